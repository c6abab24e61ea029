// attn_fwd.hip — band + global attention (Longformer / ETC) on gfx950.
//
// One launch holds two kinds of workgroups:
//   * global-row workgroups (first in the grid), one per (batch, head, query
//     tile of global rows, key chunk): each global row against a chunk of all keys,
//     written as a partial (normalised O, lse) to the workspace; the last
//     chunk workgroup of a tile to finish merges the tile's partials;
//   * band workgroups, one per query tile of one residue class of one
//     (batch, head): the sliding-window key tiles (strided by the head's
//     dilation), then the global-column tiles (keys of G outside the window).
//
// Pattern: Longformer page, §3.4 "Sliding Window Attention" (Fig. 2b),
// "Dilated Sliding Window Attention" (Fig. 2c), "Global Attention" (Fig. 2d),
// "Separate Linear Projections for Local vs. Global Attention",
// "Autoregressive Language Modeling Configuration" (causal window);
// ETC page, §3.4 "Global-Local Attention" (four pieces, two unified
// softmaxes) and "Relative Position Encoding" (clipped distance labels).
#include "tile_core.h"
#include "kernels.h"

namespace la {

// Number of residue-class query tiles (of tq rows) of a head of dilation d.
__host__ __device__ inline int32_t band_tiles_of_head(int32_t N, int32_t d, int32_t tq) {
  int32_t t = 0;
  for (int32_t c = 0; c < d && c < N; ++c) t += ((N - c + d - 1) / d + tq - 1) / tq;
  return t;
}

template <typename T>
struct OutT;
template <>
struct OutT<bf16> { typedef bf16 type; };
template <>
struct OutT<float> { typedef float type; };

// The label vocabulary per head: the 2k+1 distance labels, and with LBL the
// structural labels after them (n_labels entries in all).
template <typename T, bool LBL>
__device__ __forceinline__ void load_bias_table(typename TileTraits<T>::Smem& sm, const AttnArgs& a,
                                                int32_t h, int32_t tid) {
  if constexpr (LBL) {
    if (a.rel_bias && tid < a.n_labels)
      sm.bias[tid] = a.rel_bias[h * a.n_labels + tid] * kInvScale;
  } else {
    if (a.rel_bias && tid < 2 * a.rel_k + 1)
      sm.bias[tid] = a.rel_bias[h * (2 * a.rel_k + 1) + tid] * kInvScale;
  }
}

// With key-side label vectors a_l (ETC page, §3.4 "Relative Position
// Encoding", Step 3 and its implementation note): the workgroup's table of
// q_i . a_l for each of its query rows and each label, in q.k units, plus the
// scalar label bias (times sqrt(D)) when one is given too. Row r's query is
// q[pos(r)]; rt holds kTQ rows of V entries (every label). The head's label vectors are
// staged in `stage` (an LDS buffer not yet in use, at least V * D fp32);
// each thread holds a half row of its query in registers and sums one label
// in kTPR. Ends with a barrier.
static_assert(sizeof(TileTraits<bf16>::Smem::v) >= kMaxLabels * kD * sizeof(float) &&
                  sizeof(TileTraits<float>::Smem::v) >= kMaxLabels * kD * sizeof(float),
              "the V buffers stage the label vectors");

template <typename T, bool LBL, typename Pos>
__device__ __forceinline__ void build_row_table(float* rt, float* stage, const AttnArgs& a,
                                                int32_t h, const T* qb, Pos pos, int32_t tid) {
  using TT = TileTraits<T>;
  constexpr int32_t kTPR = TT::kThreads / TT::kTQ;  // threads per query row
  const int32_t nl = LBL ? a.n_labels : 2 * a.rel_k + 1;
  const f32x4* av = reinterpret_cast<const f32x4*>(a.rel_vec + (size_t)h * nl * kD);
  for (int32_t x = tid; x < nl * (kD / 4); x += TT::kThreads)
    reinterpret_cast<f32x4*>(stage)[x] = av[x];
  __syncthreads();
  const int32_t r = tid % TT::kTQ, sub = tid / TT::kTQ;  // sub is the same across a wave
  const T* qr = qb + (size_t)pos(r) * kD;
  const float* sb = a.rel_bias ? a.rel_bias + h * nl : nullptr;
  // Half a query row at a time in registers; this thread's labels sub,
  // sub + kTPR, ... in groups of kGroup; each partial sum goes straight to the
  // thread's own table entries (the second half adds to the first).
  constexpr int32_t kGroup = 8;
#pragma unroll 1
  for (int32_t d0 = 0; d0 < kD; d0 += 32) {
    float qv[32];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 x = ldg16(qr + d0 + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[8 * c + 2 * e] = __builtin_bit_cast(float, x[e] << 16);
          qv[8 * c + 2 * e + 1] = __builtin_bit_cast(float, x[e] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 x = __builtin_bit_cast(f32x4, ldg16(qr + d0 + 4 * c));
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * c + e] = x[e];
      }
    }
#pragma unroll 1
    for (int32_t j0 = 0; sub + j0 * kTPR < nl; j0 += kGroup) {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int32_t l = sub + (j0 + j) * kTPR;
        if (l < nl) {
          const f32x4* al = reinterpret_cast<const f32x4*>(stage + l * kD + d0);
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int c = 0; c < 8; c += 2) {
            const f32x4 x0 = al[c], x1 = al[c + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s0 = __builtin_fmaf(qv[4 * c + e], x0[e], s0);
              s1 = __builtin_fmaf(qv[4 * c + 4 + e], x1[e], s1);
            }
          }
          float* dst = rt + r * nl + l;
          *dst = (d0 == 0 ? (sb ? sb[l] * kInvScale : 0.f) : *dst) + (s0 + s1);
        }
      }
    }
  }
  __syncthreads();
}

// Segment masks: this lane's query row's segment id and the range of ids over
// the wave's rows (segb: the batch row's ids).
__device__ __forceinline__ void segment_rows(GlobInfo& gi, const int32_t* segb, int32_t qpos) {
  gi.segb = segb;
  gi.sq = segb[qpos];
  gi.sq_min = __builtin_amdgcn_readfirstlane(wave_min(gi.sq));  // uniform: scalar registers
  gi.sq_max = __builtin_amdgcn_readfirstlane(wave_max(gi.sq));
}

// ---------------------------------------------------------------------------
// band workgroup: one query tile of one residue class (positions c + d*t)
// ---------------------------------------------------------------------------
// BIAS: a relative-position bias table is given (the no-bias loops are
// compiled without its code).
template <typename T, bool BIAS, bool SEG, bool LBL>
__device__ __forceinline__ void band_workgroup(const AttnArgs& a, typename TileTraits<T>::Smem& sm,
                                               float* rowtab, int32_t bw) {
  using TT = TileTraits<T>;
  using O = typename OutT<T>::type;
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t N = a.N;
  const size_t head_elems = (size_t)N * kD;
  const int32_t bh = bw / a.band_tiles_per_head;
  int32_t tile = bw % a.band_tiles_per_head;
  const int32_t h = bh % a.H;
  const int32_t d = a.dil[h];
  int32_t c = 0, n_c = 0;
  for (; c < d && c < N; ++c) {
    n_c = (N - c + d - 1) / d;
    const int32_t tc = (n_c + kTQ - 1) / kTQ;
    if (tile < tc) break;
    tile -= tc;
  }
  if (c >= d || c >= N) return;  // padding workgroup of a less-dilated head
  const int32_t t0 = tile * kTQ;
  const int32_t qcount = min(kTQ, n_c - t0);
  const int32_t qbase = c + d * t0;
  const int32_t i_lo = qbase, i_hi = qbase + d * (qcount - 1);

  // Bounds of the global index list (uniform scalar loads, consumed late):
  // only a tile whose rows meet [G first, G last] can hold global rows.
  const int32_t ng = a.n_global;
  const int32_t g_first = ng > 0 ? a.gidx[0] : 0;
  const int32_t g_last = ng > 0 ? a.gidx[ng - 1] : -1;
  // a tile made only of global rows belongs to the global-row pass (detected
  // here when G is one run of consecutive positions)
  if (d == 1 && g_last - g_first == ng - 1 && g_first <= i_lo && g_last >= i_hi) return;
  load_bias_table<T, LBL>(sm, a, h, tid);

  const T* qb = reinterpret_cast<const T*>(a.q) + bh * head_elems;
  const T* kb = reinterpret_cast<const T*>(a.k) + bh * head_elems;
  const T* vb = reinterpret_cast<const T*>(a.v) + bh * head_elems;
  const int32_t qi = TT::qrow(wave, lane, 0);
  const int32_t qpos = qbase + d * min(qi, qcount - 1);
  const bool dead = TT::kQW * wave >= qcount;  // no valid row in this wave
  if (BIAS && a.rel_vec)  // before the wave state is live
    build_row_table<T, LBL>(rowtab, reinterpret_cast<float*>(&sm.v[0][0]), a, h, qb,
                       [&](int32_t r) { return qbase + d * min(r, qcount - 1); }, tid);
  typename TT::Wave w;
  TT::load_q(w, qb, &qpos, lane);

  // window keys in strided index space [lo, hi]
  const int32_t R = a.radius;
  const int32_t lo = max(0, t0 - R);
  const int32_t hi = a.causal ? (t0 + qcount - 1) : min(n_c - 1, t0 + qcount - 1 + R);
  const int32_t n_band = (hi - lo + 1 + kTK - 1) / kTK;
  const bool want_bias = a.rel_bias != nullptr || a.rel_vec != nullptr;
  // flags: the tiles stage their keys' global flags (for the bias, and with
  // LBL for the labels and the piece-selected segment masks)
  bool flags = want_bias;
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  LabelRule lr = {};
  if constexpr (LBL) {
    // non-global rows: the labels of their global keys; segment ids mask l2g
    // (global keys) and l2l (the others)
    lr.lab = a.llabel ? a.llabel + (size_t)(bh / a.H) * N * a.n_global : nullptr;
    lr.stride = (uint32_t)a.n_global;
    lr.V = a.n_labels;
    lr.want_rank = a.llabel != nullptr;
    lr.seg_g = (a.seg_pieces & 4) != 0;
    lr.seg_l = (a.seg_pieces & 8) != 0;
    flags = flags || a.llabel != nullptr || (a.seg && a.seg_pieces != 15);
  }
  // (the label kernel is built with SEG and may run without segment ids)
  if (SEG && (!LBL || a.seg)) segment_rows(gi, a.seg + (size_t)(bh / a.H) * N, qpos);
  if (flags && a.n_global > 0) {
    if (hi - lo + 1 <= 32 * kGMaskWords) {
      build_gmask<T>(sm, a.gidx, a.n_global, c + d * lo, d, hi - lo + 1, tid);
      gi.mode = kGlobBitmap;
    } else {
      gi.mode = kGlobSearch;
    }
  }
  BiasRule br = {!want_bias ? nullptr : a.rel_vec ? rowtab : sm.bias, a.rel_k, 0,
                 a.rel_vec ? 2 * a.rel_k + 1 : 0};
  if constexpr (LBL) br.row_stride = a.rel_vec ? a.n_labels : 0;

  auto band_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = lo + n * kTK;
    const int32_t kcount = min(kTK, hi - u0 + 1);
    kt = {nullptr, c + d * u0, d, kcount, u0 - lo, gi.mode};
    // strided index difference key - query = kj - qi - (t0 - u0)
    const int32_t dmin = u0 - t0 - (qcount - 1);
    const int32_t dmax = u0 + kcount - 1 - t0;
    const int32_t hib = a.causal ? 0 : R;
    const bool full = kcount == kTK && dmin >= -R && dmax <= hib;
    mr = {kRange, full ? 0 : 1, 0, t0 - u0, -R, hib, 0, 0, 1};
  };
  // When d = 1 and G is one run of consecutive positions, its key tiles are
  // strided views too: they follow the window tiles in the same loop (their
  // first loads overlap the last window tile). Otherwise they are gathered
  // through G in a second loop.
  const bool g_run = ng > 0 && d == 1 && g_last - g_first == ng - 1;
  if (g_run) {
    const int32_t n_gt = (ng + kTK - 1) / kTK;
    const int32_t glob_mode = flags ? kGlobAll : kGlobNone;
    // The global key tiles come first: they are the same for every query tile
    // of the head, so the workgroups' first K/V loads mostly hit in L2 while
    // their band tiles stream in behind (the online softmax is order-free).
    auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
      if (n >= n_gt) {
        band_desc(n - n_gt, kt, mr);
        return;
      }
      // keys of G outside the window (a global key in the window is counted
      // there); a tile that cannot hold an allowed pair gets count 0
      const int32_t gt = n;
      const int32_t cnt = min(kTK, ng - gt * kTK);
      const int32_t gl = g_first + gt * kTK, gh = gl + cnt - 1;
      const bool all_in_band =
          a.causal ? (gl >= i_hi - R && gh <= i_lo) : (gl >= i_hi - R && gh <= i_lo + R);
      const bool none_causal = a.causal && gl > i_hi;
      const bool keep = !all_in_band && !none_causal;
      kt = {nullptr, gl, 1, keep ? cnt : 0, 0, glob_mode, LBL ? 1 + gt * kTK : 0};
      // every key outside every row's window (and not after any row, causal):
      // no mask needed
      const bool all_out = cnt == kTK && (gh < i_lo - R || (!a.causal && gl > i_hi + R)) &&
                           (!a.causal || gh <= i_lo);
      // key gl + kj is allowed iff its distance kj - (qpos - gl) to the query
      // lies outside the window [-R, R] (causal: [-R, inf), so also j <= i)
      mr = {kOutside, all_out ? 0 : 1, 1, -gl, -R, a.causal ? kFar : R, 0, 0, 1};
    };
    run_tiles<T, false, BIAS, SEG, LBL>(sm, w, kb, vb, n_band + n_gt, desc, br, gi, lr, qi, qpos, dead,
                        a.scale_log2);
  } else {
    run_tiles<T, false, BIAS, SEG, LBL>(sm, w, kb, vb, n_band, band_desc, br, gi, lr, qi, qpos, dead,
                                        a.scale_log2);
  }

  if (a.n_global > 0 && !g_run) {
    // global-column tiles that can hold an allowed pair (bit set = keep)
    const int32_t n_gt = (a.n_global + kTK - 1) / kTK;
    uint64_t keep = ~0ull;
    if (n_gt <= 64) {
      keep = 0;
      for (int32_t gt = 0; gt < n_gt; ++gt) {
        const int32_t cnt = min(kTK, a.n_global - gt * kTK);
        const int32_t gl = a.gidx[gt * kTK], gh = a.gidx[gt * kTK + cnt - 1];
        bool all_in_band = false;
        if (d == 1)
          all_in_band = a.causal ? (gl >= i_hi - R && gh <= i_lo) : (gl >= i_hi - R && gh <= i_lo + R);
        const bool none_causal = a.causal && gl > i_hi;
        if (!all_in_band && !none_causal) keep |= (1ull << gt);
      }
    }
    const int32_t n_glob = n_gt <= 64 ? __builtin_popcountll(keep) : n_gt;
    auto glob_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
      int32_t gt = n;
      if (n_gt <= 64) {
        uint64_t m = keep;
        for (int32_t s = 0; s < n; ++s) m &= m - 1;
        gt = __builtin_ctzll(m);
      }
      const int32_t kcount = min(kTK, a.n_global - gt * kTK);
      kt = {a.gidx + gt * kTK, 0, 1, kcount, 0, flags ? kGlobAll : kGlobNone,
            LBL ? 1 + gt * kTK : 0};
      const int32_t gl = a.gidx[gt * kTK], gh = a.gidx[gt * kTK + kcount - 1];
      const bool outside = (gh < i_lo - d * R) || (gl > i_hi + d * R);
      const bool causal_ok = !a.causal || gh <= i_lo;
      const bool full = kcount == kTK && outside && causal_ok;
      mr = {kGlobCol, full ? 0 : 1, 0, 0, 0, 0, a.causal, R, d};
    };
    const GlobInfo gall = {flags ? kGlobAll : kGlobNone, a.gidx, a.n_global,
                           gi.segb, gi.sq, gi.sq_min, gi.sq_max};
    run_tiles<T, true, BIAS, SEG, LBL>(sm, w, kb, vb, n_glob, glob_desc, br, gall, lr, qi, qpos, dead,
                                       a.scale_log2);
  }

  // epilogue: rows outside G (the global-row pass owns the rest)
  const float l_tot = TT::row_sum(w.l[0]);
  if (qi < qcount) {
    const bool is_g = g_first <= i_hi && g_last >= i_lo && sorted_contains(a.gidx, ng, qpos);
    if (!is_g) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      O* dst = reinterpret_cast<O*>(a.out) + bh * head_elems + (size_t)qpos * kD;
      TT::store_row(dst, w, 0, inv, lane);
      if (a.lse && TT::row_leader(lane))
        a.lse[(size_t)bh * N + qpos] = l_tot > 0.f ? (w.m[0] + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// merge of the key-chunk partials of one tile of global rows
// ---------------------------------------------------------------------------
// lse = ln sum_c e^{lse_c}, O = sum_c e^{lse_c - lse} O_c over the n_chunks
// partials of each row (all complete and written through to memory). 8 lanes
// per row with 8 consecutive d each, 32 rows per pass; chunks are taken
// kMergeGroup at a time with all their loads issued together (a running max
// keeps the sums bounded).
constexpr int32_t kMergeGroup = 8;

template <typename T>
__device__ __forceinline__ void merge_global_tile(float* ws_o, float* ws_lse, const int32_t* gidx,
                                                  void* out, float* lse, int32_t n_global,
                                                  int32_t nc, int32_t N, int32_t bh,
                                                  int32_t r_first, int32_t qcount) {
  using O = typename OutT<T>::type;
  constexpr int32_t nt = TileTraits<T>::kThreads;
  constexpr int32_t kRowsPerPass = nt / 8;
  const int32_t tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t ro = buffer_of(ws_o), rl = buffer_of(ws_lse);
  const int32_t d8 = 8 * (tid & 7);
  for (int32_t r0 = 0; r0 < qcount; r0 += kRowsPerPass) {
    const int32_t r = r0 + tid / 8;
    if (r >= qcount) break;
    const int32_t p0 = (bh * n_global + r_first + r) * nc;
    const int32_t pos = gidx[r_first + r];
    float L = kNegInf, S = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    for (int32_t c0 = 0; c0 < nc; c0 += kMergeGroup) {
      float lc[kMergeGroup];
      f32x4 oa[kMergeGroup], ob[kMergeGroup];
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        const int32_t p = p0 + min(c0 + j, nc - 1);  // always a valid partial
        const float lj = ld_coh4(rl, p * 4);
        lc[j] = c0 + j < nc ? lj : kNegInf;
        oa[j] = ld_coh16(ro, (p * kD + d8) * 4);
        ob[j] = ld_coh16(ro, (p * kD + d8 + 4) * 4);
      }
      float Lg = L;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) Lg = fmaxf(Lg, lc[j]);
      if (Lg == kNegInf) continue;
      const float sc = L == kNegInf ? 0.f : __expf(L - Lg);
      S *= sc;
      acc0 *= sc;
      acc1 *= sc;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        const float wgt = lc[j] == kNegInf ? 0.f : __expf(lc[j] - Lg);
        S += wgt;
        acc0 += wgt * oa[j];
        acc1 += wgt * ob[j];
      }
      L = Lg;
    }
    O* dst = reinterpret_cast<O*>(out) + ((size_t)bh * N + pos) * kD + d8;
    const float inv = S > 0.f ? 1.f / S : 0.f;
    if constexpr (sizeof(O) == 2) {
      u32x4 pk;
      pk[0] = pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
      pk[1] = pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
      pk[2] = pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
      pk[3] = pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
      *reinterpret_cast<u32x4*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = acc0 * inv;
      *reinterpret_cast<f32x4*>(dst + 4) = acc1 * inv;
    }
    if (lse && d8 == 0) lse[(size_t)bh * N + pos] = S > 0.f ? L + __logf(S) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// global-row workgroup: one tile of global rows against one chunk of keys
// ---------------------------------------------------------------------------
template <typename T, bool BIAS, bool SEG, bool LBL>
__device__ __forceinline__ void global_workgroup(const AttnArgs& a,
                                                 typename TileTraits<T>::Smem& sm, float* rowtab,
                                                 int32_t gw) {
  using TT = TileTraits<T>;
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t N = a.N;
  const size_t head_elems = (size_t)N * kD;
  const int32_t per_bh = a.n_gq_tiles * a.n_chunks;
  const int32_t bh = gw / per_bh;
  const int32_t rem = gw % per_bh;
  const int32_t gq = rem / a.n_chunks, chunk = rem % a.n_chunks;
  const int32_t h = bh % a.H;
  const int32_t qcount = min(kTQ, a.n_global - gq * kTQ);
  const int32_t* qidx = a.gidx + gq * kTQ;
  const int32_t i_min = qidx[0], i_max = qidx[qcount - 1];
  const int32_t j0 = chunk * a.chunk_len;
  int32_t j1 = min(N, j0 + a.chunk_len);
  if (a.causal) j1 = min(j1, i_max + 1);
  const int32_t n_tiles = j1 > j0 ? (j1 - j0 + kTK - 1) / kTK : 0;
  load_bias_table<T, LBL>(sm, a, h, tid);
  const bool want_bias = a.rel_bias != nullptr || a.rel_vec != nullptr;
  bool flags = want_bias;  // as in the band workgroup
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  LabelRule lr = {};
  if constexpr (LBL) {
    // global rows: their label rows; segment ids mask g2g (global keys) and
    // g2l (the others)
    lr.lab = a.glabel ? a.glabel + ((size_t)(bh / a.H) * a.n_global + gq * kTQ) * N : nullptr;
    lr.rows_global = 1;
    lr.row_last = qcount - 1;  // rows past it belong to no global token
    lr.stride = (uint32_t)N;
    lr.V = a.n_labels;
    lr.seg_g = (a.seg_pieces & 1) != 0;
    lr.seg_l = (a.seg_pieces & 2) != 0;
    flags = flags || a.glabel != nullptr || (a.seg && a.seg_pieces != 15);
  }
  if (flags && n_tiles > 0) {
    build_gmask<T>(sm, a.gidx, a.n_global, j0, 1, j1 - j0, tid);  // j1 - j0 <= chunk_len
    gi.mode = kGlobBitmap;
  }

  const T* qb = reinterpret_cast<const T*>(a.qg) + bh * head_elems;
  const T* kb = reinterpret_cast<const T*>(a.kg) + bh * head_elems;
  const T* vb = reinterpret_cast<const T*>(a.vg) + bh * head_elems;
  if (BIAS && a.rel_vec)
    build_row_table<T, LBL>(rowtab, reinterpret_cast<float*>(&sm.v[0][0]), a, h, qb,
                       [&](int32_t r) { return qidx[min(r, qcount - 1)]; }, tid);
  // A tile of at most half the workgroup's rows (bf16: two key sub-tiles per
  // tile) keeps every wave busy: waves w and w + 2 take the same rows, wave w
  // the first 32 keys of each tile and wave w + 2 the last 32, and their
  // running states are folded together at the end.
  const bool split = TT::kSub == 2 && qcount <= 2 * TT::kQW;
  const int32_t wrow = split ? (wave & 1) : wave;
  const int32_t qi = TT::qrow(wrow, lane, 0);
  const int32_t qpos = qidx[min(qi, qcount - 1)];
  // (the label kernel is built with SEG and may run without segment ids)
  if (SEG && (!LBL || a.seg)) segment_rows(gi, a.seg + (size_t)(bh / a.H) * N, qpos);
  const bool dead = TT::kQW * wrow >= qcount;  // no valid row in this wave
  typename TT::Wave w;
  TT::load_q(w, qb, &qpos, lane);
  auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = j0 + n * kTK;
    const int32_t kcount = min(kTK, j1 - u0);
    kt = {nullptr, u0, 1, kcount, u0 - j0, gi.mode};
    // key position u0 + kj <= qpos  <=>  kj - (qpos - u0) <= 0
    const bool full = kcount == kTK && (!a.causal || u0 + kTK - 1 <= i_min);
    mr = {kRange, full ? 0 : 1, 1, -u0, -kFar, a.causal ? 0 : kFar, 0, 0, 1};
  };
  BiasRule br = {!want_bias ? nullptr : a.rel_vec ? rowtab : sm.bias, a.rel_k, 1,
                 a.rel_vec ? 2 * a.rel_k + 1 : 0};
  if constexpr (LBL) br.row_stride = a.rel_vec ? a.n_labels : 0;
  run_tiles<T, false, BIAS, SEG, LBL>(sm, w, kb, vb, n_tiles, desc, br, gi, lr, qi, qpos, dead,
                                      a.scale_log2,
                      split ? (wave >> 1) : -1);
  bool holds_rows = true;  // this wave holds a final running state
  if constexpr (TT::kSub == 2) {
    if (split) {
      TT::fold_pairs(sm, w, wave, lane);
      holds_rows = wave < 2;
    }
  }
  // The chunk's partial (normalised O, lse) of each row, written through to
  // memory so that the workgroup merging the chunks may run on another XCD.
  const __amdgpu_buffer_rsrc_t ro = buffer_of(a.ws_o), rl = buffer_of(a.ws_lse);
  const float l_tot = TT::row_sum(w.l[0]);
  if (holds_rows && qi < qcount) {
    const int32_t prow = ((bh * a.n_global + gq * kTQ + qi) * a.n_chunks + chunk);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    TT::store_row_coh(ro, prow * (kD * 4), w, inv, lane);
    if (TT::row_leader(lane))
      st_coh4(rl, prow * 4, l_tot > 0.f ? (w.m[0] + __log2f(l_tot)) * kLn2 : kNegInf);
  }
  // Arrival: the last chunk workgroup of this tile merges all its chunks. The
  // counter word carries the call's token in its high half; a word with any
  // other high half (zero, another call's token, stale partial data: fp32
  // values, never this NaN pattern) is taken as no arrival yet.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
  __syncthreads();
  int32_t* flag = reinterpret_cast<int32_t*>(&sm.gcls[0]);
  uint64_t* cnt = a.ws_cnt + (bh * a.n_gq_tiles + gq);
  if (tid == 0) {
    const uint64_t tag = (uint64_t)a.token << 32;
    // No load first: the CAS returns the word's value when the guess misses (a
    // device-coherent load before it made the whole launch ~3 us slower). The
    // guess is 0, what every completed call leaves.
    uint64_t old = 0;
    uint64_t nv;
    do {
      nv = (old >> 32) == (uint64_t)a.token ? old + 1u : tag + 1u;
    } while (!__hip_atomic_compare_exchange_strong(cnt, &old, nv, __ATOMIC_RELAXED,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const bool last = (uint32_t)nv == (uint32_t)a.n_chunks;
    if (last) __hip_atomic_store(cnt, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  merge_global_tile<T>(a.ws_o, a.ws_lse, a.gidx, a.out, a.lse, a.n_global, a.n_chunks, N, bh,
                       gq * kTQ, qcount);
}

// At least kMinWavesPerEU waves per SIMD (the label kernel: at most 3, as it
// needs more registers): that bounds each wave's registers.
// BIAS: a relative-position bias (scalar table and/or key-side label vectors)
// is given; SEG: segment masks are given; LBL: per-pair label matrices and/or
// segment masks of some pieces only (instantiated with BIAS and SEG). Each
// kernel carries only the code its flags need.
template <typename T, bool BIAS, bool SEG, bool LBL>
__global__ __launch_bounds__(TileTraits<T>::kThreads)
__attribute__((amdgpu_waves_per_eu(LBL && TileTraits<T>::kMinWavesPerEU > 3 ? 3 : TileTraits<T>::kMinWavesPerEU)))
void attn_fwd_kernel(AttnArgs a) {
  __shared__ typename TileTraits<T>::Smem sm;
  // per-row label table (key-side label vectors only; sized at launch, else empty)
  extern __shared__ float rowtab[];
  // Block b runs on XCD b % 8. Each XCD takes an equal share of the global-row
  // workgroups, then an equal share of the band workgroups, each share a
  // contiguous range (workgroups of one head then share K/V in that XCD's L2,
  // and no XCD is left with only the shorter global-row work).
  const int32_t x = (int32_t)blockIdx.x % kXcds, j = (int32_t)blockIdx.x / kXcds;
  const int32_t gper = (a.n_glob_wg + kXcds - 1) / kXcds;
  const int32_t bper = (a.n_band_wg + kXcds - 1) / kXcds;
  const int32_t gcnt = min(gper, max(0, a.n_glob_wg - x * gper));
  const int32_t bcnt = min(bper, max(0, a.n_band_wg - x * bper));
  if (j < gcnt)
    global_workgroup<T, BIAS, SEG, LBL>(a, sm, rowtab, x * gper + j);
  else if (j - gcnt < bcnt)
    band_workgroup<T, BIAS, SEG, LBL>(a, sm, rowtab, x * bper + (j - gcnt));
}

hipError_t launch_attn(const AttnArgs& a, int32_t dtype, hipStream_t stream) {
  if ((int64_t)a.n_band_wg + a.n_glob_wg <= 0) return hipSuccess;
  // per-XCD shares of each kind (see attn_fwd_kernel)
  const int64_t grid = (int64_t)kXcds * ((a.n_glob_wg + kXcds - 1) / kXcds +
                                         (a.n_band_wg + kXcds - 1) / kXcds);
  // dynamic LDS: the per-row label table of key-side label vectors
  const size_t rows = dtype == 1 ? TileTraits<bf16>::kTQ : TileTraits<float>::kTQ;
  const uint32_t dyn = a.rel_vec ? (uint32_t)(rows * a.n_labels * sizeof(float)) : 0u;
  const bool bias = a.rel_bias != nullptr || a.rel_vec != nullptr;
  const bool seg = a.seg != nullptr;
  // the label kernel also reads tables wider than the 2k+1 distance labels
  const bool lbl = a.glabel != nullptr || a.llabel != nullptr || (seg && a.seg_pieces != 15) ||
                   (bias && a.n_labels != 2 * a.rel_k + 1);
  const dim3 g((uint32_t)grid);
  if (dtype == 1) {
    const dim3 b(TileTraits<bf16>::kThreads);
    if (lbl) hipLaunchKernelGGL((attn_fwd_kernel<bf16, true, true, true>), g, b, dyn, stream, a);
    else if (bias && seg) hipLaunchKernelGGL((attn_fwd_kernel<bf16, true, true, false>), g, b, dyn, stream, a);
    else if (bias) hipLaunchKernelGGL((attn_fwd_kernel<bf16, true, false, false>), g, b, dyn, stream, a);
    else if (seg) hipLaunchKernelGGL((attn_fwd_kernel<bf16, false, true, false>), g, b, dyn, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<bf16, false, false, false>), g, b, dyn, stream, a);
  } else {
    const dim3 b(TileTraits<float>::kThreads);
    if (lbl) hipLaunchKernelGGL((attn_fwd_kernel<float, true, true, true>), g, b, dyn, stream, a);
    else if (bias && seg) hipLaunchKernelGGL((attn_fwd_kernel<float, true, true, false>), g, b, dyn, stream, a);
    else if (bias) hipLaunchKernelGGL((attn_fwd_kernel<float, true, false, false>), g, b, dyn, stream, a);
    else if (seg) hipLaunchKernelGGL((attn_fwd_kernel<float, false, true, false>), g, b, dyn, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<float, false, false, false>), g, b, dyn, stream, a);
  }
  return hipGetLastError();
}

int32_t host_band_tiles_of_head(int32_t N, int32_t d, int32_t tq) {
  return band_tiles_of_head(N, d, tq);
}
int32_t host_query_tile(int32_t dtype) {
  return dtype == 1 ? TileTraits<bf16>::kTQ : TileTraits<float>::kTQ;
}

}  // namespace la
