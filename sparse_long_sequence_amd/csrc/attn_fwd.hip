// attn_fwd.hip — band + global attention (Longformer / ETC) on gfx950.
//
// One launch holds two kinds of workgroups:
//   * global-row workgroups (first in the grid), one per (batch, head, 64
//     global rows, key chunk): each global row against a chunk of all keys,
//     written as a partial (normalised O, lse) to the workspace; the last
//     workgroup of a row tile to finish merges the chunk partials;
//   * band workgroups, one per 64-row query tile of one residue class of one
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

// Number of residue-class query tiles of a head of dilation d.
__host__ __device__ inline int32_t band_tiles_of_head(int32_t N, int32_t d) {
  int32_t t = 0;
  for (int32_t c = 0; c < d && c < N; ++c) t += ((N - c + d - 1) / d + kTQ - 1) / kTQ;
  return t;
}

// Number of entries of the sorted array g[0..n) that are < p.
__device__ __forceinline__ int32_t lower_bound(const int32_t* g, int32_t n, int32_t p) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    if (g[mid] < p) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <typename T>
struct OutT;
template <>
struct OutT<bf16> { typedef bf16 type; };
template <>
struct OutT<float> { typedef float type; };

template <typename T>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
  using TT = TileTraits<T>;
  using O = typename OutT<T>::type;
  __shared__ typename TT::Smem sm;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t wg = (int32_t)blockIdx.x;
  const int32_t N = a.N;
  const size_t head_elems = (size_t)N * kD;

  if (wg >= a.n_glob_wg) {
    // ---------------- band workgroup ----------------
    const int32_t bw = wg - a.n_glob_wg;
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
    // A tile made only of global rows belongs to the global-row pass.
    if (a.n_global > 0 && d == 1) {
      const int32_t ng = lower_bound(a.gidx, a.n_global, qbase + qcount) -
                         lower_bound(a.gidx, a.n_global, qbase);
      if (ng == qcount) return;
    }
    if (a.rel_bias && tid < 2 * a.rel_k + 1) sm.bias[tid] = a.rel_bias[h * (2 * a.rel_k + 1) + tid];

    const T* qb = reinterpret_cast<const T*>(a.q) + bh * head_elems;
    const T* kb = reinterpret_cast<const T*>(a.k) + bh * head_elems;
    const T* vb = reinterpret_cast<const T*>(a.v) + bh * head_elems;
    const RowMap qm = {nullptr, qbase, d, qcount};
    typename TT::Wave w;
    TT::load_q(w, qb, qm, wave, lane);
    const int32_t qi = 16 * wave + (lane & 15);
    const int32_t qpos = qbase + d * qi;

    // window keys in strided index space [lo, hi]
    const int32_t R = a.radius;
    const int32_t lo = max(0, t0 - R);
    const int32_t hi = a.causal ? (t0 + qcount - 1) : min(n_c - 1, t0 + qcount - 1 + R);
    const int32_t n_band = (hi - lo + 1 + kTK - 1) / kTK;

    // global-column tiles that can hold an allowed pair (bit set = keep)
    const int32_t n_gt = (a.n_global + kTK - 1) / kTK;
    uint64_t keep = ~0ull;
    const int32_t i_lo = qbase, i_hi = qbase + d * (qcount - 1);
    if (n_gt <= 64) {
      keep = 0;
      for (int32_t gt = 0; gt < n_gt; ++gt) {
        const int32_t cnt = min(kTK, a.n_global - gt * kTK);
        const int32_t g_lo = a.gidx[gt * kTK], g_hi = a.gidx[gt * kTK + cnt - 1];
        bool all_in_band = false;
        if (d == 1) {
          all_in_band = a.causal ? (g_lo >= i_hi - R && g_hi <= i_lo)
                                 : (g_lo >= i_hi - R && g_hi <= i_lo + R);
        }
        const bool none_allowed_causal = a.causal && g_lo > i_hi;
        if (!all_in_band && !none_allowed_causal) keep |= (1ull << gt);
      }
    }
    const int32_t n_glob = n_gt <= 64 ? __builtin_popcountll(keep) : n_gt;

    auto desc = [&](int32_t n, RowMap& km, MaskRule& mr) {
      if (n < n_band) {
        const int32_t u0 = lo + n * kTK;
        const int32_t kcount = min(kTK, hi - u0 + 1);
        km = {nullptr, c + d * u0, d, kcount};
        const int32_t dmin = u0 - t0 - (qcount - 1);
        const int32_t dmax = u0 + kcount - 1 - t0;
        const bool full = kcount == kTK && dmin >= -R && dmax <= (a.causal ? 0 : R);
        mr = {kBand, full ? 0 : 1, a.causal, R, d, t0 - u0};
      } else {
        int32_t x = n - n_band, gt = x;
        if (n_gt <= 64) {
          uint64_t m = keep;
          for (int32_t s = 0; s < x; ++s) m &= m - 1;
          gt = __builtin_ctzll(m);
        }
        const int32_t kcount = min(kTK, a.n_global - gt * kTK);
        km = {a.gidx + gt * kTK, 0, 1, kcount};
        const int32_t g_lo = a.gidx[gt * kTK], g_hi = a.gidx[gt * kTK + kcount - 1];
        const bool outside = (g_hi < i_lo - d * R) || (g_lo > i_hi + d * R);
        const bool causal_ok = !a.causal || g_hi <= i_lo;
        const bool full = kcount == kTK && outside && causal_ok;
        mr = {kGlobCol, full ? 0 : 1, a.causal, R, d, 0};
      }
    };
    const BiasRule br = {a.rel_bias ? sm.bias : nullptr, a.rel_k, 0};
    const bool need_glob = a.rel_bias != nullptr && a.n_global > 0;
    run_tiles<T>(sm, w, kb, vb, n_band + n_glob, desc, br, need_glob, a.gidx, a.n_global, qi, qpos,
                 a.scale_log2);

    // epilogue: rows outside G (the global-row pass owns the rest)
    const float l_tot = wave_sum_xor16_32(w.l);
    if (qi < qcount) {
      const bool is_g = a.n_global > 0 && sorted_contains(a.gidx, a.n_global, qpos);
      if (!is_g) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        O* dst = reinterpret_cast<O*>(a.out) + bh * head_elems + (size_t)qpos * kD;
        TT::store_row(dst, w.o, inv, lane);
        if (a.lse && (lane >> 4) == 0)
          a.lse[(size_t)bh * N + qpos] = l_tot > 0.f ? (w.m + __log2f(l_tot)) * kLn2 : kNegInf;
      }
    }
    return;
  }

  // ---------------- global-row workgroup ----------------
  // global-row workgroups come first in the grid so their merges are not the tail
  const int32_t gw = wg;
  const int32_t per_bh = a.n_gq_tiles * a.n_chunks;
  const int32_t bh = gw / per_bh;
  if (bh >= a.B * a.H) return;
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
  if (a.rel_bias && tid < 2 * a.rel_k + 1) sm.bias[tid] = a.rel_bias[h * (2 * a.rel_k + 1) + tid];

  const T* qb = reinterpret_cast<const T*>(a.qg) + bh * head_elems;
  const T* kb = reinterpret_cast<const T*>(a.kg) + bh * head_elems;
  const T* vb = reinterpret_cast<const T*>(a.vg) + bh * head_elems;
  const RowMap qm = {qidx, 0, 1, qcount};
  typename TT::Wave w;
  TT::load_q(w, qb, qm, wave, lane);
  const int32_t qi = 16 * wave + (lane & 15);
  const int32_t qpos = qi < qcount ? qidx[qi] : i_max;
  auto desc = [&](int32_t n, RowMap& km, MaskRule& mr) {
    const int32_t u0 = j0 + n * kTK;
    const int32_t kcount = min(kTK, j1 - u0);
    km = {nullptr, u0, 1, kcount};
    const bool full = kcount == kTK && (!a.causal || u0 + kTK - 1 <= i_min);
    mr = {kAll, full ? 0 : 1, a.causal, 0, 1, 0};
  };
  const BiasRule br = {a.rel_bias ? sm.bias : nullptr, a.rel_k, 1};
  const bool need_glob = a.rel_bias != nullptr;
  run_tiles<T>(sm, w, kb, vb, n_tiles, desc, br, need_glob, a.gidx, a.n_global, qi, qpos,
               a.scale_log2);
  const float l_tot = wave_sum_xor16_32(w.l);
  if (qi < qcount) {
    const size_t prow = ((size_t)bh * a.n_global + gq * kTQ + qi) * a.n_chunks + chunk;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    TileTraits<float>::store_row(a.ws_o + prow * kD, w.o, inv, lane);
    if ((lane >> 4) == 0) a.ws_lse[prow] = l_tot > 0.f ? (w.m + __log2f(l_tot)) * kLn2 : kNegInf;
  }

  // The last of the n_chunks workgroups of this row tile to finish merges the
  // partials: lse = ln sum_c e^{lse_c}, O = sum_c e^{lse_c - lse} O_c, in chunk
  // order (so the result does not depend on which workgroup merges). It then
  // returns the tile's counter to zero for the next call.
  __shared__ int32_t s_last;
  __threadfence();  // publish this workgroup's partial before counting it
  __syncthreads();
  if (tid == 0) {
    const int32_t prev = atomicAdd(&a.ws_cnt[bh * a.n_gq_tiles + gq], 1);
    s_last = prev == a.n_chunks - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // see every other workgroup's partial
  // 256 threads: 4 rows at a time, thread = d
  for (int32_t r = tid >> 6; r < qcount; r += kThreads / 64) {
    const int32_t dd = tid & 63;
    const size_t p0 = ((size_t)bh * a.n_global + gq * kTQ + r) * a.n_chunks;
    float L = kNegInf;
    for (int32_t c = 0; c < a.n_chunks; ++c) L = fmaxf(L, a.ws_lse[p0 + c]);
    float acc = 0.f, S = 0.f;
    if (L != kNegInf) {
      for (int32_t c = 0; c < a.n_chunks; ++c) {
        const float lc = a.ws_lse[p0 + c];
        if (lc == kNegInf) continue;
        const float wgt = __expf(lc - L);
        S += wgt;
        acc += wgt * a.ws_o[(p0 + c) * kD + dd];
      }
    }
    const int32_t pos = qidx[r];
    O* dst = reinterpret_cast<O*>(a.out) + bh * head_elems + (size_t)pos * kD;
    const float val = S > 0.f ? acc / S : 0.f;
    if constexpr (sizeof(O) == 2) {
      reinterpret_cast<uint16_t*>(dst)[dd] = (uint16_t)f32_to_bf16_bits(val);
    } else {
      dst[dd] = val;
    }
    if (a.lse && dd == 0) a.lse[(size_t)bh * N + pos] = S > 0.f ? L + __logf(S) : kNegInf;
  }
  if (tid == 0) atomicExch(&a.ws_cnt[bh * a.n_gq_tiles + gq], 0);
}

hipError_t launch_attn(const AttnArgs& a, int32_t dtype, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_band_wg + (int64_t)a.n_glob_wg;
  if (grid <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(attn_fwd_kernel<bf16>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<float>, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int32_t host_band_tiles_of_head(int32_t N, int32_t d) { return band_tiles_of_head(N, d); }

}  // namespace la
