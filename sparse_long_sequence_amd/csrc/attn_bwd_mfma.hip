// attn_bwd_mfma.hip — the bf16 backward of band + global attention and of the
// LongNet mixture on the MFMA tile engine (the chain rule through the masked
// softmax: LongNet page, §3.4 "Standard Self-Attention and Sparse Attention
// (Preliminaries)", Eq. 2, differentiated; the pattern as in attn_fwd.hip).
// Band + global: one launch holds the dK/dV and the dQ workgroups (D_i comes
// from a launch before, each row's label table too when labels carry vectors
// or a table), and the split global tiles' partial sums are added by a launch
// after. The forward's per-instance inputs (bias tables, key-side label
// vectors, segment ids, label matrices and piece masks) select instantiations
// of the same workgroups.
//
// For the forward's own lse (natural log) and D_i = dO_i . O_i,
//   P_ij  = exp(q_i . k_j / sqrt(D) - lse_i),   dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),                 dQ_i  = sum_j dS_ij k_j / sqrt(D).
// A workgroup owns a query tile of the non-global rows of one residue class
// (as the forward's band workgroups) and streams the same key tiles through
// LDS: the window, then the global keys outside it. Per 32-key sub-tile a
// wave forms S^T = K Q^T and dP^T = V dO^T on MFMA (its rows' Q and dO in
// registers), P from lse with no running max (lse is final), dS in bf16, and
// dQ^T += K^T dS^T on MFMA with K read transposed from LDS (the forward's PV
// step with K in place of V and dS in place of P). No atomics: each dQ row is
// written once (the global rows' ranges into partial sums).
//
// dK, dV run the same engine with the roles swapped: a workgroup owns a tile
// of non-global keys (their K and V fragments in registers) and streams the
// query rows that reach them through LDS (Q in the K slot, dO in the V slot,
// each row's negated offsets -lse / scale and -D_i next to them, where the
// score and dP MFMAs start):
//   S'^T = Q K^T and dP'^T = dO V^T per 32-row sub-tile, P and dS as above,
//   dV^T += dO^T P^T and dK^T += Q^T dS^T (transposed LDS reads of dO and Q),
// first over the window's non-global rows, then over the global rows (which
// reach every key; with separate projections through qg_i, kg_j, vg_j into
// dKg, dVg).
#include "tile_core.h"
#include "bwd_kernels.h"

namespace la {
namespace {

using TT = TileTraits<bf16>;
constexpr float kLog2e = 1.4426950408889634f;

// One wave's rows: Q and dO fragments (B operands), lse in log2 units (+inf
// for a row without keys, so its P are 0), D_i, and dQ^T (as the forward's O).
struct DqWave {
  bf16x8 qf[4];
  bf16x8 df[4];
  f32x16 acc[2];
  float lse2;
  float di;
  float c_lo, c_hi;  // key vectors: this lane's dS sums over the two clipped labels
};

__device__ __forceinline__ void load_frag(bf16x8 (&f)[4], const bf16* base, int32_t pos,
                                          int32_t lane) {
  const bf16* src = base + (size_t)pos * kD + 8 * (lane >> 5);
#pragma unroll
  for (int st = 0; st < 4; ++st) f[st] = __builtin_bit_cast(bf16x8, ldg16(src + 16 * st));
}

// D_i = dO_i . O_i of this lane's row, given its dO fragment (the row's two
// lanes hold one half each).
__device__ __forceinline__ float row_delta(const bf16x8 (&df)[4], const bf16* ob, int32_t pos,
                                           int32_t lane) {
  bf16x8 of[4];
  load_frag(of, ob, pos, lane);
  float x = 0.f;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x = __builtin_fmaf((float)df[st][e], (float)of[st][e], x);
  }
  return xor32_sum(x);
}

// s[e] = acc[e] + X[key_const(sb, e) + key_lane] . f for the staged tile X
// (K or V, [key][d] rows in the engine's swizzled layout): S^T or dP^T of
// sub-tile sb, accumulated onto acc (zero, or a per-element offset).
__device__ __forceinline__ void tile_dots(const bf16* tile, const bf16x8 (&f)[4], int32_t lane,
                                          int sb, float s[TT::kNS], f32x16 acc = {}) {
  const int32_t r = lane & 31, h = lane >> 5;
  const int32_t y = h ^ TT::swz(r);
  const bf16* row = tile + (32 * sb + r) * kD;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + 8 * ((2 * st) ^ y));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, f[st], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < TT::kNS; ++e) s[e] = acc[e];
}

// acc (X^T Y^T over sub-tile sb) += X^T . G^T, X the staged tile of buffer
// `buf` read transposed (as the forward's V in its PV step) and G the
// sub-tile's bf16 weights in the forward's P layout.
template <int32_t BUF>
__device__ __forceinline__ void acc_transposed(const bf16* tile0, f32x16 (&acc)[2], int32_t lane,
                                               int sb, const TT::PTile& G) {
  typedef short __attribute__((__vector_size__(4 * sizeof(short)))) s16x4;
  const int32_t L = lane & 15, g = (lane >> 4) & 1, h = lane >> 5;
  const int32_t kr = 4 * h + (L >> 2);
  const int32_t u = (2 * g + ((L & 3) >> 1)) ^ TT::swz(kr);
  const bf16* base = tile0 + kr * kD + 4 * (L & 1);
  const uint32_t a00 = TT::lds_addr(base + 8 * (0 ^ u));
  const uint32_t a01 = TT::lds_addr(base + 8 * kD + 8 * (0 ^ u ^ 2));
  const uint32_t a10 = TT::lds_addr(base + 8 * (4 ^ u));
  const uint32_t a11 = TT::lds_addr(base + 8 * kD + 8 * (4 ^ u ^ 2));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t off = (BUF * kTK * kD + (32 * sb + 16 * t) * kD) * 2;  // bytes
    s16x4 lo0, hi0, lo1, hi1;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo0), "=&v"(hi0), "=&v"(lo1), "=&v"(hi1)
        : "v"(a00), "v"(a01), "v"(a10), "v"(a11), "i"(off));
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo0, hi0, 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo1, hi1, 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8 y = __builtin_bit_cast(bf16x8, G.p[t]);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, y, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, y, acc[1], 0, 0, 0);
  }
}

// The forward's scalar bias table on a staged tile (ETC page, §3.4 "Relative
// Position Encoding": same-kind pairs only; br.tab null: none). From the
// tile's global flags: whether any pair takes the bias (on) and whether every
// one does (same), as the forward decides them. A tile staged without flags
// has no global position in it.
struct TileBias {
  bool on, same;
};
template <int32_t BUF>
__device__ __forceinline__ TileBias tile_bias(const TT::Smem& sm, const BiasRule& br,
                                              const KeyTile& kt) {
  if (!br.tab) return {false, false};
  const int32_t gc = kt.gmode == kGlobNone ? 0 : __builtin_amdgcn_readfirstlane(sm.gcls[BUF]);
  const bool any_g = (gc & 1) != 0, all_g = (gc & 2) != 0;
  return {br.key_global_is_same_kind ? any_g : !all_g,
          br.key_global_is_same_kind ? all_g : !any_g};
}

// The head's scalar bias table, in q.k units (times sqrt(D)), into sm.bias
// for br (visible after the next barrier). flip: entry l holds entry 2k - l,
// for the dK/dV pass, whose lanes hold the keys and whose tiles hold the rows
// (the bias of a pair depends on key - row).
__device__ __forceinline__ BiasRule bias_rule(const BwdArgs& a, TT::Smem& sm, int32_t h,
                                              bool flip, int32_t lane_is_global_kind) {
  const int32_t nb = 2 * a.rel_k + 1;
  if (!a.rel_bias) return {nullptr, 0, 0, 0};
  const int32_t tid = threadIdx.x;
  if (tid < nb) sm.bias[tid] = a.rel_bias[h * nb + (flip ? nb - 1 - tid : tid)] / a.scale;
  return {sm.bias, a.rel_k, lane_is_global_kind, 0};
}

// Per-instance segment masks (packed documents; ETC page, §3.4 "Per-instance
// attention masks"): a pair is kept only when its row and key lie in the same
// segment. gi takes the batch row's segment ids, this lane's row (or key) id
// and the min / max over the wave (every lane of the wave takes part).
template <bool SEG>
__device__ __forceinline__ void seg_info(GlobInfo& gi, const BwdArgs& a, int32_t bh, int32_t pos) {
  if constexpr (SEG) {
    if (a.seg) {
      gi.segb = a.seg + (size_t)(bh / a.H) * a.N;
      gi.sq = gi.segb[pos];
      gi.sq_min = wave_min(gi.sq);
      gi.sq_max = wave_max(gi.sq);
    }
  }
}

// A staged tile against the wave's segments: 0 no pair kept, 1 every pair
// kept as far as segments go, 2 a per-element check.
template <int32_t BUF>
__device__ __forceinline__ int32_t seg_tile(const TT::Smem& sm, const GlobInfo& gi,
                                            const KeyTile& kt) {
  if (!gi.segb || kt.count <= 0) return 1;
  const int32_t kmn = __builtin_amdgcn_readfirstlane(sm.segr[BUF][0]);
  const int32_t kmx = __builtin_amdgcn_readfirstlane(sm.segr[BUF][1]);
  if (kmx < gi.sq_min || kmn > gi.sq_max) return 0;
  return (kmn == kmx && gi.sq_min == gi.sq_max && kmn == gi.sq_min) ? 1 : 2;
}

// The pairs of sub-tile sb whose staged entry lies in another segment than
// sq (this lane's row or key) are excluded.
template <int32_t BUF>
__device__ __forceinline__ void seg_mask(float* s, const TT::Smem& sm, int32_t sq, int sb,
                                         int32_t lane) {
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call, as in mask_tile
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r)
    s[r] = sm.kseg[BUF][TT::key_const(sb, r) + kl] == sq ? s[r] : kNegInf;
}

// Per-pair label matrices and per-piece segment masks (ETC page, §3.4
// "Per-instance attention masks" and "Relative Position Encoding", Step 1 and
// its implementation note), for the tiles that hold a global token: the
// batch row's label matrices (glabel [n_global][N], llabel [N][n_global]) and
// segment ids, the vocabulary size and clip k, the pieces the segment ids
// mask (bits g2g 1, g2l 2, l2g 4, l2l 8), the lane's own global rank (its
// row in the dQ pass, its key in the dK/dV pass; -1 not global) and whether
// row tables exist.
struct LblCtx {
  const uint8_t* glabel;
  const uint8_t* llabel;
  const int32_t* segb;
  int32_t N, n_global, V, k, pieces, rank, tabs, avec;
};

__device__ __forceinline__ LblCtx lbl_ctx(const BwdArgs& a, int32_t bh, int32_t rank) {
  const int32_t b = bh / a.H;
  return {a.glabel ? a.glabel + (size_t)b * a.n_global * a.N : nullptr,
          a.llabel ? a.llabel + (size_t)b * a.N * a.n_global : nullptr,
          a.seg ? a.seg + (size_t)b * a.N : nullptr,
          a.N,  a.n_global,    a.n_labels, a.rel_k, a.seg_pieces, rank, a.rowtab != nullptr,
          a.rel_vec != nullptr};
}

// Pair (row i, key j) with global ranks gi, gj: -2 masked (a segment mask of
// its piece or a masking label), -1 kept without a label (a mixed pair keeping
// its usual label, or no tables), else its label (explicit, or the clipped
// distance of a same-kind pair).
__device__ __forceinline__ int32_t lbl_pair(const LblCtx& L, int32_t i, int32_t gi, int32_t j,
                                            int32_t gj) {
  const bool ig = gi >= 0, jg = gj >= 0;
  if (L.segb) {
    const int32_t piece = ig ? (jg ? 1 : 2) : (jg ? 4 : 8);
    if ((L.pieces & piece) && L.segb[i] != L.segb[j]) return -2;
  }
  int32_t l = kLabelDist;
  if (ig && L.glabel)
    l = L.glabel[(size_t)gi * L.N + j];
  else if (!ig && jg && L.llabel)
    l = L.llabel[(size_t)i * L.n_global + gj];
  if (l != kLabelDist && l >= L.V) return -2;
  if (!L.tabs) return -1;
  if (l == kLabelDist) {
    if (ig != jg) return -1;
    l = min(max(j - i, -L.k), L.k) + L.k;
  }
  return l;
}

// A tile holding a global token, sub-tile sb: each pair's label by lbl_pair
// (row against key), packed four to a word as label + 2 (byte r & 3 of word
// r >> 2). ROWS_IN_LANES: the lane holds the row (dQ pass; the staged entries
// are keys), else the key (dK/dV pass; the staged entries are rows). Returns
// whether any pair of the wave's sub-tile is kept.
template <int32_t BUF, bool ROWS_IN_LANES>
__device__ __forceinline__ bool lbl_labels(uint32_t (&lw)[TT::kNS / 4], const TT::Smem& sm,
                                           const LblCtx& L, int sb, int32_t pos, int32_t kl) {
  bool any = false;
#pragma unroll
  for (int g = 0; g < TT::kNS / 4; ++g) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t kj = TT::key_const(sb, 4 * g + e) + kl;
      const int32_t l = ROWS_IN_LANES
                            ? lbl_pair(L, pos, L.rank, sm.kpos[BUF][kj], sm.kgrank[BUF][kj])
                            : lbl_pair(L, sm.kpos[BUF][kj], sm.kgrank[BUF][kj], pos, L.rank);
      any = any || l != -2;
      x |= (uint32_t)(l + 2) << (8 * e);
    }
    lw[g] = x;
  }
  return __ballot(any) != 0ull;
}
__device__ __forceinline__ int32_t lbl_at(const uint32_t (&lw)[TT::kNS / 4], int r) {
  return (int32_t)((lw[r >> 2] >> (8 * (r & 3))) & 0xffu) - 2;
}

// The labels applied to the scores: masked pairs excluded, labelled ones add
// the table entry (tab(kj, l): the row's table, or null without tables).
template <typename Tab>
__device__ __forceinline__ void lbl_apply(float* s, const uint32_t (&lw)[TT::kNS / 4], int sb,
                                          int32_t kl, bool tabs, Tab tab) {
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t l = lbl_at(lw, r);
    if (l == -2) s[r] = kNegInf;
    else if (l >= 0 && tabs) s[r] += tab(TT::key_const(sb, r) + kl, l);
  }
}

// dQ pass with label vectors, a tile holding a global token: the labelled
// pairs' dS into the row's label sums, one half-wave at a time (the two lanes
// of a row may share a label; lanes of one half hold different rows).
__device__ __forceinline__ void lbl_sums_dq(const float* ds, const uint32_t (&lw)[TT::kNS / 4],
                                            float* crow, int32_t lane) {
  const int32_t hh = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (hh == half) {
#pragma unroll
      for (int r = 0; r < TT::kNS; ++r) {
        const int32_t l = lbl_at(lw, r);
        if (l >= 0) atomicAdd(crow + l, ds[r]);
      }
    }
  }
}

// Which clipped-distance label every pair of a sub-tile takes, from its keys'
// and rows' first and last positions (both non-decreasing): 1 every pair at
// key - row <= -k (label 0), 2 every pair at key - row >= k (label 2k), 0
// mixed. Wave-uniform.
__device__ __forceinline__ int32_t label_side(int32_t kfirst, int32_t klast, int32_t rfirst,
                                              int32_t rlast, int32_t k) {
  if (klast - rfirst <= -k) return 1;
  if (kfirst - rlast >= k) return 2;
  return 0;
}

// Key-side label vectors, dQ pass: the same-kind pairs' dS of sub-tile sb by
// label (clipped distance key - row): the two clipped labels into the lane's
// registers, the others into C[qi][l] in LDS (each such (row, label) pair has
// one key, so the lanes of one add never share an address).
template <int32_t BUF>
__device__ __forceinline__ void vec_label_sums(DqWave& w, const float* ds, const TT::Smem& sm,
                                               const BiasRule& br, int sb, int32_t qi,
                                               int32_t qpos, int32_t lane, bool all_same) {
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call, as in mask_tile
  const int32_t k = br.k, top = 2 * br.k;
  float* C = const_cast<float*>(br.tab) + TT::kTQ * br.row_stride + qi * br.row_stride;
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(sb, r) + kl;
    const bool same =
        all_same || ((sm.kglob[BUF][kj] != 0) == (br.key_global_is_same_kind != 0));
    const int32_t l = min(max(sm.kpos[BUF][kj] - qpos, -k), k) + k;
    const float x = same ? ds[r] : 0.f;
    w.c_lo += l == 0 ? x : 0.f;
    w.c_hi += l == top ? x : 0.f;
    if (same && l > 0 && l < top) atomicAdd(C + l, ds[r]);
  }
}

// Key-side label vectors, dQ workgroup set-up: the rows' tables (row r at
// position pos(r); rows past the tile repeat its last), the label sums
// zeroed and the head's vectors a_l (fp32 [V][D]) into the dynamic LDS; visible
// after the tile loop's first barrier.
template <bool LBL, typename Pos>
__device__ __forceinline__ BiasRule vec_rule_dq(const BwdArgs& a, float* dyn, int32_t bh,
                                                int32_t h, int32_t lane_is_global_kind,
                                                Pos pos) {
  // (without LBL the tables and vectors are always there)
  const bool tabs = !LBL || a.rowtab != nullptr, avec = !LBL || a.rel_vec != nullptr;
  const int32_t V = a.n_labels, tid = threadIdx.x;
  const float* tb = tabs ? a.rowtab + (size_t)bh * a.N * V : nullptr;
  float* rt = dyn;
  float* C = dyn + TT::kTQ * V;
  float* A = dyn + 2 * TT::kTQ * V;
  const int32_t r = tid >> 1, l0 = tid & 1;  // two threads per row
  if (tabs) {
    const float* src = tb + (size_t)pos(r) * V;
    for (int32_t l = l0; l < V; l += 2) {
      rt[r * V + l] = src[l];
      C[r * V + l] = 0.f;
    }
  }
  if (avec) {
    const float* av = a.rel_vec + (size_t)h * V * kD;
    for (int32_t x = tid; x < V * kD; x += TT::kThreads) A[x] = av[x];
  }
  return {tabs ? dyn : nullptr, a.rel_k, lane_is_global_kind, V};
}

// Key-side label vectors, dQ workgroup end: dQ_i^T += sum_l C_il a_l for the
// lane's row (the clipped labels' sums combined over the row's two lanes, in
// lane order).
__device__ __forceinline__ void vec_dq_epilogue(DqWave& w, const BiasRule& br, const float* dyn,
                                                int32_t qi, int32_t lane) {
  const int32_t V = br.row_stride, top = 2 * br.k, hh = lane >> 5;
  const float* C = dyn + TT::kTQ * V + qi * V;
  const float* A = dyn + 2 * TT::kTQ * V;
  const float olo = __shfl_xor(w.c_lo, 32), ohi = __shfl_xor(w.c_hi, 32);
  const float lo = hh == 0 ? w.c_lo + olo : olo + w.c_lo;
  const float hi = hh == 0 ? w.c_hi + ohi : ohi + w.c_hi;
  for (int32_t l = 0; l < V; ++l) {
    const float cl = C[l] + (l == 0 ? lo : 0.f) + (l == top ? hi : 0.f);
    const float* al = A + l * kD + 4 * hh;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(al + 32 * db + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) w.acc[db][4 * j + i] = __builtin_fmaf(cl, x[i], w.acc[db][4 * j + i]);
      }
    }
  }
}

// One staged key tile into dQ^T. The forward's block classes decide which
// sub-tiles run and which need the per-element mask. SEG: segment masks from
// gs (a tile of other segments only is skipped). VEC: key-side label vectors
// (ETC page, §3.4 "Relative Position Encoding": the logit is q_i . (k_j + a_l)
// / sqrt(D) for a same-kind pair of label l), br.tab holding the workgroup's
// rows' tables (row stride V) followed by the label sums C [rows][V]: the
// same-kind pairs' dS add to C[row][l] (the clipped labels 0 and 2k in the
// lane's registers), for dQ_i's term sum_l C_il a_l.
template <int32_t BUF, bool BIAS, bool SEG = false, bool VEC = false, bool LBL = false>
__device__ __forceinline__ void dq_tile(const TT::Smem& sm, DqWave& w, int32_t lane,
                                        const MaskRule& mr, const KeyTile& kt, int32_t qi,
                                        int32_t qpos, bool dead, float c, const BiasRule& br,
                                        const GlobInfo& gs, const LblCtx* lc = nullptr) {
  // LBL: a tile whose rows or keys hold a global token decides each pair by
  // lbl_pair; the others (l2l pairs only) take the paths below, with segment
  // masks only if the l2l piece has them
  bool per_pair = false, seg_on = SEG;
  if constexpr (LBL) {
    const int32_t gc = kt.gmode == kGlobNone ? 0 : __builtin_amdgcn_readfirstlane(sm.gcls[BUF]);
    per_pair = lc->rank >= 0 || (gc & 1) != 0;
    seg_on = !per_pair && (lc->pieces & 8) != 0;
  }
  bool seg_check = false;
  if constexpr (SEG) {
    if (seg_on) {
      const int32_t st = seg_tile<BUF>(sm, gs, kt);
      if (st == 0) return;
      seg_check = st == 2;
    }
  }
  const int32_t r0 = (mr.use_qpos ? __builtin_amdgcn_readlane(qpos, 0)
                                  : __builtin_amdgcn_readlane(qi, 0)) + mr.ref_off;
  const int32_t r1 = (mr.use_qpos ? __builtin_amdgcn_readlane(qpos, TT::kRowsPerBlock - 1)
                                  : __builtin_amdgcn_readlane(qi, TT::kRowsPerBlock - 1)) + mr.ref_off;
  TileBias tb = {false, false};
  int32_t q0 = 0, q1 = 0;  // the wave's first and last row positions
  if constexpr (BIAS || VEC) {
    if (!per_pair) tb = tile_bias<BUF>(sm, br, kt);
    q0 = __builtin_amdgcn_readlane(qpos, 0);
    q1 = __builtin_amdgcn_readlane(qpos, TT::kRowsPerBlock - 1);
  }
#pragma unroll
  for (int sb = 0; sb < TT::kSub; ++sb) {
    const int32_t cls = dead ? kEmpty : classify<bf16>(mr, kt.count, sb, r0, r1);
    if (cls == kEmpty) continue;
    // one clipped label for the whole sub-tile: its table entry joins the
    // exponent's offset (per lane), no per-element lookup
    int32_t side = 0;
    if constexpr (BIAS || VEC) {
      if (tb.on && tb.same)
        side = label_side(__builtin_amdgcn_readfirstlane(sm.kpos[BUF][32 * sb]),
                          __builtin_amdgcn_readfirstlane(sm.kpos[BUF][32 * sb + 31]), q0, q1, br.k);
    }
    uint32_t lw[TT::kNS / 4];
    if constexpr (LBL) {
      // a sub-tile whose pairs are all masked is skipped before its MFMAs
      if (per_pair && !lbl_labels<BUF, true>(lw, sm, *lc, sb, qpos, TT::key_lane(lane))) continue;
    }
    float s[TT::kNS], dp[TT::kNS];
    tile_dots(&sm.k[BUF][0], w.qf, lane, sb, s);
    tile_dots(&sm.v[BUF][0], w.df, lane, sb, dp);
    float off = -w.lse2;
    if constexpr (BIAS || VEC) {
      if (tb.on && side == 0) add_bias<bf16>(s, sm, BUF, br, sb, qi, qpos, lane, tb.same);
      if (side != 0)
        off = __builtin_fmaf(br.tab[qi * br.row_stride + (side == 1 ? 0 : 2 * br.k)], c, off);
    }
    if constexpr (LBL) {
      if (per_pair) {
        const float* trow = br.tab ? br.tab + qi * br.row_stride : nullptr;
        lbl_apply(s, lw, sb, TT::key_lane(lane), trow != nullptr,
                  [&](int32_t, int32_t l) { return trow[l]; });
      }
    }
    if (cls == kPartial) mask_tile<bf16>(s, sm, BUF, mr, sb, kt.count, qi, qpos, lane);
    if (SEG && seg_check) seg_mask<BUF>(s, sm, gs.sq, sb, lane);
    TT::PTile G;
    float ds[TT::kNS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 8 * t + 2 * i;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, off));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + 1], c, off));
        ds[e] = p0 * (dp[e] - w.di);
        ds[e + 1] = p1 * (dp[e + 1] - w.di);
        G.p[t][i] = pack_bf16x2(ds[e], ds[e + 1]);
      }
    }
    if constexpr (VEC) {
      const bool sums = !LBL || lc->avec;
      if (LBL && per_pair) {
        if (sums) lbl_sums_dq(ds, lw, const_cast<float*>(br.tab) + TT::kTQ * br.row_stride +
                                          qi * br.row_stride, lane);
      } else if (tb.on && side == 0) {
        if (sums) vec_label_sums<BUF>(w, ds, sm, br, sb, qi, qpos, lane, tb.same);
      } else if (side != 0) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < TT::kNS; ++e) t += ds[e];
        if (side == 1)
          w.c_lo += t;
        else
          w.c_hi += t;
      }
    }
    acc_transposed<BUF>(&sm.k[0][0], w.acc, lane, sb, G);
  }
}

// The forward's tile loop (fetch next, compute current, stage, barrier) with
// `proc(buf_tag, kt, mr)` as the per-tile work; no bias or label state. SEG:
// the staged keys' segment ids and their range, when gi has them.
template <bool GATHER, bool SEG = false, bool LBL = false, typename Desc, typename Proc>
__device__ __forceinline__ void stream_tiles(TT::Smem& sm, const bf16* kb, const bf16* vb,
                                             int32_t n_tiles, Desc desc, const GlobInfo& gi,
                                             Proc proc) {
  const int32_t tid = threadIdx.x;
  if (n_tiles <= 0) return;
  LabelRule nolab = {};
  nolab.want_rank = LBL ? 1 : 0;  // LBL: the keys' global ranks
  TT::Prefetch pf;
  KeyTile kt;
  MaskRule mr;
  desc(0, kt, mr);
  const FetchPlan fp = TT::plan(kt.stride, tid);
  TT::template fetch<GATHER>(pf, sm, 0, kb, vb, kt, fp, tid);
  TT::stage(sm, 0, pf, tid);
  stage_meta<bf16, SEG, LBL>(sm, 0, pf.meta, gi, nolab, kt.gmode, tid);
  __syncthreads();
  auto step = [&](auto buf_tag, int32_t n) {
    constexpr int32_t buf = decltype(buf_tag)::value;
    KeyTile kt_next;
    MaskRule mr_next;
    const bool more = n + 1 < n_tiles;
    if (more) {
      desc(n + 1, kt_next, mr_next);
      TT::template fetch<GATHER>(pf, sm, buf ^ 1, kb, vb, kt_next, fp, tid);
    }
    proc(buf_tag, kt, mr);
    if (more) {
      TT::stage(sm, buf ^ 1, pf, tid);
      stage_meta<bf16, SEG, LBL>(sm, buf ^ 1, pf.meta, gi, nolab, kt_next.gmode, tid);
      kt = kt_next;
      mr = mr_next;
    }
    __syncthreads();
  };
  for (int32_t n = 0; n < n_tiles; n += 2) {
    step(BufTag<0>{}, n);
    if (n + 1 < n_tiles) step(BufTag<1>{}, n + 1);
  }
}

// Number of residue-class query tiles (of tq rows) of a head of dilation d
// (the forward's enumeration).
__device__ __forceinline__ int32_t tiles_of_class(int32_t N, int32_t d, int32_t c, int32_t tq) {
  return ((N - c + d - 1) / d + tq - 1) / tq;
}

// Whether this lane's row (or key) of a tile is a global position.
__device__ __forceinline__ bool qi_is_global(const BwdArgs& a, int32_t qi, int32_t qcount,
                                             int32_t pos, int32_t g_first, int32_t g_last,
                                             int32_t lo, int32_t hi) {
  return qi < qcount && g_first <= hi && g_last >= lo && sorted_contains(a.gidx, a.n_global, pos);
}

// dQ of the non-global rows of one query tile (the forward's band workgroup:
// window tiles, then the global keys outside the window).
template <bool BIAS, bool SEG, bool VEC, bool LBL>
__device__ __forceinline__ void dq_band_workgroup(const BwdArgs& a, TT::Smem& sm, float* dyn,
                                                  int32_t bw) {
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
    const int32_t tc = tiles_of_class(N, d, c, kTQ);
    if (tile < tc) break;
    tile -= tc;
  }
  if (c >= d || c >= N) return;  // padding workgroup of a less-dilated head
  const int32_t t0 = tile * kTQ;
  const int32_t qcount = min(kTQ, n_c - t0);
  const int32_t qbase = c + d * t0;
  const int32_t i_lo = qbase, i_hi = qbase + d * (qcount - 1);
  const int32_t ng = a.n_global;
  const int32_t g_first = ng > 0 ? a.gidx[0] : 0;
  const int32_t g_last = ng > 0 ? a.gidx[ng - 1] : -1;
  // a tile made only of global rows has nothing here (the global rows' dQ
  // comes from the global-row pass)
  if (d == 1 && g_last - g_first == ng - 1 && g_first <= i_lo && g_last >= i_hi) return;

  const bf16* qb = static_cast<const bf16*>(a.q) + bh * head_elems;
  const bf16* kb = static_cast<const bf16*>(a.k) + bh * head_elems;
  const bf16* vb = static_cast<const bf16*>(a.v) + bh * head_elems;
  const bf16* dob = static_cast<const bf16*>(a.dout) + bh * head_elems;
  const int32_t qi = TT::qrow(wave, lane, 0);
  const int32_t qpos = qbase + d * min(qi, qcount - 1);
  const bool dead = TT::kQW * wave >= qcount;
  DqWave w;
  load_frag(w.qf, qb, qpos, lane);
  load_frag(w.df, dob, qpos, lane);
  const float lse = a.lse[(size_t)bh * N + qpos];
  w.lse2 = lse == kNegInf ? -kNegInf : lse * kLog2e;
  w.di = a.delta[(size_t)bh * N + qpos];  // D_i from the launch before
  w.acc[0] = f32x16{};
  w.acc[1] = f32x16{};
  w.c_lo = 0.f;
  w.c_hi = 0.f;

  const int32_t R = a.radius;
  const int32_t lo = max(0, t0 - R);
  const int32_t hi = a.causal ? (t0 + qcount - 1) : min(n_c - 1, t0 + qcount - 1 + R);
  const int32_t n_band = (hi - lo + 1 + kTK - 1) / kTK;
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  seg_info<SEG>(gi, a, bh, qpos);
  BiasRule br = {nullptr, 0, 0, 0};
  if constexpr (BIAS || VEC) {
    // the window keys' global flags decide which pairs are same-kind
    if constexpr (VEC)
      br = vec_rule_dq<LBL>(a, dyn, bh, h, 0,
                       [&](int32_t r) { return qbase + d * min(r, qcount - 1); });
    else
      br = bias_rule(a, sm, h, false, 0);
    if (ng > 0) {
      if (hi - lo + 1 <= 32 * kGMaskWords) {
        build_gmask<bf16>(sm, a.gidx, ng, c + d * lo, d, hi - lo + 1, tid);
        gi.mode = kGlobBitmap;
      } else {
        gi.mode = kGlobSearch;
      }
    }
  }
  const int32_t gkeys = (BIAS || VEC) ? kGlobAll : kGlobNone;  // mode of the global-key tiles
  const LblCtx lc = lbl_ctx(a, bh, -1);  // (LBL) the rows here count as non-global
  auto proc = [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
    constexpr int32_t buf = decltype(buf_tag)::value;
    dq_tile<buf, BIAS, SEG, VEC, LBL>(sm, w, lane, mr, kt, qi, qpos, dead, a.scale_log2, br, gi,
                                      &lc);
  };
  auto band_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = lo + n * kTK;
    const int32_t kcount = min(kTK, hi - u0 + 1);
    kt = {nullptr, c + d * u0, d, kcount, u0 - lo, gi.mode};
    const int32_t dmin = u0 - t0 - (qcount - 1);
    const int32_t dmax = u0 + kcount - 1 - t0;
    const int32_t hib = a.causal ? 0 : R;
    const bool full = kcount == kTK && dmin >= -R && dmax <= hib;
    mr = {kRange, full ? 0 : 1, 0, t0 - u0, -R, hib, 0, 0, 1};
  };
  const bool g_run = ng > 0 && d == 1 && g_last - g_first == ng - 1;
  if (g_run) {
    const int32_t n_gt = (ng + kTK - 1) / kTK;
    auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
      if (n >= n_gt) {
        band_desc(n - n_gt, kt, mr);
        return;
      }
      const int32_t gt = n;
      const int32_t cnt = min(kTK, ng - gt * kTK);
      const int32_t gl = g_first + gt * kTK, gh = gl + cnt - 1;
      const bool all_in_band =
          a.causal ? (gl >= i_hi - R && gh <= i_lo) : (gl >= i_hi - R && gh <= i_lo + R);
      const bool none_causal = a.causal && gl > i_hi;
      const bool keep = !all_in_band && !none_causal;
      kt = {nullptr, gl, 1, keep ? cnt : 0, 0, gkeys};
      const bool all_out = cnt == kTK && (gh < i_lo - R || (!a.causal && gl > i_hi + R)) &&
                           (!a.causal || gh <= i_lo);
      mr = {kOutside, all_out ? 0 : 1, 1, -gl, -R, a.causal ? kFar : R, 0, 0, 1};
    };
    stream_tiles<false, SEG, LBL>(sm, kb, vb, n_band + n_gt, desc, gi, proc);
  } else {
    stream_tiles<false, SEG, LBL>(sm, kb, vb, n_band, band_desc, gi, proc);
  }
  if (ng > 0 && !g_run) {
    const int32_t n_gt = (ng + kTK - 1) / kTK;
    uint64_t keep = ~0ull;
    if (n_gt <= 64) {
      keep = 0;
      for (int32_t gt = 0; gt < n_gt; ++gt) {
        const int32_t cnt = min(kTK, ng - gt * kTK);
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
      const int32_t kcount = min(kTK, ng - gt * kTK);
      kt = {a.gidx + gt * kTK, 0, 1, kcount, 0, gkeys};
      const int32_t gl = a.gidx[gt * kTK], gh = a.gidx[gt * kTK + kcount - 1];
      const bool outside = (gh < i_lo - d * R) || (gl > i_hi + d * R);
      const bool causal_ok = !a.causal || gh <= i_lo;
      const bool full = kcount == kTK && outside && causal_ok;
      mr = {kGlobCol, full ? 0 : 1, 0, 0, 0, 0, a.causal, R, d};
    };
    stream_tiles<true, SEG, LBL>(sm, kb, vb, n_glob, glob_desc, gi, proc);
  }

  if constexpr (VEC) {
    if (!LBL || a.rel_vec) vec_dq_epilogue(w, br, dyn, qi, lane);
  }
  // non-global rows: dQ (and, with separate projections, a zero dQ_g row)
  if (qi < qcount) {
    const bool is_g = g_first <= i_hi && g_last >= i_lo && sorted_contains(a.gidx, ng, qpos);
    if (!is_g) {
      const int32_t hh = lane >> 5;
      float* dst = a.dq + ((size_t)bh * N + qpos) * kD;
      float* dsg = a.sep ? a.dqg + ((size_t)bh * N + qpos) * kD : nullptr;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = w.acc[db][4 * j + i] * a.scale;
          *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh) = x;
          if (dsg) *reinterpret_cast<f32x4*>(dsg + 32 * db + 8 * j + 4 * hh) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV of the non-global keys
// ---------------------------------------------------------------------------

// One wave's keys: K and V fragments, dK^T and dV^T.
struct DkvWave {
  bf16x8 kf[4];
  bf16x8 vf[4];
  f32x16 dk[2];
  f32x16 dv[2];
};

// The backward's LDS: the engine's tile buffers and, for the dK/dV pass, each
// staged row tile's offsets, negated: -lse times lse_mul (1 / scale gives
// score units, the raw q.k at which P = 1; -inf for a row without keys) and
// -D_i.
struct BwdSmem : TT::Smem {
  alignas(16) float rlse[2][kTK];
  alignas(16) float rdi[2][kTK];
};
__device__ __forceinline__ float* row_lse(BwdSmem& sm, int32_t buf) { return &sm.rlse[buf][0]; }
__device__ __forceinline__ float* row_di(BwdSmem& sm, int32_t buf) { return &sm.rdi[buf][0]; }
__device__ __forceinline__ const float* row_lse(const BwdSmem& sm, int32_t buf) {
  return &sm.rlse[buf][0];
}
__device__ __forceinline__ const float* row_di(const BwdSmem& sm, int32_t buf) {
  return &sm.rdi[buf][0];
}

// Key-side label vectors, dK/dV pass: each same-kind pair of sub-tile sb adds
// its row's table entry for label clip(key - row) + k (the lane holds the key,
// the elements the staged rows).
template <int32_t BUF>
__device__ __forceinline__ void vec_add_rows(float* s, const BwdSmem& sm, const BiasRule& br,
                                             int sb, int32_t kpos, int32_t kl, bool all_same) {
  const int32_t V = br.row_stride, k = br.k;
  const float* vt = br.tab + BUF * kTK * V;
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(sb, r) + kl;
    const bool same =
        all_same || ((sm.kglob[BUF][kj] != 0) == (br.key_global_is_same_kind != 0));
    const int32_t l = min(max(kpos - sm.kpos[BUF][kj], -k), k) + k;
    const float b = vt[kj * V + l];  // always read: keeps the loop branch-free
    s[r] += same ? b : 0.f;
  }
}

// One streamed tile of query rows into dK^T, dV^T. EXCL_G: rows that are
// global are excluded (they are taken in the global-row sweep); ROWS_AFTER:
// (gathered global rows, causal) only rows at or after the lane's key.
// The score and dP MFMAs start from the rows' offsets (-lse / scale and -D_i,
// staged with the lse in score units), so those per-element values take no
// registers of their own (this lets the band kernel run 3 waves per SIMD) and
// no VALU work after the MFMAs.
// PRIO: the exponential stretch at raised wave issue priority (as in the
// forward's softmax); it pays in the LongNet sweeps (the (2048, 1) pattern's
// dK/dV launch runs about 11% faster) and costs about 1% in the band ones.
// BIAS: the scalar bias table (br: the flipped table, key_global_is_same_kind
// = the lane's key is global). SEG: segment masks from gs (the lane's key's
// segment against the staged rows'). VEC: key-side label vectors, br.tab the
// staged rows' tables (kTK rows of br.row_stride labels per buffer).
template <int32_t BUF, bool EXCL_G, bool ROWS_AFTER, bool PRIO = false, bool BIAS = false,
          bool SEG = false, bool VEC = false, bool LBL = false>
__device__ __forceinline__ void dkv_tile(const BwdSmem& sm, DkvWave& w, int32_t lane,
                                         const MaskRule& mr, const KeyTile& kt, int32_t ki,
                                         int32_t kpos, bool dead, float c, bool causal,
                                         const BiasRule& br = {nullptr, 0, 0, 0},
                                         const GlobInfo& gs = {}, const LblCtx* lc = nullptr) {
  // LBL: as in dq_tile (rows excluded as global do not count: they are masked)
  bool per_pair = false, seg_on = SEG;
  if constexpr (LBL) {
    const int32_t gc = kt.gmode == kGlobNone ? 0 : __builtin_amdgcn_readfirstlane(sm.gcls[BUF]);
    per_pair = lc->rank >= 0 || (!EXCL_G && (gc & 1) != 0);
    seg_on = !per_pair && (lc->pieces & 8) != 0;
  }
  bool seg_check = false;
  if constexpr (SEG) {
    if (seg_on) {
      const int32_t st = seg_tile<BUF>(sm, gs, kt);
      if (st == 0) return;
      seg_check = st == 2;
    }
  }
  const int32_t r0 = (mr.use_qpos ? __builtin_amdgcn_readlane(kpos, 0)
                                  : __builtin_amdgcn_readlane(ki, 0)) + mr.ref_off;
  const int32_t r1 = (mr.use_qpos ? __builtin_amdgcn_readlane(kpos, TT::kRowsPerBlock - 1)
                                  : __builtin_amdgcn_readlane(ki, TT::kRowsPerBlock - 1)) + mr.ref_off;
  bool any_g = false;
  if constexpr (EXCL_G)
    any_g = kt.gmode != kGlobNone && (__builtin_amdgcn_readfirstlane(sm.gcls[BUF]) & 1) != 0;
  TileBias tb = {false, false};
  int32_t kq0 = 0, kq1 = 0;  // the wave's first and last key positions
  if constexpr (BIAS || VEC) {
    if (!per_pair) tb = tile_bias<BUF>(sm, br, kt);
    kq0 = __builtin_amdgcn_readlane(kpos, 0);
    kq1 = __builtin_amdgcn_readlane(kpos, TT::kRowsPerBlock - 1);
  }
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call, as in mask_tile
#pragma unroll
  for (int sb = 0; sb < TT::kSub; ++sb) {
    const int32_t cls = dead ? kEmpty : classify<bf16>(mr, kt.count, sb, r0, r1);
    if (cls == kEmpty) continue;
    uint32_t lw[TT::kNS / 4];
    if constexpr (LBL) {
      // a sub-tile whose pairs are all masked is skipped before its MFMAs
      if (per_pair && !lbl_labels<BUF, false>(lw, sm, *lc, sb, kpos, kl)) continue;
    }
    // one clipped label for the whole sub-tile: VEC starts the score MFMAs
    // from the offsets with the rows' entries added; the scalar table's entry
    // joins the exponent
    int32_t side = 0;
    if constexpr (BIAS || VEC) {
      if (tb.on && tb.same)
        side = label_side(kq0, kq1, __builtin_amdgcn_readfirstlane(sm.kpos[BUF][32 * sb]),
                          __builtin_amdgcn_readfirstlane(sm.kpos[BUF][32 * sb + 31]), br.k);
    }
    const float* lsrc = row_lse(sm, BUF);
    if constexpr (VEC) {
      if (side != 0)
        lsrc = br.tab + 2 * kTK * br.row_stride + (side == 1 ? 0 : 2 * kTK) + BUF * kTK;
    }
    float coff = 0.f;
    if constexpr (BIAS) {
      if (side != 0) coff = br.tab[side == 1 ? 2 * br.k : 0] * c;  // the flipped table
    }
    // the lane's 16 rows are 4 runs of 4 (key_const): one 16-byte read per run
    const f32x4* ls = reinterpret_cast<const f32x4*>(lsrc + kl);
    const f32x4* dd = reinterpret_cast<const f32x4*>(row_di(sm, BUF) + kl);
    float s[TT::kNS], dp[TT::kNS];
    {  // s = q.k - lse / scale, dp = dO.v - D_i
      f32x16 s0, d0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 x = ls[(TT::key_const(sb, 4 * j)) / 4];
        const f32x4 y = dd[(TT::key_const(sb, 4 * j)) / 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s0[4 * j + i] = x[i];
          d0[4 * j + i] = y[i];
        }
      }
      tile_dots(&sm.k[BUF][0], w.kf, lane, sb, s, s0);
      tile_dots(&sm.v[BUF][0], w.vf, lane, sb, dp, d0);
    }
    if constexpr (BIAS) {
      if (tb.on && side == 0) add_bias<bf16>(s, sm, BUF, br, sb, ki, kpos, lane, tb.same);
    }
    if constexpr (VEC) {
      if (tb.on && side == 0) vec_add_rows<BUF>(s, sm, br, sb, kpos, kl, tb.same);
    }
    if constexpr (LBL) {
      if (per_pair) {
        const float* vt = br.tab ? br.tab + BUF * kTK * br.row_stride : nullptr;
        const int32_t V = br.row_stride;
        lbl_apply(s, lw, sb, kl, vt != nullptr,
                  [&](int32_t kj, int32_t l) { return vt[kj * V + l]; });
      }
    }
    if (cls == kPartial) mask_tile<bf16>(s, sm, BUF, mr, sb, kt.count, ki, kpos, lane);
    if (SEG && seg_check) seg_mask<BUF>(s, sm, gs.sq, sb, lane);
    if (EXCL_G && any_g) {
#pragma unroll
      for (int r = 0; r < TT::kNS; ++r)
        s[r] = sm.kglob[BUF][TT::key_const(sb, r) + kl] != 0 ? kNegInf : s[r];
    }
    if constexpr (ROWS_AFTER) {
      if (causal) {
#pragma unroll
        for (int r = 0; r < TT::kNS; ++r)
          s[r] = sm.kpos[BUF][TT::key_const(sb, r) + kl] >= kpos ? s[r] : kNegInf;
      }
    }
    TT::PTile P, G;
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 8 * t + 2 * i;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, coff));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + 1], c, coff));
        G.p[t][i] = pack_bf16x2(p0 * dp[e], p1 * dp[e + 1]);
        P.p[t][i] = pack_bf16x2(p0, p1);
      }
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    acc_transposed<BUF>(&sm.v[0][0], w.dv, lane, sb, P);
    acc_transposed<BUF>(&sm.k[0][0], w.dk, lane, sb, G);
    // one sub-tile's values live at a time (the two interleaved spill)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// stream_tiles for query rows: as stream_tiles, and each staged tile's rows'
// lse (times lse_mul) and D_i, read with the tile's loads, written to LDS
// with its staging (SEG: the rows' segment ids are staged as the keys' are).
// VEC: also the rows' label tables (tab: the head's [N][V] tables) into
// vt + buf * kTK * V, and after the two buffers' tables the rows' offsets with
// the clipped labels' entries added, -lse * lse_mul + T[row][0] ([2][kTK])
// then + T[row][vtop] ([2][kTK]; vtop = 2k).
template <bool GATHER, bool SEG = false, bool VEC = false, bool LBL = false, typename Desc,
          typename Proc>
__device__ __forceinline__ void stream_rows(BwdSmem& sm, const bf16* qb, const bf16* dob,
                                            const float* lse, const float* delta, float lse_mul,
                                            int32_t n_tiles, Desc desc, const GlobInfo& gi,
                                            Proc proc, const float* tab = nullptr,
                                            float* vt = nullptr, int32_t V = 0,
                                            int32_t vtop = 0) {
  const int32_t tid = threadIdx.x;
  if (n_tiles <= 0) return;
  LabelRule nolab = {};
  nolab.want_rank = LBL ? 1 : 0;  // LBL: the rows' global ranks
  TT::Prefetch pf;
  KeyTile kt;
  MaskRule mr;
  float pl = 0.f, pd = 0.f, plo = 0.f, phi = 0.f;
  // VEC: four threads per row, labels tid % 4 + 4u
  constexpr int32_t kVecPer = VEC ? kMaxLabels / 4 : 1;
  float pv[kVecPer];
  auto row_vals = [&](const KeyTile& t) {
    if (tid < kTK && t.count > 0) {
      const int32_t p = key_pos<GATHER>(t, min(tid, t.count - 1));
      const float l = lse[p];
      pl = l == kNegInf ? kNegInf : -(l * lse_mul);
      pd = -delta[p];
      if constexpr (VEC) {
        if (!LBL || tab) {
          plo = pl + tab[(size_t)p * V];
          phi = pl + tab[(size_t)p * V + vtop];
        }
      }
    }
    if constexpr (VEC) {
      if (t.count > 0 && (!LBL || tab)) {
        const float* src = tab + (size_t)key_pos<GATHER>(t, min(tid >> 2, t.count - 1)) * V;
#pragma unroll
        for (int u = 0; u < kVecPer; ++u) {
          const int32_t l = (tid & 3) + 4 * u;
          if (l < V) pv[u] = src[l];
        }
      }
    }
  };
  auto put_rows = [&](int32_t buf) {
    if (tid < kTK) {
      row_lse(sm, buf)[tid] = pl;
      row_di(sm, buf)[tid] = pd;
    }
    if constexpr (VEC) {
      if (LBL && !tab) return;
      if (tid < kTK) {
        vt[2 * kTK * V + buf * kTK + tid] = plo;
        vt[2 * kTK * V + 2 * kTK + buf * kTK + tid] = phi;
      }
      float* dst = vt + buf * kTK * V + (tid >> 2) * V;
#pragma unroll
      for (int u = 0; u < kVecPer; ++u) {
        const int32_t l = (tid & 3) + 4 * u;
        if (l < V) dst[l] = pv[u];
      }
    }
  };
  desc(0, kt, mr);
  const FetchPlan fp = TT::plan(kt.stride, tid);
  TT::template fetch<GATHER>(pf, sm, 0, qb, dob, kt, fp, tid);
  row_vals(kt);
  TT::stage(sm, 0, pf, tid);
  stage_meta<bf16, SEG, LBL>(sm, 0, pf.meta, gi, nolab, kt.gmode, tid);
  put_rows(0);
  __syncthreads();
  auto step = [&](auto buf_tag, int32_t n) {
    constexpr int32_t buf = decltype(buf_tag)::value;
    KeyTile kt_next;
    MaskRule mr_next;
    const bool more = n + 1 < n_tiles;
    if (more) {
      desc(n + 1, kt_next, mr_next);
      TT::template fetch<GATHER>(pf, sm, buf ^ 1, qb, dob, kt_next, fp, tid);
      row_vals(kt_next);
    }
    proc(buf_tag, kt, mr);
    if (more) {
      TT::stage(sm, buf ^ 1, pf, tid);
      stage_meta<bf16, SEG, LBL>(sm, buf ^ 1, pf.meta, gi, nolab, kt_next.gmode, tid);
      put_rows(buf ^ 1);
      kt = kt_next;
      mr = mr_next;
    }
    __syncthreads();
  };
  for (int32_t n = 0; n < n_tiles; n += 2) {
    step(BufTag<0>{}, n);
    if (n + 1 < n_tiles) step(BufTag<1>{}, n + 1);
  }
}

// Lane row of dK^T / dV^T (d = 32db + 8j + 4h + i) to an fp32 row.
__device__ __forceinline__ void store_rows_f32(float* dst, const f32x16 (&acc)[2], float sc,
                                               int32_t lane) {
  const int32_t hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = acc[db][4 * j + i] * sc;
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh) = x;
    }
  }
}

// dK, dV of the non-global keys of one key tile (a residue class of the
// head's dilation, like the forward's query tiles).
template <bool BIAS, bool SEG, bool VEC, bool LBL>
__device__ __forceinline__ void dkv_band_workgroup(const BwdArgs& a, BwdSmem& sm, float* dyn,
                                                   int32_t bw) {
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
    const int32_t tc = tiles_of_class(N, d, c, kTQ);
    if (tile < tc) break;
    tile -= tc;
  }
  if (c >= d || c >= N) return;
  const int32_t t0 = tile * kTQ;
  const int32_t kcount = min(kTQ, n_c - t0);
  const int32_t kbase = c + d * t0;
  const int32_t j_lo = kbase, j_hi = kbase + d * (kcount - 1);
  const int32_t ng = a.n_global;
  const int32_t g_first = ng > 0 ? a.gidx[0] : 0;
  const int32_t g_last = ng > 0 ? a.gidx[ng - 1] : -1;
  // a tile of global keys only: the global-key pass has them
  if (d == 1 && g_last - g_first == ng - 1 && g_first <= j_lo && g_last >= j_hi) return;

  const int32_t ki = TT::qrow(wave, lane, 0);
  const int32_t kpos = kbase + d * min(ki, kcount - 1);
  const bool dead = TT::kQW * wave >= kcount;
  DkvWave w;
  load_frag(w.kf, static_cast<const bf16*>(a.k) + bh * head_elems, kpos, lane);
  load_frag(w.vf, static_cast<const bf16*>(a.v) + bh * head_elems, kpos, lane);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    w.dk[x] = f32x16{};
    w.dv[x] = f32x16{};
  }
  const float* lse = a.lse + (size_t)bh * N;
  const float* delta = a.delta + (size_t)bh * N;
  const bf16* dob = static_cast<const bf16*>(a.dout) + bh * head_elems;

  // window rows in strided index space [lo, hi]: rows i with
  // -R <= i - j <= R (causal: 0 <= i - j <= R)
  const int32_t R = a.radius;
  const int32_t lo = a.causal ? t0 : max(0, t0 - R);
  const int32_t hi = min(n_c - 1, t0 + kcount - 1 + R);
  const int32_t n_band = (hi - lo + 1 + kTK - 1) / kTK;
  const int32_t lob = a.causal ? 0 : -R;
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  seg_info<SEG>(gi, a, bh, kpos);
  if (ng > 0) {  // the rows' global flags: global rows come in their own sweep
    if (hi - lo + 1 <= 32 * kGMaskWords) {
      build_gmask<bf16>(sm, a.gidx, ng, c + d * lo, d, hi - lo + 1, tid);
      gi.mode = kGlobBitmap;
    } else {
      gi.mode = kGlobSearch;
    }
  }
  BiasRule br = {nullptr, 0, 0, 0};
  if constexpr (BIAS) br = bias_rule(a, sm, h, true, 0);  // lanes hold keys: flipped table
  const bool tabs = !LBL || a.rowtab != nullptr;  // (without LBL always there)
  if constexpr (VEC) br = {tabs ? dyn : nullptr, a.rel_k, 0, a.n_labels};  // staged tables
  const float* vtab = VEC && tabs ? a.rowtab + (size_t)bh * N * a.n_labels : nullptr;
  const LblCtx lc = lbl_ctx(a, bh, -1);  // (LBL) the keys here count as non-global
  auto band_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = lo + n * kTK;
    const int32_t cnt = min(kTK, hi - u0 + 1);
    kt = {nullptr, c + d * u0, d, cnt, u0 - lo, gi.mode};
    // strided index difference row - key = kr - ki - (t0 - u0)
    const int32_t dmin = u0 - t0 - (kcount - 1);
    const int32_t dmax = u0 + cnt - 1 - t0;
    const bool full = cnt == kTK && dmin >= lob && dmax <= R;
    mr = {kRange, full ? 0 : 1, 0, t0 - u0, lob, R, 0, 0, 1};
  };
  const bf16* qs = static_cast<const bf16*>(a.q) + bh * head_elems;
  stream_rows<false, SEG, VEC, LBL>(sm, qs, dob, lse, delta, 1.f / a.scale, n_band, band_desc,
                                    gi,
                                    [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                                      constexpr int32_t buf = decltype(buf_tag)::value;
                                      dkv_tile<buf, true, false, false, BIAS, SEG, VEC, LBL>(
                                          sm, w, lane, mr, kt, ki, kpos, dead, a.scale_log2,
                                          a.causal, br, gi, &lc);
                                    },
                                    vtab, dyn, a.n_labels, 2 * a.rel_k);
  // the global rows reach every key (causal: rows at or after it)
  const int32_t n_gt = (ng + kTK - 1) / kTK;
  const int32_t grows = (BIAS || VEC) ? kGlobAll : kGlobNone;  // mode of the global-row tiles
  const GlobInfo gall = {grows, a.gidx, ng, gi.segb, gi.sq, gi.sq_min, gi.sq_max};
  auto glob_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t cnt = min(kTK, ng - n * kTK);
    kt = {a.gidx + n * kTK, 0, 1, cnt, 0, grows};
    // every row of the tile, unless it is past the tile's end
    mr = {kRange, cnt == kTK ? 0 : 1, 0, 0, -kFar, kFar, 0, 0, 1};
  };
  auto glob_proc = [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
    constexpr int32_t buf = decltype(buf_tag)::value;
    dkv_tile<buf, false, true, false, BIAS, SEG, VEC, LBL>(sm, w, lane, mr, kt, ki, kpos, dead,
                                                             a.scale_log2, a.causal, br, gall, &lc);
  };
  const bool mine = ki < kcount && !qi_is_global(a, ki, kcount, kpos, g_first, g_last, j_lo, j_hi);
  if (a.sep) {
    // the window's rows are done: their dK, dV; the global rows go through
    // qg_i, kg_j, vg_j into dKg, dVg
    if (mine) {
      store_rows_f32(a.dk + ((size_t)bh * N + kpos) * kD, w.dk, a.scale, lane);
      store_rows_f32(a.dv + ((size_t)bh * N + kpos) * kD, w.dv, 1.f, lane);
    }
    load_frag(w.kf, static_cast<const bf16*>(a.kg) + bh * head_elems, kpos, lane);
    load_frag(w.vf, static_cast<const bf16*>(a.vg) + bh * head_elems, kpos, lane);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      w.dk[x] = f32x16{};
      w.dv[x] = f32x16{};
    }
  }
  if (ng > 0)
    stream_rows<true, SEG, VEC, LBL>(
        sm, static_cast<const bf16*>(a.sep ? a.qg : a.q) + bh * head_elems, dob, lse, delta,
        1.f / a.scale, n_gt, glob_desc, gall, glob_proc, vtab, dyn, a.n_labels, 2 * a.rel_k);
  if (mine) {
    float* const dk = a.sep ? a.dkg : a.dk;
    float* const dv = a.sep ? a.dvg : a.dv;
    store_rows_f32(dk + ((size_t)bh * N + kpos) * kD, w.dk, a.scale, lane);
    store_rows_f32(dv + ((size_t)bh * N + kpos) * kD, w.dv, 1.f, lane);
  }
}

// ---------------------------------------------------------------------------
// The global rows' dQ and the global keys' dK, dV: a global row reaches every
// key and a global key every row, so a workgroup owns a tile of global rows
// (or keys) and streams one of glob_chunks consecutive ranges of the key (or
// row) tiles. With several ranges each writes its unscaled sums to its own
// partial rows and bwd_glob_reduce_kernel adds them in range order.
// ---------------------------------------------------------------------------

// This workgroup's range of n_all tiles: [t0, t0 + count).
__device__ __forceinline__ void chunk_range(int32_t n_all, int32_t chunks, int32_t c,
                                            int32_t& t0, int32_t& count) {
  const int32_t per = (n_all + chunks - 1) / chunks;
  t0 = min(n_all, c * per);
  count = min(n_all, t0 + per) - t0;
}

// Partial-sum row g (global index) of range c for part 0 (dQ), 1 (dK), 2 (dV).
__device__ __forceinline__ float* part_row(const BwdArgs& a, int32_t part, int32_t c, int32_t bh,
                                           int32_t g) {
  const int32_t n_gpad = (a.n_global + TT::kTQ - 1) / TT::kTQ * TT::kTQ;
  const size_t bhs = (size_t)a.B * a.H;
  return a.gpart + ((((size_t)part * a.glob_chunks + c) * bhs + bh) * n_gpad + g) * kD;
}

// Workgroup wg of the B*H*ceil(n_global/128)*glob_chunks global-row ones.
template <bool BIAS, bool SEG, bool VEC, bool LBL>
__device__ __forceinline__ void dq_glob_workgroup(const BwdArgs& a, TT::Smem& sm, float* dyn,
                                                  int32_t wg) {
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n_gq = (a.n_global + kTQ - 1) / kTQ;
  const int32_t chunks = a.glob_chunks, c = wg % chunks;
  const int32_t unit = wg / chunks;
  const int32_t bh = unit / n_gq, gq = unit % n_gq;
  const int32_t N = a.N;
  const size_t head_elems = (size_t)N * kD;
  const int32_t qcount = min(kTQ, a.n_global - gq * kTQ);
  const int32_t* qidx = a.gidx + gq * kTQ;
  const int32_t i_min = qidx[0], i_max = qidx[qcount - 1];
  const int32_t qi = TT::qrow(wave, lane, 0);
  const int32_t qpos = qidx[min(qi, qcount - 1)];
  const bool dead = TT::kQW * wave >= qcount;
  const bool sep = a.sep != 0;
  DqWave w;
  load_frag(w.qf, static_cast<const bf16*>(sep ? a.qg : a.q) + bh * head_elems, qpos, lane);
  load_frag(w.df, static_cast<const bf16*>(a.dout) + bh * head_elems, qpos, lane);
  const float lse = a.lse[(size_t)bh * N + qpos];
  w.lse2 = lse == kNegInf ? -kNegInf : lse * kLog2e;
  w.di = a.delta[(size_t)bh * N + qpos];  // D_i from the launch before
  w.acc[0] = f32x16{};
  w.acc[1] = f32x16{};
  w.c_lo = 0.f;
  w.c_hi = 0.f;
  const int32_t j1 = a.causal ? i_max + 1 : N;
  int32_t t0, n_tiles;
  chunk_range((j1 + kTK - 1) / kTK, chunks, c, t0, n_tiles);
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  seg_info<SEG>(gi, a, bh, qpos);
  BiasRule br = {nullptr, 0, 0, 0};
  if constexpr (BIAS || VEC) {
    // the keys' global flags decide which pairs are same-kind (global keys)
    if constexpr (VEC)
      br = vec_rule_dq<LBL>(a, dyn, bh, bh % a.H, 1,
                       [&](int32_t r) { return qidx[min(r, qcount - 1)]; });
    else
      br = bias_rule(a, sm, bh % a.H, false, 1);
    const int32_t ub = t0 * kTK, ue = min(j1, ub + n_tiles * kTK);
    if (n_tiles > 0) {
      if (ue - ub <= 32 * kGMaskWords) {
        build_gmask<bf16>(sm, a.gidx, a.n_global, ub, 1, ue - ub, tid);
        gi.mode = kGlobBitmap;
      } else {
        gi.mode = kGlobSearch;
      }
    }
  }
  auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = (t0 + n) * kTK;
    const int32_t kcount = min(kTK, j1 - u0);
    kt = {nullptr, u0, 1, kcount, n * kTK, gi.mode};
    // key position u0 + kj <= qpos when causal
    const bool full = kcount == kTK && (!a.causal || u0 + kTK - 1 <= i_min);
    mr = {kRange, full ? 0 : 1, 1, -u0, -kFar, a.causal ? 0 : kFar, 0, 0, 1};
  };
  const LblCtx lc = lbl_ctx(a, bh, gq * kTQ + min(qi, qcount - 1));  // (LBL) the lane's row rank
  stream_tiles<false, SEG, LBL>(
      sm, static_cast<const bf16*>(sep ? a.kg : a.k) + bh * head_elems,
      static_cast<const bf16*>(sep ? a.vg : a.v) + bh * head_elems, n_tiles, desc, gi,
      [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
        constexpr int32_t buf = decltype(buf_tag)::value;
        dq_tile<buf, BIAS, SEG, VEC, LBL>(sm, w, lane, mr, kt, qi, qpos, dead, a.scale_log2, br,
                                          gi, &lc);
      });
  if constexpr (VEC) {
    if (!LBL || a.rel_vec) vec_dq_epilogue(w, br, dyn, qi, lane);
  }
  if (qi < qcount && chunks > 1) {
    store_rows_f32(part_row(a, 0, c, bh, gq * kTQ + qi), w.acc, 1.f, lane);
  } else if (qi < qcount) {
    const size_t ro = ((size_t)bh * N + qpos) * kD;
    store_rows_f32((sep ? a.dqg : a.dq) + ro, w.acc, a.scale, lane);
    if (sep) {  // a global row's shared-projection gradient is 0
      f32x16 z[2] = {f32x16{}, f32x16{}};
      store_rows_f32(a.dq + ro, z, 0.f, lane);
    }
  }
}

// Workgroup wg of the B*H*ceil(n_global/128)*glob_chunks global-key ones.
template <bool BIAS, bool SEG, bool VEC, bool LBL>
__device__ __forceinline__ void dkv_glob_workgroup(const BwdArgs& a, BwdSmem& sm, float* dyn,
                                                   int32_t wg) {
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n_gk = (a.n_global + kTQ - 1) / kTQ;
  const int32_t chunks = a.glob_chunks, c = wg % chunks;
  const int32_t unit = wg / chunks;
  const int32_t bh = unit / n_gk, gk = unit % n_gk;
  const int32_t N = a.N;
  const size_t head_elems = (size_t)N * kD;
  const int32_t kcount = min(kTQ, a.n_global - gk * kTQ);
  const int32_t* kidx = a.gidx + gk * kTQ;
  const int32_t j_min = kidx[0], j_max = kidx[kcount - 1];
  const int32_t ki = TT::qrow(wave, lane, 0);
  const int32_t kpos = kidx[min(ki, kcount - 1)];
  const bool dead = TT::kQW * wave >= kcount;
  const bool sep = a.sep != 0;
  DkvWave w;
  load_frag(w.kf, static_cast<const bf16*>(a.k) + bh * head_elems, kpos, lane);
  load_frag(w.vf, static_cast<const bf16*>(a.v) + bh * head_elems, kpos, lane);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    w.dk[x] = f32x16{};
    w.dv[x] = f32x16{};
  }
  const float* lse = a.lse + (size_t)bh * N;
  const float* delta = a.delta + (size_t)bh * N;
  const bf16* dob = static_cast<const bf16*>(a.dout) + bh * head_elems;
  // this range of the row positions (causal: from the first key on); with
  // separate projections the global rows are left to the second sweep
  const int32_t r0 = a.causal ? j_min : 0;
  int32_t t0, n_tiles;
  chunk_range((N - r0 + kTK - 1) / kTK, chunks, c, t0, n_tiles);
  const int32_t ub = r0 + t0 * kTK, ue = min(N, ub + n_tiles * kTK);
  GlobInfo gi = {kGlobNone, a.gidx, a.n_global, nullptr, 0, 0, 0};
  seg_info<SEG>(gi, a, bh, kpos);
  BiasRule br = {nullptr, 0, 0, 0};
  if constexpr (BIAS) br = bias_rule(a, sm, bh % a.H, true, 1);  // lanes hold global keys
  const bool tabs = !LBL || a.rowtab != nullptr;  // (without LBL always there)
  if constexpr (VEC) br = {tabs ? dyn : nullptr, a.rel_k, 1, a.n_labels};  // staged tables
  const float* vtab = VEC && tabs ? a.rowtab + (size_t)bh * N * a.n_labels : nullptr;
  const LblCtx lc = lbl_ctx(a, bh, gk * kTQ + min(ki, kcount - 1));  // (LBL) the lane's key rank
  // the rows' global flags: excluded with separate projections; with a bias
  // table or label vectors, the same-kind pairs
  if ((sep || BIAS || VEC) && n_tiles > 0) {
    if (ue - ub <= 32 * kGMaskWords) {
      build_gmask<bf16>(sm, a.gidx, a.n_global, ub, 1, ue - ub, tid);
      gi.mode = kGlobBitmap;
    } else {
      gi.mode = kGlobSearch;
    }
  }
  auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = ub + n * kTK;
    const int32_t cnt = min(kTK, N - u0);
    kt = {nullptr, u0, 1, cnt, u0 - ub, gi.mode};
    // row position u0 + kr >= kpos when causal
    const bool full = cnt == kTK && (!a.causal || u0 >= j_max);
    mr = {kRange, full ? 0 : 1, 1, -u0, a.causal ? 0 : -kFar, kFar, 0, 0, 1};
  };
  const bf16* qs = static_cast<const bf16*>(a.q) + bh * head_elems;
  if (sep)
    stream_rows<false, SEG, VEC, LBL>(sm, qs, dob, lse, delta, 1.f / a.scale, n_tiles, desc, gi,
                                      [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                                        constexpr int32_t buf = decltype(buf_tag)::value;
                                        dkv_tile<buf, true, false, false, BIAS, SEG, VEC, LBL>(
                                            sm, w, lane, mr, kt, ki, kpos, dead, a.scale_log2,
                                            a.causal, br, gi, &lc);
                                      },
                                      vtab, dyn, a.n_labels, 2 * a.rel_k);
  else
    stream_rows<false, SEG, VEC, LBL>(sm, qs, dob, lse, delta, 1.f / a.scale, n_tiles, desc, gi,
                                      [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                                        constexpr int32_t buf = decltype(buf_tag)::value;
                                        dkv_tile<buf, false, false, false, BIAS, SEG, VEC, LBL>(
                                            sm, w, lane, mr, kt, ki, kpos, dead, a.scale_log2,
                                            a.causal, br, gi, &lc);
                                      },
                                      vtab, dyn, a.n_labels, 2 * a.rel_k);
  const size_t ro = ((size_t)bh * N + kpos) * kD;
  if (ki < kcount && chunks > 1) {
    store_rows_f32(part_row(a, 1, c, bh, gk * kTQ + ki), w.dk, 1.f, lane);
    store_rows_f32(part_row(a, 2, c, bh, gk * kTQ + ki), w.dv, 1.f, lane);
  } else if (ki < kcount) {
    store_rows_f32(a.dk + ro, w.dk, a.scale, lane);
    store_rows_f32(a.dv + ro, w.dv, 1.f, lane);
  }
  // separate projections: the last range also sweeps the global rows
  if (!sep || c != chunks - 1) return;
  // separate projections: the global rows through qg_i, kg_j, vg_j
  load_frag(w.kf, static_cast<const bf16*>(a.kg) + bh * head_elems, kpos, lane);
  load_frag(w.vf, static_cast<const bf16*>(a.vg) + bh * head_elems, kpos, lane);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    w.dk[x] = f32x16{};
    w.dv[x] = f32x16{};
  }
  const int32_t n_gt = (a.n_global + kTK - 1) / kTK;
  const int32_t grows = (BIAS || VEC) ? kGlobAll : kGlobNone;  // mode of the global-row tiles
  auto glob_desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t cnt = min(kTK, a.n_global - n * kTK);
    kt = {a.gidx + n * kTK, 0, 1, cnt, 0, grows};
    mr = {kRange, cnt == kTK ? 0 : 1, 0, 0, -kFar, kFar, 0, 0, 1};
  };
  const GlobInfo gall = {grows, a.gidx, a.n_global, gi.segb, gi.sq, gi.sq_min, gi.sq_max};
  stream_rows<true, SEG, VEC, LBL>(sm, static_cast<const bf16*>(a.qg) + bh * head_elems, dob,
                                   lse, delta, 1.f / a.scale, n_gt, glob_desc, gall,
                                   [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                                     constexpr int32_t buf = decltype(buf_tag)::value;
                                     dkv_tile<buf, false, true, false, BIAS, SEG, VEC, LBL>(
                                         sm, w, lane, mr, kt, ki, kpos, dead, a.scale_log2,
                                         a.causal, br, gall, &lc);
                                   },
                                   vtab, dyn, a.n_labels, 2 * a.rel_k);
  if (ki < kcount) {
    store_rows_f32(a.dkg + ro, w.dk, a.scale, lane);
    store_rows_f32(a.dvg + ro, w.dv, 1.f, lane);
  }
}

// ---------------------------------------------------------------------------
// LongNet mixture (bf16). The mixture is one softmax over the multiset of the
// patterns' keys (LongNet page, §3.4 "Mixture of Dilated Attentions"), so with
// the mixture's lse each pattern contributes its own pairs' terms and a pair
// kept by several patterns adds once per pattern. A pattern's dQ workgroups
// (or dK/dV workgroups) add its terms into dQ (or dK, dV), every kept row (or
// key) in one workgroup, and each gradient takes the patterns one launch after
// another, so the sums are deterministic. A pattern of dilation 1 keeps every
// row and key: when there is one it goes first and stores its terms;
// otherwise zeros are written first (rows no pattern keeps keep them).
// ---------------------------------------------------------------------------

// The pattern's segment geometry for head h (as the forward's dilated_tile):
// kept rows base + r * t, t in [0, n_rows).
struct DilGeom {
  int32_t base, r, n_rows;
};
__device__ __forceinline__ DilGeom dil_geom(const BwdArgs& a, int32_t k, int32_t seg, int32_t h) {
  const int32_t w = a.pw[k], r = a.pr[k];
  const int32_t sigma = seg * w;
  const int32_t L = min(w, a.N - sigma);
  const int32_t s = h % r;
  return {sigma + s, r, L > s ? (L - s + r - 1) / r : 0};
}

// Workgroup wg of a pattern launch: query (or key) tiles of kept rows, the
// heaviest (latest) tile index first.
__device__ __forceinline__ void dil_decode(const BwdArgs& a, int32_t nseg, int32_t qtiles,
                                           int64_t wg, int32_t& qt, int32_t& seg, int32_t& bh) {
  const int64_t per = (int64_t)a.B * a.H * nseg;
  qt = qtiles - 1 - (int32_t)(wg / per);
  const int64_t rest = wg % per;
  seg = (int32_t)(rest % nseg);
  bh = (int32_t)(rest / nseg);
}

// this lane's row += acc * sc (an fp32 row owned by this workgroup)
__device__ __forceinline__ void add_rows_f32(float* dst, const f32x16 (&acc)[2], float sc,
                                             int32_t lane) {
  const int32_t hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4* p = reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh);
      f32x4 x = *p;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] += acc[db][4 * j + i] * sc;
      *p = x;
    }
  }
}

// One launch's share of pattern k: its workgroups, decoded by dil_decode.
struct DilPart {
  int32_t k, nseg, qtiles, store;
};

__device__ __forceinline__ void dq_dil_workgroup(const BwdArgs& a, TT::Smem& sm, const DilPart& p,
                                                 int64_t wg) {
  const int32_t k = p.k, nseg = p.nseg, qtiles = p.qtiles, store = p.store;
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t qt, seg, bh;
  dil_decode(a, nseg, qtiles, wg, qt, seg, bh);
  const DilGeom g = dil_geom(a, k, seg, bh % a.H);
  const int32_t t0 = qt * kTQ;
  if (t0 >= g.n_rows) return;
  const int32_t qcount = min(kTQ, g.n_rows - t0);
  const size_t head_elems = (size_t)a.N * kD;
  const int32_t qi = TT::qrow(wave, lane, 0);
  const int32_t qpos = g.base + g.r * (t0 + min(qi, qcount - 1));
  const bool dead = TT::kQW * wave >= qcount;
  DqWave w;
  load_frag(w.qf, static_cast<const bf16*>(a.q) + bh * head_elems, qpos, lane);
  load_frag(w.df, static_cast<const bf16*>(a.dout) + bh * head_elems, qpos, lane);
  const float lse = a.lse[(size_t)bh * a.N + qpos];
  w.lse2 = lse == kNegInf ? -kNegInf : lse * kLog2e;
  if (store) {  // the first pattern keeps every row: D_i here, for the later launches
    w.di = row_delta(w.df, static_cast<const bf16*>(a.out) + bh * head_elems, qpos, lane);
    if (qi < qcount && lane < 32) a.delta[(size_t)bh * a.N + qpos] = w.di;
  } else {
    w.di = a.delta[(size_t)bh * a.N + qpos];
  }
  w.acc[0] = f32x16{};
  w.acc[1] = f32x16{};
  const int32_t hi = a.causal ? t0 + qcount - 1 : g.n_rows - 1;
  const int32_t n_tiles = (hi + kTK) / kTK;
  auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = n * kTK;
    const int32_t kcount = min(kTK, hi - u0 + 1);
    kt = {nullptr, g.base + g.r * u0, g.r, kcount, 0, kGlobNone};
    const bool full = kcount == kTK && (!a.causal || u0 + kTK - 1 <= t0);
    mr = {kRange, full ? 0 : 1, 0, t0 - u0, -kFar, a.causal ? 0 : kFar, 0, 0, 1};
  };
  const GlobInfo gi = {kGlobNone, nullptr, 0, nullptr, 0, 0, 0};
  stream_tiles<false>(sm, static_cast<const bf16*>(a.k) + bh * head_elems,
                      static_cast<const bf16*>(a.v) + bh * head_elems, n_tiles, desc, gi,
                      [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                        constexpr int32_t buf = decltype(buf_tag)::value;
                        dq_tile<buf, false>(sm, w, lane, mr, kt, qi, qpos, dead, a.scale_log2,
                                            BiasRule{nullptr, 0, 0, 0}, gi);
                      });
  if (qi < qcount) {
    float* dst = a.dq + ((size_t)bh * a.N + qpos) * kD;
    if (store)
      store_rows_f32(dst, w.acc, a.scale, lane);
    else
      add_rows_f32(dst, w.acc, a.scale, lane);
  }
}

__device__ __forceinline__ void dkv_dil_workgroup(const BwdArgs& a, BwdSmem& sm,
                                                  const DilPart& p, int64_t wg) {
  const int32_t k = p.k, nseg = p.nseg, qtiles = p.qtiles, store = p.store;
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t qt, seg, bh;
  dil_decode(a, nseg, qtiles, wg, qt, seg, bh);
  const DilGeom g = dil_geom(a, k, seg, bh % a.H);
  const int32_t t0 = qt * kTQ;
  if (t0 >= g.n_rows) return;
  const int32_t kcount = min(kTQ, g.n_rows - t0);
  const size_t head_elems = (size_t)a.N * kD;
  const int32_t ki = TT::qrow(wave, lane, 0);
  const int32_t kpos = g.base + g.r * (t0 + min(ki, kcount - 1));
  const bool dead = TT::kQW * wave >= kcount;
  DkvWave w;
  load_frag(w.kf, static_cast<const bf16*>(a.k) + bh * head_elems, kpos, lane);
  load_frag(w.vf, static_cast<const bf16*>(a.v) + bh * head_elems, kpos, lane);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    w.dk[x] = f32x16{};
    w.dv[x] = f32x16{};
  }
  // rows at or after the keys (causal), else every kept row
  const int32_t lo = a.causal ? t0 : 0, hi = g.n_rows - 1;
  const int32_t n_tiles = (hi - lo + 1 + kTK - 1) / kTK;
  const int32_t lob = a.causal ? 0 : -kFar;
  auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
    const int32_t u0 = lo + n * kTK;
    const int32_t cnt = min(kTK, hi - u0 + 1);
    kt = {nullptr, g.base + g.r * u0, g.r, cnt, 0, kGlobNone};
    const bool full = cnt == kTK && (!a.causal || u0 >= t0 + kcount - 1);
    mr = {kRange, full ? 0 : 1, 0, t0 - u0, lob, kFar, 0, 0, 1};
  };
  const GlobInfo gi = {kGlobNone, nullptr, 0, nullptr, 0, 0, 0};
  stream_rows<false>(sm, static_cast<const bf16*>(a.q) + bh * head_elems,
                     static_cast<const bf16*>(a.dout) + bh * head_elems,
                     a.lse + (size_t)bh * a.N, a.delta + (size_t)bh * a.N, 1.f / a.scale,
                     n_tiles, desc, gi,
                     [&](auto buf_tag, const KeyTile& kt, const MaskRule& mr) {
                       constexpr int32_t buf = decltype(buf_tag)::value;
                       dkv_tile<buf, false, false, true>(sm, w, lane, mr, kt, ki, kpos, dead, a.scale_log2,
                                                   a.causal);
                     });
  if (ki < kcount) {
    float* dk = a.dk + ((size_t)bh * a.N + kpos) * kD;
    float* dv = a.dv + ((size_t)bh * a.N + kpos) * kD;
    if (store) {
      store_rows_f32(dk, w.dk, a.scale, lane);
      store_rows_f32(dv, w.dv, 1.f, lane);
    } else {
      add_rows_f32(dk, w.dk, a.scale, lane);
      add_rows_f32(dv, w.dv, 1.f, lane);
    }
  }
}

// The launches: the global-tile workgroups first (their count rounded up to a
// multiple of 8), then the band workgroups. Block b runs on XCD b % 8; each
// XCD takes a contiguous share of the band tiles (tiles of one head then
// share K/V in that XCD's L2). The global tiles' work thus fills the chip
// while the band tiles finish, instead of running alone in a launch of its
// own.
__device__ __forceinline__ int32_t glob_wg(const BwdArgs& a) {
  return a.n_global > 0 ? a.B * a.H * ((a.n_global + TT::kTQ - 1) / TT::kTQ) * a.glob_chunks : 0;
}
__device__ __forceinline__ int32_t glob_wg_padded(const BwdArgs& a) {
  return (glob_wg(a) + kXcds - 1) / kXcds * kXcds;
}
// The band tile of block b (after the global ones), or -1.
__device__ __forceinline__ int32_t band_tile_of(const BwdArgs& a, int32_t b) {
  const int32_t x = b % kXcds, j = b / kXcds;
  const int32_t per = (a.n_band_wg + kXcds - 1) / kXcds;
  const int32_t bw = x * per + j;
  return j >= per || bw >= a.n_band_wg ? -1 : bw;
}

// dK/dV and dQ workgroups in one launch, the dK/dV ones (the longer work)
// first: the two add into different gradients, and D_i came from a launch
// before, so they run side by side and fill each other's tails.
// VEC: key-side label vectors (their tables in the dynamic LDS). LBL: label
// matrices and per-piece segment masks (with VEC and SEG; tables optional).
template <bool BIAS, bool SEG, bool VEC, bool LBL = false>
__global__ __launch_bounds__(TT::kThreads)
__attribute__((amdgpu_waves_per_eu((BIAS || VEC) ? 2 : 3)))
void bwd_mfma_kernel(BwdArgs a, int32_t grid_kv) {
  __shared__ BwdSmem sm;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int32_t gw = glob_wg_padded(a);
  const int32_t nb = grid_kv - gw;  // band slots per pass
  int32_t b = (int32_t)blockIdx.x;
  if (b < 2 * nb) {  // band: dK/dV, then dQ
    const bool kv = b < nb;
    const int32_t bw = band_tile_of(a, kv ? b : b - nb);
    if (bw < 0) return;
    if (kv)
      dkv_band_workgroup<BIAS, SEG, VEC, LBL>(a, sm, dyn, bw);
    else
      dq_band_workgroup<BIAS, SEG, VEC, LBL>(a, sm, dyn, bw);
    return;
  }
  b -= 2 * nb;  // global ranges: dK/dV, then dQ
  const bool kv = b < gw;
  if (!kv) b -= gw;
  if (b >= glob_wg(a)) return;
  if (kv)
    dkv_glob_workgroup<BIAS, SEG, VEC, LBL>(a, sm, dyn, b);
  else
    dq_glob_workgroup<BIAS, SEG, VEC, LBL>(a, sm, dyn, b);
}

// The global rows' dQ and the global keys' dK, dV from the ranges' partial
// sums, added in range order; with separate projections a global row's dq is 0.
// One thread per 4 columns of a global row of one of the three parts.
__global__ __launch_bounds__(256) void bwd_glob_reduce_kernel(BwdArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_part = (int64_t)a.B * a.H * a.n_global * (kD / 4);
  if (t >= 3 * per_part) return;
  const int32_t x = (int32_t)(t / per_part);  // 0 dQ, 1 dK, 2 dV
  const int64_t rest = t % per_part;
  const int32_t d4 = (int32_t)(rest % (kD / 4));
  const int64_t r = rest / (kD / 4);
  const int32_t g = (int32_t)(r % a.n_global), bh = (int32_t)(r / a.n_global);
  // every range's load in flight at once (at most kMaxGlobChunks), then
  // added in range order
  f32x4 v[kMaxGlobChunks];
#pragma unroll
  for (int u = 0; u < kMaxGlobChunks; ++u)
    v[u] = u < a.glob_chunks ? reinterpret_cast<const f32x4*>(part_row(a, x, u, bh, g))[d4]
                             : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMaxGlobChunks; ++u)
    if (u < a.glob_chunks) sum += v[u];
  const size_t ro = ((size_t)bh * a.N + a.gidx[g]) * kD;
  float* dst = x == 0 ? (a.sep ? a.dqg : a.dq) : (x == 1 ? a.dk : a.dv);
  reinterpret_cast<f32x4*>(dst + ro)[d4] = sum * (x == 2 ? 1.f : a.scale);
  if (x == 0 && a.sep) reinterpret_cast<f32x4*>(a.dq + ro)[d4] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One LongNet launch: the dK/dV workgroups of pattern kv.k (grid_kv of them,
// the longer work, first), then the dQ ones of pattern q.k (k < 0: none). The
// two parts add into different gradients, so they run side by side; each
// gradient still takes its patterns in launch order.
__global__ __launch_bounds__(TT::kThreads)
__attribute__((amdgpu_waves_per_eu(2)))
void bwd_dil_mfma_kernel(BwdArgs a, DilPart kv, int64_t grid_kv, DilPart q) {
  __shared__ BwdSmem sm;
  const int64_t b = blockIdx.x;
  if (b < grid_kv)
    dkv_dil_workgroup(a, sm, kv, b);
  else if (q.k >= 0)
    dq_dil_workgroup(a, sm, q, b - grid_kv);
}

// Key-side label vectors (ETC page, §3.4 "Relative Position Encoding"): each
// row's table T[row][l] = q'_row . a_l + b_l / scale (b the scalar table, if
// any), in q.k units, q' the row's query (qg for a global row with separate
// projections). 64 rows of one head per workgroup, four threads per row
// (labels l = part + 4u), the head's vectors in LDS (rows padded to D + 4
// floats: the four labels a wave reads at once, 16 bytes each, fall on
// different banks).
__global__ __launch_bounds__(256) void bwd_rowtab_kernel(BwdArgs a) {
  constexpr int32_t kRow = kD + 4;
  __shared__ __attribute__((aligned(16))) float av[kMaxLabels * kRow];
  const int32_t V = a.n_labels;
  const int32_t per = (a.N + 63) / 64;
  const int32_t bh = (int32_t)(blockIdx.x / per), t = (int32_t)(blockIdx.x % per);
  const int32_t h = bh % a.H;
  const int32_t i = t * 64 + (int32_t)(threadIdx.x >> 2), part = (int32_t)(threadIdx.x & 3);
  const bool live = i < a.N;
  // the row's query loads go out before the vectors' staging
  bf16x8 qx[kD / 8];
  if (live) {
    const bool g = a.sep && a.n_global > 0 && sorted_contains(a.gidx, a.n_global, i);
    const bf16* qr = static_cast<const bf16*>(g ? a.qg : a.q) + ((size_t)bh * a.N + i) * kD;
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) qx[c] = *reinterpret_cast<const bf16x8*>(qr + 8 * c);
  }
  if (a.rel_vec)
    for (int32_t x = threadIdx.x; x < V * kD; x += 256)
      av[(x / kD) * kRow + x % kD] = a.rel_vec[(size_t)h * V * kD + x];
  __syncthreads();
  if (!live) return;
  float qv[kD];
#pragma unroll
  for (int c = 0; c < kD / 8; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[8 * c + e] = (float)qx[c][e];
  }
  float* dst = a.rowtab + ((size_t)bh * a.N + i) * V;
  const float* sb = a.rel_bias ? a.rel_bias + (size_t)h * V : nullptr;
  for (int32_t l = part; l < V; l += 4) {
    float acc = sb ? sb[l] / a.scale : 0.f;
    if (a.rel_vec) {
      const f32x4* al = reinterpret_cast<const f32x4*>(av + l * kRow);
#pragma unroll
      for (int c = 0; c < kD / 4; ++c) {
        const f32x4 x = al[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qv[4 * c + e], x[e], acc);
      }
    }
    dst[l] = acc;
  }
}

// zeros into three fp32 buffers of n4 float4 each (a kernel: no memset)
__global__ __launch_bounds__(256) void bwd_zero3_kernel(float* x, float* y, float* z, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  reinterpret_cast<f32x4*>(x)[i] = zero;
  reinterpret_cast<f32x4*>(y)[i] = zero;
  reinterpret_cast<f32x4*>(z)[i] = zero;
}

}  // namespace

hipError_t launch_dilated_bwd_mfma(const BwdArgs& a, hipStream_t stream) {
  const int64_t n4 = (int64_t)a.B * a.H * a.N * kD / 4;
  if (n4 <= 0) return hipSuccess;
  int32_t first = -1;  // a pattern of dilation 1, launched first and storing
  for (int32_t k = 0; k < a.n_pairs && first < 0; ++k)
    if (a.pr[k] == 1) first = k;
  if (first < 0)  // zeros, then every pattern adds (D_i came from a launch before)
    hipLaunchKernelGGL(bwd_zero3_kernel, dim3((uint32_t)((n4 + 255) / 256)), dim3(256), 0, stream,
                       a.dq, a.dk, a.dv, n4);
  auto part_of = [&](int32_t k, bool store) {
    const int32_t nseg = (a.N + a.pw[k] - 1) / a.pw[k];
    const int32_t rows = (a.pw[k] + a.pr[k] - 1) / a.pr[k];
    return DilPart{k, nseg, (rows + TT::kTQ - 1) / TT::kTQ, store ? 1 : 0};
  };
  auto grid_of = [&](const DilPart& p) { return (int64_t)a.B * a.H * p.nseg * p.qtiles; };
  // order: the storing pattern, then the others taken alternately from the
  // small and the large end of their launch sizes. A pattern with few
  // workgroups (long segments at a high dilation) has the longest chains of
  // tiles per workgroup; paired with a pattern of many short workgroups, the
  // latter fill the chip around those chains.
  DilPart ord[kMaxPairs];
  int32_t n = 0;
  if (first >= 0) ord[n++] = part_of(first, true);
  for (int32_t k = 0; k < a.n_pairs; ++k) {
    if (k == first) continue;
    const DilPart p = part_of(k, false);
    int32_t x = n++;
    while (x > (first >= 0 ? 1 : 0) && grid_of(ord[x - 1]) > grid_of(p)) {
      ord[x] = ord[x - 1];
      --x;
    }
    ord[x] = p;
  }
  {
    const int32_t s0 = first >= 0 ? 1 : 0;
    DilPart alt[kMaxPairs];
    int32_t lo = s0, hi = n - 1, m = s0;
    while (lo <= hi) {
      alt[m++] = ord[lo++];
      if (lo <= hi) alt[m++] = ord[hi--];
    }
    for (int32_t x = s0; x < n; ++x) ord[x] = alt[x];
  }
  for (int32_t x = 0; x < n; ++x)
    if (grid_of(ord[x]) <= 0 || 2 * grid_of(ord[x]) > 0x7fffffffLL) return hipErrorInvalidValue;
  // launch x: dK/dV of pattern x - 1 beside dQ of pattern x
  const DilPart none = {-1, 0, 0, 0};
  for (int32_t x = 0; x <= n; ++x) {
    const DilPart kv = x > 0 ? ord[x - 1] : none;
    const DilPart q = x < n ? ord[x] : none;
    const int64_t gkv = x > 0 ? grid_of(kv) : 0, gq = x < n ? grid_of(q) : 0;
    hipLaunchKernelGGL(bwd_dil_mfma_kernel, dim3((uint32_t)(gkv + gq)), dim3(TT::kThreads), 0,
                       stream, a, kv, gkv, q);
  }
  return hipGetLastError();
}

// Blocks of a dQ or dK/dV launch: the padded global-tile ones and 8 times the
// band tiles per XCD.
static int64_t mfma_grid(const BwdArgs& a) {
  const int64_t g = a.n_global > 0 ? (int64_t)a.B * a.H * ((a.n_global + TT::kTQ - 1) / TT::kTQ) *
                                         a.glob_chunks
                                   : 0;
  return (g + kXcds - 1) / kXcds * kXcds + (int64_t)kXcds * ((a.n_band_wg + kXcds - 1) / kXcds);
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t stream) {
  if (a.n_band_wg <= 0) return hipSuccess;
  if (a.glob_chunks < 1 || (a.glob_chunks > 1 && !a.gpart)) return hipErrorInvalidValue;
  const int64_t grid = mfma_grid(a);
  if (2 * grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 g((uint32_t)(2 * grid)), t(TT::kThreads);
  const int32_t gkv = (int32_t)grid;
  const bool lbl = a.glabel || a.llabel || (a.seg && a.seg_pieces != 15) ||
                   ((a.rel_bias || a.rel_vec) && a.n_labels != 2 * a.rel_k + 1);
  if (lbl) {  // row tables when there is a table, label sums with vectors
    if ((a.rel_bias || a.rel_vec) != (a.rowtab != nullptr) || a.n_labels < 1 ||
        a.n_labels > kMaxLabels)
      return hipErrorInvalidValue;
    const int32_t V = a.n_labels < 3 ? 3 : a.n_labels;  // room for the dK/dV offset rows
    const uint32_t dyn = (uint32_t)((2 * TT::kTQ + kD) * V * sizeof(float));
    hipLaunchKernelGGL((bwd_mfma_kernel<false, true, true, true>), g, t, dyn, stream, a, gkv);
  } else if (a.rel_vec) {  // the tables (scalar bias folded in), the label sums, the vectors
    if (!a.rowtab || a.n_labels != 2 * a.rel_k + 1 || a.n_labels > kMaxLabels)
      return hipErrorInvalidValue;
    // dQ: rows' tables, label sums, vectors; dK/dV: two tiles' tables and
    // four offset rows (2 * kTQ * V >= 2 * kTK * V + 4 * kTK for V >= 3)
    const uint32_t dyn = (uint32_t)((2 * TT::kTQ + kD) * a.n_labels * sizeof(float));
    if (a.seg)
      hipLaunchKernelGGL((bwd_mfma_kernel<false, true, true>), g, t, dyn, stream, a, gkv);
    else
      hipLaunchKernelGGL((bwd_mfma_kernel<false, false, true>), g, t, dyn, stream, a, gkv);
  } else if (a.rel_bias && a.seg) {
    hipLaunchKernelGGL((bwd_mfma_kernel<true, true, false>), g, t, 0, stream, a, gkv);
  } else if (a.rel_bias) {
    hipLaunchKernelGGL((bwd_mfma_kernel<true, false, false>), g, t, 0, stream, a, gkv);
  } else if (a.seg) {
    hipLaunchKernelGGL((bwd_mfma_kernel<false, true, false>), g, t, 0, stream, a, gkv);
  } else {
    hipLaunchKernelGGL((bwd_mfma_kernel<false, false, false>), g, t, 0, stream, a, gkv);
  }
  return hipGetLastError();
}

hipError_t launch_rowtab(const BwdArgs& a, hipStream_t stream) {
  if (!a.rowtab || a.n_band_wg <= 0) return hipSuccess;
  if (!a.rowtab || a.n_labels < 1 || a.n_labels > kMaxLabels) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.B * a.H * ((a.N + 63) / 64);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_rowtab_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_glob_reduce(const BwdArgs& a, hipStream_t stream) {
  if (a.n_global <= 0 || a.glob_chunks <= 1) return hipSuccess;
  if (a.glob_chunks > kMaxGlobChunks) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)3 * a.B * a.H * a.n_global * (kD / 4);
  hipLaunchKernelGGL(bwd_glob_reduce_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

// Partial-sum rows per head that the workspace holds: the padded sequence up
// to 2048 (the ranges share them: chunks * n_gpad <= this).
int32_t host_glob_part_rows(int32_t N) {
  const int32_t padded = (N + TT::kTQ - 1) / TT::kTQ * TT::kTQ;
  return padded < 2048 ? padded : 2048;
}

// Ranges per global tile: enough workgroups to fill the chip twice over
// (about 512), at most 16, at least 4 tiles of 64 per range, and within the
// workspace's partial rows.
int32_t host_glob_chunks(int64_t bh, int32_t N, int32_t n_global) {
  if (n_global <= 0 || bh <= 0) return 1;
  const int32_t n_gpad = (n_global + TT::kTQ - 1) / TT::kTQ * TT::kTQ;
  const int64_t units = bh * (n_gpad / TT::kTQ);
  int64_t c = (512 + units - 1) / units;
  c = c < kMaxGlobChunks ? c : kMaxGlobChunks;
  const int64_t by_rows = host_glob_part_rows(N) / n_gpad;
  c = c < by_rows ? c : by_rows;
  const int64_t by_len = (N + 4 * kTK - 1) / (4 * kTK);
  c = c < by_len ? c : by_len;
  return c > 1 ? (int32_t)c : 1;
}

}  // namespace la
