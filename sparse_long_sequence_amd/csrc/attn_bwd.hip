// attn_bwd.hip — backward of band + global attention: dQ, dK, dV from the
// forward's output and lse (the training step after the forward; the forward
// keeps the softmax in fp32, Longformer page, §3.4 "Autoregressive Language
// Modeling Configuration").
//
// With P_ij = c_ij exp(s_ij - lse_i), s_ij = q_i . k_j / sqrt(D) and the mask
// c of the forward (LongNet page, §3.4 "Standard Self-Attention and Sparse
// Attention (Preliminaries)", Eq. 2, differentiated):
//   D_i   = dO_i . O_i                 dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = sum_j dS_ij k_j / sqrt(D)  dK_j = sum_i dS_ij q_i / sqrt(D)
//   dV_j  = sum_i P_ij dO_i
// Global rows with separate projections (Longformer page, §3.4 "Separate
// Linear Projections for Local vs. Global Attention") differentiate through
// qg_i, kg_j, vg_j, so their terms land in dqg, dkg, dvg.
//
// bf16 calls and the LongNet mixture run on the MFMA tile engine
// (attn_bwd_mfma.hip); this file holds their D_i launch and the fp32 path.
// The fp32 path has no atomics: after a pass that marks the global positions,
// a query-centric pass (one wave per row, one lane per vector element, dot
// products as wave sums) writes D_i and dQ_i, and a key-centric pass (one
// wave per key) visits every row that attends to its key and writes dK_j and
// dV_j in one store.
#include <hip/hip_runtime.h>
#include <math.h>

#include "bwd_kernels.h"
#include "tile_core.h"

namespace la {
namespace {

constexpr int kWavesBwd = 4;  // rows (or keys) per workgroup

__device__ __forceinline__ float load_el(const float* p) { return *p; }

// Sum over the 64 lanes, in registers; every lane gets the same value (each
// step adds a lane's value and its partner's, a commutative pair). DPP moves
// within rows of 16 lanes: quad_perm [1,0,3,2] and [2,3,0,1] (partners l^1,
// l^2), row_half_mirror (8 lanes reversed: the other quad) and row_mirror (16
// lanes reversed: the other half-row); then the gfx950 half-wave swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_partner<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_partner<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_partner<0x141>(x);  // row_half_mirror
  x += dpp_partner<0x140>(x);  // row_mirror
  return xor32_sum(xor16_sum(x));
}

// Dilated window of row i (the forward's band): j - i = t * dil, |t| <= R,
// causal t <= 0.
__device__ __forceinline__ bool in_band(int32_t i, int32_t j, int32_t R, int32_t dil,
                                        int32_t causal) {
  const int32_t delta = j - i;
  if (causal && delta > 0) return false;
  if (delta % dil != 0) return false;
  const int32_t t = delta / dil;
  return t >= -R && t <= R;
}

// Global ranks of the N positions (index in global_idx, -1: not global; in
// the workspace), so the loops below test membership with one load instead of
// a search, and find a global token's label row.
__global__ __launch_bounds__(256) void bwd_flags_kernel(BwdArgs a) {
  const int32_t p = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (p < a.N) a.grank[p] = a.n_global > 0 ? sorted_index(a.gidx, a.n_global, p) : -1;
}

// Pair (i, j) of batch row b under the forward's per-instance inputs, given
// the two global ranks (ETC page, §3.4 "Per-instance attention masks" and
// "Relative Position Encoding", Step 1): -2 when a segment mask of its piece
// or a masking label excludes it, -1 when it is kept without a label (a mixed
// pair keeping its usual label, or no bias tables), else its label.
__device__ __forceinline__ int32_t bwd_pair(const BwdArgs& a, int32_t b, int32_t i, int32_t j,
                                            int32_t gi, int32_t gj, const int32_t* segb) {
  const bool ig = gi >= 0, jg = gj >= 0;
  if (segb) {
    const int32_t piece = ig ? (jg ? 1 : 2) : (jg ? 4 : 8);  // g2g, g2l, l2g, l2l
    if ((a.seg_pieces & piece) && segb[i] != segb[j]) return -2;
  }
  int32_t l = kLabelDistance;
  if (ig && a.glabel)
    l = a.glabel[((size_t)b * a.n_global + gi) * a.N + j];
  else if (!ig && jg && a.llabel)
    l = a.llabel[((size_t)b * a.N + i) * a.n_global + gj];
  if (l != kLabelDistance && l >= a.n_labels) return -2;
  if (!a.rel_bias && !a.rel_vec) return -1;
  if (l == kLabelDistance) {
    if (ig != jg) return -1;
    l = min(max(j - i, -a.rel_k), a.rel_k) + a.rel_k;
  }
  return l;
}

// The logit's bias for label lab (>= 0) of head h, given qa = q_i . a_lab
// (unscaled; 0 without label vectors).
__device__ __forceinline__ float label_bias(const BwdArgs& a, int32_t h, int32_t lab, float qa) {
  return (a.rel_bias ? a.rel_bias[h * a.n_labels + lab] : 0.f) + qa * a.scale;
}

constexpr int kBatch = 8;  // pairs whose loads and reductions are issued together

// D_i = dO_i . O_i of every row (bf16; for the band + global MFMA path, and a
// LongNet call without a pattern of dilation 1): eight lanes per row with one
// 16-byte load each from dO and O, kDeltaPasses rows per group of eight lanes
// with all their loads in flight at once (32 * kDeltaPasses rows per
// workgroup).
constexpr int kDeltaPasses = 4;
static int64_t delta_blocks(int64_t rows) { return (rows + 32 * kDeltaPasses - 1) / (32 * kDeltaPasses); }

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int32_t part = threadIdx.x & 7;
  bf16x8 d[kDeltaPasses], y[kDeltaPasses];
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    const int64_t row = ((int64_t)blockIdx.x * kDeltaPasses + p) * 32 + (threadIdx.x >> 3);
    if (row < rows) {
      const size_t o = (size_t)row * kD + 8 * part;
      d[p] = __builtin_bit_cast(bf16x8, ldg16(static_cast<const bf16*>(a.dout) + o));
      y[p] = __builtin_bit_cast(bf16x8, ldg16(static_cast<const bf16*>(a.out) + o));
    }
  }
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    const int64_t row = ((int64_t)blockIdx.x * kDeltaPasses + p) * 32 + (threadIdx.x >> 3);
    const bool live = row < rows;
    float x = 0.f;
    if (live) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x += (float)d[p][e] * (float)y[p][e];
    }
    // sum over the row's eight lanes: partners l^1, l^2, then the other quad
    x += dpp_partner<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_partner<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_partner<0x141>(x);  // row_half_mirror
    if (live && part == 0) a.delta[row] = x;
  }
}

// Row i's gradient dQ_i (query-centric), and D_i into the workspace.
template <typename T>
__global__ __launch_bounds__(64 * kWavesBwd) void bwd_dq_kernel(BwdArgs a) {
  __shared__ float qa_s[kWavesBwd][kMaxLabels];  // q_i . a_l of this wave's row
  const int32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWavesBwd + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (row >= rows) return;
  const int32_t N = a.N;
  const int32_t i = (int32_t)(row % N);
  const int64_t bh = row / N;
  const int32_t h = (int32_t)(bh % a.H), b = (int32_t)(bh / a.H);
  const size_t hoff = (size_t)bh * N * kD;
  const int32_t gi = a.grank[i];
  const bool ig = gi >= 0;
  const bool sep = ig && a.sep;
  const T* Q = static_cast<const T*>(sep ? a.qg : a.q) + hoff;
  const T* K = static_cast<const T*>(sep ? a.kg : a.k) + hoff;
  const T* V = static_cast<const T*>(sep ? a.vg : a.v) + hoff;
  const float dov = load_el(static_cast<const T*>(a.dout) + hoff + (size_t)i * kD + lane);
  const float ov = load_el(static_cast<const T*>(a.out) + hoff + (size_t)i * kD + lane);
  const float Di = wave_sum(dov * ov);
  if (lane == 0) a.delta[row] = Di;
  const float qv = load_el(Q + (size_t)i * kD + lane);
  const float lse = a.lse[row];
  const int32_t* segb = a.seg ? a.seg + (size_t)b * N : nullptr;
  const float* avec = a.rel_vec ? a.rel_vec + (size_t)h * a.n_labels * kD : nullptr;
  if (avec)
    for (int32_t l = 0; l < a.n_labels; ++l) {
      const float t = wave_sum(qv * avec[(size_t)l * kD + lane]);
      if (lane == 0) qa_s[wv][l] = t;
    }
  float acc = 0.f;
  // keys key_of(x), x in [0, n) (-1: skip), kBatch at a time; a skipped slot
  // reads row i (always valid) and gets weight 0
  auto sweep = [&](int32_t n, auto key_of) {
    for (int32_t x0 = 0; x0 < n; x0 += kBatch) {
      int32_t j[kBatch], lb[kBatch];
      float kv[kBatch], vv[kBatch], s[kBatch], dp[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        j[e] = x0 + e < n ? key_of(x0 + e) : -1;
        lb[e] = j[e] >= 0 ? bwd_pair(a, b, i, j[e], gi, a.grank[j[e]], segb) : -1;
        if (lb[e] == -2) j[e] = -1;
        const int32_t r = j[e] >= 0 ? j[e] : i;
        kv[e] = load_el(K + (size_t)r * kD + lane);
        vv[e] = load_el(V + (size_t)r * kD + lane);
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        s[e] = wave_sum(qv * kv[e]);
        dp[e] = wave_sum(dov * vv[e]);
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const bool lab = j[e] >= 0 && lb[e] >= 0;
        const float bias = lab ? label_bias(a, h, lb[e], avec ? qa_s[wv][lb[e]] : 0.f) : 0.f;
        const float p = j[e] >= 0 ? __expf(s[e] * a.scale + bias - lse) : 0.f;
        // a label vector's share q_i . a_l of the logit adds a_l to dq
        const float av = (lab && avec) ? avec[(size_t)lb[e] * kD + lane] : 0.f;
        acc += p * (dp[e] - Di) * (kv[e] + av);
      }
    }
  };
  if (lse != kNegInf) {  // a row without keys has no gradient
    if (ig) {  // a global row attends to every key (causal: up to itself)
      sweep(a.causal ? i + 1 : N, [&](int32_t x) { return x; });
    } else {
      const int32_t d = a.dil[h], R = a.radius;
      // the window's keys inside [0, N): t in [t0, t1]
      const int32_t t0 = -min(R, i / d);
      const int32_t t1 = a.causal ? 0 : min(R, (N - 1 - i) / d);
      sweep(t1 - t0 + 1, [&](int32_t x) { return i + (t0 + x) * d; });
      // global keys outside the window (a global key in it was counted there)
      sweep(a.n_global, [&](int32_t x) {
        const int32_t j = a.gidx[x];
        const bool skip = j < 0 || j >= N || (a.causal && j > i) || in_band(i, j, R, d, a.causal);
        return skip ? -1 : j;
      });
    }
  }
  const float g = acc * a.scale;
  if (a.sep) {  // each row owns one of the two gradients; the other gets 0
    a.dq[hoff + (size_t)i * kD + lane] = ig ? 0.f : g;
    a.dqg[hoff + (size_t)i * kD + lane] = ig ? g : 0.f;
  } else {
    a.dq[hoff + (size_t)i * kD + lane] = g;
  }
}

// Key j's gradients dK_j, dV_j (and dKg_j, dVg_j), key-centric.
template <typename T>
__global__ __launch_bounds__(64 * kWavesBwd) void bwd_dkv_kernel(BwdArgs a) {
  const int32_t lane = threadIdx.x & 63;
  const int64_t key = (int64_t)blockIdx.x * kWavesBwd + (threadIdx.x >> 6);
  const int64_t keys = (int64_t)a.B * a.H * a.N;
  if (key >= keys) return;
  const int32_t N = a.N;
  const int32_t j = (int32_t)(key % N);
  const int64_t bh = key / N;
  const int32_t h = (int32_t)(bh % a.H), b = (int32_t)(bh / a.H);
  const size_t hoff = (size_t)bh * N * kD;
  const float* lse = a.lse + (size_t)bh * N;
  const float* delta = a.delta + (size_t)bh * N;
  const T* dO = static_cast<const T*>(a.dout) + hoff;
  const int32_t* segb = a.seg ? a.seg + (size_t)b * N : nullptr;
  const int32_t d = a.dil[h], R = a.radius;
  const int32_t gj = a.grank[j];
  const bool jg = gj >= 0;
  const float* avec = a.rel_vec ? a.rel_vec + (size_t)h * a.n_labels * kD : nullptr;

  // rows row_of(x), x in [0, n) (-1: skip), through projections Q with this
  // key's (kv, vv), into (dk, dv); kBatch rows at a time, a skipped slot reads
  // row j (always valid) and gets weight 0
  auto sweep = [&](int32_t n, const T* Q, float kv, float vv, float& dk, float& dv,
                   auto row_of) {
    for (int32_t x0 = 0; x0 < n; x0 += kBatch) {
      int32_t i[kBatch], lb[kBatch];
      float qv[kBatch], dov[kBatch], li[kBatch], di[kBatch], s[kBatch], dp[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        i[e] = x0 + e < n ? row_of(x0 + e) : -1;
        lb[e] = i[e] >= 0 ? bwd_pair(a, b, i[e], j, a.grank[i[e]], gj, segb) : -1;
        if (lb[e] == -2) i[e] = -1;
        const int32_t r = i[e] >= 0 ? i[e] : j;
        qv[e] = load_el(Q + (size_t)r * kD + lane);
        dov[e] = load_el(dO + (size_t)r * kD + lane);
        li[e] = lse[r];
        di[e] = delta[r];
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        s[e] = wave_sum(qv[e] * kv);
        dp[e] = wave_sum(dov[e] * vv);
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const bool on = i[e] >= 0 && li[e] != kNegInf;
        const bool lab = on && lb[e] >= 0;
        float qa = 0.f;  // q_i . a_l (uniform branch: one pair per wave)
        if (lab && avec) qa = wave_sum(qv[e] * avec[(size_t)lb[e] * kD + lane]);
        const float bias = lab ? label_bias(a, h, lb[e], qa) : 0.f;
        const float p = on ? __expf(s[e] * a.scale + bias - li[e]) : 0.f;
        dv += p * dov[e];
        dk += p * (dp[e] - di[e]) * qv[e];
      }
    }
  };

  const T* Qs = static_cast<const T*>(a.q) + hoff;
  const float kv = load_el(static_cast<const T*>(a.k) + hoff + (size_t)j * kD + lane);
  const float vv = load_el(static_cast<const T*>(a.v) + hoff + (size_t)j * kD + lane);
  float dk = 0.f, dv = 0.f;
  // non-global rows whose window holds j: i = j + u * d, causal u >= 0
  {
    const int32_t u0 = a.causal ? 0 : -min(R, j / d);
    const int32_t u1 = min(R, (N - 1 - j) / d);
    sweep(u1 - u0 + 1, Qs, kv, vv, dk, dv, [&](int32_t x) {
      const int32_t i = j + (u0 + x) * d;
      return a.grank[i] >= 0 ? -1 : i;
    });
  }
  // a global key: every other non-global row (causal: from j on)
  if (jg) {
    const int32_t i0 = a.causal ? j : 0;
    sweep(N - i0, Qs, kv, vv, dk, dv, [&](int32_t x) {
      const int32_t i = i0 + x;
      return (in_band(i, j, R, d, a.causal) || a.grank[i] >= 0) ? -1 : i;
    });
  }
  // global rows attend to every key (causal: rows from j on)
  auto grow = [&](int32_t x) {
    const int32_t i = a.gidx[x];
    return (i < 0 || i >= N || (a.causal && i < j)) ? -1 : i;
  };
  if (!a.sep) {
    sweep(a.n_global, Qs, kv, vv, dk, dv, grow);
  } else {
    const T* Qg = static_cast<const T*>(a.qg) + hoff;
    const float kgv = load_el(static_cast<const T*>(a.kg) + hoff + (size_t)j * kD + lane);
    const float vgv = load_el(static_cast<const T*>(a.vg) + hoff + (size_t)j * kD + lane);
    float dkg = 0.f, dvg = 0.f;
    sweep(a.n_global, Qg, kgv, vgv, dkg, dvg, grow);
    a.dkg[hoff + (size_t)j * kD + lane] = dkg * a.scale;
    a.dvg[hoff + (size_t)j * kD + lane] = dvg;
  }
  a.dk[hoff + (size_t)j * kD + lane] = dk * a.scale;
  a.dv[hoff + (size_t)j * kD + lane] = dv;
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a, int32_t dtype, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (rows <= 0) return hipSuccess;
  const dim3 g((uint32_t)((rows + kWavesBwd - 1) / kWavesBwd)), blk(64 * kWavesBwd);
  if (dtype == 1) {
    // D_i, then dK/dV and dQ on MFMA in one launch (no global ranks needed)
    if (a.n_band_wg <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((uint32_t)delta_blocks(rows)), dim3(256), 0, stream, a);
    hipError_t e = launch_rowtab(a, stream);  // key-side label vectors: the rows' tables
    if (e != hipSuccess) return e;
    e = launch_bwd_mfma(a, stream);
    if (e != hipSuccess) return e;
    e = launch_glob_reduce(a, stream);  // the global tiles' partial sums
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  // fp32: global ranks, then dQ and D_i, then dK and dV on the VALU
  hipLaunchKernelGGL(bwd_flags_kernel, dim3((uint32_t)((a.N + 255) / 256)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(bwd_dq_kernel<float>, g, blk, 0, stream, a);
  hipLaunchKernelGGL(bwd_dkv_kernel<float>, g, blk, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dilated_bwd(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (rows <= 0) return hipSuccess;
  // each pattern's terms on the MFMA tile engine; a pattern of dilation 1
  // goes first and its dQ launch writes D_i, else D_i comes first here
  bool r1 = false;
  for (int32_t k = 0; k < a.n_pairs; ++k) r1 = r1 || a.pr[k] == 1;
  if (!r1)
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((uint32_t)delta_blocks(rows)), dim3(256), 0, stream, a);
  return launch_dilated_bwd_mfma(a, stream);
}

}  // namespace la
