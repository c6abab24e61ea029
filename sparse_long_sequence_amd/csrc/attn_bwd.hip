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
// No atomics: after a pass that marks the global positions, a query-centric
// pass (one wave per row) writes D_i and dQ_i, and a key-centric pass (one
// wave per key) visits every row that attends to its key and writes dK_j and
// dV_j in one store. These are the scalar kernels: fp32 VALU work, no MFMA.
// The fp32 path keeps one lane per vector element (dot products as wave
// sums); the bf16 path (below) puts one key or row on each lane instead. They
// serve fp32 calls and calls with bias tables, labels or segment ids; bf16
// calls without them, and the LongNet mixture, run on the MFMA tile engine
// (attn_bwd_mfma.hip), whose dQ launches compute D_i (a LongNet call without
// a pattern of dilation 1 takes it from the launch here first).
#include <hip/hip_runtime.h>
#include <math.h>

#include "bwd_kernels.h"
#include "tile_core.h"

namespace la {
namespace {

constexpr int kWavesBwd = 4;  // rows (or keys) per workgroup

__device__ __forceinline__ float load_el(const float* p) { return *p; }
__device__ __forceinline__ float load_el(const bf16* p) { return (float)*p; }

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

// ---------------------------------------------------------------------------
// bf16 form: one lane per key (dQ) or per row (dK, dV). Each lane loads whole
// 128-byte rows and forms its own dot products against the wave's query or key
// vectors, which sit in LDS (read as broadcasts), so a pair costs no cross-lane
// work; each lane keeps a 64-wide partial gradient, summed across the lanes once
// per row (or key) at the end.
// ---------------------------------------------------------------------------

// Eight bf16 (one 16-byte chunk, element 2e in the low half of word e) to fp32.
__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __builtin_bit_cast(float, w[e] << 16);
    f[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xffff0000u);
  }
}

// A 64-element bf16 row as eight 16-byte chunks.
__device__ __forceinline__ void load_row(const bf16* row, uint4 (&c)[8]) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = p[k];
}

// x . y over 64 elements: x packed in chunks, y a wave vector in LDS.
__device__ __forceinline__ float dot_row(const uint4 (&c)[8], const float* y) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float f[8];
    unpack8(c[k], f);
    const float4 y0 = *reinterpret_cast<const float4*>(y + 8 * k);
    const float4 y1 = *reinterpret_cast<const float4*>(y + 8 * k + 4);
    s += f[0] * y0.x + f[1] * y0.y + f[2] * y0.z + f[3] * y0.w;
    s += f[4] * y1.x + f[5] * y1.y + f[6] * y1.z + f[7] * y1.w;
  }
  return s;
}

// acc += w * row (row packed in chunks). The chunk is unpacked again here
// (an opaque copy of its words) rather than kept unpacked from the dot
// product, which would hold 64 more registers per row.
__device__ __forceinline__ void axpy_row(float (&acc)[kD], float w, const uint4 (&c)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint4 u = c[k];
    asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
    float f[8];
    unpack8(u, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[8 * k + e] += w * f[e];
  }
}

// Lane d receives the sum over the lanes of acc[d].
__device__ __forceinline__ float lane_totals(const float (&acc)[kD], int32_t lane) {
  float res = 0.f;
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    const float t = wave_sum(acc[d]);
    res = lane == d ? t : res;
  }
  return res;
}

__global__ __launch_bounds__(64 * kWavesBwd) void bwd_dq_rows_kernel(BwdArgs a) {
  __shared__ float vq[kWavesBwd][kD], vdo[kWavesBwd][kD];
  __shared__ float qa_s[kWavesBwd][kMaxLabels];  // q_i . a_l of this wave's row
  const int32_t lane = threadIdx.x & 63;
  const int32_t wv = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
  const int32_t N = a.N;
  const int64_t rows = (int64_t)a.B * a.H * N;
  const int64_t row0 = (int64_t)blockIdx.x * kWavesBwd + wv;
  const bool valid = row0 < rows;
  const int64_t row = valid ? row0 : rows - 1;  // a wave past the end stages a valid row
  const int32_t i = (int32_t)(row % N);
  const int64_t bh = row / N;
  const int32_t h = (int32_t)(bh % a.H), b = (int32_t)(bh / a.H);
  const size_t hoff = (size_t)bh * N * kD;
  const int32_t gi = a.grank[i];
  const bool ig = gi >= 0;
  const bool sep = ig && a.sep;
  const bf16* Q = static_cast<const bf16*>(sep ? a.qg : a.q) + hoff;
  const bf16* K = static_cast<const bf16*>(sep ? a.kg : a.k) + hoff;
  const bf16* V = static_cast<const bf16*>(sep ? a.vg : a.v) + hoff;
  const float dov = load_el(static_cast<const bf16*>(a.dout) + hoff + (size_t)i * kD + lane);
  const float ov = load_el(static_cast<const bf16*>(a.out) + hoff + (size_t)i * kD + lane);
  const float Di = wave_sum(dov * ov);
  const float qv = load_el(Q + (size_t)i * kD + lane);
  vq[wv][lane] = qv;
  vdo[wv][lane] = dov;
  const float* avec = a.rel_vec ? a.rel_vec + (size_t)h * a.n_labels * kD : nullptr;
  if (avec)
    for (int32_t l = 0; l < a.n_labels; ++l) {
      const float t = wave_sum(qv * avec[(size_t)l * kD + lane]);
      if (lane == 0) qa_s[wv][l] = t;
    }
  __syncthreads();  // the only barrier: every wave reaches it
  if (!valid) return;
  if (lane == 0) a.delta[row] = Di;
  const float lse = a.lse[row];
  const int32_t* segb = a.seg ? a.seg + (size_t)b * N : nullptr;
  float acc[kD];
#pragma unroll
  for (int d = 0; d < kD; ++d) acc[d] = 0.f;
  // keys key_of(x), x in [0, n) (-1: skip), one per lane; a skipped lane
  // reads row i (always valid) and gets weight 0
  auto sweep = [&](int32_t n, auto key_of) {
    for (int32_t x0 = 0; x0 < n; x0 += 64) {
      const int32_t x = x0 + lane;
      int32_t j = x < n ? key_of(x) : -1;
      const int32_t lb = j >= 0 ? bwd_pair(a, b, i, j, gi, a.grank[j], segb) : -1;
      if (lb == -2) j = -1;
      if (__ballot(j >= 0) == 0ull) continue;  // no lane has a pair (masks, labels)
      const int32_t r = j >= 0 ? j : i;
      uint4 kc[8], vc[8];
      load_row(K + (size_t)r * kD, kc);
      load_row(V + (size_t)r * kD, vc);
      const float s = dot_row(kc, vq[wv]);
      const float dp = dot_row(vc, vdo[wv]);
      const bool lab = j >= 0 && lb >= 0;
      const float bias = lab ? label_bias(a, h, lb, avec ? qa_s[wv][lb] : 0.f) : 0.f;
      const float p = j >= 0 ? __expf(s * a.scale + bias - lse) : 0.f;
      const float w = p * (dp - Di);
      axpy_row(acc, w, kc);
      if (lab && avec) {  // a label vector's share q_i . a_l of the logit adds a_l to dq
        const float4* al = reinterpret_cast<const float4*>(avec + (size_t)lb * kD);
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) {
          const float4 x4 = al[c];
          acc[4 * c] += w * x4.x;
          acc[4 * c + 1] += w * x4.y;
          acc[4 * c + 2] += w * x4.z;
          acc[4 * c + 3] += w * x4.w;
        }
      }
    }
  };
  if (lse != kNegInf) {
    if (ig) {
      sweep(a.causal ? i + 1 : N, [&](int32_t x) { return x; });
    } else {
      const int32_t d = a.dil[h], R = a.radius;
      const int32_t t0 = -min(R, i / d);
      const int32_t t1 = a.causal ? 0 : min(R, (N - 1 - i) / d);
      sweep(t1 - t0 + 1, [&](int32_t x) { return i + (t0 + x) * d; });
      sweep(a.n_global, [&](int32_t x) {
        const int32_t j = a.gidx[x];
        const bool skip = j < 0 || j >= N || (a.causal && j > i) || in_band(i, j, R, d, a.causal);
        return skip ? -1 : j;
      });
    }
  }
  const float g = lane_totals(acc, lane) * a.scale;
  if (a.sep) {
    a.dq[hoff + (size_t)i * kD + lane] = ig ? 0.f : g;
    a.dqg[hoff + (size_t)i * kD + lane] = ig ? g : 0.f;
  } else {
    a.dq[hoff + (size_t)i * kD + lane] = g;
  }
}

__global__ __launch_bounds__(64 * kWavesBwd) void bwd_dkv_rows_kernel(BwdArgs a) {
  // this wave's key and value vectors, shared and (separate projections) global
  __shared__ float vk[kWavesBwd][kD], vv[kWavesBwd][kD], vkg[kWavesBwd][kD], vvg[kWavesBwd][kD];
  const int32_t lane = threadIdx.x & 63;
  const int32_t wv = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
  const int32_t N = a.N;
  const int64_t keys = (int64_t)a.B * a.H * N;
  const int64_t key0 = (int64_t)blockIdx.x * kWavesBwd + wv;
  const bool valid = key0 < keys;
  const int64_t key = valid ? key0 : keys - 1;
  const int32_t j = (int32_t)(key % N);
  const int64_t bh = key / N;
  const int32_t h = (int32_t)(bh % a.H), b = (int32_t)(bh / a.H);
  const size_t hoff = (size_t)bh * N * kD;
  const size_t jo = hoff + (size_t)j * kD + lane;
  vk[wv][lane] = load_el(static_cast<const bf16*>(a.k) + jo);
  vv[wv][lane] = load_el(static_cast<const bf16*>(a.v) + jo);
  if (a.sep) {
    vkg[wv][lane] = load_el(static_cast<const bf16*>(a.kg) + jo);
    vvg[wv][lane] = load_el(static_cast<const bf16*>(a.vg) + jo);
  }
  __syncthreads();  // the only barrier: every wave reaches it
  if (!valid) return;
  const float* lse = a.lse + (size_t)bh * N;
  const float* delta = a.delta + (size_t)bh * N;
  const bf16* dO = static_cast<const bf16*>(a.dout) + hoff;
  const int32_t* segb = a.seg ? a.seg + (size_t)b * N : nullptr;
  const int32_t d = a.dil[h], R = a.radius;
  const int32_t gj = a.grank[j];
  const bool jg = gj >= 0;
  const float* avec = a.rel_vec ? a.rel_vec + (size_t)h * a.n_labels * kD : nullptr;
  // Two passes over the same rows, one accumulator live at a time: dV (needs
  // s only) and then dK (needs s and dP).
  float acc[kD];
  // rows row_of(x), x in [0, n) (-1: skip), one per lane, through projection Q
  // against key vectors (kvec, vvec); a skipped lane reads row j and gets weight 0
  auto sweep = [&](bool dk_pass, int32_t n, const bf16* Q, const float* kvec, const float* vvec,
                   auto row_of) __attribute__((always_inline)) {
    for (int32_t x0 = 0; x0 < n; x0 += 64) {
      const int32_t x = x0 + lane;
      int32_t i = x < n ? row_of(x) : -1;
      const int32_t lb = i >= 0 ? bwd_pair(a, b, i, j, a.grank[i], gj, segb) : -1;
      if (lb == -2) i = -1;
      if (__ballot(i >= 0) == 0ull) continue;  // no lane has a pair (masks, labels)
      const int32_t r = i >= 0 ? i : j;
      uint4 qc[8], oc[8];
      load_row(Q + (size_t)r * kD, qc);
      load_row(dO + (size_t)r * kD, oc);
      const float li = lse[r];
      const float sc = dot_row(qc, kvec);
      const bool on = i >= 0 && li != kNegInf;
      float bias = 0.f;
      if (on && lb >= 0) bias = label_bias(a, h, lb, avec ? dot_row(qc, avec + (size_t)lb * kD) : 0.f);
      const float p = on ? __expf(sc * a.scale + bias - li) : 0.f;
      if (dk_pass) {
        const float dp = dot_row(oc, vvec);
        axpy_row(acc, p * (dp - delta[r]), qc);
      } else {
        axpy_row(acc, p, oc);
      }
    }
  };
  const bf16* Qs = static_cast<const bf16*>(a.q) + hoff;
  auto grow = [&](int32_t x) {
    const int32_t i = a.gidx[x];
    return (i < 0 || i >= N || (a.causal && i < j)) ? -1 : i;
  };
  // every row that reaches key j through the shared projections
  auto shared_rows = [&](bool dk_pass) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kD; ++e) acc[e] = 0.f;
    const int32_t u0 = a.causal ? 0 : -min(R, j / d);
    const int32_t u1 = min(R, (N - 1 - j) / d);
    sweep(dk_pass, u1 - u0 + 1, Qs, vk[wv], vv[wv], [&](int32_t x) {
      const int32_t i = j + (u0 + x) * d;
      return a.grank[i] >= 0 ? -1 : i;
    });
    if (jg) {
      const int32_t i0 = a.causal ? j : 0;
      sweep(dk_pass, N - i0, Qs, vk[wv], vv[wv], [&](int32_t x) {
        const int32_t i = i0 + x;
        return (in_band(i, j, R, d, a.causal) || a.grank[i] >= 0) ? -1 : i;
      });
    }
    if (!a.sep) sweep(dk_pass, a.n_global, Qs, vk[wv], vv[wv], grow);
  };
  shared_rows(false);
  a.dv[hoff + (size_t)j * kD + lane] = lane_totals(acc, lane);
  shared_rows(true);
  a.dk[hoff + (size_t)j * kD + lane] = lane_totals(acc, lane) * a.scale;
  if (a.sep) {  // the global rows, through qg_i, kg_j, vg_j
    const bf16* Qg = static_cast<const bf16*>(a.qg) + hoff;
#pragma unroll
    for (int e = 0; e < kD; ++e) acc[e] = 0.f;
    sweep(false, a.n_global, Qg, vkg[wv], vvg[wv], grow);
    a.dvg[hoff + (size_t)j * kD + lane] = lane_totals(acc, lane);
#pragma unroll
    for (int e = 0; e < kD; ++e) acc[e] = 0.f;
    sweep(true, a.n_global, Qg, vkg[wv], vvg[wv], grow);
    a.dkg[hoff + (size_t)j * kD + lane] = lane_totals(acc, lane) * a.scale;
  }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a, int32_t dtype, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (rows <= 0) return hipSuccess;
  const dim3 g((uint32_t)((rows + kWavesBwd - 1) / kWavesBwd)), blk(64 * kWavesBwd);
  if (dtype == 1 && a.n_band_wg > 0) {
    // D_i, then dK/dV and dQ on MFMA in one launch (no global ranks needed)
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((uint32_t)delta_blocks(rows)), dim3(256), 0, stream, a);
    hipError_t e = launch_rowtab(a, stream);  // key-side label vectors: the rows' tables
    if (e != hipSuccess) return e;
    e = launch_bwd_mfma(a, stream);
    if (e != hipSuccess) return e;
    e = launch_glob_reduce(a, stream);  // the global tiles' partial sums
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  hipLaunchKernelGGL(bwd_flags_kernel, dim3((uint32_t)((a.N + 255) / 256)), dim3(256), 0, stream, a);
  if (dtype == 1) {
    hipLaunchKernelGGL(bwd_dq_rows_kernel, g, blk, 0, stream, a);
    hipLaunchKernelGGL(bwd_dkv_rows_kernel, g, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<float>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(bwd_dkv_kernel<float>, g, blk, 0, stream, a);
  }
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
