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
// Two launches, no atomics: a query-centric pass (one wave per row) writes
// D_i and dQ_i; a key-centric pass (one wave per key) visits every row that
// attends to its key and writes dK_j and dV_j in one store. Lane d of a wave
// holds element d of the 64-wide vectors; dot products are wave reductions.
// This is the plain first form of the backward: fp32 VALU work, no MFMA.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"
#include "tile_core.h"

namespace la {
namespace {

constexpr int kWavesBwd = 4;  // rows (or keys) per workgroup

__device__ __forceinline__ float load_el(const float* p) { return *p; }
__device__ __forceinline__ float load_el(const bf16* p) { return (float)*p; }

// Sum over the 64 lanes; every lane gets the same value.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
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

__device__ __forceinline__ bool is_global(const BwdArgs& a, int32_t p) {
  return a.n_global > 0 && sorted_contains(a.gidx, a.n_global, p);
}

// Row i's gradient dQ_i (query-centric), and D_i into the workspace.
template <typename T>
__global__ __launch_bounds__(64 * kWavesBwd) void bwd_dq_kernel(BwdArgs a) {
  const int32_t lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWavesBwd + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (row >= rows) return;
  const int32_t N = a.N;
  const int32_t i = (int32_t)(row % N);
  const int64_t bh = row / N;
  const int32_t h = (int32_t)(bh % a.H), b = (int32_t)(bh / a.H);
  const size_t hoff = (size_t)bh * N * kD;
  const bool ig = is_global(a, i);
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
  const int32_t si = segb ? segb[i] : 0;
  float acc = 0.f;
  auto visit = [&](int32_t j) {
    const float kv = load_el(K + (size_t)j * kD + lane);
    const float vv = load_el(V + (size_t)j * kD + lane);
    const float p = __expf(wave_sum(qv * kv) * a.scale - lse);
    const float dp = wave_sum(dov * vv);
    acc += p * (dp - Di) * kv;
  };
  if (lse != kNegInf) {  // a row without keys has no gradient
    if (ig) {  // a global row attends to every key (causal: up to itself)
      const int32_t last = a.causal ? i : N - 1;
      for (int32_t j = 0; j <= last; ++j)
        if (!segb || segb[j] == si) visit(j);
    } else {
      const int32_t d = a.dil[h], R = a.radius;
      // the window's keys inside [0, N): t in [t0, t1]
      const int32_t t0 = -min(R, i / d);
      const int32_t t1 = a.causal ? 0 : min(R, (N - 1 - i) / d);
      for (int32_t t = t0; t <= t1; ++t) {
        const int32_t j = i + t * d;
        if (!segb || segb[j] == si) visit(j);
      }
      // global keys outside the window (a global key in it was counted there)
      for (int32_t g = 0; g < a.n_global; ++g) {
        const int32_t j = a.gidx[g];
        if (j < 0 || j >= N || (a.causal && j > i) || in_band(i, j, R, d, a.causal)) continue;
        if (!segb || segb[j] == si) visit(j);
      }
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
  const int32_t sj = segb ? segb[j] : 0;
  const int32_t d = a.dil[h], R = a.radius;
  const bool jg = is_global(a, j);

  // one (row, key) pair through projections (Q, K, V) into (dk, dv)
  auto pair = [&](const T* Q, float kv, float vv, int32_t i, float& dk, float& dv) {
    const float li = lse[i];
    if (li == kNegInf) return;
    const float qv = load_el(Q + (size_t)i * kD + lane);
    const float dov = load_el(dO + (size_t)i * kD + lane);
    const float p = __expf(wave_sum(qv * kv) * a.scale - li);
    const float dp = wave_sum(dov * vv);
    dv += p * dov;
    dk += p * (dp - delta[i]) * qv;
  };

  const T* Qs = static_cast<const T*>(a.q) + hoff;
  const float kv = load_el(static_cast<const T*>(a.k) + hoff + (size_t)j * kD + lane);
  const float vv = load_el(static_cast<const T*>(a.v) + hoff + (size_t)j * kD + lane);
  float dk = 0.f, dv = 0.f;
  // non-global rows whose window holds j: i = j + u * d, causal u >= 0
  {
    const int32_t u0 = a.causal ? 0 : -min(R, j / d);
    const int32_t u1 = min(R, (N - 1 - j) / d);
    for (int32_t u = u0; u <= u1; ++u) {
      const int32_t i = j + u * d;
      if (is_global(a, i) || (segb && segb[i] != sj)) continue;
      pair(Qs, kv, vv, i, dk, dv);
    }
  }
  // a global key: every other non-global row (causal: from j on)
  if (jg) {
    for (int32_t i = a.causal ? j : 0; i < N; ++i) {
      if (in_band(i, j, R, d, a.causal) || is_global(a, i) || (segb && segb[i] != sj)) continue;
      pair(Qs, kv, vv, i, dk, dv);
    }
  }
  // global rows attend to every key (causal: rows from j on)
  if (!a.sep) {
    for (int32_t g = 0; g < a.n_global; ++g) {
      const int32_t i = a.gidx[g];
      if (i < 0 || i >= N || (a.causal && i < j) || (segb && segb[i] != sj)) continue;
      pair(Qs, kv, vv, i, dk, dv);
    }
  } else {
    const T* Qg = static_cast<const T*>(a.qg) + hoff;
    const float kgv = load_el(static_cast<const T*>(a.kg) + hoff + (size_t)j * kD + lane);
    const float vgv = load_el(static_cast<const T*>(a.vg) + hoff + (size_t)j * kD + lane);
    float dkg = 0.f, dvg = 0.f;
    for (int32_t g = 0; g < a.n_global; ++g) {
      const int32_t i = a.gidx[g];
      if (i < 0 || i >= N || (a.causal && i < j) || (segb && segb[i] != sj)) continue;
      pair(Qg, kgv, vgv, i, dkg, dvg);
    }
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
    hipLaunchKernelGGL(bwd_dq_kernel<bf16>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(bwd_dkv_kernel<bf16>, g, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<float>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(bwd_dkv_kernel<float>, g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace la
