// dilated_fwd.hip — LongNet dilated attention on gfx950.
//
// For each (segment length w, dilation r) pattern and head h, every segment of
// w positions keeps the rows whose offset from the segment start is congruent
// to h mod r (LongNet page, §3.4 "Dilated Attention: Core Mechanism", Eqs. 3-5,
// and "Multi-Head Dilated Attention: Offset Mechanism", Eqs. 13-15). Those rows
// are read straight from Q, K, V as a strided view (row stride r*D): no gather
// copy is made. Dense attention runs among them (Eq. 6), causal in position
// when requested, and each pattern writes a partial (normalised O, lse) per
// kept row. A row's output is the sum of the partials of the patterns that
// kept it, weighted by exp(lse_k), i.e. by the softmax denominators (Eqs.
// 7-10, "Mixture of Dilated Attentions"); rows a pattern skipped receive
// nothing from it. When a pattern has dilation 1 it keeps every row: it runs
// last, in a launch of its own, and its workgroups mix the other patterns'
// partials into their rows. Otherwise a combine launch scatters and mixes.
#include "tile_core.h"
#include "kernels.h"

namespace la {

// One query tile (128 kept rows from t0) of pattern k, segment seg, head bh:
// dense attention (causal in position when requested) among the segment's
// kept rows, run through the tile engine. Leaves each wave's running state in
// wv; returns false if the tile holds no row.
struct DilTile {
  int32_t base, r, t0, qcount, qi, qpos;
};

__device__ __forceinline__ bool dilated_tile(const DilArgs& a, TileTraits<bf16>::Smem& sm,
                                             TileTraits<bf16>::Wave& wv, int32_t k, int32_t seg,
                                             int32_t bh, int32_t qt, DilTile& dt) {
  using TT = TileTraits<bf16>;
  constexpr int32_t kTQ = TT::kTQ;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t w = a.w[k], r = a.r[k];
  const int32_t h = bh % a.H;
  const int32_t sigma = seg * w;
  const int32_t L = min(w, a.N - sigma);
  const int32_t s = h % r;
  const int32_t n_rows = L > s ? (L - s + r - 1) / r : 0;
  const int32_t t0 = qt * kTQ;
  if (t0 >= n_rows) return false;
  const int32_t qcount = min(kTQ, n_rows - t0);
  const size_t head_elems = (size_t)a.N * kD;
  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + bh * head_elems;
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + bh * head_elems;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + bh * head_elems;
  const int32_t base = sigma + s;
  const int32_t qi = TT::qrow(wave, lane, 0);
  const int32_t qpos = base + r * (t0 + min(qi, qcount - 1));
  const bool dead = TT::kQW * wave >= qcount;  // no valid row in this wave
  TT::load_q(wv, qb, &qpos, lane);
  const BiasRule br = {nullptr, 0, 0, 0};
  const GlobInfo gi = {kGlobNone, nullptr, 0};
  const LabelRule nolab = {};
  if (a.kind[k] == 1) {
    // Fixed pattern, strided part (LongNet page, §3.4 "Standard Self-Attention
    // and Sparse Attention (Preliminaries)"): the c summary positions at block
    // offsets [toff, toff + c) of every other block (causal: every earlier
    // block). c is a multiple of 64, so a key tile is one contiguous run, and
    // every pair of it is allowed.
    const int32_t c = a.sum_c[k];
    const int32_t hp = h % max(1, w / c);
    const int32_t toff = w - c * (hp + 1);
    const int32_t n_keys = (a.causal ? seg : a.nseg[k] - 1) * c;
    auto desc_sum = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
      const int32_t x0 = n * kTK;
      const int32_t kb = x0 / c;
      const int32_t blk = (a.causal || kb < seg) ? kb : kb + 1;  // the blocks other than seg
      kt = {nullptr, blk * w + toff + (x0 - kb * c), 1, kTK, 0, kGlobNone};
      mr = {kRange, 0, 0, 0, -kFar, kFar, 0, 0, 1};
    };
    run_tiles<bf16, false, false, false, false>(sm, wv, kb, vb, n_keys / kTK, desc_sum, br, gi,
                                                nolab, qi, qpos, dead, a.scale_log2);
  } else {
    const int32_t hi = a.causal ? t0 + qcount - 1 : n_rows - 1;
    const int32_t n_tiles = (hi + kTK) / kTK;
    auto desc = [&](int32_t n, KeyTile& kt, MaskRule& mr) {
      const int32_t u0 = n * kTK;
      const int32_t kcount = min(kTK, hi - u0 + 1);
      kt = {nullptr, base + r * u0, r, kcount, 0, kGlobNone};
      // gathered index difference key - query = kj - qi - (t0 - u0) <= 0 when causal
      const bool full = kcount == kTK && (!a.causal || u0 + kTK - 1 <= t0);
      mr = {kRange, full ? 0 : 1, 0, t0 - u0, -kFar, a.causal ? 0 : kFar, 0, 0, 1};
    };
    run_tiles<bf16, false, false, false, false>(sm, wv, kb, vb, n_tiles, desc, br, gi, nolab, qi,
                                                qpos, dead, a.scale_log2);
  }
  dt = {base, r, t0, qcount, qi, qpos};
  return true;
}

// Every pattern but the finisher: a partial (normalised O, lse) per kept row.
__global__ __launch_bounds__(TileTraits<bf16>::kThreads)
__attribute__((amdgpu_waves_per_eu(TileTraits<bf16>::kMinWavesPerEU)))
void dilated_pair_kernel(DilArgs a) {
  using TT = TileTraits<bf16>;
  __shared__ TT::Smem sm;
  const int32_t lane = threadIdx.x & 63;
  // Blocks in launch order (no XCD remap: that would give one XCD all the
  // longest workgroups): query-tile level descending across all patterns.
  const int64_t wg = blockIdx.x;
  if (wg >= a.band_start[a.n_part]) return;
  int32_t j = 0;
  while (j + 1 < a.n_part && wg >= a.band_start[j + 1]) ++j;
  const int64_t off = wg - a.band_start[j];
  const int32_t qt = a.band_top[j] - (int32_t)(off / a.band_per[j]);
  const int64_t rem = off % a.band_per[j];
  int32_t oi = 0;
  while (oi < j && rem >= a.pre[oi + 1]) ++oi;
  const int32_t k = a.order[oi];
  const int32_t nseg = a.nseg[k];
  const int64_t rest = rem - a.pre[oi];
  const int32_t seg = (int32_t)(rest % nseg);
  const int32_t bh = (int32_t)(rest / nseg);
  TT::Wave wv;
  DilTile dt;
  if (!dilated_tile(a, sm, wv, k, seg, bh, qt, dt)) return;
  const float l_tot = TT::row_sum(wv.l[0]);
  if (dt.qi < dt.qcount) {
    const int64_t prow = a.row_off[k] + ((int64_t)bh * nseg + seg) * a.seg_rows[k] + dt.t0 + dt.qi;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    TT::store_row_f32(a.ws_o + prow * kD, wv, 0, inv, lane);
    if (TT::row_leader(lane))
      a.ws_lse[prow] = l_tot > 0.f ? (wv.m[0] + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

// x / d for 0 <= x < 2^24 and d >= 1 with a precomputed fp32 1/d: the
// estimate is within 2 of the quotient, and two exact integer corrections
// fix it (integer division would be a long emulated sequence per lane).
__device__ __forceinline__ int32_t div_small(int32_t x, int32_t d, float inv_d) {
  int32_t q = (int32_t)((float)x * inv_d);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int32_t rem = x - q * d;
    q += rem < 0 ? -1 : (rem >= d ? 1 : 0);
  }
  return q;
}

// Scatter + mixture. 16 output rows per 256-thread block. First one thread
// per (row, pattern) finds whether the pattern covers the row, and if so its
// partial row and lse (into LDS); then 16 lanes per row, 4 consecutive d per
// lane (16-byte loads), read the covering partials and mix them (a running max
// keeps the sums bounded).
constexpr int32_t kCombineRows = 16;

__global__ __launch_bounds__(256) void dilated_combine_kernel(DilArgs a) {
  __shared__ int64_t s_prow[kCombineRows][kMaxPairs];
  __shared__ float s_lse[kCombineRows][kMaxPairs];
  const int32_t tid = threadIdx.x;
  const int64_t total = (int64_t)a.B * a.H * a.N;
  const int64_t row0 = (int64_t)blockIdx.x * kCombineRows;
  {
    const int32_t rr = tid >> 4, k = tid & 15;  // kMaxPairs == 16
    const int64_t row = row0 + rr;
    float lse = kNegInf;
    int64_t prow = 0;
    if (k < a.n_pairs && row < total) {
      const int32_t i = (int32_t)(row % a.N);
      const int32_t bh = (int32_t)(row / a.N);
      const int32_t h = bh % a.H;
      const int32_t w = a.w[k], r = a.r[k];
      const int32_t seg = div_small(i, w, a.inv_w[k]), off = i - seg * w;
      const int32_t m = div_small(off, r, a.inv_r[k]);       // off = m r + (off mod r)
      const int32_t hs = h - div_small(h, r, a.inv_r[k]) * r;  // h mod r
      // pattern k covers row i iff its offset in the segment is congruent to h mod r
      if (off - m * r == hs) {
        prow = a.row_off[k] + ((int64_t)bh * a.nseg[k] + seg) * a.seg_rows[k] + m;
        lse = a.ws_lse[prow];
      }
    }
    s_prow[rr][k] = prow;
    s_lse[rr][k] = lse;
  }
  __syncthreads();
  const int32_t rr = tid >> 4, d4 = 4 * (tid & 15);
  const int64_t row = row0 + rr;
  if (row >= total) return;
  float L = kNegInf;
  for (int32_t k = 0; k < a.n_pairs; ++k) L = fmaxf(L, s_lse[rr][k]);
  float S = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (L != kNegInf) {
    for (int32_t k = 0; k < a.n_pairs; ++k) {
      const float lk = s_lse[rr][k];
      if (lk == kNegInf) continue;  // not covering (or an empty partial)
      const float wgt = __expf(lk - L);
      S += wgt;
      acc += wgt * *reinterpret_cast<const f32x4*>(a.ws_o + s_prow[rr][k] * kD + d4);
    }
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  u32x2 pk;
  pk[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(a.out) + row * kD + d4) = pk;
  if (a.lse && d4 == 0) a.lse[row] = S > 0.f ? L + __logf(S) : kNegInf;
}

// The finisher pattern (dilation 1: it keeps every row of its segments),
// whose workgroups, after their own tile, mix the partials of the patterns
// that also cover their rows with weights exp(lse_k) (LongNet page, §3.4
// "Mixture of Dilated Attentions", Eqs. 7-10) and write the final rows. The
// pair launch before it has written every partial. Workgroups in decreasing
// query-tile index (the longest first).
__global__ __launch_bounds__(TileTraits<bf16>::kThreads)
__attribute__((amdgpu_waves_per_eu(TileTraits<bf16>::kMinWavesPerEU)))
void dilated_finish_kernel(DilArgs a) {
  using TT = TileTraits<bf16>;
  __shared__ TT::Smem sm;
  const int32_t lane = threadIdx.x & 63;
  const int32_t kf = a.fin;
  const int32_t nseg = a.nseg[kf];
  const int64_t per = (int64_t)a.B * a.H * nseg;
  const int64_t wg = blockIdx.x;
  if (wg >= per * a.qtiles[kf]) return;
  const int32_t qt = a.qtiles[kf] - 1 - (int32_t)(wg / per);
  const int64_t rest = wg % per;
  const int32_t seg = (int32_t)(rest % nseg);
  const int32_t bh = (int32_t)(rest / nseg);
  TT::Wave wv;
  DilTile dt;
  if (!dilated_tile(a, sm, wv, kf, seg, bh, qt, dt)) return;
  const bool valid = dt.qi < dt.qcount;
  const float l_tot = TT::row_sum(wv.l[0]);
  // running mixture: M = max lse, S = sum e^{lse - M}, wv.o = sum e^{lse - M} O
  float M = l_tot > 0.f ? (wv.m[0] + __log2f(l_tot)) * kLn2 : kNegInf;
  float S = M == kNegInf ? 0.f : 1.f;
  TT::scale_acc(wv, l_tot > 0.f ? 1.f / l_tot : 0.f);
  const int32_t i = dt.qpos;  // this lane's row position (the finisher keeps every row)
  const int32_t h = bh % a.H;
  const int32_t d0 = 4 * (lane >> 5);  // this lane holds d = 32db + 8j + d0 + [0, 4)
  for (int32_t k = 0; k < a.n_pairs; ++k) {
    if (k == kf) continue;
    const int32_t w = a.w[k], r = a.r[k];
    const int32_t sg = div_small(i, w, a.inv_w[k]), off = i - sg * w;
    const int32_t m = div_small(off, r, a.inv_r[k]);
    const int32_t hs = h - div_small(h, r, a.inv_r[k]) * r;  // h mod r
    // pattern k covers row i iff its offset in the segment is congruent to h mod r
    const bool cov = valid && off - m * r == hs;
    const int64_t prow = a.row_off[k] + ((int64_t)bh * a.nseg[k] + sg) * a.seg_rows[k] + m;
    const float lk = cov ? a.ws_lse[prow] : kNegInf;
    const bool use = lk != kNegInf;
    if (__ballot(use) == 0ull) continue;
    if (use) {
      const float Mn = fmaxf(M, lk);
      const float sc = M == kNegInf ? 0.f : __expf(M - Mn);
      const float wk = __expf(lk - Mn);
      const float* src = a.ws_o + prow * kD + d0;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(src + 32 * db + 8 * jj);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv.o[db][4 * jj + e] = wv.o[db][4 * jj + e] * sc + wk * x[e];
        }
      }
      S = S * sc + wk;
      M = Mn;
    }
  }
  if (valid) {
    const float inv = S > 0.f ? 1.f / S : 0.f;
    bf16* dst = reinterpret_cast<bf16*>(a.out) + ((size_t)bh * a.N + i) * kD;
    TT::store_row(dst, wv, 0, inv, lane);
    if (a.lse && TT::row_leader(lane))
      a.lse[(size_t)bh * a.N + i] = S > 0.f ? M + __logf(S) : kNegInf;
  }
}

static_assert(kMaxPairs == 16, "one thread per (row, pattern) in a 256-thread block");

hipError_t launch_dilated(const DilArgs& a, hipStream_t stream) {
  const int64_t grid = a.band_start[a.n_part];
  if (grid > 0) {
    hipLaunchKernelGGL(dilated_pair_kernel, dim3((uint32_t)grid), dim3(TileTraits<bf16>::kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.fin >= 0) {
    const int64_t g = (int64_t)a.B * a.H * a.nseg[a.fin] * a.qtiles[a.fin];
    hipLaunchKernelGGL(dilated_finish_kernel, dim3((uint32_t)g), dim3(TileTraits<bf16>::kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  hipLaunchKernelGGL(dilated_combine_kernel, dim3((uint32_t)((rows + kCombineRows - 1) / kCombineRows)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace la
