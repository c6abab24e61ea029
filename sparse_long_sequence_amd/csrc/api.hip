// api.hip — the C ABI declared in include/longattn.h: argument checks,
// workspace sizing and launches. No allocation, no host synchronisation
// (except la_check_global_idx, a synchronous test helper).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "entry.h"
#include "kernels.h"
#include "longattn.h"

namespace {

thread_local std::string g_err;

la_status fail(la_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

using la::aligned16;
using la::align_up;
using la::is_empty;
using la::kAlign;
using la::kDHead;
constexpr int32_t kMaxN = 1 << 24;
// Keys per global-row partial: at least 8 chunks per row when that leaves a
// whole key tile each (short sequences spread their global rows over several
// workgroups), at most 10 key tiles.
constexpr int32_t kChunkMax = 640;

}  // namespace

namespace la {

la_status check_dims(const la_dims* d, bool need_bf16) {
  if (!d) return fail(LA_EINVAL, "dims is NULL");
  if (d->B < 0 || d->H < 0 || d->N < 0 || d->D < 1)
    return fail(LA_EINVAL, "dims must be non-negative (B, H, N) and D positive");
  if (d->dtype != LA_F32 && d->dtype != LA_BF16) return fail(LA_EINVAL, "unknown dtype");
  if (d->D != kDHead) return fail(LA_EUNSUPPORTED, "only D == 64 is built");
  if (need_bf16 && d->dtype != LA_BF16) return fail(LA_EUNSUPPORTED, "this call is built for bf16 only");
  const int64_t total = (int64_t)d->B * d->H * d->N;
  if (total > (int64_t)1 << 31) return fail(LA_EUNSUPPORTED, "B*H*N above 2^31 rows");
  // bf16 tiles are addressed with 32-bit byte offsets within a head (N * 128 B)
  // and the LongNet index arithmetic divides positions in fp32
  if (d->N >= kMaxN) return fail(LA_EUNSUPPORTED, "N must be below 2^24");
  return LA_OK;
}

}  // namespace la

namespace {

using la::check_dims;

// A fresh token per band + global call: a quiet-NaN bit pattern (payload
// 1 .. 2^22 - 1), which no fp32 partial or lse ever holds, so counter words
// left by earlier calls (or partial data at the same offset) never match it.
uint32_t next_token() {
  static std::atomic<uint32_t> seq{0};
  const uint32_t n = seq.fetch_add(1, std::memory_order_relaxed);
  return 0x7FC00000u | (1u + n % 0x3FFFFFu);
}

int32_t chunk_len_of(int32_t N) {
  const int32_t c = ((N + 7) / 8 + 63) / 64 * 64;
  return std::min(kChunkMax, std::max(64, c));
}
int32_t n_chunks_of(int32_t N) { return (N + chunk_len_of(N) - 1) / chunk_len_of(N); }

// Workspace of la_attn_forward: global-row partials, fp32 O then fp32 lse,
// then one 64-bit arrival counter word per tile of global rows (tagged with
// the call's token; no initialisation needed).
struct AttnWs {
  size_t o_off, lse_off, cnt_off, bytes;
};

AttnWs attn_ws_layout(const la_dims* d, int32_t n_global) {
  AttnWs w = {0, 0, 0, 0};
  if (n_global <= 0) return w;
  const size_t parts = (size_t)d->B * d->H * n_global * n_chunks_of(d->N);
  const int32_t tq = la::host_query_tile(d->dtype);
  const size_t tiles = (size_t)d->B * d->H * ((n_global + tq - 1) / tq);
  w.lse_off = align_up(parts * kDHead * sizeof(float));
  w.cnt_off = w.lse_off + align_up(parts * sizeof(float));
  w.bytes = w.cnt_off + align_up(tiles * sizeof(uint64_t));
  return w;
}

size_t attn_ws_bytes(const la_dims* d, int32_t n_global) { return attn_ws_layout(d, n_global).bytes; }

struct DilPlan {
  la::DilArgs a;
  size_t ws_bytes;
};

// kind / sum_c: per pattern (null: every pattern dilated, kind 0); see DilArgs.
la_status plan_dilated(const la_dims* d, const int32_t* w, const int32_t* r, int32_t n_pairs,
                       DilPlan& p, const int32_t* kind = nullptr,
                       const int32_t* sum_c = nullptr) {
  if (!w || !r) return fail(LA_EINVAL, "seg_lens and dil_rates are required");
  if (n_pairs < 1) return fail(LA_EINVAL, "n_pairs must be >= 1");
  if (n_pairs > la::kMaxPairs) return fail(LA_EUNSUPPORTED, "more than 16 (w, r) pairs");
  memset(&p.a, 0, sizeof(p.a));
  la::DilArgs& a = p.a;
  a.B = d->B;
  a.H = d->H;
  a.N = d->N;
  a.n_pairs = n_pairs;
  a.fin = -1;
  for (int32_t k = 0; k < n_pairs; ++k) {
    if (w[k] < 1 || r[k] < 1) return fail(LA_EINVAL, "every w and r must be >= 1");
    a.kind[k] = kind ? kind[k] : 0;
    a.sum_c[k] = sum_c ? sum_c[k] : 0;
    if (r[k] == 1 && a.kind[k] == 0 && a.fin < 0) a.fin = k;
  }
  int64_t rows = 0;
  for (int32_t k = 0; k < n_pairs; ++k) {
    a.w[k] = w[k];
    a.r[k] = r[k];
    a.inv_w[k] = 1.0f / (float)w[k];
    a.inv_r[k] = 1.0f / (float)r[k];
    a.nseg[k] = (d->N + w[k] - 1) / w[k];
    a.seg_rows[k] = (w[k] + r[k] - 1) / r[k];
    a.qtiles[k] = (a.seg_rows[k] + la::kDilatedQueryTile - 1) / la::kDilatedQueryTile;
    a.row_off[k] = rows;
    if (k != a.fin) rows += (int64_t)d->B * d->H * a.nseg[k] * a.seg_rows[k];
  }
  a.rows_total = rows;
  // Workgroups of the pair launch (every pattern but the finisher) in
  // decreasing query-tile index (the key tiles of a workgroup grow with it),
  // across all patterns, so that the longest start first. With the patterns
  // sorted by qtiles, the levels split into bands over which the set of
  // patterns having that tile index is fixed.
  std::vector<int32_t> ord;
  for (int32_t k = 0; k < n_pairs; ++k)
    if (k != a.fin) ord.push_back(k);
  const int32_t np = (int32_t)ord.size();
  a.n_part = np;
  std::stable_sort(ord.begin(), ord.end(),
                   [&](int32_t x, int32_t y) { return a.qtiles[x] > a.qtiles[y]; });
  a.pre[0] = 0;
  for (int32_t i = 0; i < np; ++i) {
    a.order[i] = ord[i];
    a.pre[i + 1] = a.pre[i] + (int64_t)d->B * d->H * a.nseg[ord[i]];
  }
  int64_t wg = 0;
  for (int32_t j = 0; j < np; ++j) {
    const int32_t lo = j + 1 < np ? a.qtiles[ord[j + 1]] : 0;
    a.band_top[j] = a.qtiles[ord[j]] - 1;
    a.band_per[j] = a.pre[j + 1];
    a.band_start[j] = wg;
    wg += (int64_t)(a.qtiles[ord[j]] - lo) * a.band_per[j];
  }
  a.band_start[np] = wg;
  if (wg > 0x7fffffffLL) return fail(LA_EUNSUPPORTED, "launch grid too large");
  if (a.fin >= 0 &&
      (int64_t)d->B * d->H * a.nseg[a.fin] * a.qtiles[a.fin] > 0x7fffffffLL)
    return fail(LA_EUNSUPPORTED, "launch grid too large");
  // (a call whose only pattern is the finisher needs no workspace)
  p.ws_bytes = rows == 0 ? 0
                         : align_up((size_t)rows * kDHead * sizeof(float)) +
                               align_up((size_t)rows * sizeof(float));
  return LA_OK;
}

}  // namespace

extern "C" {

int32_t la_version(void) { return 2; }

const char* la_last_error(void) { return g_err.c_str(); }

size_t la_attn_workspace_size(const la_dims* dims, int32_t n_global, int32_t has_separate_global) {
  (void)has_separate_global;
  if (check_dims(dims, false) != LA_OK || n_global < 0 || n_global > dims->N) return 0;
  return attn_ws_bytes(dims, n_global);
}

size_t la_dilated_workspace_size(const la_dims* dims, const int32_t* seg_lens,
                                 const int32_t* dil_rates, int32_t n_pairs) {
  if (check_dims(dims, true) != LA_OK) return 0;
  DilPlan p;
  if (plan_dilated(dims, seg_lens, dil_rates, n_pairs, p) != LA_OK) return 0;
  return p.ws_bytes;
}

}  // extern "C"

namespace la {

// la_attn_forward with its workspace given apart from ext (ext->workspace is
// not read): the caller's buffer, or the allocation-free entry point's
// device scratch. ws_limit > 0 caps the workspace a call may need.
la_status attn_forward_ws(const la_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* global_idx, int32_t n_global, int32_t radius,
                          const int32_t* dilation, int32_t causal, const float* rel_bias,
                          void* out, float* lse, hipStream_t stream, const la_attn_ext* ext,
                          WorkspaceSource src) {
  la_status st = check_dims(dims, false);
  if (st != LA_OK) return st;
  if (is_empty(dims)) return LA_OK;  // nothing to compute
  if (!q || !k || !v || !out) return fail(LA_EINVAL, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(LA_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (n_global < 0 || n_global > dims->N) return fail(LA_EINVAL, "n_global must be in [0, N]");
  if ((n_global > 0) != (global_idx != nullptr))
    return fail(LA_EINVAL, "global_idx must be non-NULL exactly when n_global > 0");
  if (radius < 0) return fail(LA_EINVAL, "radius must be >= 0");
  if (causal != 0 && causal != 1) return fail(LA_EINVAL, "causal must be 0 or 1");
  la::AttnArgs a;
  memset(&a, 0, sizeof(a));
  if (dilation) {
    for (int32_t h = 0; h < dims->H; ++h)
      if (dilation[h] < 1) return fail(LA_EINVAL, "dilation entries must be >= 1");
  }
  if (dims->H > la::kMaxHeadsDil) return fail(LA_EUNSUPPORTED, "H above 64");
  for (int32_t h = 0; h < dims->H; ++h) a.dil[h] = dilation ? dilation[h] : 1;
  const int32_t rel_k = ext ? ext->rel_k : 0;
  const float* rel_vec = ext ? ext->rel_vec : nullptr;
  if ((rel_bias || rel_vec) && rel_k < 1)
    return fail(LA_EINVAL, "rel_bias / ext->rel_vec need ext->rel_k >= 1");
  if (!rel_bias && !rel_vec && rel_k != 0)
    return fail(LA_EINVAL, "ext->rel_k set without rel_bias or ext->rel_vec");
  if (rel_vec && !aligned16(rel_vec)) return fail(LA_EINVAL, "ext->rel_vec must be 16-byte aligned");
  const int32_t* seg_ids = ext ? ext->seg_ids : nullptr;
  if (seg_ids && ((uintptr_t)seg_ids & 3u) != 0)
    return fail(LA_EINVAL, "ext->seg_ids must be 4-byte aligned");
  if (rel_k > la::kMaxRelK) return fail(LA_EUNSUPPORTED, "rel_k above 31");
  const uint8_t* glabel = ext ? ext->glabel : nullptr;
  const uint8_t* llabel = ext ? ext->llabel : nullptr;
  const int32_t n_labels = ext ? ext->n_labels : 0;
  const int32_t seg_pieces = ext ? ext->seg_pieces : 0;
  if (n_labels < 0 || (n_labels > 0 && n_labels < 2 * rel_k + 1))
    return fail(LA_EINVAL, "ext->n_labels must be 0 or at least 2*rel_k+1");
  if (n_labels > la::kMaxLabels) return fail(LA_EUNSUPPORTED, "more than 64 labels");
  if (n_labels > 0 && !rel_bias && !rel_vec)
    return fail(LA_EINVAL, "ext->n_labels set without rel_bias or ext->rel_vec");
  if ((glabel || llabel) && n_global == 0)
    return fail(LA_EINVAL, "label matrices need global tokens");
  if (seg_pieces < 0 || seg_pieces > 15) return fail(LA_EINVAL, "ext->seg_pieces must be in [0, 15]");
  if (glabel || llabel) {
    // the label matrices are addressed with 32-bit offsets per batch row
    if ((int64_t)n_global * dims->N > ((int64_t)1 << 31))
      return fail(LA_EUNSUPPORTED, "label matrices above 2^31 entries per batch row");
  }
  const void *qg = q, *kg = k, *vg = v;
  if (ext && (ext->qg || ext->kg || ext->vg)) {
    if (!(ext->qg && ext->kg && ext->vg)) return fail(LA_EINVAL, "qg, kg, vg: all three or none");
    if (!aligned16(ext->qg) || !aligned16(ext->kg) || !aligned16(ext->vg))
      return fail(LA_EINVAL, "qg, kg, vg must be 16-byte aligned");
    qg = ext->qg;
    kg = ext->kg;
    vg = ext->vg;
  }
  const size_t need = attn_ws_bytes(dims, n_global);
  void* ws = nullptr;
  if (need > 0) {
    if (src.fixed_bytes > 0) {
      if (need > src.fixed_bytes)
        return fail(LA_EUNSUPPORTED, "this call needs " + std::to_string(need) +
                                         " bytes of scratch, above the " +
                                         std::to_string(src.fixed_bytes) +
                                         " bytes the allocation-free entry point holds");
      ws = src.get();
      if (!ws) return fail(LA_EHIP, std::string("device scratch unavailable: ") + g_err);
    } else {
      if (!ext || !ext->workspace || ext->workspace_bytes < need)
        return fail(LA_EINVAL, "workspace missing or smaller than la_attn_workspace_size()");
      ws = ext->workspace;
    }
    if (((uintptr_t)ws & (kAlign - 1)) != 0)
      return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  }

  a.q = q;
  a.k = k;
  a.v = v;
  a.qg = qg;
  a.kg = kg;
  a.vg = vg;
  a.gidx = global_idx;
  a.n_global = n_global;
  a.B = dims->B;
  a.H = dims->H;
  a.N = dims->N;
  a.radius = radius;
  a.causal = causal;
  a.rel_bias = rel_bias;
  a.rel_vec = rel_vec;
  a.seg = seg_ids;
  a.glabel = glabel;
  a.llabel = llabel;
  a.n_labels = n_labels > 0 ? n_labels : 2 * rel_k + 1;
  a.seg_pieces = seg_pieces == 0 ? 15 : seg_pieces;
  a.rel_k = rel_k;
  a.out = out;
  a.lse = lse;
  if (need > 0) {
    const AttnWs lay = attn_ws_layout(dims, n_global);
    char* base = reinterpret_cast<char*>(ws);
    a.ws_o = reinterpret_cast<float*>(base + lay.o_off);
    a.ws_lse = reinterpret_cast<float*>(base + lay.lse_off);
    a.ws_cnt = reinterpret_cast<uint64_t*>(base + lay.cnt_off);
    a.token = next_token();
    // partials are addressed with 32-bit byte offsets
    if (lay.cnt_off > (size_t)0x7fffffff) return fail(LA_EUNSUPPORTED, "global-row partials above 2 GiB");
  }
  a.chunk_len = chunk_len_of(dims->N);
  a.n_chunks = n_chunks_of(dims->N);
  const int32_t tq = la::host_query_tile(dims->dtype);
  int32_t tiles = 0;
  for (int32_t h = 0; h < dims->H; ++h)
    tiles = std::max(tiles, la::host_band_tiles_of_head(dims->N, a.dil[h], tq));
  a.band_tiles_per_head = tiles;
  const int64_t band_wg = (int64_t)dims->B * dims->H * tiles;
  a.n_gq_tiles = (n_global + tq - 1) / tq;
  const int64_t glob_wg = (int64_t)dims->B * dims->H * a.n_gq_tiles * a.n_chunks;
  if (band_wg + glob_wg > 0x7fffffffLL) return fail(LA_EUNSUPPORTED, "launch grid too large");
  a.n_band_wg = (int32_t)band_wg;
  a.n_glob_wg = (int32_t)glob_wg;
  a.scale_log2 = (float)(1.0 / sqrt((double)kDHead) * 1.4426950408889634);
  hipError_t e = la::launch_attn(a, dims->dtype, stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return LA_OK;
}

la_status set_error(la_status s, const char* msg) { return fail(s, msg); }

}  // namespace la

extern "C" {

la_status la_attn_forward(const la_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* global_idx, int32_t n_global, int32_t radius,
                          const int32_t* dilation, int32_t causal, const float* rel_bias,
                          void* out, float* lse, hipStream_t stream, const la_attn_ext* ext) {
  return la::attn_forward_ws(dims, q, k, v, global_idx, n_global, radius, dilation, causal,
                             rel_bias, out, lse, stream, ext, la::WorkspaceSource{});
}

la_status la_dilated_forward(const la_dims* dims, const void* q, const void* k, const void* v,
                             const int32_t* seg_lens, const int32_t* dil_rates, int32_t n_pairs,
                             int32_t causal, void* out, hipStream_t stream,
                             const la_dilated_ext* ext) {
  la_status st = check_dims(dims, true);
  if (st != LA_OK) return st;
  if (n_pairs < 1) return fail(LA_EINVAL, "n_pairs must be >= 1");
  if (is_empty(dims)) return LA_OK;  // nothing to compute
  if (!q || !k || !v || !out) return fail(LA_EINVAL, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(LA_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (causal != 0 && causal != 1) return fail(LA_EINVAL, "causal must be 0 or 1");
  DilPlan p;
  st = plan_dilated(dims, seg_lens, dil_rates, n_pairs, p);
  if (st != LA_OK) return st;
  if (p.ws_bytes > 0) {
    if (!ext || !ext->workspace || ext->workspace_bytes < p.ws_bytes)
      return fail(LA_EINVAL, "workspace missing or smaller than la_dilated_workspace_size()");
    if (((uintptr_t)ext->workspace & (kAlign - 1)) != 0)
      return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  }
  la::DilArgs& a = p.a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.causal = causal;
  a.out = out;
  a.lse = ext ? ext->lse : nullptr;
  if (p.ws_bytes > 0) {
    a.ws_o = reinterpret_cast<float*>(ext->workspace);
    a.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(ext->workspace) +
                                        align_up((size_t)a.rows_total * kDHead * sizeof(float)));
  }
  a.scale_log2 = (float)(1.0 / sqrt((double)kDHead) * 1.4426950408889634);
  hipError_t e = la::launch_dilated(a, stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return LA_OK;
}

// Sparse Transformer fixed pattern: the causal (or full) local block as a
// dilated pattern (w = l, r = 1), which finishes and mixes, and the strided
// summary keys as a second pattern of kind 1. The two key sets of a row are
// disjoint, so mixing them by their softmax denominators is one softmax over
// their union.
static la_status plan_fixed(const la_dims* dims, int32_t l, int32_t c, DilPlan& p) {
  if (l < 1 || c < 1 || c > l) return fail(LA_EINVAL, "need 1 <= summary_len <= block_len");
  if (c % 64 != 0) return fail(LA_EUNSUPPORTED, "summary_len must be a multiple of 64");
  if (dims->N % l != 0) return fail(LA_EUNSUPPORTED, "N must be a multiple of block_len");
  const int32_t w[2] = {l, l}, r[2] = {1, 1}, kind[2] = {0, 1}, cs[2] = {0, c};
  return plan_dilated(dims, w, r, 2, p, kind, cs);
}

size_t la_fixed_workspace_size(const la_dims* dims, int32_t block_len, int32_t summary_len) {
  if (check_dims(dims, true) != LA_OK) return 0;
  DilPlan p;
  if (plan_fixed(dims, block_len, summary_len, p) != LA_OK) return 0;
  return p.ws_bytes;
}

la_status la_fixed_forward(const la_dims* dims, const void* q, const void* k, const void* v,
                           int32_t block_len, int32_t summary_len, int32_t causal, void* out,
                           hipStream_t stream, const la_dilated_ext* ext) {
  la_status st = check_dims(dims, true);
  if (st != LA_OK) return st;
  if (is_empty(dims)) return LA_OK;
  if (!q || !k || !v || !out) return fail(LA_EINVAL, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(LA_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (causal != 0 && causal != 1) return fail(LA_EINVAL, "causal must be 0 or 1");
  DilPlan p;
  st = plan_fixed(dims, block_len, summary_len, p);
  if (st != LA_OK) return st;
  if (p.ws_bytes > 0) {
    if (!ext || !ext->workspace || ext->workspace_bytes < p.ws_bytes)
      return fail(LA_EINVAL, "workspace missing or smaller than la_fixed_workspace_size()");
    if (((uintptr_t)ext->workspace & (kAlign - 1)) != 0)
      return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  }
  la::DilArgs& a = p.a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.causal = causal;
  a.out = out;
  a.lse = ext ? ext->lse : nullptr;
  if (p.ws_bytes > 0) {
    a.ws_o = reinterpret_cast<float*>(ext->workspace);
    a.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(ext->workspace) +
                                        align_up((size_t)a.rows_total * kDHead * sizeof(float)));
  }
  a.scale_log2 = (float)(1.0 / sqrt((double)kDHead) * 1.4426950408889634);
  hipError_t e = la::launch_dilated(a, stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return LA_OK;
}

la_status la_check_global_idx(const int32_t* global_idx, int32_t n_global, int32_t N,
                              hipStream_t stream) {
  if (n_global < 0 || n_global > N) return fail(LA_EINVAL, "n_global must be in [0, N]");
  if (n_global == 0) return global_idx ? fail(LA_EINVAL, "global_idx given with n_global == 0") : LA_OK;
  if (!global_idx) return fail(LA_EINVAL, "global_idx is NULL");
  std::vector<int32_t> h(n_global);
  hipError_t e = hipMemcpyAsync(h.data(), global_idx, sizeof(int32_t) * n_global,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("copy failed: ") + hipGetErrorString(e));
  for (int32_t i = 0; i < n_global; ++i) {
    if (h[i] < 0 || h[i] >= N) return fail(LA_EINVAL, "global_idx entry outside [0, N)");
    if (i > 0 && h[i] <= h[i - 1]) return fail(LA_EINVAL, "global_idx not strictly increasing");
  }
  return LA_OK;
}

}  // extern "C"
