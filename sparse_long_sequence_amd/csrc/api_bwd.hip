// api_bwd.hip — the C ABI's backward calls declared in include/longattn.h
// (la_attn_backward, la_dilated_backward and their workspace sizes): argument
// checks, workspace layout and launches. No allocation, no synchronisation.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "bwd_kernels.h"
#include "entry.h"
#include "longattn.h"

namespace {

la_status fail(la_status s, const std::string& msg) { return la::set_error(s, msg.c_str()); }

using la::aligned16;
using la::align_up;
using la::check_dims;
using la::is_empty;
using la::kAlign;
using la::kDHead;

// The partial sums of the split global-row and global-key passes (bf16):
// dQ, dK and dV for host_glob_part_rows(N) rows per head.
size_t bwd_part_bytes(const la_dims* dims) {
  if (dims->dtype != LA_BF16) return 0;
  return align_up((size_t)3 * dims->B * dims->H * la::host_glob_part_rows(dims->N) * kDHead *
                  sizeof(float));
}

// Each row's label table for key-side label vectors (bf16): up to
// kMaxLabels fp32 entries per row.
size_t bwd_rowtab_bytes(const la_dims* dims) {
  if (dims->dtype != LA_BF16) return 0;
  return align_up((size_t)dims->B * dims->H * dims->N * la::kMaxLabels * sizeof(float));
}

}  // namespace

extern "C" {

size_t la_attn_backward_workspace_size(const la_dims* dims) {
  if (check_dims(dims, false) != LA_OK) return 0;
  // D_i per row, each position's global rank, the partial sums, the row tables
  return align_up((size_t)dims->B * dims->H * dims->N * sizeof(float)) +
         align_up((size_t)dims->N * sizeof(int32_t)) + bwd_part_bytes(dims) +
         bwd_rowtab_bytes(dims);
}

la_status la_attn_backward(const la_dims* dims, const void* q, const void* k, const void* v,
                           const int32_t* global_idx, int32_t n_global, int32_t radius,
                           const int32_t* dilation, int32_t causal, const void* out,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           hipStream_t stream, const la_attn_bwd_ext* ext) {
  la_status st = check_dims(dims, false);
  if (st != LA_OK) return st;
  if (is_empty(dims)) return LA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
    return fail(LA_EINVAL, "q, k, v, out, lse, dout, dq, dk and dv are required");
  const void* ptrs[] = {q, k, v, out, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(LA_EINVAL, "tensors must be 16-byte aligned");
  if (n_global < 0 || n_global > dims->N) return fail(LA_EINVAL, "n_global must be in [0, N]");
  if ((n_global > 0) != (global_idx != nullptr))
    return fail(LA_EINVAL, "global_idx must be non-NULL exactly when n_global > 0");
  if (radius < 0) return fail(LA_EINVAL, "radius must be >= 0");
  if (causal != 0 && causal != 1) return fail(LA_EINVAL, "causal must be 0 or 1");
  if (dims->H > la::kMaxHeadsDil) return fail(LA_EUNSUPPORTED, "H above 64");
  la::BwdArgs a;
  memset(&a, 0, sizeof(a));
  for (int32_t h = 0; h < dims->H; ++h) {
    a.dil[h] = dilation ? dilation[h] : 1;
    if (a.dil[h] < 1) return fail(LA_EINVAL, "dilation entries must be >= 1");
  }
  if (!ext || !ext->workspace || ext->workspace_bytes < la_attn_backward_workspace_size(dims))
    return fail(LA_EINVAL, "workspace missing or smaller than la_attn_backward_workspace_size()");
  if (((uintptr_t)ext->workspace & (kAlign - 1)) != 0)
    return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  const bool sep_in = ext->qg || ext->kg || ext->vg;
  const bool sep_out = ext->dqg || ext->dkg || ext->dvg;
  if (sep_in || sep_out) {
    if (!(ext->qg && ext->kg && ext->vg && ext->dqg && ext->dkg && ext->dvg))
      return fail(LA_EINVAL, "qg, kg, vg and dqg, dkg, dvg: all six or none");
    const void* gp[] = {ext->qg, ext->kg, ext->vg, ext->dqg, ext->dkg, ext->dvg};
    for (const void* p : gp)
      if (!aligned16(p)) return fail(LA_EINVAL, "tensors must be 16-byte aligned");
  }
  if (ext->seg_ids && ((uintptr_t)ext->seg_ids & 3u) != 0)
    return fail(LA_EINVAL, "ext->seg_ids must be 4-byte aligned");
  // the forward's tables and structured inputs (the forward's checks)
  const int32_t rel_k = ext->rel_k;
  if ((ext->rel_bias || ext->rel_vec) && rel_k < 1)
    return fail(LA_EINVAL, "ext->rel_bias / ext->rel_vec need ext->rel_k >= 1");
  if (!ext->rel_bias && !ext->rel_vec && rel_k != 0)
    return fail(LA_EINVAL, "ext->rel_k set without ext->rel_bias or ext->rel_vec");
  if (ext->rel_vec && !aligned16(ext->rel_vec))
    return fail(LA_EINVAL, "ext->rel_vec must be 16-byte aligned");
  if (rel_k > la::kMaxRelK) return fail(LA_EUNSUPPORTED, "rel_k above 31");
  if (ext->n_labels < 0 || (ext->n_labels > 0 && ext->n_labels < 2 * rel_k + 1))
    return fail(LA_EINVAL, "ext->n_labels must be 0 or at least 2*rel_k+1");
  if (ext->n_labels > la::kMaxLabels) return fail(LA_EUNSUPPORTED, "more than 64 labels");
  if (ext->n_labels > 0 && !ext->rel_bias && !ext->rel_vec)
    return fail(LA_EINVAL, "ext->n_labels set without ext->rel_bias or ext->rel_vec");
  if ((ext->glabel || ext->llabel) && n_global == 0)
    return fail(LA_EINVAL, "label matrices need global tokens");
  if (ext->seg_pieces < 0 || ext->seg_pieces > 15)
    return fail(LA_EINVAL, "ext->seg_pieces must be in [0, 15]");
  if ((ext->glabel || ext->llabel) && (int64_t)n_global * dims->N > ((int64_t)1 << 31))
    return fail(LA_EUNSUPPORTED, "label matrices above 2^31 entries per batch row");
  a.rel_bias = ext->rel_bias;
  a.rel_vec = ext->rel_vec;
  a.glabel = ext->glabel;
  a.llabel = ext->llabel;
  a.rel_k = rel_k;
  a.n_labels = ext->n_labels > 0 ? ext->n_labels : 2 * rel_k + 1;
  a.seg_pieces = ext->seg_pieces == 0 ? 15 : ext->seg_pieces;
  a.q = q;
  a.k = k;
  a.v = v;
  a.qg = ext->qg;
  a.kg = ext->kg;
  a.vg = ext->vg;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.gidx = global_idx;
  a.seg = ext->seg_ids;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dqg = ext->dqg;
  a.dkg = ext->dkg;
  a.dvg = ext->dvg;
  a.delta = reinterpret_cast<float*>(ext->workspace);
  a.grank = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ext->workspace) +
                                       align_up((size_t)dims->B * dims->H * dims->N * sizeof(float)));
  a.n_global = n_global;
  a.B = dims->B;
  a.H = dims->H;
  a.N = dims->N;
  a.radius = radius;
  a.causal = causal;
  a.sep = sep_in ? 1 : 0;
  a.scale = (float)(1.0 / sqrt((double)kDHead));
  a.scale_log2 = (float)(1.0 / sqrt((double)kDHead) * 1.4426950408889634);
  a.glob_chunks = 1;
  // the MFMA path: every bf16 call
  if (dims->dtype == LA_BF16) {
    const int32_t tq = la::host_query_tile(dims->dtype);
    int32_t tiles = 0;
    for (int32_t h = 0; h < dims->H; ++h)
      tiles = std::max(tiles, la::host_band_tiles_of_head(dims->N, a.dil[h], tq));
    a.band_tiles_per_head = tiles;
    const int64_t band_wg = (int64_t)dims->B * dims->H * tiles;
    if (band_wg > 0x7fffffffLL) return fail(LA_EUNSUPPORTED, "launch grid too large");
    a.n_band_wg = (int32_t)band_wg;
    a.glob_chunks = la::host_glob_chunks((int64_t)dims->B * dims->H, dims->N, n_global);
    a.gpart = reinterpret_cast<float*>(reinterpret_cast<char*>(a.grank) +
                                       align_up((size_t)dims->N * sizeof(int32_t)));
    // row tables: with label vectors, and with a scalar table under label
    // matrices, piece masks or a wider vocabulary
    const bool lbl = a.glabel || a.llabel || (a.seg && a.seg_pieces != 15) ||
                     ((a.rel_bias || a.rel_vec) && a.n_labels != 2 * rel_k + 1);
    if (a.rel_vec || (lbl && a.rel_bias))
      a.rowtab = reinterpret_cast<float*>(reinterpret_cast<char*>(a.gpart) + bwd_part_bytes(dims));
  }
  hipError_t e = la::launch_attn_bwd(a, dims->dtype, stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return LA_OK;
}

size_t la_dilated_backward_workspace_size(const la_dims* dims) {
  if (check_dims(dims, true) != LA_OK) return 0;
  return align_up((size_t)dims->B * dims->H * dims->N * sizeof(float));
}

la_status la_dilated_backward(const la_dims* dims, const void* q, const void* k, const void* v,
                              const int32_t* seg_lens, const int32_t* dil_rates, int32_t n_pairs,
                              int32_t causal, const void* out, const float* lse, const void* dout,
                              float* dq, float* dk, float* dv, hipStream_t stream, void* workspace,
                              size_t workspace_bytes) {
  la_status st = check_dims(dims, true);
  if (st != LA_OK) return st;
  if (is_empty(dims)) return LA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
    return fail(LA_EINVAL, "q, k, v, out, lse, dout, dq, dk and dv are required");
  const void* ptrs[] = {q, k, v, out, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(LA_EINVAL, "tensors must be 16-byte aligned");
  if (!seg_lens || !dil_rates || n_pairs < 1)
    return fail(LA_EINVAL, "seg_lens, dil_rates and n_pairs >= 1 are required");
  if (n_pairs > la::kMaxPairs) return fail(LA_EUNSUPPORTED, "more than 16 patterns");
  if (causal != 0 && causal != 1) return fail(LA_EINVAL, "causal must be 0 or 1");
  la::BwdArgs a;
  memset(&a, 0, sizeof(a));
  for (int32_t p = 0; p < n_pairs; ++p) {
    if (seg_lens[p] < 1 || dil_rates[p] < 1)
      return fail(LA_EINVAL, "segment lengths and dilation rates must be >= 1");
    a.pw[p] = seg_lens[p];
    a.pr[p] = dil_rates[p];
  }
  if (!workspace || workspace_bytes < la_dilated_backward_workspace_size(dims))
    return fail(LA_EINVAL, "workspace missing or smaller than la_dilated_backward_workspace_size()");
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = reinterpret_cast<float*>(workspace);
  a.B = dims->B;
  a.H = dims->H;
  a.N = dims->N;
  a.causal = causal;
  a.n_pairs = n_pairs;
  a.scale = (float)(1.0 / sqrt((double)kDHead));
  a.scale_log2 = (float)(1.0 / sqrt((double)kDHead) * 1.4426950408889634);
  hipError_t e = la::launch_dilated_bwd(a, stream);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return LA_OK;
}

}  // extern "C"
