// bwd_kernels.h — the backward kernels' argument block and launchers, shared
// by the C ABI (api_bwd.hip) and the kernels.
#pragma once

#include "kernels.h"

namespace la {

// Backward of band + global attention (attn_bwd.hip). Tensors are [B,H,N,64];
// q, k, v, qg, kg, vg, out, dout in the call's dtype; gradients fp32.
struct BwdArgs {
  const void *q, *k, *v, *qg, *kg, *vg, *out, *dout;
  const float* lse;
  const int32_t* gidx;
  const int32_t* seg;
  float *dq, *dk, *dv, *dqg, *dkg, *dvg;
  float* delta;  // workspace: D_i = dO_i . O_i per row
  int32_t* grank;  // workspace: each position's index in global_idx, -1 if not global
  // the forward's bias tables and per-instance inputs (as in AttnArgs; tables
  // not differentiated): rel_bias [H][n_labels], rel_vec [H][n_labels][D]
  const float* rel_bias;
  const float* rel_vec;
  const uint8_t* glabel;
  const uint8_t* llabel;
  int32_t rel_k, n_labels, seg_pieces;  // seg_pieces: bits g2g 1, g2l 2, l2g 4, l2l 8
  int32_t n_global, B, H, N, radius, causal, sep;
  int32_t dil[kMaxHeadsDil];
  float scale;
  // MFMA backward (bf16 without tables, labels or segment ids): the forward's
  // residue-class tiles (of query rows for dQ, of keys for dK, dV)
  float scale_log2;
  int32_t band_tiles_per_head, n_band_wg;
  // the global rows' dQ and the global keys' dK, dV split over glob_chunks
  // key (row) ranges: fp32 partial sums [3][glob_chunks][B*H][n_gpad][D] in
  // the workspace (n_gpad: n_global rounded up to the query tile), added in
  // chunk order by a reduce launch; glob_chunks == 1 writes directly
  float* gpart;
  int32_t glob_chunks;
  // key-side label vectors on the MFMA path: each row's label table
  // [B*H*N][n_labels] (q . a_l plus the scalar bias over scale, in q.k units),
  // written by a launch before the MFMA one
  float* rowtab;
  // LongNet mixture (launch_dilated_bwd only): patterns (w, r)
  int32_t n_pairs;
  int32_t pw[kMaxPairs], pr[kMaxPairs];
};

constexpr int32_t kMaxGlobChunks = 16;  // key (row) ranges per global tile

hipError_t launch_attn_bwd(const BwdArgs& a, int32_t dtype, hipStream_t stream);
hipError_t launch_glob_reduce(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t stream);  // dK/dV and dQ, D_i given
hipError_t launch_rowtab(const BwdArgs& a, hipStream_t stream);    // a.rowtab from q, qg, rel_vec
hipError_t launch_dilated_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_dilated_bwd_mfma(const BwdArgs& a, hipStream_t stream);
int32_t host_glob_part_rows(int32_t N);  // partial-sum rows per head in the workspace
int32_t host_glob_chunks(int64_t bh, int32_t N, int32_t n_global);

}  // namespace la
