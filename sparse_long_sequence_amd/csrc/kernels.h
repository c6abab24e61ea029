// kernels.h — the forward kernels' argument blocks and launchers, shared by the
// C ABI and the kernels (the backward's are in bwd_kernels.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int32_t kMaxHeadsDil = 64;  // per-head dilation table size
constexpr int32_t kMaxPairs = 16;     // LongNet patterns per call
constexpr int32_t kMaxRelK = 31;      // 2k+1 <= 63 bias entries per head
constexpr int32_t kMaxLabels = 64;    // label vocabulary (distance + structural) per head
constexpr int32_t kLabelDistance = 0xFE;  // per-pair label: the pair's usual clipped-distance label

struct AttnArgs {
  const void *q, *k, *v;
  const void *qg, *kg, *vg;  // the global rows' projections (== q, k, v when shared)
  const int32_t* gidx;
  int32_t n_global;
  int32_t B, H, N;
  int32_t radius, causal;
  int32_t dil[kMaxHeadsDil];
  const float* rel_bias;
  const float* rel_vec;  // [H][2k+1][D] key-side label vectors, or null
  const int32_t* seg;    // [B][N] segment id per position (packed documents), or null
  // Per-pair labels of the pieces with a global token: glabel [B][n_global][N]
  // (global queries), llabel [B][N][n_global] (non-global queries, global
  // keys); a vocabulary index < n_labels, kLabelDistance, or a masked pair.
  const uint8_t* glabel;
  const uint8_t* llabel;
  int32_t n_labels;      // vocabulary size (2*rel_k+1 without structural labels)
  int32_t seg_pieces;    // pieces segment ids mask: bits g2g 1, g2l 2, l2g 4, l2l 8
  int32_t rel_k;
  void* out;
  float* lse;
  float* ws_o;      // [B*H][n_global][n_chunks][D] global-row partials
  float* ws_lse;    // [B*H][n_global][n_chunks]
  // [B*H][n_gq_tiles] chunk arrivals per global-row tile: (token << 32) | count.
  // A word whose high half is not this call's token counts as 0, so whatever
  // an earlier call left there is ignored; the tile's last arrival writes 0.
  uint64_t* ws_cnt;
  uint32_t token;   // unique per call: a quiet-NaN bit pattern no fp32 partial holds
  int32_t chunk_len, n_chunks;
  int32_t band_tiles_per_head;
  int32_t n_band_wg;
  int32_t n_glob_wg;  // B*H*n_gq_tiles*n_chunks, placed first in the grid
  int32_t n_gq_tiles;
  float scale_log2;
};

struct DilArgs {
  const void *q, *k, *v;
  int32_t B, H, N, causal, n_pairs;
  int32_t w[kMaxPairs], r[kMaxPairs];
  // kind 0: a dilated pattern (w, r); kind 1 (r = 1): the strided summary
  // keys of Sparse Transformer's fixed pattern, c = sum_c[k] positions per
  // block of length w, the run per head as in la_fixed_forward
  int32_t kind[kMaxPairs], sum_c[kMaxPairs];
  float inv_w[kMaxPairs], inv_r[kMaxPairs];  // 1/w, 1/r (fp32) for division without divides
  int32_t nseg[kMaxPairs];      // segments of pattern k: ceil(N / w)
  int32_t seg_rows[kMaxPairs];  // partial rows reserved per segment: ceil(w / r)
  int32_t qtiles[kMaxPairs];    // query tiles per segment: ceil(seg_rows / query tile)
  // Launch order: by query-tile index t descending (a workgroup's key tiles
  // grow with t), all patterns together. order[] lists the patterns by qtiles
  // descending; band j holds the levels t in [qtiles[order[j+1]], band_top[j]]
  // (the last band down to 0), where exactly patterns order[0..j] have a tile
  // t, band_per[j] workgroups per level. pre[i]: workgroups of one level that
  // belong to order[0..i-1].
  // Finisher: a pattern of dilation 1 (it covers every row), or -1. When
  // there is one, the pair launch runs the other n_part patterns, and the
  // finisher's own launch mixes their partials into its rows; otherwise all
  // patterns write partials (n_part == n_pairs) and a combine launch mixes.
  int32_t fin, n_part;
  int32_t order[kMaxPairs];
  int32_t band_top[kMaxPairs];
  int64_t band_per[kMaxPairs];
  int64_t pre[kMaxPairs + 1];
  int64_t band_start[kMaxPairs + 1];  // first workgroup of band j; [n_pairs]: total
  int64_t row_off[kMaxPairs];   // first partial row of pattern k (not the finisher's)
  int64_t rows_total;           // partial rows of all patterns
  float* ws_o;                  // [rows_total][D]
  float* ws_lse;                // [rows_total]
  void* out;
  float* lse;
  float scale_log2;
};

hipError_t launch_attn(const AttnArgs& a, int32_t dtype, hipStream_t stream);
hipError_t launch_dilated(const DilArgs& a, hipStream_t stream);
int32_t host_band_tiles_of_head(int32_t N, int32_t d, int32_t tq);
int32_t host_query_tile(int32_t dtype);  // query rows per workgroup
constexpr int32_t kDilatedQueryTile = 128;  // bf16 workgroup rows of the LongNet kernel

}  // namespace la
