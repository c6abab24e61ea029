/* longattn.h — C ABI of the sparse long-sequence attention forward pass (gfx950).
 *
 * Two operations, both exact masked softmax attention (LongNet page, §3.4
 * "Standard Self-Attention and Sparse Attention (Preliminaries)", Eq. 2):
 *
 *   la_attn_forward     sliding-window attention of radius R (optionally dilated
 *                       per head and causal), unioned with a set G of global
 *                       tokens that attend to every key and that every query
 *                       attends to, with optional separate projections for the
 *                       global rows and an optional per-head scalar relative-
 *                       position bias.
 *                       Longformer page, §3.4 "Sliding Window Attention"
 *                       (Fig. 2b), "Dilated Sliding Window Attention" (Fig. 2c,
 *                       head-specific dilation), "Global Attention" (Fig. 2d),
 *                       "Separate Linear Projections for Local vs. Global
 *                       Attention", "Autoregressive Language Modeling
 *                       Configuration" (causal window). ETC page, §3.4
 *                       "Global-Local Attention" (g2g/g2l/l2g full, l2l within
 *                       radius r, two unified softmaxes) and "Relative Position
 *                       Encoding" (labels clipped at distance k).
 *
 *   la_dilated_forward  LongNet dilated attention: for every (segment length w,
 *                       dilation r) pattern, each length-w segment keeps the
 *                       positions whose offset from the segment start is
 *                       congruent to (head mod r), attends densely among them,
 *                       and the per-pattern outputs are mixed with weights
 *                       proportional to their softmax denominators.
 *                       LongNet page, §3.4 "Dilated Attention: Core Mechanism"
 *                       (Eqs. 3-8), "Mixture of Dilated Attentions" (Eqs. 9-10),
 *                       "Multi-Head Dilated Attention: Offset Mechanism"
 *                       (Eqs. 13-15).
 *
 * Conventions for every call:
 *   - B, H, N >= 0; a call with B, H or N equal to 0 does nothing and returns
 *     LA_OK (after the remaining argument checks that need no pointer).
 *     N must be below 2^24 and B*H*N at most 2^31 (LA_EUNSUPPORTED otherwise):
 *     the kernels address a head's rows with 32-bit byte offsets.
 *   - q, k, v, out (and qg, kg, vg) are device tensors, contiguous [B,H,N,D]
 *     row-major, 16-byte aligned, of the dtype in la_dims (bf16 or fp32);
 *     D must be 64 and la_attn_forward takes H <= 64 (LA_EUNSUPPORTED above).
 *   - logits are (q_i . k_j) / sqrt(D) + bias_ij in fp32; softmax and both
 *     products accumulate in fp32; out is rounded to its dtype (RNE).
 *   - lse (optional) is device fp32 [B,H,N]: the natural-log softmax
 *     denominator, lse_i = ln sum_j c_ij exp(s_ij).
 *   - Ownership: the caller owns every buffer. The library allocates nothing,
 *     keeps no pointer after returning, never writes its inputs, and fully
 *     overwrites out and lse. The workspace is scratch whose contents on entry
 *     do not matter (nothing in it needs initialisation). out must not alias
 *     an input.
 *   - All work is enqueued on `stream` (0 = the null stream); the call returns
 *     without synchronising and issues no device-to-host copy.
 *   - Errors: host-detectable argument errors return LA_EINVAL and enqueue
 *     nothing; valid but unbuilt combinations return LA_EUNSUPPORTED; a failed
 *     launch returns LA_EHIP. la_last_error() then describes the failure.
 *     Facts that live in device memory (global_idx sorted and in range) are
 *     the caller's contract; la_check_global_idx() verifies them synchronously.
 *   - Thread safety: calls may come from several host threads; the only state
 *     is the thread-local error message.
 */
#ifndef LONGATTN_H
#define LONGATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LA_OK = 0, LA_EINVAL = -1, LA_EUNSUPPORTED = -2, LA_EHIP = -3 } la_status;
typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Shape and element type shared by q, k, v, out: [B,H,N,D]. */
typedef struct {
  int32_t B, H, N, D;
  int32_t dtype; /* la_dtype */
} la_dims;

/* Optional extras of la_attn_forward; pass NULL for none. */
typedef struct {
  /* rel_bias holds H*V fp32 entries (V = n_labels, or 2*rel_k+1 when that is
   * 0); entry [h][clamp(j-i,-rel_k,rel_k)+rel_k] is added to the logit of every
   * pair (i,j) whose members are of the same kind (both global or both
   * non-global), unless a label matrix gives the pair another label. Required
   * (> 0) iff rel_bias != NULL or rel_vec != NULL. */
  int32_t rel_k;
  /* Separate projections for the global rows: all three or none, dims as q.
   * A global row i then uses qg_i, kg_j, vg_j for every key j; non-global rows
   * keep q, k, v (for their global columns too). */
  const void *qg, *kg, *vg;
  /* Device scratch of at least la_attn_workspace_size() bytes, 256-byte aligned;
   * required when n_global > 0. Its contents on entry do not matter and need no
   * initialisation: it holds the global rows' key-chunk partials, which the call
   * writes before reading, and one arrival counter word per tile of global rows,
   * tagged with a token unique to the call (a quiet-NaN bit pattern no fp32
   * value this library writes can hold), so words left by earlier calls of any
   * shape are ignored. Calls that share a workspace must not overlap in time. */
  void *workspace;
  size_t workspace_bytes;
  /* Key-side relative-position vectors (ETC page, §3.4 "Relative Position
   * Encoding", Steps 2-3): device fp32 [H][V][D] (V as for rel_bias), 16-byte aligned, or
   * NULL. For a same-kind pair (i,j) with label l = clamp(j-i,-rel_k,rel_k) the
   * logit becomes q_i . (k_j + a_{h,l}) / sqrt(D) (plus rel_bias when both are
   * given). The kernels precompute q_i . a_{h,l} per query row and label, as the
   * page's implementation note describes; such calls use V fp32 of LDS per
   * query row of a workgroup beyond the usual. */
  const float *rel_vec;
  /* Per-instance segment masks for packed documents (ETC page, §3.4
   * "Per-instance attention masks"): device int32 [B][N], a segment id per
   * position, or NULL. A pair (i,j) whose positions carry different ids is
   * excluded in every piece (band, global rows, global columns), on top of the
   * pattern. Any int32 values; a segment need not be contiguous. seg_pieces
   * (below) can restrict this to some pieces. */
  const int32_t *seg_ids;
  /* Per-instance per-piece masks and structural relation labels for the pieces
   * with a global token (ETC page, §3.4 "Global-Local Attention": a binary mask
   * M per piece; "Per-instance attention masks": hard g2l masking;
   * "Relative Position Encoding", Step 1: labels for structural relations, and
   * its implementation note: a label gathered per pair). The piece of a pair
   * (i,j) follows from whether i and j are in global_idx.
   *  glabel   device uint8 [B][n_global][N] or NULL: the label of every pair
   *           whose query is global_idx[g] (g2g and g2l pieces);
   *  llabel   device uint8 [B][N][n_global] or NULL: the label of every pair of
   *           a non-global query i and the key global_idx[g] (l2g piece).
   * A label value l < n_labels selects entry l of rel_bias [H][n_labels] and of
   * rel_vec [H][n_labels][D] for that pair, whatever its piece; 0xFE keeps the
   * pair's usual label (the clipped distance for same-kind pairs, none for
   * mixed pairs); any other value masks the pair (M = 0). Entries of pairs the
   * pattern excludes are not read. Label matrices need n_global > 0 and at most
   * 2^31 entries per batch row.
   *  n_labels   size of the label vocabulary: 0 (the 2*rel_k+1 distance labels
   *             only) or in [2*rel_k+1, 64]; the structural labels follow the
   *             distance labels. Needs rel_bias or rel_vec when non-zero.
   *  seg_pieces the pieces seg_ids mask, as bits g2g 1, g2l 2, l2g 4, l2l 8
   *             (0 = all four: packed documents), e.g. 8 to mask l2l across
   *             contexts while every word piece still reads every global token. */
  const uint8_t *glabel;
  const uint8_t *llabel;
  int32_t n_labels;
  int32_t seg_pieces;
} la_attn_ext;

/* Optional extras of la_dilated_forward; pass NULL for none. */
typedef struct {
  float *lse;      /* device fp32 [B,H,N] or NULL; -inf where no pattern covers a row */
  void *workspace; /* device scratch of la_dilated_workspace_size() bytes, 256-byte aligned
                    * (NULL when that size is 0) */
  size_t workspace_bytes;
} la_dilated_ext;

/* Band + global attention.
 *  global_idx  device int32[n_global], strictly increasing, each in [0,N); NULL iff n_global == 0.
 *  radius      R >= 0, counted in dilation steps: row i sees keys i + d*m for |m| <= R
 *              (causal: -R <= m <= 0), inside [0,N).
 *  dilation    host int32[H], each >= 1; NULL means 1 for every head.
 *  causal      0 or 1; when 1, every pair (band, global row, global column) needs j <= i.
 *  rel_bias    device fp32 [H][2*rel_k+1] or NULL (see la_attn_ext.rel_k).
 *  out         device [B,H,N,D], dtype as q.   lse: device fp32 [B,H,N] or NULL.
 * Requires ext->workspace when n_global > 0 (ext may be NULL otherwise). */
la_status la_attn_forward(const la_dims *dims, const void *q, const void *k, const void *v,
                          const int32_t *global_idx, int32_t n_global, int32_t radius,
                          const int32_t *dilation, int32_t causal, const float *rel_bias,
                          void *out, float *lse, hipStream_t stream, const la_attn_ext *ext);

/* Allocation-free variant of la_attn_forward, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Arguments, results and errors are those of
 * la_attn_forward, except that no workspace is passed (ext may be NULL; if
 * given, ext->workspace must be NULL and ext->workspace_bytes 0, else
 * LA_EINVAL): the call uses a fixed 32 MiB scratch array in the library's
 * device memory instead, one copy per GPU, held from the first call on that
 * GPU (its address is looked up then, with that GPU current) until the process
 * ends. A call whose la_attn_workspace_size() exceeds 32 MiB returns
 * LA_EUNSUPPORTED and enqueues nothing. The call allocates nothing and needs
 * nothing cleared between calls. All calls on one GPU share the array: calls
 * that overlap in time on one GPU (other streams or host threads) race, and
 * the caller must serialise them. */
la_status la_attn_forward_noalloc(const la_dims *dims, const void *q, const void *k,
                                  const void *v, const int32_t *global_idx, int32_t n_global,
                                  int32_t radius, const int32_t *dilation, int32_t causal,
                                  const float *rel_bias, void *out, float *lse,
                                  hipStream_t stream, const la_attn_ext *ext);

/* LongNet dilated attention mixture (bf16 only).
 *  seg_lens, dil_rates  host int32[n_pairs]: segment length w_k >= 1 and dilation r_k >= 1.
 *                       1 <= n_pairs <= 16. The last segment of a pattern is
 *                       truncated at N. Head h uses offset h mod r_k.
 *  causal               0 or 1: within a segment, key position <= query position.
 *  out                  device bf16 [B,H,N,D]; rows no pattern covers are 0.
 * The first pattern with r_k == 1 (it keeps every row) runs last and mixes the
 * other patterns' partials into its rows, so it needs no workspace of its own.
 * Requires ext->workspace of la_dilated_workspace_size() bytes when that size is
 * non-zero (it needs no initialisation); ext may be NULL when it is zero. */
la_status la_dilated_forward(const la_dims *dims, const void *q, const void *k, const void *v,
                             const int32_t *seg_lens, const int32_t *dil_rates, int32_t n_pairs,
                             int32_t causal, void *out, hipStream_t stream,
                             const la_dilated_ext *ext);

/* Sparse Transformer fixed pattern (LongNet page, §3.4 "Standard Self-Attention
 * and Sparse Attention (Preliminaries)"; bf16 only). Query i attends the keys of
 * its own block of block_len positions (local part) and, in every other block
 * (causal: every earlier block), the summary_len positions at block offsets
 * [t, t + summary_len), t = block_len - summary_len * (h' + 1) for head h,
 * h' = h mod floor(block_len / summary_len): head 0 takes each block's last
 * summary_len tokens, further heads distinct sub-blocks. One softmax over the
 * union; causal 0 or 1 (key position <= query position).
 *  block_len    >= 1; N must be a multiple of it (else LA_EUNSUPPORTED).
 *  summary_len  in [1, block_len]; a multiple of 64 (else LA_EUNSUPPORTED).
 *  out          device bf16 [B,H,N,D]; ext->lse optional as for la_dilated_forward.
 * Requires ext->workspace of la_fixed_workspace_size() bytes (256-byte aligned,
 * no initialisation needed). */
la_status la_fixed_forward(const la_dims *dims, const void *q, const void *k, const void *v,
                           int32_t block_len, int32_t summary_len, int32_t causal, void *out,
                           hipStream_t stream, const la_dilated_ext *ext);

/* Bytes of workspace la_fixed_forward needs (0 for invalid arguments). */
size_t la_fixed_workspace_size(const la_dims *dims, int32_t block_len, int32_t summary_len);

/* Optional arguments of la_attn_backward. */
typedef struct {
  const void *qg, *kg, *vg; /* separate global projections as given to the forward (all or none) */
  float *dqg, *dkg, *dvg;   /* their gradients, fp32 [B,H,N,D]: required iff qg, kg, vg are */
  const int32_t *seg_ids;   /* device int32 [B][N] segment ids as given to the forward, or NULL */
  void *workspace;          /* la_attn_backward_workspace_size() bytes, 256-byte aligned */
  size_t workspace_bytes;
  /* The forward's bias tables and structured-input arguments, as given to it
   * (la_attn_ext; the scalar table here instead of la_attn_forward's rel_bias
   * argument): read, not differentiated. Zero / NULL: none. */
  int32_t rel_k;
  const float *rel_bias;    /* device fp32 [H][V], or NULL */
  const float *rel_vec;     /* device fp32 [H][V][D], 16-byte aligned, or NULL */
  const uint8_t *glabel;    /* device uint8 [B][n_global][N], or NULL */
  const uint8_t *llabel;    /* device uint8 [B][N][n_global], or NULL */
  int32_t n_labels;         /* V: 0 (2*rel_k+1) or the vocabulary size, <= 64 */
  int32_t seg_pieces;       /* pieces seg_ids masks (bits g2g 1, g2l 2, l2g 4, l2l 8; 0 = all) */
} la_attn_bwd_ext;

/* Backward of la_attn_forward for the band + global pattern (the training step
 * after it; the chain rule through masked softmax attention, LongNet page,
 * §3.4 "Standard Self-Attention and Sparse Attention (Preliminaries)", Eq. 2).
 * With P_ij = c_ij exp(q_i.k_j / sqrt(D) - lse_i) over the forward's mask c:
 *   D_i = dO_i . O_i,  dS_ij = P_ij (dO_i . v_j - D_i),
 *   dq_i = sum_j dS_ij k_j / sqrt(D),  dk_j = sum_i dS_ij q_i / sqrt(D),
 *   dv_j = sum_i P_ij dO_i.
 * With separate global projections a global row's terms go to ext->dqg,
 * ext->dkg, ext->dvg (through qg_i, kg_j, vg_j), every other row's to dq, dk, dv;
 * each of the six is fully written (rows that receive nothing get 0).
 * With the forward's bias tables the logit is q_i . (k_j + a_l) / sqrt(D) + b_l
 * for the pair's label l (ETC page, §3.4 "Relative Position Encoding"), so P
 * is recomputed with it and dq_i gains sum_j dS_ij a_l / sqrt(D); the tables
 * get no gradient. Label matrices and segment pieces mask pairs as in the
 * forward.
 *  q, k, v, global_idx, n_global, radius, dilation, causal: as given to the
 *               forward (its bias tables, labels and segment ids through ext).
 *  out, lse     the forward's output (dims/dtype as q) and its lse (fp32 [B,H,N],
 *               required).
 *  dout         device [B,H,N,D] in q's dtype: the loss gradient w.r.t. out.
 *  dq, dk, dv   device fp32 [B,H,N,D] outputs; must not alias any input.
 * Requires ext->workspace (its contents on entry are ignored). Pointers 16-byte
 * aligned. Errors as for la_attn_forward. Two to four launches on `stream`
 * (bf16: D_i, with label vectors, or a scalar table under label matrices,
 * piece masks or a wider vocabulary, each row's label table, then one MFMA
 * launch for dQ, dK and dV, the global rows and keys split over up to 16 key
 * or row ranges, and with several ranges one launch adding their partial sums
 * in a fixed order; fp32: global ranks, dQ and D_i, dK and dV), no
 * allocation; results are bitwise reproducible. */
la_status la_attn_backward(const la_dims *dims, const void *q, const void *k, const void *v,
                           const int32_t *global_idx, int32_t n_global, int32_t radius,
                           const int32_t *dilation, int32_t causal, const void *out,
                           const float *lse, const void *dout, float *dq, float *dk, float *dv,
                           hipStream_t stream, const la_attn_bwd_ext *ext);

/* Bytes of workspace la_attn_backward needs (0 for invalid dims): fp32 D_i per
 * row, each position's int32 rank in global_idx and, for bf16, fp32 partial
 * sums of dQ, dK and dV for min(N rounded up to 128, 2048) rows per head and
 * a label table of 64 fp32 entries per row (used with label vectors); each
 * part padded to 256 bytes. */
size_t la_attn_backward_workspace_size(const la_dims *dims);

/* Backward of la_dilated_forward (bf16 only). The mixture is one softmax over
 * the multiset of the patterns' keys (LongNet page, §3.4 "Mixture of Dilated
 * Attentions"), so with c_ij the number of patterns that pair i with j and lse
 * the forward's (mixture) lse, P_ij = c_ij exp(q_i.k_j / sqrt(D) - lse_i), and
 * the gradients follow the formulas of la_attn_backward.
 *  q, k, v, seg_lens, dil_rates, n_pairs, causal: as given to the forward.
 *  out, lse     the forward's output and its ext->lse (fp32 [B,H,N], required).
 *  dout         device bf16 [B,H,N,D]: the loss gradient w.r.t. out.
 *  dq, dk, dv   device fp32 [B,H,N,D] outputs (fully written; must not alias inputs).
 *  workspace    la_dilated_backward_workspace_size() bytes, 256-byte aligned.
 * Errors as for la_dilated_forward. n_pairs + 1 launches on `stream`: each
 * pattern's dQ terms, then its dK/dV terms in the next launch beside the next
 * pattern's dQ terms. A pattern of dilation 1, which keeps every row and key,
 * goes first, computes D_i and stores its terms; the others add theirs in a
 * fixed order (deterministic). Without one, a D_i and a zeroing launch come
 * first and every pattern adds. No allocation. */
la_status la_dilated_backward(const la_dims *dims, const void *q, const void *k, const void *v,
                              const int32_t *seg_lens, const int32_t *dil_rates, int32_t n_pairs,
                              int32_t causal, const void *out, const float *lse,
                              const void *dout, float *dq, float *dk, float *dv,
                              hipStream_t stream, void *workspace, size_t workspace_bytes);

/* Bytes of workspace la_dilated_backward needs (0 for invalid dims): fp32 D_i per row. */
size_t la_dilated_backward_workspace_size(const la_dims *dims);

/* Bytes of workspace la_attn_forward needs for these dims and n_global
 * (0 when n_global == 0). has_separate_global is accepted for symmetry and
 * does not change the size. Returns 0 for invalid dims. */
size_t la_attn_workspace_size(const la_dims *dims, int32_t n_global, int32_t has_separate_global);

/* Bytes of workspace la_dilated_forward needs for these dims and patterns
 * (host arrays as in la_dilated_forward). Returns 0 for invalid arguments. */
size_t la_dilated_workspace_size(const la_dims *dims, const int32_t *seg_lens,
                                 const int32_t *dil_rates, int32_t n_pairs);

/* Synchronous test helper: LA_OK iff global_idx (device int32[n_global]) is
 * strictly increasing and inside [0,N). Copies the array to the host on `stream`
 * and waits for it. */
la_status la_check_global_idx(const int32_t *global_idx, int32_t n_global, int32_t N,
                              hipStream_t stream);

/* Message of the last non-OK status on this thread ("" if none). */
const char *la_last_error(void);

/* ABI version of this library (2: la_attn_ext carries label matrices, n_labels
 * and seg_pieces after seg_ids). */
int32_t la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LONGATTN_H */
