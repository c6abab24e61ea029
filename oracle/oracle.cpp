// oracle.cpp — TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
//
// A plain, slow, fp64 CPU reference ("the oracle") for the forward pass of
// sparse long-sequence self-attention. Only the tests, the smoke check and the
// benchmark's CPU-baseline leg load it. It shares no code, header, helper or
// constant with the HIP library in sparse_long_sequence_amd/, and it never
// reads anything that library produced.
//
// Sparse attention is exact masked softmax attention, so the oracle is that
// definition written out (LongNet page, §3.4 "Standard Self-Attention and
// Sparse Attention (Preliminaries)", Eq. 2: entries outside the mask S are set
// to -inf before the softmax):
//
//   s_ij   = (q_i . k_j) / sqrt(D) + bias_ij
//   M_i    = max over allowed j of s_ij
//   Z_i    = sum_j c_ij exp(s_ij - M_i)
//   O_i    = sum_j c_ij exp(s_ij - M_i) v_j / Z_i,   lse_i = M_i + ln Z_i
//
// where c_ij is the explicit mask (0/1) or, for the LongNet mixture, an integer
// key multiplicity. The mask is evaluated by its predicate for every key j of
// every requested row; the n x n matrix is materialised one row at a time (a
// full n x n byte matrix for n = 32768 would be 1 GiB per head).
//
// Readings of points the pages leave open (each is listed in the design doc):
//   * scale 1/sqrt(D) everywhere, LongNet included;
//   * masked pairs are excluded (-inf), not given ETC's -10000;
//   * the window is inclusive, |j-i| <= d*R, and keys outside [0,N) are dropped;
//   * causal means j <= i for every pair, band, global row and global column;
//   * a global key inside the band counts once (set union);
//   * the scalar relative bias and the relative key vectors apply only to
//     pairs of the same kind (both global or both non-global), indexed by the
//     label clamp(j-i, -k, k); mixed pairs get neither;
//   * with separate global projections, a global row i uses qg_i, kg_j, vg_j
//     for every key j; non-global rows use q, k, v, also for global columns;
//   * per-instance masks for packed documents: with a segment id per token,
//     a pair whose tokens carry different ids is masked in all four pieces
//     (g2g, g2l, l2g, l2l), on top of the pattern;
//   * LongNet head h keeps, in each segment, the positions whose offset from
//     the segment start is congruent to h mod r; the last segment is truncated
//     to N; attention inside a segment is causal in position when causal != 0;
//     a row that no pattern covers gets O = 0 and lse = -inf.
//
// Threads: rows are split over std::threads; each row is summed sequentially
// in fp64, so the result does not depend on the thread count.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <limits>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Pattern predicates
// ---------------------------------------------------------------------------

// Membership of position p in the strictly increasing global index set G.
bool in_global(const int32_t* gidx, int32_t n_global, int32_t p) {
  return std::binary_search(gidx, gidx + n_global, p);
}

// Dilated sliding window, one side of the union that forms the mask.
// Longformer page, §3.4 "Sliding Window Attention" (w/2 keys per side plus the
// token itself, Fig. 2b) and "Dilated Sliding Window Attention" (keys at
// i + d*m for |m| <= w/2, Fig. 2c); causal: "Autoregressive Language Modeling
// Configuration" (only keys to the left). Here R = w/2.
bool band_allows(int32_t i, int32_t j, int32_t radius, int32_t dil, int32_t causal) {
  const int64_t delta = (int64_t)j - (int64_t)i;
  if (causal && delta > 0) return false;
  if (delta % dil != 0) return false;
  const int64_t steps = delta / dil;
  return steps >= -(int64_t)radius && steps <= (int64_t)radius;
}

// The full mask entry c_ij in {0,1}. Global tokens attend to every key and
// every query attends to them (Longformer page, §3.4 "Global Attention",
// Fig. 2d; ETC page, §3.4 "Global-Local Attention": g2g, g2l and l2g pieces are
// full, l2l is banded with radius r). Causal restricts all of them to j <= i.
uint8_t mask_entry(int32_t i, int32_t j, bool i_glob, bool j_glob, int32_t radius,
                   int32_t dil, int32_t causal) {
  if (causal && j > i) return 0;
  if (i_glob || j_glob) return 1;
  return band_allows(i, j, radius, dil, causal) ? 1 : 0;
}

// LongNet sparsification membership: position p is kept by pattern (w, r) for
// head h iff (p - segment_start) mod r == h mod r. LongNet page, §3.4
// "Dilated Attention: Core Mechanism" (Eqs. 3-5) and "Multi-Head Dilated
// Attention: Offset Mechanism" (Eqs. 13-15, offset s_j = j mod r).
bool longnet_kept(int32_t p, int32_t w, int32_t r, int32_t head) {
  const int32_t seg_start = (p / w) * w;
  return ((p - seg_start) % r) == (head % r);
}

// Sparse Transformer fixed pattern (LongNet page, §3.4 "Standard
// Self-Attention and Sparse Attention (Preliminaries)"): the local part keeps
// the keys of the query's own block of length l, the strided part the keys at
// block offsets [t, t + c) of every block, here with t = l - c (h' + 1) for
// head h, h' = h mod floor(l / c): head 0 takes the last c tokens of each
// block, and further heads distinct sub-blocks (the page's baseline setup).
// The mask is the union; causal adds j <= i.
bool fixed_allows(int32_t i, int32_t j, int32_t head, int32_t l, int32_t c, int32_t causal) {
  if (causal && j > i) return false;
  if (i / l == j / l) return true;
  const int32_t hp = head % std::max(1, l / c);
  const int32_t t = l - c * (hp + 1);
  const int32_t o = j % l;
  return o >= t && o < t + c;
}

// Integer multiplicity of key j for query i under the mixture of patterns:
// the number of patterns whose sparsified segment holds both i and j. By the
// page's equivalence statement ("Mixture of Dilated Attentions": mixing with
// alpha_i = s_i / sum_j s_j equals one softmax over the gathered keys of all
// patterns), this multiplicity weights one joint softmax.
int32_t longnet_mult(int32_t i, int32_t j, int32_t head, const int32_t* w, const int32_t* r,
                     int32_t n_pairs, int32_t causal) {
  if (causal && j > i) return 0;
  int32_t m = 0;
  for (int32_t k = 0; k < n_pairs; ++k) {
    if (i / w[k] != j / w[k]) continue;  // same segment
    if (longnet_kept(i, w[k], r[k], head) && longnet_kept(j, w[k], r[k], head)) ++m;
  }
  return m;
}

// A pair's label in the per-pair label inputs: its usual clipped-distance
// label (kLabelDistance) or an index into the label vocabulary; every other
// value masks the pair.
constexpr int32_t kLabelDistance = 0xFE;

// ---------------------------------------------------------------------------
// Masked dense softmax attention of one query row (the definition above).
// weight[j] is c_ij (0 excludes the key). bias(j) adds to the scaled logit.
// ---------------------------------------------------------------------------
template <class Bias>
void attend_row(int32_t N, int32_t D, const double* qi, const double* kbase, const double* vbase,
                const std::vector<double>& weight, Bias bias, double* out, double* lse) {
  const double scale = 1.0 / std::sqrt((double)D);
  std::vector<double> logit(N, 0.0);
  double M = -std::numeric_limits<double>::infinity();
  for (int32_t j = 0; j < N; ++j) {
    if (weight[j] == 0.0) continue;  // excluded keys carry weight exactly 0
    const double* kj = kbase + (size_t)j * D;
    double dot = 0.0;
    for (int32_t c = 0; c < D; ++c) dot += qi[c] * kj[c];
    logit[j] = dot * scale + bias(j);
    M = std::max(M, logit[j]);
  }
  for (int32_t c = 0; c < D; ++c) out[c] = 0.0;
  if (M == -std::numeric_limits<double>::infinity()) {  // no allowed key
    *lse = M;
    return;
  }
  double Z = 0.0;
  for (int32_t j = 0; j < N; ++j) {
    if (weight[j] == 0.0) continue;
    const double p = weight[j] * std::exp(logit[j] - M);
    Z += p;
    const double* vj = vbase + (size_t)j * D;
    for (int32_t c = 0; c < D; ++c) out[c] += p * vj[c];
  }
  for (int32_t c = 0; c < D; ++c) out[c] /= Z;
  *lse = M + std::log(Z);
}

// Run fn(row_index) for row_index in [0, n) over n_threads threads.
template <class Fn>
void parallel_rows(int64_t n, int32_t n_threads, Fn fn) {
  int32_t T = n_threads > 0 ? n_threads : (int32_t)std::thread::hardware_concurrency();
  if (T < 1) T = 1;
  if ((int64_t)T > n) T = (int32_t)std::max<int64_t>(n, 1);
  std::vector<std::thread> pool;
  for (int32_t t = 0; t < T; ++t) {
    pool.emplace_back([=, &fn]() {
      for (int64_t x = t; x < n; x += T) fn(x);
    });
  }
  for (auto& th : pool) th.join();
}

// Decode the (b, h, i) of the x-th requested row: `sel` holds triples, or is
// null for all rows in [B, H, N] order.
inline void decode_row(const int32_t* sel, int64_t x, int32_t H, int32_t N, int32_t& b, int32_t& h,
                       int32_t& i) {
  if (sel) {
    b = sel[3 * x];
    h = sel[3 * x + 1];
    i = sel[3 * x + 2];
  } else {
    i = (int32_t)(x % N);
    h = (int32_t)((x / N) % H);
    b = (int32_t)(x / ((int64_t)N * H));
  }
}

}  // namespace

extern "C" {

int32_t lo_version(void) { return 1; }

// Explicit 0/1 mask rows of the band + global pattern for one head.
// mask is [n_rows][N]; rows == null means every row 0..N-1 (the n x n matrix).
int32_t lo_mask_rows(int32_t N, const int32_t* gidx, int32_t n_global, int32_t radius,
                     int32_t dilation, int32_t causal, const int32_t* rows, int32_t n_rows,
                     uint8_t* mask) {
  if (N <= 0 || radius < 0 || dilation < 1 || n_global < 0 || (n_global > 0 && !gidx)) return -1;
  const int32_t nr = rows ? n_rows : N;
  for (int32_t x = 0; x < nr; ++x) {
    const int32_t i = rows ? rows[x] : x;
    const bool ig = in_global(gidx, n_global, i);
    for (int32_t j = 0; j < N; ++j)
      mask[(size_t)x * N + j] = mask_entry(i, j, ig, in_global(gidx, n_global, j), radius, dilation, causal);
  }
  return 0;
}

// LongNet key multiplicity rows for one head; mult is [n_rows][N].
int32_t lo_longnet_mult_rows(int32_t N, int32_t head, const int32_t* w, const int32_t* r,
                             int32_t n_pairs, int32_t causal, const int32_t* rows, int32_t n_rows,
                             int32_t* mult) {
  if (N <= 0 || n_pairs < 1) return -1;
  for (int32_t k = 0; k < n_pairs; ++k)
    if (w[k] < 1 || r[k] < 1) return -1;
  const int32_t nr = rows ? n_rows : N;
  for (int32_t x = 0; x < nr; ++x) {
    const int32_t i = rows ? rows[x] : x;
    for (int32_t j = 0; j < N; ++j)
      mult[(size_t)x * N + j] = longnet_mult(i, j, head, w, r, n_pairs, causal);
  }
  return 0;
}

// The pairs of one row of the band + global pattern with its per-instance
// inputs (segment ids, the pieces they mask, per-pair label matrices; see
// lo_attn_rows): for query i of batch row b and head h, weight[j] is the mask
// entry c_ij (0 or 1) and lab[j] the pair's label in the vocabulary of V
// entries, -1 when the pair takes no label (a mixed pair keeping its usual
// label, or no bias tables at all).
struct RowRule {
  int32_t N, radius, causal, rel_k, V, pieces, n_global;
  const int32_t* dilation;
  const int32_t* seg;
  const uint8_t* glabel;
  const uint8_t* llabel;
  const uint8_t* is_glob;
  const int32_t* grank;
  bool has_tables;

  void fill(int32_t b, int32_t h, int32_t i, double* weight, int32_t* lab) const {
    const int32_t dil = dilation ? dilation[h] : 1;
    const bool ig = is_glob[i] != 0;
    const int32_t* sb = seg ? seg + (size_t)b * N : nullptr;
    for (int32_t j = 0; j < N; ++j) {
      const bool jg = is_glob[j] != 0;
      weight[j] = mask_entry(i, j, ig, jg, radius, dil, causal);
      const int32_t piece = ig ? (jg ? 1 : 2) : (jg ? 4 : 8);  // g2g, g2l, l2g, l2l
      if (sb && (pieces & piece) && sb[j] != sb[i]) weight[j] = 0.0;  // another segment
      int32_t l = kLabelDistance;
      if (ig && glabel)
        l = glabel[((size_t)b * n_global + grank[i]) * N + j];
      else if (!ig && jg && llabel)
        l = llabel[((size_t)b * N + i) * n_global + grank[j]];
      if (l != kLabelDistance && l >= V) weight[j] = 0.0;  // M = 0
      if (l == kLabelDistance) {
        if (jg != ig) {
          l = -1;  // mixed global/non-global pair: no label
        } else {
          int64_t dlt = (int64_t)j - i;
          dlt = std::max<int64_t>(-rel_k, std::min<int64_t>(rel_k, dlt));
          l = (int32_t)(dlt + rel_k);
        }
      }
      lab[j] = (has_tables && weight[j] != 0.0) ? l : -1;
    }
  }
};

// Band + global attention (Longformer / ETC), fp64. seg: [B][N] segment ids
// or null; with it, c_ij also needs seg[b][i] == seg[b][j] (ETC page, §3.4
// "Per-instance attention masks": documents packed into one input are masked
// from each other in l2l and through the global tokens; §3.4 Global-Local
// Attention, the binary masks M of each piece).
// q, k, v: [B,H,N,D]; qg, kg, vg: all null (shared projections) or all
// [B,H,N,D] (Longformer page, §3.4 "Separate Linear Projections for Local vs.
// Global Attention"). dilation: [H] (null = all 1). rel_bias: [H][2*rel_k+1]
// or null, a scalar added to the scaled logit per label. rel_vec:
// [H][2*rel_k+1][D] or null, the learned key-side vector a_l of each label:
// the logit becomes q_i . (k_j + a_l) / sqrt(D) (ETC page, §3.4 "Relative
// Position Encoding", Steps 1-3: labels clip j - i at k; one vector per label
// and head). Either, both or neither may be given. sel: n_sel (b,h,i) triples
// or null for all B*H*N rows. out: [n_sel][D]; lse: [n_sel].
//
// Per-instance per-piece masks and structural labels (ETC page, §3.4
// "Global-Local Attention": the binary masks M^{g2g}, M^{g2l}, M^{l2g},
// M^{l2l}; "Per-instance attention masks"; "Relative Position Encoding",
// Step 1: labels for relations such as "token belongs to this sentence", and
// its implementation note: one label per (i, j) pair, gathered). The piece of
// a pair follows from whether i and j are global. glabel [B][n_global][N]
// gives the label of each pair whose query is the g-th global token (g2g,
// g2l); llabel [B][N][n_global] the label of each pair of a non-global query
// and the g-th global key (l2g). A label is an index into the vocabulary of
// n_labels entries (rel_bias [H][n_labels], rel_vec [H][n_labels][D];
// n_labels == 0: the 2k+1 distance labels alone), kLabelDistance for the
// pair's usual label (the clipped distance for same-kind pairs, none for mixed
// pairs), or any other value for a masked pair (M = 0). An explicit label
// applies to any pair, mixed ones included. seg_pieces selects the pieces that
// segment ids mask (bits g2g 1, g2l 2, l2g 4, l2l 8; 0 means all four).
int32_t lo_attn_rows(int32_t B, int32_t H, int32_t N, int32_t D, const double* q, const double* k,
                     const double* v, const double* qg, const double* kg, const double* vg,
                     const int32_t* gidx, int32_t n_global, int32_t radius, const int32_t* dilation,
                     int32_t causal, const double* rel_bias, const double* rel_vec, int32_t rel_k,
                     const int32_t* seg, const int32_t* sel, int64_t n_sel, double* out,
                     double* lse, int32_t n_threads, const uint8_t* glabel,
                     const uint8_t* llabel, int32_t n_labels, int32_t seg_pieces) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || radius < 0 || n_global < 0) return -1;
  if (!q || !k || !v || !out || !lse) return -1;
  if ((qg || kg || vg) && !(qg && kg && vg)) return -1;
  if (n_global > 0 && !gidx) return -1;
  if ((rel_bias || rel_vec) && rel_k < 0) return -1;
  const int32_t V = n_labels > 0 ? n_labels : 2 * rel_k + 1;  // vocabulary size
  if (n_labels > 0 && n_labels < 2 * rel_k + 1) return -1;
  if ((glabel || llabel) && n_global == 0) return -1;
  const int32_t pieces = seg_pieces ? seg_pieces : 15;
  if (dilation)
    for (int32_t h = 0; h < H; ++h)
      if (dilation[h] < 1) return -1;
  const int64_t rows = sel ? n_sel : (int64_t)B * H * N;
  std::vector<uint8_t> is_glob(N, 0);
  std::vector<int32_t> grank(N, -1);  // index of a global position in global_idx
  for (int32_t g = 0; g < n_global; ++g)
    if (gidx[g] >= 0 && gidx[g] < N) {
      is_glob[gidx[g]] = 1;
      grank[gidx[g]] = g;
    }
  const RowRule rule = {N, radius, causal, rel_k, V, pieces, n_global, dilation, seg, glabel,
                        llabel, is_glob.data(), grank.data(), rel_bias || rel_vec};
  parallel_rows(rows, n_threads, [&](int64_t x) {
    int32_t b, h, i;
    decode_row(sel, x, H, N, b, h, i);
    const bool ig = is_glob[i] != 0;
    const size_t head_off = ((size_t)b * H + h) * (size_t)N * D;
    // Global rows with separate projections use qg_i, kg_j, vg_j.
    const bool sep = ig && qg;
    const double* qi = (sep ? qg : q) + head_off + (size_t)i * D;
    const double* kb = (sep ? kg : k) + head_off;
    const double* vb = (sep ? vg : v) + head_off;
    std::vector<double> weight(N);  // the explicit mask row c_i,:
    std::vector<int32_t> label(N);  // each pair's label (-1: none)
    rule.fill(b, h, i, weight.data(), label.data());
    const double* tab = rel_bias ? rel_bias + (size_t)h * V : nullptr;
    const double* vec = rel_vec ? rel_vec + (size_t)h * V * D : nullptr;
    const double scale = 1.0 / std::sqrt((double)D);
    auto bias = [&](int32_t j) -> double {
      const int32_t l = label[j];
      if (l < 0) return 0.0;
      double b = tab ? tab[l] : 0.0;
      if (vec) {  // q_i . a_l / sqrt(D): the key-side vector's share of the logit
        const double* al = vec + (size_t)l * D;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qi[d] * al[d];
        b += dot * scale;
      }
      return b;
    };
    attend_row(N, D, qi, kb, vb, weight, bias, out + (size_t)x * D, lse + x);
  });
  return 0;
}

// Backward of band + global attention, fp64: the chain rule through the
// definition above (LongNet page, §3.4 "Standard Self-Attention and Sparse
// Attention (Preliminaries)", Eq. 2, differentiated), for a loss whose gradient
// with respect to O is dout. With P_ij = c_ij exp(s_ij) / Z_i from this
// oracle's own forward:
//   dV_j  = sum_i P_ij dO_i           dP_ij = dO_i . v_j
//   D_i   = sum_j P_ij dP_ij          dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = sum_j dS_ij k_j / sqrt(D)  dK_j = sum_i dS_ij q_i / sqrt(D)
// The mask and the logits are lo_attn_rows's (pattern, causal, segment ids and
// their pieces, per-pair labels, the scalar bias b_l and the key-side vectors
// a_l of the pair's label l): z_ij = q_i . (k_j + a_l) / sqrt(D) + b_l. The
// tables are inputs, not differentiated; a_l adds dS_ij a_l / sqrt(D) to dQ_i.
// A global row with separate projections differentiates through qg_i, kg_j,
// vg_j, so its terms go to dqg, dkg, dvg (given iff qg, kg, vg are). Heads are
// split over threads; rows are visited in order within a head, so sums are
// deterministic.
int32_t lo_attn_backward(int32_t B, int32_t H, int32_t N, int32_t D, const double* q,
                         const double* k, const double* v, const double* qg, const double* kg,
                         const double* vg, const int32_t* gidx, int32_t n_global, int32_t radius,
                         const int32_t* dilation, int32_t causal, const int32_t* seg,
                         const double* dout, double* dq, double* dk, double* dv, double* dqg,
                         double* dkg, double* dvg, int32_t n_threads, const double* rel_bias,
                         const double* rel_vec, int32_t rel_k, const uint8_t* glabel,
                         const uint8_t* llabel, int32_t n_labels, int32_t seg_pieces) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || radius < 0 || n_global < 0) return -1;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  const bool sep_all = qg && kg && vg && dqg && dkg && dvg;
  if ((qg || kg || vg || dqg || dkg || dvg) && !sep_all) return -1;
  if (n_global > 0 && !gidx) return -1;
  if ((rel_bias || rel_vec) && rel_k < 0) return -1;
  const int32_t V = n_labels > 0 ? n_labels : 2 * rel_k + 1;  // vocabulary size
  if (n_labels > 0 && n_labels < 2 * rel_k + 1) return -1;
  if ((glabel || llabel) && n_global == 0) return -1;
  if (dilation)
    for (int32_t h = 0; h < H; ++h)
      if (dilation[h] < 1) return -1;
  std::vector<uint8_t> is_glob(N, 0);
  std::vector<int32_t> grank(N, -1);
  for (int32_t g = 0; g < n_global; ++g)
    if (gidx[g] >= 0 && gidx[g] < N) {
      is_glob[gidx[g]] = 1;
      grank[gidx[g]] = g;
    }
  const RowRule rule = {N, radius, causal, rel_k, V, seg_pieces ? seg_pieces : 15, n_global,
                        dilation, seg, glabel, llabel, is_glob.data(), grank.data(),
                        rel_bias || rel_vec};
  const double scale = 1.0 / std::sqrt((double)D);
  const size_t head_elems = (size_t)N * D;
  parallel_rows((int64_t)B * H, n_threads, [&](int64_t bh) {
    const int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
    const size_t off = (size_t)bh * head_elems;
    double* outs[6] = {dq, dk, dv, dqg, dkg, dvg};
    for (double* o : outs)
      if (o) std::fill(o + off, o + off + head_elems, 0.0);
    const double* tab = rel_bias ? rel_bias + (size_t)h * V : nullptr;
    const double* vec = rel_vec ? rel_vec + (size_t)h * V * D : nullptr;
    std::vector<double> P(N), dP(N), weight(N);
    std::vector<int32_t> lab(N);
    for (int32_t i = 0; i < N; ++i) {
      const bool ig = is_glob[i] != 0;
      const bool sep = ig && sep_all;
      const double* qi = (sep ? qg : q) + off + (size_t)i * D;
      const double* kb = (sep ? kg : k) + off;
      const double* vb = (sep ? vg : v) + off;
      double* dqi = (sep ? dqg : dq) + off + (size_t)i * D;
      double* dkb = (sep ? dkg : dk) + off;
      double* dvb = (sep ? dvg : dv) + off;
      const double* doi = dout + off + (size_t)i * D;
      // forward of row i: the allowed keys' probabilities
      rule.fill(b, h, i, weight.data(), lab.data());
      double M = -std::numeric_limits<double>::infinity();
      for (int32_t j = 0; j < N; ++j) {
        if (weight[j] == 0.0) {
          P[j] = -std::numeric_limits<double>::infinity();
          continue;
        }
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qi[d] * kb[(size_t)j * D + d];
        if (lab[j] >= 0 && vec)
          for (int32_t d = 0; d < D; ++d) dot += qi[d] * vec[(size_t)lab[j] * D + d];
        P[j] = dot * scale + (lab[j] >= 0 && tab ? tab[lab[j]] : 0.0);  // the logit for now
        M = std::max(M, P[j]);
      }
      if (M == -std::numeric_limits<double>::infinity()) continue;  // no key: O = 0, no gradient
      double Z = 0.0;
      for (int32_t j = 0; j < N; ++j) {
        P[j] = std::exp(P[j] - M);  // exp(-inf) = 0 for excluded keys
        Z += P[j];
      }
      double Di = 0.0;
      for (int32_t j = 0; j < N; ++j) {
        P[j] /= Z;
        if (P[j] == 0.0) {
          dP[j] = 0.0;
          continue;
        }
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += doi[d] * vb[(size_t)j * D + d];
        dP[j] = dot;
        Di += P[j] * dot;
      }
      for (int32_t j = 0; j < N; ++j) {
        if (P[j] == 0.0) continue;
        const double dS = P[j] * (dP[j] - Di);
        const double* al = lab[j] >= 0 && vec ? vec + (size_t)lab[j] * D : nullptr;
        for (int32_t d = 0; d < D; ++d) {
          dvb[(size_t)j * D + d] += P[j] * doi[d];
          dqi[d] += dS * (kb[(size_t)j * D + d] + (al ? al[d] : 0.0)) * scale;
          dkb[(size_t)j * D + d] += dS * qi[d] * scale;
        }
      }
    }
  });
  return 0;
}

// Backward of the LongNet mixture, fp64. By the mixture's equivalence (one
// softmax over the multiset of the patterns' keys, "Mixture of Dilated
// Attentions"), P_ij = c_ij exp(s_ij) / Z_i with c the integer multiplicity of
// longnet_mult, and the gradients follow the same chain rule as
// lo_attn_backward. A row no pattern covers has no gradient.
int32_t lo_longnet_backward(int32_t B, int32_t H, int32_t N, int32_t D, const double* q,
                            const double* k, const double* v, const int32_t* w, const int32_t* r,
                            int32_t n_pairs, int32_t causal, const double* dout, double* dq,
                            double* dk, double* dv, int32_t n_threads) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || n_pairs < 1 || !q || !k || !v || !dout || !dq ||
      !dk || !dv)
    return -1;
  for (int32_t p = 0; p < n_pairs; ++p)
    if (w[p] < 1 || r[p] < 1) return -1;
  const double scale = 1.0 / std::sqrt((double)D);
  const size_t head_elems = (size_t)N * D;
  parallel_rows((int64_t)B * H, n_threads, [&](int64_t bh) {
    const int32_t h = (int32_t)(bh % H);
    const size_t off = (size_t)bh * head_elems;
    for (double* o : {dq, dk, dv}) std::fill(o + off, o + off + head_elems, 0.0);
    std::vector<double> P(N), dP(N);
    for (int32_t i = 0; i < N; ++i) {
      const double* qi = q + off + (size_t)i * D;
      const double* doi = dout + off + (size_t)i * D;
      double M = -std::numeric_limits<double>::infinity();
      for (int32_t j = 0; j < N; ++j) {
        const int32_t c = longnet_mult(i, j, h, w, r, n_pairs, causal);
        P[j] = c;  // the multiplicity for now
        if (c == 0) continue;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qi[d] * k[off + (size_t)j * D + d];
        dP[j] = dot * scale;  // the logit for now
        M = std::max(M, dP[j]);
      }
      if (M == -std::numeric_limits<double>::infinity()) continue;
      double Z = 0.0;
      for (int32_t j = 0; j < N; ++j) {
        if (P[j] == 0.0) continue;
        P[j] *= std::exp(dP[j] - M);
        Z += P[j];
      }
      double Di = 0.0;
      for (int32_t j = 0; j < N; ++j) {
        if (P[j] == 0.0) continue;
        P[j] /= Z;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += doi[d] * v[off + (size_t)j * D + d];
        dP[j] = dot;
        Di += P[j] * dot;
      }
      for (int32_t j = 0; j < N; ++j) {
        if (P[j] == 0.0) continue;
        const double g = P[j] * (dP[j] - Di);
        for (int32_t d = 0; d < D; ++d) {
          dv[off + (size_t)j * D + d] += P[j] * doi[d];
          dq[off + (size_t)i * D + d] += g * k[off + (size_t)j * D + d] * scale;
          dk[off + (size_t)j * D + d] += g * qi[d] * scale;
        }
      }
    }
  });
  return 0;
}

}  // extern "C"

// The same gradients for chosen outputs only, for shapes where the full
// backward is too slow: dq of the chosen rows (b, h, i), and dk, dv of the
// chosen keys (b, h, j). Each row that enters is evaluated in full by the
// definition: its multiplicity row c_i,:, logits, lse_i = ln sum_j c_ij e^s_ij
// and D_i = sum_j P_ij (dO_i . v_j); a chosen key j then sums over every row i
// with c_ij > 0. A row no pattern covers contributes nothing.
namespace {

struct LongnetRow {
  std::vector<double> c, logit;  // c_i,: and the scaled logits where c > 0
  double lse = 0.0, Di = 0.0;
  bool covered = false;
};

void longnet_row(int32_t N, int32_t D, int32_t h, int32_t i, const double* q, const double* k,
                 const double* v, const double* dout, const int32_t* w, const int32_t* r,
                 int32_t n_pairs, int32_t causal, LongnetRow& row) {
  const double scale = 1.0 / std::sqrt((double)D);
  row.c.assign(N, 0.0);
  row.logit.assign(N, 0.0);
  const double* qi = q + (size_t)i * D;
  double M = -std::numeric_limits<double>::infinity();
  for (int32_t j = 0; j < N; ++j) {
    row.c[j] = longnet_mult(i, j, h, w, r, n_pairs, causal);
    if (row.c[j] == 0.0) continue;
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += qi[d] * k[(size_t)j * D + d];
    row.logit[j] = dot * scale;
    M = std::max(M, row.logit[j]);
  }
  row.covered = M != -std::numeric_limits<double>::infinity();
  if (!row.covered) return;
  double Z = 0.0;
  for (int32_t j = 0; j < N; ++j)
    if (row.c[j] != 0.0) Z += row.c[j] * std::exp(row.logit[j] - M);
  row.lse = M + std::log(Z);
  const double* doi = dout + (size_t)i * D;
  row.Di = 0.0;
  for (int32_t j = 0; j < N; ++j) {
    if (row.c[j] == 0.0) continue;
    double dp = 0.0;
    for (int32_t d = 0; d < D; ++d) dp += doi[d] * v[(size_t)j * D + d];
    row.Di += row.c[j] * std::exp(row.logit[j] - row.lse) * dp;
  }
}

}  // namespace

extern "C" {

int32_t lo_longnet_backward_sel(int32_t B, int32_t H, int32_t N, int32_t D, const double* q,
                                const double* k, const double* v, const int32_t* w,
                                const int32_t* r, int32_t n_pairs, int32_t causal,
                                const double* dout, const int32_t* rows, int64_t n_rows,
                                double* dq_rows, const int32_t* keys, int64_t n_keys,
                                double* dk_keys, double* dv_keys, int32_t n_threads) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || n_pairs < 1 || !q || !k || !v || !dout) return -1;
  if ((n_rows > 0 && (!rows || !dq_rows)) || (n_keys > 0 && (!keys || !dk_keys || !dv_keys)))
    return -1;
  for (int32_t p = 0; p < n_pairs; ++p)
    if (w[p] < 1 || r[p] < 1) return -1;
  const double scale = 1.0 / std::sqrt((double)D);
  const size_t head_elems = (size_t)N * D;
  // dq_i = sum_j P_ij (dP_ij - D_i) k_j / sqrt(D)
  parallel_rows(n_rows, n_threads, [&](int64_t x) {
    const int32_t b = rows[3 * x], h = rows[3 * x + 1], i = rows[3 * x + 2];
    const size_t off = ((size_t)b * H + h) * head_elems;
    double* dqi = dq_rows + (size_t)x * D;
    for (int32_t d = 0; d < D; ++d) dqi[d] = 0.0;
    LongnetRow row;
    longnet_row(N, D, h, i, q + off, k + off, v + off, dout + off, w, r, n_pairs, causal, row);
    if (!row.covered) return;
    const double* doi = dout + off + (size_t)i * D;
    for (int32_t j = 0; j < N; ++j) {
      if (row.c[j] == 0.0) continue;
      const double P = row.c[j] * std::exp(row.logit[j] - row.lse);
      double dp = 0.0;
      for (int32_t d = 0; d < D; ++d) dp += doi[d] * v[off + (size_t)j * D + d];
      const double g = P * (dp - row.Di);
      for (int32_t d = 0; d < D; ++d) dqi[d] += g * k[off + (size_t)j * D + d] * scale;
    }
  });
  // dk_j = sum_i P_ij (dP_ij - D_i) q_i / sqrt(D),  dv_j = sum_i P_ij dO_i
  parallel_rows(n_keys, n_threads, [&](int64_t x) {
    const int32_t b = keys[3 * x], h = keys[3 * x + 1], j = keys[3 * x + 2];
    const size_t off = ((size_t)b * H + h) * head_elems;
    double* dkj = dk_keys + (size_t)x * D;
    double* dvj = dv_keys + (size_t)x * D;
    for (int32_t d = 0; d < D; ++d) dkj[d] = dvj[d] = 0.0;
    LongnetRow row;
    for (int32_t i = 0; i < N; ++i) {
      if (longnet_mult(i, j, h, w, r, n_pairs, causal) == 0) continue;
      longnet_row(N, D, h, i, q + off, k + off, v + off, dout + off, w, r, n_pairs, causal, row);
      const double* qi = q + off + (size_t)i * D;
      const double* doi = dout + off + (size_t)i * D;
      const double P = row.c[j] * std::exp(row.logit[j] - row.lse);
      double dp = 0.0;
      for (int32_t d = 0; d < D; ++d) dp += doi[d] * v[off + (size_t)j * D + d];
      const double g = P * (dp - row.Di);
      for (int32_t d = 0; d < D; ++d) {
        dkj[d] += g * qi[d] * scale;
        dvj[d] += P * doi[d];
      }
    }
  });
  return 0;
}

}  // extern "C"

extern "C" {

// Sparse Transformer fixed pattern, fp64: masked dense softmax over
// fixed_allows. q, k, v: [B,H,N,D]; sel as in lo_attn_rows.
int32_t lo_fixed_rows(int32_t B, int32_t H, int32_t N, int32_t D, const double* q, const double* k,
                      const double* v, int32_t l, int32_t c, int32_t causal, const int32_t* sel,
                      int64_t n_sel, double* out, double* lse, int32_t n_threads) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || l < 1 || c < 1 || c > l || !q || !k || !v || !out ||
      !lse)
    return -1;
  const int64_t rows = sel ? n_sel : (int64_t)B * H * N;
  parallel_rows(rows, n_threads, [&](int64_t x) {
    int32_t b, h, i;
    decode_row(sel, x, H, N, b, h, i);
    const size_t head_off = ((size_t)b * H + h) * (size_t)N * D;
    std::vector<double> weight(N);
    for (int32_t j = 0; j < N; ++j) weight[j] = fixed_allows(i, j, h, l, c, causal) ? 1.0 : 0.0;
    attend_row(N, D, q + head_off + (size_t)i * D, k + head_off, v + head_off, weight,
               [](int32_t) { return 0.0; }, out + (size_t)x * D, lse + x);
  });
  return 0;
}

// LongNet mixture of dilated attentions, path 1: one softmax per row over the
// integer key multiplicity (the page's equivalence statement).
int32_t lo_longnet_rows(int32_t B, int32_t H, int32_t N, int32_t D, const double* q, const double* k,
                        const double* v, const int32_t* w, const int32_t* r, int32_t n_pairs,
                        int32_t causal, const int32_t* sel, int64_t n_sel, double* out, double* lse,
                        int32_t n_threads) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || n_pairs < 1 || !q || !k || !v || !out || !lse) return -1;
  for (int32_t p = 0; p < n_pairs; ++p)
    if (w[p] < 1 || r[p] < 1) return -1;
  const int64_t rows = sel ? n_sel : (int64_t)B * H * N;
  parallel_rows(rows, n_threads, [&](int64_t x) {
    int32_t b, h, i;
    decode_row(sel, x, H, N, b, h, i);
    const size_t head_off = ((size_t)b * H + h) * (size_t)N * D;
    std::vector<double> weight(N);
    for (int32_t j = 0; j < N; ++j) weight[j] = longnet_mult(i, j, h, w, r, n_pairs, causal);
    attend_row(N, D, q + head_off + (size_t)i * D, k + head_off, v + head_off, weight,
               [](int32_t) { return 0.0; }, out + (size_t)x * D, lse + x);
  });
  return 0;
}

// LongNet mixture of dilated attentions, path 2, in the page's order:
// for each pattern (w_k, r_k): sparsify the row's segment (Eqs. 3-5 with the
// head offset of Eqs. 13-15), dense softmax attention on the sparsified
// segment (Eq. 6), scatter back with zeros for rows the pattern skips
// (Eqs. 7-8); then mix O = sum_k alpha_k O_k with alpha_k = s_k / sum_j s_j,
// s_k the softmax denominator sum exp(s) of pattern k (Eqs. 9-10; "Mixture of
// Dilated Attentions"). s_k is carried as lse_k = ln s_k.
// Optional per-pattern outputs: out_k [n_pairs][n_sel][D], lse_k [n_pairs][n_sel]
// (lse_k = -inf where pattern k skips the row).
int32_t lo_longnet_mixture_rows(int32_t B, int32_t H, int32_t N, int32_t D, const double* q,
                                const double* k, const double* v, const int32_t* w, const int32_t* r,
                                int32_t n_pairs, int32_t causal, const int32_t* sel, int64_t n_sel,
                                double* out, double* lse, double* out_k, double* lse_k,
                                int32_t n_threads) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || n_pairs < 1 || !q || !k || !v || !out || !lse) return -1;
  for (int32_t p = 0; p < n_pairs; ++p)
    if (w[p] < 1 || r[p] < 1) return -1;
  const int64_t rows = sel ? n_sel : (int64_t)B * H * N;
  const double NEG_INF = -std::numeric_limits<double>::infinity();
  parallel_rows(rows, n_threads, [&](int64_t x) {
    int32_t b, h, i;
    decode_row(sel, x, H, N, b, h, i);
    const size_t head_off = ((size_t)b * H + h) * (size_t)N * D;
    const double* qi = q + head_off + (size_t)i * D;
    std::vector<double> Ok((size_t)n_pairs * D, 0.0), Lk(n_pairs, NEG_INF);
    for (int32_t p = 0; p < n_pairs; ++p) {
      const int32_t seg_start = (i / w[p]) * w[p];
      const int32_t seg_end = std::min<int64_t>((int64_t)seg_start + w[p], N);
      const int32_t off = h % r[p];
      if ((i - seg_start) % r[p] != off) continue;  // scattered zero row
      // Gather the sparsified keys of this segment: seg_start + off + m*r.
      std::vector<double> weight(N, 0.0);
      for (int64_t j = (int64_t)seg_start + off; j < seg_end; j += r[p])
        if (!causal || j <= i) weight[j] = 1.0;
      attend_row(N, D, qi, k + head_off, v + head_off, weight, [](int32_t) { return 0.0; },
                 &Ok[(size_t)p * D], &Lk[p]);
    }
    // alpha_k = s_k / sum_j s_j with s_k = exp(lse_k); evaluated stably.
    double Lmax = NEG_INF;
    for (int32_t p = 0; p < n_pairs; ++p) Lmax = std::max(Lmax, Lk[p]);
    double* o = out + (size_t)x * D;
    for (int32_t c = 0; c < D; ++c) o[c] = 0.0;
    if (Lmax == NEG_INF) {
      lse[x] = NEG_INF;
    } else {
      double S = 0.0;
      for (int32_t p = 0; p < n_pairs; ++p)
        if (Lk[p] != NEG_INF) S += std::exp(Lk[p] - Lmax);
      for (int32_t p = 0; p < n_pairs; ++p) {
        if (Lk[p] == NEG_INF) continue;
        const double alpha = std::exp(Lk[p] - Lmax) / S;
        for (int32_t c = 0; c < D; ++c) o[c] += alpha * Ok[(size_t)p * D + c];
      }
      lse[x] = Lmax + std::log(S);
    }
    if (out_k && lse_k) {
      for (int32_t p = 0; p < n_pairs; ++p) {
        for (int32_t c = 0; c < D; ++c) out_k[((size_t)p * rows + x) * D + c] = Ok[(size_t)p * D + c];
        lse_k[(size_t)p * rows + x] = Lk[p];
      }
    }
  });
  return 0;
}

}  // extern "C"
