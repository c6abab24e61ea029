// tile_core.h — the attention tile engine shared by every kernel of the library.
//
// One workgroup = 4 wave64s = one tile of 64 query rows. Keys arrive in tiles of
// 64 rows staged through LDS (double-buffered, register prefetch of the next
// tile). Each wave owns 16 query rows and computes, per key tile,
//
//   S^T (64 keys x 16 queries) = K_tile . Q^T       (MFMA, fp32 accumulate)
//   online softmax on S^T in the log2 domain        (registers, fp32)
//   O^T (64 d x 16 queries)   += V_tile^T . P^T     (MFMA, fp32 accumulate)
//
// The S^T orientation puts one query column per lane (16 keys per lane, the
// other keys of that query in the three lanes 16, 32, 48 apart), so the row
// max needs only two cross-lane steps and the row sum none until the end.
// The same lane layout is exactly the B operand that the PV product needs
// (after a fixed permutation of the key order, applied to V^T as well).
//
// Layouts of the CDNA3/CDNA4 MFMA operands used here (lane l, g = l / 16):
//   v_mfma_f32_16x16x32_bf16: A[m = l%16][k = 8g..8g+7], B[k = 8g..8g+7][n = l%16],
//                             C[m = 4g..4g+3][n = l%16].
//   v_mfma_f32_16x16x4_f32:   A[m = l%16][k = g], B[k = g][n = l%16], C as above.
//
// This engine computes exact masked softmax attention (LongNet page, §3.4
// "Standard Self-Attention and Sparse Attention (Preliminaries)", Eq. 2) with
// the softmax kept in fp32 (Longformer page, §3.4 "Autoregressive Language
// Modeling Configuration": attention in fp32 to avoid overflow).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kTQ = 64;       // query rows per workgroup
constexpr int kTK = 64;       // keys per key tile
constexpr int kD = 64;        // head dimension
constexpr int kThreads = 256; // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// LDS row pitches (elements). Padding keeps the MFMA operand reads free of
// most bank conflicts.
constexpr int kKPitchBf16 = 72;  // K tile [key][d], 144 B rows
constexpr int kVPitchBf16 = 68;  // V^T tile [d][key], 136 B rows
constexpr int kPitchF32 = 68;    // fp32 K and V tiles [key][d], 272 B rows

// A sequence of rows of one [N, D] matrix: either positions base + stride*x
// for x < count, or positions idx[x] for x < count (a gather).
struct RowMap {
  const int32_t* idx;  // non-null for a gather
  int32_t base;
  int32_t stride;
  int32_t count;
  __device__ __forceinline__ int32_t pos(int32_t x) const {
    return idx ? idx[x] : base + stride * x;
  }
};

// Per-element mask/bias rules of one key tile (positions are sequence
// positions of the query row i and key row j).
enum TileKind : int32_t {
  kBand = 0,    // sliding-window tile in strided index space
  kGlobCol = 1, // global-column tile: keys are global tokens outside the band
  kAll = 2,     // plain range of keys (global rows): causal only
  kSeg = 3,     // LongNet gathered segment: causal in gathered index
};

struct MaskRule {
  int32_t kind;
  int32_t need_mask;  // 0: every (query, key) of the tile is allowed
  int32_t causal;
  int32_t radius;     // band half-width in dilation steps
  int32_t dil;        // dilation of the head
  int32_t qoff;       // kBand / kSeg: strided index of query row 0 minus that of key row 0
};

// fp32 -> bf16 with round-to-nearest-even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Membership of p in the strictly increasing array g[0..n).
__device__ __forceinline__ bool sorted_contains(const int32_t* g, int32_t n, int32_t p) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    int32_t x = g[mid];
    if (x == p) return true;
    if (x < p) lo = mid + 1; else hi = mid;
  }
  return false;
}

// Is (query position i, key position j) allowed by the rule? kq/kk are the
// row indices inside the tiles.
__device__ __forceinline__ bool allowed(const MaskRule& r, int32_t qi, int32_t kj, int32_t i,
                                        int32_t j, int32_t kcount) {
  if (kj >= kcount) return false;
  switch (r.kind) {
    case kBand: {
      // strided index difference key - query
      const int32_t dlt = kj - qi - r.qoff;
      if (r.causal) return dlt <= 0 && dlt >= -r.radius;
      return dlt >= -r.radius && dlt <= r.radius;
    }
    case kGlobCol: {
      if (r.causal && j > i) return false;
      const int32_t dl = j - i;
      const bool in_band = (dl % r.dil == 0) && (dl / r.dil <= r.radius) &&
                           (dl / r.dil >= -r.radius) && (!r.causal || dl <= 0);
      return !in_band;  // the band tile already counted it
    }
    case kAll:
      return !r.causal || j <= i;
    default: {  // kSeg
      const int32_t dlt = kj - qi - r.qoff;
      return !r.causal || dlt <= 0;
    }
  }
}

// Bias source: the scalar relative-position table of one head (ETC page,
// §3.4 "Relative Position Encoding": labels clip j - i to [-k, k]).
struct BiasRule {
  const float* tab;   // LDS copy of the head's 2k+1 entries, or null
  int32_t k;
  int32_t key_global_is_same_kind;  // 1: pair is same-kind iff the key is global
};

template <typename T>
struct TileTraits;

// ---------------------------------------------------------------------------
// bf16 engine
// ---------------------------------------------------------------------------
template <>
struct TileTraits<bf16> {
  struct Smem {
    bf16 k[2][kTK][kKPitchBf16];
    bf16 vt[2][kD][kVPitchBf16];
    int32_t kpos[2][kTK];
    uint8_t kglob[2][kTK];
    float bias[64];
  };
  struct Prefetch {
    u32x4 k0, k1, v0, v1;
    int32_t pos;
    uint8_t glob;
  };
  struct Wave {
    bf16x8 qf[2];
    f32x4 o[4];
    float m;  // running max, log2 domain
    float l;  // this lane's share of the running sum
  };

  // Issue the global loads of one key tile into registers.
  static __device__ __forceinline__ void fetch(Prefetch& pf, const bf16* kb, const bf16* vb,
                                               const RowMap& km, int32_t tid, bool need_glob,
                                               const int32_t* gidx, int32_t n_global) {
    const int32_t kk = tid >> 2, ck = tid & 3;
    const int32_t vp = tid >> 3, cv = tid & 7;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (kk < km.count) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kb + (size_t)km.pos(kk) * kD + 16 * ck);
      pf.k0 = src[0];
      pf.k1 = src[1];
    } else {
      pf.k0 = z;
      pf.k1 = z;
    }
    const int32_t ka = 2 * vp, kb2 = 2 * vp + 1;
    pf.v0 = ka < km.count ? *reinterpret_cast<const u32x4*>(vb + (size_t)km.pos(ka) * kD + 8 * cv) : z;
    pf.v1 = kb2 < km.count ? *reinterpret_cast<const u32x4*>(vb + (size_t)km.pos(kb2) * kD + 8 * cv) : z;
    if (tid < kTK) {
      pf.pos = tid < km.count ? km.pos(tid) : 0;
      pf.glob = (need_glob && tid < km.count) ? (uint8_t)sorted_contains(gidx, n_global, pf.pos) : 0;
    }
  }

  // Move a prefetched tile into LDS buffer `buf` (V transposed to [d][key]).
  static __device__ __forceinline__ void stage(Smem& sm, int32_t buf, const Prefetch& pf,
                                               int32_t tid) {
    const int32_t kk = tid >> 2, ck = tid & 3;
    *reinterpret_cast<u32x4*>(&sm.k[buf][kk][16 * ck]) = pf.k0;
    *reinterpret_cast<u32x4*>(&sm.k[buf][kk][16 * ck + 8]) = pf.k1;
    const int32_t vp = tid >> 3, cv = tid & 7;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // two bf16 of one key share a dword; pair keys 2vp and 2vp+1
      const uint32_t a = pf.v0[e], b = pf.v1[e];
      const uint32_t lo = (a & 0xffffu) | (b << 16);
      const uint32_t hi = (a >> 16) | (b & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&sm.vt[buf][8 * cv + 2 * e][2 * vp]) = lo;
      *reinterpret_cast<uint32_t*>(&sm.vt[buf][8 * cv + 2 * e + 1][2 * vp]) = hi;
    }
    if (tid < kTK) {
      sm.kpos[buf][tid] = pf.pos;
      sm.kglob[buf][tid] = pf.glob;
    }
  }

  static __device__ __forceinline__ void load_q(Wave& w, const bf16* qb, const RowMap& qm,
                                                int32_t wave, int32_t lane) {
    const int32_t qq = 16 * wave + (lane & 15), g = lane >> 4;
    if (qq < qm.count) {
      const bf16x8* src = reinterpret_cast<const bf16x8*>(qb + (size_t)qm.pos(qq) * kD + 8 * g);
      w.qf[0] = src[0];
      w.qf[1] = src[4];
    } else {
      const bf16x8 z = {};
      w.qf[0] = z;
      w.qf[1] = z;
    }
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i) w.o[i] = zf;
    w.m = kNegInf;
    w.l = 0.f;
  }

  // S^T for this wave: s[kb][i] = K[16kb + 4g + i] . Q[16*wave + lane%16].
  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, f32x4 s[4]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[buf][16 * kb + r][32 * st + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w.qf[st], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }
  }

  // O^T += V^T . P^T with P in s[][] (already exponentiated).
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, const f32x4 p[4]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 pb;
      pb[0] = pack_bf16x2(p[2 * ks][0], p[2 * ks][1]);
      pb[1] = pack_bf16x2(p[2 * ks][2], p[2 * ks][3]);
      pb[2] = pack_bf16x2(p[2 * ks + 1][0], p[2 * ks + 1][1]);
      pb[3] = pack_bf16x2(p[2 * ks + 1][2], p[2 * ks + 1][3]);
      const bf16x8 b = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(&sm.vt[buf][16 * db + r][32 * ks + 4 * g]);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(&sm.vt[buf][16 * db + r][32 * ks + 16 + 4 * g]);
        u32x4 av;
        av[0] = v0[0];
        av[1] = v0[1];
        av[2] = v1[0];
        av[3] = v1[1];
        w.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), b,
                                                           w.o[db], 0, 0, 0);
      }
    }
  }

  // out row (16 lanes per row): this lane holds d = 16db + 4g + i.
  static __device__ __forceinline__ void store_row(bf16* dst, const f32x4 o[4], float inv,
                                                   int32_t lane) {
    const int32_t g = lane >> 4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      u32x2 pk;
      pk[0] = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      pk[1] = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      *reinterpret_cast<u32x2*>(dst + 16 * db + 4 * g) = pk;
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 engine (fp32 MFMA; P kept in fp32)
// ---------------------------------------------------------------------------
template <>
struct TileTraits<float> {
  struct Smem {
    float k[2][kTK][kPitchF32];
    float v[2][kTK][kPitchF32];
    int32_t kpos[2][kTK];
    uint8_t kglob[2][kTK];
    float bias[64];
  };
  struct Prefetch {
    u32x4 k[4], v[4];
    int32_t pos;
    uint8_t glob;
  };
  struct Wave {
    float qf[16];
    f32x4 o[4];
    float m;
    float l;
  };

  static __device__ __forceinline__ void fetch(Prefetch& pf, const float* kb, const float* vb,
                                               const RowMap& km, int32_t tid, bool need_glob,
                                               const int32_t* gidx, int32_t n_global) {
    const int32_t kk = tid >> 2, c = tid & 3;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (kk < km.count) {
      const size_t row = (size_t)km.pos(kk) * kD + 16 * c;
      const u32x4* ks = reinterpret_cast<const u32x4*>(kb + row);
      const u32x4* vs = reinterpret_cast<const u32x4*>(vb + row);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pf.k[x] = ks[x];
        pf.v[x] = vs[x];
      }
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pf.k[x] = z;
        pf.v[x] = z;
      }
    }
    if (tid < kTK) {
      pf.pos = tid < km.count ? km.pos(tid) : 0;
      pf.glob = (need_glob && tid < km.count) ? (uint8_t)sorted_contains(gidx, n_global, pf.pos) : 0;
    }
  }

  static __device__ __forceinline__ void stage(Smem& sm, int32_t buf, const Prefetch& pf,
                                               int32_t tid) {
    const int32_t kk = tid >> 2, c = tid & 3;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      *reinterpret_cast<u32x4*>(&sm.k[buf][kk][16 * c + 4 * x]) = pf.k[x];
      *reinterpret_cast<u32x4*>(&sm.v[buf][kk][16 * c + 4 * x]) = pf.v[x];
    }
    if (tid < kTK) {
      sm.kpos[buf][tid] = pf.pos;
      sm.kglob[buf][tid] = pf.glob;
    }
  }

  // The contraction over d runs in the order d = 16g + step, so each lane
  // reads 16 contiguous floats of its Q row and of each K row.
  static __device__ __forceinline__ void load_q(Wave& w, const float* qb, const RowMap& qm,
                                                int32_t wave, int32_t lane) {
    const int32_t qq = 16 * wave + (lane & 15), g = lane >> 4;
    if (qq < qm.count) {
      const float* src = qb + (size_t)qm.pos(qq) * kD + 16 * g;
#pragma unroll
      for (int x = 0; x < 16; ++x) w.qf[x] = src[x];
    } else {
#pragma unroll
      for (int x = 0; x < 16; ++x) w.qf[x] = 0.f;
    }
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i) w.o[i] = zf;
    w.m = kNegInf;
    w.l = 0.f;
  }

  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, f32x4 s[4]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* krow = &sm.k[buf][16 * kb + r][16 * g];
#pragma unroll
      for (int st = 0; st < 16; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(krow[st], w.qf[st], acc, 0, 0, 0);
      s[kb] = acc;
    }
  }

  // k-slot g of step (kb, i) is key 16kb + 4g + i: A = V[key][d = 16db + r].
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, const f32x4 p[4]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vrow = &sm.v[buf][16 * kb + 4 * g + i][r];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          w.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], p[kb][i], w.o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store_row(float* dst, const f32x4 o[4], float inv,
                                                   int32_t lane) {
    const int32_t g = lane >> 4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4 x = o[db] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = x;
    }
  }
};

// ---------------------------------------------------------------------------
// One key tile through the online softmax (shared by both engines).
// qpos: this lane's query position; qi: its row index in the query tile.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void process_tile(const typename TileTraits<T>::Smem& sm, int32_t buf,
                                             typename TileTraits<T>::Wave& w, int32_t lane,
                                             const MaskRule& mr, const BiasRule& br, int32_t kcount,
                                             int32_t qi, int32_t qpos, float scale_log2) {
  using TT = TileTraits<T>;
  f32x4 s[4];
  TT::scores(sm, buf, w, lane, s);
  const int32_t g = lane >> 4;
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t kj = 16 * kb + 4 * g + i;
      float t = s[kb][i] * scale_log2;
      if (br.tab) {
        const int32_t j = sm.kpos[buf][kj];
        const bool kglob = sm.kglob[buf][kj] != 0;
        if (kglob == (br.key_global_is_same_kind != 0)) {
          int32_t dl = j - qpos;
          dl = dl < -br.k ? -br.k : (dl > br.k ? br.k : dl);
          t += br.tab[dl + br.k] * kLog2e;
        }
      }
      if (mr.need_mask && !allowed(mr, qi, kj, qpos, sm.kpos[buf][kj], kcount)) t = kNegInf;
      s[kb][i] = t;
      mx = fmaxf(mx, t);
    }
  }
  mx = wave_max_xor16_32(mx);
  const float m_new = fmaxf(w.m, mx);
  // A row with every key masked so far keeps m = -inf; shift by 0 then.
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(w.m - m_use);
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[kb][i] - m_use);
      s[kb][i] = p;
      rs += p;
    }
  }
  w.m = m_new;
  w.l = w.l * alpha + rs;
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] *= alpha;
  TT::accumulate(sm, buf, w, lane, s);
}

// The key-tile loop: tiles 0..n_tiles-1 described by desc(n, RowMap&, MaskRule&).
template <typename T, typename Desc>
__device__ __forceinline__ void run_tiles(typename TileTraits<T>::Smem& sm,
                                          typename TileTraits<T>::Wave& w, const T* kb,
                                          const T* vb, int32_t n_tiles, Desc desc,
                                          const BiasRule& br, bool need_glob,
                                          const int32_t* gidx, int32_t n_global, int32_t qi,
                                          int32_t qpos, float scale_log2) {
  using TT = TileTraits<T>;
  const int32_t tid = threadIdx.x, lane = tid & 63;
  if (n_tiles <= 0) return;
  typename TT::Prefetch pf;
  RowMap km;
  MaskRule mr;
  desc(0, km, mr);
  TT::fetch(pf, kb, vb, km, tid, need_glob, gidx, n_global);
  TT::stage(sm, 0, pf, tid);
  __syncthreads();
  for (int32_t n = 0; n < n_tiles; ++n) {
    const int32_t buf = n & 1;
    RowMap km_next;
    MaskRule mr_next;
    const bool more = n + 1 < n_tiles;
    if (more) {
      desc(n + 1, km_next, mr_next);
      TT::fetch(pf, kb, vb, km_next, tid, need_glob, gidx, n_global);
    }
    process_tile<T>(sm, buf, w, lane, mr, br, km.count, qi, qpos, scale_log2);
    if (more) {
      TT::stage(sm, buf ^ 1, pf, tid);
      km = km_next;
      mr = mr_next;
    }
    __syncthreads();
  }
}

}  // namespace la
