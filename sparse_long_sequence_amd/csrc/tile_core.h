// tile_core.h — the attention tile engine shared by every kernel of the library.
//
// One workgroup = 4 wave64s = one tile of query rows (128 for bf16, 64 for
// fp32). Keys arrive in tiles of 64 rows staged through LDS (double-buffered,
// register prefetch of the next tile). Each wave owns kQW query rows and
// computes, per key tile,
//
//   S^T (64 keys x kQW queries) = K_tile . Q^T      (MFMA, fp32 accumulate)
//   online softmax on S^T in the log2 domain        (registers, fp32)
//   O^T (64 d x kQW queries)   += V_tile^T . P^T    (MFMA, fp32 accumulate)
//
// The S^T orientation puts one query column per lane (its other keys sit in
// the lane 32 apart for bf16, in the lanes 16/32/48 apart for fp32), so the
// row max needs one (bf16) or two (fp32) cross-lane swaps and the row sum none
// until the end. The same lane layout is exactly the B operand of the PV
// product (after a fixed permutation of the key order, applied to V^T too).
//
// MFMA operand layouts used here (lane l; measured on gfx950):
//   v_mfma_f32_32x32x16_bf16: A[m = l%32][k = 8h..8h+7], B[k = 8h..8h+7][n = l%32],
//                             C[m = 8j + 4h + i][n = l%32] in element 4j+i, h = l/32.
//   v_mfma_f32_16x16x4_f32:   A[m = l%16][k = g], B[k = g][n = l%16],
//                             C[m = 4g + i][n = l%16] in element i, g = l/16.
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
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kTK = 64;       // keys per key tile
constexpr int kD = 64;        // head dimension
constexpr int kThreads = 256; // 4 waves
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kInvScale = 8.0f;  // sqrt(kD): the bias table is stored in q.k units
constexpr int kGMaskWords = 256;   // LDS bitmap of global positions: 8192 key rows
constexpr int32_t kFar = 0x3fffffff;

// LDS row pitches (elements). Padding keeps the MFMA operand reads free of
// most bank conflicts.
constexpr int kKPitchBf16 = 72;  // K tile [key][d], 144 B rows
constexpr int kVPitchBf16 = 68;  // V^T tile [d][key], 136 B rows
constexpr int kPitchF32 = 68;    // fp32 K and V tiles [key][d], 272 B rows

// fp32 -> bf16, round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum with the lane 32 (resp. 16) apart: gfx950 v_permlane32_swap and
// v_permlane16_swap exchange half-waves (resp. rows of 16) in registers. With
// a = b = x, afterwards {a, b} = {x[l], x[l ^ 32]} (resp. ^16) in every lane.
// Issued through inline asm: this compiler folds max/add of the two results
// of the builtins to the first result, which drops the partner lane. The
// s_nop 1 pairs cover the VALU -> permlane -> VALU dependency wait states.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xor32_max(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a = x, b = x;
  permlane32_swap(a, b);
  return a + b;
}
__device__ __forceinline__ float xor16_max(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor16_sum(float x) {
  float a = x, b = x;
  permlane16_swap(a, b);
  return a + b;
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

// Key rows of one tile: positions base + stride*x (strided view) or idx[x]
// (gather through the global index list), for x < count (count >= 1).
struct KeyTile {
  const int32_t* idx;
  int32_t base, stride, count;
  int32_t gbit0;  // bit of row 0 in the workgroup's global bitmap (strided tiles)
};

// Which (query, key) pairs of a tile are allowed.
//   kRange:   key row kj of the tile, reference ref = (use_qpos ? qpos : qi) + ref_off;
//             allowed iff kj < count and lo <= kj - ref <= hi.
//   kGlobCol: key j = global position outside the query's window (j <= i if causal).
enum MaskKind : int32_t { kRange = 0, kGlobCol = 1 };

struct MaskRule {
  int32_t kind;
  int32_t need_mask;  // 0: every (query, key) of the tile is allowed
  int32_t use_qpos;
  int32_t ref_off;
  int32_t lo, hi;
  // kGlobCol only
  int32_t causal, radius, dil;
};

// How the per-key "is global" flags of a tile are found (needed by the bias).
enum GlobMode : int32_t { kGlobNone = 0, kGlobBitmap = 1, kGlobSearch = 2, kGlobAll = 3 };

struct GlobInfo {
  int32_t mode;
  const int32_t* gidx;
  int32_t n_global;
};

// Bias source: the scalar relative-position table of one head (ETC page,
// §3.4 "Relative Position Encoding": labels clip j - i to [-k, k]).
struct BiasRule {
  const float* tab;   // LDS copy of the head's 2k+1 entries (times sqrt(D)), or null
  int32_t k;
  int32_t key_global_is_same_kind;  // 1: pair is same-kind iff the key is global
};

// Position of key row x of a tile (x clamped into [0, count) by the caller).
template <bool GATHER>
__device__ __forceinline__ int32_t key_pos(const KeyTile& kt, int32_t x) {
  if constexpr (GATHER) return kt.idx[x];
  else return kt.base + kt.stride * x;
}

// Per-key metadata: position and bit index in the global bitmap.
struct KeyMeta {
  int32_t pos;
  int32_t gbit;
};

// Per-thread element offsets of a full strided tile (stride fixed per loop).
struct FetchPlan {
  int32_t ok, oa, ob;  // K row chunk, V row chunks of the key pair
};

template <typename T>
struct TileTraits;

// ---------------------------------------------------------------------------
// bf16 engine: 32 queries per wave, v_mfma_f32_32x32x16_bf16
// ---------------------------------------------------------------------------
template <>
struct TileTraits<bf16> {
  static constexpr int kQW = 32;        // query rows per wave
  static constexpr int kTQ = 4 * kQW;   // query rows per workgroup
  static constexpr int kNS = 32;        // scores per lane per key tile

  // 16-byte alignment lets the operand reads use ds_read_b128 / ds_read_b64.
  struct __attribute__((aligned(16))) Smem {
    alignas(16) bf16 k[2][kTK][kKPitchBf16];
    alignas(16) bf16 vt[2][kD][kVPitchBf16];
    alignas(16) int32_t kpos[2][kTK];
    alignas(16) float bias[64];
    alignas(16) uint32_t gmask[kGMaskWords];
    alignas(16) uint8_t kglob[2][kTK];
  };
  struct Prefetch {
    u32x4 k0, k1, v0, v1;
    KeyMeta meta;
  };
  struct Wave {
    bf16x8 qf[4];
    f32x16 o[2];
    float m;  // running max, log2 domain
    float l;  // this lane's share of the running sum
  };

  static __device__ __forceinline__ int32_t qrow(int32_t wave, int32_t lane) {
    return kQW * wave + (lane & 31);
  }
  // Key row of score element r: a constant part and a lane part.
  static __device__ __forceinline__ constexpr int32_t key_const(int r) {
    return 32 * (r >> 4) + 8 * ((r >> 2) & 3) + (r & 3);
  }
  static __device__ __forceinline__ int32_t key_lane(int32_t lane) { return 4 * (lane >> 5); }
  static __device__ __forceinline__ float row_max(float x) { return xor32_max(x); }
  static __device__ __forceinline__ float row_sum(float x) { return xor32_sum(x); }
  // one lane per query row writes the row's scalars
  static __device__ __forceinline__ bool row_leader(int32_t lane) { return lane < 32; }

  static __device__ __forceinline__ FetchPlan plan(int32_t stride, int32_t tid) {
    FetchPlan p;
    p.ok = (tid >> 2) * stride * kD + 16 * (tid & 3);
    p.oa = 2 * (tid >> 3) * stride * kD + 8 * (tid & 7);
    p.ob = p.oa + stride * kD;
    return p;
  }

  // Issue the global loads of one key tile into registers. Rows past the
  // tile's end re-read its last row: those keys are masked, and a valid row
  // keeps every value finite.
  template <bool GATHER>
  static __device__ __forceinline__ void fetch(Prefetch& pf, const bf16* kb, const bf16* vb,
                                               const KeyTile& kt, const FetchPlan& fp,
                                               int32_t tid) {
    const int32_t last = kt.count - 1;
    const bf16 *pk, *pa, *pb;
    if (!GATHER && kt.count == kTK) {
      const size_t b0 = (size_t)kt.base * kD;
      pk = kb + b0 + fp.ok;
      pa = vb + b0 + fp.oa;
      pb = vb + b0 + fp.ob;
    } else {
      pk = kb + (size_t)key_pos<GATHER>(kt, min(tid >> 2, last)) * kD + 16 * (tid & 3);
      pa = vb + (size_t)key_pos<GATHER>(kt, min(2 * (tid >> 3), last)) * kD + 8 * (tid & 7);
      pb = vb + (size_t)key_pos<GATHER>(kt, min(2 * (tid >> 3) + 1, last)) * kD + 8 * (tid & 7);
    }
    const u32x4* ks = reinterpret_cast<const u32x4*>(pk);
    pf.k0 = ks[0];
    pf.k1 = ks[1];
    pf.v0 = *reinterpret_cast<const u32x4*>(pa);
    pf.v1 = *reinterpret_cast<const u32x4*>(pb);
    if (tid < kTK) {
      pf.meta.pos = key_pos<GATHER>(kt, min(tid, last));
      pf.meta.gbit = kt.gbit0 + min(tid, last);
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
      *reinterpret_cast<uint32_t*>(&sm.vt[buf][8 * cv + 2 * e][2 * vp]) =
          __builtin_amdgcn_perm(b, a, 0x05040100u);
      *reinterpret_cast<uint32_t*>(&sm.vt[buf][8 * cv + 2 * e + 1][2 * vp]) =
          __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
  }

  static __device__ __forceinline__ void load_q(Wave& w, const bf16* qb, int32_t qrow_pos,
                                                int32_t lane) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(qb + (size_t)qrow_pos * kD + 8 * (lane >> 5));
#pragma unroll
    for (int st = 0; st < 4; ++st) w.qf[st] = src[2 * st];
    const f32x16 zf = {};
    w.o[0] = zf;
    w.o[1] = zf;
    w.m = kNegInf;
    w.l = 0.f;
  }

  // S^T for this wave: s[16kb + e] = K[key_const(16kb+e) + key_lane] . Q[qrow].
  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, float s[kNS]) {
    const int32_t r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * kb + r][16 * st + 8 * h]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[st], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s[16 * kb + e] = acc[e];
    }
  }

  // O^T += V^T . P^T with P in p[] (already exponentiated). MFMA step (kb, t)
  // takes the 16 keys 32kb + 16t + [0, 16): this lane's p[16kb + 8t + 0..7].
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, const float p[kNS]) {
    const int32_t r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e0 = 16 * kb + 8 * t;
        u32x4 pb;
        pb[0] = pack_bf16x2(p[e0 + 0], p[e0 + 1]);
        pb[1] = pack_bf16x2(p[e0 + 2], p[e0 + 3]);
        pb[2] = pack_bf16x2(p[e0 + 4], p[e0 + 5]);
        pb[3] = pack_bf16x2(p[e0 + 6], p[e0 + 7]);
        const bf16x8 b = __builtin_bit_cast(bf16x8, pb);
        const int c0 = 32 * kb + 16 * t + 4 * h;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(&sm.vt[buf][32 * db + r][c0]);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(&sm.vt[buf][32 * db + r][c0 + 8]);
          u32x4 av;
          av[0] = v0[0];
          av[1] = v0[1];
          av[2] = v1[0];
          av[3] = v1[1];
          w.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), b,
                                                             w.o[db], 0, 0, 0);
        }
      }
    }
  }

  // Output row of this lane's query; the lane holds d = 32db + 8j + 4h + i.
  static __device__ __forceinline__ void store_row(bf16* dst, const Wave& w, float inv,
                                                   int32_t lane) {
    const int32_t h = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 pk;
        pk[0] = pack_bf16x2(w.o[db][4 * j + 0] * inv, w.o[db][4 * j + 1] * inv);
        pk[1] = pack_bf16x2(w.o[db][4 * j + 2] * inv, w.o[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * j + 4 * h) = pk;
      }
    }
  }
  // Same, fp32 (partials of split computations).
  static __device__ __forceinline__ void store_row_f32(float* dst, const Wave& w, float inv,
                                                       int32_t lane) {
    const int32_t h = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
        for (int i = 0; i < 4; ++i) x[i] = w.o[db][4 * j + i] * inv;
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * h) = x;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 engine: 16 queries per wave, fp32 MFMA; P kept in fp32
// ---------------------------------------------------------------------------
template <>
struct TileTraits<float> {
  static constexpr int kQW = 16;
  static constexpr int kTQ = 4 * kQW;
  static constexpr int kNS = 16;

  struct __attribute__((aligned(16))) Smem {
    alignas(16) float k[2][kTK][kPitchF32];
    alignas(16) float v[2][kTK][kPitchF32];
    alignas(16) int32_t kpos[2][kTK];
    alignas(16) float bias[64];
    alignas(16) uint32_t gmask[kGMaskWords];
    alignas(16) uint8_t kglob[2][kTK];
  };
  struct Prefetch {
    u32x4 k[4], v[4];
    KeyMeta meta;
  };
  struct Wave {
    float qf[16];
    f32x4 o[4];
    float m;
    float l;
  };

  static __device__ __forceinline__ int32_t qrow(int32_t wave, int32_t lane) {
    return kQW * wave + (lane & 15);
  }
  static __device__ __forceinline__ constexpr int32_t key_const(int r) {
    return 16 * (r >> 2) + (r & 3);
  }
  static __device__ __forceinline__ int32_t key_lane(int32_t lane) { return 4 * (lane >> 4); }
  static __device__ __forceinline__ float row_max(float x) { return xor32_max(xor16_max(x)); }
  static __device__ __forceinline__ float row_sum(float x) { return xor32_sum(xor16_sum(x)); }
  static __device__ __forceinline__ bool row_leader(int32_t lane) { return lane < 16; }

  static __device__ __forceinline__ FetchPlan plan(int32_t stride, int32_t tid) {
    FetchPlan p;
    p.ok = (tid >> 2) * stride * kD + 16 * (tid & 3);
    p.oa = p.ok;
    p.ob = p.ok;
    return p;
  }

  template <bool GATHER>
  static __device__ __forceinline__ void fetch(Prefetch& pf, const float* kb, const float* vb,
                                               const KeyTile& kt, const FetchPlan& fp,
                                               int32_t tid) {
    const int32_t last = kt.count - 1;
    size_t row;
    if (!GATHER && kt.count == kTK)
      row = (size_t)kt.base * kD + fp.ok;
    else
      row = (size_t)key_pos<GATHER>(kt, min(tid >> 2, last)) * kD + 16 * (tid & 3);
    const u32x4* ks = reinterpret_cast<const u32x4*>(kb + row);
    const u32x4* vs = reinterpret_cast<const u32x4*>(vb + row);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pf.k[x] = ks[x];
      pf.v[x] = vs[x];
    }
    if (tid < kTK) {
      pf.meta.pos = key_pos<GATHER>(kt, min(tid, last));
      pf.meta.gbit = kt.gbit0 + min(tid, last);
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
  }

  // The contraction over d runs in the order d = 16g + step, so each lane
  // reads 16 contiguous floats of its Q row and of each K row.
  static __device__ __forceinline__ void load_q(Wave& w, const float* qb, int32_t qrow_pos,
                                                int32_t lane) {
    const float* src = qb + (size_t)qrow_pos * kD + 16 * (lane >> 4);
#pragma unroll
    for (int x = 0; x < 16; ++x) w.qf[x] = src[x];
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i) w.o[i] = zf;
    w.m = kNegInf;
    w.l = 0.f;
  }

  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, float s[kNS]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* krow = &sm.k[buf][16 * kb + r][16 * g];
#pragma unroll
      for (int st = 0; st < 16; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(krow[st], w.qf[st], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * kb + i] = acc[i];
    }
  }

  // k-slot g of step (kb, i) is key 16kb + 4g + i: A = V[key][d = 16db + r].
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, const float p[kNS]) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vrow = &sm.v[buf][16 * kb + 4 * g + i][r];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          w.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], p[4 * kb + i], w.o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store_row(float* dst, const Wave& w, float inv,
                                                   int32_t lane) {
    const int32_t g = lane >> 4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4 x = w.o[db] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = x;
    }
  }
  static __device__ __forceinline__ void store_row_f32(float* dst, const Wave& w, float inv,
                                                       int32_t lane) {
    store_row(dst, w, inv, lane);
  }
};

// Per-key position and global flag of a staged tile (tid < 64 write them).
template <typename T>
__device__ __forceinline__ void stage_meta(typename TileTraits<T>::Smem& sm, int32_t buf,
                                           const KeyMeta& mt, const GlobInfo& gi, int32_t tid) {
  if (tid < kTK) {
    sm.kpos[buf][tid] = mt.pos;
    uint8_t f = 0;
    if (gi.mode == kGlobBitmap)
      f = (uint8_t)((sm.gmask[mt.gbit >> 5] >> (mt.gbit & 31)) & 1u);
    else if (gi.mode == kGlobSearch)
      f = (uint8_t)sorted_contains(gi.gidx, gi.n_global, mt.pos);
    else if (gi.mode == kGlobAll)
      f = 1;
    sm.kglob[buf][tid] = f;
  }
}

// Mark in sm.gmask the rows u in [0, count) whose position base + stride*u is
// global. Needs count <= 32 * kGMaskWords. Ends with a barrier.
template <typename T>
__device__ __forceinline__ void build_gmask(typename TileTraits<T>::Smem& sm, const int32_t* gidx,
                                            int32_t n_global, int32_t base, int32_t stride,
                                            int32_t count, int32_t tid) {
  for (int32_t x = tid; x < kGMaskWords; x += kThreads) sm.gmask[x] = 0u;
  __syncthreads();
  for (int32_t x = tid; x < n_global; x += kThreads) {
    const int32_t dl = gidx[x] - base;
    if (dl >= 0 && dl % stride == 0 && dl / stride < count) {
      const int32_t u = dl / stride;
      atomicOr(&sm.gmask[u >> 5], 1u << (u & 31));
    }
  }
  __syncthreads();
}

// Scores stay raw dot products q.k until the exponent; the bias table in LDS
// is pre-multiplied by sqrt(D) so that it adds in the same units.
template <typename T>
__device__ __forceinline__ void add_bias(float* s, const typename TileTraits<T>::Smem& sm,
                                         int32_t buf, const BiasRule& br, int32_t qpos,
                                         int32_t lane) {
  using TT = TileTraits<T>;
  const int32_t kl = TT::key_lane(lane);
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(r) + kl;
    const bool same = (sm.kglob[buf][kj] != 0) == (br.key_global_is_same_kind != 0);
    const int32_t dl = min(max(sm.kpos[buf][kj] - qpos, -br.k), br.k);
    const float b = br.tab[dl + br.k];  // always read: keeps the loop branch-free
    s[r] += same ? b : 0.f;
  }
}

// Set excluded (query, key) pairs of a partial tile to -inf. One uniform
// branch per tile; the per-element tests are a few integer ops.
template <typename T>
__device__ __forceinline__ void mask_tile(float* s, const typename TileTraits<T>::Smem& sm,
                                          int32_t buf, const MaskRule& mr, int32_t kcount,
                                          int32_t qi, int32_t qpos, int32_t lane) {
  using TT = TileTraits<T>;
  const int32_t kl = TT::key_lane(lane);
  if (mr.kind == kRange) {
    const int32_t base = kl - (mr.use_qpos ? qpos : qi) - mr.ref_off;
#pragma unroll
    for (int r = 0; r < TT::kNS; ++r) {
      const int32_t kj = TT::key_const(r) + kl;
      const int32_t dlt = base + TT::key_const(r);
      const bool ok = (kj < kcount) & (dlt >= mr.lo) & (dlt <= mr.hi);
      s[r] = ok ? s[r] : kNegInf;
    }
  } else {  // kGlobCol
#pragma unroll
    for (int r = 0; r < TT::kNS; ++r) {
      const int32_t kj = TT::key_const(r) + kl;
      const int32_t dl = sm.kpos[buf][kj] - qpos;
      const bool in_band = (dl % mr.dil == 0) & (dl >= -mr.radius * mr.dil) &
                           (dl <= mr.radius * mr.dil) & (!mr.causal | (dl <= 0));
      const bool ok = (kj < kcount) & (!mr.causal | (dl <= 0)) & !in_band;
      s[r] = ok ? s[r] : kNegInf;
    }
  }
}

// The running max moves only when a row's tile max exceeds it by more than
// this many log2 units; p = 2^(t - m) then stays below 2^8, and the final
// O = sum p v / sum p is unchanged, so most tiles skip the O rescale.
constexpr float kRescaleSlack = 8.0f;

template <typename W>
__device__ __forceinline__ void scale_acc(W& w, float alpha);
template <>
__device__ __forceinline__ void scale_acc(TileTraits<bf16>::Wave& w, float alpha) {
  w.o[0] *= alpha;
  w.o[1] *= alpha;
}
template <>
__device__ __forceinline__ void scale_acc(TileTraits<float>::Wave& w, float alpha) {
#pragma unroll
  for (int db = 0; db < 4; ++db) w.o[db] *= alpha;
}

// One key tile through the online softmax (shared by both engines).
// qpos: this lane's query position; qi: its row index in the query tile.
template <typename T>
__device__ __forceinline__ void process_tile(const typename TileTraits<T>::Smem& sm, int32_t buf,
                                             typename TileTraits<T>::Wave& w, int32_t lane,
                                             const MaskRule& mr, const BiasRule& br, int32_t kcount,
                                             int32_t qi, int32_t qpos, float scale_log2) {
  using TT = TileTraits<T>;
  float s[TT::kNS];
  TT::scores(sm, buf, w, lane, s);
  if (br.tab) add_bias<T>(s, sm, buf, br, qpos, lane);
  if (mr.need_mask) mask_tile<T>(s, sm, buf, mr, kcount, qi, qpos, lane);
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < TT::kNS; ++r) mx = fmaxf(mx, s[r]);
  mx = TT::row_max(mx);
  const float mt = mx * scale_log2;  // tile max in log2 units (-inf if all masked)
  const bool up = mt > w.m + kRescaleSlack;
  if (__ballot(up) != 0ull) {
    const float alpha = !up ? 1.f : (w.m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(w.m - mt));
    w.m = up ? mt : w.m;
    w.l *= alpha;
    scale_acc(w, alpha);
  }
  // A row with every key masked so far keeps m = -inf; shift by 0 then.
  const float nm = (w.m == kNegInf) ? 0.f : -w.m;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, nm));
    s[r] = p;
    rs += p;
  }
  w.l += rs;
  TT::accumulate(sm, buf, w, lane, s);
}

// The key-tile loop: tiles 0..n_tiles-1 described by desc(n, KeyTile&, MaskRule&),
// all strided with one stride or all gathered (GATHER).
template <typename T, bool GATHER, typename Desc>
__device__ __forceinline__ void run_tiles(typename TileTraits<T>::Smem& sm,
                                          typename TileTraits<T>::Wave& w, const T* kb,
                                          const T* vb, int32_t n_tiles, Desc desc,
                                          const BiasRule& br, const GlobInfo& gi, int32_t qi,
                                          int32_t qpos, float scale_log2) {
  using TT = TileTraits<T>;
  const int32_t tid = threadIdx.x, lane = tid & 63;
  if (n_tiles <= 0) return;
  typename TT::Prefetch pf;
  KeyTile kt;
  MaskRule mr;
  desc(0, kt, mr);
  const FetchPlan fp = TT::plan(kt.stride, tid);
  TT::template fetch<GATHER>(pf, kb, vb, kt, fp, tid);
  TT::stage(sm, 0, pf, tid);
  stage_meta<T>(sm, 0, pf.meta, gi, tid);
  __syncthreads();
  for (int32_t n = 0; n < n_tiles; ++n) {
    const int32_t buf = n & 1;
    KeyTile kt_next;
    MaskRule mr_next;
    const bool more = n + 1 < n_tiles;
    if (more) {
      desc(n + 1, kt_next, mr_next);
      TT::template fetch<GATHER>(pf, kb, vb, kt_next, fp, tid);
    }
    process_tile<T>(sm, buf, w, lane, mr, br, kt.count, qi, qpos, scale_log2);
    if (more) {
      TT::stage(sm, buf ^ 1, pf, tid);
      stage_meta<T>(sm, buf ^ 1, pf.meta, gi, tid);
      kt = kt_next;
      mr = mr_next;
    }
    __syncthreads();
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin (block b on XCD b % 8).
// Map them so that each XCD runs one contiguous range of logical tiles: query
// tiles of one head then share K/V tiles in that XCD's L2. The grid is padded
// to a multiple of 8; returns -1 for a padding block.
constexpr int32_t kXcds = 8;
__device__ __forceinline__ int32_t xcd_logical_block(int32_t b, int32_t total) {
  const int32_t per = (total + kXcds - 1) / kXcds;
  const int32_t lg = (b % kXcds) * per + b / kXcds;
  return lg < total ? lg : -1;
}

}  // namespace la
