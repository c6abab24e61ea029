// tile_core.h — the attention tile engine shared by every kernel of the library.
//
// One workgroup = one tile of query rows (128 for bf16, 64 for fp32). Keys
// arrive in tiles of 64 rows, double-buffered in LDS; the next tile's loads
// are issued while the current one computes (bf16: straight from global
// memory into LDS; fp32: through registers). Each wave owns kQW query rows,
// held as kQB blocks of 32 (bf16) or 16 (fp32) rows, and computes, per key
// sub-tile,
//
//   S^T (keys x queries) = K_sub . Q^T                (MFMA, fp32 accumulate)
//   online softmax on S^T in the log2 domain          (registers, fp32)
//   O^T (64 d x queries) += V_sub^T . P^T             (MFMA, fp32 accumulate)
//
// The S^T orientation puts one query column per lane (its other keys sit in
// the lane 32 apart for bf16, in the lanes 16/32/48 apart for fp32), so the
// row max needs one (bf16) or two (fp32) cross-lane swaps and the row sum none
// until the end. The same lane layout is exactly the B operand of the PV
// product, once the A operand (V^T) takes its keys in the matching order.
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
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// The running max of a row before any allowed key: far below any real
// score (log2 units), so that the first allowed key always moves it and keys
// masked to -inf give p = 0 against it, without tests for -inf.
constexpr float kMFloor = -1e30f;
constexpr float kInvScale = 8.0f;  // sqrt(kD): the bias table is stored in q.k units
constexpr int kGMaskWords = 256;   // LDS bitmap of global positions: 8192 key rows
constexpr int32_t kFar = 0x3fffffff;

// LDS row pitch of the fp32 K and V tiles [key][d] (elements): 272-byte rows
// put the operand reads of consecutive rows on disjoint banks.
constexpr int kPitchF32 = 68;

// 16-byte load from global memory. The explicit address space makes it a
// global_load: through a generic pointer the compiler may emit a flat_load,
// which also counts against the LDS wait counter, so every later wait for an
// LDS read would wait for this load as well.
typedef const u32x4 __attribute__((address_space(1)))* gptr_u32x4;
typedef const u32x2 __attribute__((address_space(1)))* gptr_u32x2;
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(gptr_u32x4)(p); }
__device__ __forceinline__ u32x2 ldg8(const void* p) { return *(gptr_u32x2)(p); }

// Buffer loads: a 128-bit resource (base address, size, format) held in
// scalar registers, a per-lane 32-bit byte offset and a uniform 32-bit byte
// offset. Per-lane address state is one register per load instead of a 64-bit
// pointer. Word 3 selects 32-bit data format for untyped loads.
constexpr int32_t kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufWord3);
}
__device__ __forceinline__ u32x4 ldb16(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 ldb8(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Device-coherent buffer stores and loads (cache policy sc1): a store is
// written through to memory, a load does not return a line another XCD's
// writes may have made stale. Workgroups on different XCDs can then hand data
// to each other through an atomic counter without writing back or
// invalidating a whole L2.
constexpr int32_t kCoherent = 16;  // sc1
__device__ __forceinline__ void st_coh16(__amdgpu_buffer_rsrc_t r, int32_t voff, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, 0, kCoherent);
}
__device__ __forceinline__ void st_coh4(__amdgpu_buffer_rsrc_t r, int32_t voff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, 0, kCoherent);
}
__device__ __forceinline__ f32x4 ld_coh16(__amdgpu_buffer_rsrc_t r, int32_t voff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCoherent));
}
__device__ __forceinline__ float ld_coh4(__amdgpu_buffer_rsrc_t r, int32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, kCoherent));
}

// fp32 -> bf16, round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pk, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, acc, false);
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

// Index of p in the strictly increasing array g[0..n), or -1.
__device__ __forceinline__ int32_t sorted_index(const int32_t* g, int32_t n, int32_t p) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    int32_t x = g[mid];
    if (x == p) return mid;
    if (x < p) lo = mid + 1; else hi = mid;
  }
  return -1;
}

// Key rows of one tile: positions base + stride*x (strided view) or idx[x]
// (gather through the global index list), for x < count (count >= 1).
struct KeyTile {
  const int32_t* idx;
  int32_t base, stride, count;  // count 0: nothing to load, every query block is empty
  int32_t gbit0;  // bit of row 0 in the workgroup's global bitmap (strided tiles)
  int32_t gmode;  // how the keys' "is global" flags are found (GlobMode)
  // 1 + the global rank of key row 0 when the tile's keys are global tokens of
  // consecutive ranks (per-pair label rows are then read contiguously), else 0
  int32_t rank_run;
};

// Which (query, key) pairs of a tile are allowed.
//   kRange:   key row kj of the tile, reference ref = (use_qpos ? qpos : qi) + ref_off;
//             allowed iff kj < count and lo <= kj - ref <= hi.
//   kGlobCol: key j = global position outside the query's window (j <= i if causal).
//   kOutside: as kRange with the interval's complement: kj < count and
//             kj - ref < lo or kj - ref > hi.
enum MaskKind : int32_t { kRange = 0, kGlobCol = 1, kOutside = 2 };

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
  // Per-instance segment masks (packed documents; ETC page, §3.4 "Per-instance
  // attention masks"): the batch row's segment id per position, or null; this
  // lane's query row's id and the min / max id over the wave's rows.
  const int32_t* segb;
  int32_t sq, sq_min, sq_max;
};

// min / max over the 64 lanes of a wave
__device__ __forceinline__ int32_t wave_min(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Bias source (ETC page, §3.4 "Relative Position Encoding": labels clip
// j - i to [-k, k]): the head's table of 2k+1 scalars, or, with key-side label
// vectors a_l, a table per query row of q_i . a_l (plus the scalar when both
// are given), the precompute the page describes.
struct BiasRule {
  const float* tab;   // LDS, in q.k units (scalars times sqrt(D)), or null
  int32_t k;
  int32_t key_global_is_same_kind;  // 1: pair is same-kind iff the key is global
  int32_t row_stride;               // 0: one table; else query row qi's table at tab + qi * row_stride
};

// Structured inputs (only the kernels built for them read this). Per-pair
// labels (ETC page, §3.4 "Relative Position Encoding", Step 1 and its
// implementation note; a masked label is an entry M = 0 of "Per-instance
// attention masks"), or lab = null. Global query rows (rows_global): row qi's
// labels are lab[min(qi, row_last) * stride + key position] (the lanes past
// the workgroup's last row read that row's); non-global rows: the labels of
// their global keys are lab[qpos * stride + key's global rank] (want_rank:
// the tiles stage each key's rank). seg_g / seg_l: the segment ids mask the
// pairs whose key is global / non-global.
struct LabelRule {
  const uint8_t* lab;
  int32_t rows_global;
  int32_t row_last;  // rows_global: the workgroup's last query row
  uint32_t stride;
  int32_t V;  // vocabulary size: a label >= V other than kLabelDist masks the pair
  int32_t want_rank;
  int32_t seg_g, seg_l;
};

// A per-pair label value keeping the pair's usual clipped-distance label.
constexpr int32_t kLabelDist = 0xFE;

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
  int32_t ok;  // this thread's K chunk
  int32_t ov;  // this thread's first V chunk
  int32_t rs;  // elements between consecutive key rows
};

template <typename T>
struct TileTraits;

// ---------------------------------------------------------------------------
// bf16 engine: 4 waves x 32 queries, v_mfma_f32_32x32x16_bf16
// ---------------------------------------------------------------------------
template <>
struct TileTraits<bf16> {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQB = 1;              // one 32-row query block per wave
  static constexpr int kQW = 32;             // query rows per wave
  static constexpr int kTQ = kWaves * kQW;   // query rows per workgroup
  static constexpr int kSub = 2;             // key sub-tiles of 32 keys
  static constexpr int kSubKeys = kTK / kSub;
  static constexpr int kNS = 16;             // scores per lane and sub-tile
  static constexpr int kRowsPerBlock = 32;   // lanes 0..31 hold the block's rows in order
  static constexpr int kMinWavesPerEU = 4;

  // K and V tiles are kept as loaded, [key][d] in 128-byte rows, and go from
  // global memory straight into LDS (no register staging). The 16-byte chunk
  // c of row k sits at chunk position c ^ swz(k), so that both the K operand
  // reads (one chunk of 16 consecutive rows) and the transposing V reads (two
  // chunks of 4 consecutive rows) fall on distinct banks.
  struct __attribute__((aligned(16))) Smem {
    alignas(16) bf16 k[2][kTK * kD];
    alignas(16) bf16 v[2][kTK * kD];
    alignas(16) int32_t kpos[2][kTK];
    alignas(16) float bias[64];
    alignas(16) uint32_t gmask[kGMaskWords];
    alignas(16) uint8_t kglob[2][kTK];
    alignas(16) int32_t kseg[2][kTK];  // segment ids of the staged keys (segment masks only)
    alignas(16) int32_t kgrank[2][kTK];  // the keys' index in the global list, -1 if not global (labels only)
    int32_t segr[2][2];                // per staged tile: min and max of kseg
    int32_t gcls[2];  // per staged tile: bit 0 some key is global, bit 1 every key is
  };
  struct Prefetch {
    KeyMeta meta;
  };
  struct Wave {
    bf16x8 qf[4];
    f32x16 o[2];
    float m[kQB];  // running max, log2 domain
    float l[kQB];  // this lane's share of the running sum
  };
  // P of one sub-tile as bf16: the B operands of its two PV MFMA steps.
  struct PTile {
    u32x4 p[2];
  };

  // Chunk-position swizzle of row k (depends on k mod 16): within 8 aligned
  // rows it is a permutation of 0..7, the 8 even (odd) rows of 16 aligned rows
  // take distinct values, and for 4 aligned rows bits 1-2 are distinct while
  // bit 2 differs between rows k and k + 2.
  static __device__ __forceinline__ int32_t swz(int32_t k) {
    return (((k & 3) << 1) | ((k >> 2) & 1)) ^ ((k >> 2) & 2);
  }

  static __device__ __forceinline__ int32_t qrow(int32_t wave, int32_t lane, int) {
    return kQW * wave + (lane & 31);
  }
  // Key row of score element r of sub-tile sb: a constant part and a lane part.
  static __device__ __forceinline__ constexpr int32_t key_const(int sb, int r) {
    return 32 * sb + 8 * (r >> 2) + (r & 3);
  }
  static __device__ __forceinline__ int32_t key_lane(int32_t lane) { return 4 * (lane >> 5); }
  static __device__ __forceinline__ float row_max(float x) { return xor32_max(x); }
  static __device__ __forceinline__ float row_sum(float x) { return xor32_sum(x); }
  // one lane per query row writes the row's scalars
  static __device__ __forceinline__ bool row_leader(int32_t lane) { return lane < 32; }

  // Wave w loads the key rows 16w + 8i + (lane >> 3), i = 0, 1, of both K and
  // V; lane l writes chunk position l & 7 of its row, so it reads the chunk
  // (l & 7) ^ swz(row). ok / ov: byte offsets of the two reads from the start
  // of a full strided tile.
  static __device__ __forceinline__ int32_t load_row(int32_t tid, int i) {
    return 16 * (tid >> 6) + 8 * i + ((tid & 63) >> 3);
  }
  static __device__ __forceinline__ int32_t load_chunk(int32_t tid, int i) {
    return (tid & 7) ^ swz(load_row(tid, i));
  }
  static __device__ __forceinline__ FetchPlan plan(int32_t stride, int32_t tid) {
    FetchPlan p;
    p.rs = stride * kD;
    p.ok = (load_row(tid, 0) * p.rs + 8 * load_chunk(tid, 0)) * 2;
    p.ov = (load_row(tid, 1) * p.rs + 8 * load_chunk(tid, 1)) * 2;
    return p;
  }

  // 16 bytes per lane from a buffer into LDS at dst + 16 * lane (dst uniform).
  static __device__ __forceinline__ void to_lds(__amdgpu_buffer_rsrc_t r, bf16* dst, int32_t voff,
                                                int32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                             voff, soff, 0, 0);
  }

  // Issue the loads of one key tile into LDS buffer `buf` (buffer loads
  // relative to the head's K and V; byte offsets fit in 32 bits for N < 2^24).
  // Rows past the tile's end re-read its last row: those keys are masked, and
  // a valid row keeps every value finite. `buf` must not be read until
  // stage() and a barrier have followed.
  template <bool GATHER>
  static __device__ __forceinline__ void fetch(Prefetch& pf, Smem& sm, int32_t buf,
                                               const bf16* kb, const bf16* vb,
                                               const KeyTile& kt, const FetchPlan& fp,
                                               int32_t tid) {
    if (kt.count <= 0) return;
    const __amdgpu_buffer_rsrc_t rk = buffer_of(kb), rv = buffer_of(vb);
    const int32_t last = kt.count - 1;
    // the destination is per wave: uniform, so it is formed in scalar registers
    const int32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    bf16* kd = &sm.k[buf][16 * wv * kD];
    bf16* vd = &sm.v[buf][16 * wv * kD];
    if (!GATHER && kt.count == kTK) {
      const int32_t sb = kt.base * (kD * 2);  // tile base, bytes (uniform)
      to_lds(rk, kd, fp.ok, sb);
      to_lds(rk, kd + 8 * kD, fp.ov, sb);
      to_lds(rv, vd, fp.ok, sb);
      to_lds(rv, vd + 8 * kD, fp.ov, sb);
    } else {
      // lane values recomputed here from an opaque copy of tid: kept across the
      // loop they would be spilled, and a spill reload waits for the loads
      // just issued
      int32_t t = tid;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int32_t off =
            (key_pos<GATHER>(kt, min(load_row(t, i), last)) * kD + 8 * load_chunk(t, i)) * 2;
        to_lds(rk, kd + 8 * i * kD, off, 0);
        to_lds(rv, vd + 8 * i * kD, off, 0);
      }
    }
    if (tid < kTK) {
      pf.meta.pos = key_pos<GATHER>(kt, min(tid, last));
      pf.meta.gbit = kt.gbit0 + min(tid, last);
    }
  }

  // The tile's loads have landed in LDS for this wave (a barrier must follow
  // before other waves read them).
  static __device__ __forceinline__ void stage(Smem&, int32_t, const Prefetch&, int32_t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }

  static __device__ __forceinline__ void load_q(Wave& w, const bf16* qb, const int32_t* qpos,
                                                int32_t lane) {
    const bf16* src = qb + (size_t)qpos[0] * kD + 8 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < 4; ++st) w.qf[st] = __builtin_bit_cast(bf16x8, ldg16(src + 16 * st));
    const f32x16 zf = {};
    w.o[0] = zf;
    w.o[1] = zf;
    w.m[0] = kMFloor;
    w.l[0] = 0.f;
  }

  // S^T of sub-tile sb: s[e] = K[key_const(sb, e) + key_lane] . Q[qrow].
  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, int sb, float s[kNS]) {
    const int32_t r = lane & 31, h = lane >> 5;
    const int32_t y = h ^ swz(r);  // chunk 2st + h of row r sits at position 2st ^ y
    const bf16* row = &sm.k[buf][(32 * sb + r) * kD];
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(row + 8 * ((2 * st) ^ y));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[st], acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < kNS; ++e) s[e] = acc[e];
  }

  // p = 2^(s * c + nm) rounded to bf16; the row sum adds exactly these values.
  // The wave runs this exponential stretch at raised issue priority: with
  // several waves on a SIMD, the one in its VALU phase then issues ahead of
  // waves that are starting their next MFMAs, which keeps both pipes busier
  // (the forward's headline shape runs about 4% faster, the unmasked
  // R = 4096 band about 5%).
  static __device__ __forceinline__ void softmax_p(const float s[kNS], float nm, float c,
                                                   PTile& P, float& l) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * t + 2 * i], c, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * t + 2 * i + 1], c, nm));
        const uint32_t pk = pack_bf16x2(p0, p1);
        P.p[t][i] = pk;
        l = add_bf16x2(pk, l);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // O^T += V^T . P^T over sub-tile sb. MFMA step t takes the keys
  // 32sb + 16t + [0, 16): in k-slot 8h + e the key 32sb + 16t + 8(e >> 2) + 4h + (e & 3),
  // i.e. this lane's score elements 8t + e. The A operand (V^T, d = 32db + l % 32)
  // comes from two ds_read_b64_tr_b16: in each group of 16 lanes, lane L
  // addresses d 4(L & 3)..+3 of key K0 + L / 4 and receives keys K0..K0+3 of
  // its own d.
  //
  // The reads are issued through inline asm that also waits for them: for the
  // builtin, the compiler cannot tell that the read does not touch the LDS
  // buffer the next tile is being loaded into, and waits for those loads
  // first, which leaves the prefetch only part of a tile to land. Both key
  // steps' reads go out together, so the sub-tile waits for LDS once.
  static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  }
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, int sb, const PTile& P) {
    typedef short __attribute__((__vector_size__(4 * sizeof(short)))) s16x4;
    const int32_t L = lane & 15, g = (lane >> 4) & 1, h = lane >> 5;
    const int32_t kr = 4 * h + (L >> 2);  // key row mod 16 of the first read; +8 for the second
    const int32_t u = (2 * g + ((L & 3) >> 1)) ^ swz(kr);
    const bf16* base = &sm.v[0][kr * kD + 4 * (L & 1)];
    // lane addresses of the (d block, key half) reads; buffer, sub-tile and
    // step go into the instruction's offset
    const uint32_t a00 = lds_addr(base + 8 * (0 ^ u));
    const uint32_t a01 = lds_addr(base + 8 * kD + 8 * (0 ^ u ^ 2));
    const uint32_t a10 = lds_addr(base + 8 * (4 ^ u));
    const uint32_t a11 = lds_addr(base + 8 * kD + 8 * (4 ^ u ^ 2));
    const int32_t off = (buf * kTK * kD + (32 * sb) * kD) * 2;  // bytes
    constexpr int32_t o16 = 16 * kD * 2;  // the second key step
    s16x4 lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo0), "=&v"(hi0), "=&v"(lo1), "=&v"(hi1), "=&v"(lo2), "=&v"(hi2), "=&v"(lo3), "=&v"(hi3)
        : "v"(a00), "v"(a01), "v"(a10), "v"(a11), "i"(off), "i"(off + o16));
    {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo0, hi0, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo1, hi1, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 b = __builtin_bit_cast(bf16x8, P.p[0]);
      w.o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, w.o[0], 0, 0, 0);
      w.o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, w.o[1], 0, 0, 0);
    }
    {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo3, hi3, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 b = __builtin_bit_cast(bf16x8, P.p[1]);
      w.o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, w.o[0], 0, 0, 0);
      w.o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, w.o[1], 0, 0, 0);
    }
  }

  static __device__ __forceinline__ void scale_acc(Wave& w, float alpha) {
    w.o[0] *= alpha;
    w.o[1] *= alpha;
  }

  // Waves w and w + 2 (w = 0, 1) held the same query rows over different key
  // sub-tiles: fold the running state of wave w + 2 into wave w through LDS
  // (reusing the K/V buffers). Each side's O and l are relative to its own
  // reference max; both are rescaled to the larger one. Call from all waves
  // after the tile loop; waves 2 and 3 are spent afterwards.
  static __device__ __forceinline__ void fold_pairs(Smem& sm, Wave& w, int32_t wave,
                                                    int32_t lane) {
    float* xo = reinterpret_cast<float*>(&sm.k[0][0]);  // [2][32][64]: 16 KB
    float* xs = reinterpret_cast<float*>(&sm.v[0][0]);  // [2][2][64]
    __syncthreads();  // every wave is done with the last staged tile
    if (wave >= 2) {
      const int32_t p = wave - 2;
#pragma unroll
      for (int e = 0; e < 32; ++e) xo[(p * 32 + e) * 64 + lane] = w.o[e >> 4][e & 15];
      xs[(p * 2 + 0) * 64 + lane] = w.m[0];
      xs[(p * 2 + 1) * 64 + lane] = w.l[0];
    }
    __syncthreads();
    if (wave < 2) {
      const float mb = xs[(wave * 2 + 0) * 64 + lane], lb = xs[(wave * 2 + 1) * 64 + lane];
      const float ma = w.m[0];
      const float m = fmaxf(ma, mb);
      const float sa = __builtin_amdgcn_exp2f(ma - m);  // 0 for a side at the floor
      const float sb = __builtin_amdgcn_exp2f(mb - m);
#pragma unroll
      for (int e = 0; e < 32; ++e)
        w.o[e >> 4][e & 15] = w.o[e >> 4][e & 15] * sa + xo[(wave * 32 + e) * 64 + lane] * sb;
      w.l[0] = w.l[0] * sa + lb * sb;
      w.m[0] = m;
    }
  }

  // Output row of this lane's query; the lane holds d = 32db + 8j + 4h + i.
  static __device__ __forceinline__ void store_row(bf16* dst, const Wave& w, int, float inv,
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
  static __device__ __forceinline__ void store_row_f32(float* dst, const Wave& w, int, float inv,
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
  // Same, device-coherent: the row at byte offset voff of buffer r.
  // byte offset voff of buffer r.
  static __device__ __forceinline__ void store_row_coh(__amdgpu_buffer_rsrc_t r, int32_t voff,
                                                       const Wave& w, float inv, int32_t lane) {
    const int32_t h = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
        for (int i = 0; i < 4; ++i) x[i] = w.o[db][4 * j + i] * inv;
        st_coh16(r, voff + 4 * (32 * db + 8 * j + 4 * h), __builtin_bit_cast(u32x4, x));
      }
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 engine: 4 waves x 16 queries, fp32 MFMA; P kept in fp32
// ---------------------------------------------------------------------------
template <>
struct TileTraits<float> {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQB = 1;
  static constexpr int kQW = 16;
  static constexpr int kTQ = kWaves * kQW;
  static constexpr int kSub = 1;
  static constexpr int kSubKeys = kTK / kSub;
  static constexpr int kNS = 16;
  static constexpr int kRowsPerBlock = 16;
  static constexpr int kMinWavesPerEU = 2;

  struct __attribute__((aligned(16))) Smem {
    alignas(16) float k[2][kTK][kPitchF32];
    alignas(16) float v[2][kTK][kPitchF32];
    alignas(16) int32_t kpos[2][kTK];
    alignas(16) float bias[64];
    alignas(16) uint32_t gmask[kGMaskWords];
    alignas(16) uint8_t kglob[2][kTK];
    alignas(16) int32_t kseg[2][kTK];  // segment ids of the staged keys (segment masks only)
    alignas(16) int32_t kgrank[2][kTK];  // the keys' index in the global list, -1 if not global (labels only)
    int32_t segr[2][2];                // per staged tile: min and max of kseg
    int32_t gcls[2];  // per staged tile: bit 0 some key is global, bit 1 every key is
  };
  struct Prefetch {
    u32x4 k[4], v[4];
    KeyMeta meta;
  };
  struct Wave {
    float qf[16];
    f32x4 o[4];
    float m[kQB];
    float l[kQB];
  };
  struct PTile {
    float p[kNS];
  };

  static __device__ __forceinline__ int32_t qrow(int32_t wave, int32_t lane, int) {
    return kQW * wave + (lane & 15);
  }
  static __device__ __forceinline__ constexpr int32_t key_const(int, int r) {
    return 16 * (r >> 2) + (r & 3);
  }
  static __device__ __forceinline__ int32_t key_lane(int32_t lane) { return 4 * (lane >> 4); }
  static __device__ __forceinline__ float row_max(float x) { return xor32_max(xor16_max(x)); }
  static __device__ __forceinline__ float row_sum(float x) { return xor32_sum(xor16_sum(x)); }
  static __device__ __forceinline__ bool row_leader(int32_t lane) { return lane < 16; }

  static __device__ __forceinline__ FetchPlan plan(int32_t stride, int32_t tid) {
    FetchPlan p;
    p.rs = stride * kD;
    p.ok = (tid >> 2) * p.rs + 16 * (tid & 3);
    p.ov = p.ok;
    return p;
  }

  template <bool GATHER>
  static __device__ __forceinline__ void fetch(Prefetch& pf, Smem&, int32_t, const float* kb,
                                               const float* vb,
                                               const KeyTile& kt, const FetchPlan& fp,
                                               int32_t tid) {
    if (kt.count <= 0) return;
    const int32_t last = kt.count - 1;
    size_t row;
    if (!GATHER && kt.count == kTK)
      row = (size_t)kt.base * kD + fp.ok;
    else
      row = (size_t)key_pos<GATHER>(kt, min(tid >> 2, last)) * kD + 16 * (tid & 3);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pf.k[x] = ldg16(kb + row + 4 * x);
      pf.v[x] = ldg16(vb + row + 4 * x);
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
  static __device__ __forceinline__ void load_q(Wave& w, const float* qb, const int32_t* qpos,
                                                int32_t lane) {
    const float* src = qb + (size_t)qpos[0] * kD + 16 * (lane >> 4);
#pragma unroll
    for (int x = 0; x < 16; ++x) w.qf[x] = src[x];
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i) w.o[i] = zf;
    w.m[0] = kMFloor;
    w.l[0] = 0.f;
  }

  static __device__ __forceinline__ void scores(const Smem& sm, int32_t buf, const Wave& w,
                                                int32_t lane, int, float s[kNS]) {
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

  static __device__ __forceinline__ void softmax_p(const float s[kNS], float nm, float c,
                                                   PTile& P, float& l) {
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < kNS; ++r) {
      P.p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, nm));
      rs += P.p[r];
    }
    l += rs;
  }

  // k-slot g of step (kb, i) is key 16kb + 4g + i: A = V[key][d = 16db + r].
  static __device__ __forceinline__ void accumulate(const Smem& sm, int32_t buf, Wave& w,
                                                    int32_t lane, int, const PTile& P) {
    const int32_t r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vrow = &sm.v[buf][16 * kb + 4 * g + i][r];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          w.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], P.p[4 * kb + i], w.o[db], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void scale_acc(Wave& w, float alpha) {
#pragma unroll
    for (int db = 0; db < 4; ++db) w.o[db] *= alpha;
  }

  static __device__ __forceinline__ void store_row(float* dst, const Wave& w, int, float inv,
                                                   int32_t lane) {
    const int32_t g = lane >> 4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4 x = w.o[db] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = x;
    }
  }
  static __device__ __forceinline__ void store_row_coh(__amdgpu_buffer_rsrc_t r, int32_t voff,
                                                       const Wave& w, float inv, int32_t lane) {
    const int32_t g = lane >> 4;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4 x = w.o[db] * inv;
      st_coh16(r, voff + 4 * (16 * db + 4 * g), __builtin_bit_cast(u32x4, x));
    }
  }
};

// Per-key position and global flag of a staged tile (tid < 64 write them);
// SEG: also the keys' segment ids and their range, when gi has them; LBL: the
// keys' global ranks, when gi asks for them.
template <typename T, bool SEG, bool LBL>
__device__ __forceinline__ void stage_meta(typename TileTraits<T>::Smem& sm, int32_t buf,
                                           const KeyMeta& mt, const GlobInfo& gi,
                                           const LabelRule& lr, int32_t mode, int32_t tid) {
  if (tid < kTK) {
    sm.kpos[buf][tid] = mt.pos;
    uint8_t f = 0;
    if (mode == kGlobBitmap)
      f = (uint8_t)((sm.gmask[mt.gbit >> 5] >> (mt.gbit & 31)) & 1u);
    else if (mode == kGlobSearch)
      f = (uint8_t)sorted_contains(gi.gidx, gi.n_global, mt.pos);
    else if (mode == kGlobAll)
      f = 1;
    sm.kglob[buf][tid] = f;
    if constexpr (LBL) {
      if (lr.want_rank) sm.kgrank[buf][tid] = f ? sorted_index(gi.gidx, gi.n_global, mt.pos) : -1;
    }
    if (mode != kGlobNone) {
      // the rows past the tile's end repeat its last key, so the whole wave
      // (tid < 64) gives the tile's any / all
      const uint64_t g = __ballot(f != 0);
      if (tid == 0) sm.gcls[buf] = (g != 0ull ? 1 : 0) | (g == ~0ull ? 2 : 0);
    }
    if (SEG && gi.segb) {  // the keys' segment ids and their range (wave 0: tid < 64)
      const int32_t sk = gi.segb[mt.pos];
      sm.kseg[buf][tid] = sk;
      const int32_t mn = wave_min(sk), mx = wave_max(sk);
      if (tid == 0) {
        sm.segr[buf][0] = mn;
        sm.segr[buf][1] = mx;
      }
    }
  }
}

// Mark in sm.gmask the rows u in [0, count) whose position base + stride*u is
// global. Needs count <= 32 * kGMaskWords. Ends with a barrier.
template <typename T>
__device__ __forceinline__ void build_gmask(typename TileTraits<T>::Smem& sm, const int32_t* gidx,
                                            int32_t n_global, int32_t base, int32_t stride,
                                            int32_t count, int32_t tid) {
  constexpr int32_t nt = TileTraits<T>::kThreads;
  for (int32_t x = tid; x < kGMaskWords; x += nt) sm.gmask[x] = 0u;
  __syncthreads();
  for (int32_t x = tid; x < n_global; x += nt) {
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
// all_same: every key of the tile is of the query's kind (no per-key test).
template <typename T>
__device__ __forceinline__ void add_bias(float* s, const typename TileTraits<T>::Smem& sm,
                                         int32_t buf, const BiasRule& br, int sb, int32_t qi,
                                         int32_t qpos, int32_t lane, bool all_same) {
  using TT = TileTraits<T>;
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call: keeps kl-derived per-element values out of loop-invariant hoisting
  const float* tab = br.tab + qi * br.row_stride + br.k;
  if (all_same) {
#pragma unroll
    for (int r = 0; r < TT::kNS; ++r) {
      const int32_t kj = TT::key_const(sb, r) + kl;
      const int32_t dl = min(max(sm.kpos[buf][kj] - qpos, -br.k), br.k);
      s[r] += tab[dl];
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(sb, r) + kl;
    const bool same = (sm.kglob[buf][kj] != 0) == (br.key_global_is_same_kind != 0);
    const int32_t dl = min(max(sm.kpos[buf][kj] - qpos, -br.k), br.k);
    const float b = tab[dl];  // always read: keeps the loop branch-free
    s[r] += same ? b : 0.f;
  }
}

// add_bias for a tile of consecutive positions whose keys are all of the
// query's kind: key kj sits at base + kj, so a pair's distance is
// (base - qpos) + kj with kj a compile-time constant plus the lane's part,
// and no key position is read from LDS.
template <typename T>
__device__ __forceinline__ void add_bias_run(float* s, const BiasRule& br, int sb, int32_t qi,
                                             int32_t off, int32_t lane) {
  using TT = TileTraits<T>;
  const int32_t c = off + TT::key_lane(lane);
  const float* tab = br.tab + qi * br.row_stride + br.k;
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t dl = min(max(c + TT::key_const(sb, r), -br.k), br.k);
    s[r] += tab[dl];
  }
}

// The labels of the lane's kNS pairs of sub-tile sb, four per word (element
// r in byte r & 3 of word r >> 2; the lane's keys come in runs of four):
// issued before the sub-tile's score MFMAs so that their latency overlaps
// them. Global query rows read their label row at the keys' positions (the
// tiles of the global-row pass are contiguous runs of positions); other rows
// read theirs at the keys' global ranks, contiguous for a run of global keys
// (kt.rank_run) and else looked up per key (kgrank, -1: not global, no label).
template <typename T>
__device__ __forceinline__ void load_labels(uint32_t lw[TileTraits<T>::kNS / 4],
                                            const typename TileTraits<T>::Smem& sm, int32_t buf,
                                            const LabelRule& lr, const KeyTile& kt, int sb,
                                            int32_t qi, int32_t qpos, int32_t lane) {
  using TT = TileTraits<T>;
  static_assert(TT::kNS % 4 == 0, "runs of four keys per lane");
  const int32_t kl = TT::key_lane(lane);
  const int32_t row = lr.rows_global ? min(qi, lr.row_last) : qpos;
  const uint8_t* lrow = lr.lab + (size_t)(uint32_t)row * lr.stride;
  const int32_t last = kt.count - 1;
  const bool run = lr.rows_global ? kt.stride == 1 : kt.rank_run > 0;
  if (run) {
    const uint8_t* lt = lrow + (lr.rows_global ? kt.base : kt.rank_run - 1);
    if (kt.count == kTK && ((uintptr_t)lt & 3) == 0) {
#pragma unroll
      for (int g = 0; g < TT::kNS / 4; ++g)
        lw[g] = *reinterpret_cast<const uint32_t*>(lt + TT::key_const(sb, 4 * g) + kl);
    } else {  // a ragged or unaligned run: byte loads, clamped into the tile
#pragma unroll
      for (int g = 0; g < TT::kNS / 4; ++g) {
        uint32_t x = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x |= (uint32_t)lt[min(TT::key_const(sb, 4 * g + e) + kl, last)] << (8 * e);
        lw[g] = x;
      }
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < TT::kNS / 4; ++g) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t kj = TT::key_const(sb, 4 * g + e) + kl;
      uint32_t b = (uint32_t)kLabelDist;
      if (lr.rows_global) {
        b = lrow[(uint32_t)sm.kpos[buf][kj]];
      } else {
        const int32_t gr = sm.kgrank[buf][kj];
        if (gr >= 0) b = lrow[(uint32_t)gr];
      }
      x |= b << (8 * e);
    }
    lw[g] = x;
  }
}

// Bias and masks from per-pair labels: a pair with an explicit label l < V
// takes table entry l (whatever its piece), kLabelDist keeps the usual
// distance label for same-kind pairs (none for mixed ones), and any other
// value masks the pair (-inf).
template <typename T>
__device__ __forceinline__ void add_bias_labels(float* s, const uint32_t* lw,
                                                const typename TileTraits<T>::Smem& sm,
                                                int32_t buf, const BiasRule& br,
                                                const LabelRule& lr, int sb, int32_t qi,
                                                int32_t qpos, int32_t lane) {
  using TT = TileTraits<T>;
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call, as in add_bias
  const float* tab = br.tab ? br.tab + qi * br.row_stride : nullptr;
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(sb, r) + kl;
    const int32_t lbl = (int32_t)((lw[r >> 2] >> (8 * (r & 3))) & 0xFFu);
    const bool same = (sm.kglob[buf][kj] != 0) == (br.key_global_is_same_kind != 0);
    const int32_t dl = min(max(sm.kpos[buf][kj] - qpos, -br.k), br.k);
    const int32_t idx = lbl == kLabelDist ? (same ? dl + br.k : -1) : lbl;
    const bool masked = lbl != kLabelDist && lbl >= lr.V;
    const float b = (tab && idx >= 0 && !masked) ? tab[idx] : 0.f;
    s[r] = masked ? kNegInf : s[r] + b;
  }
}

// Set excluded (query, key) pairs of a partial tile to -inf. One uniform
// branch per tile; the per-element tests are a few integer ops.
template <typename T>
__device__ __forceinline__ void mask_tile(float* s, const typename TileTraits<T>::Smem& sm,
                                          int32_t buf, const MaskRule& mr, int sb, int32_t kcount,
                                          int32_t qi, int32_t qpos, int32_t lane) {
  using TT = TileTraits<T>;
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call: keeps kl-derived per-element values out of loop-invariant hoisting
  if (mr.kind != kGlobCol) {
    // The lane's allowed key rows (kRange) or excluded ones (kOutside) form
    // one interval [a, a + span]; element r's row kj = key_const(sb, r) + kl
    // is inside iff (unsigned)(kj - a) <= (unsigned)span: one add, one compare.
    const int32_t ref = (mr.use_qpos ? qpos : qi) + mr.ref_off;
    int32_t a = ref + mr.lo, span = mr.hi - mr.lo;
    if (mr.kind == kRange) {
      span = min(ref + mr.hi, kcount - 1) - a;  // rows past the tile's end are excluded too
      // nothing allowed: an interval no row reaches
      a = span < 0 ? 0x40000000 : a;
      span = max(span, 0);
    }
    const int32_t c = kl - a;
    if (mr.kind == kRange) {
#pragma unroll
      for (int r = 0; r < TT::kNS; ++r) {
        const bool in = (uint32_t)(TT::key_const(sb, r) + c) <= (uint32_t)span;
        s[r] = in ? s[r] : kNegInf;
      }
    } else {
      const int32_t lim = kcount - kl;  // rows past the tile's end stay excluded
#pragma unroll
      for (int r = 0; r < TT::kNS; ++r) {
        const bool in = (uint32_t)(TT::key_const(sb, r) + c) <= (uint32_t)span;
        s[r] = (!in & (TT::key_const(sb, r) < lim)) ? s[r] : kNegInf;
      }
    }
  } else {  // kGlobCol
#pragma unroll
    for (int r = 0; r < TT::kNS; ++r) {
      const int32_t kj = TT::key_const(sb, r) + kl;
      const int32_t dl = sm.kpos[buf][kj] - qpos;
      const bool in_band = (dl % mr.dil == 0) & (dl >= -mr.radius * mr.dil) &
                           (dl <= mr.radius * mr.dil) & (!mr.causal | (dl <= 0));
      const bool ok = (kj < kcount) & (!mr.causal | (dl <= 0)) & !in_band;
      s[r] = ok ? s[r] : kNegInf;
    }
  }
}

// Exclude the pairs of sub-tile sb whose key lies in another segment than
// this lane's query row (segment masks).
// LBL: only the pieces gi names are checked (pairs with a global key: seg_g,
// with a non-global key: seg_l); otherwise every pair.
template <typename T, bool LBL>
__device__ __forceinline__ void mask_segments(float* s, const typename TileTraits<T>::Smem& sm,
                                              int32_t buf, int sb, const GlobInfo& gi,
                                              const LabelRule& lr, int32_t lane) {
  using TT = TileTraits<T>;
  int32_t kl = TT::key_lane(lane);
  asm("" : "+v"(kl));  // opaque per call, as in mask_tile
#pragma unroll
  for (int r = 0; r < TT::kNS; ++r) {
    const int32_t kj = TT::key_const(sb, r) + kl;
    bool check = true;
    if constexpr (LBL) check = sm.kglob[buf][kj] != 0 ? lr.seg_g != 0 : lr.seg_l != 0;
    s[r] = (!check || sm.kseg[buf][kj] == gi.sq) ? s[r] : kNegInf;
  }
}

// The running max moves only when a row's sub-tile max exceeds it by more
// than this many log2 units; p = 2^(t - m) then stays below 2^8, and the final
// O = sum p v / sum p is unchanged, so most sub-tiles skip the O rescale.
constexpr float kRescaleSlack = 8.0f;

// Which pairs of (query block, key sub-tile sb) a rule allows: 0 none,
// 1 all, 2 some. ref0 <= ref1 bound the block's reference values (the rule's
// query index or position plus ref_off, non-decreasing along the block).
enum BlockClass : int32_t { kEmpty = 0, kFull = 1, kPartial = 2 };

template <typename T>
__device__ __forceinline__ int32_t classify(const MaskRule& mr, int32_t kcount, int sb,
                                            int32_t ref0, int32_t ref1) {
  constexpr int32_t SK = TileTraits<T>::kSubKeys;
  const int32_t k0 = SK * sb, k1 = k0 + SK - 1;
  if (k0 >= kcount) return kEmpty;
  if (mr.kind == kGlobCol) return mr.need_mask ? kPartial : kFull;
  const int32_t dmin = k0 - ref1, dmax = k1 - ref0;
  const bool inside = dmin >= mr.lo && dmax <= mr.hi;  // every pair in [lo, hi]
  const bool apart = dmax < mr.lo || dmin > mr.hi;     // no pair in [lo, hi]
  if (mr.kind == kOutside) {
    if (inside) return kEmpty;
    return (k1 < kcount && apart) ? kFull : kPartial;
  }
  if (apart) return kEmpty;
  return (k1 < kcount && inside) ? kFull : kPartial;
}

// Online softmax and PV of key sub-tile sb given its final logits s (raw
// q.k, with bias, -inf where excluded). ADD: the logits are s + badd, badd
// the same for every pair of the sub-tile (folded into the row max and the
// exponent's shift instead of added to each score).
template <typename T, bool ADD = false>
__device__ __forceinline__ void sub_update(const typename TileTraits<T>::Smem& sm, int32_t buf,
                                           typename TileTraits<T>::Wave& w, int32_t lane, int sb,
                                           const float* s, float scale_log2, float badd = 0.f) {
  using TT = TileTraits<T>;
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < TT::kNS; ++r) mx = fmaxf(mx, s[r]);
  if constexpr (ADD) mx += badd;
  const float mxr = TT::row_max(mx);  // sub-tile max, q.k units (-inf if all masked)
  const float m_old = w.m[0];
  // the running max moves when the sub-tile's exceeds it by the slack
  const bool up = __builtin_fmaf(mxr, scale_log2, -m_old) > kRescaleSlack;
  if (__ballot(up) != 0ull) {
    const float mt = mxr * scale_log2;  // log2 units
    const float alpha = !up ? 1.f : __builtin_amdgcn_exp2f(m_old - mt);  // 0 from the floor
    w.m[0] = up ? mt : m_old;
    w.l[0] *= alpha;
    TT::scale_acc(w, alpha);
  }
  // A row with no allowed key so far keeps the floor: its keys here are all
  // masked (-inf), and p = 2^-inf = 0.
  float nm = -w.m[0];
  if constexpr (ADD) nm += badd * scale_log2;
  typename TT::PTile P;
  TT::softmax_p(s, nm, scale_log2, P, w.l[0]);
  TT::accumulate(sm, buf, w, lane, sb, P);
}

// One staged key tile through the online softmax (shared by both engines).
// qpos: this lane's query position; qi: its row index in the query tile;
// dead: the wave holds no valid query row (it only helps stage tiles).
//
// Each (wave's query block, key sub-tile) is classified from the block's row
// range. When every sub-tile is full and no bias applies, the fast path runs
// the sub-tiles one after the other with no mask or bias code. Otherwise each
// sub-tile is skipped (no allowed pair), or biased and masked as needed.
template <typename T, bool BIAS, bool SEG, bool LBL>
__device__ __forceinline__ void process_tile(const typename TileTraits<T>::Smem& sm, int32_t buf,
                                             typename TileTraits<T>::Wave& w, int32_t lane,
                                             const MaskRule& mr, const BiasRule& br,
                                             const GlobInfo& gi, const LabelRule& lr,
                                             const KeyTile& kt, bool strided,
                                             int32_t qi, int32_t qpos, bool dead,
                                             float scale_log2, int32_t only_sb) {
  using TT = TileTraits<T>;
  constexpr int SB = TT::kSub;
  const int32_t kcount = kt.count;
  // the block's first and last reference values (loop-invariant lane reads,
  // plus the tile's scalar offset)
  const int32_t r0 = (mr.use_qpos ? __builtin_amdgcn_readlane(qpos, 0)
                                  : __builtin_amdgcn_readlane(qi, 0)) + mr.ref_off;
  const int32_t r1 = (mr.use_qpos ? __builtin_amdgcn_readlane(qpos, TT::kRowsPerBlock - 1)
                                  : __builtin_amdgcn_readlane(qi, TT::kRowsPerBlock - 1)) + mr.ref_off;
  // Bias (ETC page, §3.4 "Relative Position Encoding": same-kind pairs only).
  // From the staged tile's global flags: no key of the query's kind means no
  // bias at all; every key of its kind means no per-key kind test.
  bool bias_on = false, all_same = false, lab_on = false;
  bool any_g = false, all_g = false;
  if constexpr (BIAS) {
    // (kGlobNone: no key is global, and the class word was not written)
    const int32_t gc = kt.gmode == kGlobNone ? 0 : __builtin_amdgcn_readfirstlane(sm.gcls[buf]);
    any_g = (gc & 1) != 0;
    all_g = (gc & 2) != 0;
    bias_on = br.tab != nullptr && (br.key_global_is_same_kind ? any_g : !all_g);
    if constexpr (LBL) {
      // per-pair labels: every pair of a global row, the global keys of others
      lab_on = lr.lab != nullptr && (lr.rows_global || any_g);
      bias_on = bias_on || lab_on;
    }
    all_same = br.key_global_is_same_kind ? all_g : !any_g;
  }
  // A tile every pair of which is allowed for all of the workgroup's rows
  // (the rule needs no mask) and that takes no bias is full for every wave
  // holding rows: a uniform test instead of the per-wave classification.
  int32_t cls[SB];
  bool fast = !bias_on;
  if (!bias_on && mr.need_mask == 0 && only_sb < 0) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) cls[sb] = dead ? kEmpty : kFull;
    fast = !dead;
  } else {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      cls[sb] = (dead || (only_sb >= 0 && sb != only_sb)) ? kEmpty : classify<T>(mr, kcount, sb, r0, r1);
      fast = fast && cls[sb] == kFull;
    }
  }
  // Segment masks (SEG): keys of one other segment only: nothing allowed;
  // keys and rows all of one segment: no change; otherwise every computed
  // sub-tile is masked per element.
  bool seg_check = false;
  if constexpr (SEG) {
    // LBL: the segment ids mask the pieces lr names only. A tile whose keys
    // are all of masked pieces is checked as usual, one with none of them not
    // at all, and one with keys of both per element.
    bool seg_some = true, seg_mixed = false;
    if constexpr (LBL) {
      const bool chk_g = lr.seg_g && any_g, chk_l = lr.seg_l && !all_g;
      const bool unchk = (!lr.seg_g && any_g) || (!lr.seg_l && !all_g);
      seg_some = chk_g || chk_l;
      seg_mixed = seg_some && unchk;
    }
    if (LBL && gi.segb && kcount > 0 && seg_mixed) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) cls[sb] = cls[sb] == kFull ? kPartial : cls[sb];
      fast = false;
      seg_check = true;
    } else if (gi.segb && kcount > 0 && seg_some) {
      const int32_t kmn = __builtin_amdgcn_readfirstlane(sm.segr[buf][0]);
      const int32_t kmx = __builtin_amdgcn_readfirstlane(sm.segr[buf][1]);
      if (kmx < gi.sq_min || kmn > gi.sq_max) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) cls[sb] = kEmpty;
        fast = false;
      } else if (!(kmn == kmx && gi.sq_min == gi.sq_max && kmn == gi.sq_min)) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) cls[sb] = cls[sb] == kFull ? kPartial : cls[sb];
        fast = false;
        seg_check = true;
      }
    }
  }
  if (fast) {
    // Every sub-tile's scores first: the later sub-tiles' score MFMAs then
    // run on the matrix core while this wave does the earlier ones' softmax.
    float s[SB][TT::kNS];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) TT::scores(sm, buf, w, lane, sb, s[sb]);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) sub_update<T>(sm, buf, w, lane, sb, s[sb], scale_log2);
    return;
  }
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) {
    if (cls[sb] == kEmpty) continue;  // no allowed pair: no scores, no softmax, no PV
    float s[TT::kNS];
    uint32_t lw[TT::kNS / 4];
    if (LBL && lab_on) load_labels<T>(lw, sm, buf, lr, kt, sb, qi, qpos, lane);
    TT::scores(sm, buf, w, lane, sb, s);
    float badd = 0.f;  // a bias shared by every pair of the sub-tile
    if (BIAS && bias_on) {
      // A strided sub-tile whose clipped distances are all +k (or all -k) for
      // the block's rows takes one table entry for every pair.
      bool uniform = false;
      int32_t ue = 0;
      if (strided && all_same && !lab_on) {
        constexpr int32_t SK = TT::kSubKeys;
        const int32_t q0 = __builtin_amdgcn_readlane(qpos, 0);
        const int32_t q1 = __builtin_amdgcn_readlane(qpos, TT::kRowsPerBlock - 1);
        const int32_t k0 = kt.base + kt.stride * (SK * sb);
        const int32_t k1 = kt.base + kt.stride * min(SK * sb + SK - 1, kcount - 1);
        if (k0 - q1 >= br.k) { uniform = true; ue = 2 * br.k; }
        else if (k1 - q0 <= -br.k) { uniform = true; ue = 0; }
      }
      if (LBL && lab_on) add_bias_labels<T>(s, lw, sm, buf, br, lr, sb, qi, qpos, lane);
      else if (uniform) badd = br.tab[qi * br.row_stride + ue];  // per query row with label vectors
      else if (strided && all_same && kt.stride == 1)
        add_bias_run<T>(s, br, sb, qi, kt.base - qpos, lane);
      else add_bias<T>(s, sm, buf, br, sb, qi, qpos, lane, all_same);
    }
    if (cls[sb] == kPartial) mask_tile<T>(s, sm, buf, mr, sb, kcount, qi, qpos, lane);
    if (SEG && seg_check) mask_segments<T, LBL>(s, sm, buf, sb, gi, lr, lane);
    sub_update<T, BIAS>(sm, buf, w, lane, sb, s, scale_log2, badd);
  }
}

// A compile-time LDS buffer index.
template <int32_t B>
struct BufTag {
  static constexpr int32_t value = B;
};

// The key-tile loop: tiles 0..n_tiles-1 described by desc(n, KeyTile&, MaskRule&),
// all strided with one stride or all gathered (GATHER); BIAS: br holds a bias
// table (compiled out otherwise); SEG: gi holds segment ids (compiled out
// otherwise); LBL: br may hold per-pair labels and gi may restrict the segment
// mask to some pieces (compiled out otherwise). only_sb >= 0: this
// wave computes only that key sub-tile of every tile (the others are left to
// other waves holding the same rows).
template <typename T, bool GATHER, bool BIAS, bool SEG, bool LBL, typename Desc>
__device__ __forceinline__ void run_tiles(typename TileTraits<T>::Smem& sm,
                                          typename TileTraits<T>::Wave& w, const T* kb,
                                          const T* vb, int32_t n_tiles, Desc desc,
                                          const BiasRule& br, const GlobInfo& gi,
                                          const LabelRule& lr, int32_t qi, int32_t qpos,
                                          bool dead, float scale_log2, int32_t only_sb = -1) {
  using TT = TileTraits<T>;
  const int32_t tid = threadIdx.x, lane = tid & 63;
  if (n_tiles <= 0) return;
  typename TT::Prefetch pf;
  KeyTile kt;
  MaskRule mr;
  desc(0, kt, mr);
  const FetchPlan fp = TT::plan(kt.stride, tid);
  TT::template fetch<GATHER>(pf, sm, 0, kb, vb, kt, fp, tid);
  TT::stage(sm, 0, pf, tid);
  stage_meta<T, SEG, LBL>(sm, 0, pf.meta, gi, lr, kt.gmode, tid);
  __syncthreads();
  // Tile n computes from LDS buffer n & 1 while tile n + 1 loads into the
  // other. The loop is unrolled by two so that the buffer of each step is a
  // compile-time constant: LDS addresses then fold into instruction offsets.
  auto step = [&](auto buf_tag, int32_t n) {
    constexpr int32_t buf = decltype(buf_tag)::value;
    KeyTile kt_next;
    MaskRule mr_next;
    const bool more = n + 1 < n_tiles;
    if (more) {
      desc(n + 1, kt_next, mr_next);
      TT::template fetch<GATHER>(pf, sm, buf ^ 1, kb, vb, kt_next, fp, tid);
    }
    process_tile<T, BIAS, SEG, LBL>(sm, buf, w, lane, mr, br, gi, lr, kt, !GATHER, qi, qpos, dead, scale_log2,
                          only_sb);
    if (more) {
      TT::stage(sm, buf ^ 1, pf, tid);
      stage_meta<T, SEG, LBL>(sm, buf ^ 1, pf.meta, gi, lr, kt_next.gmode, tid);
      kt = kt_next;
      mr = mr_next;
    }
    __syncthreads();
  };
  for (int32_t n = 0; n < n_tiles; n += 2) {
    step(BufTag<0>{}, n);
    if (n + 1 < n_tiles) step(BufTag<1>{}, n + 1);
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
