// entry.h — internal entry points shared by the C ABI's source files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "longattn.h"

namespace la {

// Where la_attn_forward's workspace comes from: the caller's buffer in
// ext->workspace (fixed_bytes == 0), or a fixed device buffer of fixed_bytes
// bytes that get() returns (null on failure, with the reason already set as
// the thread's error message).
struct WorkspaceSource {
  size_t fixed_bytes = 0;
  void* (*get)() = nullptr;
};

la_status attn_forward_ws(const la_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* global_idx, int32_t n_global, int32_t radius,
                          const int32_t* dilation, int32_t causal, const float* rel_bias,
                          void* out, float* lse, hipStream_t stream, const la_attn_ext* ext,
                          WorkspaceSource src);

// Sets the thread's error message; returns s.
la_status set_error(la_status s, const char* msg);

// dims checks shared by every call (D == 64, dtype, size limits; bf16 only
// when need_bf16), setting the thread's error message on failure.
la_status check_dims(const la_dims* d, bool need_bf16);

constexpr int32_t kDHead = 64;  // the one head size built
constexpr size_t kAlign = 256;  // workspace alignment and part padding
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool is_empty(const la_dims* d) { return d->B == 0 || d->H == 0 || d->N == 0; }

}  // namespace la
