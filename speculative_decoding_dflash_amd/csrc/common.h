// Internal definitions shared by the kernels and the host side of libdflash (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DF_HOST_DEVICE __host__ __device__ __forceinline__
#define DF_DEVICE __device__ __forceinline__

namespace df {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 stored as raw 16-bit words; conversions are explicit.
struct bf16 {
  uint16_t bits;
};

DF_HOST_DEVICE float bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  return __builtin_bit_cast(float, u);
}

// Round to nearest, ties to even (inputs are finite in this library).
DF_HOST_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<bf16> {
  static DF_DEVICE float load(const bf16 *p) { return bf16_to_f32(p->bits); }
  static DF_DEVICE void store(bf16 *p, float v) { p->bits = f32_to_bf16(v); }
  static constexpr int kPerVec = 8;  // elements per 16-byte vector
};
template <> struct Elem<float> {
  static DF_DEVICE float load(const float *p) { return *p; }
  static DF_DEVICE void store(float *p, float v) { *p = v; }
  static constexpr int kPerVec = 4;
};

// Device state of one sequence slot (lives in the workspace).
struct SlotState {
  int32_t seq_len;    // committed positions 0 .. seq_len-1 (both caches)
  int32_t anchor;     // last emitted token, at position seq_len
  int32_t pend_start; // start position of the last verified block
  int32_t pend_qlen;  // its length
  int32_t inj_base;   // first position whose target features still need injecting
  int32_t inj_rows;   // how many (rows 0 .. inj_rows-1 of the last verified block)
  int32_t pad[2];
};

// Sticky device-side error flags (workspace).
enum ErrFlag { ERR_TOKEN = 0, ERR_PAGE = 1, ERR_STATE = 2, ERR_COUNT = 4 };

DF_DEVICE void raise_err(int32_t *err, int which) {
  __hip_atomic_store(err + which, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-row information of a call (workspace arrays, indexed by row).
struct Rows {
  int32_t *pos;   // absolute position
  int32_t *slot;  // sequence slot
  int32_t *valid; // 0: row is padding (its KV is not written)
  int32_t *tok;   // token id (embedding input)
};

// Paged KV addressing inside one layer's pool: page = [2 (K, V)][kv_heads][page_tokens * head_dim].
// K of a head is stored token-major ([tok][dim]), V dim-major ([dim][tok]), so that both attention
// products read their MFMA operands with contiguous loads.
struct KVLayout {
  int32_t page_tokens, kv_heads, head_dim;
  DF_HOST_DEVICE size_t page_elems() const { return (size_t)2 * kv_heads * page_tokens * head_dim; }
  DF_HOST_DEVICE size_t block(int page, int kv, int head) const {
    return (((size_t)page * 2 + kv) * kv_heads + head) * (size_t)page_tokens * head_dim;
  }
  DF_HOST_DEVICE size_t k_index(int page, int head, int tok, int dim) const {
    return block(page, 0, head) + (size_t)tok * head_dim + dim;
  }
  DF_HOST_DEVICE size_t v_index(int page, int head, int tok, int dim) const {
    return block(page, 1, head) + (size_t)dim * page_tokens + tok;
  }
};

constexpr int kWave = 64;

}  // namespace df
