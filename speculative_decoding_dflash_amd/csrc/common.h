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

// IEEE binary16 stored as raw 16-bit words: the attention operands (q, the KV cache) of bf16 models.
struct f16 {
  uint16_t bits;
};

// Element access for the storage types.
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
// Round to nearest even; magnitudes beyond the largest finite half (65504) saturate to it.
DF_DEVICE uint16_t f32_to_f16(float f) {
  const _Float16 h = (_Float16)fminf(fmaxf(f, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, h);
}
DF_DEVICE float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
template <> struct Elem<f16> {
  static DF_DEVICE float load(const f16 *p) { return f16_to_f32(p->bits); }
  static DF_DEVICE void store(f16 *p, float v) { p->bits = f32_to_f16(v); }
  static constexpr int kPerVec = 8;
};

// Storage type of the attention operands (q, K, V) for a model whose weights are T: fp16 for bf16
// models (11 significant bits where bf16 keeps 8; q and k are RMS-normalised and the softmax weights
// lie in [0, 1]), fp32 for fp32 models.
template <typename T> struct KvOf;
template <> struct KvOf<bf16> { using type = f16; };
template <> struct KvOf<float> { using type = float; };
// and back: the projection-input type that goes with a KV storage type
template <typename K> struct XOf;
template <> struct XOf<f16> { using type = bf16; };
template <> struct XOf<float> { using type = float; };

// Projection inputs (the X operand of every weight product) of bf16 models are held as two bf16
// planes, hi = bf16(v) and lo = bf16(v - hi) (v - hi is exact in fp32), so that hi + lo carries v to
// about 16 significant bits and the product W (hi + lo) = W hi + W lo loses nothing to the storage of
// X.  Calls over many rows instead hold one fp16 plane (lo null: the 16-bit words at hi are fp16), for
// the tiled fp16 kernel.  fp32 models keep one plane (lo is null).
DF_DEVICE void store_x(bf16 *hi, bf16 *lo, size_t i, float v) {
  if (!lo) {
    hi[i].bits = f32_to_f16(v);
    return;
  }
  const uint16_t h = f32_to_bf16(v);
  hi[i].bits = h;
  if (lo) lo[i].bits = f32_to_bf16(v - bf16_to_f32(h));
}
DF_DEVICE void store_x(float *hi, float *, size_t i, float v) { hi[i] = v; }

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
