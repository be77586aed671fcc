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

// Storage type of the activations that feed the matrix cores -- q, the KV cache, and the X operand of
// every weight product (normed hidden rows, attention output, SwiGLU activation, target features) --
// for a model whose weights are T: fp16 for bf16 models, fp32 for fp32 models.  fp16 keeps 11
// significant bits where bf16 keeps 8: rounding every one of these operands to bf16 would put a 64-layer
// forward's logits about 5e-2 from exact arithmetic (independent roundings adding up like the square
// root of the depth), rounding them to fp16 keeps it near 5e-3.  The bf16 weights enter the fp16
// products converted exactly (see bf16x2_to_f16x2).  q and k are RMS-normalised, the softmax weights lie
// in [0, 1]; every other stored magnitude saturates at 65504.
template <typename T> struct KvOf;
template <> struct KvOf<bf16> { using type = f16; };
template <> struct KvOf<float> { using type = float; };
template <typename T> using ActOf = typename KvOf<T>::type;

// Store v as element i of a projection input (X operand) of storage type A (fp16 or fp32).
template <typename A> DF_DEVICE void store_x(A *x, size_t i, float v) { Elem<A>::store(x + i, v); }

// Two bf16 weights (element 0 in the low half) -> two fp16, exact wherever fp16 is normal (|w| in
// [2^-14, 65504]: bf16's 8 significant bits fit in fp16's 11); smaller magnitudes land on fp16's
// subnormal grid, truncated (error below 2^-24).
DF_DEVICE uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float e0 = __builtin_bit_cast(float, w << 16), e1 = __builtin_bit_cast(float, w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
}

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
