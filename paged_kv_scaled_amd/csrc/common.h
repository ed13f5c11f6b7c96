// Shared device helpers of libpkv (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Storage tags: the kernels see raw 16-bit or 32-bit words.
struct BF16 { using storage = uint16_t; static constexpr int bytes = 2; };
struct F16  { using storage = uint16_t; static constexpr int bytes = 2; };
struct F32  { using storage = uint32_t; static constexpr int bytes = 4; };

// An FP8 (E4M3) KV cache read with a bf16 / fp16 query: the query, output and arithmetic
// are those of the base tag; keys and values are widened from their codes on load.
struct BF16K8 : BF16 {};
struct F16K8 : F16 {};
template <typename T> struct KvFp8 { static constexpr bool value = false; };
template <> struct KvFp8<BF16K8> { static constexpr bool value = true; };
template <> struct KvFp8<F16K8> { static constexpr bool value = true; };
// The compute tag of a tag (BF16 for BF16K8, F16 for F16K8, else itself).
template <typename T> struct BaseOf { using type = T; };
template <> struct BaseOf<BF16K8> { using type = BF16; };
template <> struct BaseOf<F16K8> { using type = F16; };

// ---- scalar conversions ---------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Two fp32 -> packed pair of the storage type, round to nearest even.
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  f16x2_t v = __builtin_convertvector((f32x2_t){a, b}, f16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Widen the two halves of a packed word.
__device__ __forceinline__ float lo_of(BF16, uint32_t w) { return bf16_lo(w); }
__device__ __forceinline__ float hi_of(BF16, uint32_t w) { return bf16_hi(w); }
__device__ __forceinline__ float lo_of(F16, uint32_t w) { return f16_lo(w); }
__device__ __forceinline__ float hi_of(F16, uint32_t w) { return f16_hi(w); }

// acc + a.x*b.x + a.y*b.y on packed 16-bit pairs (fp32 accumulate): v_dot2_f32_{bf16,f16}.
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                acc, false);
}

// Two E4M3 codes (bytes 0-1, or 2-3 with HI) of a word -> the packed pair of the compute
// type (exact: every E4M3 value is a bf16 and an fp16 value).
template <bool HI>
__device__ __forceinline__ uint32_t widen_fp8x2(BF16, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t widen_fp8x2(F16, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
}

// ---- cross-lane helpers ---------------------------------------------------------------

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  return __shfl_xor(x, m, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Masks of the prefill kernels (the first three are pkv_mask_mode; SPANS is the span-list
// entry point).
constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskBlockCausal = 2, kMaskSpans = 3;

// End of the visible key prefix of the query at absolute position a of a sequence of L
// keys.  Every mask here sees a prefix [0, end): NONE all keys; CAUSAL p <= a; BLOCK_CAUSAL
// up to the end of a's span of `span` tokens; SPANS up to the end of the full span
// holding a, if any (spans[2i], spans[2i+1]) for i in [n0, n1), sorted), else p <= a.
// The end never decreases with a.
__device__ __forceinline__ int visible_end(int mask, int a, int L, int span,
                                           const int32_t* spans = nullptr, int n0 = 0, int n1 = 0) {
  if (mask == kMaskCausal) return min(L, a + 1);
  if (mask == kMaskBlockCausal) return min(L, (a / span + 1) * span);
  if (mask == kMaskSpans) {
    int e = a + 1;
    for (int i = n0; i < n1; ++i) {
      const int s0 = spans[2 * i];
      if (s0 > a) break;
      const int s1 = spans[2 * i + 1];
      if (a < s1) {
        e = s1;
        break;
      }
    }
    return min(L, e);
  }
  return L;
}

// log2 of a power of two (block sizes, tiling factors).
inline int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// True when a device-side precondition check on this device has failed (the guard is
// the error word, null when checks are off): every kernel then returns before it
// reads or writes anything else.
__device__ __forceinline__ bool guard_tripped(const uint32_t* guard) {
  return guard != nullptr && *guard != 0u;
}

}  // namespace pkv
