// slot_mapping scatter of new K/V rows into the paged cache, and the test-only gather.
//
// Scatter: Spyre paged-attention PR (vllm-spyre #853), "Description", step 1 -- new
// key/value tokens are written into the paged KV cache by a vectorised scatter through
// slot_mapping.  Gather: the same page's step 2 -- rows are collected from scattered
// blocks into compact per-sequence tensors (the attention kernels fuse this step into
// their loads; the exported gather exists so tests can check the addressing bit-exactly).
//
// The FP8 variant of the scatter quantises each element to an E4M3 code on the way (FP8
// staging of cache rows: CSA2 Vanilla golden PR, "Description"; the pages fix no scale
// convention, the one used here is stated in pkv.h).
//
// Both plain kernels are raw copies, so they are written on bytes: one lane moves one VEC-byte
// vector of a token row (num_kv_heads * head_dim elements, dense in source and in
// cache), consecutive lanes take consecutive vectors of the same row, so every wave
// reads and writes whole contiguous row segments (coalesced, HBM-bound).
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

template <int VEC>
struct VecT;
template <> struct VecT<16> { using type = u32x4_t; };
template <> struct VecT<8> { using type = u32x2_t; };
template <> struct VecT<4> { using type = uint32_t; };
template <> struct VecT<2> { using type = uint16_t; };

constexpr int kScatterThreads = 256;

// grid.x covers (token, vector) pairs in a grid-stride loop; K and V move together.
template <int VEC>
__global__ void __launch_bounds__(kScatterThreads)
kv_scatter_kernel(const char* __restrict__ key, const char* __restrict__ value,
                  int64_t token_stride_b, const int64_t* __restrict__ slots, int32_t num_tokens,
                  char* __restrict__ kc, char* __restrict__ vc, int64_t block_stride_b,
                  int32_t block_shift, int32_t row_vecs, int64_t num_slots, const uint32_t* guard) {
  using V = typename VecT<VEC>::type;
  if (guard_tripped(guard)) return;
  const int64_t total = (int64_t)num_tokens * row_vecs;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int32_t bmask = (1 << block_shift) - 1;
  const int64_t row_b = (int64_t)row_vecs * VEC;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int32_t t = (int32_t)(i / row_vecs);
    const int32_t v = (int32_t)(i - (int64_t)t * row_vecs);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;   // padding token (negative slot)
    const int64_t blk = slot >> block_shift;
    const int64_t off = slot & bmask;
    const int64_t src = (int64_t)t * token_stride_b + (int64_t)v * VEC;
    const int64_t dst = blk * block_stride_b + off * row_b + (int64_t)v * VEC;
    const V kv = *reinterpret_cast<const V*>(key + src);
    const V vv = *reinterpret_cast<const V*>(value + src);
    *reinterpret_cast<V*>(kc + dst) = kv;
    *reinterpret_cast<V*>(vc + dst) = vv;
  }
}

// grid = (ceil(max_seq_len*row_vecs / threads), num_seqs)
template <int VEC>
__global__ void __launch_bounds__(kScatterThreads)
kv_gather_kernel(char* __restrict__ kout, char* __restrict__ vout,
                 const int32_t* __restrict__ cu_seq_lens, const char* __restrict__ kc,
                 const char* __restrict__ vc, int64_t block_stride_b,
                 const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
                 int32_t block_shift, int32_t row_vecs, const uint32_t* guard) {
  using V = typename VecT<VEC>::type;
  if (guard_tripped(guard)) return;
  const int s = blockIdx.y;
  const int32_t r0 = cu_seq_lens[s];
  const int32_t L = cu_seq_lens[s + 1] - r0;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)L * row_vecs) return;
  const int32_t p = (int32_t)(i / row_vecs);
  const int32_t v = (int32_t)(i - (int64_t)p * row_vecs);
  const int64_t row_b = (int64_t)row_vecs * VEC;
  const int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + (p >> block_shift)];
  const int64_t off = p & ((1 << block_shift) - 1);
  const int64_t src = blk * block_stride_b + off * row_b + (int64_t)v * VEC;
  const int64_t dst = ((int64_t)r0 + p) * row_b + (int64_t)v * VEC;
  *reinterpret_cast<V*>(kout + dst) = *reinterpret_cast<const V*>(kc + src);
  *reinterpret_cast<V*>(vout + dst) = *reinterpret_cast<const V*>(vc + src);
}

// ---- quantising scatter into an FP8 (E4M3) cache ---------------------------------------
// One lane turns N source elements of a row into N code bytes.  code = E4M3 of
// clamp(x * inv_scale, +-448), the product rounded once to fp32 and the conversion rounding
// to nearest even (v_cvt_pk_fp8_f32); a NaN stays NaN (the comparisons below pass it through).

__device__ __forceinline__ float src_value(BF16, uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ float src_value(F16, uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ __forceinline__ float src_value(F32, uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ float clamp_e4m3(float y) {
  return y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
}

// Two values -> two codes in the low (HI false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b, float inv, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a * inv), clamp_e4m3(b * inv),
                                                   (int)old, HI);
}

template <typename S, int N>
struct alignas(N * sizeof(typename S::storage)) SrcChunk {
  typename S::storage e[N];
};

template <int N> struct CodeChunk;
template <> struct CodeChunk<8> { using type = u32x2_t; };
template <> struct CodeChunk<4> { using type = uint32_t; };

template <typename S, int N>
__device__ __forceinline__ typename CodeChunk<N>::type quantize_chunk(const SrcChunk<S, N>& x,
                                                                     float inv) {
  uint32_t w[N / 4];
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const float f0 = src_value(S{}, x.e[4 * j]), f1 = src_value(S{}, x.e[4 * j + 1]);
    const float f2 = src_value(S{}, x.e[4 * j + 2]), f3 = src_value(S{}, x.e[4 * j + 3]);
    w[j] = to_e4m3x2<true>(f2, f3, inv, to_e4m3x2<false>(f0, f1, inv, 0u));
  }
  if constexpr (N == 8) return (u32x2_t){w[0], w[1]};
  else return w[0];
}

// Rows hold num_kv_heads * head_dim elements, a multiple of 16, so N in {4, 8} divides them.
template <typename S, int N>
__global__ void __launch_bounds__(kScatterThreads)
kv_scatter_fp8_kernel(const typename S::storage* __restrict__ key,
                      const typename S::storage* __restrict__ value, int64_t token_stride,
                      const int64_t* __restrict__ slots, int32_t num_tokens,
                      uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int64_t block_stride,
                      int32_t block_shift, int32_t row_chunks, int64_t num_slots, float k_inv,
                      float v_inv, const uint32_t* guard) {
  using C = typename CodeChunk<N>::type;
  if (guard_tripped(guard)) return;
  const int64_t total = (int64_t)num_tokens * row_chunks;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int32_t bmask = (1 << block_shift) - 1;
  const int64_t row = (int64_t)row_chunks * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int32_t t = (int32_t)(i / row_chunks);
    const int32_t v = (int32_t)(i - (int64_t)t * row_chunks);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;   // padding token (negative slot)
    const int64_t src = (int64_t)t * token_stride + (int64_t)v * N;
    const int64_t dst = (slot >> block_shift) * block_stride + (slot & bmask) * row + (int64_t)v * N;
    const SrcChunk<S, N> kx = *reinterpret_cast<const SrcChunk<S, N>*>(key + src);
    const SrcChunk<S, N> vx = *reinterpret_cast<const SrcChunk<S, N>*>(value + src);
    *reinterpret_cast<C*>(kc + dst) = quantize_chunk<S, N>(kx, k_inv);
    *reinterpret_cast<C*>(vc + dst) = quantize_chunk<S, N>(vx, v_inv);
  }
}

// Widest vector that divides every byte offset the kernel forms.
int pick_vec(int64_t row_b, int64_t a, int64_t b, const void* p0, const void* p1, const void* p2,
             const void* p3) {
  const uint64_t bits = (uint64_t)row_b | (uint64_t)a | (uint64_t)b | (uint64_t)(uintptr_t)p0 |
                        (uint64_t)(uintptr_t)p1 | (uint64_t)(uintptr_t)p2 |
                        (uint64_t)(uintptr_t)p3;
  for (int v : {16, 8, 4})
    if ((bits & (uint64_t)(v - 1)) == 0) return v;
  return 2;
}

}  // namespace

hipError_t launch_kv_scatter(const ScatterArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int eb = dtype_bytes(a.dtype);
  const int64_t row_b = (int64_t)a.num_kv_heads * a.head_dim * eb;
  const int64_t ts_b = a.token_stride * eb, bs_b = a.block_stride * eb;
  const int vec = pick_vec(row_b, ts_b, bs_b, a.key, a.value, a.key_cache, a.value_cache);
  const int32_t row_vecs = (int32_t)(row_b / vec);
  const int64_t total = (int64_t)a.num_tokens * row_vecs;
  const int64_t blocks64 = (total + kScatterThreads - 1) / kScatterThreads;
  const int blocks = (int)(blocks64 < 65536 ? blocks64 : 65536);
  const int shift = log2_exact(a.block_size);
  const int64_t num_slots = (int64_t)a.num_blocks * a.block_size;
  PKV_LOG_LAUNCH("kv_scatter_kernel", blocks, kScatterThreads, "vector=%dB tokens=%d", vec,
                 a.num_tokens);
#define PKV_SCATTER(V)                                                                       \
  hipLaunchKernelGGL(kv_scatter_kernel<V>, dim3(blocks), dim3(kScatterThreads), 0, stream,  \
                     (const char*)a.key, (const char*)a.value, ts_b, a.slots, a.num_tokens,  \
                     (char*)a.key_cache, (char*)a.value_cache, bs_b, shift, row_vecs, num_slots,  \
                     a.guard)
  switch (vec) {
    case 16: PKV_SCATTER(16); break;
    case 8: PKV_SCATTER(8); break;
    case 4: PKV_SCATTER(4); break;
    default: PKV_SCATTER(2); break;
  }
#undef PKV_SCATTER
  return hipGetLastError();
}

hipError_t launch_kv_scatter_fp8(const ScatterArgs& a, float k_inv, float v_inv,
                                 hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int eb = dtype_bytes(a.dtype);
  const int64_t row = (int64_t)a.num_kv_heads * a.head_dim;
  // 8 elements per lane when every source chunk is 8-element aligned and every code chunk
  // 8-byte aligned, else 4
  const uint64_t bits8 = (uint64_t)(a.token_stride * eb) | (uint64_t)(uintptr_t)a.key |
                         (uint64_t)(uintptr_t)a.value;
  const uint64_t bits1 = (uint64_t)a.block_stride | (uint64_t)(uintptr_t)a.key_cache |
                         (uint64_t)(uintptr_t)a.value_cache;
  const int n = ((bits8 & (uint64_t)(8 * eb - 1)) == 0 && (bits1 & 7u) == 0) ? 8 : 4;
  if ((bits8 & (uint64_t)(4 * eb - 1)) != 0 || (bits1 & 3u) != 0) return hipErrorInvalidValue;
  const int32_t row_chunks = (int32_t)(row / n);
  const int64_t total = (int64_t)a.num_tokens * row_chunks;
  const int64_t blocks64 = (total + kScatterThreads - 1) / kScatterThreads;
  const int blocks = (int)(blocks64 < 65536 ? blocks64 : 65536);
  const int shift = log2_exact(a.block_size);
  const int64_t num_slots = (int64_t)a.num_blocks * a.block_size;
  PKV_LOG_LAUNCH("kv_scatter_fp8_kernel", blocks, kScatterThreads, "elements_per_lane=%d tokens=%d",
                 n, a.num_tokens);
#define PKV_SCATTER8(S, N)                                                                     \
  hipLaunchKernelGGL((kv_scatter_fp8_kernel<S, N>), dim3(blocks), dim3(kScatterThreads), 0,    \
                     stream, (const S::storage*)a.key, (const S::storage*)a.value,            \
                     a.token_stride, a.slots, a.num_tokens, (uint8_t*)a.key_cache,             \
                     (uint8_t*)a.value_cache, a.block_stride, shift, row_chunks, num_slots,    \
                     k_inv, v_inv, a.guard)
  switch (a.dtype) {
    case kBF16: if (n == 8) PKV_SCATTER8(BF16, 8); else PKV_SCATTER8(BF16, 4); break;
    case kF16: if (n == 8) PKV_SCATTER8(F16, 8); else PKV_SCATTER8(F16, 4); break;
    default: if (n == 8) PKV_SCATTER8(F32, 8); else PKV_SCATTER8(F32, 4); break;
  }
#undef PKV_SCATTER8
  return hipGetLastError();
}

hipError_t launch_kv_gather(const GatherArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.total_tokens == 0 || a.max_seq_len == 0) return hipSuccess;
  const int eb = dtype_bytes(a.dtype);
  const int64_t row_b = (int64_t)a.num_kv_heads * a.head_dim * eb;
  const int64_t bs_b = a.block_stride * eb;
  const int vec = pick_vec(row_b, bs_b, 0, a.key_out, a.value_out, a.key_cache, a.value_cache);
  const int32_t row_vecs = (int32_t)(row_b / vec);
  const int64_t per_seq = (int64_t)a.max_seq_len * row_vecs;
  const dim3 grid((unsigned)((per_seq + kScatterThreads - 1) / kScatterThreads), a.num_seqs);
  const int shift = log2_exact(a.block_size);
  PKV_LOG_LAUNCH("kv_gather_kernel", (long long)grid.x * grid.y, kScatterThreads, "vector=%dB seqs=%d",
                 vec, a.num_seqs);
#define PKV_GATHER(V)                                                                           \
  hipLaunchKernelGGL(kv_gather_kernel<V>, grid, dim3(kScatterThreads), 0, stream,              \
                     (char*)a.key_out, (char*)a.value_out, a.cu_seq_lens,                      \
                     (const char*)a.key_cache, (const char*)a.value_cache, bs_b,                \
                     a.block_tables, a.max_blocks_per_seq, shift, row_vecs, a.guard)
  switch (vec) {
    case 16: PKV_GATHER(16); break;
    case 8: PKV_GATHER(8); break;
    case 4: PKV_GATHER(4); break;
    default: PKV_GATHER(2); break;
  }
#undef PKV_GATHER
  return hipGetLastError();
}

}  // namespace pkv
