// Achievable-ceiling kernels for the benchmark (not part of the attention ABI; built
// into libpkv_ceilings.so, which only bench.py loads).
//
//  * stream_read_kernel: every workgroup reads one contiguous range of a buffer in 16-byte
//    vectors and folds them into one word -- the HBM read rate a plain streaming kernel
//    reaches on this chip, the ceiling the decode kernels are held to;
//  * mfma_loop_kernel: every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on four
//    independent accumulators (the prefill kernel's matrix instruction) with nothing
//    else in the loop -- the matrix-core rate reachable at the clock the chip holds
//    under that load.  Wave 0 of workgroup 0 also records the shader clock counter
//    (s_memtime) and the constant 100 MHz counter (s_memrealtime) around its loop, so
//    the clock during the loop is their ratio times 100 MHz.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each workgroup reads one contiguous range of the buffer, UNROLL 16-byte loads in flight
// per lane (nontemporal: the data is used once).
template <int UNROLL>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf, size_t n,
                                                          uint32_t* __restrict__ sink) {
  const size_t per_block = (n + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * per_block;
  const size_t end = begin + per_block < n ? begin + per_block : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = begin + threadIdx.x;
  constexpr size_t kStep = 256;
  for (; i + (UNROLL - 1) * kStep < end; i += UNROLL * kStep) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kStep);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < end; i += kStep) acc ^= buf[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, x);
}

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* __restrict__ sink,
                                                        unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  // operands that never change: the loop measures the matrix pipe alone
  const u32x4 ua = {0x3F803F80u ^ (uint32_t)lane, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4 ub = {0x3C003C00u, 0x3C003C00u ^ (uint32_t)lane, 0x3C003C00u, 0x3C003C00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua);
  const bf16x8 b = __builtin_bit_cast(bf16x8, ub);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (timer) {
    // the accumulators feed the sum, so the loop has finished when the counters are read
    clocks[0] = __builtin_amdgcn_s_memtime() - t0 + (s == 12345.f ? 1ull : 0ull);
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  if (lane == 0) sink[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = s;
}

}  // namespace

extern "C" {

// Reads n16 16-byte vectors of buf with `blocks` workgroups of 256 threads, 4 or 8 loads in
// flight per lane (`unroll`); sink holds `blocks` words (XOR-accumulated).  Returns a
// hipError_t.
int pkv_ceiling_stream_read(const void* buf, size_t n16, uint32_t* sink, int blocks, int unroll,
                            void* stream) {
  if (!buf || !sink || blocks <= 0) return (int)hipErrorInvalidValue;
  const u32x4* b = static_cast<const u32x4*>(buf);
  if (unroll >= 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, b, n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, b, n16, sink);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave 4 * iters MFMAs of 32x32x16 (32768 flops each);
// sink holds blocks * 4 floats, clocks two counters (shader clock ticks, 100 MHz ticks).
int pkv_ceiling_mfma(int blocks, int iters, float* sink, unsigned long long* clocks, void* stream) {
  if (!sink || !clocks || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters,
                     sink, clocks);
  return (int)hipGetLastError();
}

}  // extern "C"
