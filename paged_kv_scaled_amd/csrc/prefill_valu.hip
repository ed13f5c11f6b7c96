// Prefill / chunked-prefill attention on the vector ALU, fp32 throughout.
//
// Covers what the MFMA kernel does not: fp32 inputs (any head_dim) and head_dim 16 (also
// over an FP8 cache, whose codes are widened exactly to fp32).
// Semantics are those of the MFMA kernel (Spyre paged-attention PR, "Description"
// steps 2-6 on a flat query batch; bottom-right causal and block-causal masks of the
// vllm-omni piecewise block-causal PR).  Probabilities stay fp32 here.
//
// One wave per (query row, head).  Keys are visited in chunks of 64, one key per lane:
// the lane forms its score from K read through the block table (the fused gather), the
// wave keeps a running max / sum, parks the chunk's probabilities in LDS and then
// accumulates P.V with lanes over the head dimension (coalesced V reads).
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kValuThreads = 256;
constexpr int kValuWaves = kValuThreads / kWave;

template <typename T>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (T::bytes == 4) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    const uint32_t b = reinterpret_cast<const uint16_t*>(base)[idx];
    return lo_of(T{}, b);
  }
}

// One K or V element: an E4M3 code widened exactly for an FP8 cache, else as load_elem.
template <typename T>
__device__ __forceinline__ float load_kv(const void* base, int64_t idx) {
  if constexpr (KvFp8<T>::value) {
    return __builtin_amdgcn_cvt_f32_fp8((int)reinterpret_cast<const uint8_t*>(base)[idx], 0);
  } else {
    return load_elem<T>(base, idx);
  }
}

template <typename T>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (T::bytes == 4) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)(pack2(T{}, x, 0.f) & 0xFFFFu);
  }
}

// Index of the sequence owning flat query row t (cu is non-decreasing, cu[0] = 0).
__device__ __forceinline__ int owner_seq(const int32_t* __restrict__ cu, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One past the last key visible to the query at absolute position a.

template <typename T, int DMAX>
__global__ void __launch_bounds__(kValuThreads)
prefill_valu_kernel(const AttnArgs p, float scale_log2, float out_scale) {
  if (guard_tripped(p.guard)) return;
  __shared__ float s_q[kValuWaves][DMAX];
  __shared__ float s_p[kValuWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int64_t item = (int64_t)blockIdx.x * kValuWaves + wv;
  if (item >= (int64_t)p.num_tokens * p.num_heads) return;
  const int t = (int)(item / p.num_heads);
  const int h = (int)(item % p.num_heads);
  const int D = p.head_dim;
  const int s = owner_seq(p.cu_seqlens_q, p.num_seqs, t);
  const int L = p.seq_lens[s];
  const int q0 = p.cu_seqlens_q[s];
  const int qn = p.cu_seqlens_q[s + 1] - q0;
  const int a = L - qn + (t - q0);
  const int n0 = p.cu_spans ? p.cu_spans[s] : 0, n1 = p.cu_spans ? p.cu_spans[s + 1] : 0;
  const int vend = visible_end(p.mask, a, L, p.span_len, p.full_spans, n0, n1);
  const int kvh = h / (p.num_heads / p.num_kv_heads);
  const int bmask = p.block_size - 1;
  int shift = 0;
  while ((1 << shift) < p.block_size) ++shift;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  const int32_t* table = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

  for (int d = lane; d < D; d += kWave)
    s_q[wv][d] = load_elem<T>(p.query, ((int64_t)t * p.num_heads + h) * D + d);
  __builtin_amdgcn_wave_barrier();

  float m = -INFINITY, l = 0.f;
  constexpr int DPL = (DMAX + kWave - 1) / kWave;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;

  for (int k0 = 0; k0 < vend; k0 += kWave) {
    const int pos = k0 + lane;
    float z = -INFINITY;
    if (pos < vend) {
      const int64_t blk = table[pos >> shift];
      const int64_t row = blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + (int64_t)kvh * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(s_q[wv][d], load_kv<T>(p.key_cache, row + d), dot);
      z = dot * scale_log2;
    }
    float cmax = z;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) cmax = fmaxf(cmax, shfl_xor_f(cmax, off));
    const float mn = fmaxf(m, cmax);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float pr = (pos < vend) ? exp2f(z - mn) : 0.f;
    float psum = pr;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) psum += shfl_xor_f(psum, off);
    l = l * alpha + psum;
    m = mn;
    s_p[wv][lane] = pr;
    __builtin_amdgcn_wave_barrier();
    const int n = min(kWave, vend - k0);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    for (int j = 0; j < n; ++j) {
      const int pj = k0 + j;
      const int64_t blk = table[pj >> shift];
      const int64_t row = blk * p.block_stride + (int64_t)(pj & bmask) * row_elems + (int64_t)kvh * D;
      const float w = s_p[wv][j];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + i * kWave;
        if (d < D) acc[i] = __builtin_fmaf(w, load_kv<T>(p.value_cache, row + d), acc[i]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = l > 0.f ? out_scale / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = lane + i * kWave;
    if (d < D) store_elem<T>(p.out, ((int64_t)t * p.num_heads + h) * D + d, acc[i] * inv);
  }
}

template <typename T>
void launch_valu_t(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.num_tokens * a.num_heads;
  const int blocks = (int)((items + kValuWaves - 1) / kValuWaves);
  const float sl2 = a.scale * (a.kv_fp8 ? a.k_scale : 1.f) * kLog2e;
  PKV_LOG_LAUNCH("prefill_valu_kernel", blocks, kValuThreads, "D=%d rows=%d heads=%d mask=%d fp8=%d",
                 a.head_dim, a.num_tokens, a.num_heads, a.mask, a.kv_fp8);
  const float osc = a.kv_fp8 ? a.v_scale : 1.f;
  if (a.head_dim <= 64)
    hipLaunchKernelGGL((prefill_valu_kernel<T, 64>), dim3(blocks), dim3(kValuThreads), 0, stream, a, sl2, osc);
  else
    hipLaunchKernelGGL((prefill_valu_kernel<T, 128>), dim3(blocks), dim3(kValuThreads), 0, stream, a, sl2, osc);
}

}  // namespace

hipError_t launch_prefill_valu(const AttnArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  if (a.kv_fp8) {
    if (a.dtype == kBF16) launch_valu_t<BF16K8>(a, stream);
    else launch_valu_t<F16K8>(a, stream);
    return hipGetLastError();
  }
  switch (a.dtype) {
    case kBF16: launch_valu_t<BF16>(a, stream); break;
    case kF16: launch_valu_t<F16>(a, stream); break;
    default: launch_valu_t<F32>(a, stream); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
