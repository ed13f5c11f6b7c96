// Prefill / chunked-prefill attention on MFMA: host side.  The kernel, and what it
// computes, are in prefill_device.h.
#include "prefill_device.h"

namespace pkv {

bool prefill_mfma_supported(const AttnArgs& a) {
  // the row max is taken on raw scores, which needs a positive scale; a block offset is a
  // 32 x 32 -> 64-bit product, which needs a block of less than 4 GiB
  const uint64_t block_bytes = (uint64_t)a.block_stride * (a.kv_fp8 ? 1u : 2u);
  return (a.dtype == kBF16 || a.dtype == kF16) && (a.head_dim == 64 || a.head_dim == 128) &&
         a.scale > 0.f && block_bytes < ((uint64_t)1 << 32);
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t stream) {
  if (!prefill_mfma_supported(a)) return hipErrorNotSupported;
  if (a.num_tokens == 0 || a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  PrefillParams p{};
  int64_t nb = 0;
  if (!prefill_params(a, p, nb)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nb), block(kWaves * 64);
  PKV_LOG_LAUNCH("prefill_mfma_kernel", nb, kWaves * 64,
                 "D=%d heads_per_wg=%d rows_per_wg=%d groups=%d qtiles=%d mask=%d fp8=%d xcds=%d "
                 "ranked=%d",
                 a.head_dim, p.hw, 32 << p.rb_log2, p.ngroups, p.qtiles, p.mask, a.kv_fp8, p.nxcd,
                 p.rank_items);
#define PKV_PREFILL(TT)                                                                        \
  if (a.head_dim == 128) hipLaunchKernelGGL((prefill_mfma_kernel<TT, 128>), grid, block, 0, stream, p); \
  else hipLaunchKernelGGL((prefill_mfma_kernel<TT, 64>), grid, block, 0, stream, p)
  if (a.kv_fp8) {
    if (a.dtype == kBF16) { PKV_PREFILL(BF16K8); } else { PKV_PREFILL(F16K8); }
  } else {
    if (a.dtype == kBF16) { PKV_PREFILL(BF16); } else { PKV_PREFILL(F16); }
  }
#undef PKV_PREFILL
  return hipGetLastError();
}

}  // namespace pkv
