// Mixed batch: context rows (prefill / chunked prefill) and generation rows (single-token
// decode) of one step in one launch.
//
// What is computed: exactly what pkv_paged_attention_prefill computes for the context
// sequences and pkv_paged_attention_decode for the generation sequences.  The batch is
// ordered context first, generation after, and the two phases never share a tile (CSA2
// Vanilla golden PR, "Description": query tiles must not cross the context/generation
// boundary).  The Spyre paged-attention PR ("Description") runs prefill and decode
// sequences of a step through one attention call; here they also share one grid.
//
// How: one grid, two kinds of blocks.  Its first blocks are the prefill workgroups (the
// MFMA kernel's tiles, in its XCD-aware order, longest first); the blocks after them run
// eight decode waves each, one item per wave: up to 1024 generation sequences the
// stream-mode ranges (2048 equal slices of the concatenated key axis over all head groups,
// as in the decode kernel), beyond that split-mode (sequence, split, head group) items.
// The hardware starts the decode blocks on the CUs that the prefill workgroups free, so
// the decode work fills the prefill tail, which two launches on one stream cannot do.
// (acc, m, l) partials of sequences cut by ranges or splits are combined by the matching
// merge kernel afterwards.  Measured against a work queue (waves taking items from an
// atomic counter): the queue's atomics cost more than the balance they bring.
#include "decode_device.h"
#include "prefill_device.h"

namespace pkv {

namespace {

struct MixedParams {
  PrefillParams pf;
  DecodeParams dc;
  int32_t prefill_blocks;   // blocks [0, prefill_blocks) are prefill workgroups
};

constexpr int kMixedMaxDecodeBlocks = 4096;   // 8 waves each; more items: grid stride

template <typename T, int D, int HPW, int NSTEP>
__global__ void __launch_bounds__(kWaves * 64)
mixed_kernel(const MixedParams mp) {
  if (guard_tripped(mp.pf.guard)) return;
  const int bid = blockIdx.x;
  if (bid < mp.prefill_blocks) {
    prefill_tile<T, D>(mp.pf, bid);
    return;
  }
  const int64_t nw = (int64_t)(gridDim.x - mp.prefill_blocks) * kWaves;
  for (int64_t it = (int64_t)(bid - mp.prefill_blocks) * kWaves + threadIdx.x / kWave;
       it < mp.dc.total_items; it += nw) {
    if (mp.dc.nranges > 0)
      stream_item<T, D, HPW, NSTEP>(mp.dc, it);
    else
      split_item<T, D, HPW, NSTEP>(mp.dc, it);
  }
}

template <typename T, int D, int HPW>
void launch_mixed_t(const MixedParams& mp, unsigned blocks, hipStream_t stream) {
  constexpr int NS = DecodeSteps<T, D, HPW>::value;
  hipLaunchKernelGGL((mixed_kernel<T, D, HPW, NS>), dim3(blocks), dim3(kWaves * 64), 0, stream, mp);
}

// At most 4 heads per decode wave: 8 would not fit the prefill kernel's 256 registers.
template <typename T, int D>
void launch_mixed_d(const MixedParams& mp, int hpw, unsigned blocks, hipStream_t stream) {
  switch (hpw) {
    case 1: launch_mixed_t<T, D, 1>(mp, blocks, stream); break;
    case 2: launch_mixed_t<T, D, 2>(mp, blocks, stream); break;
    default: launch_mixed_t<T, D, 4>(mp, blocks, stream); break;
  }
}

template <typename T, int D>
void launch_mixed_merge_d(const DecodeParams& dp, bool stream_mode, hipStream_t stream) {
  const int blocks = (int)(((int64_t)dp.S * dp.H + kWavesPerBlock - 1) / kWavesPerBlock);
  if (stream_mode)
    hipLaunchKernelGGL((decode_merge_stream_kernel<T, D>), dim3(blocks), dim3(kDecodeThreads), 0,
                       stream, dp);
  else
    hipLaunchKernelGGL((decode_merge_split_kernel<T, D>), dim3(blocks), dim3(kDecodeThreads), 0,
                       stream, dp);
}

template <typename T>
void launch_mixed_merge(const DecodeParams& dp, int d, bool stream_mode, hipStream_t stream) {
  if (d == 128) launch_mixed_merge_d<T, 128>(dp, stream_mode, stream);
  else launch_mixed_merge_d<T, 64>(dp, stream_mode, stream);
}

}  // namespace

bool mixed_fused_supported(int dtype, int head_dim, float scale, bool kv_fp8) {
  return !kv_fp8 && prefill_mfma_supported(dtype, head_dim, scale);
}

hipError_t launch_mixed(const AttnArgs& ctx, const AttnArgs& gen, const DecodePlan& pl,
                        hipStream_t stream) {
  if (!mixed_fused_supported(ctx.dtype, ctx.head_dim, ctx.scale, ctx.kv_fp8 != 0) ||
      pl.heads_per_wave > 4)
    return hipErrorNotSupported;
  MixedParams mp{};
  int64_t pblocks = 0;
  if (ctx.num_seqs > 0 && ctx.num_tokens > 0 && ctx.max_q_len > 0) {
    if (!prefill_params(ctx, mp.pf, pblocks)) return hipErrorInvalidValue;
  }
  mp.pf.guard = ctx.guard;
  mp.prefill_blocks = (int32_t)pblocks;
  int64_t dblocks = 0;
  if (gen.num_seqs > 0) {
    mp.dc = decode_params(gen, pl);
    dblocks = (mp.dc.total_items + kWaves - 1) / kWaves;
    if (dblocks > kMixedMaxDecodeBlocks) dblocks = kMixedMaxDecodeBlocks;
  }
  const int64_t blocks = pblocks + dblocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int hpw = pl.heads_per_wave;
  PKV_LOG_LAUNCH("mixed_kernel", blocks, kWaves * 64,
                 "prefill_blocks=%lld decode_blocks=%lld decode=%s items=%lld heads_per_wave=%d",
                 (long long)pblocks, (long long)dblocks, pl.stream ? "stream" : "split",
                 (long long)mp.dc.total_items, hpw);
  if (ctx.dtype == kBF16) {
    if (ctx.head_dim == 128) launch_mixed_d<BF16, 128>(mp, hpw, (unsigned)blocks, stream);
    else launch_mixed_d<BF16, 64>(mp, hpw, (unsigned)blocks, stream);
  } else {
    if (ctx.head_dim == 128) launch_mixed_d<F16, 128>(mp, hpw, (unsigned)blocks, stream);
    else launch_mixed_d<F16, 64>(mp, hpw, (unsigned)blocks, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || gen.num_seqs == 0 || !(pl.stream || pl.num_splits > 1)) return e;
  if (ctx.dtype == kBF16) launch_mixed_merge<BF16>(mp.dc, gen.head_dim, pl.stream, stream);
  else launch_mixed_merge<F16>(mp.dc, gen.head_dim, pl.stream, stream);
  return hipGetLastError();
}

}  // namespace pkv
