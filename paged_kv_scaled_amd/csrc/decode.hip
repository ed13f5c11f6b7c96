// Single-token decode: host side (plan and launches).  The kernels, and what they
// compute, are in decode_device.h.
#include <mutex>

#include "decode_device.h"

namespace pkv {

namespace {

// The decode workspace of the allocation-free entry point: a device array of the
// library, one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel: it takes the device address that hipGetSymbolAddress gives
// for the current device (decode_scratch) and passes that.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

constexpr int kMaxScratchDevices = 64;

// ---- dispatch --------------------------------------------------------------------------

int heads_per_wave(int g) {
  if (g <= 1) return 1;
  if (g == 2) return 2;
  if (g <= 4) return 4;
  return 8;
}

// Stream and split mode run on the matrix-core core (decode_mfma.h) where the vector
// core's arithmetic per key is the larger cost, for bf16 / fp16 queries at head_dim 64 or
// 128 with pages of at least 8 tokens.
//  * Stream mode (one wave per SIMD; with a bf16 / fp16 cache the core keeps a rolling
//    double buffer): from 4 heads per wave.  Measured per launch at 1024 stream waves:
//    decode batch (4 heads) 99.3 -> 96.4 us, 32 sequences of 1000..3000 keys at 4 heads
//    52.2 -> 50.0 us and at 8 heads 55.9 -> 51.4 us; at 1 and 2 heads the vector core
//    stays ahead (46.2 vs 48.5 us, 48.0 vs 49.8 us).
//  * Split mode (many short items, bound by occupancy: the matrix-core kernel allows 2
//    waves per SIMD, the vector kernel 4): from 8 heads per wave, or 4 with an FP8 cache
//    (whose codes the vector core widens per head group) or at head_dim 64.  Measured
//    when batches beyond 1024 sequences still took split mode: 1100 sequences at 4
//    heads 149 us (vector) against 175 us (bf16), but 119 -> 95 us over FP8.
// Item mode, fp32 and the other shapes always take the vector core.
template <typename T, int D>
constexpr bool mfma_decode_type() {
  return T::bytes == 2 && (D == 64 || D == 128);
}

template <typename T, int D, int HPW>
constexpr bool mfma_stream_shape() {
  return mfma_decode_type<T, D>() && HPW >= 4;
}

template <typename T, int D, int HPW>
constexpr bool mfma_split_shape() {
  return mfma_decode_type<T, D>() && HPW >= ((KvFp8<T>::value || D == 64) ? 4 : 8);
}

template <typename T, int D, int HPW>
bool launch_main_mfma(const DecodeParams& dp, const DecodePlan& pl, hipStream_t stream) {
  if (dp.block_shift < 3) return false;
  // the core's offsets inside a page are 32-bit: pages of 4 GiB and more take the vector core
  if ((uint64_t)dp.block_stride * (KvFp8<T>::value ? 1u : 2u) >= ((uint64_t)1 << 32)) return false;
  constexpr int MS = MSteps<T>::value;
  if (pl.stream) {
    if constexpr (mfma_stream_shape<T, D, HPW>()) {
      const int blocks = (int)((dp.total_items + kWavesPerBlock - 1) / kWavesPerBlock);
      PKV_LOG_LAUNCH("decode_stream_kernel", blocks, kDecodeThreads,
                     "core=mfma D=%d heads_per_wave=%d steps=%d ranges=%d items=%lld cus=%d", D,
                     HPW, MS, dp.nranges, (long long)dp.total_items, device_shape().cus);
      if (pl.prefix)
        hipLaunchKernelGGL((decode_stream_kernel<T, D, HPW, MS, true, true>), dim3(blocks),
                           dim3(kDecodeThreads), 0, stream, dp);
      else
        hipLaunchKernelGGL((decode_stream_kernel<T, D, HPW, MS, true>), dim3(blocks),
                           dim3(kDecodeThreads), 0, stream, dp);
      return true;
    }
    return false;
  }
  if constexpr (mfma_split_shape<T, D, HPW>()) {
    using C = DecodeShape<T, D>;
    if constexpr (C::LPT == 8 && C::TPR == 8) {
      if (pl.num_splits == 1 && pl.max_seq_len <= kItemPages << dp.block_shift) return false;
    }
    const int64_t wanted = (dp.total_items + kWavesPerBlock - 1) / kWavesPerBlock;
    const int blocks = (int)(wanted < 8192 ? wanted : 8192);
    PKV_LOG_LAUNCH("decode_split_kernel", blocks, kDecodeThreads,
                   "core=mfma D=%d heads_per_wave=%d split_len=%d splits=%d items=%lld", D, HPW,
                   dp.split_len, dp.nsplit, (long long)dp.total_items);
    hipLaunchKernelGGL((decode_split_kernel<T, D, HPW, MS, true>), dim3(blocks),
                       dim3(kDecodeThreads), 0, stream, dp);
    return true;
  }
  return false;
}

template <typename T, int D, int HPW>
void launch_main(const DecodeParams& dp, const DecodePlan& pl, hipStream_t stream) {
  using C = DecodeShape<T, D>;
  constexpr int NS = DecodeSteps<T, D, HPW>::value;
  if (launch_main_mfma<T, D, HPW>(dp, pl, stream)) return;
  if (pl.stream) {
    const int blocks = (int)((dp.total_items + kWavesPerBlock - 1) / kWavesPerBlock);
    PKV_LOG_LAUNCH("decode_stream_kernel", blocks, kDecodeThreads,
                   "core=vector D=%d heads_per_wave=%d steps=%d ranges=%d items=%lld cus=%d", D,
                   HPW, NS, dp.nranges, (long long)dp.total_items, device_shape().cus);
    if (pl.prefix)
      hipLaunchKernelGGL((decode_stream_kernel<T, D, HPW, NS, false, true>), dim3(blocks),
                         dim3(kDecodeThreads), 0, stream, dp);
    else
      hipLaunchKernelGGL((decode_stream_kernel<T, D, HPW, NS>), dim3(blocks), dim3(kDecodeThreads),
                         0, stream, dp);
    return;
  }
  if constexpr (C::LPT == 8 && C::TPR == 8) {
    if (pl.num_splits == 1 && pl.max_seq_len <= kItemPages << dp.block_shift) {
      const int64_t waves = (dp.total_items + C::TPR - 1) / C::TPR;
      const int blocks = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
      PKV_LOG_LAUNCH("decode_items_kernel", blocks, kDecodeThreads,
                     "core=vector D=%d heads_per_wave=%d items=%lld (8 per wave)", D, HPW,
                     (long long)dp.total_items);
      hipLaunchKernelGGL((decode_items_kernel<T, D, HPW, kItemSteps>), dim3(blocks),
                         dim3(kDecodeThreads), 0, stream, dp);
      return;
    }
  }
  const int64_t wanted = (dp.total_items + kWavesPerBlock - 1) / kWavesPerBlock;
  const int blocks = (int)(wanted < 8192 ? wanted : 8192);
  PKV_LOG_LAUNCH("decode_split_kernel", blocks, kDecodeThreads,
                 "core=vector D=%d heads_per_wave=%d split_len=%d splits=%d items=%lld", D, HPW,
                 dp.split_len, dp.nsplit, (long long)dp.total_items);
  if (pl.max_seq_len <= C::STEP)
    hipLaunchKernelGGL((decode_split_kernel<T, D, HPW, 1>), dim3(blocks), dim3(kDecodeThreads),
                       0, stream, dp);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, HPW, NS>), dim3(blocks), dim3(kDecodeThreads),
                       0, stream, dp);
}

template <typename T, int D>
void launch_hpw(const DecodeParams& dp, const DecodePlan& pl, hipStream_t stream) {
  switch (pl.heads_per_wave) {
    case 1: launch_main<T, D, 1>(dp, pl, stream); break;
    case 2: launch_main<T, D, 2>(dp, pl, stream); break;
    case 4: launch_main<T, D, 4>(dp, pl, stream); break;
    default: launch_main<T, D, 8>(dp, pl, stream); break;
  }
}

template <typename T, int D>
void launch_merge(const DecodeParams& dp, const DecodePlan& pl, hipStream_t stream) {
  if (pl.wide_merge) {
    const int rows = dp.S * dp.H;
    PKV_LOG_LAUNCH("decode_merge_stream_wide_kernel", rows, kDecodeThreads, "rows=%d", rows);
    hipLaunchKernelGGL((decode_merge_stream_wide_kernel<T, D>), dim3(rows), dim3(kDecodeThreads),
                       0, stream, dp);
    return;
  }
  const int blocks = (int)(((int64_t)dp.S * dp.H + kWavesPerBlock - 1) / kWavesPerBlock);
  PKV_LOG_LAUNCH(pl.stream ? "decode_merge_stream_kernel" : "decode_merge_split_kernel", blocks,
                 kDecodeThreads, "rows=%lld", (long long)dp.S * dp.H);
  if (pl.stream) {
    if (pl.prefix)
      hipLaunchKernelGGL((decode_merge_stream_kernel<T, D, true>), dim3(blocks),
                         dim3(kDecodeThreads), 0, stream, dp);
    else
      hipLaunchKernelGGL((decode_merge_stream_kernel<T, D>), dim3(blocks), dim3(kDecodeThreads), 0,
                         stream, dp);
  } else
    hipLaunchKernelGGL((decode_merge_split_kernel<T, D>), dim3(blocks), dim3(kDecodeThreads), 0,
                       stream, dp);
}

template <typename T>
void launch_all(const DecodeParams& dp, const DecodePlan& pl, int d, bool merge,
                hipStream_t stream) {
  switch (d) {
    case 16: merge ? launch_merge<T, 16>(dp, pl, stream) : launch_hpw<T, 16>(dp, pl, stream); break;
    case 64: merge ? launch_merge<T, 64>(dp, pl, stream) : launch_hpw<T, 64>(dp, pl, stream); break;
    default: merge ? launch_merge<T, 128>(dp, pl, stream) : launch_hpw<T, 128>(dp, pl, stream); break;
  }
}

}  // namespace

DecodePlan decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_seq_len) {
  DecodePlan pl{};
  const int g = num_kv_heads > 0 ? num_heads / num_kv_heads : 1;
  pl.heads_per_wave = heads_per_wave(g);
  pl.groups_per_kv = (g + pl.heads_per_wave - 1) / pl.heads_per_wave;
  const int64_t groups = (int64_t)num_kv_heads * pl.groups_per_kv;
  // Split mode: splits of >= 256 keys within 64 blocks, lengthened until the item count
  // is at most 16384 (about 16 waves per CU on 256 CUs).
  const int max_split = kWave * block_size;
  int split = 256 < max_split ? 256 : max_split;
  while (split < max_seq_len && split * 2 <= max_split &&
         (int64_t)num_seqs * groups * (((int64_t)max_seq_len + split - 1) / split) > 16384)
    split *= 2;
  pl.split_len = split;
  pl.max_seq_len = max_seq_len;
  pl.num_splits = max_seq_len > 0 ? (max_seq_len + split - 1) / split : 1;
  if (pl.num_splits < 1) pl.num_splits = 1;
  // Stream mode whenever some sequence needs more than one split.  Up to kStreamScanSeqs
  // sequences every wave scans the lengths itself; beyond, a planning kernel writes
  // prefix sums and range starts for the waves to read.  Measured (interleaved A/B, 32 q
  // / 8 kv heads, D 128): 1024 sequences of <= 1024 keys 5.26 -> 5.92 TB/s and 512 of
  // <= 2048 keys 5.97 -> 6.16 TB/s with the tables; 256 sequences equal either way.
  pl.stream = pl.num_splits > 1;
  pl.prefix = pl.stream && num_seqs > kStreamScanSeqs;
  const int waves = device_shape().cus * kStreamWavesPerCu;
  pl.num_ranges = pl.stream ? (int)(waves / groups > 1 ? waves / groups : 1) : 0;
  // A workgroup per (sequence, head) merges where a sequence averages 16 ranges or more.
  pl.wide_merge = pl.stream && (int64_t)num_seqs * 16 <= pl.num_ranges;
  const size_t slots = pl.stream ? (size_t)num_heads * pl.num_ranges * 2
                                 : (pl.num_splits > 1 ? (size_t)num_seqs * num_heads * pl.num_splits : 0);
  pl.workspace_bytes = slots * (size_t)head_dim * sizeof(float) + slots * 2 * sizeof(float);
  if (pl.prefix)   // cu[S + 1] and rpos[ranges] (int64), rstart[ranges] (int32)
    pl.workspace_bytes += ((size_t)num_seqs + 1 + pl.num_ranges) * sizeof(int64_t) +
                          (size_t)pl.num_ranges * sizeof(int32_t);
  return pl;
}

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* table[kMaxScratchDevices] = {};
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (table[dev] == nullptr) {
    // once per device, with that device current: its own copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    table[dev] = p;
  }
  *ptr = table[dev];
  return hipSuccess;
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& pl, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const DecodeParams dp = decode_params(a, pl);
  auto dispatch = [&](bool merge) {
    if (a.kv_fp8) {
      if (a.dtype == kBF16) launch_all<BF16K8>(dp, pl, a.head_dim, merge, stream);
      else launch_all<F16K8>(dp, pl, a.head_dim, merge, stream);
      return;
    }
    switch (a.dtype) {
      case kBF16: launch_all<BF16>(dp, pl, a.head_dim, merge, stream); break;
      case kF16: launch_all<F16>(dp, pl, a.head_dim, merge, stream); break;
      default: launch_all<F32>(dp, pl, a.head_dim, merge, stream); break;
    }
  };
  if (pl.prefix) {
    PKV_LOG_LAUNCH("decode_stream_plan_kernel", 1, kPlanThreads, "seqs=%d ranges=%d",
                   a.num_seqs, pl.num_ranges);
    hipLaunchKernelGGL(decode_stream_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, dp);
  }
  dispatch(false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(pl.stream || pl.num_splits > 1)) return e;
  dispatch(true);
  return hipGetLastError();
}

}  // namespace pkv
