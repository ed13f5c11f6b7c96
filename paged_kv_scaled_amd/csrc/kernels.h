// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Every argument here has already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2, kFp8E4M3 = 3 };

// The span-list mask (beyond the three pkv_mask_mode values), as the kernels number it.
constexpr int kMaskSpansHost = 3;

inline int dtype_bytes(int dt) { return dt == kF32 ? 4 : (dt == kFp8E4M3 ? 1 : 2); }

struct ScatterArgs {
  const void* key;
  const void* value;
  int64_t token_stride;        // elements
  const int64_t* slots;
  int32_t num_tokens;
  void* key_cache;
  void* value_cache;
  int64_t block_stride;        // elements
  int32_t num_blocks, block_size, num_kv_heads, head_dim;
  int dtype;
  const uint32_t* guard = nullptr;   // device error word when device checks are on
};

struct GatherArgs {
  void* key_out;
  void* value_out;
  const int32_t* cu_seq_lens;
  const void* key_cache;
  const void* value_cache;
  int64_t block_stride;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq, num_seqs, total_tokens, num_blocks, block_size, num_kv_heads,
      head_dim, max_seq_len;
  int dtype;
  const uint32_t* guard = nullptr;
};

struct AttnArgs {
  void* out;
  const void* query;
  const int32_t* cu_seqlens_q;   // prefill only
  const int32_t* seq_lens;
  const void* key_cache;
  const void* value_cache;
  int64_t block_stride;          // elements
  const int32_t* block_tables;
  int32_t max_blocks_per_seq, num_seqs, num_tokens, num_heads, num_kv_heads, head_dim,
      num_blocks, block_size;
  float scale;
  int mask;                      // kMaskNone / kMaskCausal / kMaskBlockCausal / kMaskSpans
  int32_t span_len, max_q_len, max_seq_len;
  const int32_t* full_spans;     // SPANS: (start, end) pairs, sequence by sequence
  const int32_t* cu_spans;       // SPANS: [S+1] offsets into full_spans
  int dtype;
  void* workspace;               // decode only
  const uint32_t* guard;         // device error word when device checks are on, else null
  int kv_fp8;                    // the caches hold E4M3 codes (value = code * scale)
  float k_scale, v_scale;
};

// What the sequence check kernel reads: lengths from seq_lens (attention) or from
// cu_seq_lens (gather); cu_seqlens_q only for prefill.
struct CheckSeqArgs {
  const int32_t* full_spans;     // prefill with span lists only
  const int32_t* cu_spans;
  int32_t num_spans;
  const int32_t* seq_lens;
  const int32_t* cu_seq_lens;
  const int32_t* cu_seqlens_q;
  const int32_t* block_tables;
  int32_t num_seqs, max_blocks_per_seq, num_blocks, block_size, max_seq_len, max_q_len;
  int64_t num_tokens, total_tokens;
};

// Device-side precondition checks: the device address of this device's error word
// (null if the runtime cannot give it), the two check kernels, and a synchronising
// read-and-clear of the word.
const uint32_t* check_guard();
hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t num_slots, hipStream_t stream);
hipError_t launch_check_seqs(const CheckSeqArgs& a, hipStream_t stream);
hipError_t take_check_word(hipStream_t stream, uint32_t* bits);
// Duplicate-slot check of one slot_mapping over a caller bitmap of ceil(num_slots / 32)
// words that is all zero on entry and left all zero (two launches).
hipError_t launch_check_duplicate_slots(const int64_t* slots, int32_t n, int64_t num_slots,
                                        uint32_t* marks, hipStream_t stream);

// Decode split plan: a pure function of the sizes, shared by the workspace query
// and the launch so that both agree.
struct DecodePlan {
  int heads_per_wave;   // query heads of one kv group handled by one wave (power of 2)
  int groups_per_kv;    // waves needed to cover the g = H / Hkv heads of one kv head
  int split_len;        // keys per split (split mode)
  int num_splits;       // splits of the longest sequence (split mode)
  bool stream;          // equal ranges of the concatenated key axis instead of splits
  bool prefix;          // stream mode over more sequences than a wave can scan: a planning
                        // kernel first writes the length prefix sums and every range's
                        // first sequence into the workspace
  int num_ranges;       // ranges per head group (stream mode)
  bool wide_merge;      // stream mode over few long sequences: one workgroup merges each
                        // (sequence, head)
  int max_seq_len;
  size_t workspace_bytes;
};
DecodePlan decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_seq_len);

// The current device's shape, read once per device from its properties: compute units,
// and XCDs (chiplets of 32 CUs on gfx950, so 8 on a whole MI355X, fewer on a partition).
// Without a device (host-only use, the workspace size queries) the whole chip is assumed.
struct DeviceShape {
  int cus;
  int xcds;
};
DeviceShape device_shape();

hipError_t launch_kv_scatter(const ScatterArgs& a, hipStream_t stream);
// Launch log: with PKV_LOG=1 in the environment (read once), every kernel launch prints
// one line to stderr -- the kernel, its grid and block, and the variant chosen.
bool log_enabled();
void log_launch(const char* kernel, long long grid, int block, const char* fmt, ...);
#define PKV_LOG_LAUNCH(...) \
  do { if (::pkv::log_enabled()) ::pkv::log_launch(__VA_ARGS__); } while (0)

// Small-seq training path (one query row per sequence, at most 16 keys).
struct SmallArgs {
  void* out;                     // forward output [S, H, D]
  void* weights;                 // [S, H, max_seq_len] attention weights, query type
  const void* query;             // [S, H, D]
  const void* d_out;             // backward: [S, H, D]
  void* d_query;                 // backward: [S, H, D]
  void* d_key;                   // backward: [total_kv, Hkv, D], THD by cu_seq_lens
  void* d_value;
  const void* key_cache;
  const void* value_cache;
  int64_t block_stride;          // elements
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* cu_seq_lens;    // backward
  int32_t max_blocks_per_seq, num_seqs, num_heads, num_kv_heads, head_dim, block_size;
  int32_t max_seq_len;           // <= 16: the weights' row length
  float scale;
  int dtype;
  const uint32_t* guard;
};
hipError_t launch_smallseq(const SmallArgs& a, bool backward, hipStream_t stream);

// Quantising scatter into an FP8 (E4M3) cache: a.dtype is the source type, the cache
// element is one byte; code = E4M3(clamp(x * inv_scale, +-448)).
hipError_t launch_kv_scatter_fp8(const ScatterArgs& a, float k_inv_scale, float v_inv_scale,
                                 hipStream_t stream);
hipError_t launch_kv_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, const DecodePlan& plan, hipStream_t stream);
// Size of the library's own decode workspace (the allocation-free decode entry point), and
// its device address on the current device, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);
// Returns hipErrorNotSupported when no MFMA variant covers the shape.
hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t stream);
hipError_t launch_prefill_valu(const AttnArgs& a, hipStream_t stream);
// bf16 / fp16 queries, head_dim 64 or 128, scale > 0, cache blocks below 4 GiB
bool prefill_mfma_supported(const AttnArgs& a);

}  // namespace pkv
