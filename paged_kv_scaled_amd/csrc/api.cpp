// C ABI of libpkv: host-side validation, then kernel launches on the caller's stream.
// Every check runs before anything is enqueued, and a rejected call touches no memory
// (CSA2 Vanilla golden PR, "Description": rejected before anything is written).
#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/pkv.h"
#include "kernels.h"

static_assert(pkv::kDecodeScratchBytes == PKV_DECODE_NOALLOC_MAX_WORKSPACE,
              "the scratch array and its documented size must agree");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

bool is_pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

int check_dtype(int dtype) {
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not one of PKV_F32, PKV_F16, PKV_BF16", dtype);
  return PKV_OK;
}

// FP8 cache scales: finite and positive (their reciprocal must be finite too).
int check_fp8_scales(float k_scale, float v_scale) {
  const float lim = 3.0e38f;
  if (!(k_scale > 0.f && k_scale < lim && 1.f / k_scale < lim) ||
      !(v_scale > 0.f && v_scale < lim && 1.f / v_scale < lim))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite "
                "with finite reciprocals (got %g, %g)", (double)k_scale, (double)v_scale);
  return PKV_OK;
}

bool aligned(const void* p, unsigned n) { return ((uintptr_t)p & (n - 1)) == 0; }

// The attention kernels read cache rows and query/output rows in 16-byte vectors (8-byte
// ones for 64-dim FP8 rows): every row start must be 16-byte aligned.
int check_attn_alignment(const void* out, const void* query, const void* kc, const void* vc,
                         int64_t cache_block_stride, int elem_bytes) {
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(kc, 16) || !aligned(vc, 16) ||
      (cache_block_stride * elem_bytes) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "out, query, key_cache and value_cache must be 16-byte "
                "aligned and cache_block_stride a multiple of 16 bytes");
  return PKV_OK;
}

// Geometry shared by every call that reads or writes the cache.
int check_cache(const void* kc, const void* vc, int64_t block_stride, int32_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim) {
  if (!kc || !vc) return fail(PKV_ERR_INVALID_ARG, "key_cache/value_cache must not be NULL");
  if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be > 0 (got %d)", num_blocks);
  if (!is_pow2_in(block_size, 1, 256))
    return fail(PKV_ERR_INVALID_ARG, "block_size must be a power of two in [1, 256] (got %d)",
                block_size);
  if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", num_kv_heads);
  if (!PKV_HEAD_DIM_SUPPORTED(head_dim))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d is not compiled (16, 64, 128)", head_dim);
  const int64_t min_stride = (int64_t)block_size * num_kv_heads * head_dim;
  if (block_stride < min_stride)
    return fail(PKV_ERR_INVALID_ARG,
                "cache_block_stride %lld is smaller than block_size*num_kv_heads*head_dim = %lld",
                (long long)block_stride, (long long)min_stride);
  return PKV_OK;
}

int check_heads(int32_t num_heads, int32_t num_kv_heads) {
  if (num_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_heads must be > 0 (got %d)", num_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  return PKV_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

std::atomic<int> g_device_checks{0};

// With device checks on: the device error word that every kernel of the call takes as
// its guard (null when checks are off).  The call's check kernel is enqueued by the
// caller of this function, before the kernels it guards.
int guard_word(const uint32_t** guard, const char* what) {
  *guard = nullptr;
  if (!g_device_checks.load(std::memory_order_relaxed)) return PKV_OK;
  *guard = pkv::check_guard();
  if (*guard == nullptr)
    return fail(PKV_ERR_LAUNCH, "%s: the device error word of the current device is unavailable", what);
  return PKV_OK;
}

// Validation and launch shared by the two prefill entry points (mask already checked).
int prefill_common(void* out, const void* query, const int32_t* cu_seqlens_q,
                   const int32_t* seq_lens, const void* key_cache, const void* value_cache,
                   int64_t cache_block_stride, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_tokens,
                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                   int32_t block_size, float scale, int mask, int32_t span_len,
                   const int32_t* full_spans, const int32_t* cu_spans, int32_t num_spans,
                   int32_t max_q_len, int32_t max_seq_len, pkv_dtype dtype, void* stream,
                   const char* what, bool kv_fp8 = false, float k_scale = 1.f,
                   float v_scale = 1.f) {
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || max_seq_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs, num_tokens, max_q_len, max_seq_len must be >= 0");
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if ((rc = check_heads(num_heads, num_kv_heads)) != PKV_OK) return rc;
  if (!(scale == scale)) return fail(PKV_ERR_INVALID_ARG, "scale is NaN");
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !query || !cu_seqlens_q || !seq_lens || !block_tables)
    return fail(PKV_ERR_INVALID_ARG,
                "out, query, cu_seqlens_q, seq_lens and block_tables must not be NULL");
  if (max_q_len > max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_q_len (%d) > max_seq_len (%d)", max_q_len, max_seq_len);
  if (num_tokens > 0 && max_q_len == 0)
    return fail(PKV_ERR_INVALID_ARG, "max_q_len must be > 0 when num_tokens > 0");
  if ((int64_t)max_q_len * num_seqs < num_tokens)
    return fail(PKV_ERR_INVALID_ARG, "num_tokens (%d) > num_seqs*max_q_len (%lld)", num_tokens,
                (long long)max_q_len * num_seqs);
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq*block_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  if ((rc = check_attn_alignment(out, query, key_cache, value_cache, cache_block_stride,
                                 kv_fp8 ? 1 : (dtype == PKV_F32 ? 4 : 2))) != PKV_OK)
    return rc;
  pkv::AttnArgs a{};
  a.kv_fp8 = kv_fp8 ? 1 : 0;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.query = query;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens = seq_lens;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_stride = cache_block_stride;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.scale = scale;
  a.mask = mask;
  a.span_len = mask == PKV_MASK_BLOCK_CAUSAL ? span_len : 1;
  a.full_spans = full_spans;
  a.cu_spans = cu_spans;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.dtype = (int)dtype;
  if ((rc = guard_word(&a.guard, what)) != PKV_OK) return rc;
  if (a.guard != nullptr) {
    pkv::CheckSeqArgs c{full_spans, cu_spans, num_spans, seq_lens, nullptr, cu_seqlens_q,
                        block_tables, num_seqs, max_blocks_per_seq, num_blocks, block_size,
                        max_seq_len, max_q_len, num_tokens, 0};
    if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream), what)) != PKV_OK) return rc;
  }
  if (pkv::prefill_mfma_supported(a))
    return launched(pkv::launch_prefill_mfma(a, (hipStream_t)stream), what);
  return launched(pkv::launch_prefill_valu(a, (hipStream_t)stream), what);
}

// Validation and launch shared by the two decode entry points (dtype already checked).
int decode_common(void* out, const void* query, const void* key_cache, const void* value_cache,
                  int64_t cache_block_stride, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                  int32_t block_size, float scale, bool kv_fp8, float k_scale, float v_scale,
                  int32_t max_seq_len, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                  void* stream, const char* what) {
  int rc;
  if (num_seqs < 0 || max_seq_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs and max_seq_len must be >= 0");
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if ((rc = check_heads(num_heads, num_kv_heads)) != PKV_OK) return rc;
  if (!(scale == scale)) return fail(PKV_ERR_INVALID_ARG, "scale is NaN");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !block_tables || !seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "out, query, block_tables and seq_lens must not be NULL");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq*block_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  if ((rc = check_attn_alignment(out, query, key_cache, value_cache, cache_block_stride,
                                 kv_fp8 ? 1 : (dtype == PKV_F32 ? 4 : 2))) != PKV_OK)
    return rc;
  const pkv::DecodePlan plan =
      pkv::decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(PKV_ERR_WORKSPACE, "decode workspace of %zu bytes required (got %zu at %p)",
                plan.workspace_bytes, workspace_bytes, workspace);
  // the partials are stored as 16-byte vectors and the planning tables as int64
  if (plan.workspace_bytes > 0 && !aligned(workspace, 16))
    return fail(PKV_ERR_INVALID_ARG, "the decode workspace must be 16-byte aligned (got %p)",
                workspace);
  pkv::AttnArgs a{};
  a.out = out;
  a.query = query;
  a.seq_lens = seq_lens;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_stride = cache_block_stride;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.scale = scale;
  a.mask = PKV_MASK_NONE;
  a.max_seq_len = max_seq_len;
  a.max_q_len = 1;
  a.dtype = (int)dtype;
  a.workspace = workspace;
  a.kv_fp8 = kv_fp8 ? 1 : 0;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if ((rc = guard_word(&a.guard, what)) != PKV_OK) return rc;
  if (a.guard != nullptr) {
    pkv::CheckSeqArgs c{nullptr, nullptr, 0, seq_lens, nullptr, nullptr, block_tables, num_seqs, max_blocks_per_seq,
                        num_blocks, block_size, max_seq_len, 1, 0, 0};
    if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream),
                       what)) != PKV_OK)
      return rc;
  }
  return launched(pkv::launch_decode(a, plan, (hipStream_t)stream), what);
}

// Validation shared by the small-seq forward and backward (dtype already checked).
int smallseq_common(pkv::SmallArgs& a, const void* query, const void* key_cache,
                    const void* value_cache, int64_t cache_block_stride,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t block_size, float scale, int32_t max_seq_len, pkv_dtype dtype,
                    const char* what) {
  int rc;
  if (dtype != PKV_BF16 && dtype != PKV_F16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: dtype %d is not PKV_BF16 or PKV_F16", what, (int)dtype);
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (max_seq_len < 1 || max_seq_len > 16)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_seq_len must be in [1, 16] (got %d)", what, max_seq_len);
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if ((rc = check_heads(num_heads, num_kv_heads)) != PKV_OK) return rc;
  if (!(scale == scale)) return fail(PKV_ERR_INVALID_ARG, "scale is NaN");
  if (num_seqs == 0) return PKV_OK;
  if (!query || !seq_lens || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "query, seq_lens and block_tables must not be NULL");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq*block_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  if (!aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
      (cache_block_stride * 2) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "query and the caches must be 16-byte aligned and "
                "cache_block_stride a multiple of 16 bytes");
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_stride = cache_block_stride;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_seq_len = max_seq_len;
  a.scale = scale;
  a.dtype = (int)dtype;
  return guard_word(&a.guard, what);
}

}  // namespace

namespace pkv {

DeviceShape device_shape() {
  constexpr int kMaxDev = 64;
  constexpr int kCusPerXcd = 32;
  static std::mutex mu;
  static DeviceShape table[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return DeviceShape{256, 8};
  std::lock_guard<std::mutex> lock(mu);
  DeviceShape& d = table[dev];
  if (d.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return DeviceShape{256, 8};
    d.cus = cus;
    d.xcds = cus >= kCusPerXcd ? cus / kCusPerXcd : 1;
  }
  return d;
}

// -1: not read yet; then 0 / 1 (PKV_LOG in the environment, or pkv_set_log)
static std::atomic<int> g_log{-1};

bool log_enabled() {
  int v = g_log.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("PKV_LOG");
    const int on = (e != nullptr && e[0] != '\0' && e[0] != '0') ? 1 : 0;
    int expected = -1;
    g_log.compare_exchange_strong(expected, on, std::memory_order_relaxed);
    v = g_log.load(std::memory_order_relaxed);
  }
  return v == 1;
}

void log_launch(const char* kernel, long long grid, int block, const char* fmt, ...) {
  char detail[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(detail, sizeof(detail), fmt, ap);
  va_end(ap);
  fprintf(stderr, "pkv: %s grid=%lld block=%d %s\n", kernel, grid, block, detail);
}

}  // namespace pkv

extern "C" {

int pkv_version(void) { return (1 << 16) | 0; }

const char* pkv_last_error(void) { return g_err; }

int pkv_set_log(int enable) {
  clear_error();
  pkv::g_log.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_set_device_checks(int enable) {
  clear_error();
  g_device_checks.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_check_device_error(void* stream, uint32_t* bits) {
  clear_error();
  uint32_t v = 0;
  const hipError_t e = pkv::take_check_word((hipStream_t)stream, &v);
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "pkv_check_device_error: %s", hipGetErrorString(e));
  if (bits) *bits = v;
  if (v == 0) return PKV_OK;
  char list[256] = "";
  const struct { uint32_t bit; const char* name; } names[] = {
      {PKV_CHECK_SLOT_RANGE, "slot_mapping entry >= num_blocks*block_size"},
      {PKV_CHECK_SEQ_LEN, "sequence length outside [0, min(max_seq_len, max_blocks_per_seq*block_size)]"},
      {PKV_CHECK_TABLE, "block_tables entry outside [0, num_blocks)"},
      {PKV_CHECK_CU_Q, "cu_seqlens_q inconsistent"},
      {PKV_CHECK_SPANS, "span lists inconsistent"},
      {PKV_CHECK_DUP_SLOT, "slot_mapping holds a slot twice"}};
  for (const auto& n : names) {
    if (!(v & n.bit)) continue;
    if (list[0]) strncat(list, "; ", sizeof(list) - strlen(list) - 1);
    strncat(list, n.name, sizeof(list) - strlen(list) - 1);
  }
  return fail(PKV_ERR_INVALID_ARG, "device checks failed (bits 0x%x): %s", v, list);
}

int pkv_check_slots_unique(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, void* marks, size_t marks_bytes, void* stream) {
  clear_error();
  const char* what = "pkv_check_slots_unique";
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "%s: num_tokens must be >= 0 (got %d)", what, num_tokens);
  if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "%s: num_blocks must be > 0 (got %d)", what, num_blocks);
  if (!is_pow2_in(block_size, 1, 256))
    return fail(PKV_ERR_INVALID_ARG, "%s: block_size must be a power of two in [1, 256] (got %d)",
                what, block_size);
  if (num_tokens == 0) return PKV_OK;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const size_t need = (size_t)((num_slots + 31) / 32) * sizeof(uint32_t);
  if (!slot_mapping || !marks)
    return fail(PKV_ERR_INVALID_ARG, "%s: slot_mapping and marks must not be NULL", what);
  if (marks_bytes < need || !aligned(marks, 4))
    return fail(PKV_ERR_INVALID_ARG, "%s: marks must be a 4-byte aligned bitmap of at least %zu "
                "bytes (got %zu at %p)", what, need, marks_bytes, marks);
  return launched(pkv::launch_check_duplicate_slots(slot_mapping, num_tokens, num_slots,
                                                    static_cast<uint32_t*>(marks),
                                                    (hipStream_t)stream),
                  what);
}

int pkv_kv_cache_write(const void* key, const void* value, int64_t kv_token_stride,
                       const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                       void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                       pkv_dtype dtype, void* stream) {
  clear_error();
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "key, value and slot_mapping must not be NULL");
  if (kv_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "kv_token_stride %lld < num_kv_heads*head_dim = %lld",
                (long long)kv_token_stride, (long long)num_kv_heads * head_dim);
  pkv::ScatterArgs a{key, value, kv_token_stride, slot_mapping, num_tokens, key_cache,
                     value_cache, cache_block_stride, num_blocks, block_size, num_kv_heads,
                     head_dim, (int)dtype};
  if ((rc = guard_word(&a.guard, "pkv_kv_cache_write")) != PKV_OK) return rc;
  if (a.guard != nullptr &&
      (rc = launched(pkv::launch_check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                             (hipStream_t)stream),
                     "pkv_kv_cache_write (device checks)")) != PKV_OK)
    return rc;
  return launched(pkv::launch_kv_scatter(a, (hipStream_t)stream), "pkv_kv_cache_write");
}

int pkv_kv_cache_write_fp8(const void* key, const void* value, int64_t kv_token_stride,
                           const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                           void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           float k_scale, float v_scale, pkv_dtype dtype, void* stream) {
  clear_error();
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  if ((rc = check_fp8_scales(k_scale, v_scale)) != PKV_OK) return rc;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "key, value and slot_mapping must not be NULL");
  if (kv_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "kv_token_stride %lld < num_kv_heads*head_dim = %lld",
                (long long)kv_token_stride, (long long)num_kv_heads * head_dim);
  const unsigned eb = dtype == PKV_F32 ? 4u : 2u;
  if (kv_token_stride % 4 != 0 || !aligned(key, 4 * eb) || !aligned(value, 4 * eb) ||
      cache_block_stride % 4 != 0 || !aligned(key_cache, 4) || !aligned(value_cache, 4))
    return fail(PKV_ERR_INVALID_ARG, "pkv_kv_cache_write_fp8: kv_token_stride and "
                "cache_block_stride must be multiples of 4 and key/value/cache pointers aligned "
                "to 4 elements");
  pkv::ScatterArgs a{key, value, kv_token_stride, slot_mapping, num_tokens, key_cache,
                     value_cache, cache_block_stride, num_blocks, block_size, num_kv_heads,
                     head_dim, (int)dtype};
  if ((rc = guard_word(&a.guard, "pkv_kv_cache_write_fp8")) != PKV_OK) return rc;
  if (a.guard != nullptr &&
      (rc = launched(pkv::launch_check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                             (hipStream_t)stream),
                     "pkv_kv_cache_write_fp8 (device checks)")) != PKV_OK)
    return rc;
  // the reciprocals are rounded once to fp32 here; the kernel multiplies by them
  return launched(pkv::launch_kv_scatter_fp8(a, 1.f / k_scale, 1.f / v_scale, (hipStream_t)stream),
                  "pkv_kv_cache_write_fp8");
}

int pkv_kv_cache_gather(void* key_out, void* value_out, const int32_t* cu_seq_lens,
                        const void* key_cache, const void* value_cache,
                        int64_t cache_block_stride, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_tokens,
                        int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_seq_len, pkv_dtype dtype, void* stream) {
  clear_error();
  int rc;
  if (dtype != PKV_FP8_E4M3 && (rc = check_dtype(dtype)) != PKV_OK) return rc;
  if (num_seqs < 0 || total_tokens < 0 || max_seq_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs, total_tokens and max_seq_len must be >= 0");
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if (num_seqs == 0 || total_tokens == 0) return PKV_OK;
  if (!key_out || !value_out || !cu_seq_lens || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "key_out, value_out, cu_seq_lens and block_tables must not be NULL");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq*block_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  pkv::GatherArgs a{key_out, value_out, cu_seq_lens, key_cache, value_cache, cache_block_stride,
                    block_tables, max_blocks_per_seq, num_seqs, total_tokens, num_blocks,
                    block_size, num_kv_heads, head_dim, max_seq_len, (int)dtype};
  if ((rc = guard_word(&a.guard, "pkv_kv_cache_gather")) != PKV_OK) return rc;
  if (a.guard != nullptr) {
    pkv::CheckSeqArgs c{nullptr, nullptr, 0, nullptr, cu_seq_lens, nullptr, block_tables, num_seqs, max_blocks_per_seq,
                        num_blocks, block_size, max_seq_len, 0, 0, total_tokens};
    if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream),
                       "pkv_kv_cache_gather (device checks)")) != PKV_OK)
      return rc;
  }
  return launched(pkv::launch_kv_gather(a, (hipStream_t)stream), "pkv_kv_cache_gather");
}

size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !PKV_HEAD_DIM_SUPPORTED(head_dim) || !is_pow2_in(block_size, 1, 256) || max_seq_len < 0)
    return 0;
  return pkv::decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len)
      .workspace_bytes;
}

int pkv_paged_attention_decode(void* out, const void* query, const void* key_cache,
                               const void* value_cache, int64_t cache_block_stride,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               int32_t block_size, float scale, int32_t max_seq_len,
                               void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                               void* stream) {
  clear_error();
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  return decode_common(out, query, key_cache, value_cache, cache_block_stride, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                       num_blocks, block_size, scale, false, 1.f, 1.f, max_seq_len, workspace,
                       workspace_bytes, dtype, stream, "pkv_paged_attention_decode");
}

int pkv_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, int64_t cache_block_stride,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t num_blocks, int32_t block_size, float scale,
                                       int32_t max_seq_len, pkv_dtype dtype, void* stream) {
  clear_error();
  const char* what = "pkv_paged_attention_decode_noalloc";
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  // the plan's workspace must fit the library's scratch array; checked before the lookup
  // so that an oversized call touches no device state
  if (num_seqs > 0 && num_heads > 0 && num_kv_heads > 0 && num_heads % num_kv_heads == 0 &&
      PKV_HEAD_DIM_SUPPORTED(head_dim) && is_pow2_in(block_size, 1, 256) && max_seq_len >= 0) {
    const size_t need = pkv::decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                         max_seq_len).workspace_bytes;
    if (need > pkv::kDecodeScratchBytes)
      return fail(PKV_ERR_WORKSPACE, "%s: these sizes need %zu bytes of decode workspace, more "
                  "than the %zu bytes of the library's scratch; use pkv_paged_attention_decode "
                  "with a caller workspace", what, need, (size_t)pkv::kDecodeScratchBytes);
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    const hipError_t e = pkv::decode_scratch(&ws);
    if (e != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "%s: the scratch array of the current device is unavailable: %s",
                  what, hipGetErrorString(e));
  }
  return decode_common(out, query, key_cache, value_cache, cache_block_stride, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                       num_blocks, block_size, scale, false, 1.f, 1.f, max_seq_len, ws,
                       ws ? pkv::kDecodeScratchBytes : 0, dtype, stream, what);
}

int pkv_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, int64_t cache_block_stride,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                   int32_t block_size, float scale, float k_scale, float v_scale,
                                   int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                                   pkv_dtype dtype, void* stream) {
  clear_error();
  int rc;
  if (dtype != PKV_BF16 && dtype != PKV_F16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_attention_decode_fp8: query dtype %d is not "
                "PKV_BF16 or PKV_F16", (int)dtype);
  if ((rc = check_fp8_scales(k_scale, v_scale)) != PKV_OK) return rc;
  return decode_common(out, query, key_cache, value_cache, cache_block_stride, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                       num_blocks, block_size, scale, true, k_scale, v_scale, max_seq_len,
                       workspace, workspace_bytes, dtype, stream, "pkv_paged_attention_decode_fp8");
}

int pkv_paged_attention_prefill(void* out, const void* query, const int32_t* cu_seqlens_q,
                                const int32_t* seq_lens, const void* key_cache,
                                const void* value_cache, int64_t cache_block_stride,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                int32_t block_size, float scale, pkv_mask_mode mask,
                                int32_t span_len, int32_t max_q_len, int32_t max_seq_len,
                                pkv_dtype dtype, void* stream) {
  clear_error();
  if (mask != PKV_MASK_NONE && mask != PKV_MASK_CAUSAL && mask != PKV_MASK_BLOCK_CAUSAL)
    return fail(PKV_ERR_INVALID_ARG, "unknown mask mode %d", (int)mask);
  if (mask == PKV_MASK_BLOCK_CAUSAL && span_len <= 0)
    return fail(PKV_ERR_INVALID_ARG, "BLOCK_CAUSAL needs span_len > 0 (got %d)", span_len);
  return prefill_common(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                        cache_block_stride, block_tables, max_blocks_per_seq, num_seqs, num_tokens,
                        num_heads, num_kv_heads, head_dim, num_blocks, block_size, scale, (int)mask,
                        span_len, nullptr, nullptr, 0, max_q_len, max_seq_len, dtype, stream,
                        "pkv_paged_attention_prefill");
}

int pkv_paged_attention_prefill_fp8(void* out, const void* query, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens, const void* key_cache,
                                    const void* value_cache, int64_t cache_block_stride,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                    int32_t block_size, float scale, float k_scale, float v_scale,
                                    pkv_mask_mode mask, int32_t span_len, int32_t max_q_len,
                                    int32_t max_seq_len, pkv_dtype dtype, void* stream) {
  clear_error();
  int rc;
  if (dtype != PKV_BF16 && dtype != PKV_F16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_attention_prefill_fp8: query dtype %d is not "
                "PKV_BF16 or PKV_F16", (int)dtype);
  if ((rc = check_fp8_scales(k_scale, v_scale)) != PKV_OK) return rc;
  if (mask != PKV_MASK_NONE && mask != PKV_MASK_CAUSAL && mask != PKV_MASK_BLOCK_CAUSAL)
    return fail(PKV_ERR_INVALID_ARG, "unknown mask mode %d", (int)mask);
  if (mask == PKV_MASK_BLOCK_CAUSAL && span_len <= 0)
    return fail(PKV_ERR_INVALID_ARG, "BLOCK_CAUSAL needs span_len > 0 (got %d)", span_len);
  return prefill_common(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                        cache_block_stride, block_tables, max_blocks_per_seq, num_seqs, num_tokens,
                        num_heads, num_kv_heads, head_dim, num_blocks, block_size, scale, (int)mask,
                        span_len, nullptr, nullptr, 0, max_q_len, max_seq_len, dtype, stream,
                        "pkv_paged_attention_prefill_fp8", true, k_scale, v_scale);
}

size_t pkv_mixed_workspace_size(int32_t num_gen_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_seq_len) {
  if (num_gen_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !PKV_HEAD_DIM_SUPPORTED(head_dim) || !is_pow2_in(block_size, 1, 256) || max_seq_len < 0)
    return 0;
  return pkv::decode_plan(num_gen_seqs, num_heads, num_kv_heads, head_dim, block_size,
                          max_seq_len)
      .workspace_bytes;
}

int pkv_paged_attention_mixed(void* out, const void* query, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens, const void* key_cache,
                              const void* value_cache, int64_t cache_block_stride,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              int32_t num_seqs, int32_t num_tokens, int32_t num_ctx_seqs,
                              int32_t num_ctx_tokens, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t block_size,
                              float scale, pkv_mask_mode mask, int32_t span_len,
                              int32_t max_q_len, int32_t max_seq_len, void* workspace,
                              size_t workspace_bytes, pkv_dtype dtype, void* stream) {
  clear_error();
  const char* what = "pkv_paged_attention_mixed";
  int rc;
  if ((rc = check_dtype(dtype)) != PKV_OK) return rc;
  if (mask != PKV_MASK_NONE && mask != PKV_MASK_CAUSAL && mask != PKV_MASK_BLOCK_CAUSAL)
    return fail(PKV_ERR_INVALID_ARG, "unknown mask mode %d", (int)mask);
  if (mask == PKV_MASK_BLOCK_CAUSAL && span_len <= 0)
    return fail(PKV_ERR_INVALID_ARG, "BLOCK_CAUSAL needs span_len > 0 (got %d)", span_len);
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || max_seq_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs, num_tokens, max_q_len, max_seq_len must be >= 0");
  if (num_ctx_seqs < 0 || num_ctx_seqs > num_seqs || num_ctx_tokens < 0 ||
      num_ctx_tokens > num_tokens)
    return fail(PKV_ERR_INVALID_ARG, "need 0 <= num_ctx_seqs <= num_seqs and 0 <= num_ctx_tokens "
                "<= num_tokens (got %d of %d, %d of %d)", num_ctx_seqs, num_seqs, num_ctx_tokens,
                num_tokens);
  const int32_t num_gen = num_seqs - num_ctx_seqs;
  if (num_tokens - num_ctx_tokens != num_gen)
    return fail(PKV_ERR_INVALID_ARG, "generation sequences take one query row each: "
                "num_tokens - num_ctx_tokens (%d) != num_seqs - num_ctx_seqs (%d)",
                num_tokens - num_ctx_tokens, num_gen);
  if (num_ctx_seqs == 0 && num_ctx_tokens != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_ctx_tokens must be 0 without context sequences");
  if ((rc = check_cache(key_cache, value_cache, cache_block_stride, num_blocks, block_size,
                        num_kv_heads, head_dim)) != PKV_OK)
    return rc;
  if ((rc = check_heads(num_heads, num_kv_heads)) != PKV_OK) return rc;
  if (!(scale == scale)) return fail(PKV_ERR_INVALID_ARG, "scale is NaN");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !seq_lens || !block_tables || (num_ctx_seqs > 0 && !cu_seqlens_q))
    return fail(PKV_ERR_INVALID_ARG,
                "out, query, seq_lens, block_tables (and cu_seqlens_q with context sequences) "
                "must not be NULL");
  if (num_ctx_tokens > 0 && max_q_len == 0)
    return fail(PKV_ERR_INVALID_ARG, "max_q_len must be > 0 when num_ctx_tokens > 0");
  if (max_q_len > max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_q_len (%d) > max_seq_len (%d)", max_q_len, max_seq_len);
  if ((int64_t)max_q_len * num_ctx_seqs < num_ctx_tokens)
    return fail(PKV_ERR_INVALID_ARG, "num_ctx_tokens (%d) > num_ctx_seqs*max_q_len (%lld)",
                num_ctx_tokens, (long long)max_q_len * num_ctx_seqs);
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size < max_seq_len)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq*block_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  if ((rc = check_attn_alignment(out, query, key_cache, value_cache, cache_block_stride,
                                 dtype == PKV_F32 ? 4 : 2)) != PKV_OK)
    return rc;
  const pkv::DecodePlan plan = pkv::decode_plan(num_gen > 0 ? num_gen : 1, num_heads,
                                                num_kv_heads, head_dim, block_size, max_seq_len);
  if (num_gen > 0 && plan.workspace_bytes > 0 &&
      (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(PKV_ERR_WORKSPACE, "mixed-batch workspace of %zu bytes required (got %zu at %p)",
                plan.workspace_bytes, workspace_bytes, workspace);
  if (num_gen > 0 && plan.workspace_bytes > 0 && !aligned(workspace, 16))
    return fail(PKV_ERR_INVALID_ARG, "the mixed-batch workspace must be 16-byte aligned (got %p)",
                workspace);
  const size_t eb = dtype == PKV_F32 ? 4 : 2;
  const size_t row_bytes = (size_t)num_heads * head_dim * eb;
  pkv::AttnArgs ctx{};
  ctx.out = out;
  ctx.query = query;
  ctx.cu_seqlens_q = cu_seqlens_q;
  ctx.seq_lens = seq_lens;
  ctx.key_cache = key_cache;
  ctx.value_cache = value_cache;
  ctx.block_stride = cache_block_stride;
  ctx.block_tables = block_tables;
  ctx.max_blocks_per_seq = max_blocks_per_seq;
  ctx.num_seqs = num_ctx_seqs;
  ctx.num_tokens = num_ctx_tokens;
  ctx.num_heads = num_heads;
  ctx.num_kv_heads = num_kv_heads;
  ctx.head_dim = head_dim;
  ctx.num_blocks = num_blocks;
  ctx.block_size = block_size;
  ctx.scale = scale;
  ctx.mask = mask;
  ctx.span_len = mask == PKV_MASK_BLOCK_CAUSAL ? span_len : 1;
  ctx.max_q_len = max_q_len;
  ctx.max_seq_len = max_seq_len;
  ctx.dtype = (int)dtype;
  pkv::AttnArgs gen = ctx;
  gen.out = static_cast<char*>(out) + (size_t)num_ctx_tokens * row_bytes;
  gen.query = static_cast<const char*>(query) + (size_t)num_ctx_tokens * row_bytes;
  gen.cu_seqlens_q = nullptr;
  gen.seq_lens = seq_lens + num_ctx_seqs;
  gen.block_tables = block_tables + (size_t)num_ctx_seqs * max_blocks_per_seq;
  gen.num_seqs = num_gen;
  gen.num_tokens = num_gen;
  gen.mask = PKV_MASK_NONE;
  gen.max_q_len = 1;
  gen.workspace = workspace;
  if ((rc = guard_word(&ctx.guard, what)) != PKV_OK) return rc;
  gen.guard = ctx.guard;
  if (ctx.guard != nullptr) {
    if (num_ctx_seqs > 0) {
      pkv::CheckSeqArgs c{nullptr, nullptr, 0, seq_lens, nullptr, cu_seqlens_q, block_tables,
                          num_ctx_seqs, max_blocks_per_seq, num_blocks, block_size, max_seq_len,
                          max_q_len, num_ctx_tokens, 0};
      if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream), what)) != PKV_OK) return rc;
    }
    if (num_gen > 0) {
      pkv::CheckSeqArgs c{nullptr, nullptr, 0, gen.seq_lens, nullptr, nullptr, gen.block_tables,
                          num_gen, max_blocks_per_seq, num_blocks, block_size, max_seq_len, 1, 0, 0};
      if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream), what)) != PKV_OK) return rc;
    }
  }
  // the context rows through the prefill kernel, then the generation rows through the
  // decode kernels, on the caller's stream
  if (num_ctx_seqs > 0 && num_ctx_tokens > 0) {
    const hipError_t e = pkv::prefill_mfma_supported(ctx)
                             ? pkv::launch_prefill_mfma(ctx, (hipStream_t)stream)
                             : pkv::launch_prefill_valu(ctx, (hipStream_t)stream);
    if ((rc = launched(e, what)) != PKV_OK) return rc;
  }
  if (num_gen > 0) return launched(pkv::launch_decode(gen, plan, (hipStream_t)stream), what);
  return PKV_OK;
}

int pkv_smallseq_attention_fwd(void* out, void* weights, const void* query,
                               const void* key_cache, const void* value_cache,
                               int64_t cache_block_stride, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks, int32_t block_size,
                               float scale, int32_t max_seq_len, pkv_dtype dtype, void* stream) {
  clear_error();
  const char* what = "pkv_smallseq_attention_fwd";
  pkv::SmallArgs a{};
  int rc = smallseq_common(a, query, key_cache, value_cache, cache_block_stride, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads,
                           head_dim, num_blocks, block_size, scale, max_seq_len, dtype, what);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (!out || !weights)
    return fail(PKV_ERR_INVALID_ARG, "out and weights must not be NULL");
  if (!aligned(out, 16) || !aligned(weights, 2))
    return fail(PKV_ERR_INVALID_ARG, "out must be 16-byte aligned and weights 2-byte aligned");
  a.out = out;
  a.weights = weights;
  if (a.guard != nullptr) {
    pkv::CheckSeqArgs c{nullptr, nullptr, 0, seq_lens, nullptr, nullptr, block_tables, num_seqs,
                        max_blocks_per_seq, num_blocks, block_size, max_seq_len, 1, 0, 0};
    if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream), what)) != PKV_OK) return rc;
  }
  return launched(pkv::launch_smallseq(a, false, (hipStream_t)stream), what);
}

int pkv_smallseq_attention_bwd(void* d_query, void* d_key, void* d_value, const void* d_out,
                               const void* query, const void* weights, const void* key_cache,
                               const void* value_cache, int64_t cache_block_stride,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, const int32_t* cu_seq_lens,
                               int32_t num_seqs, int32_t total_kv, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               int32_t block_size, float scale, int32_t max_seq_len,
                               pkv_dtype dtype, void* stream) {
  clear_error();
  const char* what = "pkv_smallseq_attention_bwd";
  pkv::SmallArgs a{};
  int rc = smallseq_common(a, query, key_cache, value_cache, cache_block_stride, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_heads, num_kv_heads,
                           head_dim, num_blocks, block_size, scale, max_seq_len, dtype, what);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (total_kv < 0) return fail(PKV_ERR_INVALID_ARG, "total_kv must be >= 0 (got %d)", total_kv);
  if (!d_query || !d_out || !weights || !cu_seq_lens || (total_kv > 0 && (!d_key || !d_value)))
    return fail(PKV_ERR_INVALID_ARG,
                "d_query, d_out, weights, cu_seq_lens (and d_key, d_value) must not be NULL");
  if (!aligned(d_query, 16) || !aligned(d_out, 16) || !aligned(weights, 2) ||
      (total_kv > 0 && (!aligned(d_key, 16) || !aligned(d_value, 16))))
    return fail(PKV_ERR_INVALID_ARG, "gradient rows must be 16-byte aligned, weights 2-byte");
  a.d_query = d_query;
  a.d_key = d_key;
  a.d_value = d_value;
  a.d_out = d_out;
  a.weights = const_cast<void*>(weights);
  a.cu_seq_lens = cu_seq_lens;
  if (a.guard != nullptr) {
    pkv::CheckSeqArgs c{nullptr, nullptr, 0, seq_lens, cu_seq_lens, nullptr, block_tables, num_seqs,
                        max_blocks_per_seq, num_blocks, block_size, max_seq_len, 0, 0, total_kv};
    if ((rc = launched(pkv::launch_check_seqs(c, (hipStream_t)stream), what)) != PKV_OK) return rc;
  }
  return launched(pkv::launch_smallseq(a, true, (hipStream_t)stream), what);
}

int pkv_paged_attention_prefill_spans(void* out, const void* query, const int32_t* cu_seqlens_q,
                                      const int32_t* seq_lens, const void* key_cache,
                                      const void* value_cache, int64_t cache_block_stride,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                      int32_t block_size, float scale, const int32_t* full_spans,
                                      const int32_t* cu_spans, int32_t num_spans,
                                      int32_t max_q_len, int32_t max_seq_len, pkv_dtype dtype,
                                      void* stream) {
  clear_error();
  if (num_spans < 0) return fail(PKV_ERR_INVALID_ARG, "num_spans must be >= 0 (got %d)", num_spans);
  if (num_spans > 0 && (!full_spans || !cu_spans))
    return fail(PKV_ERR_INVALID_ARG, "full_spans and cu_spans must not be NULL when num_spans > 0");
  // no full span: plain causal prefill
  const int mask = num_spans > 0 ? pkv::kMaskSpansHost : (int)PKV_MASK_CAUSAL;
  return prefill_common(out, query, cu_seqlens_q, seq_lens, key_cache, value_cache,
                        cache_block_stride, block_tables, max_blocks_per_seq, num_seqs, num_tokens,
                        num_heads, num_kv_heads, head_dim, num_blocks, block_size, scale, mask, 1,
                        num_spans > 0 ? full_spans : nullptr, num_spans > 0 ? cu_spans : nullptr,
                        num_spans, max_q_len, max_seq_len, dtype, stream,
                        "pkv_paged_attention_prefill_spans");
}

}  // extern "C"
