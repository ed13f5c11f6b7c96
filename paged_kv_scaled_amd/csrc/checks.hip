// Device-side checks of the preconditions on device memory that the host cannot see
// without a copy (the calls never copy to the host): slot range, sequence lengths
// against the host hints, the block-table entries a sequence uses, and cu_seqlens_q.
// A failed check ORs its bit into a per-device word; while that word is non-zero every
// kernel of the library returns before touching memory (the guard argument).
#include <mutex>

#include "../../include/pkv.h"
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kMaxDevices = 64;

__device__ uint32_t g_check_word;   // OR of pkv_check_bits since the last read
__device__ uint32_t g_check_taken;  // the value the last read took

__global__ void __launch_bounds__(kCheckThreads)
check_slots_kernel(const int64_t* __restrict__ slots, int32_t n, int64_t num_slots,
                   uint32_t* word) {
  bool bad = false;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    bad |= slots[i] >= num_slots;
  if (__any(bad) && (threadIdx.x & (kWave - 1)) == 0) atomicOr(word, (uint32_t)PKV_CHECK_SLOT_RANGE);
}

// One wave per sequence.
__global__ void __launch_bounds__(kCheckThreads)
check_seqs_kernel(const CheckSeqArgs a, uint32_t* word) {
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x * (kCheckThreads / kWave) + threadIdx.x / kWave;
  if (s >= a.num_seqs) return;
  uint32_t bits = 0;
  int64_t L;
  if (a.cu_seq_lens != nullptr) {        // gather: lengths are differences of cu_seq_lens
    const int64_t c0 = a.cu_seq_lens[s], c1 = a.cu_seq_lens[s + 1];
    L = c1 - c0;
    if ((s == 0 && c0 != 0) || (s == a.num_seqs - 1 && c1 != a.total_tokens)) bits |= PKV_CHECK_SEQ_LEN;
    // both given (small-seq backward): they must agree
    if (a.seq_lens != nullptr && a.seq_lens[s] != L) bits |= PKV_CHECK_SEQ_LEN;
  } else {
    L = a.seq_lens[s];
  }
  const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
  if (L < 0 || L > a.max_seq_len || L > cap) bits |= PKV_CHECK_SEQ_LEN;
  const int64_t Lc = L < 0 ? 0 : (L > cap ? cap : L);
  const int64_t pages = (Lc + a.block_size - 1) / a.block_size;
  bool bad = false;
  for (int64_t j = lane; j < pages; j += kWave) {
    const int32_t b = a.block_tables[(int64_t)s * a.max_blocks_per_seq + j];
    bad |= b < 0 || b >= a.num_blocks;
  }
  if (__any(bad)) bits |= PKV_CHECK_TABLE;
  if (a.cu_seqlens_q != nullptr) {       // prefill: this sequence's query segment
    const int64_t q0 = a.cu_seqlens_q[s], q1 = a.cu_seqlens_q[s + 1];
    const int64_t q = q1 - q0;
    if ((s == 0 && q0 != 0) || q < 0 || q > a.max_q_len || q > L ||
        (s == a.num_seqs - 1 && q1 != a.num_tokens))
      bits |= PKV_CHECK_CU_Q;
  }
  if (a.cu_spans != nullptr) {           // prefill with span lists: sorted, disjoint, inside the list
    const int64_t n0 = a.cu_spans[s], n1 = a.cu_spans[s + 1];
    bool bad_sp = (s == 0 && n0 != 0) || n1 < n0 || n0 < 0 || n1 > a.num_spans ||
                  (s == a.num_seqs - 1 && n1 != a.num_spans);
    if (!bad_sp) {
      bool b2 = false;
      for (int64_t i = n0 + lane; i < n1; i += kWave) {
        const int32_t st = a.full_spans[2 * i], en = a.full_spans[2 * i + 1];
        b2 |= st < 0 || en <= st || (i > n0 && st < a.full_spans[2 * i - 1]);
      }
      bad_sp = __any(b2);
    }
    if (bad_sp) bits |= PKV_CHECK_SPANS;
  }
  if (bits != 0 && lane == 0) atomicOr(word, bits);
}

// Duplicate slots of one kv_cache_write call (two tokens with one slot race in the
// scatter): one bit per cache slot in a caller-owned bitmap, all clear between calls.
// Pass 1 sets each valid slot's bit and flags a bit that was already set; pass 2, a
// separate launch on the same stream, clears the bits again.  Negative and
// out-of-range slots are skipped (the range check covers the latter).
__global__ void __launch_bounds__(kCheckThreads)
mark_slots_kernel(const int64_t* __restrict__ slots, int32_t n, int64_t num_slots,
                  uint32_t* __restrict__ marks, uint32_t* word) {
  bool dup = false;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
    const int64_t sl = slots[i];
    if (sl < 0 || sl >= num_slots) continue;
    const uint32_t bit = 1u << (sl & 31);
    dup |= (atomicOr(marks + (sl >> 5), bit) & bit) != 0u;
  }
  if (__any(dup) && (threadIdx.x & (kWave - 1)) == 0) atomicOr(word, (uint32_t)PKV_CHECK_DUP_SLOT);
}

__global__ void __launch_bounds__(kCheckThreads)
clear_slots_kernel(const int64_t* __restrict__ slots, int32_t n, int64_t num_slots,
                   uint32_t* __restrict__ marks) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
    const int64_t sl = slots[i];
    if (sl < 0 || sl >= num_slots) continue;
    atomicAnd(marks + (sl >> 5), ~(1u << (sl & 31)));
  }
}

// Move the word into g_check_taken and clear it, in one atomic step.
__global__ void take_word_kernel(uint32_t* word, uint32_t* taken) {
  if (threadIdx.x == 0) *taken = atomicExch(word, 0u);
}

struct Symbols {
  uint32_t* word = nullptr;
  uint32_t* taken = nullptr;
};

// Device addresses of the two words on the current device (each GPU has its own copy).
bool symbols(Symbols& out) {
  static std::mutex mu;
  static Symbols table[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  Symbols& s = table[dev];
  if (s.word == nullptr) {
    void* w = nullptr;
    void* t = nullptr;
    if (hipGetSymbolAddress(&w, HIP_SYMBOL(g_check_word)) != hipSuccess) return false;
    if (hipGetSymbolAddress(&t, HIP_SYMBOL(g_check_taken)) != hipSuccess) return false;
    s.word = static_cast<uint32_t*>(w);
    s.taken = static_cast<uint32_t*>(t);
  }
  out = s;
  return true;
}

}  // namespace

const uint32_t* check_guard() {
  Symbols s;
  return symbols(s) ? s.word : nullptr;
}

hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t num_slots, hipStream_t stream) {
  Symbols s;
  if (!symbols(s)) return hipErrorInvalidSymbol;
  if (n <= 0) return hipSuccess;
  const int64_t want = ((int64_t)n + kCheckThreads - 1) / kCheckThreads;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(check_slots_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream, slots, n,
                     num_slots, s.word);
  return hipGetLastError();
}

hipError_t launch_check_seqs(const CheckSeqArgs& a, hipStream_t stream) {
  Symbols s;
  if (!symbols(s)) return hipErrorInvalidSymbol;
  if (a.num_seqs <= 0) return hipSuccess;
  const int per_block = kCheckThreads / kWave;
  const int blocks = (a.num_seqs + per_block - 1) / per_block;
  hipLaunchKernelGGL(check_seqs_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream, a, s.word);
  return hipGetLastError();
}

hipError_t launch_check_duplicate_slots(const int64_t* slots, int32_t n, int64_t num_slots,
                                        uint32_t* marks, hipStream_t stream) {
  Symbols s;
  if (!symbols(s)) return hipErrorInvalidSymbol;
  if (n <= 0) return hipSuccess;
  const int64_t want = ((int64_t)n + kCheckThreads - 1) / kCheckThreads;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(mark_slots_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream, slots, n,
                     num_slots, marks, s.word);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_slots_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream, slots, n,
                     num_slots, marks);
  return hipGetLastError();
}

hipError_t take_check_word(hipStream_t stream, uint32_t* bits) {
  Symbols s;
  if (!symbols(s)) return hipErrorInvalidSymbol;
  hipLaunchKernelGGL(take_word_kernel, dim3(1), dim3(kWave), 0, stream, s.word, s.taken);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t v = 0;
  if ((e = hipMemcpyAsync(&v, s.taken, sizeof(v), hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  *bits = v;
  return hipSuccess;
}

}  // namespace pkv
