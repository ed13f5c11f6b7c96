// Small-seq training path: attention with saved weights, and its backward.
//
// What is computed (ROCm TransformerEngine small-seq PR, description: varlen cross
// attention with one query token per sequence and at most 16 keys; the forward writes the
// attention weights, the backward reads them and computes grad_V, grad_attn, the softmax
// backward and grad_Q / grad_K).  For sequence s, query head h, kv head j = h / g and keys
// k < L_s (read from the paged cache through the block table):
//   forward   P[h, k] = softmax_k(scale <q[h], K[k, j]>),   out[h] = sum_k P[h, k] V[k, j]
//   backward  dV[k, j] = sum_{h of j} P[h, k] dO[h]                         (grad_V)
//             dP[h, k] = <dO[h], V[k, j]>                                   (grad_attn)
//             dS[h, k] = P[h, k] (dP[h, k] - sum_k' P[h, k'] dP[h, k'])     (softmax bwd)
//             dQ[h]    = scale sum_k dS[h, k] K[k, j]                       (grad_Q)
//             dK[k, j] = scale sum_{h of j} dS[h, k] q[h]                   (grad_K)
// The backward takes P from the weights the forward saved (in the query type, as the
// page's attention-weights buffer is), not from a recomputation.
//
// How (MI355X, HBM / latency bound, vector ALU): one wave owns one (sequence, kv head)
// item.  Lanes = (key t of a round, column c): LPT lanes share a key row, each holding EPL
// contiguous elements (one or two 16-byte loads), and TPR = 64 / LPT keys make a round;
// with at most 16 keys an item takes one or two rounds.  K and V of the item stay in
// registers while the wave walks the g query heads of its kv head, so dK and dV sum over
// the group in registers and are written once.  Dot products reduce over the LPT lanes of
// a key with xor shuffles; sums over keys reduce over the key lanes and the rounds.
#include "decode_device.h"

namespace pkv {

namespace {

constexpr int kSmallThreads = 256;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallMaxKv = 16;

template <int D>
struct SmallShape {
  static constexpr int LPT = D / 8 < 8 ? D / 8 : 8;     // lanes per key row
  static constexpr int EPL = D / LPT;                   // elements per lane (8 or 16)
  static constexpr int TPR = kWave / LPT;               // keys per round
  static constexpr int NR = (kSmallMaxKv + TPR - 1) / TPR;   // rounds
  static constexpr int NV = EPL / 8;                    // 16-byte vectors per lane
};

struct SmallParams {
  void* out;              // forward: [S, H, D]
  void* weights;          // [S, H, max_kv], query type
  const void* query;      // [S, H, D]
  const void* d_out;      // backward: [S, H, D]
  void* d_query;          // backward: [S, H, D]
  void* d_key;            // backward: [total_kv, Hkv, D] (THD rows cu_kv[s] + k)
  void* d_value;
  const void* kc;
  const void* vc;
  int64_t block_stride;   // elements
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* cu_kv;   // backward only
  int32_t mb, S, H, Hkv, g, block_shift, max_kv;
  float scale;
  const uint32_t* guard;
};

// The lane's EPL elements of a row of D storage elements starting at `row`, as packed
// pairs (word i holds elements 2i, 2i+1).
template <typename T, int D>
__device__ __forceinline__ void load_words(const typename T::storage* base, int64_t row, int c,
                                           uint32_t (&x)[SmallShape<D>::EPL / 2]) {
  using C = SmallShape<D>;
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + row + c * C::EPL);
#pragma unroll
  for (int v = 0; v < C::NV; ++v) {
    const u32x4_t w = p[v];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[v * 4 + i] = w[i];
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_row(typename T::storage* base, int64_t row, int c,
                                          const float (&x)[SmallShape<D>::EPL]) {
  using C = SmallShape<D>;
  u32x4_t* p = reinterpret_cast<u32x4_t*>(base + row + c * C::EPL);
#pragma unroll
  for (int v = 0; v < C::NV; ++v) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2(T{}, x[v * 8 + 2 * i], x[v * 8 + 2 * i + 1]);
    p[v] = w;
  }
}

// Store of the lane's D/8 contiguous elements (8 lanes per row).
template <typename T, int D>
__device__ __forceinline__ void store_row_c(typename T::storage* base, int64_t row, int c,
                                            const float (&x)[D / 8]) {
  constexpr int EPL = D / 8;
  u32x4_t* p = reinterpret_cast<u32x4_t*>(base + row + c * EPL);
#pragma unroll
  for (int v = 0; v < EPL / 8; ++v) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack2(T{}, x[v * 8 + 2 * i], x[v * 8 + 2 * i + 1]);
    p[v] = w;
  }
}

// <a, b> over the lane's elements (packed pairs, fp32 accumulate).
template <typename T, int N>
__device__ __forceinline__ float dot_words(const uint32_t (&a)[N], const uint32_t (&b)[N]) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) d = dot2(T{}, a[i], b[i], d);
  return d;
}

// Sum over the LPT lanes of one key row (lanes t*LPT .. t*LPT+LPT-1).
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < LPT; off <<= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Sum / max over the key lanes of a round (lanes with the same column).
template <int LPT>
__device__ __forceinline__ float keys_sum(float x) {
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
  return x;
}
template <int LPT>
__device__ __forceinline__ float keys_max(float x) {
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

// K and V rows of the item's keys (key t + r*TPR in round r) as packed pairs.  The length
// and the page ids load together (ids for keys past the length are read but not used:
// the table row holds max_blocks_per_seq >= pages of max_kv entries); keys past L re-read
// key 0.  Returns L (clamped to max_kv); nothing is loaded when it is 0.
template <typename T, int D>
__device__ __forceinline__ int load_kv(const SmallParams& p, int s, int kvh, int t, int c,
                                       uint32_t (&k)[SmallShape<D>::NR][SmallShape<D>::EPL / 2],
                                       uint32_t (&v)[SmallShape<D>::NR][SmallShape<D>::EPL / 2]) {
  using C = SmallShape<D>;
  using S = typename T::storage;
  const int32_t* table = p.block_tables + (int64_t)s * p.mb;
  const int bmask = (1 << p.block_shift) - 1;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  int ids[C::NR];
#pragma unroll
  for (int r = 0; r < C::NR; ++r) ids[r] = table[min(t + r * C::TPR, p.max_kv - 1) >> p.block_shift];
  const int id0 = table[0];
  const int L = min(p.seq_lens[s], p.max_kv);
  if (L <= 0) return 0;
#pragma unroll
  for (int r = 0; r < C::NR; ++r) {
    const int pos_raw = t + r * C::TPR;
    const bool in = pos_raw < L;
    const int pos = in ? pos_raw : 0;
    const int64_t blk = in ? ids[r] : id0;
    const int64_t row = blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + (int64_t)kvh * D;
    load_words<T, D>(reinterpret_cast<const S*>(p.kc), row, c, k[r]);
    load_words<T, D>(reinterpret_cast<const S*>(p.vc), row, c, v[r]);
  }
  return L;
}

template <typename T, int D>
__global__ void __launch_bounds__(kSmallThreads)
smallseq_fwd_kernel(const SmallParams p) {
  if (guard_tripped(p.guard)) return;
  using C = SmallShape<D>;
  using S = typename T::storage;
  constexpr int W = C::EPL / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int64_t item = (int64_t)blockIdx.x * kSmallWaves + threadIdx.x / kWave;
  if (item >= (int64_t)p.S * p.Hkv) return;
  const int s = (int)(item / p.Hkv), kvh = (int)(item % p.Hkv);
  uint32_t k[C::NR][W], v[C::NR][W], q[W];
  // the first head's query row loads together with the length, page ids and K/V
  load_words<T, D>(reinterpret_cast<const S*>(p.query), ((int64_t)s * p.H + kvh * p.g) * D, c, q);
  const int L = load_kv<T, D>(p, s, kvh, t, c, k, v);
  for (int hi = 0; hi < p.g; ++hi) {
    const int h = kvh * p.g + hi;
    const int64_t qrow = ((int64_t)s * p.H + h) * D;
    float pr[C::NR], o[C::EPL];
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int r = 0; r < C::NR; ++r) pr[r] = 0.f;
    if (L > 0) {
      if (hi > 0) load_words<T, D>(reinterpret_cast<const S*>(p.query), qrow, c, q);
      float z[C::NR];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < C::NR; ++r) {
        const float d = row_sum<C::LPT>(dot_words<T>(q, k[r])) * p.scale;
        z[r] = (t + r * C::TPR < L) ? d : -INFINITY;
        mx = fmaxf(mx, z[r]);
      }
      mx = keys_max<C::LPT>(mx);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < C::NR; ++r) {
        pr[r] = (t + r * C::TPR < L) ? __expf(z[r] - mx) : 0.f;
        sum += pr[r];
      }
      sum = keys_sum<C::LPT>(sum);
      const float inv = 1.f / sum;
#pragma unroll
      for (int r = 0; r < C::NR; ++r) {
        pr[r] *= inv;
#pragma unroll
        for (int i = 0; i < W; ++i) {
          o[2 * i] = __builtin_fmaf(pr[r], lo_of(T{}, v[r][i]), o[2 * i]);
          o[2 * i + 1] = __builtin_fmaf(pr[r], hi_of(T{}, v[r][i]), o[2 * i + 1]);
        }
      }
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) o[e] = keys_sum<C::LPT>(o[e]);
    }
    // weights: one lane per key writes P (zero past L, up to max_kv)
    S* wrow = reinterpret_cast<S*>(p.weights) + ((int64_t)s * p.H + h) * p.max_kv;
#pragma unroll
    for (int r = 0; r < C::NR; ++r) {
      const int key = t + r * C::TPR;
      if (c == 0 && key < p.max_kv) wrow[key] = (S)(pack2(T{}, pr[r], 0.f) & 0xFFFFu);
    }
    if (t == 0) store_row<T, D>(reinterpret_cast<S*>(p.out), qrow, c, o);
  }
}

// GROUP: more than one query head per kv head, so dK and dV sum over the heads in fp32
// registers; with one head per kv head each key row is written as soon as it is known.
template <typename T, int D, bool GROUP>
__global__ void __launch_bounds__(kSmallThreads)
smallseq_bwd_kernel(const SmallParams p) {
  if (guard_tripped(p.guard)) return;
  using C = SmallShape<D>;
  using S = typename T::storage;
  constexpr int W = C::EPL / 2;
  constexpr int NA = GROUP ? C::NR : 1;       // rounds of fp32 dK / dV accumulators
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int64_t item = (int64_t)blockIdx.x * kSmallWaves + threadIdx.x / kWave;
  if (item >= (int64_t)p.S * p.Hkv) return;
  const int s = (int)(item / p.Hkv), kvh = (int)(item % p.Hkv);
  uint32_t k[C::NR][W], v[C::NR][W];
  float dk[NA][C::EPL], dv[NA][C::EPL];
#pragma unroll
  for (int r = 0; r < NA; ++r)
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) dk[r][e] = dv[r][e] = 0.f;
  // the first head's query and output-gradient rows load together with the length, page
  // ids and K/V
  uint32_t q[W], go[W];
  const int64_t qrow0 = ((int64_t)s * p.H + kvh * p.g) * D;
  load_words<T, D>(reinterpret_cast<const S*>(p.query), qrow0, c, q);
  load_words<T, D>(reinterpret_cast<const S*>(p.d_out), qrow0, c, go);
  const int L = load_kv<T, D>(p, s, kvh, t, c, k, v);
  const int64_t base = p.cu_kv[s];
  for (int hi = 0; hi < p.g; ++hi) {
    const int h = kvh * p.g + hi;
    const int64_t qrow = ((int64_t)s * p.H + h) * D;
    float dq[C::EPL];
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) dq[e] = 0.f;
    if (L > 0) {
      if (hi > 0) {
        load_words<T, D>(reinterpret_cast<const S*>(p.query), qrow, c, q);
        load_words<T, D>(reinterpret_cast<const S*>(p.d_out), qrow, c, go);
      }
      const S* wrow = reinterpret_cast<const S*>(p.weights) + ((int64_t)s * p.H + h) * p.max_kv;
      float pr[C::NR], dp[C::NR];
      float dsum = 0.f;
#pragma unroll
      for (int r = 0; r < C::NR; ++r) {
        const int key = t + r * C::TPR;
        pr[r] = key < L ? lo_of(T{}, (uint32_t)wrow[key]) : 0.f;
        dp[r] = row_sum<C::LPT>(dot_words<T>(go, v[r]));            // grad_attn
        dsum = __builtin_fmaf(pr[r], dp[r], dsum);
      }
      dsum = keys_sum<C::LPT>(dsum);
#pragma unroll
      for (int r = 0; r < C::NR; ++r) {
        const int key = t + r * C::TPR;
        const float ds = pr[r] * (dp[r] - dsum) * p.scale;           // softmax bwd (scaled)
        float rk[C::EPL], rv[C::EPL];
#pragma unroll
        for (int i = 0; i < W; ++i) {
          dq[2 * i] = __builtin_fmaf(ds, lo_of(T{}, k[r][i]), dq[2 * i]);          // grad_Q
          dq[2 * i + 1] = __builtin_fmaf(ds, hi_of(T{}, k[r][i]), dq[2 * i + 1]);
          rk[2 * i] = ds * lo_of(T{}, q[i]);                                       // grad_K
          rk[2 * i + 1] = ds * hi_of(T{}, q[i]);
          rv[2 * i] = pr[r] * lo_of(T{}, go[i]);                                   // grad_V
          rv[2 * i + 1] = pr[r] * hi_of(T{}, go[i]);
        }
        if constexpr (GROUP) {
#pragma unroll
          for (int e = 0; e < C::EPL; ++e) {
            dk[r][e] += rk[e];
            dv[r][e] += rv[e];
          }
        } else if (key < L) {
          const int64_t row = ((base + key) * p.Hkv + kvh) * D;
          store_row<T, D>(reinterpret_cast<S*>(p.d_key), row, c, rk);
          store_row<T, D>(reinterpret_cast<S*>(p.d_value), row, c, rv);
        }
      }
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) dq[e] = keys_sum<C::LPT>(dq[e]);
    }
    if (t == 0) store_row<T, D>(reinterpret_cast<S*>(p.d_query), qrow, c, dq);
  }
  if constexpr (GROUP) {
    // dK, dV rows of the item's keys, THD at cu_kv[s] + key
#pragma unroll
    for (int r = 0; r < C::NR; ++r) {
      const int key = t + r * C::TPR;
      if (key < L) {
        const int64_t row = ((base + key) * p.Hkv + kvh) * D;
        store_row<T, D>(reinterpret_cast<S*>(p.d_key), row, c, dk[r]);
        store_row<T, D>(reinterpret_cast<S*>(p.d_value), row, c, dv[r]);
      }
    }
  }
}

// Backward with one query head per kv head, eight items per wave (as decode item mode):
// each group of 8 lanes owns one (sequence, head) item and walks its keys itself, so the
// dependent loads of eight items overlap.  Lane c holds elements c*EPL .. c*EPL+EPL-1 of
// every row and page c of the item.  Pass 1 reads the V rows (grad_attn, then the
// softmax-backward mean); pass 2 reads the K rows, accumulates grad_Q in the lane and
// writes the grad_K and grad_V rows of each key.
template <typename T, int D>
__global__ void __launch_bounds__(kSmallThreads)
smallseq_bwd_items_kernel(const SmallParams p) {
  if (guard_tripped(p.guard)) return;
  using S = typename T::storage;
  constexpr int LPT = 8;
  constexpr int EPL = D / LPT;
  constexpr int W = EPL / 2;
  constexpr int NV = EPL / 8;
  constexpr int KB = 4;                                   // keys whose loads go together
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / LPT, c = lane % LPT;
  const int64_t wave = (int64_t)blockIdx.x * kSmallWaves + threadIdx.x / kWave;
  const int64_t items = (int64_t)p.S * p.Hkv;
  if (wave * 8 >= items) return;                          // uniform over the wave
  const int64_t item_raw = wave * 8 + t;
  const bool live = item_raw < items;
  const int64_t item = live ? item_raw : items - 1;
  const int s = (int)(item / p.Hkv), kvh = (int)(item % p.Hkv);
  const int L = min(p.seq_lens[s], p.max_kv);
  const int last_page = L > 0 ? (L - 1) >> p.block_shift : -1;
  const int32_t pid = c <= last_page ? p.block_tables[(int64_t)s * p.mb + c] : 0;
  const int64_t qrow = ((int64_t)s * p.H + kvh) * D;       // g == 1: head = kv head
  uint32_t q[W], go[W];
  {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const S*>(p.query) + qrow + c * EPL);
    const u32x4_t* gp = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const S*>(p.d_out) + qrow + c * EPL);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const u32x4_t a = qp[v], b = gp[v];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[v * 4 + i] = a[i];
        go[v * 4 + i] = b[i];
      }
    }
  }
  // the item's weights (every lane of the group reads the same row); keys past L re-read
  // entry min(k, L-1), inside the row, and count as 0
  float pr[kSmallMaxKv];
  {
    const S* wrow = reinterpret_cast<const S*>(p.weights) + ((int64_t)s * p.H + kvh) * p.max_kv;
#pragma unroll
    for (int k = 0; k < kSmallMaxKv; ++k) {
      const uint32_t w = wrow[min(k, max(L - 1, 0))];
      pr[k] = k < L ? lo_of(T{}, w) : 0.f;
    }
  }
  int Lw = L;
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) Lw = max(Lw, __shfl_xor(Lw, off, kWave));
  const int bmask = (1 << p.block_shift) - 1;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  auto row_of = [&](int k) -> int64_t {                    // cache row of key k (a real key)
    const int pos = min(k, max(L - 1, 0));
    const int64_t blk = __shfl(pid, t * LPT + (pos >> p.block_shift), kWave);
    return blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + (int64_t)kvh * D + c * EPL;
  };
  // pass 1: dP = <dO, V[k]> and the mean sum_k P dP
  float dp[kSmallMaxKv];
  float dsum = 0.f;
#pragma unroll
  for (int k0 = 0; k0 < kSmallMaxKv; k0 += KB) {
#pragma unroll
    for (int k = k0; k < k0 + KB; ++k) dp[k] = 0.f;
    if (k0 < Lw) {
      uint32_t vr[KB][W];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const S*>(p.vc) + row_of(k0 + kk));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const u32x4_t a = vp[v];
#pragma unroll
          for (int i = 0; i < 4; ++i) vr[kk][v * 4 + i] = a[i];
        }
      }
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < W; ++i) d = dot2(T{}, go[i], vr[kk][i], d);
#pragma unroll
        for (int off = 1; off < LPT; off <<= 1) d += __shfl_xor(d, off, kWave);
        dp[k0 + kk] = d;
        dsum = __builtin_fmaf(pr[k0 + kk], d, dsum);
      }
    }
  }
  // pass 2: dS, grad_Q (in the lane), grad_K and grad_V rows
  float dq[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) dq[e] = 0.f;
  const int64_t base = p.cu_kv[s];
#pragma unroll
  for (int k0 = 0; k0 < kSmallMaxKv; k0 += KB) {
    if (k0 < Lw) {
      uint32_t kr[KB][W];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const S*>(p.kc) + row_of(k0 + kk));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const u32x4_t a = kp[v];
#pragma unroll
          for (int i = 0; i < 4; ++i) kr[kk][v * 4 + i] = a[i];
        }
      }
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int k = k0 + kk;
        const float ds = pr[k] * (dp[k] - dsum) * p.scale;
        float rk[EPL], rv[EPL];
#pragma unroll
        for (int i = 0; i < W; ++i) {
          dq[2 * i] = __builtin_fmaf(ds, lo_of(T{}, kr[kk][i]), dq[2 * i]);
          dq[2 * i + 1] = __builtin_fmaf(ds, hi_of(T{}, kr[kk][i]), dq[2 * i + 1]);
          rk[2 * i] = ds * lo_of(T{}, q[i]);
          rk[2 * i + 1] = ds * hi_of(T{}, q[i]);
          rv[2 * i] = pr[k] * lo_of(T{}, go[i]);
          rv[2 * i + 1] = pr[k] * hi_of(T{}, go[i]);
        }
        if (live && k < L) {
          const int64_t row = ((base + k) * p.Hkv + kvh) * D;
          store_row_c<T, D>(reinterpret_cast<S*>(p.d_key), row, c, rk);
          store_row_c<T, D>(reinterpret_cast<S*>(p.d_value), row, c, rv);
        }
      }
    }
  }
  if (live) store_row_c<T, D>(reinterpret_cast<S*>(p.d_query), qrow, c, dq);
}

// The forward with one or two query heads per kv head and head_dim 64 / 128 runs as the
// decode item mode with weights (eight items per wave, so that their dependent loads
// overlap); other shapes take smallseq_fwd_kernel.
template <typename T>
bool launch_fwd_items(const SmallParams& sp, int d, hipStream_t stream) {
  if (!(d == 128 || d == 64) || sp.g > 2) return false;
  DecodeParams p{};
  p.out = sp.out;
  p.query = sp.query;
  p.kc = sp.kc;
  p.vc = sp.vc;
  p.block_stride = sp.block_stride;
  p.block_tables = sp.block_tables;
  p.seq_lens = sp.seq_lens;
  p.mb = sp.mb;
  p.S = sp.S;
  p.H = sp.H;
  p.Hkv = sp.Hkv;
  p.g = sp.g;
  p.block_shift = sp.block_shift;
  p.groups_per_kv = 1;
  p.nsplit = 1;
  p.split_len = sp.max_kv;
  p.total_items = (int64_t)sp.S * sp.Hkv;
  p.scale_log2 = sp.scale * kLog2e;
  p.out_scale = 1.f;
  p.guard = sp.guard;
  p.weights = sp.weights;
  p.max_kv = sp.max_kv;
  const int64_t waves = (p.total_items + 7) / 8;
  const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)), block(kDecodeThreads);
  PKV_LOG_LAUNCH("decode_items_weights_kernel", grid.x, kDecodeThreads,
                 "D=%d heads_per_item=%d items=%lld max_kv=%d", d, sp.g, (long long)p.total_items,
                 sp.max_kv);
#define PKV_ITEMS(DD, HH) \
  hipLaunchKernelGGL((decode_items_weights_kernel<T, DD, HH>), grid, block, 0, stream, p)
  if (d == 128) {
    if (sp.g == 1) PKV_ITEMS(128, 1); else PKV_ITEMS(128, 2);
  } else {
    if (sp.g == 1) PKV_ITEMS(64, 1); else PKV_ITEMS(64, 2);
  }
#undef PKV_ITEMS
  return true;
}

template <typename T>
void launch_small(const SmallParams& p, int d, bool backward, hipStream_t stream) {
  if (!backward && launch_fwd_items<T>(p, d, stream)) return;
  if (backward && p.g == 1 && (d == 128 || d == 64)) {
    const int64_t waves = ((int64_t)p.S * p.Hkv + 7) / 8;
    const dim3 grid((unsigned)((waves + kSmallWaves - 1) / kSmallWaves)), block(kSmallThreads);
    PKV_LOG_LAUNCH("smallseq_bwd_items_kernel", grid.x, kSmallThreads, "D=%d items=%lld max_kv=%d",
                   d, (long long)p.S * p.Hkv, p.max_kv);
    if (d == 128) hipLaunchKernelGGL((smallseq_bwd_items_kernel<T, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((smallseq_bwd_items_kernel<T, 64>), grid, block, 0, stream, p);
    return;
  }
  const int64_t items = (int64_t)p.S * p.Hkv;
  const dim3 grid((unsigned)((items + kSmallWaves - 1) / kSmallWaves)), block(kSmallThreads);
  PKV_LOG_LAUNCH(backward ? "smallseq_bwd_kernel" : "smallseq_fwd_kernel", grid.x, kSmallThreads,
                 "D=%d heads_per_kv=%d items=%lld max_kv=%d", d, p.g, (long long)items, p.max_kv);
#define PKV_SMALL(DD)                                                                        \
  if (!backward) hipLaunchKernelGGL((smallseq_fwd_kernel<T, DD>), grid, block, 0, stream, p); \
  else if (p.g > 1) hipLaunchKernelGGL((smallseq_bwd_kernel<T, DD, true>), grid, block, 0, stream, p); \
  else hipLaunchKernelGGL((smallseq_bwd_kernel<T, DD, false>), grid, block, 0, stream, p)
  switch (d) {
    case 16: PKV_SMALL(16); break;
    case 64: PKV_SMALL(64); break;
    default: PKV_SMALL(128); break;
  }
#undef PKV_SMALL
}

}  // namespace

hipError_t launch_smallseq(const SmallArgs& a, bool backward, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if ((int64_t)a.num_seqs * a.num_kv_heads > (int64_t)0x7FFFFFFF / kSmallWaves * kSmallWaves)
    return hipErrorInvalidValue;
  SmallParams p{};
  p.out = a.out;
  p.weights = a.weights;
  p.query = a.query;
  p.d_out = a.d_out;
  p.d_query = a.d_query;
  p.d_key = a.d_key;
  p.d_value = a.d_value;
  p.kc = a.key_cache;
  p.vc = a.value_cache;
  p.block_stride = a.block_stride;
  p.block_tables = a.block_tables;
  p.seq_lens = a.seq_lens;
  p.cu_kv = a.cu_seq_lens;
  p.mb = a.max_blocks_per_seq;
  p.S = a.num_seqs;
  p.H = a.num_heads;
  p.Hkv = a.num_kv_heads;
  p.g = a.num_heads / a.num_kv_heads;
  p.block_shift = log2_exact(a.block_size);
  p.max_kv = a.max_seq_len;
  p.scale = a.scale;
  p.guard = a.guard;
  if (a.dtype == kBF16) launch_small<BF16>(p, a.head_dim, backward, stream);
  else launch_small<F16>(p, a.head_dim, backward, stream);
  return hipGetLastError();
}

}  // namespace pkv
