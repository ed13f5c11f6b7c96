// Single-token decode over a paged KV cache: split-K flash decoding + log-sum-exp merge.
//
// What is computed (Spyre paged-attention PR, "Description": gather from scattered
// blocks, GQA by repeat_interleave, per-sequence attention): for each sequence s and
// query head h, out = softmax(scale * q K^T) V over the L_s cached keys of kv head
// h / (H / Hkv).  The ROCm TransformerEngine small-seq PR's s_q = 1, s_kv <= 16 varlen
// cross attention is the same call with one sequence per query token.
//
// How (MI355X design, HBM-bound, vector ALU only):
//  * one wave = one work item (sequence, group of HPW query heads sharing a kv head,
//    split of split_len keys); waves walk items in a grid-stride loop;
//  * lanes = (token t of a round, column c): a round covers TPR tokens, each token's
//    D-element row of one kv head is read by LPT lanes with 16-byte loads, so a wave
//    load instruction reads TPR contiguous row segments; the block-table gather is the
//    address computation of those loads (no gathered copy exists);
//  * q . k with packed dot2 (v_dot2_f32_bf16 / _f16) and a DPP reduction over the LPT
//    lanes of a token; every lane keeps a private online-softmax state (m, l, acc) over
//    the tokens it sees, the max is only moved when it grows by more than 2^8 (the
//    probabilities stay <= 256, exact after the final division);
//  * probabilities of two rounds are paired and multiplied into V with dot2 as well;
//  * at the end of the item the lanes of a column merge their states (shuffles), and
//    the wave writes either the final output (one split) or (acc, m, l) to the
//    workspace for the merge kernel.
#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kDecodeThreads = 256;
constexpr float kLazyRescale = 8.0f;   // log2 units

template <typename T, int D>
struct DecodeShape {
  static constexpr int EB = T::bytes;
  static constexpr int EPV = 16 / EB;              // elements per 16-byte vector
  static constexpr int NV = D / EPV;               // vectors per row of one head
  static constexpr int LPT = NV < 8 ? NV : 8;      // lanes per token
  static constexpr int VPL = NV / LPT;             // vectors per lane
  static constexpr int TPR = kWave / LPT;          // tokens per round
  static constexpr int WPL = VPL * 4;              // 32-bit words per lane per row
  static constexpr int EPL = VPL * EPV;            // elements per lane per row
  static_assert(NV >= 1 && NV % LPT == 0, "head_dim / dtype combination");
};

struct DecodeParams {
  void* out;
  const void* query;
  const void* kc;
  const void* vc;
  int64_t block_stride;     // elements
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;            // [S, H, nsplit, D]
  float* ws_ml;             // [S, H, nsplit, 2]  (max in log2 units, sum)
  int64_t total_items;
  int32_t mb, S, H, Hkv, g, block_shift, split_len, nsplit, groups_per_kv;
  float scale_log2;
};

template <typename T, int D>
struct Step {
  using C = DecodeShape<T, D>;
  uint32_t k[2][C::WPL];
  uint32_t v[2][C::WPL];
  bool valid[2];
};

template <typename T, int D>
__device__ __forceinline__ void load_step(Step<T, D>& st, const DecodeParams& p,
                                          const int32_t* __restrict__ table, int64_t head_off,
                                          int base, int end, int t, int c) {
  using C = DecodeShape<T, D>;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  const int bmask = (1 << p.block_shift) - 1;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int pos = base + r * C::TPR + t;
    st.valid[r] = pos < end;
    if (st.valid[r]) {
      const int64_t blk = table[pos >> p.block_shift];
      const int64_t row = blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + head_off;
      const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(
          reinterpret_cast<const typename T::storage*>(p.kc) + row);
      const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(
          reinterpret_cast<const typename T::storage*>(p.vc) + row);
#pragma unroll
      for (int v = 0; v < C::VPL; ++v) {
        const u32x4_t kk = kp[v * C::LPT + c];
        const u32x4_t vv = vp[v * C::LPT + c];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          st.k[r][v * 4 + w] = kk[w];
          st.v[r][v * 4 + w] = vv[w];
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < C::WPL; ++w) {
        st.k[r][w] = 0u;
        st.v[r][w] = 0u;
      }
    }
  }
}

// Sum over the LPT lanes that hold one token's row (DPP, no LDS).
template <int LPT>
__device__ __forceinline__ float reduce_token(float x) {
  if constexpr (LPT >= 2) x += dpp_f<kDppQuadXor1>(x);
  if constexpr (LPT >= 4) x += dpp_f<kDppQuadXor2>(x);
  if constexpr (LPT >= 8) x += dpp_f<kDppRowHalfMirror>(x);
  return x;
}

template <typename T, int D, int HPW>
__device__ __forceinline__ void compute_step(const Step<T, D>& st, const uint32_t (&q)[HPW][DecodeShape<T, D>::WPL],
                                             float (&m)[HPW], float (&l)[HPW],
                                             float (&acc)[HPW][DecodeShape<T, D>::EPL],
                                             float scale_log2) {
  using C = DecodeShape<T, D>;
  constexpr bool kHalf = T::bytes == 2;
  float sc[2][HPW];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < C::WPL; ++w) {
        if constexpr (kHalf) {
          d = dot2(T{}, q[hh][w], st.k[r][w], d);
        } else {
          d = __builtin_fmaf(__uint_as_float(q[hh][w]), __uint_as_float(st.k[r][w]), d);
        }
      }
      d = reduce_token<C::LPT>(d);
      sc[r][hh] = st.valid[r] ? d * scale_log2 : -INFINITY;
    }
  }
  // lazy max update: rescale only when a score exceeds the running max by > 2^8
  bool grow = false;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) grow |= fmaxf(sc[0][hh], sc[1][hh]) > m[hh] + kLazyRescale;
  if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float mn = fmaxf(m[hh], fmaxf(sc[0][hh], sc[1][hh]));
      const float alpha = (m[hh] == -INFINITY) ? 0.f : fast_exp2(m[hh] - mn);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) acc[hh][e] *= alpha;
      m[hh] = mn;
    }
  }
  float pr[2][HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int r = 0; r < 2; ++r) pr[r][hh] = st.valid[r] ? fast_exp2(sc[r][hh] - m[hh]) : 0.f;
    l[hh] += pr[0][hh] + pr[1][hh];
  }
  if constexpr (kHalf) {
    // pair the two rounds: x = (v0.lo, v1.lo), y = (v0.hi, v1.hi) for every word
#pragma unroll
    for (int w = 0; w < C::WPL; ++w) {
      const uint32_t a = st.v[0][w], b = st.v[1][w];
      const uint32_t x = (a & 0xFFFFu) | (b << 16);
      const uint32_t y = (a >> 16) | (b & 0xFFFF0000u);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const uint32_t pp = pack2(T{}, pr[0][hh], pr[1][hh]);
        acc[hh][2 * w] = dot2(T{}, pp, x, acc[hh][2 * w]);
        acc[hh][2 * w + 1] = dot2(T{}, pp, y, acc[hh][2 * w + 1]);
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < C::WPL; ++w) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        acc[hh][w] = __builtin_fmaf(pr[0][hh], __uint_as_float(st.v[0][w]), acc[hh][w]);
        acc[hh][w] = __builtin_fmaf(pr[1][hh], __uint_as_float(st.v[1][w]), acc[hh][w]);
      }
    }
  }
}

template <typename T, int D, int HPW>
__global__ void __launch_bounds__(kDecodeThreads)
decode_split_kernel(const DecodeParams p) {
  using C = DecodeShape<T, D>;
  using S = typename T::storage;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int64_t wave = (int64_t)blockIdx.x * (kDecodeThreads / kWave) + (threadIdx.x / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * (kDecodeThreads / kWave);
  const int HG = p.Hkv * p.groups_per_kv;

  for (int64_t item = wave; item < p.total_items; item += nwaves) {
    const int hg = (int)(item % HG);
    const int64_t sj = item / HG;
    const int j = (int)(sj % p.nsplit);
    const int s = (int)(sj / p.nsplit);
    const int L = p.seq_lens[s];
    const int start = j * p.split_len;
    if (j > 0 && start >= L) continue;
    const int end = min(L, start + p.split_len);
    const int ns = L > 0 ? (L + p.split_len - 1) / p.split_len : 1;
    const int kvh = hg / p.groups_per_kv, sub = hg % p.groups_per_kv;
    const int h0 = kvh * p.g + sub * HPW;
    const int nh = min(HPW, p.g - sub * HPW);

    uint32_t q[HPW][C::WPL];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (hh < nh) {
        const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const S*>(p.query) + ((int64_t)s * p.H + h0 + hh) * D);
#pragma unroll
        for (int v = 0; v < C::VPL; ++v) {
          const u32x4_t qq = qp[v * C::LPT + c];
#pragma unroll
          for (int w = 0; w < 4; ++w) q[hh][v * 4 + w] = qq[w];
        }
      } else {
#pragma unroll
        for (int w = 0; w < C::WPL; ++w) q[hh][w] = 0u;
      }
    }

    float m[HPW], l[HPW], acc[HPW][C::EPL];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) acc[hh][e] = 0.f;
    }

    const int32_t* table = p.block_tables + (int64_t)s * p.mb;
    const int64_t head_off = (int64_t)kvh * D;
    constexpr int STEP = 2 * C::TPR;
    if (start < end) {
      Step<T, D> a, b;
      load_step<T, D>(a, p, table, head_off, start, end, t, c);
      int base = start;
      while (true) {
        if (base + STEP < end) load_step<T, D>(b, p, table, head_off, base + STEP, end, t, c);
        compute_step<T, D, HPW>(a, q, m, l, acc, p.scale_log2);
        base += STEP;
        if (base >= end) break;
        if (base + STEP < end) load_step<T, D>(a, p, table, head_off, base + STEP, end, t, c);
        compute_step<T, D, HPW>(b, q, m, l, acc, p.scale_log2);
        base += STEP;
        if (base >= end) break;
      }
    }

    // merge the private states of the TPR token lanes of each column
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float M = m[hh];
#pragma unroll
      for (int off = C::LPT; off < kWave; off <<= 1) M = fmaxf(M, shfl_xor_f(M, off));
      const float f = (m[hh] == -INFINITY) ? 0.f : fast_exp2(m[hh] - M);
      float ll = l[hh] * f;
#pragma unroll
      for (int off = C::LPT; off < kWave; off <<= 1) ll += shfl_xor_f(ll, off);
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) {
        float x = acc[hh][e] * f;
#pragma unroll
        for (int off = C::LPT; off < kWave; off <<= 1) x += shfl_xor_f(x, off);
        acc[hh][e] = x;
      }
      m[hh] = M;
      l[hh] = ll;
    }

    if (t == 0) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        if (hh >= nh) continue;
        const int h = h0 + hh;
        if (ns == 1) {
          const float inv = l[hh] > 0.f ? 1.f / l[hh] : 0.f;
          u32x4_t* op = reinterpret_cast<u32x4_t*>(reinterpret_cast<S*>(p.out) +
                                                   ((int64_t)s * p.H + h) * D);
#pragma unroll
          for (int v = 0; v < C::VPL; ++v) {
            u32x4_t o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              if constexpr (T::bytes == 2) {
                const int e = (v * 4 + w) * 2;
                o[w] = pack2(T{}, acc[hh][e] * inv, acc[hh][e + 1] * inv);
              } else {
                o[w] = __float_as_uint(acc[hh][v * 4 + w] * inv);
              }
            }
            op[v * C::LPT + c] = o;
          }
        } else {
          const int64_t slot = ((int64_t)s * p.H + h) * p.nsplit + j;
          f32x4_t* wp = reinterpret_cast<f32x4_t*>(p.ws_acc + slot * D);
#pragma unroll
          for (int v = 0; v < C::VPL; ++v) {
#pragma unroll
            for (int q4 = 0; q4 < C::EPV / 4; ++q4) {
              const int e = v * C::EPV + q4 * 4;
              wp[(v * C::LPT + c) * (C::EPV / 4) + q4] =
                  (f32x4_t){acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]};
            }
          }
          if (c == 0) {
            p.ws_ml[slot * 2] = m[hh];
            p.ws_ml[slot * 2 + 1] = l[hh];
          }
        }
      }
    }
  }
}

// One wave per (sequence, head): combine the splits of sequences that had more than one.
template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_merge_kernel(const DecodeParams p) {
  using S = typename T::storage;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sh = (int64_t)blockIdx.x * (kDecodeThreads / kWave) + (threadIdx.x / kWave);
  if (sh >= (int64_t)p.S * p.H) return;
  const int s = (int)(sh / p.H);
  const int L = p.seq_lens[s];
  const int ns = L > 0 ? (L + p.split_len - 1) / p.split_len : 1;
  if (ns <= 1) return;
  const float* ml = p.ws_ml + sh * p.nsplit * 2;
  float M = -INFINITY;
  for (int j = lane; j < ns; j += kWave) M = fmaxf(M, ml[2 * j]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) M = fmaxf(M, shfl_xor_f(M, off));
  constexpr int DPL = (D + kWave - 1) / kWave;
  float num[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) num[i] = 0.f;
  float den = 0.f;
  const float* acc = p.ws_acc + sh * p.nsplit * D;
  for (int j = 0; j < ns; ++j) {
    const float mj = ml[2 * j];
    const float w = (mj == -INFINITY) ? 0.f : fast_exp2(mj - M);
    den += w * ml[2 * j + 1];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = lane + i * kWave;
      if (d < D) num[i] += w * acc[(int64_t)j * D + d];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  S* o = reinterpret_cast<S*>(p.out) + sh * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = lane + i * kWave;
    if (d >= D) continue;
    const float x = num[i] * inv;
    if constexpr (T::bytes == 2) {
      o[d] = (S)(pack2(T{}, x, 0.f) & 0xFFFFu);
    } else {
      o[d] = __float_as_uint(x);
    }
  }
}

int heads_per_wave(int g) {
  if (g <= 1) return 1;
  if (g == 2) return 2;
  if (g <= 4) return 4;
  return 8;
}

template <typename T, int D, int HPW>
void launch_split(const DecodeParams& dp, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D, HPW>), dim3(blocks), dim3(kDecodeThreads), 0,
                     stream, dp);
}

template <typename T, int D>
void launch_split_hpw(const DecodeParams& dp, int hpw, int blocks, hipStream_t stream) {
  switch (hpw) {
    case 1: launch_split<T, D, 1>(dp, blocks, stream); break;
    case 2: launch_split<T, D, 2>(dp, blocks, stream); break;
    case 4: launch_split<T, D, 4>(dp, blocks, stream); break;
    default: launch_split<T, D, 8>(dp, blocks, stream); break;
  }
}

template <typename T>
void launch_split_d(const DecodeParams& dp, int d, int hpw, int blocks, hipStream_t stream) {
  switch (d) {
    case 16: launch_split_hpw<T, 16>(dp, hpw, blocks, stream); break;
    case 64: launch_split_hpw<T, 64>(dp, hpw, blocks, stream); break;
    default: launch_split_hpw<T, 128>(dp, hpw, blocks, stream); break;
  }
}

template <typename T>
void launch_merge_d(const DecodeParams& dp, int d, int blocks, hipStream_t stream) {
  switch (d) {
    case 16: hipLaunchKernelGGL((decode_merge_kernel<T, 16>), dim3(blocks), dim3(kDecodeThreads), 0, stream, dp); break;
    case 64: hipLaunchKernelGGL((decode_merge_kernel<T, 64>), dim3(blocks), dim3(kDecodeThreads), 0, stream, dp); break;
    default: hipLaunchKernelGGL((decode_merge_kernel<T, 128>), dim3(blocks), dim3(kDecodeThreads), 0, stream, dp); break;
  }
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

DecodePlan decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int max_seq_len) {
  DecodePlan pl{};
  const int g = num_kv_heads > 0 ? num_heads / num_kv_heads : 1;
  pl.heads_per_wave = heads_per_wave(g);
  pl.groups_per_kv = (g + pl.heads_per_wave - 1) / pl.heads_per_wave;
  const int64_t items_per_split = (int64_t)num_seqs * num_kv_heads * pl.groups_per_kv;
  // Splits of >= 256 keys; lengthen them until the item count is at most 16384
  // (about 16 waves per CU on 256 CUs), so the per-split merge traffic stays small.
  int split = 256;
  while (split < max_seq_len &&
         items_per_split * (((int64_t)max_seq_len + split - 1) / split) > 16384)
    split *= 2;
  pl.split_len = split;
  pl.num_splits = max_seq_len > 0 ? (max_seq_len + split - 1) / split : 1;
  if (pl.num_splits < 1) pl.num_splits = 1;
  pl.workspace_bytes = 0;
  if (pl.num_splits > 1) {
    const size_t slots = (size_t)num_seqs * num_heads * pl.num_splits;
    pl.workspace_bytes = slots * (size_t)head_dim * sizeof(float) + slots * 2 * sizeof(float);
  }
  return pl;
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& pl, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  DecodeParams dp{};
  dp.out = a.out;
  dp.query = a.query;
  dp.kc = a.key_cache;
  dp.vc = a.value_cache;
  dp.block_stride = a.block_stride;
  dp.block_tables = a.block_tables;
  dp.seq_lens = a.seq_lens;
  dp.mb = a.max_blocks_per_seq;
  dp.S = a.num_seqs;
  dp.H = a.num_heads;
  dp.Hkv = a.num_kv_heads;
  dp.g = a.num_heads / a.num_kv_heads;
  dp.block_shift = log2_exact(a.block_size);
  dp.split_len = pl.split_len;
  dp.nsplit = pl.num_splits;
  dp.groups_per_kv = pl.groups_per_kv;
  dp.scale_log2 = a.scale * kLog2e;
  const size_t slots = (size_t)a.num_seqs * a.num_heads * pl.num_splits;
  dp.ws_acc = pl.num_splits > 1 ? reinterpret_cast<float*>(a.workspace) : nullptr;
  dp.ws_ml = pl.num_splits > 1 ? dp.ws_acc + slots * a.head_dim : nullptr;
  dp.total_items = (int64_t)a.num_seqs * pl.num_splits * a.num_kv_heads * pl.groups_per_kv;
  const int64_t wanted = (dp.total_items + 3) / 4;
  const int blocks = (int)(wanted < 8192 ? wanted : 8192);
  switch (a.dtype) {
    case kBF16: launch_split_d<BF16>(dp, a.head_dim, pl.heads_per_wave, blocks, stream); break;
    case kF16: launch_split_d<F16>(dp, a.head_dim, pl.heads_per_wave, blocks, stream); break;
    default: launch_split_d<F32>(dp, a.head_dim, pl.heads_per_wave, blocks, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.num_splits <= 1) return e;
  const int mblocks = (int)(((int64_t)a.num_seqs * a.num_heads + 3) / 4);
  switch (a.dtype) {
    case kBF16: launch_merge_d<BF16>(dp, a.head_dim, mblocks, stream); break;
    case kF16: launch_merge_d<F16>(dp, a.head_dim, mblocks, stream); break;
    default: launch_merge_d<F32>(dp, a.head_dim, mblocks, stream); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
