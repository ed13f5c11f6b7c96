// Single-token decode on the matrix cores: the stream- and split-mode core for bf16 /
// fp16 queries (bf16 / fp16 or FP8 caches), head_dim 64 or 128, pages of >= 8 tokens.
//
// What is computed is the same as the vector-ALU core of decode_device.h (the
// per-sequence attention of the Spyre paged-attention PR, "Description"); only the
// arithmetic is arranged for v_mfma_f32_16x16x32:
//  * scores S^T = K Q^T per tile of 16 keys: rows are keys, columns the query heads of
//    the wave (up to 8 of the 16 columns carry a head), the product runs over head_dim;
//  * outputs O = P V per step of 32 keys: rows are heads, columns 16 dims, the product
//    runs over the 32 keys.
// Measured before this core existed: the vector-ALU loop issued about 650 instructions
// per 32 keys, so even with every key in L2 the decode batch took ~61 us (bf16) and
// ~62 us (FP8); the dot products are a dense contraction and belong on MFMA.
//
// Lane l = 16a + n (a = l / 16, n = l % 16) of the wave:
//  * K tile T (T = 0, 1) of a step: row n is key 8(n/4) + 4T + (n%4).  The row's
//    16-byte units go to the four lane groups in turn (unit u to group u % 4, loaded by
//    the group's instruction u / 4), so one load instruction reads 64 contiguous bytes
//    of each of its 16 keys; product j takes 8 dims of the lane's units.  Q^T: column
//    n is head h0 + n with the same dims in the same registers, so the contraction
//    pairs equal dims whatever order the hardware gives the k slots;
//  * a 16x16 accumulator gives lane l rows 4a + i of column n, so after the two tiles
//    the lane holds the scores of keys 8a .. 8a+7 for head n: exactly the P operand
//    (row n = head, k slots = keys 8a .. 8a+7) of O = P V;
//  * V: the lane loads keys 8a .. 8a+7 at dims [n D/16, (n+1) D/16) and pairs the keys
//    per dim with byte permutes (FP8 codes are paired first, then widened), giving the
//    B operand of product i: column n = dim n D/16 + i, k slots = keys 8a .. 8a+7.
//    No LDS and no cross-lane traffic;
//  * O: lane l holds heads 4a + j (j < 4), dims n D/16 + i of product i.
// Steps start at multiples of 8 keys of the sequence (the segment start rounded down), so
// every 8-key group lies in one page.  Keys of a step outside the segment [lo, hi) get probability 0 and their V
// words are zeroed (a stale slot of a page may hold anything, NaN included); groups
// entirely past the end re-read the last group instead of following a table entry
// that may not exist.  Softmax: the same lazy running max as the vector core (move
// only when a score passes it by 2^8), kept per head and equal in the four lanes that
// hold that head's keys.
#pragma once

#include "common.h"

namespace pkv {

namespace {

constexpr int kMStep = 32;          // keys per MFMA step
constexpr int kMGroup = 8;          // keys of one lane's page group

// Steps whose loads are issued together (64 registers of K / V per lane and step for a
// bf16 / fp16 cache at head_dim 128, 32 for FP8).
template <typename T>
struct MSteps {
  static constexpr int value = KvFp8<T>::value ? 2 : 1;
};

template <typename T>
struct Mma;

template <>
struct Mma<BF16> {
  static __device__ __forceinline__ f32x4_t run(const u32x4_t& a, const u32x4_t& b,
                                                const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<F16> {
  static __device__ __forceinline__ f32x4_t run(const u32x4_t& a, const u32x4_t& b,
                                                const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

template <typename T, int D>
struct MShape {
  using B = typename BaseOf<T>::type;                  // compute type
  static constexpr bool kFp8 = KvFp8<T>::value;
  static constexpr int KQ = D / 4;                      // dims of a lane's K / Q slice
  static constexpr int U = kFp8 ? 16 : 8;               // dims of one 16-byte K unit
  static constexpr int NSC = D / 32;                    // score products per tile
  static constexpr int VD = D / 16;                     // dims of a lane's V slice
  static constexpr int KW = kFp8 ? KQ / 4 : KQ / 2;     // raw words of one key's K slice
  static constexpr int VW = kFp8 ? VD / 4 : VD / 2;     // raw words of one key's V slice
  static_assert(D == 64 || D == 128, "MFMA decode takes head_dim 64 or 128");
};

// First of the 8 dims that lane group a feeds to score product j (K and Q alike).
template <typename T, int D>
__device__ __forceinline__ int kdim(int j, int a) {
  using M = MShape<T, D>;
  constexpr int JPU = M::U / 8;                         // products per unit
  return (4 * (j / JPU) + a) * M::U + (j % JPU) * 8;
}

template <typename T, int D>
struct MStep {
  uint32_t k[2][MShape<T, D>::KW];    // K slice of tile T's row-n key
  uint32_t v[kMGroup][MShape<T, D>::VW];   // V slices of keys 8a .. 8a+7
};

// Attention state of a wave (see the layout above).
template <int D>
struct MState {
  float m;                    // running max of head n (log2 units)
  float l;                    // this lane's share of the sum of head n
  f32x4_t acc[D / 16];        // O rows 4a + j, dim n D/16 + i, in acc[i][j]
};

// N raw words at byte address b (16-, 8- or 4-byte aligned as N requires).
template <int N>
__device__ __forceinline__ void load_words(uint32_t* dst, const uint8_t* b) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(b) + i);
#pragma unroll
      for (int w = 0; w < 4; ++w) dst[4 * i + w] = x[w];
    }
  } else if constexpr (N == 2) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(b));
    dst[0] = x[0];
    dst[1] = x[1];
  } else {
    static_assert(N == 1, "slice width");
    dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(b));
  }
}

// Byte geometry of a wave's loads that holds for the whole segment.  A page is under
// 4 GiB (the launch checks it), so the offset inside a page is 32-bit and a page's own
// offset is one 32 x 32 -> 64-bit multiply of its id.
struct MAddr {
  const uint8_t* kc;
  const uint8_t* vc;
  uint32_t row_bytes;         // one token row (all kv heads)
  uint32_t blk_bytes;         // one page
  uint32_t k_lane;            // the lane's K slice in its row: kv head, unit a, key n % 4
  uint32_t v_lane;            // the lane's V slice in its row: kv head, dims n D/16
};

template <typename T, int D>
__device__ __forceinline__ MAddr maddr(const DecodeParams& p, int kvh, int a, int n) {
  using M = MShape<T, D>;
  constexpr uint32_t E = M::kFp8 ? 1u : 2u;         // bytes per cache element
  MAddr m;
  m.kc = reinterpret_cast<const uint8_t*>(p.kc);
  m.vc = reinterpret_cast<const uint8_t*>(p.vc);
  m.row_bytes = (uint32_t)p.Hkv * D * E;
  m.blk_bytes = (uint32_t)((uint64_t)p.block_stride * E);
  const uint32_t head = (uint32_t)kvh * D * E;
  m.k_lane = head + (uint32_t)a * 16u + (uint32_t)(n & 3) * m.row_bytes;
  m.v_lane = head + (uint32_t)n * (M::VD * E);
  return m;
}

// Loads of the step starting at key sb (a multiple of 8) of a segment ending at hi.
template <typename T, int D>
__device__ __forceinline__ void mload_step(MStep<T, D>& st, const DecodeParams& p,
                                           const TableWindow& tw, const MAddr& ma, int sb,
                                           int hi, int a, int n) {
  using M = MShape<T, D>;
  const uint32_t bmask = (1u << p.block_shift) - 1u;
  const int last_group = (hi - 1) & ~(kMGroup - 1);
  // K: group of row n; V: group a
  const int gk = min(sb + kMGroup * (n >> 2), last_group);
  const int gv = min(sb + kMGroup * a, last_group);
  const uint32_t bk = (uint32_t)__shfl(tw.ids, ((gk >> p.block_shift) - tw.chunk_base) & (kWave - 1), kWave);
  const uint32_t bv = (uint32_t)__shfl(tw.ids, ((gv >> p.block_shift) - tw.chunk_base) & (kWave - 1), kWave);
  const uint8_t* kp = ma.kc + ((uint64_t)bk * ma.blk_bytes + (((uint32_t)gk & bmask) * ma.row_bytes + ma.k_lane));
  const uint8_t* vp = ma.vc + ((uint64_t)bv * ma.blk_bytes + (((uint32_t)gv & bmask) * ma.row_bytes + ma.v_lane));
  // tile t: key 4t + n % 4 of the group; instruction i: units 4i .. 4i+3 of the row
  // (64 contiguous bytes, unit a of them for this lane)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < M::KW / 4; ++i)
      load_words<4>(st.k[t] + 4 * i, kp + (uint64_t)(4 * t) * ma.row_bytes + 64 * i);
#pragma unroll
  for (int k = 0; k < kMGroup; ++k)
    load_words<M::VW>(st.v[k], vp + (uint64_t)k * ma.row_bytes);
}

// Compute-type words 4j .. 4j+3 of a K slice (product j's A operand).
template <typename T, int D>
__device__ __forceinline__ u32x4_t k_operand(const uint32_t (&raw)[MShape<T, D>::KW], int j) {
  using M = MShape<T, D>;
  if constexpr (M::kFp8) {
    const uint32_t c0 = raw[2 * j], c1 = raw[2 * j + 1];
    return (u32x4_t){widen_fp8x2<false>(typename M::B{}, c0), widen_fp8x2<true>(typename M::B{}, c0),
                     widen_fp8x2<false>(typename M::B{}, c1), widen_fp8x2<true>(typename M::B{}, c1)};
  } else {
    return (u32x4_t){raw[4 * j], raw[4 * j + 1], raw[4 * j + 2], raw[4 * j + 3]};
  }
}

// One step: scores, softmax update, O += P V.  FULL: every key of the step lies in
// [lo, hi) (decided per step, uniformly over the wave).  scale_log2 >= 0 (a negative
// scale is taken by negating the queries), so the largest raw score is the largest
// scaled one and each exponent is one fma of the raw score.
template <typename T, int D, bool FULL>
__device__ __forceinline__ void mcompute_step(MStep<T, D>& st, const u32x4_t (&q)[MShape<T, D>::NSC],
                                              MState<D>& s, float scale_log2, int sb, int lo,
                                              int hi, int a) {
  using M = MShape<T, D>;
  using B = typename M::B;
  // scores of keys 8a + 4t + i for head n
  f32x4_t sc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sc[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < M::NSC; ++j) sc[t] = Mma<B>::run(k_operand<T, D>(st.k[t], j), q[j], sc[t]);
  }
  float x[kMGroup];                          // raw scores q . k
  bool in[kMGroup];
  const int k0 = sb + kMGroup * a;           // this lane's first key
#pragma unroll
  for (int r = 0; r < kMGroup; ++r) {
    in[r] = FULL || (k0 + r >= lo && k0 + r < hi);
    x[r] = in[r] ? sc[r >> 2][r & 3] : -INFINITY;
  }
  if constexpr (!FULL) {
    // keys outside the segment: zero V so that nothing but finite zeros reaches O
#pragma unroll
    for (int r = 0; r < kMGroup; ++r)
#pragma unroll
      for (int w = 0; w < M::VW; ++w) st.v[r][w] = in[r] ? st.v[r][w] : 0u;
  }
  float mx = x[0];
#pragma unroll
  for (int r = 1; r < kMGroup; ++r) mx = fmaxf(mx, x[r]);
  mx *= scale_log2;
  if (__builtin_expect(__any(mx > s.m + kLazyRescale), 0)) {
    float mt = fmaxf(mx, shfl_xor_f(mx, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float mn = fmaxf(s.m, mt);
    const float alpha = (s.m == -INFINITY) ? 0.f : fast_exp2(s.m - mn);
    s.l *= alpha;
    // O rows are heads 4a + j: their factor sits in lane 4a + j (column 4a + j)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float f = __shfl(alpha, 4 * a + j, kWave);
#pragma unroll
      for (int i = 0; i < M::VD; ++i) s.acc[i][j] *= f;
    }
    s.m = mn;
  }
  // (at an edge the running max may still be -inf: masked keys get 0 explicitly)
  float pr[kMGroup];
  const float nm = -s.m;
#pragma unroll
  for (int r = 0; r < kMGroup; ++r) {
    const float e = fast_exp2(__builtin_fmaf(x[r], scale_log2, nm));
    pr[r] = FULL ? e : (in[r] ? e : 0.f);
  }
  u32x4_t pp;
#pragma unroll
  for (int w = 0; w < 4; ++w) pp[w] = pack2(B{}, pr[2 * w], pr[2 * w + 1]);
  // row sum of the rounded probabilities (the values the product consumes)
  const uint32_t ones = pack2(B{}, 1.f, 1.f);
#pragma unroll
  for (int w = 0; w < 4; ++w) s.l = dot2(B{}, pp[w], ones, s.l);
  // B operands: for each dim of the slice, keys (0,1) (2,3) (4,5) (6,7) of the group
#pragma unroll
  for (int i = 0; i < M::VD; ++i) {
    u32x4_t vb;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int k0r = 2 * w, k1r = 2 * w + 1;
      if constexpr (M::kFp8) {
        // code word i/4 holds dims 4(i/4) .. +3; pair the two keys' bytes, then widen
        const uint32_t c0 = st.v[k0r][i >> 2], c1 = st.v[k1r][i >> 2];
        const uint32_t pr = (i & 2) ? __builtin_amdgcn_perm(c1, c0, 0x07030602u)
                                    : __builtin_amdgcn_perm(c1, c0, 0x05010400u);
        vb[w] = (i & 1) ? widen_fp8x2<true>(B{}, pr) : widen_fp8x2<false>(B{}, pr);
      } else {
        // word i/2 holds dims 2(i/2), 2(i/2)+1; take the same half of both keys
        const uint32_t e0 = st.v[k0r][i >> 1], e1 = st.v[k1r][i >> 1];
        vb[w] = (i & 1) ? __builtin_amdgcn_perm(e1, e0, 0x07060302u)
                        : __builtin_amdgcn_perm(e1, e0, 0x05040100u);
      }
    }
    s.acc[i] = Mma<B>::run(pp, vb, s.acc[i]);
  }
}

// State of one wave over keys [lo, hi) of sequence s for heads h0 .. h0+nh-1 (nh <= 8)
// of kv head kvh.  On return s.l is the head's full sum in every lane of column n.
// ROLL: a rolling double buffer of NSTEP steps each (the loads of batch k + 2 go out as soon
// as batch k is computed), for the stream grid, whose single wave per SIMD has no other
// wave to hide its arithmetic behind; otherwise batches of NSTEP steps loaded together.
template <typename T, int D, int NSTEP, bool ROLL = false>
__device__ __forceinline__ void attend_segment_mfma(const DecodeParams& p, int s, int kvh, int h0,
                                                    int nh, int lo, int hi, int lane,
                                                    MState<D>& st) {
  using M = MShape<T, D>;
  using S = typename T::storage;
  const int a = lane >> 4, n = lane & 15;
  // the bounds are the same in every lane: scalar registers, scalar branches
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  // a negative scale: negated queries (exact) give negated raw scores, and the scale's
  // magnitude then applies
  const float sl2 = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4_t q[M::NSC];
  {
    // columns past the group's heads get zeros (finite scores, never written)
    const S* qrow = reinterpret_cast<const S*>(p.query) + ((int64_t)s * p.H + h0 + (n < nh ? n : 0)) * D;
#pragma unroll
    for (int j = 0; j < M::NSC; ++j) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + kdim<T, D>(j, a));
#pragma unroll
      for (int w = 0; w < 4; ++w) q[j][w] = n < nh ? (v[w] ^ qsign) : 0u;
    }
  }
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < M::VD; ++i) st.acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  if (lo < hi) {
    const int32_t* table = p.block_tables + (int64_t)s * p.mb;
    const MAddr ma = maddr<T, D>(p, kvh, a, n);
    const int last_page = (hi - 1) >> p.block_shift;
    const int start = lo & ~(kMGroup - 1);
    TableWindow tw;
    table_window_load(tw, table, start >> p.block_shift, last_page, lane);
    auto compute = [&](MStep<T, D>& b, int sb) {
      if (sb >= lo && sb + kMStep <= hi)
        mcompute_step<T, D, true>(b, q, st, sl2, sb, lo, hi, a);
      else
        mcompute_step<T, D, false>(b, q, st, sl2, sb, lo, hi, a);
    };
    if constexpr (ROLL) {
      // batches past the end re-read the last group (no branch around a load) and are
      // never computed
      constexpr int BATCH = NSTEP * kMStep;
      const int last_group = (hi - 1) & ~(kMGroup - 1);
      auto load = [&](MStep<T, D> (&b)[NSTEP], int base) {
        const int need = (min(base + BATCH, hi) - 1) >> p.block_shift;
        if (need >= tw.chunk_base + kWave) {
          table_window_load(tw, table, min(base, last_group) >> p.block_shift, last_page, lane);
          // wait for the new page ids here, on this rare path: a wait after the branch
          // would be one for every load in flight (the counter is in order) on every batch,
          // and the other buffer's loads would never overlap this batch's
          asm volatile("" ::"v"(tw.ids));
        }
#pragma unroll
        for (int k = 0; k < NSTEP; ++k)
          mload_step<T, D>(b[k], p, tw, ma, base + k * kMStep, hi, a, n);
      };
      auto compute_batch = [&](MStep<T, D> (&b)[NSTEP], int base) {
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
          const int sb = base + k * kMStep;
          if (sb >= hi) break;
          compute(b[k], sb);
        }
      };
      MStep<T, D> b0[NSTEP], b1[NSTEP];
      load(b0, start);
      load(b1, start + BATCH);
      for (int base = start;; base += 2 * BATCH) {
        compute_batch(b0, base);
        if (base + BATCH >= hi) break;
        load(b0, base + 2 * BATCH);
        compute_batch(b1, base + BATCH);
        if (base + 2 * BATCH >= hi) break;
        load(b1, base + 3 * BATCH);
      }
    } else {
      for (int base = start; base < hi; base += NSTEP * kMStep) {
        const int it_last = (min(base + NSTEP * kMStep, hi) - 1) >> p.block_shift;
        if (it_last >= tw.chunk_base + kWave)
          table_window_load(tw, table, base >> p.block_shift, last_page, lane);
        MStep<T, D> ms[NSTEP];
#pragma unroll
        for (int k = 0; k < NSTEP; ++k)
          mload_step<T, D>(ms[k], p, tw, ma, base + k * kMStep, hi, a, n);
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
          const int sb = base + k * kMStep;
          if (sb >= hi) break;
          compute(ms[k], sb);
        }
      }
    }
  }
  st.l += shfl_xor_f(st.l, 16);
  st.l += shfl_xor_f(st.l, 32);
}

// Final rows of heads h0 .. h0+nh-1: lane (a, n) writes dims n D/16 .. of heads 4a + j.
template <typename T, int D>
__device__ __forceinline__ void write_output_mfma(const DecodeParams& p, int s, int h0, int nh,
                                                  int lane, const MState<D>& st) {
  using M = MShape<T, D>;
  using S = typename T::storage;
  using B = typename M::B;
  const int a = lane >> 4, n = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * a + j;
    const float lh = __shfl(st.l, hh & 15, kWave);
    if (hh >= nh) continue;
    const float inv = lh > 0.f ? p.out_scale / lh : 0.f;
    uint32_t w[M::VD / 2];
#pragma unroll
    for (int i = 0; i < M::VD / 2; ++i)
      w[i] = pack2(B{}, st.acc[2 * i][j] * inv, st.acc[2 * i + 1][j] * inv);
    S* o = reinterpret_cast<S*>(p.out) + ((int64_t)s * p.H + h0 + hh) * D + n * M::VD;
    if constexpr (M::VD == 8) {
      *reinterpret_cast<u32x4_t*>(o) = (u32x4_t){w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<u32x2_t*>(o) = (u32x2_t){w[0], w[1]};
    }
  }
}

// Partial state of heads h0 .. into workspace slot `slot` of each head (same layout as
// the vector core's partials, so the merge kernels are shared).
template <typename T, int D>
__device__ __forceinline__ void write_partial_mfma(const DecodeParams& p, int64_t slots_per_head,
                                                   int64_t slot, int h0, int nh, int lane,
                                                   const MState<D>& st) {
  using M = MShape<T, D>;
  const int a = lane >> 4, n = lane & 15;
  const float o = p.out_scale;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * a + j;
    if (hh >= nh) continue;
    const int64_t idx = (int64_t)(h0 + hh) * slots_per_head + slot;
    f32x4_t* wp = reinterpret_cast<f32x4_t*>(p.ws_acc + idx * D + n * M::VD);
#pragma unroll
    for (int i4 = 0; i4 < M::VD / 4; ++i4)
      wp[i4] = (f32x4_t){st.acc[4 * i4][j] * o, st.acc[4 * i4 + 1][j] * o,
                         st.acc[4 * i4 + 2][j] * o, st.acc[4 * i4 + 3][j] * o};
  }
  if (a == 0 && n < nh) {
    const int64_t idx = (int64_t)(h0 + n) * slots_per_head + slot;
    p.ws_ml[idx * 2] = st.m;
    p.ws_ml[idx * 2 + 1] = st.l;
  }
}

}  // namespace

}  // namespace pkv
