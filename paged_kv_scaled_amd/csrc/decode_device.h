// Single-token decode over a paged KV cache: flash decoding + log-sum-exp merge.
//
// What is computed (Spyre paged-attention PR, "Description": gather from scattered
// blocks, GQA by repeat_interleave, per-sequence attention): for each sequence s and
// query head h, out = softmax(scale * q K^T) V over the L_s cached keys of kv head
// h / (H / Hkv).  The ROCm TransformerEngine small-seq PR's s_q = 1, s_kv <= 16 varlen
// cross attention is the same call with one sequence per query token.
//
// How (MI355X design, HBM-bound; this is the vector-ALU core, and decode_mfma.h holds the
// matrix-core core that stream and split mode use where the arithmetic per key weighs):
//  * a wave handles one group of HPW query heads sharing a kv head over a contiguous
//    segment of one sequence's keys;
//  * lanes = (token t of a round, column c): a round covers TPR tokens, each token's
//    D-element row of one kv head is read by LPT lanes with 16-byte loads, so one wave
//    load instruction reads TPR contiguous row segments.  The block-table gather is the
//    address computation of those loads (no gathered copy exists); the segment's block
//    ids sit in one register per lane and are fetched with a lane shuffle;
//  * q . k with packed dot2 (v_dot2_f32_bf16 / _f16) and a DPP reduction over the LPT
//    lanes of a token; every lane keeps a private online-softmax state (m, l, acc) over
//    the tokens it sees; the max only moves when a score exceeds it by more than 2^8
//    (probabilities stay <= 256, exact after the final division);
//  * probabilities of two rounds are paired and multiplied into V with dot2 as well;
//  * at the end of a segment the lanes of a column merge their states (shuffles).
//
// Work decomposition (picked on the host from the sizes):
//  * stream mode (some sequence longer than one split): the concatenated key axis of
//    all sequences is cut into `nranges` equal ranges per head group, one wave each,
//    so every wave does the same work whatever the length mix.  On that axis every
//    sequence after the first is preceded by kStreamSeqCost positions that hold no key: a
//    wave pays about that much for each sequence it starts (page ids, the first loads,
//    the partial it leaves), so a range that crosses more sequence boundaries holds
//    fewer keys.  A
//    sequence that lies inside one range is finished by that wave; a range boundary
//    inside a sequence leaves (acc, m, l) partials that the merge kernel combines.  Up to kStreamScanSeqs
//    sequences each wave finds its range's first sequence by scanning the lengths;
//    beyond, a one-block planning kernel writes the length prefix sums and every range's
//    first sequence into the workspace, and the waves read them;
//  * split mode (every sequence within one split): fixed splits of split_len keys per
//    sequence, waves
//    walk (sequence, split, head group) items in a grid-stride loop; sequences with one
//    split are written directly.
// The merge combines one (sequence, head)'s partials by their log-sum-exp weights: one wave
// per (sequence, head), or one workgroup per (sequence, head) when a stream-mode batch has
// so few sequences that each spans dozens of ranges.
#pragma once

#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kDecodeThreads = 256;
constexpr int kWavesPerBlock = kDecodeThreads / kWave;
constexpr float kLazyRescale = 8.0f;   // log2 units
constexpr int kStreamScanSeqs = 256;   // plain decode: up to here every stream wave scans
                                       // seq_lens, beyond the planning kernel's tables
constexpr int kStreamWavesPerCu = 4;       // waves of the stream grid (all head groups): one
                                           // wave per SIMD (1024 on a whole MI355X)
constexpr int kStreamMinRange = 64;    // shortest range, keys
// Positions charged on the stream key axis for each sequence a range starts (measured:
// a segment costs a wave ~1.2-1.8 us besides its keys, 30-45 keys of an FP8 decode and
// 20-25 of a bf16 one; waves crossing three sequences ended ~4.5 us after those with one).
constexpr int kStreamSeqCost = 32;

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
  static constexpr int STEP = 2 * TPR;             // keys per step (two rounds)
  static_assert(NV >= 1 && NV % LPT == 0, "head_dim / dtype combination");
  // 16-byte vector (of the query / output row) that lane column c holds as its v-th:
  // interleaved over the columns, or, with an FP8 cache, the lane's own contiguous
  // EPL elements (the elements its one FP8 load covers).
  static __device__ __forceinline__ int vec(int v, int c) {
    return KvFp8<T>::value ? c * VPL + v : v * LPT + c;
  }
};

// 32-bit words of one K (or V) row that a lane holds in flight: the elements themselves,
// or for an FP8 cache the raw codes (half as many words; widened when used).
template <typename T, int D>
constexpr int raw_words() {
  return KvFp8<T>::value ? DecodeShape<T, D>::WPL / 2 : DecodeShape<T, D>::WPL;
}

// Steps whose loads are issued together: keep the K/V registers of one batch of steps
// at about 64 per lane (2 rounds x 2 tensors x raw words per step).
template <typename T, int D, int HPW>
struct DecodeSteps {
  static constexpr int words = 4 * raw_words<T, D>();
  static constexpr int value =
      KvFp8<T>::value ? (HPW >= 8 ? 1 : 2)
                      : ((HPW >= 8 || words > 32) ? 1 : (words > 16 || HPW >= 4 ? 2 : 4));
};

struct DecodeParams {
  void* out;
  const void* query;
  const void* kc;
  const void* vc;
  int64_t block_stride;     // elements
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;            // [H, slots_per_head, D]
  float* ws_ml;             // [H, slots_per_head, 2]  (max in log2 units, sum)
  int64_t total_items;      // split mode: S*nsplit*HG; stream mode: HG*nranges
  int32_t mb, S, H, Hkv, g, block_shift, split_len, nsplit, groups_per_kv, nranges;
  float scale_log2;         // scale * log2(e) (times k_scale for an FP8 cache)
  float out_scale;          // v_scale for an FP8 cache, else 1
  const uint32_t* guard;    // device error word when device checks are on, else null
  void* weights;            // small-seq training forward: [S, H, max_kv] attention weights
  int32_t max_kv;
  // prefix stream mode (workspace, after the partials): cu[s] = keys of sequences < s
  // (cu[S] = total), and for range r its first sequence rstart[r] starting at rpos[r]
  int64_t* cu;
  int64_t* rpos;
  int32_t* rstart;
};

template <typename T, int D>
struct Step {
  static constexpr int RW = raw_words<T, D>();
  uint32_t k[2][RW];
  uint32_t v[2][RW];
  bool valid[2];
};

// Word w (a pair of compute-type elements) of a lane's row held as `raw`.
template <typename T, int RW>
__device__ __forceinline__ uint32_t row_word(const uint32_t (&raw)[RW], int w) {
  if constexpr (KvFp8<T>::value) {
    return (w & 1) ? widen_fp8x2<true>(T{}, raw[w >> 1]) : widen_fp8x2<false>(T{}, raw[w >> 1]);
  } else {
    return raw[w];
  }
}

// Block ids of 64 consecutive pages, one per lane (lane i: page chunk_base + i).
struct TableWindow {
  int32_t ids;
  int chunk_base;
};

__device__ __forceinline__ void table_window_load(TableWindow& tw, const int32_t* __restrict__ table,
                                                  int first_page, int last_page, int lane) {
  tw.chunk_base = first_page;
  tw.ids = table[min(first_page + lane, last_page)];
}

// Round r of a step: this lane's part of the K and V rows at element offset `row`.
template <typename T, int D>
__device__ __forceinline__ void load_row(Step<T, D>& st, int r, const DecodeParams& p, int64_t row,
                                         int c) {
  using C = DecodeShape<T, D>;
  if constexpr (KvFp8<T>::value) {
    // EPL codes per lane, one load each for K and V (widened when used)
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(p.kc) + row + c * C::EPL;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(p.vc) + row + c * C::EPL;
    constexpr int NW = C::EPL / 4;                  // code words per lane
    uint32_t kw[NW], vw[NW];
    if constexpr (NW == 4) {
      const u32x4_t kk = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb));
      const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kw[i] = kk[i];
        vw[i] = vv[i];
      }
    } else {
      static_assert(NW == 2, "FP8 rows of 8 or 16 codes per lane");
      const u32x2_t kk = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(kb));
      const u32x2_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vb));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        kw[i] = kk[i];
        vw[i] = vv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      st.k[r][i] = kw[i];
      st.v[r][i] = vw[i];
    }
  } else {
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const typename T::storage*>(p.kc) + row);
    const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const typename T::storage*>(p.vc) + row);
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const u32x4_t kk = __builtin_nontemporal_load(kp + v * C::LPT + c);
      const u32x4_t vv = __builtin_nontemporal_load(vp + v * C::LPT + c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        st.k[r][v * 4 + w] = kk[w];
        st.v[r][v * 4 + w] = vv[w];
      }
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_step(Step<T, D>& st, const DecodeParams& p,
                                          const TableWindow& tw, int64_t head_off, int base,
                                          int end, int t, int c) {
  using C = DecodeShape<T, D>;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  const int bmask = (1 << p.block_shift) - 1;
  // Loads are branch-free: a lane past the end of the segment re-reads its last key
  // (finite data) and gets probability 0.  Divergent branches around the loads would
  // make the compiler wait for every load in flight.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int pos_raw = base + r * C::TPR + t;
    st.valid[r] = pos_raw < end;
    const int pos = min(pos_raw, end - 1);
    const int idx = ((pos >> p.block_shift) - tw.chunk_base) & (kWave - 1);
    const int64_t blk = __shfl(tw.ids, idx, kWave);
    const int64_t row = blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + head_off;
    load_row<T, D>(st, r, p, row, c);
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

// Scores of the two keys of a step for every head, in log2 units (-inf past the end).
template <typename T, int D, int HPW>
__device__ __forceinline__ void score_step(const Step<T, D>& st,
                                           const uint32_t (&q)[HPW][DecodeShape<T, D>::WPL],
                                           float scale_log2, float (&sc)[2][HPW]) {
  using C = DecodeShape<T, D>;
  constexpr bool kHalf = T::bytes == 2;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < C::WPL; ++w) {
        if constexpr (kHalf) {
          d = dot2(T{}, q[hh][w], row_word<T>(st.k[r], w), d);
        } else {
          d = __builtin_fmaf(__uint_as_float(q[hh][w]), __uint_as_float(st.k[r][w]), d);
        }
      }
      d = reduce_token<C::LPT>(d);
      sc[r][hh] = st.valid[r] ? d * scale_log2 : -INFINITY;
    }
  }
}

// Online-softmax update of (m, l, acc) with a step's scores and V rows.
template <typename T, int D, int HPW>
__device__ __forceinline__ void update_step(const Step<T, D>& st, const float (&sc)[2][HPW],
                                            float (&m)[HPW], float (&l)[HPW],
                                            float (&acc)[HPW][DecodeShape<T, D>::EPL]) {
  using C = DecodeShape<T, D>;
  constexpr bool kHalf = T::bytes == 2;
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
  if constexpr (KvFp8<T>::value) {
    // pair the two rounds on the codes (one byte permute per two pairs), then widen:
    // raw word i holds elements 4i..4i+3 of a row
#pragma unroll
    for (int i = 0; i < Step<T, D>::RW; ++i) {
      const uint32_t r0 = st.v[0][i], r1 = st.v[1][i];
      const uint32_t p01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0.b0 r1.b0 r0.b1 r1.b1
      const uint32_t p23 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);   // r0.b2 r1.b2 r0.b3 r1.b3
      const uint32_t xy[4] = {widen_fp8x2<false>(T{}, p01), widen_fp8x2<true>(T{}, p01),
                              widen_fp8x2<false>(T{}, p23), widen_fp8x2<true>(T{}, p23)};
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const uint32_t pp = pack2(T{}, pr[0][hh], pr[1][hh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[hh][4 * i + e] = dot2(T{}, pp, xy[e], acc[hh][4 * i + e]);
      }
    }
  } else if constexpr (kHalf) {
    // pair the two rounds: x = (v0.lo, v1.lo), y = (v0.hi, v1.hi) for every word
#pragma unroll
    for (int w = 0; w < C::WPL; ++w) {
      const uint32_t a = row_word<T>(st.v[0], w), b = row_word<T>(st.v[1], w);
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
__device__ __forceinline__ void compute_step(const Step<T, D>& st,
                                             const uint32_t (&q)[HPW][DecodeShape<T, D>::WPL],
                                             float (&m)[HPW], float (&l)[HPW],
                                             float (&acc)[HPW][DecodeShape<T, D>::EPL],
                                             float scale_log2) {
  float sc[2][HPW];
  score_step<T, D, HPW>(st, q, scale_log2, sc);
  update_step<T, D, HPW>(st, sc, m, l, acc);
}

// Attention state of one wave over keys [lo, hi) of sequence s for the query heads
// h0 .. h0+nh-1 of kv head kvh.  On return every lane of column c holds the merged
// (m, l, acc) for the dimensions of that column (acc relative to m, unnormalised).
template <typename T, int D, int HPW, int NSTEP>
__device__ __forceinline__ void attend_segment(const DecodeParams& p, int s, int kvh, int h0,
                                               int nh, int lo, int hi, int lane, float (&m)[HPW],
                                               float (&l)[HPW],
                                               float (&acc)[HPW][DecodeShape<T, D>::EPL]) {
  using C = DecodeShape<T, D>;
  using S = typename T::storage;
  const int t = lane / C::LPT, c = lane % C::LPT;
  uint32_t q[HPW][C::WPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    // heads past the group re-read the group's first head and are never written
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const S*>(p.query) + ((int64_t)s * p.H + h0 + (hh < nh ? hh : 0)) * D);
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const u32x4_t qq = qp[C::vec(v, c)];
#pragma unroll
      for (int w = 0; w < 4; ++w) q[hh][v * 4 + w] = qq[w];
    }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) acc[hh][e] = 0.f;
  }
  if (lo < hi) {
    const int32_t* table = p.block_tables + (int64_t)s * p.mb;
    const int64_t head_off = (int64_t)kvh * D;
    const int last_page = (hi - 1) >> p.block_shift;
    TableWindow tw;
    table_window_load(tw, table, lo >> p.block_shift, last_page, lane);
    // Each iteration issues the loads of NSTEP steps before computing any of them;
    // no register buffer is carried across iterations.
    for (int base = lo; base < hi; base += NSTEP * C::STEP) {
      const int it_last = (min(base + NSTEP * C::STEP, hi) - 1) >> p.block_shift;
      if (it_last >= tw.chunk_base + kWave)
        table_window_load(tw, table, base >> p.block_shift, last_page, lane);
      Step<T, D> st[NSTEP];
#pragma unroll
      for (int k = 0; k < NSTEP; ++k)
        load_step<T, D>(st[k], p, tw, head_off, base + k * C::STEP, hi, t, c);
#pragma unroll
      for (int k = 0; k < NSTEP; ++k) compute_step<T, D, HPW>(st[k], q, m, l, acc, p.scale_log2);
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
}

// Final output rows of heads h0.. (lanes of round-token 0 write, one 16-byte vector each).
template <typename T, int D, int HPW>
__device__ __forceinline__ void write_output(const DecodeParams& p, int s, int h0, int nh, int c,
                                             const float (&l)[HPW],
                                             const float (&acc)[HPW][DecodeShape<T, D>::EPL]) {
  using C = DecodeShape<T, D>;
  using S = typename T::storage;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (hh >= nh) continue;
    const float inv = l[hh] > 0.f ? p.out_scale / l[hh] : 0.f;
    u32x4_t* op = reinterpret_cast<u32x4_t*>(reinterpret_cast<S*>(p.out) +
                                             ((int64_t)s * p.H + h0 + hh) * D);
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
      op[C::vec(v, c)] = o;
    }
  }
}

// Partial state of heads h0.. into workspace slot `slot` of each head.
template <typename T, int D, int HPW>
__device__ __forceinline__ void write_partial(const DecodeParams& p, int64_t slots_per_head,
                                              int64_t slot, int h0, int nh, int c,
                                              const float (&m)[HPW], const float (&l)[HPW],
                                              const float (&acc)[HPW][DecodeShape<T, D>::EPL]) {
  using C = DecodeShape<T, D>;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (hh >= nh) continue;
    const int64_t idx = (int64_t)(h0 + hh) * slots_per_head + slot;
    f32x4_t* wp = reinterpret_cast<f32x4_t*>(p.ws_acc + idx * D);
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
#pragma unroll
      for (int q4 = 0; q4 < C::EPV / 4; ++q4) {
        const int e = v * C::EPV + q4 * 4;
        const float o = p.out_scale;
        wp[C::vec(v, c) * (C::EPV / 4) + q4] =
            (f32x4_t){acc[hh][e] * o, acc[hh][e + 1] * o, acc[hh][e + 2] * o, acc[hh][e + 3] * o};
      }
    }
    if (c == 0) {
      p.ws_ml[idx * 2] = m[hh];
      p.ws_ml[idx * 2 + 1] = l[hh];
    }
  }
}

}  // namespace

}  // namespace pkv

#include "decode_mfma.h"

namespace pkv {

namespace {

// ---- split mode ------------------------------------------------------------------------

// One (sequence, split, head group) item of split mode, walked by the calling wave (MF:
// on the matrix-core core of decode_mfma.h).
template <typename T, int D, int HPW, int NSTEP, bool MF = false>
__device__ __forceinline__ void split_item(const DecodeParams& p, int64_t item) {
  using C = DecodeShape<T, D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int HG = p.Hkv * p.groups_per_kv;
  const int hg = (int)(item % HG);
  const int64_t sj = item / HG;
  const int j = (int)(sj % p.nsplit);
  const int s = (int)(sj / p.nsplit);
  const int L = p.seq_lens[s];
  const int start = j * p.split_len;
  if (j > 0 && start >= L) return;
  const int end = min(L, start + p.split_len);
  const int ns = L > 0 ? (L + p.split_len - 1) / p.split_len : 1;
  const int kvh = hg / p.groups_per_kv, sub = hg % p.groups_per_kv;
  const int h0 = kvh * p.g + sub * HPW;
  const int nh = min(HPW, p.g - sub * HPW);
  if constexpr (MF) {
    MState<D> ms;
    attend_segment_mfma<T, D, NSTEP>(p, s, kvh, h0, nh, start, end, lane, ms);
    if (ns == 1)
      write_output_mfma<T, D>(p, s, h0, nh, lane, ms);
    else
      write_partial_mfma<T, D>(p, (int64_t)p.S * p.nsplit, (int64_t)s * p.nsplit + j, h0, nh,
                               lane, ms);
    return;
  } else {
    float m[HPW], l[HPW], acc[HPW][C::EPL];
    attend_segment<T, D, HPW, NSTEP>(p, s, kvh, h0, nh, start, end, lane, m, l, acc);
    if (t == 0) {
      if (ns == 1)
        write_output<T, D, HPW>(p, s, h0, nh, c, l, acc);
      else
        write_partial<T, D, HPW>(p, (int64_t)p.S * p.nsplit, (int64_t)s * p.nsplit + j, h0, nh,
                                 c, m, l, acc);
    }
  }
}

// Waves wave, wave + nwaves, ... walk the items.
template <typename T, int D, int HPW, int NSTEP, bool MF = false>
__device__ __forceinline__ void split_items(const DecodeParams& p, int64_t wave, int64_t nwaves) {
  for (int64_t item = wave; item < p.total_items; item += nwaves)
    split_item<T, D, HPW, NSTEP, MF>(p, item);
}

template <typename T, int D, int HPW, int NSTEP, bool MF = false>
__global__ void __launch_bounds__(kDecodeThreads)
decode_split_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  split_items<T, D, HPW, NSTEP, MF>(p, (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave),
                                    (int64_t)gridDim.x * kWavesPerBlock);
}

// ---- item mode -------------------------------------------------------------------------
// Short sequences (each one split and at most kItemPages pages): every group of LPT = 8
// lanes owns one item (sequence, head group) and walks its keys two per step, so the 8
// items of a wave run side by side.  Their dependent loads (length, page ids, K/V)
// overlap, and no cross-lane merge is needed at the end.
constexpr int kItemPages = 8;   // page ids of an item: one per lane of its group
constexpr int kItemSteps = 2;   // steps whose loads are issued together

template <typename T, int D>
__device__ __forceinline__ void load_item_step(Step<T, D>& st, const DecodeParams& p, int32_t pid,
                                               int64_t head_off, int base, int L, int t, int c) {
  using C = DecodeShape<T, D>;
  const int64_t row_elems = (int64_t)p.Hkv * D;
  const int bmask = (1 << p.block_shift) - 1;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int pos_raw = base + r;
    st.valid[r] = pos_raw < L;
    const int pos = min(pos_raw, max(L - 1, 0));          // branch-free: re-read a real key
    const int64_t blk = __shfl(pid, t * C::LPT + (pos >> p.block_shift), kWave);
    const int64_t row = blk * p.block_stride + (int64_t)(pos & bmask) * row_elems + head_off;
    load_row<T, D>(st, r, p, row, c);
  }
}

template <typename T, int D, int HPW, int NSTEP>
__global__ void __launch_bounds__(kDecodeThreads)
decode_items_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  using C = DecodeShape<T, D>;
  using S = typename T::storage;
  static_assert(C::LPT == 8 && C::TPR == 8, "item mode needs 8 lanes per row");
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  if (wave * C::TPR >= p.total_items) return;            // uniform over the wave
  const int64_t item_raw = wave * C::TPR + t;
  const bool live = item_raw < p.total_items;
  const int64_t item = live ? item_raw : p.total_items - 1;
  const int HG = p.Hkv * p.groups_per_kv;
  const int hg = (int)(item % HG);
  const int s = (int)(item / HG);
  const int L = p.seq_lens[s];
  const int kvh = hg / p.groups_per_kv, sub = hg % p.groups_per_kv;
  const int h0 = kvh * p.g + sub * HPW;
  const int nh = min(HPW, p.g - sub * HPW);
  // lane c of the group holds page c of the item; block 0 stands in past the last page
  const int last_page = L > 0 ? (L - 1) >> p.block_shift : -1;
  const int32_t pid = c <= last_page ? p.block_tables[(int64_t)s * p.mb + c] : 0;
  uint32_t q[HPW][C::WPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const S*>(p.query) + ((int64_t)s * p.H + h0 + (hh < nh ? hh : 0)) * D);
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const u32x4_t qq = qp[C::vec(v, c)];
#pragma unroll
      for (int w = 0; w < 4; ++w) q[hh][v * 4 + w] = qq[w];
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
  // the longest item of the wave bounds the steps (uniform loop)
  int Lw = live ? L : 0;
#pragma unroll
  for (int off = C::LPT; off < kWave; off <<= 1) Lw = max(Lw, __shfl_xor(Lw, off, kWave));
  const int64_t head_off = (int64_t)kvh * D;
  for (int base = 0; base < Lw; base += 2 * NSTEP) {
    Step<T, D> st[NSTEP];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) load_item_step<T, D>(st[k], p, pid, head_off, base + 2 * k, L, t, c);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) compute_step<T, D, HPW>(st[k], q, m, l, acc, p.scale_log2);
  }
  if (live) write_output<T, D, HPW>(p, s, h0, nh, c, l, acc);
}

// Item mode that also writes the attention weights (the small-seq training forward, at
// most kWeightKeys keys): the scores of the item's keys stay in registers (log2 units),
// and once the final max and sum are known every lane of the group writes the weights of
// keys c and c + 8, P = 2^(z - m) / l, zero past the length.
constexpr int kWeightKeys = 16;

template <typename T, int D, int HPW>
__global__ void __launch_bounds__(kDecodeThreads)
decode_items_weights_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  using C = DecodeShape<T, D>;
  using S = typename T::storage;
  static_assert(C::LPT == 8 && C::TPR == 8, "item mode needs 8 lanes per row");
  constexpr int NSTEP = 2;
  constexpr int ITER = kWeightKeys / (2 * NSTEP);
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  if (wave * C::TPR >= p.total_items) return;            // uniform over the wave
  const int64_t item_raw = wave * C::TPR + t;
  const bool live = item_raw < p.total_items;
  const int64_t item = live ? item_raw : p.total_items - 1;
  const int HG = p.Hkv * p.groups_per_kv;
  const int hg = (int)(item % HG);
  const int s = (int)(item / HG);
  const int L = min(p.seq_lens[s], p.max_kv);
  const int kvh = hg / p.groups_per_kv, sub = hg % p.groups_per_kv;
  const int h0 = kvh * p.g + sub * HPW;
  const int nh = min(HPW, p.g - sub * HPW);
  const int last_page = L > 0 ? (L - 1) >> p.block_shift : -1;
  const int32_t pid = c <= last_page ? p.block_tables[(int64_t)s * p.mb + c] : 0;
  uint32_t q[HPW][C::WPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const S*>(p.query) + ((int64_t)s * p.H + h0 + (hh < nh ? hh : 0)) * D);
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const u32x4_t qq = qp[C::vec(v, c)];
#pragma unroll
      for (int w = 0; w < 4; ++w) q[hh][v * 4 + w] = qq[w];
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
  int Lw = L;
#pragma unroll
  for (int off = C::LPT; off < kWave; off <<= 1) Lw = max(Lw, __shfl_xor(Lw, off, kWave));
  const int64_t head_off = (int64_t)kvh * D;
  float z[ITER * NSTEP][2][HPW];                           // key 2*i + r at z[i][r]
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
#pragma unroll
    for (int k = 0; k < NSTEP; ++k)
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) z[it * NSTEP + k][r][hh] = -INFINITY;
    const int base = it * 2 * NSTEP;
    if (base < Lw) {                                       // uniform over the wave
      Step<T, D> st[NSTEP];
#pragma unroll
      for (int k = 0; k < NSTEP; ++k) load_item_step<T, D>(st[k], p, pid, head_off, base + 2 * k, L, t, c);
#pragma unroll
      for (int k = 0; k < NSTEP; ++k) {
        score_step<T, D, HPW>(st[k], q, p.scale_log2, z[it * NSTEP + k]);
        update_step<T, D, HPW>(st[k], z[it * NSTEP + k], m, l, acc);
      }
    }
  }
  if (!live) return;
  write_output<T, D, HPW>(p, s, h0, nh, c, l, acc);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (hh >= nh) continue;
    S* wrow = reinterpret_cast<S*>(p.weights) + ((int64_t)s * p.H + h0 + hh) * p.max_kv;
    const float inv = L > 0 ? 1.f / l[hh] : 0.f;
    const float mh = L > 0 ? m[hh] : 0.f;
#pragma unroll
    for (int key = 0; key < kWeightKeys; ++key) {
      if ((key & (C::LPT - 1)) != c || key >= p.max_kv) continue;
      const float zk = z[key >> 1][key & 1][hh];
      const float pk = key < L ? fast_exp2(zk - mh) * inv : 0.f;
      wrow[key] = (S)(pack2(T{}, pk, 0.f) & 0xFFFFu);
    }
  }
}

// ---- stream mode -----------------------------------------------------------------------

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

// Length of the stream key axis (every key, plus kStreamSeqCost before each sequence but
// the first), from which every stream kernel derives the range length.  len0: this lane's
// entry of the first 64 lengths (0 past the batch), loaded once.
__device__ __forceinline__ int64_t stream_total(const DecodeParams& p, int lane, int len0) {
  int64_t total = (int64_t)(p.S - 1) * kStreamSeqCost;
  for (int c0 = 0; c0 < p.S; c0 += kWave) {
    int x = c0 == 0 ? len0 : ((c0 + lane < p.S) ? p.seq_lens[c0 + lane] : 0);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    total += x;
  }
  return total;
}

__device__ __forceinline__ int64_t stream_range_len(int64_t total, int nranges) {
  const int64_t r = (total + nranges - 1) / nranges;
  return r < kStreamMinRange ? kStreamMinRange : r;
}

// First sequence whose span (its charge, then its keys) reaches past position x of the
// stream key axis, and the position of that sequence's first key.
__device__ __forceinline__ void stream_locate(const DecodeParams& p, int64_t x, int lane, int len0,
                                              int& s0, int64_t& start0) {
  int count = 0;
  int64_t carry = 0, before = 0;
  for (int c0 = 0; c0 < p.S; c0 += kWave) {
    const bool in = c0 + lane < p.S;
    const int Ls = (c0 == 0 ? len0 : (in ? p.seq_lens[c0 + lane] : 0)) + (in ? kStreamSeqCost : 0);
    // incl: first key of the next sequence; this one's span ends kStreamSeqCost before
    const int64_t incl = carry + wave_inclusive_scan(Ls, lane);
    const bool done = in && incl - kStreamSeqCost <= x;   // sequence ends at or before x
    count += __popcll(__ballot(done));
    int64_t b = done ? incl : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t o = __shfl_xor(b, off, kWave);
      b = o > b ? o : b;
    }
    before = b > before ? b : before;
    carry = __shfl(incl, kWave - 1, kWave);
  }
  s0 = count;
  start0 = before;
}

// One stream-mode item (head group, key range), walked by the calling wave (MF: on the
// matrix-core core of decode_mfma.h).
// PFX: the batch has more sequences than a wave scans; the planning kernel's prefix sums
// and range starts in the workspace take the place of the scans.
template <typename T, int D, int HPW, int NSTEP, bool MF = false, bool PFX = false>
__device__ __forceinline__ void stream_item(const DecodeParams& p, int64_t item) {
  using C = DecodeShape<T, D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane / C::LPT, c = lane % C::LPT;
  const int HG = p.Hkv * p.groups_per_kv;
  const int hg = (int)(item % HG);
  const int r = (int)(item / HG);
  int len0 = 0;
  int64_t total;
  if constexpr (PFX) {
    total = p.cu[p.S] + (int64_t)(p.S - 1) * kStreamSeqCost;
  } else {
    len0 = lane < p.S ? p.seq_lens[lane] : 0;
    total = stream_total(p, lane, len0);
  }
  const int64_t R = stream_range_len(total, p.nranges);
  const int64_t lo = (int64_t)r * R;
  const int64_t hi = min(total, lo + R);
  if (lo >= hi) return;
  const int kvh = hg / p.groups_per_kv, sub = hg % p.groups_per_kv;
  const int h0 = kvh * p.g + sub * HPW;
  const int nh = min(HPW, p.g - sub * HPW);
  int s;
  int64_t P;
  if constexpr (PFX) {
    s = p.rstart[r];
    P = p.rpos[r];
  } else {
    stream_locate(p, lo, lane, len0, s, P);
  }
  // P: position of sequence s's first key.  A range leaves at most two partials: slot 0
  // for a sequence begun before the range, slot 1 for one that runs past its end.
  for (; s < p.S && P < hi; ++s) {
    const int L = p.seq_lens[s];
    const int seg_lo = (int)((lo > P ? lo : P) - P);
    const int seg_hi = (int)((hi < P + L ? hi : P + L) - P);
    if (seg_hi > seg_lo) {
      const int64_t slot = (int64_t)r * 2 + (seg_lo > 0 ? 0 : 1);
      if constexpr (MF) {
        MState<D> ms;
        // one wave per SIMD: a rolling buffer where a load batch would be one step
        attend_segment_mfma<T, D, NSTEP, NSTEP == 1>(p, s, kvh, h0, nh, seg_lo, seg_hi, lane,
                                                      ms);
        if (seg_lo == 0 && seg_hi == L)
          write_output_mfma<T, D>(p, s, h0, nh, lane, ms);
        else
          write_partial_mfma<T, D>(p, (int64_t)p.nranges * 2, slot, h0, nh, lane, ms);
      } else {
        float m[HPW], l[HPW], acc[HPW][C::EPL];
        attend_segment<T, D, HPW, NSTEP>(p, s, kvh, h0, nh, seg_lo, seg_hi, lane, m, l, acc);
        if (t == 0) {
          if (seg_lo == 0 && seg_hi == L)
            write_output<T, D, HPW>(p, s, h0, nh, c, l, acc);
          else
            write_partial<T, D, HPW>(p, (int64_t)p.nranges * 2, slot, h0, nh, c, m, l, acc);
        }
      }
    }
    P += L + kStreamSeqCost;
  }
}

template <typename T, int D, int HPW, int NSTEP, bool MF = false, bool PFX = false>
__global__ void __launch_bounds__(kDecodeThreads)
decode_stream_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  if (wave >= p.total_items) return;
  stream_item<T, D, HPW, NSTEP, MF, PFX>(p, wave);
}

// Prefix stream mode, one block before the stream kernel: cu = exclusive prefix sums of
// the lengths (cu[S] = total), then for every range r the first sequence whose keys reach
// past its start r * R (empty sequences before it skipped) and where that sequence starts.
constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
decode_stream_plan_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  constexpr int NW = kPlanThreads / kWave;
  __shared__ int64_t s_wave[NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int64_t carry = 0;
  for (int c0 = 0; c0 < p.S; c0 += kPlanThreads) {
    const int i = c0 + tid;
    int64_t v = i < p.S ? (int64_t)p.seq_lens[i] : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t y = __shfl_up(v, off, kWave);
      if (lane >= off) v += y;
    }
    if (lane == kWave - 1) s_wave[w] = v;
    __syncthreads();
    int64_t before = 0, chunk = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int64_t x = s_wave[k];
      before += k < w ? x : 0;
      chunk += x;
    }
    if (i < p.S) p.cu[i + 1] = carry + before + v;
    carry += chunk;
    __syncthreads();                 // s_wave is rewritten by the next chunk
  }
  if (tid == 0) p.cu[0] = 0;
  __threadfence_block();
  __syncthreads();                   // cu complete and visible to the block
  // the stream key axis: sequence s's keys start at cu[s] + s kStreamSeqCost
  const int64_t R = stream_range_len(carry + (int64_t)(p.S - 1) * kStreamSeqCost, p.nranges);
  for (int r = tid; r < p.nranges; r += kPlanThreads) {
    const int64_t x = (int64_t)r * R;
    // smallest s whose span ends past x (S when the range is empty)
    int a = 0, b = p.S;
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (p.cu[mid + 1] + (int64_t)mid * kStreamSeqCost > x) b = mid; else a = mid + 1;
    }
    p.rstart[r] = a;
    p.rpos[r] = p.cu[min(a, p.S)] + (int64_t)a * kStreamSeqCost;   // its first key
  }
}

// ---- merge -----------------------------------------------------------------------------

template <typename T, int D>
__device__ __forceinline__ void store_row(const DecodeParams& p, int64_t sh, int lane,
                                          const float* num, float inv) {
  using S = typename T::storage;
  constexpr int DPL = (D + kWave - 1) / kWave;
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

// Combine partials (acc, m, l) of one head with the log-sum-exp rule: slot0 for partial
// 0, slot1 + (j - 1) * slot_step for partial j > 0.  The partials are taken in batches of
// MB whose (m, l) pairs and accumulator rows are all loaded before any is used; the
// running max moves between batches with a rescale of the sums.  Batches of 8 hold the
// usual two or three partials of a head in one round of loads; batches of 32 serve the
// workgroup merge of a stream-mode batch of few sequences, where one sequence spans
// dozens of ranges.
constexpr int kMergeBatch = 8;
constexpr int kMergeBatchWide = 32;

// One wave's running merge state: max M, sum den (this lane's share until summed over
// the wave) and this lane's dims d = lane + i * 64 of the numerator.
template <int D>
struct MergeState {
  static constexpr int DPL = (D + kWave - 1) / kWave;
  float M = -INFINITY, den = 0.f, num[DPL];
  __device__ MergeState() {
#pragma unroll
    for (int i = 0; i < DPL; ++i) num[i] = 0.f;
  }
  __device__ void sum_den() {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) den += shfl_xor_f(den, off);
  }
};

// Fold partials j_begin <= j < j_end into st.
template <int D, int MB>
__device__ __forceinline__ void merge_run(const DecodeParams& p, int h, int64_t slots_per_head,
                                          int j_begin, int j_end, int lane, int64_t slot0,
                                          int64_t slot1, int64_t slot_step, MergeState<D>& st) {
  constexpr int DPL = MergeState<D>::DPL;
  auto slot_of = [&](int j) -> int64_t {
    return (int64_t)h * slots_per_head + (j == 0 ? slot0 : slot1 + (int64_t)(j - 1) * slot_step);
  };
  for (int j0 = j_begin; j0 < j_end; j0 += MB) {
    const int cnt = min(MB, j_end - j0);
    // lane k < cnt: (m, l) of partial j0 + k; every lane: its dims of each row (rows past
    // cnt re-read the last one and get weight 0)
    const int64_t my = slot_of(j0 + min(lane, cnt - 1));
    float mj = p.ws_ml[my * 2], lj = p.ws_ml[my * 2 + 1];
    float acc[MB][DPL];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const float* row = p.ws_acc + slot_of(j0 + min(k, cnt - 1)) * D;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + i * kWave;
        acc[k][i] = d < D ? row[d] : 0.f;
      }
    }
    if (lane >= cnt) mj = -INFINITY;
    float bm = mj;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) bm = fmaxf(bm, shfl_xor_f(bm, off));
    const float Mn = fmaxf(st.M, bm);
    const float alpha = (st.M == -INFINITY) ? 0.f : fast_exp2(st.M - Mn);
    const float w = (mj == -INFINITY) ? 0.f : fast_exp2(mj - Mn);
    st.den = st.den * alpha + w * lj;
#pragma unroll
    for (int i = 0; i < DPL; ++i) st.num[i] *= alpha;
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const float wk = __shfl(w, k, kWave);
#pragma unroll
      for (int i = 0; i < DPL; ++i) st.num[i] += wk * acc[k][i];
    }
    st.M = Mn;
  }
}

// Merge the n partials of one head in one wave and write its output row.
template <typename T, int D>
__device__ __forceinline__ void merge_slots(const DecodeParams& p, int64_t sh, int h,
                                            int64_t slots_per_head, int n, int lane,
                                            int64_t slot0, int64_t slot1, int64_t slot_step) {
  MergeState<D> st;
  merge_run<D, kMergeBatch>(p, h, slots_per_head, 0, n, lane, slot0, slot1, slot_step, st);
  st.sum_den();
  store_row<T, D>(p, sh, lane, st.num, st.den > 0.f ? 1.f / st.den : 0.f);
}

template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_merge_split_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sh = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  if (sh >= (int64_t)p.S * p.H) return;
  const int s = (int)(sh / p.H), h = (int)(sh % p.H);
  const int L = p.seq_lens[s];
  const int ns = L > 0 ? (L + p.split_len - 1) / p.split_len : 1;
  if (ns <= 1) return;
  const int64_t base = (int64_t)s * p.nsplit;
  merge_slots<T, D>(p, sh, h, (int64_t)p.S * p.nsplit, ns, lane, base, base + 1, 1);
}

// Where sequence s sits on the stream key axis: its length L, the position P of its first
// key and the axis length, all from one round of loads: the planning kernel's prefix sums,
// or one pass of the wave over the lengths (L taken from the pass itself).
struct SeqPos {
  int64_t total = 0, P = 0;
  int L = 0;
};

template <bool PFX>
__device__ __forceinline__ SeqPos stream_seq_pos(const DecodeParams& p, int s, int lane) {
  SeqPos q;
  if constexpr (PFX) {
    q.L = p.seq_lens[s];
    q.total = p.cu[p.S];
    q.P = p.cu[s];
  } else {
    for (int c0 = 0; c0 < p.S; c0 += kWave) {
      const int x = (c0 + lane < p.S) ? p.seq_lens[c0 + lane] : 0;
      if (c0 == (s & ~(kWave - 1))) q.L = __shfl(x, s & (kWave - 1), kWave);
      int before = (c0 + lane < s) ? x : 0;
      int all = x;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        all += __shfl_xor(all, off, kWave);
        before += __shfl_xor(before, off, kWave);
      }
      q.total += all;
      q.P += before;
    }
  }
  q.total += (int64_t)(p.S - 1) * kStreamSeqCost;
  q.P += (int64_t)s * kStreamSeqCost;
  return q;
}

template <typename T, int D>
__device__ __forceinline__ void store_zero_row(const DecodeParams& p, int64_t sh, int lane) {
  float zero[MergeState<D>::DPL];
#pragma unroll
  for (int i = 0; i < MergeState<D>::DPL; ++i) zero[i] = 0.f;
  store_row<T, D>(p, sh, lane, zero, 0.f);
}

// Stream mode: one wave per (sequence, head).  Sequences inside one range were written
// by the stream kernel; empty sequences get zeros; the others combine one partial per
// range they touch: the second slot of the range holding their first key, the first slot
// of every later one.
template <typename T, int D, bool PFX = false>
__global__ void __launch_bounds__(kDecodeThreads)
decode_merge_stream_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sh = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  if (sh >= (int64_t)p.S * p.H) return;
  const int s = (int)(sh / p.H), h = (int)(sh % p.H);
  const SeqPos q = stream_seq_pos<PFX>(p, s, lane);
  if (q.L == 0) {
    store_zero_row<T, D>(p, sh, lane);
    return;
  }
  const int64_t R = stream_range_len(q.total, p.nranges);
  const int64_t r0 = q.P / R, r1 = (q.P + q.L - 1) / R;
  if (r0 == r1) return;
  const int64_t slot0 = r0 * 2 + 1;
  merge_slots<T, D>(p, sh, h, (int64_t)p.nranges * 2, (int)(r1 - r0 + 1), lane, slot0,
                    (r0 + 1) * 2, 2);
}

// Stream mode over a few long sequences (each spanning dozens of ranges; no planning
// tables): one workgroup per (sequence, head).  Its waves fold equal runs of the
// partials, 32 per round of loads, and wave 0 combines the waves' states through LDS.
// Every early return depends on (sequence, head) alone, so the whole workgroup takes it
// before the barrier.
template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_merge_stream_wide_kernel(const DecodeParams p) {
  if (guard_tripped(p.guard)) return;
  constexpr int DPL = MergeState<D>::DPL;
  __shared__ float s_m[kWavesPerBlock], s_den[kWavesPerBlock], s_num[kWavesPerBlock][D];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t sh = blockIdx.x;
  const int s = (int)(sh / p.H), h = (int)(sh % p.H);
  const SeqPos q = stream_seq_pos<false>(p, s, lane);
  if (q.L == 0) {
    if (wave == 0) store_zero_row<T, D>(p, sh, lane);
    return;
  }
  const int64_t R = stream_range_len(q.total, p.nranges);
  const int64_t r0 = q.P / R, r1 = (q.P + q.L - 1) / R;
  if (r0 == r1) return;
  const int64_t slot0 = r0 * 2 + 1;
  const int n = (int)(r1 - r0 + 1);
  const int per = (n + kWavesPerBlock - 1) / kWavesPerBlock;
  const int jb = min(n, wave * per), je = min(n, jb + per);
  MergeState<D> st;
  merge_run<D, kMergeBatchWide>(p, h, (int64_t)p.nranges * 2, jb, je, lane, slot0, (r0 + 1) * 2,
                                2, st);
  st.sum_den();
  if (lane == 0) {
    s_m[wave] = st.M;
    s_den[wave] = st.den;
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = lane + i * kWave;
    if (d < D) s_num[wave][d] = st.num[i];
  }
  __syncthreads();
  if (wave != 0) return;
  float Mg = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) Mg = fmaxf(Mg, s_m[w]);
  float den = 0.f, num[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) num[i] = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    const float a = (s_m[w] == -INFINITY) ? 0.f : fast_exp2(s_m[w] - Mg);
    den += a * s_den[w];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = lane + i * kWave;
      if (d < D) num[i] += a * s_num[w][d];
    }
  }
  store_row<T, D>(p, sh, lane, num, den > 0.f ? 1.f / den : 0.f);
}

// ---- host: kernel parameters from the call's arguments and plan --------------------------

inline DecodeParams decode_params(const AttnArgs& a, const DecodePlan& pl) {
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
  dp.nranges = pl.num_ranges;
  dp.scale_log2 = a.scale * (a.kv_fp8 ? a.k_scale : 1.f) * kLog2e;
  dp.out_scale = a.kv_fp8 ? a.v_scale : 1.f;
  dp.guard = a.guard;
  const size_t slots = pl.workspace_bytes / ((size_t)(a.head_dim + 2) * sizeof(float));
  // partial slots (the prefix mode's tables follow them in the workspace)
  const size_t nslots = pl.prefix ? (size_t)a.num_heads * pl.num_ranges * 2 : slots;
  dp.ws_acc = pl.workspace_bytes ? reinterpret_cast<float*>(a.workspace) : nullptr;
  dp.ws_ml = pl.workspace_bytes ? dp.ws_acc + nslots * a.head_dim : nullptr;
  if (pl.prefix) {
    // after the partials (a multiple of 8 bytes: the slot count is even)
    uint8_t* base = reinterpret_cast<uint8_t*>(dp.ws_ml + nslots * 2);
    dp.cu = reinterpret_cast<int64_t*>(base);
    dp.rpos = dp.cu + (a.num_seqs + 1);
    dp.rstart = reinterpret_cast<int32_t*>(dp.rpos + pl.num_ranges);
  }
  const int64_t groups = (int64_t)a.num_kv_heads * pl.groups_per_kv;
  dp.total_items = pl.stream ? groups * pl.num_ranges : (int64_t)a.num_seqs * pl.num_splits * groups;
  return dp;
}

}  // namespace

}  // namespace pkv
