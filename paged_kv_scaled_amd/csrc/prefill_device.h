// Prefill / chunked-prefill attention on bf16 / fp16 MFMA (gfx950, v_mfma_f32_32x32x16).
//
// What is computed (Spyre paged-attention PR, "Description" steps 2-6 on a flat query
// batch; bottom-right causal and the block-causal "(q >= kv) or same block" mask of the
// vllm-omni piecewise block-causal PR): out[t, h] = softmax(scale * q K^T) V over the
// visible keys of the sequence owning row t, kv head h / (H / Hkv).
//
// How:
//  * a workgroup (8 waves, two per SIMD) owns one sequence, one kv head, a group of HW
//    query heads of that kv head and 32*RB consecutive query rows, with HW * RB = 8
//    column blocks of (one head, 32 rows), one per wave.  Two waves per SIMD let the
//    hardware overlap one wave's MFMA with the other's softmax and LDS traffic;
//  * keys are visited in tiles of 64.  K and V rows are gathered through the block table
//    (page ids staged in LDS) with 16-byte loads into registers one tile ahead, then
//    written to LDS: K row-major, V transposed (dims x tokens); both XOR-swizzled so the
//    MFMA operand reads hit distinct banks;
//  * S^T = K Q^T on MFMA (A = K rows from LDS, B = Q rows held in registers): each lane
//    then holds 32 scores of one query row, so the row max needs one cross-lane step;
//  * online softmax in fp32 registers (exp2 with scale*log2(e) folded).  The probabilities
//    are taken against the running max as it stands, and the tile's row max is computed
//    (and O rescaled) only when a row's probabilities of the tile sum past 2^13, which
//    is rare after the first tile;
//  * the probabilities stay where the S^T accumulator put them and are used directly as
//    the B operand of O^T = V^T P^T: the V^T tile stores each 16-token group in the
//    token order that accumulator layout implies;
//  * every wave computes every key tile of its workgroup (tiles past a row's visible end
//    get probability 0); fully visible tiles skip the mask;
//  * an FP8 (E4M3) cache is read as codes, widened exactly to bf16 / fp16 on the way to
//    LDS; k_scale is folded into the score scale and v_scale into the final 1/l.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWaves = 8;          // waves per workgroup: 2 per SIMD
constexpr int kBN = 64;            // keys per tile
constexpr int kTableChunk = 1024;  // page ids staged in LDS at a time
// bound on the sum of one lane's 32 probabilities of a key tile before the running max
// moves (log2 13: every probability stays <= 2^13)
constexpr float kSumCap = 8192.0f;
static_assert(kTableChunk % (kWaves * 64) == 0, "page-id staging: whole loads per thread");

struct PrefillParams {
  void* out;
  const void* query;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const void* kc;
  const void* vc;
  int64_t block_stride;
  const int32_t* block_tables;
  const int32_t* full_spans;                  // SPANS mask only
  const int32_t* cu_spans;
  int32_t mb, S, H, Hkv, g, block_shift, mask, span;
  int32_t hw, rb_log2, head_groups, qtiles;   // WG tiling
  int32_t ngroups;                            // (sequence, kv head, head group) groups
  int32_t nxcd;                               // XCDs of the device (workgroup dealing)
  int32_t rank_items;                         // order each XCD's query tiles longest first
  int32_t rank_bits;                          // bits of (key tiles per query tile + 2)
  float scale_log2;                           // scale * log2(e) (times k_scale for FP8)
  float out_scale;                            // v_scale for an FP8 cache, else 1
  const uint32_t* guard;                      // device error word when checks are on
};

template <typename T> struct Mfma;
template <> struct Mfma<BF16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// (1, 1) in the storage type, for row sums by dot2
template <typename T> __device__ __forceinline__ uint32_t kOnes2();
template <> __device__ __forceinline__ uint32_t kOnes2<BF16>() { return 0x3F803F80u; }
template <> __device__ __forceinline__ uint32_t kOnes2<F16>() { return 0x3C003C00u; }


// LDS layouts.  K: [kBN tokens][D] with 16-byte chunk kc of row r at kc ^ (r & (NC-1)).
// V^T: [D dims][kBN tokens], chunk (8 tokens) kc of row r at kc ^ vswz(r).
template <int D>
struct Lds {
  static constexpr int NC = D / 8;                 // 16-byte chunks per K row
  static constexpr int KBYTES = kBN * D * 2;
  static constexpr int VROW = kBN * 2;             // bytes per V^T row
  static constexpr int VBYTES = D * VROW;
  __device__ static __forceinline__ int k_off(int row, int kc) {
    return row * (D * 2) + ((kc ^ (row & (NC - 1))) << 4);
  }
  __device__ static __forceinline__ int vswz(int row) { return ((row >> 1) ^ (row >> 4)) & 7; }
  __device__ static __forceinline__ int v_off(int row, int pos) {   // pos: token slot 0..63
    return row * VROW + (((pos >> 3) ^ vswz(row)) << 4) + ((pos & 7) << 1);
  }
};

// Position of token t (0..63) of a tile in the V^T row: inside each 16-token group the
// 4-token runs 1 and 2 trade places, the order in which the S^T accumulator holds them.
__device__ __forceinline__ int vt_pos(int t) {
  const int run = (t >> 2) & 3;
  const int swapped = (run == 1) ? 2 : (run == 2 ? 1 : run);
  return (t & ~15) | (swapped << 2) | (t & 3);
}

// One workgroup of kWaves waves (one 32-column block each); bid is its index in the
// prefill grid.
template <typename T, int D>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, int bid) {
  using TB = typename BaseOf<T>::type;          // MFMA / packing type
  constexpr bool kK8 = KvFp8<T>::value;         // the caches hold E4M3 codes
  constexpr int NT = kWaves * 64;     // threads
  constexpr int NCB = 1;              // column blocks per wave
  using L = Lds<D>;
  constexpr int NC = L::NC;
  constexpr int KS = D / 16;          // k-steps of the QK^T product
  constexpr int DB = D / 32;          // 32-dim blocks of O^T
  constexpr int TG = kBN * (D / 8) / NT;         // tokens per thread (1, 2 or 4)
  // two tile slots: tile k is stored into slot k % 2 while the waves may still compute
  // tile k - 1 from the other, so one barrier per tile suffices
  __shared__ __align__(16) uint8_t s_k2[2][L::KBYTES];
  __shared__ __align__(16) uint8_t s_v2[2][L::VBYTES];
  __shared__ int32_t s_tbl[kTableChunk];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int hl = lane >> 5;           // lane half
  const int lc = lane & 31;           // lane column

  // ---- workgroup -> (sequence, kv head, head group, query tile) ----------------------
  // Workgroups go to the XCDs round-robin (XCD = blockIdx % nxcd).  Group u = (sequence,
  // kv head, head group) is dealt to XCD u % nxcd, and all query tiles of a group stay on
  // its XCD (they read the same keys: one L2 holds them); the groups of one sequence
  // spread over all XCDs, so a long sequence does not load one XCD only.
  const int nx = p.nxcd;
  const int xcd = bid % nx;
  const int slot = bid / nx;
  int grp, qt;
  int q0 = 0, qn = 0, Ls = 0;   // the sequence's first query row, chunk length, key count
  bool have_lens = false;
  if (p.rank_items) {
    // Few workgroups per CU: the order in which an XCD starts its query tiles sets the
    // makespan (a long tile started late finishes last), so each XCD starts them longest
    // first across all its groups.  Every wave ranks the XCD's (group, query tile) items,
    // one per lane, by their key tiles, and the workgroup takes the item of rank `slot`.
    const int items = ((p.ngroups + nx - 1) / nx) * p.qtiles;   // <= 64 (host)
    int cnt = -2;                     // lanes past the items rank last
    int c0 = 0, n = 0, L = 0;
    if (lane < items) {
      cnt = -1;                       // an empty query tile ranks after every real one
      const int g = (lane / p.qtiles) * nx + xcd;
      if (g < p.ngroups) {
        const int sq = g / (p.head_groups * p.Hkv);
        c0 = p.cu_q[sq];
        n = p.cu_q[sq + 1] - c0;
        L = p.seq_lens[sq];
        const int r0 = (lane % p.qtiles) * (32 << p.rb_log2);
        if (r0 < n) {
          const int z0 = p.cu_spans ? p.cu_spans[sq] : 0, z1 = p.cu_spans ? p.cu_spans[sq + 1] : 0;
          const int last = min(r0 + (32 << p.rb_log2), n) - 1;
          cnt = (visible_end(p.mask, L - n + last, L, p.span, p.full_spans, z0, z1) + kBN - 1) / kBN;
        }
      }
    }
    // rank = lanes with a larger count, plus lanes with an equal count and a lower index
    // (a permutation of 0..63), by a most-significant-bit-first radix pass over ballots:
    // `eq` keeps the lanes whose count agrees with this lane's on the bits seen so far
    const uint32_t key = (uint32_t)(cnt + 2);
    uint64_t eq = ~0ull;
    int rank = 0;
    for (int b = p.rank_bits - 1; b >= 0; --b) {
      const bool bit = (key >> b) & 1u;
      const uint64_t ones = __ballot(bit);
      const uint64_t agree = bit ? (eq & ones) : (eq & ~ones);
      if (!bit) rank += __builtin_popcountll(eq & ones);
      eq = agree;
    }
    rank += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
    const uint64_t hit = __ballot(rank == slot);
    const int who = hit ? (int)__builtin_ctzll(hit) : 0;
    grp = (who / p.qtiles) * nx + xcd;
    qt = who % p.qtiles;
    // the lane that ranked the item already holds its sequence's lengths
    q0 = __builtin_amdgcn_readlane(c0, who);
    qn = __builtin_amdgcn_readlane(n, who);
    Ls = __builtin_amdgcn_readlane(L, who);
    have_lens = true;
  } else {
    // inside a group the longest query tiles start first
    grp = (slot / p.qtiles) * nx + xcd;
    qt = p.qtiles - 1 - slot % p.qtiles;
  }
  if (grp >= p.ngroups) return;
  int rest = grp;
  const int hgrp = rest % p.head_groups;
  rest /= p.head_groups;
  const int kvh = rest % p.Hkv;
  const int s = rest / p.Hkv;
  // ---- page ids of this sequence, loaded first: they need only the sequence index, and
  // the K / V gather waits on them.  The first window is the row's first kTableChunk
  // entries (clamped to the row); entries past the sequence's last page are never used.
  const int32_t* table = p.block_tables + (int64_t)s * p.mb;
  constexpr int kTblPer = kTableChunk / NT;
  int32_t tv[kTblPer];
#pragma unroll
  for (int k = 0; k < kTblPer; ++k) tv[k] = table[min(tid + k * NT, p.mb - 1)];
  if (!have_lens) {
    q0 = p.cu_q[s];
    qn = p.cu_q[s + 1] - q0;
    Ls = p.seq_lens[s];
  }
  const int RB = 1 << p.rb_log2;
  const int wg_rows = 32 * RB;
  const int row0 = qt * wg_rows;
  if (row0 >= qn) return;
  const int ctx = Ls - qn;
  const int sp0 = p.cu_spans ? p.cu_spans[s] : 0, sp1 = p.cu_spans ? p.cu_spans[s + 1] : 0;

  // ---- this wave's column block -------------------------------------------------------
  int head[NCB], rbase[NCB], vis[NCB];
  bool hvalid[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int cb = wv * NCB + j;
    const int hw_i = cb % p.hw;
    const int rb_i = cb / p.hw;
    const int hin = hgrp * p.hw + hw_i;          // head index inside the kv group
    hvalid[j] = hin < p.g;
    head[j] = kvh * p.g + (hvalid[j] ? hin : 0);
    rbase[j] = row0 + rb_i * 32;
    const int row = min(rbase[j] + lc, qn - 1);  // rows past the chunk repeat the last one
    vis[j] = visible_end(p.mask, ctx + row, Ls, p.span, p.full_spans, sp0, sp1);
  }
  // smallest visible end over the wave's rows: tiles below it need no mask.  Tiles that
  // no row of the wave sees are still computed: their probabilities are exactly 0
  // (every row saw key 0 in the first tile, so the running max is finite), and the
  // accumulators stay free of branch copies.
  // (the visible end never decreases with the row, so it is lane 0's: the wave's first row)
  int wmin = vis[0];
#pragma unroll
  for (int j = 1; j < NCB; ++j) wmin = min(wmin, vis[j]);
  wmin = __builtin_amdgcn_readfirstlane(wmin);
  // keys the whole workgroup needs: the last row of its tile sees the most
  const int last_row = min(row0 + wg_rows, qn) - 1;
  // (uniform over the workgroup: kept in a scalar register, so the per-tile tests against
  // it are scalar branches)
  const int kv_end = __builtin_amdgcn_readfirstlane(
      visible_end(p.mask, ctx + last_row, Ls, p.span, p.full_spans, sp0, sp1));

  const int last_page = (kv_end - 1) >> p.block_shift;
  int tbl_base = 0;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds q[row lc][dims ks*16+hl*8..+8]
  using S = typename T::storage;
  u32x4_t qf[NCB][KS];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int row = min(rbase[j] + lc, qn - 1);
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const S*>(p.query) + ((int64_t)(q0 + row) * p.H + head[j]) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[j][ks] = qp[ks * 2 + hl];
  }

  // ---- page ids staged in LDS ------------------------------------------------------
#pragma unroll
  for (int k = 0; k < kTblPer; ++k) s_tbl[tid + k * NT] = tv[k];
  __syncthreads();

  // ---- K / V tile loads into registers (clamped to the last key: finite data) -------
  // Thread (token group vg, 8-dim chunk vc) loads K and V of the TG tokens vg*TG.. for
  // dims vc*8..+8: one block-id lookup serves both tensors, 16 lanes read one 256-byte
  // row segment (128 bytes of FP8 codes), and V arrives ready for its transposed store.
  // FP8 codes stay packed in flight and are widened (exactly) on the way to LDS.
  constexpr uint32_t CE = kK8 ? 1 : 2;      // cache element bytes
  using KR = typename std::conditional<kK8, u32x2_t, u32x4_t>::type;
  const uint32_t row_bytes = (uint32_t)p.Hkv * D * CE;
  const uint32_t head_bytes = (uint32_t)kvh * D * CE;
  // bytes per cache block: below 2^32 (the host routes larger strides elsewhere), so a
  // block offset is one 32 x 32 -> 64-bit multiply
  const uint32_t blk_bytes = (uint32_t)((uint64_t)p.block_stride * CE);
  const int bmask = (1 << p.block_shift) - 1;
  const int vc_ld = tid % NC;               // 8-dim chunk
  const int vg_ld = tid / NC;               // token group of TG tokens
  KR kra[TG], vra[TG], krb[TG], vrb[TG];    // two tiles in flight
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.vc);

  // keys past kv_end (seen by no row of this workgroup) re-read key kv_end-1: finite
  // data whose page id is inside the staged window
  // PAIRS (pages of >= 2 tokens, two tokens per thread): the thread's tokens k, k + 1
  // (k even) share a page, so one page-id lookup and one block offset serve both; the
  // second is the next row, or the same clamped row at the end.
  auto load_tile = [&](int k0, KR (&kreg)[TG], KR (&vreg)[TG], auto pairs) {
    if constexpr (decltype(pairs)::value && TG == 2) {
      const int t0 = k0 + vg_ld * 2;
      const int pos = min(t0, kv_end - 1);
      const uint32_t blk = (uint32_t)s_tbl[(pos >> p.block_shift) - tbl_base];
      const uint64_t off0 = (uint64_t)blk * blk_bytes +
                            ((uint32_t)(pos & bmask) * row_bytes + head_bytes + vc_ld * 8u * CE);
      const uint64_t off1 = off0 + (t0 + 1 < kv_end ? row_bytes : 0u);
      kreg[0] = *reinterpret_cast<const KR*>(kbase + off0);
      vreg[0] = *reinterpret_cast<const KR*>(vbase + off0);
      kreg[1] = *reinterpret_cast<const KR*>(kbase + off1);
      vreg[1] = *reinterpret_cast<const KR*>(vbase + off1);
    } else {
#pragma unroll
      for (int i = 0; i < TG; ++i) {
        const int pos = min(k0 + vg_ld * TG + i, kv_end - 1);
        const uint32_t blk = (uint32_t)s_tbl[(pos >> p.block_shift) - tbl_base];
        const uint64_t off = (uint64_t)blk * blk_bytes +
                             ((uint32_t)(pos & bmask) * row_bytes + head_bytes + vc_ld * 8u * CE);
        kreg[i] = *reinterpret_cast<const KR*>(kbase + off);
        vreg[i] = *reinterpret_cast<const KR*>(vbase + off);
      }
    }
  };
  // 8 elements of the compute type from what one load brought
  auto widen8 = [&](const KR& x) -> u32x4_t {
    if constexpr (kK8) {
      return (u32x4_t){widen_fp8x2<false>(TB{}, x[0]), widen_fp8x2<true>(TB{}, x[0]),
                       widen_fp8x2<false>(TB{}, x[1]), widen_fp8x2<true>(TB{}, x[1])};
    } else {
      return x;
    }
  };
  auto store_tile = [&](const KR (&kraw)[TG], const KR (&vraw)[TG], uint8_t* s_k, uint8_t* s_v) {
    u32x4_t vreg[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      *reinterpret_cast<u32x4_t*>(s_k + L::k_off(vg_ld * TG + i, vc_ld)) = widen8(kraw[i]);
      vreg[i] = widen8(vraw[i]);
    }
    // transpose TG tokens x 8 dims into 8 dims x TG tokens
    const int pos = vt_pos(vg_ld * TG);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int w = d >> 1;
      const bool hi = d & 1;
      auto el = [&](int i) -> uint32_t { return hi ? (vreg[i][w] >> 16) : (vreg[i][w] & 0xFFFFu); };
      // the same half of two tokens' words, packed by one byte permute: low halves
      // (bytes 1:0 of each) or high halves (bytes 3:2 of each)
      auto pair = [&](int i0, int i1) -> uint32_t {
        return __builtin_amdgcn_perm(vreg[i1][w], vreg[i0][w], hi ? 0x07060302u : 0x05040100u);
      };
      const int vrow = vc_ld * 8 + d;
      if constexpr (TG == 4) {
        const uint32_t lo = pair(0, 1);
        const uint32_t hi2 = pair(2, 3);
        *reinterpret_cast<u32x2_t*>(s_v + L::v_off(vrow, pos)) = (u32x2_t){lo, hi2};
      } else if constexpr (TG == 2) {
        *reinterpret_cast<uint32_t*>(s_v + L::v_off(vrow, pos)) = pair(0, 1);
      } else {
        *reinterpret_cast<uint16_t*>(s_v + L::v_off(vrow, pos)) = (uint16_t)el(0);
      }
    }
  };

  // ---- accumulators --------------------------------------------------------------------
  f32x16_t oacc[NCB][DB];
  float m[NCB], lsum[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[j][db] = (f32x16_t){};
  }

  const float c = p.scale_log2;
  // One key tile: its K/V registers (loaded two tiles earlier) go to LDS, the registers are
  // refilled with the tile two ahead, then every wave computes on the LDS tile.  Two tiles
  // in flight cover the gather latency when the keys come from HBM rather than L2.
  auto tile_step = [&](int k0, KR (&kreg)[TG], KR (&vreg)[TG], auto pairs) {
    // Slot (k0 / kBN) % 2 last held tile k0 - 2 kBN, which every wave finished computing
    // before it reached the previous tile's barrier.
    uint8_t* s_k = s_k2[(k0 / kBN) & 1];
    uint8_t* s_v = s_v2[(k0 / kBN) & 1];
    store_tile(kreg, vreg, s_k, s_v);
    __syncthreads();
    const int k2 = k0 + 2 * kBN;
    if (k2 < kv_end) {
      // restage page ids when tile k2 leaves the staged window; the loads of the tile
      // in between already took their page ids
      if ((((min(k2 + kBN, kv_end) - 1) >> p.block_shift) - tbl_base) >= kTableChunk) {
        tbl_base = k2 >> p.block_shift;
        for (int i = tid; i < kTableChunk; i += NT)
          s_tbl[i] = table[min(tbl_base + i, last_page)];
        __syncthreads();
      }
      load_tile(k2, kreg, vreg, pairs);
    }
    {  // every wave computes every tile of the workgroup (see the note on wmin)
      // ---- S^T = K Q^T for the wave's column block ------------------------------------
      f32x16_t sacc[NCB][2];
      auto scores = [&]() {
        // K fragments read one k-step ahead of their MFMAs (two register sets)
        u32x4_t ka[2][2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          ka[0][tb] = *reinterpret_cast<const u32x4_t*>(s_k + L::k_off(tb * 32 + lc, hl));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              ka[(ks + 1) & 1][tb] =
                  *reinterpret_cast<const u32x4_t*>(s_k + L::k_off(tb * 32 + lc, (ks + 1) * 2 + hl));
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int j = 0; j < NCB; ++j)
              sacc[j][tb] = Mfma<TB>::run(ka[ks & 1][tb], qf[j][ks], ks == 0 ? (f32x16_t){} : sacc[j][tb]);
        }
        // keep the read-ahead: the scheduler would otherwise pull each read down to its MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);      // LDS reads of k-steps 0, 1
#pragma unroll
        for (int ks = 0; ks + 2 < KS; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NCB, 0);   // MFMAs of k-step ks
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // reads of k-step ks + 2
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * NCB, 0);     // the last two k-steps
        // keys a row cannot see get -inf (only tiles that cross some row's visible end)
        if (k0 + kBN > wmin) {
#pragma unroll
          for (int j = 0; j < NCB; ++j) {
            // element i of token block tb holds key k0 + tb*32 + (i/4)*8 + hl*4 + i%4;
            // compare its compile-time part against a per-lane threshold
            const int thr = vis[j] - k0 - hl * 4;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if (tb * 32 + (i >> 2) * 8 + (i & 3) >= thr) sacc[j][tb][i] = -INFINITY;
          }
        }
      };
      scores();
      // ---- online softmax (lane = one query row of each column block) ---------------
      // probabilities -> packed B fragments of O^T = V^T P^T, against the running max as
      // it stands; the lane's sum of its rounded probabilities (dot2 against ones: the
      // values the P.V product consumes) comes with them
      u32x4_t pf[NCB][4];
      float lt[NCB];
      auto probabilities = [&]() {
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
          float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float pr[8];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                pr[e] = fast_exp2(__builtin_fmaf(sacc[j][tb][h2 * 8 + e], c, -m[j]));
              const u32x4_t q4 = (u32x4_t){pack2(TB{}, pr[0], pr[1]), pack2(TB{}, pr[2], pr[3]),
                                           pack2(TB{}, pr[4], pr[5]), pack2(TB{}, pr[6], pr[7])};
              ls0 = dot2(TB{}, q4[0], kOnes2<TB>(), ls0);
              ls1 = dot2(TB{}, q4[1], kOnes2<TB>(), ls1);
              ls0 = dot2(TB{}, q4[2], kOnes2<TB>(), ls0);
              ls1 = dot2(TB{}, q4[3], kOnes2<TB>(), ls1);
              pf[j][tb * 2 + h2] = q4;
            }
          lt[j] = ls0 + ls1;
        }
      };
      // The running max moves only when the probabilities of some row of this tile sum past
      // kSumCap (so each of them stays <= kSumCap, finite in bf16 and fp32), or on the
      // workgroup's first tile, where it is still -inf (every row sees key 0, so it is
      // finite afterwards).  Only then is the tile's row max taken, O and l rescaled, and
      // the probabilities recomputed.
      bool redo = k0 == 0;
      if (!redo) {
        probabilities();
        bool over = false;
#pragma unroll
        for (int j = 0; j < NCB; ++j) over |= !(lt[j] <= kSumCap);
        redo = __any(over);
      }
      if (__builtin_expect(redo, 0)) {
        // the scores again (the K tile is still in its slot): the first ones are not kept
        // alive past the probabilities, which keeps the tile within 256 registers
        if (k0 != 0) scores();
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
          // row max on raw scores (scale > 0 on this path), scaled to log2 units
          float mx = -INFINITY;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 16; i += 2)
              mx = __builtin_fmaxf(__builtin_fmaxf(mx, sacc[j][tb][i]), sacc[j][tb][i + 1]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
          const float mn = fmaxf(m[j], mx);
          const float alpha = (m[j] == -INFINITY) ? 0.f : fast_exp2(m[j] - mn);
          lsum[j] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[j][db] *= alpha;
          m[j] = mn;
        }
        probabilities();
      }
#pragma unroll
      for (int j = 0; j < NCB; ++j) lsum[j] += lt[j];
      // ---- O^T += V^T P^T --------------------------------------------------------------
#pragma unroll
      for (int ks = 0; ks < kBN / 16; ++ks) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(s_v + L::v_off(db * 32 + lc, ks * 16 + hl * 8));
#pragma unroll
          for (int j = 0; j < NCB; ++j) oacc[j][db] = Mfma<TB>::run(a, pf[j][ks], oacc[j][db]);
        }
      }
    }
  };
  auto run = [&](auto pairs) {
    if (kv_end > 0) {
      load_tile(0, kra, vra, pairs);
      if (kBN < kv_end) load_tile(kBN, krb, vrb, pairs);
    }
    int k0 = 0;
    for (; k0 + kBN < kv_end; k0 += 2 * kBN) {
      tile_step(k0, kra, vra, pairs);
      tile_step(k0 + kBN, krb, vrb, pairs);
    }
    if (k0 < kv_end) tile_step(k0, kra, vra, pairs);
  };
  if (TG == 2 && p.block_shift >= 1)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- normalise and write O (lane: one row, 4 runs of 4 dims per 32-dim block) -------
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const float lt = lsum[j] + __shfl_xor(lsum[j], 32, 64);
    const int row = rbase[j] + lc;
    if (!hvalid[j] || row >= qn) continue;
    const float inv = lt > 0.f ? p.out_scale / lt : 0.f;
    S* op = reinterpret_cast<S*>(p.out) + ((int64_t)(q0 + row) * p.H + head[j]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + hl * 4;
        const f32x16_t& o = oacc[j][db];
        *reinterpret_cast<u32x2_t*>(op + d0) =
            (u32x2_t){pack2(TB{}, o[g4 * 4 + 0] * inv, o[g4 * 4 + 1] * inv),
                      pack2(TB{}, o[g4 * 4 + 2] * inv, o[g4 * 4 + 3] * inv)};
      }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(kWaves * 64)
prefill_mfma_kernel(const PrefillParams p) {
  if (guard_tripped(p.guard)) return;
  prefill_tile<T, D>(p, blockIdx.x);
}

// ---- host: kernel parameters and grid size from the call's arguments ------------------
// The grid is nb workgroups: 8 XCDs x groups per XCD x query tiles.  False when it does
// not fit the grid limit.
inline bool prefill_params(const AttnArgs& a, PrefillParams& p, int64_t& nb) {
  p.out = a.out;
  p.query = a.query;
  p.cu_q = a.cu_seqlens_q;
  p.seq_lens = a.seq_lens;
  p.kc = a.key_cache;
  p.vc = a.value_cache;
  p.block_stride = a.block_stride;
  p.block_tables = a.block_tables;
  p.mb = a.max_blocks_per_seq;
  p.S = a.num_seqs;
  p.H = a.num_heads;
  p.Hkv = a.num_kv_heads;
  p.g = a.num_heads / a.num_kv_heads;
  p.block_shift = log2_exact(a.block_size);
  p.mask = a.mask;
  p.span = a.span_len;
  p.full_spans = a.full_spans;
  p.cu_spans = a.cu_spans;
  // kWaves column blocks per workgroup: HW heads of the kv group x RB row blocks
  int hw = 1;
  while (hw * 2 <= p.g && hw < kWaves) hw *= 2;
  p.hw = hw;
  p.rb_log2 = log2_exact(kWaves / hw);
  p.head_groups = (p.g + hw - 1) / hw;
  const int rows = 32 * (kWaves / hw);
  p.qtiles = (a.max_q_len + rows - 1) / rows;
  const int64_t ng = (int64_t)p.head_groups * p.Hkv * p.S;
  const int nx = device_shape().xcds;
  nb = (ng + nx - 1) / nx * nx * p.qtiles;   // XCDs x groups per XCD x tiles
  if (nb > 0x7FFFFFFF) return false;
  p.ngroups = (int)ng;
  p.nxcd = nx;
  // rank the query tiles when an XCD's items fit one wave's lanes: a grid of at most
  // 64 workgroups per XCD, where one workgroup per CU at a time leaves their order to
  // decide the makespan
  const int64_t items = (ng + nx - 1) / nx * p.qtiles;
  p.rank_items = items <= 64 ? 1 : 0;
  // a query tile's key tiles never exceed ceil(max_seq_len / kBN); the rank compares
  // count + 2 (empty and absent items rank last) over that many bits
  const int64_t max_key = ((int64_t)a.max_seq_len + kBN - 1) / kBN + 2;
  p.rank_bits = 1;
  while (((int64_t)1 << p.rank_bits) <= max_key) ++p.rank_bits;
  p.scale_log2 = a.scale * (a.kv_fp8 ? a.k_scale : 1.f) * kLog2e;
  p.out_scale = a.kv_fp8 ? a.v_scale : 1.f;
  p.guard = a.guard;
  return true;
}

}  // namespace

}  // namespace pkv
