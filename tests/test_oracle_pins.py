"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the passage or the mathematical fact it rests on.  The last block
plants plausible mistakes into the oracle (on the CPU, by monkeypatching) and checks
that at least one pin catches each of them, following the fail-before / pass-after
evidence protocol of the vllm-omni piecewise block-causal PR (review thread).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import reference as ref
from paged_kv_scaled_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_seq(rng, L, H, Hkv, D):
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    return q, k, v


def _one_seq(q, k, v, q_len, mask, span=0, scale=0.3, Hkv=None):
    """Oracle for one sequence whose last q_len tokens are the queries."""
    L = k.shape[0]
    cu = np.array([0, q_len], np.int32)
    return ref.paged_attention(q, [k], [v], cu, np.array([L], np.int32), Hkv or k.shape[1],
                               scale, mask, span)


def _sdpa(q, k, v, scale, attn_mask=None, is_causal=False, gqa=False):
    """torch CPU float64 SDPA on [n, H, D] / [L, Hkv, D] arrays (the textbook routine)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask, is_causal=is_causal,
                                       scale=scale, enable_gqa=gqa)
    return o[0].permute(1, 0, 2).numpy()


# ----------------------------------------------------------------------------------------
# exact widening of the storage bits
# ----------------------------------------------------------------------------------------

def test_widen_known_bit_patterns():
    bf = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x4049], np.uint16)
    assert list(ref.widen(bf, "bf16")) == [1.0, -2.0, 0.25, 0.0, -0.0, 3.140625]
    h = np.array([0x3C00, 0xC000, 0x3400, 0x7BFF], np.uint16)
    assert list(ref.widen(h, "f16")) == [1.0, -2.0, 0.25, 65504.0]
    f = np.array([0x3F800000, 0x40490FDB], np.uint32)
    assert ref.widen(f, "f32")[0] == 1.0
    assert ref.widen(f, "f32")[1] == float(np.float32(np.pi))


def test_generator_rounding_matches_torch():
    """The generator's RNE cast agrees with torch's own float32 -> bf16/f16 conversion."""
    x = np.random.default_rng(7).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # ties at bf16 precision
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.round_to_storage(x, "bf16"), tb)
    th = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.round_to_storage(x, "f16"), th)
    # the widened value is the torch value exactly
    assert np.array_equal(ref.widen(tb, "bf16"),
                          torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ----------------------------------------------------------------------------------------
# brute force (P12) and the textbook routine (P7)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(24))
def test_brute_force_agrees(seed):
    w = wl.random_small(seed, "f32")
    q = ref.widen(w.query, "f32")
    ks = ref.split_logical(ref.widen(w.key, "f32"), w.cu_seq_lens)
    vs = ref.split_logical(ref.widen(w.value, "f32"), w.cu_seq_lens)
    o, _ = ref.paged_attention(q, ks, vs, w.cu_seqlens_q, w.seq_lens, w.num_kv_heads, w.scale,
                               w.mask, w.span_len)
    b = ref.brute_force(q, ks, vs, w.cu_seqlens_q, w.seq_lens, w.num_kv_heads, w.scale, w.mask,
                        w.span_len)
    assert np.max(np.abs(o - b)) <= 1e-12


def test_tiny_prefill_brute_force():
    w = wl.tiny_prefill()
    o, _ = ref.workload_attention(w)
    q = ref.widen(w.query, "f32")
    ks = ref.split_logical(ref.widen(w.key, "f32"), w.cu_seq_lens)
    vs = ref.split_logical(ref.widen(w.value, "f32"), w.cu_seq_lens)
    b = ref.brute_force(q, ks, vs, w.cu_seqlens_q, w.seq_lens, 2, 0.25, wl.MASK_CAUSAL)
    assert np.max(np.abs(o - b)) <= 1e-12


@pytest.mark.parametrize("mask", [ref.MASK_NONE, ref.MASK_CAUSAL])
def test_full_prefill_equals_sdpa(mask):
    rng = np.random.default_rng(11)
    q, k, v = _rand_seq(rng, 37, 6, 2, 16)
    o, _ = _one_seq(q, k, v, 37, mask, scale=0.21)
    t = _sdpa(q, k, v, 0.21, is_causal=(mask == ref.MASK_CAUSAL), gqa=True)
    assert np.max(np.abs(o - t)) <= 1e-12


@pytest.mark.parametrize("q_len", [1, 5, 19])
def test_chunked_causal_is_bottom_right(q_len):
    """A chunk of q_len new tokens after L - q_len cached ones: torch's lower-right causal bias."""
    rng = np.random.default_rng(q_len)
    L = 23
    q, _, _ = _rand_seq(rng, q_len, 4, 4, 8)
    _, k, v = _rand_seq(rng, L, 4, 4, 8)
    o, _ = _one_seq(q, k, v, q_len, ref.MASK_CAUSAL, scale=0.4)
    t = _sdpa(q, k, v, 0.4, attn_mask=causal_lower_right(q_len, L)._materialize())
    assert np.max(np.abs(o - t)) <= 1e-12


# ----------------------------------------------------------------------------------------
# invariants from the pages
# ----------------------------------------------------------------------------------------

def test_gqa_equals_repeat_interleave():
    """Spyre PR, "Description": GQA by repeat_interleave of the KV heads to num_heads."""
    rng = np.random.default_rng(3)
    q, k, v = _rand_seq(rng, 20, 8, 2, 8)
    o, _ = _one_seq(q, k, v, 9, ref.MASK_CAUSAL)
    ke, ve = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, _ = _one_seq(q, ke, ve, 9, ref.MASK_CAUSAL)
    assert np.array_equal(o, o2)
    # torch's own expansion does the same
    te = torch.from_numpy(k).repeat_interleave(4, dim=1).numpy()
    assert np.array_equal(te, ke)


@pytest.mark.parametrize("mask,span", [(ref.MASK_CAUSAL, 0), (ref.MASK_NONE, 0),
                                       (ref.MASK_BLOCK_CAUSAL, 4)])
def test_fused_head_block_diagonal_form(mask, span):
    """Spyre PR, "Description": all heads in one 2D matmul with a block-diagonal mask."""
    rng = np.random.default_rng(5)
    L, n, H, Hkv, D = 13, 6, 4, 2, 8
    q, k, v = _rand_seq(rng, L, H, Hkv, D)
    qn = q[:n]
    o, _ = _one_seq(qn, k, v, n, mask, span, scale=0.35)
    pos = np.arange(L - n, L)
    vis = ref.visibility_matrix(pos, L, mask, span)
    f = ref.fused_head_attention(qn, k, v, vis, 0.35, Hkv)
    assert np.max(np.abs(o - f)) <= 1e-12


def test_additive_mask_constant_is_exclusion():
    """Spyre PR review thread: mask values 0.0 valid / -65504.0 masked.  In fp64 the additive
    form equals exclusion whenever a row has a visible key (reading A5)."""
    g = json.load(open(os.path.join(GOLDEN, "mask_constant.json")))
    rng = np.random.default_rng(9)
    q, k, v = _rand_seq(rng, 11, 2, 2, 8)
    vis = ref.visibility_matrix(np.arange(11), 11, ref.MASK_CAUSAL, 0)
    for h in range(2):
        z = 0.3 * q[:, h] @ k[:, h].T + np.where(vis, g["valid"], g["masked"])
        w = np.exp(z - z.max(axis=1, keepdims=True))
        oa = (w @ v[:, h]) / w.sum(axis=1, keepdims=True)
        oe, _ = ref.attend(q[:, h], k[:, h], v[:, h], vis, 0.3)
        assert np.max(np.abs(oa - oe)) <= 1e-15


def test_padding_never_changes_real_rows():
    """Spyre PR, "Description" steps 3-6: padded KV (to a 256 multiple) and padded query rows
    (to a 32 multiple) are masked and dropped; real rows are unchanged, exactly."""
    rng = np.random.default_rng(4)
    L, n, H, D = 45, 7, 2, 8
    q, k, v = _rand_seq(rng, n, H, H, D)
    k0, v0 = rng.standard_normal((L, H, D)), rng.standard_normal((L, H, D))
    o, _ = _one_seq(q, k0, v0, n, ref.MASK_CAUSAL)
    kp = np.concatenate([k0, np.full((256 - L, H, D), np.nan)])
    vp = np.concatenate([v0, np.full((256 - L, H, D), np.nan)])
    qp = np.concatenate([q, np.full((32 - n, H, D), 7.0)])
    pos = np.arange(L - n, L)
    vis = np.zeros((32, 256), bool)
    vis[:n, :L] = ref.visibility_matrix(pos, L, ref.MASK_CAUSAL, 0)
    for h in range(H):
        op, _ = ref.attend(qp[:, h], kp[:, h], vp[:, h], vis, 0.3)
        assert np.array_equal(op[:n], o[:, h])
        assert np.all(op[n:] == 0.0)


def test_single_visible_key_returns_its_value_row():
    """Causal row 0 with no cached context sees only key 0: out = V[0] exactly."""
    w = wl.tiny_prefill()
    o, lse = ref.workload_attention(w)
    v = ref.widen(w.value, "f32")
    for s in range(w.num_seqs):
        r0 = w.cu_seqlens_q[s]
        for h in range(w.num_heads):
            assert np.array_equal(o[r0, h], v[w.cu_seq_lens[s], h // 2])


def test_constant_value_rows_return_the_constant():
    rng = np.random.default_rng(12)
    q, k, _ = _rand_seq(rng, 30, 4, 2, 8)
    v = np.full((30, 2, 8), -1.375)
    for mask, span in [(ref.MASK_NONE, 0), (ref.MASK_CAUSAL, 0), (ref.MASK_BLOCK_CAUSAL, 7)]:
        o, _ = _one_seq(q[:12], k, v, 12, mask, span)
        assert np.max(np.abs(o + 1.375)) <= 1e-14


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(13)
    L, n = 17, 6
    _, k, v = _rand_seq(rng, L, 2, 2, 8)
    q = np.zeros((n, 2, 8))
    o, _ = _one_seq(q, k, v, n, ref.MASK_CAUSAL)
    for i in range(n):
        a = L - n + i
        assert np.max(np.abs(o[i] - v[:a + 1].mean(axis=0))) <= 1e-14


def test_block_causal_equals_piecewise_segments():
    """vllm-omni piecewise PR: each span is a segment; a full segment attends K[:end] without
    a mask (textbook routine per segment), and the composition equals the dense rule."""
    rng = np.random.default_rng(21)
    L, span, H, Hkv, D = 29, 8, 4, 2, 8
    q, k, v = _rand_seq(rng, L, H, Hkv, D)
    for q_len in (L, 11):        # whole sequence, and a chunk with cached context
        o, _ = _one_seq(q[:q_len], k, v, q_len, ref.MASK_BLOCK_CAUSAL, span, scale=0.3)
        ctx = L - q_len
        comp = np.zeros_like(o)
        for (s, e, kv_end, causal) in ref.piecewise_segments(ref.uniform_spans(L, span), L):
            lo, hi = max(s, ctx), e
            if lo >= hi:
                continue
            assert not causal
            qs = q[:q_len][lo - ctx:hi - ctx]
            comp[lo - ctx:hi - ctx] = _sdpa(qs, k[:kv_end], v[:kv_end], 0.3, gqa=True)
        assert np.max(np.abs(o - comp)) <= 1e-12


def test_block_causal_reductions():
    """span 1 is CAUSAL; a span covering the whole sequence is NONE."""
    rng = np.random.default_rng(22)
    q, k, v = _rand_seq(rng, 19, 2, 1, 8)
    bc1, _ = _one_seq(q[:9], k, v, 9, ref.MASK_BLOCK_CAUSAL, 1)
    ca, _ = _one_seq(q[:9], k, v, 9, ref.MASK_CAUSAL)
    assert np.array_equal(bc1, ca)
    bcl, _ = _one_seq(q[:9], k, v, 9, ref.MASK_BLOCK_CAUSAL, 19)
    no, _ = _one_seq(q[:9], k, v, 9, ref.MASK_NONE)
    assert np.array_equal(bcl, no)


def test_piecewise_golden_two_segment_shapes():
    g = json.load(open(os.path.join(GOLDEN, "piecewise_two_segment.json")))
    segs = ref.piecewise_segments([tuple(x) for x in g["spans"]], g["seq_len"])
    (cs, ce, ckv, ccausal), (fs, fe, fkv, fcausal) = segs
    assert (ce - cs, ckv, ccausal) == (g["expected_causal_segment"]["q_rows"],
                                       g["expected_causal_segment"]["kv_rows"], True)
    assert (fe - fs, fkv, fcausal) == (g["expected_full_segment"]["q_rows"],
                                       g["expected_full_segment"]["kv_rows"], False)
    # and the segment composition equals the dense "(q >= kv) or same block" rule
    rng = np.random.default_rng(1)
    H, D, L = g["num_heads"], g["head_dim"], g["seq_len"]
    q, k, v = _rand_seq(rng, L, H, H, D)
    comp = np.zeros((L, H, D))
    for (s, e, kv_end, causal) in segs:
        m = causal_lower_right(e - s, kv_end)._materialize() if causal else None
        comp[s:e] = _sdpa(q[s:e], k[:kv_end], v[:kv_end], 0.5, attn_mask=m)
    dense = np.zeros((L, H, D))
    same_block = lambda a, b: (a >= 2) and (b >= 2)          # the image block is [2, 5)
    vis = np.array([[(i >= j) or same_block(i, j) for j in range(L)] for i in range(L)])
    for h in range(H):
        dense[:, h], _ = ref.attend(q[:, h], k[:, h], v[:, h], vis, 0.5)
    assert np.max(np.abs(comp - dense)) <= 1e-12


def _cover(full, L):
    """(start, end, kind) list covering [0, L): the text runs between the full spans."""
    cover, pos = [], 0
    for (s, e) in full:
        if pos < s:
            cover.append((pos, s, "causal"))
        cover.append((s, e, "full"))
        pos = e
    if pos < L:
        cover.append((pos, L, "causal"))
    return cover


def _spans_one_seq(q, k, v, q_len, full, scale=0.3):
    L = k.shape[0]
    return ref.paged_attention(q, [k], [v], np.array([0, q_len], np.int32), np.array([L], np.int32),
                               k.shape[1], scale, ref.MASK_SPANS, spans=[full])[0]


@pytest.mark.parametrize("seed", range(4))
def test_spans_equal_piecewise_segments(seed):
    """vllm-omni piecewise PR: text runs are causal segments attending K[:end] bottom-right
    aligned, image blocks are full segments attending K[:end] without a mask, one textbook
    SDPA call per segment; their composition equals the general span rule, for the whole
    sequence and for a chunk after cached context (the PR's four-segment check against
    the dense `(q >= kv) or same_image_block` reference, on random layouts)."""
    rng = np.random.default_rng(31 + seed)
    L, H, Hkv, D = 41, 4, 2, 8
    q, k, v = _rand_seq(rng, L, H, Hkv, D)
    full = wl.span_layout(rng, L, (1, 6), (2, 9))
    for q_len in (L, 17, 1):
        ctx = L - q_len
        o = _spans_one_seq(q[ctx:], k, v, q_len, full)
        comp = np.zeros_like(o)
        for (s, e, kv_end, causal) in ref.piecewise_segments(_cover(full, L), L):
            lo, hi = max(s, ctx), e
            if lo >= hi:
                continue
            m = causal_lower_right(hi - lo, kv_end)._materialize() if causal else None
            comp[lo - ctx:hi - ctx] = _sdpa(q[lo:hi], k[:kv_end], v[:kv_end], 0.3, attn_mask=m,
                                            gqa=True)
        assert np.max(np.abs(o - comp)) <= 1e-12


def test_spans_reductions():
    """Full spans tiling [0, L) in steps of S are BLOCK_CAUSAL(S); no full span is CAUSAL;
    one full span over the whole sequence is NONE."""
    rng = np.random.default_rng(32)
    L = 23
    q, k, v = _rand_seq(rng, L, 2, 1, 8)
    for q_len in (L, 9):
        qq = q[L - q_len:]
        tiled = [(s, min(s + 5, L)) for s in range(0, L, 5)]
        assert np.array_equal(_spans_one_seq(qq, k, v, q_len, tiled),
                              _one_seq(qq, k, v, q_len, ref.MASK_BLOCK_CAUSAL, 5)[0])
        assert np.array_equal(_spans_one_seq(qq, k, v, q_len, []),
                              _one_seq(qq, k, v, q_len, ref.MASK_CAUSAL)[0])
        assert np.array_equal(_spans_one_seq(qq, k, v, q_len, [(0, L)]),
                              _one_seq(qq, k, v, q_len, ref.MASK_NONE)[0])


@pytest.mark.parametrize("seed", range(8))
def test_spans_brute_force_agrees(seed):
    rng = np.random.default_rng(400 + seed)
    S, H, Hkv, D = 2, 4, 2, 4
    lens = rng.integers(3, 16, size=S).astype(np.int32)
    qls = np.array([rng.integers(1, l + 1) for l in lens], np.int32)
    cu = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), H, D))
    ks = [rng.standard_normal((int(l), Hkv, D)) for l in lens]
    vs = [rng.standard_normal((int(l), Hkv, D)) for l in lens]
    spans = [wl.span_layout(rng, int(l), (1, 4), (1, 6)) for l in lens]
    o, _ = ref.paged_attention(q, ks, vs, cu, lens, Hkv, 0.35, ref.MASK_SPANS, spans=spans)
    b = ref.brute_force(q, ks, vs, cu, lens, Hkv, 0.35, ref.MASK_SPANS, spans=spans)
    assert np.max(np.abs(o - b)) <= 1e-12


def test_chunked_prefill_consistency_and_decode_is_last_row():
    """Prefilling in chunks gives the rows of a one-shot causal prefill; decode is its last row."""
    rng = np.random.default_rng(31)
    L = 40
    q, k, v = _rand_seq(rng, L, 4, 2, 8)
    full, _ = _one_seq(q, k, v, L, ref.MASK_CAUSAL)
    for (a, b) in [(0, 13), (13, 14), (14, 33), (33, 40)]:
        part, _ = _one_seq(q[a:b], k[:b], v[:b], b - a, ref.MASK_CAUSAL)
        assert np.max(np.abs(part - full[a:b])) <= 1e-12
    dec, _ = _one_seq(q[L - 1:], k, v, 1, ref.MASK_NONE)
    assert np.max(np.abs(dec[0] - full[L - 1])) <= 1e-12


def test_lse_merge_of_any_partition_equals_unsplit():
    rng = np.random.default_rng(41)
    L, n = 50, 5
    q, k, v = _rand_seq(rng, n, 1, 1, 8)
    k, v = rng.standard_normal((L, 1, 8)), rng.standard_normal((L, 1, 8))
    vis = ref.visibility_matrix(np.arange(L - n, L), L, ref.MASK_CAUSAL, 0)
    full, lfull = ref.attend(q[:, 0], k[:, 0], v[:, 0], vis, 0.3)
    for parts in (2, 3, 7):
        owner = rng.integers(0, parts, size=L)
        outs, lses = [], []
        for j in range(parts):
            vj = vis & (owner == j)[None, :]
            o, l = ref.attend(q[:, 0], k[:, 0], v[:, 0], vj, 0.3)
            outs.append(o)
            lses.append(l)
        mo, ml = ref.lse_merge(outs, lses)
        assert np.max(np.abs(mo - full)) <= 1e-12
        assert np.max(np.abs(ml - lfull)) <= 1e-12
    # lse is log sum exp of the visible scores (closed form)
    z = 0.3 * q[:, 0] @ k[:, 0].T
    for i in range(n):
        assert abs(lfull[i] - math.log(np.exp(z[i, vis[i]]).sum())) <= 1e-12


def test_empty_rows_give_zeros():
    """CSA2 Vanilla golden PR, "Description": an empty selection gives zeros (reading A6)."""
    rng = np.random.default_rng(2)
    q, k, v = _rand_seq(rng, 3, 2, 2, 4)
    o, l = ref.attend(q[:, 0], k[:, 0], v[:, 0], np.zeros((3, 3), bool), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    out, lse = ref.paged_attention(np.zeros((0, 2, 4)), [k[:0]], [v[:0]], np.array([0, 0]),
                                   np.array([0]), 2, 0.5, ref.MASK_NONE)
    assert out.shape == (0, 2, 4)


# ----------------------------------------------------------------------------------------
# scatter / gather (P10)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("maker", [wl.tiny_prefill, lambda: wl.random_small(3, "bf16"),
                                   lambda: wl.chunked_prefill(num_seqs=2, ctx_hi=64, q_hi=40)])
def test_scatter_gather_round_trip_bit_exact(maker):
    w = maker()
    st = wl.DTYPES[w.dtype][0]
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = np.full(shape, wl.nan_bits(w.dtype), st)
    vc = np.full(shape, wl.nan_bits(w.dtype), st)
    kc2, vc2 = ref.kv_cache_write(kc, vc, w.key, w.value, w.slots, w.block_size)
    # a second formulation of the scatter: flat fancy-index assignment
    kf = kc.reshape(-1, w.num_kv_heads, w.head_dim).copy()
    kf[w.slots] = w.key
    assert np.array_equal(kf.reshape(shape), kc2)
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        g = ref.gather_sequence(kc2, w.block_tables[s], L, w.block_size)
        assert np.array_equal(g, w.key[w.cu_seq_lens[s]:w.cu_seq_lens[s + 1]])
        g = ref.gather_sequence(vc2, w.block_tables[s], L, w.block_size)
        assert np.array_equal(g, w.value[w.cu_seq_lens[s]:w.cu_seq_lens[s + 1]])
    touched = np.zeros(w.num_blocks * w.block_size, bool)
    touched[w.slots] = True
    untouched = kc2.reshape(-1, w.num_kv_heads, w.head_dim)[~touched]
    assert np.all(untouched == wl.nan_bits(w.dtype))


def test_scatter_skips_negative_slots_and_rejects_duplicates():
    kc = np.zeros((2, 2, 1, 1), np.uint32)
    vc = np.zeros((2, 2, 1, 1), np.uint32)
    key = np.arange(1, 4, dtype=np.uint32).reshape(3, 1, 1)
    k2, _ = ref.kv_cache_write(kc, vc, key, key, np.array([3, -1, 0]), 2)
    assert k2.reshape(-1).tolist() == [3, 0, 0, 1]
    with pytest.raises(AssertionError):
        ref.kv_cache_write(kc, vc, key, key, np.array([1, 1, 0]), 2)


def test_generator_layout_is_consistent():
    w = wl.tiny_prefill()
    assert w.num_blocks == 8 and sorted(w.block_tables[:, :3].reshape(-1).tolist())[:0] == []
    used = np.concatenate([w.block_tables[0, :2], w.block_tables[1, :3]])
    assert len(set(used.tolist())) == 5 and used.max() < 8
    assert w.seq_lens.tolist() == [5, 9] and w.num_tokens == 14
    # same seed -> same arrays
    w2 = wl.tiny_prefill()
    assert np.array_equal(w.query, w2.query) and np.array_equal(w.block_tables, w2.block_tables)


# ----------------------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ----------------------------------------------------------------------------------------

def _caught(test_fn, *args):
    try:
        test_fn(*args)
    except AssertionError:
        return True
    return False


def test_planted_wrong_gqa_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(ref, "kv_head_of", lambda h, H, Hkv: h % Hkv)
    assert _caught(test_gqa_equals_repeat_interleave)
    assert _caught(test_full_prefill_equals_sdpa, ref.MASK_CAUSAL)


def test_visibility_matrix_equals_the_scalar_rules():
    """The grid form of the masks equals is_visible / span_visible entry by entry: every
    mask, random chunk offsets, spans and lengths (including spans past the sequence)."""
    rng = np.random.default_rng(77)
    for _ in range(60):
        L = int(rng.integers(1, 70))
        q = int(rng.integers(1, L + 1))
        pos = np.arange(L - q, L)
        for mask in (ref.MASK_NONE, ref.MASK_CAUSAL, ref.MASK_BLOCK_CAUSAL, ref.MASK_SPANS):
            span = int(rng.integers(1, 20))
            spans = None
            if mask == ref.MASK_SPANS:
                cuts = np.sort(rng.choice(np.arange(0, L + 10), size=4, replace=False))
                spans = [(int(cuts[0]), int(cuts[1])), (int(cuts[2]), int(cuts[3]))]
            got = ref.visibility_matrix(pos, L, mask, span, spans)
            want = np.zeros((q, L), bool)
            for i, a in enumerate(pos):
                for k in range(L):
                    want[i, k] = (ref.span_visible(k, int(a), L, spans) if mask == ref.MASK_SPANS
                                  else ref.is_visible(k, int(a), L, mask, span))
            assert np.array_equal(got, want), (L, q, mask, span, spans)


def test_planted_top_left_causal_is_caught(monkeypatch):
    orig = ref.visibility_matrix

    def top_left(positions, L, mask, span, spans=None):
        # a chunk's row index instead of its absolute position: top-left alignment
        if mask == ref.MASK_CAUSAL and L == 23:
            return orig(np.asarray(positions) - (L - 19), L, mask, span, spans)
        return orig(positions, L, mask, span, spans)
    monkeypatch.setattr(ref, "visibility_matrix", top_left)
    assert _caught(test_chunked_causal_is_bottom_right, 19)


def test_planted_block_rule_off_by_one_is_caught(monkeypatch):
    orig = ref.visibility_matrix

    def wrong(positions, L, mask, span, spans=None):
        if mask == ref.MASK_BLOCK_CAUSAL:
            a = np.asarray(positions).reshape(-1, 1)
            p = np.arange(L).reshape(1, -1)
            return (p <= a) | ((p // span) == (a // span) + 1)
        return orig(positions, L, mask, span, spans)
    monkeypatch.setattr(ref, "visibility_matrix", wrong)
    assert _caught(test_block_causal_equals_piecewise_segments)


def test_planted_span_end_off_by_one_is_caught(monkeypatch):
    orig = ref.visibility_matrix

    def inclusive_end(positions, L, mask, span, spans=None):
        # the span end taken as inclusive: one key past each image block leaks in
        if mask == ref.MASK_SPANS:
            a = np.asarray(positions).reshape(-1, 1)
            p = np.arange(L).reshape(1, -1)
            vis = p <= a
            for (b, e) in spans or []:
                vis |= ((a >= b) & (a <= e)) & ((p >= b) & (p <= e))
            return vis
        return orig(positions, L, mask, span, spans)
    monkeypatch.setattr(ref, "visibility_matrix", inclusive_end)
    assert _caught(test_spans_equal_piecewise_segments, 0)


def test_planted_missing_scale_and_unstable_softmax_are_caught(monkeypatch):
    orig = ref.attend

    def no_scale(q, k, v, vis, scale):
        return orig(q, k, v, vis, 1.0)
    monkeypatch.setattr(ref, "attend", no_scale)
    assert _caught(test_full_prefill_equals_sdpa, ref.MASK_NONE)
    monkeypatch.setattr(ref, "attend", orig)

    def transposed_v(q, k, v, vis, scale):
        o, l = orig(q, k, v, vis, scale)
        return o[:, ::-1].copy(), l
    monkeypatch.setattr(ref, "attend", transposed_v)
    assert _caught(test_full_prefill_equals_sdpa, ref.MASK_NONE)


# ----------------------------------------------------------------------------------------
# FP8 (E4M3) cache quantisation
# ----------------------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_float8():
    """Every one of the 256 codes decodes as torch's float8_e4m3fn does (the OCP format)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([ref.e4m3_value(c) for c in range(256)])
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(t[~nan], mine[~nan])
    assert ref.e4m3_value(0x7E) == 448.0 and ref.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_quantize_matches_torch_on_random_and_tie_values():
    rng = np.random.default_rng(91)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 40,
                        rng.standard_normal(2000).astype(np.float32) * 0.01])
    # every midpoint between neighbouring codes: the ties
    mags = np.array([ref.e4m3_value(c) for c in range(0x7F)])
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    mine = ref.quantize_e4m3(x, np.float32(1))
    t = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, t)


def test_e4m3_quantize_round_trip_ties_and_saturation():
    """Definition checks: each finite code's value maps back to that code; a midpoint goes
    to the even code; values past 448 saturate; the product with 1/scale is one float32
    rounding."""
    vals = np.array([ref.e4m3_value(c) for c in range(0x7F)], np.float32)
    assert np.array_equal(ref.quantize_e4m3(vals, np.float32(1)), np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(ref.quantize_e4m3(-vals[1:], np.float32(1)),
                          (np.arange(1, 0x7F) | 0x80).astype(np.uint8))
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    got = ref.quantize_e4m3(mids, np.float32(1)).astype(int)
    assert np.all(got % 2 == 0) and np.all((got == np.arange(0x7E)) | (got == np.arange(1, 0x7F)))
    assert list(ref.quantize_e4m3(np.float32([1e6, -1e6, 449.0]), np.float32(1))) == [0x7E, 0xFE, 0x7E]
    inv = np.float32(1) / np.float32(0.0173)
    x = np.float32([1.2345, -3.5, 0.01])
    assert np.array_equal(ref.quantize_e4m3(x, inv), ref.quantize_e4m3((x * inv).astype(np.float32), np.float32(1)))


def test_fp8_workload_oracle_uses_dequantised_rows():
    w = wl.with_fp8_cache(wl.random_small(5, "bf16", head_dim=8))
    k, v = ref.workload_kv(w)
    kc = ref.quantize_e4m3(ref.widen(w.key, "bf16"), np.float32(1) / np.float32(w.k_scale))
    assert np.array_equal(k, ref.dequantize_e4m3(kc, w.k_scale))
    # the quantisation error stays inside half a code step (relative 2^-4) plus the subnormal step
    kw = ref.widen(w.key, "bf16")
    assert np.all(np.abs(k - kw) <= np.abs(kw) * 2.0 ** -4 + 2.0 ** -10 * w.k_scale)


# ---- small-seq training path: attention weights and backward ---------------------------

def _smallseq_case(seed, S=3, H=4, Hkv=2, D=5, lens=(1, 3, 7)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, H, D))
    keys = [rng.standard_normal((L, Hkv, D)) for L in lens]
    values = [rng.standard_normal((L, Hkv, D)) for L in lens]
    d_out = rng.standard_normal((S, H, D))
    return q, keys, values, d_out


def _loss(q, keys, values, d_out, Hkv, scale):
    out, _ = ref.smallseq_forward(q, keys, values, Hkv, scale)
    return float(np.sum(out * d_out))


def test_smallseq_forward_matches_paged_attention_decode_rows():
    """The forward is the decode case of the general oracle (one row per sequence), and
    its weights are a distribution over the first L_s keys."""
    q, keys, values, _ = _smallseq_case(11)
    out, P = ref.smallseq_forward(q, keys, values, 2, 0.37)
    lens = np.array([k.shape[0] for k in keys], np.int32)
    cu = np.arange(len(lens) + 1, dtype=np.int32)
    want, _ = ref.paged_attention(q, keys, values, cu, lens, 2, 0.37, ref.MASK_NONE)
    assert np.allclose(out, want, rtol=0, atol=1e-13)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-14)
    for s, L in enumerate(lens):
        assert np.all(P[s, :, L:] == 0)


def test_smallseq_backward_matches_finite_differences():
    """Central differences of sum(d_out * out) in every coordinate of q, K and V."""
    Hkv, scale, eps = 2, 0.41, 1e-6
    q, keys, values, d_out = _smallseq_case(12)
    dq, dk, dv = ref.smallseq_backward(q, keys, values, d_out, Hkv, scale)

    def fd(arr, idx, rebuild):
        a = arr.copy(); a[idx] += eps
        b = arr.copy(); b[idx] -= eps
        return (_loss(*rebuild(a), d_out, Hkv, scale) - _loss(*rebuild(b), d_out, Hkv, scale)) / (2 * eps)

    for idx in np.ndindex(q.shape):
        g = fd(q, idx, lambda a: (a, keys, values))
        assert abs(g - dq[idx]) < 1e-7 * max(1.0, abs(g)), ("dq", idx, g, dq[idx])
    for s in range(len(keys)):
        for idx in np.ndindex(keys[s].shape):
            def rk(a, s=s):
                ks = list(keys); ks[s] = a
                return (q, ks, values)
            def rv(a, s=s):
                vs = list(values); vs[s] = a
                return (q, keys, vs)
            gk = fd(keys[s], idx, rk)
            gv = fd(values[s], idx, rv)
            assert abs(gk - dk[s][idx]) < 1e-7 * max(1.0, abs(gk)), ("dk", s, idx)
            assert abs(gv - dv[s][idx]) < 1e-7 * max(1.0, abs(gv)), ("dv", s, idx)


def test_smallseq_backward_matches_torch_autograd():
    """torch float64 autograd of softmax attention written with torch ops (GQA by
    repeat_interleave), on several random batches."""
    for seed in range(4):
        rng = np.random.default_rng(100 + seed)
        H, Hkv, D = 6, 3, 8
        lens = list(rng.integers(1, 17, size=5))
        q, keys, values, d_out = _smallseq_case(100 + seed, S=5, H=H, Hkv=Hkv, D=D, lens=lens)
        dq, dk, dv = ref.smallseq_backward(q, keys, values, d_out, Hkv, 0.3)
        for s in range(5):
            tq = torch.tensor(q[s], requires_grad=True)                       # [H, D]
            tk = torch.tensor(keys[s], requires_grad=True)                    # [L, Hkv, D]
            tv = torch.tensor(values[s], requires_grad=True)
            ke = tk.repeat_interleave(H // Hkv, dim=1)                        # [L, H, D]
            ve = tv.repeat_interleave(H // Hkv, dim=1)
            z = 0.3 * torch.einsum("hd,lhd->hl", tq, ke)
            o = torch.einsum("hl,lhd->hd", torch.softmax(z, dim=-1), ve)
            (o * torch.tensor(d_out[s])).sum().backward()
            assert np.allclose(tq.grad.numpy(), dq[s], atol=1e-12)
            assert np.allclose(tk.grad.numpy(), dk[s], atol=1e-12)
            assert np.allclose(tv.grad.numpy(), dv[s], atol=1e-12)


def test_smallseq_backward_closed_forms():
    """One key: P = 1, so dV = the sum of dO over the group's heads and dQ = dK = 0.
    Any length: the key gradients of a query sum to zero (the softmax backward removes
    the mean), so sum_k dK[k] = 0."""
    q, keys, values, d_out = _smallseq_case(13, lens=(1, 1, 1))
    dq, dk, dv = ref.smallseq_backward(q, keys, values, d_out, 2, 0.5)
    assert np.all(dq == 0)
    for s in range(3):
        assert np.all(dk[s] == 0)
        assert np.allclose(dv[s][0], d_out[s].reshape(2, 2, -1).sum(axis=1), atol=1e-15)
    q, keys, values, d_out = _smallseq_case(14, lens=(16, 5, 9))
    _, dk, _ = ref.smallseq_backward(q, keys, values, d_out, 2, 0.5)
    for s in range(3):
        assert np.allclose(dk[s].sum(axis=0), 0.0, atol=1e-13)


def test_smallseq_backward_gqa_equals_mha_with_repeated_kv():
    """Grouped heads: the same as MHA on repeated K/V with dK, dV summed over the group."""
    q, keys, values, d_out = _smallseq_case(15, S=2, H=6, Hkv=2, D=4, lens=(5, 12))
    dq, dk, dv = ref.smallseq_backward(q, keys, values, d_out, 2, 0.7)
    kr = [np.repeat(k, 3, axis=1) for k in keys]
    vr = [np.repeat(v, 3, axis=1) for v in values]
    dq2, dk2, dv2 = ref.smallseq_backward(q, kr, vr, d_out, 6, 0.7)
    assert np.allclose(dq, dq2, atol=1e-14)
    for s in range(2):
        assert np.allclose(dk[s], dk2[s].reshape(dk2[s].shape[0], 2, 3, -1).sum(axis=2), atol=1e-14)
        assert np.allclose(dv[s], dv2[s].reshape(dv2[s].shape[0], 2, 3, -1).sum(axis=2), atol=1e-14)


def test_smallseq_backward_planted_mistake_is_caught():
    """A softmax backward without the mean term fails the finite-difference pin."""
    Hkv, scale, eps = 2, 0.41, 1e-6
    q, keys, values, d_out = _smallseq_case(16)
    _, P = ref.smallseq_forward(q, keys, values, Hkv, scale)
    s, h, L = 2, 1, keys[2].shape[0]
    p = P[s, h, :L]
    dp = values[s][:, h // 2, :] @ d_out[s, h]
    wrong = scale * ((p * dp) @ keys[s][:, h // 2, :])       # dS = P dP, mean dropped
    a = q.copy(); a[s, h, 0] += eps
    b = q.copy(); b[s, h, 0] -= eps
    g = (_loss(a, keys, values, d_out, Hkv, scale) - _loss(b, keys, values, d_out, Hkv, scale)) / (2 * eps)
    assert abs(g - wrong[0]) > 1e-4


def test_smallseq_train_workload_feeds_the_oracle():
    """The training workload's rows, split per sequence, run through the oracle; with one
    query row per sequence its forward equals the general oracle's decode rows."""
    w = wl.smallseq_train(num_seqs=40)
    q = ref.widen(w.query, w.dtype)
    k = ref.split_logical(ref.widen(w.key, w.dtype), w.cu_seq_lens)
    v = ref.split_logical(ref.widen(w.value, w.dtype), w.cu_seq_lens)
    out, P = ref.smallseq_forward(q, k, v, w.num_kv_heads, w.scale, max_kv=16)
    want, _ = ref.workload_attention(w)
    assert np.allclose(out, want, atol=1e-13)
    assert P.shape == (40, 16, 16) and w.d_out.shape == (40, 16, 128)
