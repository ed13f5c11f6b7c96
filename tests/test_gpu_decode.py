"""paged_attention_decode on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, compare, to_dev

pytestmark = pytest.mark.gpu


def _run(w, combined=False, rows=None):
    d = Dev(w, combined=combined)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got, want = got[rows], want[rows]
    return compare(got, want, w.dtype, w.name)


def test_decode_batch_full_size(gpu):
    """64 sequences, contexts 256..4096, 32 q / 8 kv heads, D 128, bf16: every output."""
    _run(wl.decode_batch())


@pytest.mark.timeout(400)
def test_smallseq_full_size_every_row(gpu):
    """30720 sequences with s_kv in {2..16}, MHA 16 heads: every output row and head."""
    _run(wl.smallseq_varlen())


def test_smallseq_small_all_rows(gpu):
    _run(wl.smallseq_varlen(num_seqs=700))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_dtypes(gpu, dtype):
    _run(wl.decode_batch(seed=11, num_seqs=5, lo=1, hi=1500, dtype=dtype))


def test_decode_combined_cache_layout(gpu):
    _run(wl.decode_batch(seed=12, num_seqs=4, lo=100, hi=900), combined=True)


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(gpu, seed):
    """Random GQA ratios (incl. 3), head_dim 16/64/128, block sizes 1..4, lengths 1..12."""
    rng = np.random.default_rng(100 + seed)
    d = int(rng.choice([16, 64, 128]))
    dt = str(rng.choice(["bf16", "f16", "f32"]))
    _run(wl.random_small(seed, dt, head_dim=d, decode=True, max_len=40))


def test_decode_long_sequence_many_splits(gpu):
    """One 40k-token sequence next to short ones: many splits plus the LSE merge."""
    lens = np.array([40000, 3, 1, 700], np.int32)
    w = wl.build("long_decode", 21, "bf16", lens, np.ones(4, np.int32), 16, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    _run(w)


@pytest.mark.parametrize("H", [8, 16])
def test_decode_stream_vector_core(gpu, H):
    """Stream mode at 1 and 2 query heads per kv head (8 kv heads, D 128, bf16): the vector
    core, which the matrix cores take over from 4 heads per wave."""
    lens = np.random.default_rng(25).integers(1, 3000, size=20).astype(np.int32)
    lens[:3] = [1, 33, 2999]
    w = wl.build("stream_vector", 25, "bf16", lens, np.ones(len(lens), np.int32), H, 8, 128, 16,
                 wl.MASK_NONE, decode=True)
    _run(w)


def test_decode_gqa_wide(gpu):
    """g = 16 (two 8-head waves per kv head) and g = 6 (a partly filled wave)."""
    for H, Hkv in [(32, 2), (12, 2)]:
        lens = np.array([300, 1000, 17], np.int32)
        w = wl.build("gqa_wide", 22, "bf16", lens, np.ones(3, np.int32), H, Hkv, 64, 16,
                     wl.MASK_NONE, decode=True)
        _run(w)


def test_decode_empty_and_single_token_sequences(gpu):
    lens = np.array([0, 1, 0, 2, 513], np.int32)
    w = wl.build("edge_decode", 23, "bf16", lens, np.minimum(lens, 1), 8, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    # sequences with L = 0 own no query row in the generator; give every sequence one
    # query row (decode layout [S, H, D]) by rebuilding the query array
    q = wl.round_to_storage(np.random.default_rng(3).standard_normal((5, 8, 128)).astype(np.float32), "bf16")
    w.query = q
    w.q_lens = np.ones(5, np.int32)
    w.cu_seqlens_q = np.arange(6, dtype=np.int32)
    d = Dev(w)
    B.kv_cache_write(d.key, d.value, d.slots, d.kc, d.vc)
    out = d.decode()
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    # single visible key: the output is that key's V row, bit-exact after rounding
    v = ref.widen(w.value, "bf16")
    for h in range(8):
        assert np.array_equal(got[1, h], v[w.cu_seq_lens[1], h // 4])
    # sequences with keys: the oracle's decode (the query is the newest of L_s tokens)
    keys = ref.split_logical(ref.widen(w.key, "bf16"), w.cu_seq_lens)
    vals = ref.split_logical(v, w.cu_seq_lens)
    live = [1, 3, 4]
    want, _ = ref.paged_attention(ref.widen(q[live], "bf16"), [keys[i] for i in live],
                                  [vals[i] for i in live], np.arange(4, dtype=np.int32),
                                  lens[live], 2, w.scale, wl.MASK_NONE)
    compare(got[live], want, "bf16", "edge_decode")


def test_decode_constant_value_rows(gpu):
    """Constant V returns the constant for any query (closed form), exactly in bf16."""
    w = wl.decode_batch(seed=13, num_seqs=6, lo=1, hi=2000)
    w.value[:] = wl.round_to_storage(np.full(1, -0.625, np.float32), "bf16")[0]
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    assert np.all(as_f64(out) == -0.625)


def test_decode_rejects_small_workspace(gpu):
    w = wl.decode_batch(seed=14, num_seqs=8, lo=2000, hi=4096)
    d = Dev(w)
    need = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.max_seq_len)
    assert need > 0
    out = torch.full_like(d.query, 3.0)
    ws = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.PkvError) as e:
        B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                 w.max_seq_len, ws)
    assert e.value.code == B.PKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_decode_shared_workspace_back_to_back(gpu):
    """Decode batches of different shape on one workspace, one after another: nothing a
    call leaves in the workspace changes the next call's result."""
    w1 = wl.decode_batch(seed=15, num_seqs=12, lo=300, hi=4096)
    w2 = wl.decode_batch(seed=16, num_seqs=5, lo=1000, hi=6000)
    need = max(B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                       w.block_size, w.max_seq_len) for w in (w1, w2))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")   # garbage, not zeros
    for w in (w1, w2, w1):
        d = Dev(w)
        d.write_all()
        out = torch.empty_like(d.query)
        B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                 w.max_seq_len, ws)
        torch.cuda.synchronize()
        want, _ = ref.workload_attention(w)
        compare(as_f64(out), want, w.dtype, w.name)


def test_decode_all_empty_batch_with_long_hint(gpu):
    """seq_lens all 0 with a long max_seq_len hint (the long-context work split): zeros."""
    lens = np.zeros(6, np.int32)
    w = wl.build("all_empty", 24, "bf16", lens, lens, 8, 2, 128, 16, wl.MASK_NONE, decode=True,
                 max_blocks_per_seq=512)
    q = wl.round_to_storage(np.random.default_rng(4).standard_normal((6, 8, 128)).astype(np.float32), "bf16")
    w.query = q
    d = Dev(w)
    out = torch.full_like(d.query, 5.0)
    need = B.decode_workspace_size(6, 8, 2, 128, 16, 8192)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale, 8192, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_smallseq_thd_zero_copy_view(gpu):
    """K/V packed THD [sum s_kv, Hkv, D] used in place as a block_size-1 cache, with
    block_tables[s][j] = cu_kv[s] + j: no scatter, the same decode kernel."""
    w = wl.smallseq_varlen(num_seqs=500)
    key = to_dev(w.key, w.dtype)
    value = to_dev(w.value, w.dtype)
    kc = key.view(-1, 1, w.num_kv_heads, w.head_dim)
    vc = value.view(-1, 1, w.num_kv_heads, w.head_dim)
    mb = int(w.seq_lens.max())
    tables = np.zeros((w.num_seqs, mb), np.int32)
    for s in range(w.num_seqs):
        tables[s, :w.seq_lens[s]] = w.cu_seq_lens[s] + np.arange(w.seq_lens[s])
    q = to_dev(w.query, w.dtype)
    out = torch.empty_like(q)
    need = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, 1, mb)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    B.paged_attention_decode(out, q, kc, vc, torch.from_numpy(tables).cuda(),
                             torch.from_numpy(w.seq_lens).cuda(), w.scale, mb, ws if need else None)
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w)
    compare(as_f64(out), want, w.dtype, "thd_view")


@pytest.mark.parametrize("H,Hkv", [(16, 16), (8, 4), (12, 3), (32, 4), (16, 2)])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_decode_item_mode(gpu, H, Hkv, dtype, head_dim):
    """Short sequences (at most 8 pages, one split): eight items per wave, one per group
    of 8 lanes.  Item counts that leave the last wave part-filled, empty sequences, every
    length from 0 to 8 pages, and 1, 2, 4 and 8 heads per item."""
    bs = 4
    lens = np.arange(0, 8 * bs + 1, dtype=np.int32)
    lens = np.concatenate([lens, np.array([8 * bs, 1, 0, 3, 17], np.int32)])
    w = wl.build("item_mode", 60 + H, dtype, lens, np.minimum(lens, 1), H, Hkv, head_dim, bs,
                 wl.MASK_NONE, decode=True)
    # one query row per sequence, also for the empty ones (decode layout [S, H, D])
    q = wl.round_to_storage(np.random.default_rng(61).standard_normal((len(lens), H, head_dim))
                            .astype(np.float32), dtype)
    w.query = q
    w.q_lens = np.ones(len(lens), np.int32)
    w.cu_seqlens_q = np.arange(len(lens) + 1, dtype=np.int32)
    d = Dev(w)
    B.kv_cache_write(d.key, d.value, d.slots, d.kc, d.vc)
    out = d.decode()
    torch.cuda.synchronize()
    got = as_f64(out)
    empty = lens == 0
    assert np.all(got[empty] == 0)
    live = np.nonzero(~empty)[0]
    keys = ref.split_logical(ref.widen(w.key, dtype), w.cu_seq_lens)
    vals = ref.split_logical(ref.widen(w.value, dtype), w.cu_seq_lens)
    want, _ = ref.paged_attention(ref.widen(q[live], dtype), [keys[i] for i in live],
                                  [vals[i] for i in live], np.arange(len(live) + 1, dtype=np.int32),
                                  lens[live], Hkv, w.scale, wl.MASK_NONE)
    compare(got[live], want, dtype, f"item_mode H{H} Hkv{Hkv}")


def test_decode_prefix_stream_mode(gpu):
    """More than 256 sequences with contexts past one split: stream mode with the planning
    kernel (prefix sums and range starts in the workspace), partials and the stream
    merge; sequences spanning range boundaries and ranges spanning many sequences."""
    rng = np.random.default_rng(81)
    lens = rng.integers(1, 900, size=1100).astype(np.int32)
    lens[:4] = [256, 257, 512, 899]
    w = wl.build("split_mode", 81, "bf16", lens, np.ones(len(lens), np.int32), 8, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    need = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                   w.block_size, w.max_seq_len)
    assert need > 0                                   # partials and planning tables
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(len(lens), 200, replace=False)]))
    _run(w, rows=rows)


@pytest.mark.parametrize("H", [8, 32])
def test_decode_prefix_stream_empty_sequences(gpu, H):
    """1200 sequences, some empty (first, last and scattered), 8 kv heads at 1 and 4
    query heads per kv head (vector and matrix-core cores): empty rows are zero, the
    others match the oracle."""
    rng = np.random.default_rng(83)
    S, Hkv, D = 1200, 8, 128
    lens = rng.integers(1, 700, size=S).astype(np.int32)
    lens[[0, 5, 6, 500, S - 2, S - 1]] = 0
    w = wl.build("prefix_empty", 83, "bf16", lens, np.minimum(lens, 1), H, Hkv, D, 16,
                 wl.MASK_NONE, decode=True)
    # the generator gives empty sequences no query row: one per sequence ([S, H, D])
    q = wl.round_to_storage(rng.standard_normal((S, H, D)).astype(np.float32), "bf16")
    w.query = q
    w.q_lens = np.ones(S, np.int32)
    w.cu_seqlens_q = np.arange(S + 1, dtype=np.int32)
    d = Dev(w)
    B.kv_cache_write(d.key, d.value, d.slots, d.kc, d.vc)
    out = d.decode()
    torch.cuda.synchronize()
    got = as_f64(out)
    empty = np.flatnonzero(lens == 0)
    assert np.all(got[empty] == 0)
    live = np.sort(np.concatenate([[1, 4, 7, 499, 501, S - 3],
                                   rng.choice(np.flatnonzero(lens > 0), 60, replace=False)]))
    live = np.unique(live)
    keys = ref.split_logical(ref.widen(w.key, "bf16"), w.cu_seq_lens)
    vals = ref.split_logical(ref.widen(w.value, "bf16"), w.cu_seq_lens)
    want, _ = ref.paged_attention(ref.widen(q[live], "bf16"), [keys[i] for i in live],
                                  [vals[i] for i in live], np.arange(len(live) + 1, dtype=np.int32),
                                  lens[live], Hkv, w.scale, wl.MASK_NONE)
    compare(got[live], want, "bf16", f"prefix_empty H{H}")


def test_decode_one_split_mode(gpu):
    """Every sequence fits one split (at most 256 keys) but some exceed the 8 pages of
    item mode: the split kernel with one split per sequence, written directly."""
    lens = np.random.default_rng(84).integers(1, 257, size=300).astype(np.int32)
    lens[:3] = [256, 129, 1]
    w = wl.build("one_split", 84, "bf16", lens, np.ones(len(lens), np.int32), 32, 8, 128, 16,
                 wl.MASK_NONE, decode=True)
    assert B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                   w.block_size, w.max_seq_len) == 0
    _run(w)


@pytest.mark.parametrize("case", ["f16_bs8", "bf16_d64", "fp8", "f32"])
def test_decode_prefix_stream_variants(gpu, case):
    """Stream mode with the planning kernel across the other shapes: fp16 on pages of 8,
    head_dim 64, an FP8 cache, fp32 (vector core): sampled rows against the oracle."""
    rng = np.random.default_rng(85)
    S = 1100
    lens = rng.integers(1, 800, size=S).astype(np.int32)
    dtype = {"f16_bs8": "f16", "bf16_d64": "bf16", "fp8": "bf16", "f32": "f32"}[case]
    D = 64 if case == "bf16_d64" else 128
    bs = 8 if case == "f16_bs8" else 16
    w = wl.build(f"prefix_{case}", 85, dtype, lens, np.ones(S, np.int32), 16, 4, D, bs,
                 wl.MASK_NONE, decode=True)
    if case == "fp8":
        w = wl.with_fp8_cache(w)
    rows = np.unique(np.concatenate([np.arange(4), [S - 1], rng.choice(S, 100, replace=False)]))
    _run(w, rows=rows)


def test_decode_prefix_stream_mid_batch(gpu):
    """400 sequences of up to 3000 keys (32 q / 8 kv heads, bf16): past the 256 sequences a
    wave scans, so the planning kernel's tables serve them."""
    rng = np.random.default_rng(86)
    lens = rng.integers(1, 3000, size=400).astype(np.int32)
    w = wl.build("prefix_mid", 86, "bf16", lens, np.ones(len(lens), np.int32), 32, 8, 128, 16,
                 wl.MASK_NONE, decode=True)
    rows = np.unique(np.concatenate([np.arange(4), [399], rng.choice(400, 60, replace=False)]))
    _run(w, rows=rows)
