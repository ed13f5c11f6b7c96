"""The matrix-core decode core (stream and split mode at 8 query heads per wave with a
bf16 / fp16 cache at head_dim 128; 4 or more with an FP8 cache or at head_dim 64) against
the fp64 oracle.

Every cache slot that no token was written to holds NaN (the Dev sentinel), so a key
outside a segment that leaked into a probability or a V product would show up as NaN.
"""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, compare

pytestmark = pytest.mark.gpu


def _run(w, rows=None):
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    got = as_f64(out)
    assert not np.isnan(got).any(), "NaN reached an output row"
    want, _ = ref.workload_attention(w, rows=rows)
    if rows is not None:
        got, want = got[rows], want[rows]
    return compare(got, want, w.dtype, w.name)


def _batch(name, seed, dtype, lens, H, Hkv, D, bs=16):
    lens = np.asarray(lens, np.int32)
    return wl.build(name, seed, dtype, lens, np.minimum(lens, 1), H, Hkv, D, bs, wl.MASK_NONE,
                    decode=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("head_dim", [128, 64])
def test_mfma_stream_g8(gpu, dtype, head_dim):
    """Stream mode, 64 q / 8 kv heads: lengths that are not multiples of 8 or 32, so range
    boundaries and sequence ends fall inside steps and inside 8-key groups."""
    rng = np.random.default_rng(60 + head_dim)
    lens = rng.integers(1, 2500, size=12)
    lens[:4] = [1, 31, 33, 257]
    _run(_batch("mfma_stream", 61, dtype, lens, 64, 8, head_dim))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mfma_stream_d64_g4(gpu, dtype):
    """head_dim 64 at 4 heads per wave (32 q / 8 kv heads) runs on the matrix cores too."""
    rng = np.random.default_rng(70)
    lens = rng.integers(1, 3000, size=16)
    lens[:3] = [7, 8, 4095]
    _run(_batch("mfma_d64_g4", 70, dtype, lens, 32, 8, 64))


def test_mfma_decode_batch_shape_g8(gpu):
    """The decode batch's length mix (256..4096) with 64 q heads: every output row."""
    lens = np.random.default_rng(1).integers(256, 4097, size=24)
    _run(_batch("mfma_batch_g8", 62, "bf16", lens, 64, 8, 128))


@pytest.mark.parametrize("bs", [8, 32, 64])
def test_mfma_block_sizes(gpu, bs):
    """Pages of 8 tokens (one 8-key group per page: every group its own table entry, many
    table windows per sequence) up to 64."""
    lens = np.array([3000, 8, 9, 700, 1234], np.int32)
    _run(_batch("mfma_bs", 63, "bf16", lens, 16, 2, 128, bs=bs))


def test_mfma_small_pages_take_vector_core(gpu):
    """Pages of 4 tokens cannot hold an 8-key group: the vector core runs, same results."""
    lens = np.array([900, 5, 333], np.int32)
    _run(_batch("mfma_bs4", 64, "bf16", lens, 16, 2, 128, bs=4))


def test_mfma_prefix_stream(gpu):
    """More than 256 sequences: stream mode with the planning kernel's tables."""
    rng = np.random.default_rng(65)
    lens = rng.integers(1, 900, size=1100).astype(np.int32)
    w = _batch("mfma_split", 65, "f16", lens, 16, 2, 128)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(len(lens), 160, replace=False)]))
    _run(w, rows=rows)


def test_mfma_prefix_stream_d64_g4(gpu):
    """More than 256 sequences at head_dim 64 and 4 heads per wave (bf16)."""
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 1200, size=1030).astype(np.int32)
    w = _batch("mfma_split_d64", 71, "bf16", lens, 32, 8, 64)
    rows = np.unique(np.concatenate([np.arange(6), rng.choice(len(lens), 120, replace=False)]))
    _run(w, rows=rows)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mfma_one_split_mode(gpu, dtype):
    """Split mode on the matrix cores: every sequence within one 256-key split, some past
    the 8 pages of item mode, 8 heads per wave."""
    lens = np.random.default_rng(72).integers(1, 257, size=200).astype(np.int32)
    lens[:3] = [256, 129, 1]
    _run(_batch("mfma_one_split", 72, dtype, lens, 64, 8, 128))


def test_mfma_empty_and_tiny_sequences(gpu):
    """Empty sequences give zero rows; one-key sequences return that key's V row exactly."""
    lens = np.array([0, 1, 0, 2, 513, 3000, 0], np.int32)
    S, H, Hkv, D = len(lens), 16, 2, 128
    w = _batch("mfma_edge", 66, "bf16", lens, H, Hkv, D)
    # the generator gives empty sequences no query row: one per sequence ([S, H, D])
    q = wl.round_to_storage(np.random.default_rng(6).standard_normal((S, H, D)).astype(np.float32), "bf16")
    w.query = q
    w.q_lens = np.ones(S, np.int32)
    w.cu_seqlens_q = np.arange(S + 1, dtype=np.int32)
    d = Dev(w)
    B.kv_cache_write(d.key, d.value, d.slots, d.kc, d.vc)
    out = d.decode()
    torch.cuda.synchronize()
    got = as_f64(out)
    for s in (0, 2, 6):
        assert np.all(got[s] == 0)
    v = ref.widen(w.value, "bf16")
    g = H // Hkv
    for h in range(H):
        assert np.array_equal(got[1, h], v[w.cu_seq_lens[1], h // g])
    keys = ref.split_logical(ref.widen(w.key, "bf16"), w.cu_seq_lens)
    vals = ref.split_logical(v, w.cu_seq_lens)
    live = [1, 3, 4, 5]
    want, _ = ref.paged_attention(ref.widen(q[live], "bf16"), [keys[i] for i in live],
                                  [vals[i] for i in live], np.arange(len(live) + 1, dtype=np.int32),
                                  lens[live], Hkv, w.scale, wl.MASK_NONE)
    compare(got[live], want, "bf16", "mfma_edge")


def test_mfma_constant_value_rows(gpu):
    """Constant V gives the constant for any query (closed form), exactly."""
    w = _batch("mfma_const", 67, "bf16", np.random.default_rng(7).integers(1, 3000, size=9), 64, 8, 128)
    w.value[:] = wl.round_to_storage(np.full(1, 0.8125, np.float32), "bf16")[0]
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    assert np.all(as_f64(out) == 0.8125)


def test_mfma_large_scores_rescale(gpu):
    """Scores spread over hundreds of log2 units: the running max moves many times (the
    lazy rescale) and the result stays on the oracle."""
    w = _batch("mfma_rescale", 68, "bf16", [2000, 777, 64], 64, 8, 128)
    w.scale = 2.0
    _run(w)


def test_mfma_fp8_g8(gpu):
    """FP8 cache at 8 heads per wave, stream mode, D 128 and 64."""
    for D in (128, 64):
        lens = np.random.default_rng(69).integers(1, 3000, size=10)
        _run(wl.with_fp8_cache(_batch("mfma_fp8_g8", 69, "bf16", lens, 64, 8, D)))


@pytest.mark.parametrize("case", ["bf16_one_long", "f16_d64_four", "fp8_two", "f32_mha_one"])
def test_wide_merge_few_sequences(gpu, case):
    """Few long sequences in stream mode: every head merges dozens of partials, 32 to a
    load round (the running max moves between rounds), also past a partial round."""
    rng = np.random.default_rng(73)
    if case == "bf16_one_long":
        w = _batch("wide_one", 73, "bf16", [41000], 64, 8, 128)
    elif case == "f16_d64_four":
        w = _batch("wide_four", 74, "f16", [9000, 1, 20000, 777], 32, 8, 64)
    elif case == "fp8_two":
        w = wl.with_fp8_cache(_batch("wide_fp8", 75, "bf16", [30000, 12345], 64, 8, 128))
    else:
        w = _batch("wide_mha", 76, "f32", [int(rng.integers(20000, 30000))], 16, 16, 128)
    w.scale = 1.5 * w.scale
    _run(w)


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_long_shapes(gpu, seed):
    """Random batch sizes (1..300), GQA ratios, head_dim, page sizes, dtypes and FP8
    caches with sequences past one split: whichever core (vector / matrix), mode (stream
    with scans or tables, split) and merge (per wave, per workgroup) the host picks, the
    sampled rows stay on the oracle and no unwritten slot leaks in."""
    rng = np.random.default_rng(500 + seed)
    S = int(rng.choice([1, 2, 3, 5, 8, 17, 64, 200, 300]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    dtype = str(rng.choice(["bf16", "f16"]))
    fp8 = bool(rng.integers(0, 4) == 0)
    # at most ~40M cached K elements so the host-side generation stays quick
    cap = max(300, min(30000, 40_000_000 // (S * Hkv * D)))
    lens = rng.integers(1, cap + 1, size=S).astype(np.int32)
    lens[rng.integers(0, S)] = max(int(lens.max()), 257)      # some sequence past one split
    w = _batch(f"rand_long_{seed}", 500 + seed, dtype, lens, g * Hkv, Hkv, D, bs=bs)
    if fp8:
        w = wl.with_fp8_cache(w)
    rows = np.unique(np.concatenate([[0, S - 1], rng.choice(S, min(S, 40), replace=False)]))
    _run(w, rows=rows)
