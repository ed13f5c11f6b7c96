"""FP8 (E4M3) KV cache on the GPU: the quantising scatter bit-exact against the oracle's
quantiser, and decode over the codes against the oracle's attention over the dequantised
rows (the scale convention is the one include/pkv.h states)."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, compare, to_dev

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F


def _batch(seed, dtype, lens, H=32, Hkv=8, head_dim=128, bs=16):
    lens = np.asarray(lens, np.int32)
    return wl.build("fp8_batch", seed, dtype, lens, np.ones(len(lens), np.int32), H, Hkv,
                    head_dim, bs, wl.MASK_NONE, decode=True)


def _expected_codes(w, key_rows, value_rows, slots):
    """Cache bytes after the scatter: 0x7F everywhere, the oracle's codes at the slots."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kq = ref.quantize_e4m3(ref.widen(key_rows, w.dtype), np.float32(1) / np.float32(w.k_scale))
    vq = ref.quantize_e4m3(ref.widen(value_rows, w.dtype), np.float32(1) / np.float32(w.v_scale))
    kc = np.full(shape, NAN_CODE, np.uint8)
    vc = np.full(shape, NAN_CODE, np.uint8)
    return ref.kv_cache_write(kc, vc, kq, vq, slots, w.block_size)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("head_dim", [128, 64, 16])
def test_fp8_write_bit_exact(gpu, dtype, head_dim):
    lens = np.random.default_rng(31).integers(1, 301, size=6)
    w = wl.with_fp8_cache(_batch(31, dtype, lens, head_dim=head_dim))
    d = Dev(w)
    d.write_all()
    torch.cuda.synchronize()
    ek, ev = _expected_codes(w, w.key, w.value, w.slots)
    assert np.array_equal(d.kc.cpu().numpy(), ek)
    assert np.array_equal(d.vc.cpu().numpy(), ev)


def test_fp8_write_edge_values(gpu):
    """Rounding ties, subnormal codes, the clamp at +-448 and beyond, zeros of both signs,
    in f32 rows (exactly what the kernel scales): every code against the oracle."""
    w = wl.with_fp8_cache(_batch(32, "f32", [64], H=8, Hkv=8), k_scale=1.0, v_scale=0.5)
    rng = np.random.default_rng(33)
    mags = np.array([e for e in (ref.e4m3_value(c) for c in range(0x7F))])
    mids = (mags[:-1] + mags[1:]) / 2                       # exact ties (fp32-representable)
    special = np.concatenate([mags, mids, [448.0, 449.0, 464.0, 480.0, 1e6, 3e38, 2.0 ** -10,
                                           2.0 ** -11, 0.0]])
    vals = np.concatenate([special, -special])
    T, n = w.key.shape[0], w.num_kv_heads * w.head_dim
    k = rng.choice(vals, size=(T, n)).astype(np.float32)
    assert vals.size <= n
    k[0, :vals.size] = vals
    v = rng.choice(vals, size=(T, n)).astype(np.float32) * np.float32(0.5)
    w.key = k.reshape(w.key.shape).view(np.uint32)
    w.value = v.reshape(w.value.shape).view(np.uint32)
    d = Dev(w)
    d.write_all(split_new=False)
    torch.cuda.synchronize()
    ek, ev = _expected_codes(w, w.key, w.value, w.slots)
    assert np.array_equal(d.kc.cpu().numpy(), ek)
    assert np.array_equal(d.vc.cpu().numpy(), ev)


def test_fp8_write_nan_gives_nan_code(gpu):
    w = wl.with_fp8_cache(_batch(34, "bf16", [16], H=8, Hkv=8, head_dim=64))
    d = Dev(w, fill="zero")
    key = d.key.clone()
    key[3, 0, 5] = float("nan")
    B.kv_cache_write_fp8(key, d.value, d.slots, d.kc, d.vc, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    slot = int(w.slots[3])
    code = int(d.kc[slot // w.block_size, slot % w.block_size, 0, 5])
    assert code & 0x7F == 0x7F


def test_fp8_gather_round_trip(gpu):
    w = wl.with_fp8_cache(wl.decode_batch(seed=35, num_seqs=5, lo=1, hi=200))
    d = Dev(w)
    d.write_all()
    ko = torch.empty((w.key.shape[0],) + tuple(d.kc.shape[2:]), dtype=torch.uint8, device="cuda")
    vo = torch.empty_like(ko)
    B.kv_cache_gather(ko, vo, d.cu_k, d.kc, d.vc, d.tables, w.max_seq_len)
    torch.cuda.synchronize()
    kq = ref.quantize_e4m3(ref.widen(w.key, w.dtype), np.float32(1) / np.float32(w.k_scale))
    vq = ref.quantize_e4m3(ref.widen(w.value, w.dtype), np.float32(1) / np.float32(w.v_scale))
    assert np.array_equal(ko.cpu().numpy(), kq) and np.array_equal(vo.cpu().numpy(), vq)


def _decode(w, rows=None):
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got, want = got[rows], want[rows]
    return compare(got, want, w.dtype, w.name)


def test_fp8_decode_batch_full_size(gpu):
    """The decode batch (64 sequences, 256..4096 keys, 32 q / 8 kv heads, D 128) over an
    FP8 cache, stream mode: every output row."""
    _decode(wl.decode_batch_fp8())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("head_dim", [128, 64, 16])
def test_fp8_decode_dtypes_and_head_dims(gpu, dtype, head_dim):
    lens = np.random.default_rng(36).integers(1, 1501, size=5)
    _decode(wl.with_fp8_cache(_batch(36, dtype, lens, head_dim=head_dim)))


def test_fp8_decode_item_mode(gpu):
    """Short sequences (at most 8 pages): the eight-items-per-wave kernel."""
    lens = np.concatenate([np.arange(1, 8 * 16 + 1, 7), [128, 1, 2]]).astype(np.int32)
    w = wl.build("item_fp8", 37, "bf16", lens, np.ones(len(lens), np.int32), 16, 4, 128, 16,
                 wl.MASK_NONE, decode=True)
    _decode(wl.with_fp8_cache(w))


def test_fp8_decode_prefix_stream(gpu):
    """More than 256 sequences with contexts past one split: stream mode with the
    planning kernel's tables and the stream merge."""
    rng = np.random.default_rng(38)
    lens = rng.integers(1, 900, size=1100).astype(np.int32)
    w = wl.build("split_fp8", 38, "f16", lens, np.ones(len(lens), np.int32), 8, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(len(lens), 150, replace=False)]))
    _decode(wl.with_fp8_cache(w), rows=rows)


def test_fp8_decode_long_sequence(gpu):
    lens = np.array([40000, 3, 1, 700], np.int32)
    w = wl.build("long_fp8", 39, "bf16", lens, np.ones(4, np.int32), 16, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    _decode(wl.with_fp8_cache(w, k_scale=0.05, v_scale=0.003))


def test_fp8_decode_rejects_f32_query(gpu):
    w = wl.with_fp8_cache(wl.decode_batch(seed=40, num_seqs=2, lo=4, hi=20, dtype="f32"))
    d = Dev(w)
    out = torch.empty_like(d.query)
    with pytest.raises(B.PkvError) as e:
        B.paged_attention_decode_fp8(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                     w.k_scale, w.v_scale, w.max_seq_len)
    assert e.value.code == B.PKV_ERR_UNSUPPORTED


def _prefill(w, rows=None, heads=None):
    d = Dev(w)
    d.write_all()
    out = d.prefill()
    torch.cuda.synchronize()
    got = as_f64(out)
    want, _ = ref.workload_attention(w, rows=rows, heads=heads)
    if rows is not None:
        got, want = got[rows], want[rows]
    if heads is not None:
        got, want = got[:, heads], want[:, heads]
    return compare(got, want, w.dtype, w.name)


@pytest.mark.parametrize("mask", [wl.MASK_NONE, wl.MASK_CAUSAL, wl.MASK_BLOCK_CAUSAL])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_prefill_chunked_masks(gpu, mask, dtype):
    """Chunked prefill over an FP8 cache (MFMA kernel, D 128): several tiles, ragged tails."""
    w = wl.chunked_prefill(seed=50 + mask, num_seqs=4, ctx_hi=300, q_lo=1, q_hi=200, dtype=dtype)
    w.mask = mask
    w.span_len = 48
    _prefill(wl.with_fp8_cache(w))


@pytest.mark.parametrize("seed", range(8))
def test_fp8_prefill_random_shapes(gpu, seed):
    """head_dim 16 (vector-ALU kernel), 64 and 128 (MFMA), random GQA, lengths and masks."""
    rng = np.random.default_rng(400 + seed)
    d = int(rng.choice([16, 64, 128]))
    dt = str(rng.choice(["bf16", "f16"]))
    _prefill(wl.with_fp8_cache(wl.random_small(seed, dt, head_dim=d, max_len=70)))


def test_fp8_chunked_prefill_scaled(gpu):
    """The chunked-prefill shape (8 seqs, ctx <= 2048, chunk 32..512, 32q/8kv, D 128)."""
    _prefill(wl.with_fp8_cache(wl.chunked_prefill()))


def test_fp8_long_block_causal_sampled(gpu):
    """4 x 8192 tokens, 64 q heads, block-causal spans of 2048, FP8 cache: sampled rows."""
    w = wl.with_fp8_cache(wl.long_block_causal())
    rows = []
    for s in range(w.num_seqs):
        rows += [s * 8192 + p for p in (0, 1, 2047, 2048, 5000, 6144, 8191)]
    _prefill(w, rows=np.array(rows), heads=[0, 9, 63])


def test_fp8_prefill_single_key_rows_are_scaled_codes(gpu):
    """A causal row that sees only key 0 returns that key's V row: its codes times v_scale,
    rounded once to the output type."""
    w = wl.with_fp8_cache(wl.chunked_prefill(seed=55, num_seqs=2, ctx_hi=0, q_lo=40, q_hi=90))
    d = Dev(w)
    d.write_all()
    out = d.prefill()
    torch.cuda.synchronize()
    got = as_f64(out)
    _, vv = ref.workload_kv(w)
    g = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        r0 = w.cu_seqlens_q[s]
        want = vv[w.cu_seq_lens[s]][np.arange(w.num_heads) // g]
        want = ref.widen(wl.round_to_storage(want.astype(np.float32), w.dtype), w.dtype)
        assert np.array_equal(got[r0], want)
