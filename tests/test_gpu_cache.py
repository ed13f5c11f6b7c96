"""kv_cache_write / kv_cache_gather on the GPU: bit-exact against the oracle's scatter model."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, bits_of

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_prefill": wl.tiny_prefill,
    "random_bf16": lambda: wl.random_small(5, "bf16", head_dim=64, max_len=40),
    "random_f16_bs1": lambda: wl.random_small(6, "f16", head_dim=16, block_size=1),
    "decode_small": lambda: wl.decode_batch(num_seqs=6, lo=1, hi=300),
    "chunked_small": lambda: wl.chunked_prefill(num_seqs=3, ctx_hi=200, q_hi=100),
    "smallseq_small": lambda: wl.smallseq_varlen(num_seqs=500),
}


def _expected_cache(w):
    st = wl.DTYPES[w.dtype][0]
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = np.full(shape, wl.nan_bits(w.dtype), st)
    vc = np.full(shape, wl.nan_bits(w.dtype), st)
    return ref.kv_cache_write(kc, vc, w.key, w.value, w.slots, w.block_size)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("combined", [False, True])
def test_scatter_bit_exact(gpu, name, combined):
    w = CASES[name]()
    d = Dev(w, combined=combined)
    d.write_all()
    torch.cuda.synchronize()
    ek, ev = _expected_cache(w)
    assert np.array_equal(bits_of(d.kc), ek)
    assert np.array_equal(bits_of(d.vc), ev)


def test_scatter_skips_padding_slots(gpu):
    w = wl.random_small(8, "bf16", head_dim=64, max_len=30)
    d = Dev(w)
    slots = w.slots.copy()
    pad = np.arange(0, slots.size, 3)
    slots[pad] = -1
    B.kv_cache_write(d.key, d.value, torch.from_numpy(slots).cuda(), d.kc, d.vc)
    torch.cuda.synchronize()
    st = wl.DTYPES[w.dtype][0]
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    ek, ev = ref.kv_cache_write(np.full(shape, wl.nan_bits(w.dtype), st),
                                np.full(shape, wl.nan_bits(w.dtype), st), w.key, w.value, slots,
                                w.block_size)
    assert np.array_equal(bits_of(d.kc), ek) and np.array_equal(bits_of(d.vc), ev)


def test_scatter_strided_token_rows(gpu):
    """key/value as views into a fused [T, 3, Hkv, D] projection output (token stride 3x)."""
    w = wl.random_small(9, "bf16", head_dim=64, max_len=25)
    d = Dev(w)
    T = w.key.shape[0]
    fused = torch.empty((T, 3, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    fused[:, 1] = d.key
    fused[:, 2] = d.value
    B.kv_cache_write(fused[:, 1], fused[:, 2], d.slots, d.kc, d.vc)
    torch.cuda.synchronize()
    ek, ev = _expected_cache(w)
    assert np.array_equal(bits_of(d.kc), ek) and np.array_equal(bits_of(d.vc), ev)


@pytest.mark.parametrize("name", list(CASES))
def test_gather_round_trip_bit_exact(gpu, name):
    w = CASES[name]()
    d = Dev(w)
    d.write_all()
    ko = torch.empty_like(d.key)
    vo = torch.empty_like(d.value)
    ko.fill_(0)
    vo.fill_(0)
    B.kv_cache_gather(ko, vo, d.cu_k, d.kc, d.vc, d.tables, w.max_seq_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(ko), w.key)
    assert np.array_equal(bits_of(vo), w.value)


def test_scatter_full_size_smallseq(gpu):
    """The 30720-sequence small-seq batch (about 2 GB of K+V): sampled blocks bit-exact,
    every unmapped slot still holds its sentinel."""
    w = wl.smallseq_varlen()
    d = Dev(w)
    d.write_all(split_new=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for s in rng.choice(w.num_seqs, 64, replace=False):
        blk = int(w.block_tables[s, 0])
        L = int(w.seq_lens[s])
        got = bits_of(d.kc[blk])
        assert np.array_equal(got[:L], w.key[w.cu_seq_lens[s]:w.cu_seq_lens[s + 1]])
        assert np.all(got[L:] == wl.nan_bits("bf16"))
        gotv = bits_of(d.vc[blk])
        assert np.array_equal(gotv[:L], w.value[w.cu_seq_lens[s]:w.cu_seq_lens[s + 1]])
    used = set(w.block_tables[:, 0].tolist())
    free = [b for b in range(w.num_blocks) if b not in used]
    for b in free:
        assert np.all(bits_of(d.kc[b]) == wl.nan_bits("bf16"))


FULL = {
    "decode_batch": wl.decode_batch,
    "chunked_prefill": wl.chunked_prefill,
    "long_block_causal": wl.long_block_causal,
}


@pytest.mark.parametrize("name", list(FULL))
def test_scatter_and_gather_full_size_bit_exact(gpu, name):
    """The full decode batch (about 140k tokens), chunked prefill and long block-causal
    (32768 tokens x 8 kv heads) caches: every byte of both caches equals the oracle's
    scatter model (written rows and the untouched NaN sentinels alike), and the exported
    gather of every sequence returns the generator's logical rows bit for bit."""
    w = FULL[name]()
    print(f"full-size scatter/gather: {name} tokens={w.key.shape[0]}", flush=True)
    d = Dev(w)
    d.write_all()
    torch.cuda.synchronize()
    ek, ev = _expected_cache(w)
    assert np.array_equal(bits_of(d.kc), ek)
    assert np.array_equal(bits_of(d.vc), ev)
    del ek, ev
    ko = torch.zeros_like(d.key)
    vo = torch.zeros_like(d.value)
    B.kv_cache_gather(ko, vo, d.cu_k, d.kc, d.vc, d.tables, w.max_seq_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(ko), w.key)
    assert np.array_equal(bits_of(vo), w.value)
