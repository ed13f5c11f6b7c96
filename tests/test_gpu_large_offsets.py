"""Cache byte offsets past 2^32: block pools larger than 4 GiB per cache tensor.

The sequences' blocks are drawn from a pool of about 150k blocks of 32 KB (bf16,
8 kv heads, head_dim 128, 16-token pages: 4.9 GB per tensor; FP8 pools are twice as
many blocks of half the size), so many of their rows lie beyond 4 GiB from the cache
base. Scatter, gather, decode and prefill all address those rows; every output is
compared with the oracle and the gather round trip is bit-exact."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, bits_of, compare

pytestmark = pytest.mark.gpu


def _block_bytes(w):
    elt = 1 if getattr(w, "kv_dtype", None) == "fp8" else 2
    return w.block_size * w.num_kv_heads * w.head_dim * elt


def _past_4gib(w):
    """Blocks the tables use whose first byte lies at or beyond 2^32 from the cache base."""
    used = np.concatenate([w.block_tables[s, :(int(w.seq_lens[s]) + w.block_size - 1) // w.block_size]
                           for s in range(w.num_seqs)])
    return int(np.sum(used.astype(np.int64) * _block_bytes(w) >= (1 << 32)))


def test_decode_blocks_past_4gib(gpu):
    w = wl.decode_batch(seed=30, num_seqs=16, spare_blocks=150000)
    n = _past_4gib(w)
    print(f"decode: pool {w.num_blocks} blocks, {n} used blocks past 4 GiB", flush=True)
    assert n > 100
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w)
    compare(as_f64(out), want, w.dtype, "decode, blocks past 4 GiB")
    del d, out
    torch.cuda.empty_cache()


def test_decode_fp8_blocks_past_4gib(gpu):
    w = wl.with_fp8_cache(wl.decode_batch(seed=31, num_seqs=16, spare_blocks=300000))
    n = _past_4gib(w)
    print(f"decode fp8: pool {w.num_blocks} blocks, {n} used blocks past 4 GiB", flush=True)
    assert n > 100
    d = Dev(w)
    d.write_all()
    out = d.decode()
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w)
    compare(as_f64(out), want, w.dtype, "FP8 decode, blocks past 4 GiB")
    del d, out
    torch.cuda.empty_cache()


def test_prefill_scatter_gather_blocks_past_4gib(gpu):
    w = wl.chunked_prefill(seed=32, num_seqs=4, spare_blocks=150000)
    n = _past_4gib(w)
    print(f"prefill: pool {w.num_blocks} blocks, {n} used blocks past 4 GiB", flush=True)
    assert n > 20
    d = Dev(w)
    d.write_all()
    out = d.prefill()
    ko = torch.zeros_like(d.key)
    vo = torch.zeros_like(d.value)
    B.kv_cache_gather(ko, vo, d.cu_k, d.kc, d.vc, d.tables, w.max_seq_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(ko), w.key) and np.array_equal(bits_of(vo), w.value)
    want, _ = ref.workload_attention(w)
    compare(as_f64(out), want, w.dtype, "prefill, blocks past 4 GiB")
    del d, out, ko, vo
    torch.cuda.empty_cache()
