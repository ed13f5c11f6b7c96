"""pkv_paged_attention_decode_noalloc on the GPU: the allocation-free decode (the library's
own per-GPU scratch array as workspace) against pkv_paged_attention_decode with a caller
workspace, and both against the fp64 oracle.

Two calls in a row, the second smaller, so that the second runs over what the first left
in the shared scratch array; the plain decode's workspace is filled with 0xFF bytes (NaN
floats) first, so neither result can lean on cleared memory.  The two entry points run the
same kernels, so their outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, bits_of, compare

pytestmark = pytest.mark.gpu


def _both(w):
    """(no-alloc output, caller-workspace output, the device copies)."""
    d = Dev(w)
    d.write_all()
    ws_bytes = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                       w.block_size, w.max_seq_len)
    ws = torch.full((max(ws_bytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    ref_out = torch.empty_like(d.query)
    B.paged_attention_decode(ref_out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                             w.max_seq_len, ws if ws_bytes else None)
    out = torch.full_like(d.query, float("nan"))
    B.paged_attention_decode_noalloc(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                     w.max_seq_len)
    torch.cuda.synchronize()
    return out, ref_out


def _check(w, rows=None):
    print(f"noalloc decode: {w.name} seqs={w.num_seqs} max_len={w.max_seq_len} dtype={w.dtype}",
          flush=True)
    out, ref_out = _both(w)
    assert np.array_equal(bits_of(out), bits_of(ref_out)), f"{w.name}: outputs differ"
    want, _ = ref.workload_attention(w, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got, want = got[rows], want[rows]
    compare(got, want, w.dtype, w.name)


def test_noalloc_decode_batch_then_smaller(gpu):
    """The decode batch (64 sequences of 256..4096 keys, stream mode with partials), then 9
    sequences of 100..2500 keys over the scratch the first call left behind."""
    _check(wl.decode_batch())
    _check(wl.decode_batch(seed=21, num_seqs=9, lo=100, hi=2500))


def test_noalloc_planning_tables_then_smaller(gpu):
    """300 sequences (beyond 256: the planning kernel writes its tables into the scratch),
    then 40 sequences (scanned, no tables) and an fp16 batch of 3."""
    w = wl.decode_batch(seed=22, num_seqs=300, lo=300, hi=1200)
    rows = np.sort(np.random.default_rng(3).choice(w.num_seqs, 48, replace=False))
    _check(w, rows=rows)
    _check(wl.decode_batch(seed=23, num_seqs=40, lo=50, hi=900))
    _check(wl.decode_batch(seed=24, num_seqs=3, lo=600, hi=3000, dtype="f16"))


def test_noalloc_one_split_needs_no_scratch(gpu):
    """Every sequence within one split (the small-seq shape): no partials at all."""
    _check(wl.smallseq_varlen(num_seqs=500))
