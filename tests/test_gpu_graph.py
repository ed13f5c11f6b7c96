"""The library under HIP graph capture (torch.cuda.CUDAGraph on ROCm): a serving step --
scatter of the new tokens, then decode -- and a prefill call, captured once and replayed
several times with eager work and synchronisations between the replays.  Every replay
must reproduce the eager result bit for bit (same kernels, same inputs): the calls
enqueue kernels only (no host synchronisation, no allocation, no memset), so they are
capturable."""
import numpy as np
import pytest
import torch

from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, bits_of

pytestmark = pytest.mark.gpu


def test_decode_step_replays_bit_exactly(gpu):
    _replay_decode_step(wl.decode_batch(seed=90, num_seqs=16, lo=200, hi=3000))


def test_decode_prefix_stream_step_replays_bit_exactly(gpu):
    """More than 256 sequences: the planning kernel is captured with the stream kernel
    and the merge."""
    lens = np.random.default_rng(92).integers(10, 600, size=1100).astype(np.int32)
    w = wl.build("graph_prefix", 92, "bf16", lens, np.ones(len(lens), np.int32), 8, 2, 128, 16,
                 wl.MASK_NONE, decode=True)
    _replay_decode_step(w)


def test_decode_few_long_sequences_step_replays_bit_exactly(gpu):
    """Two long sequences: the workgroup merge (LDS and a barrier) is captured with the
    stream kernel."""
    w = wl.build("graph_wide", 93, "bf16", np.array([9000, 15000], np.int32),
                 np.ones(2, np.int32), 32, 8, 128, 16, wl.MASK_NONE, decode=True)
    _replay_decode_step(w)


def _replay_decode_step(w):
    d = Dev(w, fill="zero")
    ctx = torch.from_numpy(w.context_rows()).cuda()
    B.kv_cache_write(d.key[ctx], d.value[ctx], d.slots[ctx], d.kc, d.vc)
    new = torch.from_numpy(w.new_token_rows()).cuda()
    nk, nv, ns = d.key[new].contiguous(), d.value[new].contiguous(), d.slots[new].contiguous()
    need = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                   w.block_size, w.max_seq_len)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(d.query)

    def step():
        B.kv_cache_write(nk, nv, ns, d.kc, d.vc)
        B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                 w.max_seq_len, ws if need else None)

    step()
    torch.cuda.synchronize()
    eager = bits_of(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), f"replay {i}"
        assert torch.isfinite(junk)


def test_prefill_replays_bit_exactly(gpu):
    w = wl.chunked_prefill(seed=91, num_seqs=3, ctx_hi=400, q_hi=200)
    d = Dev(w, fill="zero")
    d.write_all()
    out = torch.zeros_like(d.query)
    call = lambda: d.prefill(out)
    call()
    torch.cuda.synchronize()
    eager = bits_of(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), eager), f"replay {i}"
