"""paged_attention_mixed on the GPU: context (chunked-prefill) rows and generation (decode)
rows of one step in one call, against the fp64 oracle over the whole THD batch."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, bits_of, compare

pytestmark = pytest.mark.gpu


def _run(w, rows=None):
    d = Dev(w)
    d.write_all()
    out = d.mixed()
    torch.cuda.synchronize()
    want, _ = ref.workload_attention(w, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got, want = got[rows], want[rows]
    compare(got, want, w.dtype, w.name)
    return d, out


def test_mixed_batch_full_size(gpu):
    """8 chunked-prefill sequences then 64 decode sequences (contexts up to 4096): every row."""
    _run(wl.mixed_batch())


@pytest.mark.parametrize("mask", [wl.MASK_NONE, wl.MASK_CAUSAL, wl.MASK_BLOCK_CAUSAL])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_mixed_masks_and_dtypes(gpu, mask, dtype):
    """bf16/fp16 take the one-launch path, fp32 the vector-ALU prefill plus decode."""
    w = wl.mixed_batch(seed=60 + mask, num_ctx=3, num_gen=9, ctx_hi=300, q_lo=1, q_hi=150,
                       lo=1, hi=700, dtype=dtype, mask=mask, span_len=48)
    _run(w)


@pytest.mark.parametrize("H,Hkv,D", [(8, 8, 128), (16, 8, 64), (12, 4, 128), (32, 4, 128),
                                     (8, 1, 64), (4, 2, 16)])
def test_mixed_gqa_and_head_dims(gpu, H, Hkv, D):
    """g = 1, 2, 3, 8 (decode waves hold at most 4 heads here), 8 (MQA), head_dim 16."""
    w = wl.mixed_batch(seed=70 + H + D, num_ctx=2, num_gen=7, ctx_hi=200, q_lo=20, q_hi=140,
                       lo=1, hi=1300, num_heads=H, num_kv_heads=Hkv, head_dim=D)
    _run(w)


def test_mixed_context_rows_equal_prefill_call_bit_for_bit(gpu):
    """The context rows come from the prefill kernel's own code with the same parameters."""
    w = wl.mixed_batch(seed=80, num_ctx=4, num_gen=20, ctx_hi=900, q_hi=300)
    d, out = _run(w)
    nc, T_ctx = w.num_ctx_seqs, int(w.cu_seqlens_q[w.num_ctx_seqs])
    ref_out = torch.zeros_like(d.query)
    B.paged_attention_prefill(ref_out[:T_ctx], d.query[:T_ctx], d.cu_q[:nc + 1], d.seq_lens[:nc],
                              d.kc, d.vc, d.tables[:nc], w.scale, w.mask, w.span_len,
                              int(w.q_lens[:nc].max()), w.max_seq_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out[:T_ctx]), bits_of(ref_out[:T_ctx]))


def test_mixed_only_context_or_only_generation(gpu):
    w = wl.mixed_batch(seed=81, num_ctx=3, num_gen=0, ctx_hi=500, q_hi=200)
    _run(w)
    w = wl.mixed_batch(seed=82, num_ctx=0, num_gen=30, lo=1, hi=3000)
    _run(w)


def test_mixed_empty_chunk_and_long_generation(gpu):
    """A context sequence with no new rows, one-key generation sequences and one with 40k
    keys (many splits and the merge)."""
    lens = np.array([300, 120, 40000, 1, 1, 700], np.int32)
    ql = np.array([40, 0, 1, 1, 1, 1], np.int32)
    w = wl.build("mixed_edges", 83, "bf16", lens, ql, 16, 4, 128, 16, wl.MASK_CAUSAL)
    w.num_ctx_seqs = 2
    _run(w)


def test_mixed_many_generation_items_grid_stride(gpu):
    """More decode items than the launch's decode blocks hold: the waves stride."""
    rng = np.random.default_rng(84)
    gl = rng.integers(1, 2000, size=1500).astype(np.int32)
    lens = np.concatenate([[600], gl]).astype(np.int32)
    ql = np.concatenate([[100], np.ones(1500, np.int32)]).astype(np.int32)
    w = wl.build("mixed_stride", 84, "bf16", lens, ql, 8, 8, 128, 16, wl.MASK_CAUSAL)
    w.num_ctx_seqs = 1
    rows = np.unique(np.concatenate([np.arange(110), rng.choice(w.num_tokens, 300, replace=False)]))
    _run(w, rows=rows)


def test_mixed_rejects_bad_boundary_and_workspace(gpu):
    w = wl.mixed_batch(seed=85, num_ctx=2, num_gen=5, ctx_hi=100, q_hi=50, lo=300, hi=2000)
    d = Dev(w)
    nc = w.num_ctx_seqs
    out = torch.full_like(d.query, 7.0)
    tc = int(w.cu_seqlens_q[nc])
    with pytest.raises(B.PkvError) as e:      # one generation row missing
        B.paged_attention_mixed(out, d.query, d.cu_q[:nc + 1], d.seq_lens, d.kc, d.vc, d.tables,
                                w.scale, w.mask, 0, 64, w.max_seq_len, nc, tc + 1)
    assert e.value.code == B.PKV_ERR_INVALID_ARG
    need = B.mixed_workspace_size(w.num_seqs - nc, w.num_heads, w.num_kv_heads, w.head_dim,
                                  w.block_size, w.max_seq_len)
    assert need > 0
    with pytest.raises(B.PkvError) as e:
        B.paged_attention_mixed(out, d.query, d.cu_q[:nc + 1], d.seq_lens, d.kc, d.vc, d.tables,
                                w.scale, w.mask, 0, 64, w.max_seq_len, nc, tc, None)
    assert e.value.code == B.PKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


@pytest.mark.parametrize("seed", range(10))
def test_mixed_random_shapes(gpu, seed):
    """Random steps: 0..4 context sequences (context 0..1200, chunks 1..300) then 0..300
    generation sequences of 1..6000 keys; GQA ratios, head_dim, pages, masks, spans and
    dtypes drawn; sampled rows (every context chunk's first and last) against the oracle."""
    rng = np.random.default_rng(900 + seed)
    nc = int(rng.integers(0, 5))
    ng = int(rng.choice([0, 1, 7, 64, 300])) if nc else int(rng.choice([1, 7, 64, 300]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    mask = int(rng.integers(0, 3))
    ql = rng.integers(1, 301, size=nc)
    ctx = rng.integers(0, 1201, size=nc)
    # at most ~40M cached generation K elements so the host-side generation stays quick
    gl = rng.integers(1, max(300, min(6000, 40_000_000 // (max(ng, 1) * Hkv * D))) + 1, size=ng)
    lens = np.concatenate([ctx + ql, gl]).astype(np.int32)
    qls = np.concatenate([ql, np.ones(ng, np.int64)]).astype(np.int32)
    w = wl.build(f"rand_mixed_{seed}", 900 + seed, dtype, lens, qls, g * Hkv, Hkv, D, bs, mask,
                 span_len=int(rng.choice([16, 48, 256])), scale=float(rng.uniform(0.05, 0.2)),
                 rng=rng)
    w.num_ctx_seqs = nc
    cu = w.cu_seqlens_q
    T = int(cu[-1])
    ends = np.concatenate([cu[:nc], cu[1:nc + 1] - 1])
    rows = np.unique(np.concatenate([ends, [T - 1], rng.choice(T, min(T, 200), replace=False)]))
    _run(w, rows=rows.astype(np.int64))
