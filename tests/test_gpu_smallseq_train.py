"""Small-seq training path on the GPU: the forward with saved attention weights and the
backward (grad_V, grad_attn, softmax backward, grad_Q / grad_K) against the fp64 oracle.

Bars for the backward, derived from its arithmetic: the weights are stored in the query
type (relative rounding 2^-9 for bf16), products accumulate in fp32 and results are
rounded once more to the query type.  Simulating exactly that arithmetic on the
small-seq distribution gives max-abs 1.8e-2 and rel-L2 2.4e-3 against the exact
gradients, whose entries reach about 6; the bar is |got - want| <= 2e-2 + 1e-2 |want|
per element and rel-L2 <= 1e-2."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, bits_of, compare

pytestmark = pytest.mark.gpu

W_BAR = {"bf16": 4e-3, "f16": 1e-3}     # weights: half an ulp at 1 plus the fp32 softmax


def _grad_bar(got, want, what):
    assert np.all(np.isfinite(got)), what
    d = np.abs(got - want)
    worst = float(np.max(d - 1e-2 * np.abs(want))) if d.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert worst <= 2e-2 and rel <= 1e-2, f"{what}: excess {worst:.3e}, rel_l2 {rel:.3e}"


def _run(w, max_kv=16, check_seqs=None):
    d = Dev(w)
    d.write_all(split_new=False)
    S, H, D = w.num_seqs, w.num_heads, w.head_dim
    dt = d.query.dtype
    out = torch.empty_like(d.query)
    weights = torch.full((S, H, max_kv), float("nan"), dtype=dt, device="cuda")
    B.smallseq_attention_fwd(out, weights, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                             max_kv)
    d_out = torch.from_numpy(w.d_out.view(np.int16)).cuda().view(dt)
    dq = torch.full_like(d.query, float("nan"))
    dk = torch.full_like(d.key, float("nan"))
    dv = torch.full_like(d.value, float("nan"))
    B.smallseq_attention_bwd(dq, dk, dv, d_out, d.query, weights, d.kc, d.vc, d.tables,
                             d.seq_lens, d.cu_k, w.scale, max_kv)
    torch.cuda.synchronize()
    seqs = np.arange(S) if check_seqs is None else np.asarray(check_seqs)
    q = ref.widen(w.query, w.dtype)[seqs]
    keys_all = ref.split_logical(ref.widen(w.key, w.dtype), w.cu_seq_lens)
    vals_all = ref.split_logical(ref.widen(w.value, w.dtype), w.cu_seq_lens)
    keys = [keys_all[s] for s in seqs]
    vals = [vals_all[s] for s in seqs]
    g_out = ref.widen(w.d_out, w.dtype)[seqs]
    want_o, want_p = ref.smallseq_forward(q, keys, vals, w.num_kv_heads, w.scale, max_kv)
    want_dq, want_dk, want_dv = ref.smallseq_backward(q, keys, vals, g_out, w.num_kv_heads, w.scale)
    compare(as_f64(out)[seqs], want_o, w.dtype, "forward out")
    got_p = as_f64(weights)[seqs]
    assert np.max(np.abs(got_p - want_p)) <= W_BAR[w.dtype]
    for i, s in enumerate(seqs):
        assert np.all(got_p[i, :, int(w.seq_lens[s]):] == 0)
    _grad_bar(as_f64(dq)[seqs], want_dq, "dq")
    gk, gv = as_f64(dk), as_f64(dv)
    rows = np.concatenate([np.arange(w.cu_seq_lens[s], w.cu_seq_lens[s + 1]) for s in seqs])
    _grad_bar(gk[rows], np.concatenate(want_dk), "dk")
    _grad_bar(gv[rows], np.concatenate(want_dv), "dv")
    return dict(out=out, weights=weights, dq=dq, dk=dk, dv=dv, d=d)


@pytest.mark.timeout(400)
def test_smallseq_train_full_size_every_sequence(gpu):
    """30720 sequences with s_kv in {2..16}, 16 heads MHA, D 128: the forward output and
    weights and all three gradients of every sequence."""
    _run(wl.smallseq_train())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 64, 16])
def test_smallseq_train_dtypes_and_head_dims(gpu, dtype, D):
    _run(wl.smallseq_train(seed=20 + D, num_seqs=300, dtype=dtype, head_dim=D))


@pytest.mark.parametrize("H,Hkv", [(8, 2), (12, 3), (4, 1), (8, 4), (6, 3)])
def test_smallseq_train_gqa(gpu, H, Hkv):
    """Grouped heads: dK and dV sum over the heads of a kv head."""
    _run(wl.smallseq_train(seed=30 + H, num_seqs=200, num_heads=H, num_kv_heads=Hkv,
                           kv_choices=tuple(range(1, 17))))


def test_smallseq_train_short_rows_and_one_key(gpu):
    """Every length 1..16 with max_seq_len 16, then max_seq_len 5 with lengths 1..5 (a
    shorter weights row).  One key: P = 1 exactly, so dQ and dK are exactly zero and dV is
    d_out itself."""
    w = wl.smallseq_train(seed=40, num_seqs=160, kv_choices=tuple(range(1, 17)))
    r = _run(w)
    one = np.nonzero(w.seq_lens == 1)[0]
    assert one.size > 0
    assert np.all(as_f64(r["dq"])[one] == 0)
    rows = w.cu_seq_lens[one]
    assert np.all(as_f64(r["dk"])[rows] == 0)
    assert np.array_equal(bits_of(r["dv"])[rows], w.d_out[one].reshape(len(one), w.num_kv_heads, -1))
    _run(wl.smallseq_train(seed=41, num_seqs=100, kv_choices=(1, 2, 3, 4, 5)), max_kv=5)


def test_smallseq_train_rejects_bad_arguments(gpu):
    w = wl.smallseq_train(seed=42, num_seqs=8)
    d = Dev(w)
    out = torch.empty_like(d.query)
    weights = torch.empty((8, 16, 17), dtype=d.query.dtype, device="cuda")
    with pytest.raises(B.PkvError) as e:
        B.smallseq_attention_fwd(out, weights, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale, 17)
    assert e.value.code == B.PKV_ERR_INVALID_ARG
    q32 = d.query.float()
    with pytest.raises(B.PkvError) as e:
        B.smallseq_attention_fwd(q32.clone(), torch.empty((8, 16, 16), device="cuda"), q32, d.kc.float(),
                                 d.vc.float(), d.tables, d.seq_lens, w.scale, 16)
    assert e.value.code == B.PKV_ERR_UNSUPPORTED
