"""Device-side precondition checks (pkv_set_device_checks / pkv_check_device_error).

Each invalid input below is backed by allocated memory (tables and caches carry slack
past what the call is told, the workspace is oversized), so even a check that failed
to fire could not make a kernel read or write outside an allocation."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev, as_f64, bits_of, compare

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks(gpu):
    B.set_device_checks(True)
    B.check_device_error()          # start from a clear word
    try:
        yield
    finally:
        B.set_device_checks(False)
        B.check_device_error()


def _decode_ws(w, max_seq_len=None, factor=1):
    need = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                   max_seq_len or w.max_seq_len)
    return need, torch.zeros(max(need * factor, 1), dtype=torch.uint8, device="cuda")


def test_checks_pass_and_change_nothing_on_valid_inputs(checks):
    """Valid calls with checks on: no bit set, outputs bit-identical to calls without."""
    w = wl.decode_batch(seed=50, num_seqs=6, lo=100, hi=3000)
    p = wl.chunked_prefill(seed=51, num_seqs=3, ctx_hi=300, q_hi=200)
    outs = []
    for on in (True, False):
        B.set_device_checks(on)
        dd, dp = Dev(w), Dev(p)
        dd.write_all()
        dp.write_all()
        od, op = dd.decode(), dp.prefill()
        kg = torch.empty_like(dp.key)
        vg = torch.empty_like(dp.value)
        B.kv_cache_gather(kg, vg, dp.cu_k, dp.kc, dp.vc, dp.tables, p.max_seq_len)
        torch.cuda.synchronize()
        outs.append((bits_of(od), bits_of(op), bits_of(kg), bits_of(vg)))
        if on:
            assert B.check_device_error() == (0, "")
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    B.set_device_checks(True)


def test_checks_flag_slot_out_of_range(checks):
    w = wl.random_small(3, "bf16", head_dim=64)
    d = Dev(w)
    slots = d.slots.clone()
    slots[-1] = w.num_blocks * w.block_size + 5
    B.kv_cache_write(d.key, d.value, slots, d.kc, d.vc)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_SLOT_RANGE and "slot_mapping" in msg
    assert torch.isnan(d.kc).all() and torch.isnan(d.vc).all()        # nothing written
    # the word was cleared by the read: a valid call works again
    B.kv_cache_write(d.key, d.value, d.slots, d.kc, d.vc)
    assert B.check_device_error() == (0, "")
    kg, vg = torch.empty_like(d.key), torch.empty_like(d.value)
    B.kv_cache_gather(kg, vg, d.cu_k, d.kc, d.vc, d.tables, w.max_seq_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(kg), bits_of(d.key)) and np.array_equal(bits_of(vg), bits_of(d.value))


def test_checks_flag_table_entry_and_stay_set_until_read(checks):
    """A block id one past the pool (two slack blocks are allocated behind it): flagged,
    the output is untouched, and a later valid call is a no-op until the word is read."""
    w = wl.decode_batch(seed=52, num_seqs=4, lo=200, hi=900)
    d = Dev(w)
    d.write_all()
    shape = (w.num_blocks + 2, w.block_size, w.num_kv_heads, w.head_dim)
    kbig = torch.zeros(shape, dtype=d.kc.dtype, device="cuda")
    vbig = torch.zeros(shape, dtype=d.vc.dtype, device="cuda")
    kbig[:w.num_blocks] = d.kc
    vbig[:w.num_blocks] = d.vc
    kc, vc = kbig[:w.num_blocks], vbig[:w.num_blocks]
    tables = d.tables.clone()
    tables[2, 1] = w.num_blocks
    need, ws = _decode_ws(w)
    out = torch.full_like(d.query, 3.0)
    B.paged_attention_decode(out, d.query, kc, vc, tables, d.seq_lens, w.scale, w.max_seq_len,
                             ws if need else None)
    # a valid call before the read: still guarded, writes nothing
    out2 = torch.full_like(d.query, 4.0)
    B.paged_attention_decode(out2, d.query, kc, vc, d.tables, d.seq_lens, w.scale, w.max_seq_len,
                             ws if need else None)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_TABLE and "block_tables" in msg
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(out2 == 4.0)
    B.paged_attention_decode(out2, d.query, kc, vc, d.tables, d.seq_lens, w.scale, w.max_seq_len,
                             ws if need else None)
    assert B.check_device_error() == (0, "")
    want, _ = ref.workload_attention(w)
    compare(as_f64(out2), want, w.dtype, "after clear")


def test_checks_flag_length_over_hint(checks):
    """seq_lens[1] = 1000 with max_seq_len = 900 (the table covers 1008 keys; the
    workspace is 4x the size the hint asks for)."""
    lens = np.array([300, 1000, 17, 700], np.int32)
    w = wl.build("over_hint", 53, "bf16", lens, np.ones(4, np.int32), 8, 2, 128, 16, wl.MASK_NONE,
                 decode=True, max_blocks_per_seq=63)
    d = Dev(w)
    d.write_all()
    need, ws = _decode_ws(w, max_seq_len=900, factor=4)
    out = torch.full_like(d.query, 2.0)
    B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale, 900,
                             ws if need else None)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_SEQ_LEN and "sequence length" in msg
    assert torch.all(out == 2.0)


def test_checks_flag_cu_seqlens_q(checks):
    """A decreasing cu_seqlens_q (a negative query segment) in prefill."""
    w = wl.chunked_prefill(seed=54, num_seqs=3, ctx_hi=200, q_lo=20, q_hi=60)
    d = Dev(w)
    d.write_all()
    cu = d.cu_q.clone()
    cu[1], cu[2] = cu[2], cu[1]
    out = torch.full_like(d.query, 5.0)
    B.paged_attention_prefill(out, d.query, cu, d.seq_lens, d.kc, d.vc, d.tables, w.scale, w.mask,
                              w.span_len, w.max_q_len, w.max_seq_len)
    bits, msg = B.check_device_error()
    assert bits & B.PKV_CHECK_CU_Q and "cu_seqlens_q" in msg
    assert torch.all(out == 5.0)


def test_checks_flag_length_over_table_capacity(checks):
    """The last sequence is 16 keys longer than max_blocks_per_seq * block_size; the
    table rows sit in a larger buffer, so the row after the last exists."""
    lens = np.array([100, 200, 256], np.int32)
    w = wl.build("over_cap", 55, "bf16", lens, lens, 8, 2, 128, 16, wl.MASK_CAUSAL)
    d = Dev(w)
    d.write_all()
    mb = d.tables.shape[1]
    buf = torch.zeros(d.tables.numel() + 4 * mb, dtype=torch.int32, device="cuda")
    buf[:d.tables.numel()] = d.tables.flatten()
    tables = buf[:d.tables.numel()].view(d.tables.shape)
    seq_lens = d.seq_lens.clone()
    seq_lens[2] = mb * w.block_size + 16
    out = torch.full_like(d.query, 6.0)
    B.paged_attention_prefill(out, d.query, d.cu_q, seq_lens, d.kc, d.vc, tables, w.scale, w.mask,
                              w.span_len, w.max_q_len, mb * w.block_size)
    bits, msg = B.check_device_error()
    assert bits & B.PKV_CHECK_SEQ_LEN
    assert torch.all(out == 6.0)


def test_checks_flag_unsorted_spans(checks):
    """Two spans of one sequence swapped (the offsets stay consistent, so every read stays
    inside the span array)."""
    w = wl.mixed_spans(seed=74, num_seqs=2, seq_len=300, text=(5, 30), image=(10, 60))
    d = Dev(w)
    d.write_all()
    fs = d.full_spans.clone()
    n0 = int(w.span_arrays()[1][0]), int(w.span_arrays()[1][1])
    assert n0[1] - n0[0] >= 2
    fs[[n0[0], n0[0] + 1]] = fs[[n0[0] + 1, n0[0]]]
    out = torch.full_like(d.query, 8.0)
    B.paged_attention_prefill_spans(out, d.query, d.cu_q, d.seq_lens, d.kc, d.vc, d.tables, w.scale,
                                    fs, d.cu_spans, w.max_q_len, w.max_seq_len)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_SPANS
    assert torch.all(out == 8.0)


def test_checks_cover_fp8_write(checks):
    """The quantising scatter takes the same slot check; nothing is written when it fails."""
    w = wl.with_fp8_cache(wl.random_small(4, "bf16", head_dim=64))
    d = Dev(w)
    slots = d.slots.clone()
    slots[0] = w.num_blocks * w.block_size
    B.kv_cache_write_fp8(d.key, d.value, slots, d.kc, d.vc, w.k_scale, w.v_scale)
    bits, _ = B.check_device_error()
    assert bits == B.PKV_CHECK_SLOT_RANGE
    torch.cuda.synchronize()
    assert bool(torch.all(d.kc == 0x7F)) and bool(torch.all(d.vc == 0x7F))


def test_checks_cover_mixed_batch(checks):
    """A generation sequence's block id one past the pool (two slack blocks behind it), then
    a context segment longer than its sequence: each flagged, the output untouched."""
    w = wl.mixed_batch(seed=56, num_ctx=2, num_gen=5, ctx_hi=200, q_lo=20, q_hi=80, lo=100, hi=600)
    d = Dev(w)
    d.write_all()
    shape = (w.num_blocks + 2, w.block_size, w.num_kv_heads, w.head_dim)
    kbig = torch.zeros(shape, dtype=d.kc.dtype, device="cuda")
    vbig = torch.zeros(shape, dtype=d.vc.dtype, device="cuda")
    kbig[:w.num_blocks] = d.kc
    vbig[:w.num_blocks] = d.vc
    d.kc, d.vc = kbig[:w.num_blocks], vbig[:w.num_blocks]
    d.tables[4, 0] = w.num_blocks
    out = torch.full_like(d.query, 6.0)
    d.mixed(out)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_TABLE and "block_tables" in msg
    torch.cuda.synchronize()
    assert bool(torch.all(out == 6.0))
    d.tables[4, 0] = int(w.block_tables[4, 0])
    d.seq_lens[0] = int(w.q_lens[0]) - 1          # fewer keys than the chunk's rows
    d.mixed(out)
    bits, msg = B.check_device_error()
    assert bits & B.PKV_CHECK_CU_Q
    torch.cuda.synchronize()
    assert bool(torch.all(out == 6.0))


def test_checks_cover_smallseq_backward(checks):
    """cu_seq_lens that disagree with seq_lens (dK / dV carry 32 slack rows): flagged, and
    the gradients stay untouched."""
    w = wl.smallseq_train(seed=57, num_seqs=20)
    d = Dev(w)
    d.write_all(split_new=False)
    dt = d.query.dtype
    weights = torch.zeros((20, 16, 16), dtype=dt, device="cuda")
    B.smallseq_attention_fwd(torch.empty_like(d.query), weights, d.query, d.kc, d.vc, d.tables,
                             d.seq_lens, w.scale, 16)
    assert B.check_device_error() == (0, "")
    cu = d.cu_k.clone()
    cu[5] += 1
    d_out = torch.from_numpy(w.d_out.view(np.int16)).cuda().view(dt)
    dq = torch.full_like(d.query, 8.0)
    dk = torch.full((w.key.shape[0] + 32,) + tuple(d.key.shape[1:]), 8.0, dtype=dt, device="cuda")
    dv = torch.full_like(dk, 8.0)
    B.smallseq_attention_bwd(dq, dk[:w.key.shape[0]], dv[:w.key.shape[0]], d_out, d.query, weights,
                             d.kc, d.vc, d.tables, d.seq_lens, cu, w.scale, 16)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_SEQ_LEN
    torch.cuda.synchronize()
    assert bool(torch.all(dq == 8.0)) and bool(torch.all(dk == 8.0)) and bool(torch.all(dv == 8.0))


def test_checks_flag_duplicate_slot(checks):
    """pkv_check_slots_unique before a write: unique slots (one padding token, slot -1) leave
    no bit; a slot held twice sets PKV_CHECK_DUP_SLOT and the guarded write after it writes
    nothing.  Every call leaves the bitmap all zero."""
    w = wl.random_small(5, "bf16", head_dim=64)
    d = Dev(w)
    nslots = w.num_blocks * w.block_size
    marks = torch.zeros((nslots + 31) // 32 + 3, dtype=torch.int32, device="cuda")
    slots = d.slots.clone()
    slots[0] = -1
    B.check_slots_unique(slots, w.num_blocks, w.block_size, marks)
    assert B.check_device_error() == (0, "")
    assert int(marks.count_nonzero()) == 0
    slots = d.slots.clone()
    slots[-1] = slots[len(slots) // 2]
    B.check_slots_unique(slots, w.num_blocks, w.block_size, marks)
    B.kv_cache_write(d.key, d.value, slots, d.kc, d.vc)
    bits, msg = B.check_device_error()
    assert bits == B.PKV_CHECK_DUP_SLOT and "twice" in msg
    torch.cuda.synchronize()
    assert int(marks.count_nonzero()) == 0
    assert torch.isnan(d.kc).all() and torch.isnan(d.vc).all()        # nothing written
    # with checks off the bit is still recorded, and read once
    B.set_device_checks(False)
    B.check_slots_unique(slots, w.num_blocks, w.block_size, marks)
    bits, _ = B.check_device_error()
    assert bits == B.PKV_CHECK_DUP_SLOT
    assert B.check_device_error() == (0, "")
    assert int(marks.count_nonzero()) == 0
