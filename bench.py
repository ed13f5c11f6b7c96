#!/usr/bin/env python3
"""Throughput of paged-KV attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode_batch,...]

Default workload (the `value`): the decode batch -- 64 sequences with contexts
U[256, 4096], 32 query / 8 kv heads, head_dim 128, block_size 16, bf16.  One step is
one pass of the hot path over the batch: slot_mapping scatter of the 64 new K/V tokens
into the paged cache, then paged decode attention (block-table gather fused into its
loads, GQA by index, split-K with the log-sum-exp merge).  `value` is algorithmic bytes
per step (each K/V row of every sequence read once, Q read, O written, tables and
lengths, plus the scatter's reads and writes) over the measured step time.

The other workloads (chunked prefill, s_q=1 small-seq varlen, long block-causal
prefill, and prefill with general span lists) are measured with the same library and
reported in `workloads`.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
METRIC = "decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA peak); GPU vs CPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(w) -> int:
    """Algorithmic bytes of one decode launch: K and V rows of every sequence once, Q in,
    O out, the block-table entries used and the lengths."""
    import numpy as np
    eb = 2 if w.dtype != "f32" else 4
    cb = 1 if getattr(w, "kv_dtype", None) == "fp8" else eb      # cache element bytes
    L = w.seq_lens.astype(np.int64)
    kv = int(L.sum()) * w.num_kv_heads * w.head_dim * cb * 2
    qo = 2 * w.num_seqs * w.num_heads * w.head_dim * eb
    tables = int(((L + w.block_size - 1) // w.block_size).sum()) * 4
    return kv + qo + tables + w.num_seqs * 4


def scatter_bytes(w, rows) -> int:
    """K and V rows read in the source type and written in the cache type, plus slots."""
    eb = 2 if w.dtype != "f32" else 4
    cb = 1 if getattr(w, "kv_dtype", None) == "fp8" else eb
    return len(rows) * w.num_kv_heads * w.head_dim * (eb + cb) * 2 + len(rows) * 8


def prefill_flops(w) -> float:
    """4*D per visible (query, key) pair per head: QK^T and PV, masked pairs excluded."""
    import numpy as np
    tot = 0
    for s in range(w.num_seqs):
        L, q = int(w.seq_lens[s]), int(w.q_lens[s])
        a = np.arange(L - q, L, dtype=np.int64)
        if w.mask == 0:
            vis = np.full(q, L, np.int64)
        elif w.mask == 1:
            vis = np.minimum(L, a + 1)
        elif w.mask == 2:
            vis = np.minimum(L, (a // w.span_len + 1) * w.span_len)
        else:                               # span lists: up to the end of a's full span
            vis = a + 1
            for (b, e) in w.spans[s]:
                inside = (a >= b) & (a < e)
                vis = np.where(inside, e, vis)
            vis = np.minimum(L, vis)
        tot += int(vis.sum())
    return 4.0 * w.head_dim * w.num_heads * tot


def prefill_bytes(w) -> int:
    import numpy as np
    eb = 2 if w.dtype != "f32" else 4
    cb = 1 if getattr(w, "kv_dtype", None) == "fp8" else eb
    kv = int(w.seq_lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * cb * 2
    return kv + 2 * w.num_tokens * w.num_heads * w.head_dim * eb


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((e0, e))

    def ms(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.pairs]


def flush_llc(buf):
    """Read a 512 MB buffer so that neither L2 nor the 256 MB MALL hold the inputs.  A read
    (not a write) leaves clean lines behind: a rewrite would leave the caches full of dirty
    lines whose write-back the next kernel would pay for."""
    buf.sum()


def run_decode_step_bench(w, steps, warmup):
    """The default step: scatter the new tokens, then decode."""
    import numpy as np
    import torch
    from paged_kv_scaled_amd.harness import Dev
    from paged_kv_scaled_amd import binding as B

    d = Dev(w, fill="zero")
    ctx = w.context_rows()
    new = w.new_token_rows()
    ci = torch.from_numpy(ctx).cuda()
    B.kv_cache_write(d.key[ci], d.value[ci], d.slots[ci], d.kc, d.vc)      # untimed context
    ni = torch.from_numpy(new).cuda()
    nk, nv, ns = d.key[ni].contiguous(), d.value[ni].contiguous(), d.slots[ni].contiguous()
    out = torch.empty_like(d.query)
    wsb = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.max_seq_len)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def step(tw=None, ts=None):
        e0 = ts.start() if ts else None
        B.kv_cache_write(nk, nv, ns, d.kc, d.vc)
        e1 = tw.start() if tw else None
        B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                 w.max_seq_len, ws if wsb else None)
        if tw:
            tw.stop(e1)
            ts.stop(e0)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    # event-timed pass: per-launch decode durations and whole-step durations
    tw, ts = Timer(), Timer()
    for _ in range(steps):
        step(tw, ts)
    dec_ms = tw.ms()
    step_ms = ts.ms()
    # decode launches back to back between two events: the per-launch average without
    # the cost of an event pair around every launch
    tb = Timer()
    e = tb.start()
    for _ in range(steps):
        B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens, w.scale,
                                 w.max_seq_len, ws if wsb else None)
    tb.stop(e)
    dec_avg_ms = tb.ms()[0] / steps
    return dict(wall_ms=wall_ms, dec_ms=dec_ms, dec_avg_ms=dec_avg_ms, step_ms=step_ms,
                num_new=len(new), ws_bytes=wsb)


def run_attention_bench(w, kind, steps, warmup, flush=False):
    """Per-launch event timing of one attention entry point (cache written untimed)."""
    import torch
    from paged_kv_scaled_amd.harness import Dev
    from paged_kv_scaled_amd import binding as B

    d = Dev(w, fill="zero")
    d.write_all(split_new=False)
    out = torch.empty_like(d.query)
    if kind == "decode":
        wsb = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.max_seq_len)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        if d.fp8:
            call = lambda: B.paged_attention_decode_fp8(out, d.query, d.kc, d.vc, d.tables,
                                                        d.seq_lens, w.scale, w.k_scale, w.v_scale,
                                                        w.max_seq_len, ws if wsb else None)
        else:
            call = lambda: B.paged_attention_decode(out, d.query, d.kc, d.vc, d.tables, d.seq_lens,
                                                    w.scale, w.max_seq_len, ws if wsb else None)
    else:
        call = lambda: d.prefill(out)
    buf = torch.zeros(128 * 1024 * 1024, dtype=torch.float32, device="cuda") if flush else None
    for _ in range(warmup):
        call()
    tm = Timer()
    for _ in range(steps):
        if flush:
            flush_llc(buf)
        e = tm.start()
        call()
        tm.stop(e)
    ms = tm.ms()
    if kind == "decode":
        # the same launches back to back between one event pair (inputs may stay in the
        # caches between launches: reported beside the flushed figure, not instead of it)
        tb = Timer()
        e = tb.start()
        for _ in range(steps):
            call()
        tb.stop(e)
        ms_b2b = tb.ms()[0] / steps
        # an empty event pair: what the pair itself adds to a per-launch figure
        te = Timer()
        for _ in range(steps):
            e = te.start()
            te.stop(e)
        ms_pair = med(te.ms())
    else:
        ms_b2b = ms_pair = None
    # scatter of the whole batch as its own HBM workload
    ts = Timer()
    for _ in range(max(3, steps // 4)):
        e = ts.start()
        d.write(d.key, d.value, d.slots)
        ts.stop(e)
    return ms, ts.ms(), ms_b2b, ms_pair


def run_mixed_bench(w, steps, warmup):
    """The mixed batch through paged_attention_mixed (one call: the prefill launch over the
    context rows, then the decode launches over the generation rows) against the same rows
    as two calls (prefill of the context sequences, then decode of the generation
    sequences), both per step between event pairs, with the caches flushed from L2 and
    MALL before each step."""
    import torch
    from paged_kv_scaled_amd.harness import Dev
    from paged_kv_scaled_amd import binding as B

    d = Dev(w, fill="zero")
    d.write_all(split_new=False)
    nc = w.num_ctx_seqs
    tc = int(w.cu_seqlens_q[nc])
    ng = w.num_seqs - nc
    out = torch.empty_like(d.query)
    mb = B.mixed_workspace_size(ng, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.max_seq_len)
    mws = torch.zeros(max(mb, 1), dtype=torch.uint8, device="cuda")
    db = B.decode_workspace_size(ng, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.max_seq_len)
    dws = torch.zeros(max(db, 1), dtype=torch.uint8, device="cuda")
    ctx_q = int(w.q_lens[:nc].max())
    fused = lambda: d.mixed(out, mws if mb else None)

    def separate():
        B.paged_attention_prefill(out[:tc], d.query[:tc], d.cu_q[:nc + 1], d.seq_lens[:nc], d.kc, d.vc,
                                  d.tables[:nc], w.scale, w.mask, w.span_len, ctx_q, w.max_seq_len)
        B.paged_attention_decode(out[tc:], d.query[tc:], d.kc, d.vc, d.tables[nc:], d.seq_lens[nc:],
                                 w.scale, w.max_seq_len, dws if db else None)

    buf = torch.zeros(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
    calls = (("fused", fused), ("separate", separate))
    for _ in range(warmup):
        for _, call in calls:
            call()
    # the two forms alternate step by step, so that the clock's ramp under load (the
    # first launches of a run are slower) favours neither
    tms = {name: Timer() for name, _ in calls}
    for _ in range(steps):
        for name, call in calls:
            flush_llc(buf)
            e = tms[name].start()
            call()
            tms[name].stop(e)
    return {name: tm.ms() for name, tm in tms.items()}


def smallseq_train_bytes(w, max_kv=16):
    """Algorithmic bytes of the small-seq forward (K, V, Q in; O and the weights out) and
    backward (K, V, Q, dO and the weights in; dQ, dK, dV out), plus lengths and tables."""
    import numpy as np
    eb = 2
    kv = int(w.seq_lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * eb
    qrow = w.num_seqs * w.num_heads * w.head_dim * eb
    wts = w.num_seqs * w.num_heads * max_kv * eb
    meta = w.num_seqs * 4 * 2
    return 2 * kv + 2 * qrow + wts + meta, 2 * kv + 3 * qrow + wts + 2 * kv + meta + w.num_seqs * 4


def run_train_bench(w, steps, warmup, max_kv=16):
    """Per-launch event timing of the small-seq forward and backward (cache written untimed)."""
    import numpy as np
    import torch
    from paged_kv_scaled_amd.harness import Dev
    from paged_kv_scaled_amd import binding as B

    d = Dev(w, fill="zero")
    d.write_all(split_new=False)
    dt = d.query.dtype
    out = torch.empty_like(d.query)
    weights = torch.empty((w.num_seqs, w.num_heads, max_kv), dtype=dt, device="cuda")
    d_out = torch.from_numpy(w.d_out.view(np.int16)).cuda().view(dt)
    dq, dk, dv = torch.empty_like(d.query), torch.empty_like(d.key), torch.empty_like(d.value)
    fwd = lambda: B.smallseq_attention_fwd(out, weights, d.query, d.kc, d.vc, d.tables, d.seq_lens,
                                           w.scale, max_kv)
    bwd = lambda: B.smallseq_attention_bwd(dq, dk, dv, d_out, d.query, weights, d.kc, d.vc, d.tables,
                                           d.seq_lens, d.cu_k, w.scale, max_kv)
    res = {}
    for name, call in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(warmup):
            call()
        tm = Timer()
        for _ in range(steps):
            e = tm.start()
            call()
            tm.stop(e)
        res[name] = tm.ms()
    return res


def med(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def visible_keys_per_row(w):
    """Visible keys of every flat query row (the count the prefill flops are made of)."""
    import numpy as np
    out = np.zeros(w.num_tokens, np.int64)
    for s in range(w.num_seqs):
        L, q = int(w.seq_lens[s]), int(w.q_lens[s])
        a = np.arange(L - q, L, dtype=np.int64)
        if w.mask == 0:
            vis = np.full(q, L, np.int64)
        elif w.mask == 1:
            vis = np.minimum(L, a + 1)
        elif w.mask == 2:
            vis = np.minimum(L, (a // w.span_len + 1) * w.span_len)
        else:
            vis = a + 1
            for (b, e) in w.spans[s]:
                vis = np.where((a >= b) & (a < e), e, vis)
            vis = np.minimum(L, vis)
        r0 = int(w.cu_seqlens_q[s])
        out[r0:r0 + q] = vis
    return out


def _host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s=8.0):
    """The fp64 oracle as it stands, timed on the host cores of this machine.

    BLAS threads = the affinity count (the oracle's matrix products); its visibility
    matrices and per-row softmax are Python loops and run on one thread.  The widening
    of the storage bits to fp64 happens outside the timed region.

    Headline (the `value` of this entry, the unit of the benchmark's metric): whole passes
    over the decode batch (every sequence, every head) for about budget_s seconds,
    bytes counted as for the GPU figure.  per_config: the same oracle on the other
    workloads, each on a bounded sample (named in its entry) scaled to the workload's
    metric: the tiny prefill whole (and its brute-force scalar twin), sampled query rows
    of the chunked and long block-causal prefills (TFLOP/s of their visible pairs), a
    sample of the small-seq sequences (GB/s of their K/V, Q and O)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import reference as ref
    from paged_kv_scaled_amd import workloads as wl

    cores = len(os.sched_getaffinity(0))
    eb = 2 if w.dtype != "f32" else 4
    res = {"unit": "GB/s", "cores": cores, "kind": "oracle", "host_cpu": _host_cpu(),
           "threads_note": f"BLAS threads = {cores} (affinity count); the oracle's Python "
                           "loops (visibility, per-row softmax) run on one thread"}
    with threadpool_limits(limits=cores):
        # ---- decode batch (the headline): whole passes ------------------------------
        q = ref.widen(w.query, w.dtype)
        k = ref.split_logical(ref.widen(w.key, w.dtype), w.cu_seq_lens)
        v = ref.split_logical(ref.widen(w.value, w.dtype), w.cu_seq_lens)
        pass_bytes = (int(w.seq_lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * eb * 2
                      + 2 * w.num_tokens * w.num_heads * w.head_dim * eb)
        passes, t0 = 0, time.perf_counter()
        while True:
            ref.paged_attention(q, k, v, w.cu_seqlens_q, w.seq_lens, w.num_kv_heads, w.scale,
                                w.mask, w.span_len)
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        res.update(value=round(passes * pass_bytes / el / 1e9, 4),
                   sample=f"{passes} full passes over the decode batch ({w.num_seqs} sequences, "
                          f"{w.num_heads} heads), fp64 numpy, {el:.1f} s",
                   seconds=round(el, 2))
        per = {}
        # ---- tiny prefill: whole, and the brute-force twin ---------------------------
        t = wl.tiny_prefill()
        tq = ref.widen(t.query, t.dtype)
        tk = ref.split_logical(ref.widen(t.key, t.dtype), t.cu_seq_lens)
        tv = ref.split_logical(ref.widen(t.value, t.dtype), t.cu_seq_lens)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            ref.paged_attention(tq, tk, tv, t.cu_seqlens_q, t.seq_lens, t.num_kv_heads, t.scale, t.mask,
                                t.span_len)
            reps += 1
        vec_ms = (time.perf_counter() - t0) / reps * 1e3
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            ref.brute_force(tq, tk, tv, t.cu_seqlens_q, t.seq_lens, t.num_kv_heads, t.scale, t.mask,
                            t.span_len)
            reps += 1
        bf_ms = (time.perf_counter() - t0) / reps * 1e3
        per["tiny_prefill"] = {"value": round(vec_ms, 3), "unit": "ms per call",
                               "brute_force_ms": round(bf_ms, 3), "sample": "the whole workload"}
        # ---- prefill workloads: sampled query rows ----------------------------------
        for name, gen in (("chunked_prefill", wl.chunked_prefill), ("long_block_causal", wl.long_block_causal)):
            pw = gen()
            pq = ref.widen(pw.query, pw.dtype)
            pk = ref.split_logical(ref.widen(pw.key, pw.dtype), pw.cu_seq_lens)
            pv = ref.split_logical(ref.widen(pw.value, pw.dtype), pw.cu_seq_lens)
            vis = visible_keys_per_row(pw)
            # distinct random rows: a fixed permutation taken in growing chunks
            order = np.random.default_rng(11).permutation(pw.num_tokens)
            n, spent, flops, rows_done = 8, 0.0, 0.0, 0
            while spent < budget_s / 2 and rows_done < pw.num_tokens:
                rows = np.sort(order[rows_done:rows_done + n])
                t0 = time.perf_counter()
                ref.paged_attention(pq, pk, pv, pw.cu_seqlens_q, pw.seq_lens, pw.num_kv_heads, pw.scale,
                                    pw.mask, pw.span_len, rows=rows)
                spent += time.perf_counter() - t0
                flops += 4.0 * pw.head_dim * pw.num_heads * float(vis[rows].sum())
                rows_done += len(rows)
                n *= 2
            per[name] = {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s",
                         "sample": f"{rows_done} random query rows (all heads) of {pw.num_tokens}, "
                                   f"{spent:.1f} s", "seconds": round(spent, 2)}
            del pq, pk, pv
        # ---- small-seq: the first sequences ----------------------------------------
        sw = wl.smallseq_varlen()
        n, spent, by, seqs_done = 64, 0.0, 0, 0
        while spent < budget_s / 2 and seqs_done < sw.num_seqs:
            s0, s1 = seqs_done, min(seqs_done + n, sw.num_seqs)
            k0, k1 = int(sw.cu_seq_lens[s0]), int(sw.cu_seq_lens[s1])
            sq = ref.widen(sw.query[s0:s1], sw.dtype)
            sk = ref.split_logical(ref.widen(sw.key[k0:k1], sw.dtype), sw.cu_seq_lens[s0:s1 + 1] - k0)
            sv = ref.split_logical(ref.widen(sw.value[k0:k1], sw.dtype), sw.cu_seq_lens[s0:s1 + 1] - k0)
            t0 = time.perf_counter()
            ref.paged_attention(sq, sk, sv, np.arange(s1 - s0 + 1, dtype=np.int32), sw.seq_lens[s0:s1],
                                sw.num_kv_heads, sw.scale, sw.mask, sw.span_len)
            spent += time.perf_counter() - t0
            by += (k1 - k0) * sw.num_kv_heads * sw.head_dim * 2 * 2 + 2 * (s1 - s0) * sw.num_heads * sw.head_dim * 2
            seqs_done = s1
            n *= 2
        per["smallseq_varlen"] = {"value": round(by / spent / 1e9, 4), "unit": "GB/s",
                                  "sample": f"the first {seqs_done} of {sw.num_seqs} sequences, {spent:.1f} s",
                                  "seconds": round(spent, 2)}
        res["per_config"] = per
    return res


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size (torch's copy kernel), run so that a
    counter pass over this process sees FETCH_SIZE / WRITE_SIZE for nbytes read and
    nbytes written.  Returns the measured copy bandwidth (read + write bytes per s)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    tm = Timer()
    for _ in range(reps):
        e = tm.start()
        b.copy_(a)
        tm.stop(e)
    ms = med(tm.ms())
    del a, b
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def _ceilings_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_scaled_amd", "libpkv_ceilings.so"))
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.pkv_ceiling_stream_read.argtypes = [P, SZ, P, I, I, P]
    lib.pkv_ceiling_mfma.argtypes = [I, I, P, P, P]
    return lib


def stream_read_ceiling(nbytes=4 << 30, reps=4):
    """Achievable HBM read rate: the ceiling kernel streams a 4 GiB buffer (16x the MALL)
    with a small sweep of grid sizes and loads in flight; the best median is reported."""
    import ctypes
    import torch
    lib = _ceilings_lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    best = None
    for blocks in (2048, 4096, 8192):
        for unroll in (4, 8):
            sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
            tm = Timer()
            for _ in range(reps):
                e = tm.start()
                rc = lib.pkv_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes // 16,
                                                 ctypes.c_void_p(sink.data_ptr()), blocks, unroll, st)
                tm.stop(e)
                assert rc == 0, rc
            gbs = nbytes / (med(tm.ms()) * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, unroll)
    del buf
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "blocks": best[1], "loads_in_flight": best[2],
            "note": "plain streaming read of 4 GiB (16-byte nontemporal loads), best of a grid sweep"}


def mfma_ceiling(iters=4000, reps=3):
    """Achievable bf16 MFMA rate: back-to-back v_mfma_f32_32x32x16_bf16 on four independent
    accumulators, one workgroup of 4 waves per 256 threads; also the shader clock during
    the loop (its clock counter against the 100 MHz constant counter)."""
    import ctypes
    import torch
    lib = _ceilings_lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for blocks in (256, 512):   # one and two waves per SIMD
        sink = torch.zeros(blocks * 4, dtype=torch.float32, device="cuda")
        clk = torch.zeros(2, dtype=torch.int64, device="cuda")
        tm = Timer()
        for _ in range(reps):
            e = tm.start()
            rc = lib.pkv_ceiling_mfma(blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.c_void_p(clk.data_ptr()), st)
            tm.stop(e)
            assert rc == 0, rc
        ms = med(tm.ms())
        ticks, ref = (int(x) for x in clk.cpu().tolist())
        tf = blocks * 4 * iters * 4 * 32768.0 / (ms * 1e-3) / 1e12
        if best is None or tf > best[0]:
            best = (tf, blocks, ticks, ref)
    tf, blocks, ticks, ref = best
    ghz = ticks / (ref / 100e6) / 1e9 if ref > 0 else None
    return {"TFLOPs": round(tf, 1), "clock_GHz_during_loop": round(ghz, 3) if ghz else None,
            "cycles_per_mfma": round(ticks / (iters * 4), 2) if ticks else None,
            "TFLOPs_at_2.4GHz_equivalent": round(tf * 2.4 / ghz, 1) if ghz else None,
            "note": f"back-to-back 32x32x16 bf16 MFMAs, 4 accumulators per wave, {blocks} "
                    "workgroups of 4 waves (best of 1 and 2 waves per SIMD)"}


def device_info():
    """What the run was measured on (device properties; the clock under load is measured
    by the MFMA ceiling loop, not read from an idle DPM level)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count, "memory_GB": round(pr.total_memory / 1e9, 1)}


DECODE_SOURCES = ("decode_device.h", "decode_mfma.h", "decode.hip", "common.h")


def kernel_sources_sha(files=DECODE_SOURCES) -> str:
    """sha256 over the sources that make the decode kernels (in this order)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "paged_kv_scaled_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def committed_traffic(profile: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on the
    current decode kernel sources (their sha256 matches); else None."""
    import re
    prof = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(prof):
        return None
    text = open(prof).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_val) or m_sha.group(1) != kernel_sources_sha():
        return None
    return float(m_val.group(1))


def run_workloads(args, names):
    """Every named workload but the default decode step: one entry each."""
    import numpy as np
    import torch
    from paged_kv_scaled_amd import workloads as wl
    result_wl = {}
    for name in names:
        if name == "decode_batch":
            continue
        log(f"generating {name}")
        wk = wl.CONFIGS[name]()
        if wk.d_out is not None:
            rt = run_train_bench(wk, args.steps, args.warmup)
            fb, bb = smallseq_train_bytes(wk)
            fm, bm = med(rt["fwd"]), med(rt["bwd"])
            entry = {"metric": "small-seq training attention HBM GB/s", "unit": "GB/s",
                     "fwd_us_median": round(fm * 1e3, 2), "bwd_us_median": round(bm * 1e3, 2),
                     "fwd_GBps": round(fb / (fm * 1e-3) / 1e9, 1),
                     "bwd_GBps": round(bb / (bm * 1e-3) / 1e9, 1),
                     "fwd_frac_of_peak": round(fb / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "bwd_frac_of_peak": round(bb / (bm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "fwd_bytes": fb, "bwd_bytes": bb}
            log(f"{name}: {entry}")
            result_wl[name] = entry
            del wk
            torch.cuda.empty_cache()
            continue
        if wk.num_ctx_seqs is not None:
            rmx = run_mixed_bench(wk, args.steps, args.warmup)
            fm, sm = med(rmx["fused"]), med(rmx["separate"])
            nc = wk.num_ctx_seqs
            entry = {"metric": "mixed step attention us (one call vs two)", "unit": "us",
                     "launch_us_median": round(fm * 1e3, 2), "launch_us_min": round(min(rmx["fused"]) * 1e3, 2),
                     "separate_calls_us_median": round(sm * 1e3, 2),
                     "speedup_vs_separate": round(sm / fm, 3),
                     "ctx_seqs": nc, "gen_seqs": wk.num_seqs - nc,
                     "ctx_rows": int(wk.cu_seqlens_q[nc])}
            log(f"{name}: {entry}")
            result_wl[name] = entry
            del wk
            torch.cuda.empty_cache()
            continue
        kind = "decode" if wk.decode else "prefill"
        # every launch timed after a 512 MB rewrite, so that neither L2 nor the MALL
        # holds its inputs
        ms, sc_ms, ms_b2b, ms_pair = run_attention_bench(wk, kind, args.steps, args.warmup, flush=True)
        m = med(ms)
        entry = {"launch_us_median": round(m * 1e3, 2), "launch_us_min": round(min(ms) * 1e3, 2),
                 "flushed": True}
        if kind == "decode":
            by = decode_bytes(wk)
            entry.update(metric="decode attn HBM GB/s", value=round(by / (m * 1e-3) / 1e9, 1),
                         unit="GB/s", frac_of_peak=round(by / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         bytes_per_launch=by,
                         event_pair_us=round(ms_pair * 1e3, 2),
                         back_to_back_us=round(ms_b2b * 1e3, 2),
                         back_to_back_GBps=round(by / (ms_b2b * 1e-3) / 1e9, 1))
        else:
            fl = prefill_flops(wk)
            tf = fl / (m * 1e-3) / 1e12
            entry.update(metric="prefill attn TFLOP/s", value=round(tf, 2), unit="TFLOP/s",
                         frac_of_peak=round(tf / BF16_PEAK_TFLOPS, 4), flops_per_launch=fl,
                         bytes_min=prefill_bytes(wk))
        sb = scatter_bytes(wk, np.arange(wk.key.shape[0]))
        entry["scatter_GBps"] = round(sb / (med(sc_ms) * 1e-3) / 1e9, 1)
        log(f"{name}: {entry}")
        result_wl[name] = entry
        del wk
        torch.cuda.empty_cache()

    return result_wl


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads",
                    default="decode_batch,smallseq_varlen,chunked_prefill,long_block_causal,mixed_spans,"
                            "decode_batch_fp8,decode_long_seq,mixed_batch,smallseq_train")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="kept for old command lines: the 1 GiB device copy (the reference kernel "
                         "of the counter passes) now always runs")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured streaming-read and MFMA-loop ceilings")
    ap.add_argument("--workloads-only", action="store_true",
                    help="profiling runs: skip the default decode step (and the ceilings and "
                         "the CPU baseline) and print only the per-workload entries")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_kv_scaled_amd import binding as B
    from paged_kv_scaled_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    B.load()
    names = [n for n in args.workloads.split(",") if n]

    if args.workloads_only:
        result_wl = run_workloads(args, names)
        print(json.dumps({"workloads": result_wl}), flush=True)
        return

    # ---- default workload: decode batch step -------------------------------------------
    log("generating decode_batch")
    w = wl.decode_batch()
    r = run_decode_step_bench(w, args.steps, args.warmup)
    dbytes = decode_bytes(w)
    sbytes = scatter_bytes(w, w.new_token_rows())
    step_bytes = dbytes + sbytes
    ms_step = r["wall_ms"] / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dec_ms = r["dec_avg_ms"]
    achieved = dbytes / (dec_ms * 1e-3) / 1e9
    log(f"decode_batch: step {ms_step*1e3:.1f} us, decode launch {dec_ms*1e3:.1f} us "
        f"(back to back; {med(r['dec_ms'])*1e3:.1f} us with an event pair around each), "
        f"{achieved:.0f} GB/s ({achieved/HBM_PEAK_GBS*100:.1f}% of HBM peak)")
    traffic = committed_traffic("decode_batch_traffic.md")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "paged_attention_decode (decode_stream_kernel + decode_merge_stream_kernel)",
                "bytes_per_launch": dbytes, "launch_us_avg": round(dec_ms * 1e3, 2),
                "launch_us_median_event_pair": round(med(r["dec_ms"]) * 1e3, 2)}

    result_wl = run_workloads(args, names)

    copy_gbs = copy_calibration()
    ceil = None
    if not args.no_ceilings:
        log("measuring the ceilings")
        ceil = {"hbm_read": stream_read_ceiling(), "mfma_bf16": mfma_ceiling()}
        roofline["frac_of_measured_read_ceiling"] = round(achieved / ceil["hbm_read"]["GBps"], 4)
        for name, e in result_wl.items():
            if e.get("unit") == "TFLOP/s":
                e["frac_of_measured_mfma_ceiling"] = round(e["value"] / ceil["mfma_bf16"]["TFLOPs"], 4)
            elif e.get("metric", "").startswith("decode") and e.get("value"):
                e["frac_of_measured_read_ceiling"] = round(e["value"] / ceil["hbm_read"]["GBps"], 4)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(w, args.cpu_seconds)
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1) if cpu["value"] > 0 else None
        for name, e in cpu["per_config"].items():
            g = result_wl.get(name)
            if g and g.get("unit") == e["unit"] and e["value"] > 0:
                e["gpu_over_cpu"] = round(g["value"] / e["value"], 1)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, shuffled block pool)",
        "config": {"workload": "decode_batch", "num_seqs": 64, "context": "U[256,4096]",
                   "num_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "seed": 1, "sum_seq_lens": int(w.seq_lens.sum()),
                   "step": "kv_cache_write(64 new tokens) + paged_attention_decode",
                   "bytes_per_step": step_bytes, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": result_wl,
        "step_us_event_median": round(med(r["step_ms"]) * 1e3, 2),
    }
    line["ceilings"] = dict(ceil or {}, hbm_spec_GBps=HBM_PEAK_GBS, bf16_spec_TFLOPs=BF16_PEAK_TFLOPS,
                            counter_calibration_copy_GBps=copy_gbs,
                            counter_calibration_note="1 GiB device copy (read + write bytes): the "
                            "reference kernel of the FETCH_SIZE / WRITE_SIZE calibration")
    line["device"] = device_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
