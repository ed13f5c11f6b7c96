"""Device copies of a generated workload and the library calls that run on them.

Used by the benchmark, the smoke run and the GPU tests.  It only uploads host arrays
(torch is the allocator) and forwards to the ctypes binding; it computes nothing.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import workloads as wl

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
INT_DT = {"f32": (torch.int32, np.int32), "f16": (torch.int16, np.int16), "bf16": (torch.int16, np.int16)}

# Bars for bf16/fp16 outputs against the fp64 oracle (max-abs, relative L2).


def to_dev(bits: np.ndarray, dtype: str, device="cuda"):
    tdt, ndt = INT_DT[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(ndt)).to(device).view(TORCH_DT[dtype])


def bits_of(t: torch.Tensor) -> np.ndarray:
    ndt = {torch.float32: np.uint32, torch.float16: np.uint16, torch.bfloat16: np.uint16}[t.dtype]
    idt = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}[t.dtype]
    return t.detach().contiguous().view(idt).cpu().numpy().view(ndt)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Dev:
    """Device copies of a workload plus a NaN-sentinel cache."""

    def __init__(self, w: wl.Workload, fill: str = "nan", combined: bool = False):
        self.w = w
        self.fp8 = getattr(w, "kv_dtype", None) == "fp8"
        dt = torch.uint8 if self.fp8 else TORCH_DT[w.dtype]     # FP8 caches hold E4M3 codes
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        if combined:
            # the (num_blocks, 2, block_size, Hkv, D) layout passed as two strided views
            base = torch.empty((w.num_blocks, 2) + shape[1:], dtype=dt, device="cuda")
            self.kc, self.vc = base[:, 0], base[:, 1]
        else:
            self.kc = torch.empty(shape, dtype=dt, device="cuda")
            self.vc = torch.empty(shape, dtype=dt, device="cuda")
        if fill == "nan":
            nan = 0x7F if self.fp8 else float("nan")
            self.kc.fill_(nan)
            self.vc.fill_(nan)
        else:
            self.kc.zero_()
            self.vc.zero_()
        self.query = to_dev(w.query, w.dtype)
        self.key = to_dev(w.key, w.dtype)
        self.value = to_dev(w.value, w.dtype)
        self.slots = torch.from_numpy(w.slots).cuda()
        self.tables = torch.from_numpy(w.block_tables).cuda()
        self.seq_lens = torch.from_numpy(w.seq_lens).cuda()
        self.cu_q = torch.from_numpy(w.cu_seqlens_q).cuda()
        self.cu_k = torch.from_numpy(w.cu_seq_lens).cuda()
        if w.spans is not None:
            fs, cs = w.span_arrays()
            self.full_spans = torch.from_numpy(np.ascontiguousarray(fs)).cuda()
            self.cu_spans = torch.from_numpy(cs).cuda()

    def write_all(self, split_new: bool = True):
        """Scatter every logical row into the cache: the cached context first, then the
        new tokens of this call (two kv_cache_write calls, as a serving step does)."""
        w = self.w
        if split_new:
            for rows in (w.context_rows(), w.new_token_rows()):
                if rows.size == 0:
                    continue
                idx = torch.from_numpy(rows).cuda()
                self.write(self.key[idx], self.value[idx], self.slots[idx])
        else:
            self.write(self.key, self.value, self.slots)

    def write(self, key, value, slots):
        if self.fp8:
            B.kv_cache_write_fp8(key, value, slots, self.kc, self.vc, self.w.k_scale, self.w.v_scale)
        else:
            B.kv_cache_write(key, value, slots, self.kc, self.vc)

    def decode(self, out=None):
        w = self.w
        out = out if out is not None else torch.empty_like(self.query)
        ws_bytes = B.decode_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                           w.max_seq_len)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        if self.fp8:
            B.paged_attention_decode_fp8(out, self.query, self.kc, self.vc, self.tables,
                                         self.seq_lens, w.scale, w.k_scale, w.v_scale,
                                         w.max_seq_len, ws if ws_bytes else None)
        else:
            B.paged_attention_decode(out, self.query, self.kc, self.vc, self.tables, self.seq_lens,
                                     w.scale, w.max_seq_len, ws if ws_bytes else None)
        return out

    def mixed(self, out=None, ws=None):
        """The whole batch through paged_attention_mixed (context sequences first)."""
        w = self.w
        nc = w.num_ctx_seqs
        out = out if out is not None else torch.empty_like(self.query)
        if ws is None:
            ws_bytes = B.mixed_workspace_size(w.num_seqs - nc, w.num_heads, w.num_kv_heads,
                                              w.head_dim, w.block_size, w.max_seq_len)
            ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
        ctx_q = int(w.q_lens[:nc].max()) if nc else 0
        B.paged_attention_mixed(out, self.query, self.cu_q[:nc + 1], self.seq_lens, self.kc,
                                self.vc, self.tables, w.scale, w.mask, w.span_len, ctx_q,
                                w.max_seq_len, nc, int(w.cu_seqlens_q[nc]), ws)
        return out

    def prefill(self, out=None):
        w = self.w
        out = out if out is not None else torch.empty_like(self.query)
        if self.fp8:
            B.paged_attention_prefill_fp8(out, self.query, self.cu_q, self.seq_lens, self.kc,
                                          self.vc, self.tables, w.scale, w.k_scale, w.v_scale,
                                          w.mask, w.span_len, w.max_q_len, w.max_seq_len)
        elif w.mask == wl.MASK_SPANS:
            B.paged_attention_prefill_spans(out, self.query, self.cu_q, self.seq_lens, self.kc,
                                            self.vc, self.tables, w.scale, self.full_spans,
                                            self.cu_spans, w.max_q_len, w.max_seq_len)
        else:
            B.paged_attention_prefill(out, self.query, self.cu_q, self.seq_lens, self.kc, self.vc,
                                      self.tables, w.scale, w.mask, w.span_len, w.max_q_len,
                                      w.max_seq_len)
        return out
