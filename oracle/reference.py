"""fp64 CPU oracle for paged-KV scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or tables) and never reads
anything the GPU produced: attention is computed from the logical per-sequence
K/V rows as the input generator drew them, not from the paged cache or a block
table (the independence rule of the CSA2 Vanilla golden PR, "Description":
geometry from independent sources; the golden never reads kernel-produced
slot or page tables).

Everything is float64.  Inputs arrive as raw storage bits and are widened
exactly (bf16 -> f32 is a 16-bit shift; f16 and f32 widen exactly to f64).

What the method computes (the Spyre paged-attention PR, "Description", six
steps; the vllm-omni piecewise block-causal PR for the block-causal mask):
  scatter  : cache[slot // B][slot % B] = new row, raw copy, slot < 0 skipped
  gather   : logical row p of sequence s = cache[table[s][p // B]][p % B]
  positions: query row i of a chunk of q_s new tokens sits at a = (L_s - q_s) + i
  visible  : key p < L_s and   NONE: always
                               CAUSAL: p <= a (bottom-right aligned)
                               BLOCK_CAUSAL(span): p <= a or p // span == a // span
                               SPANS(full spans): p <= a or p and a inside one full span
  scores   : z_p = scale * <q, k_p>, q head h reads kv head h // (H / Hkv)
  softmax  : stable: m = max z, w = exp(z - m), out = sum w v / sum w, lse = m + log sum w
  empty row: no visible key -> out = 0, lse = -inf
  small-seq training path (ROCm TransformerEngine small-seq PR): the forward also returns
  the attention weights P; the backward is the gradient of sum(d_out * out) taken in the
  pages' steps (grad_V, grad_attn, softmax backward, grad_Q / grad_K)

Parity status of each function is stated in its docstring; every function here
is pinned by `tests/test_oracle_pins.py` against something other than itself.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_BLOCK_CAUSAL, MASK_SPANS = 0, 1, 2, 3


# ----------------------------------------------------------------------------------------
# exact widening of storage bits
# ----------------------------------------------------------------------------------------

def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits -> float64, exactly (no rounding happens in any branch)."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------
# FP8 (E4M3) KV cache: quantisation and dequantisation (the FP8 KV-cache row after the five
# shapes; the pages name FP8 paths but no scale convention, so the convention is a reading:
# one float scale per tensor, code = E4M3(round(clamp(x * (1/scale)))), value = code * scale)
# ----------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one OCP 8-bit floating-point E4M3 code: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; no infinities; the codes
    with all exponent and mantissa bits set are NaN."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_MAGS = np.array([e4m3_value(c) for c in range(0x7F)])   # codes 0x00..0x7E, increasing


def quantize_e4m3(x: np.ndarray, inv_scale: np.float32) -> np.ndarray:
    """uint8 codes of float values x (finite): y = float32(float32(x) * inv_scale) (one
    rounded product), clamped to [-448, 448], then the nearest E4M3 value, a tie going to
    the even code; the sign of y (zero included) becomes the sign bit."""
    y = (np.asarray(x, np.float32) * np.float32(inv_scale)).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    a = np.abs(y).astype(np.float64).ravel()
    hi = np.clip(np.searchsorted(_E4M3_MAGS, a), 0, len(_E4M3_MAGS) - 1)   # first mag >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y.ravel()), code | np.uint8(0x80), code).astype(np.uint8)
    return code.reshape(np.shape(y))


def dequantize_e4m3(codes: np.ndarray, scale: float) -> np.ndarray:
    """float64 values of E4M3 codes times the tensor scale (exact: every code value is a
    float64 and the product of two such values with <= 24 significant bits is exact)."""
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, np.int64)] * float(scale)


# ----------------------------------------------------------------------------------------
# step 1: slot_mapping scatter (raw copy) -- Spyre PR, "Description", step 1
# ----------------------------------------------------------------------------------------

def kv_cache_write(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                   value: np.ndarray, slot_mapping: np.ndarray, block_size: int):
    """Return copies of the caches [NB, B, Hkv, D] with each token's row written at its slot.

    A negative slot marks a padding token and is skipped (reading A1).  Slots must be
    unique within one call and inside the pool.  Untouched slots keep their old bits.
    """
    kc, vc = key_cache.copy(), value_cache.copy()
    nb = kc.shape[0]
    seen = set()
    for t in range(slot_mapping.shape[0]):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        assert slot < nb * block_size, "slot outside the block pool"
        assert slot not in seen, "duplicate slot within one call"
        seen.add(slot)
        blk, off = slot // block_size, slot % block_size
        kc[blk, off] = key[t]
        vc[blk, off] = value[t]
    return kc, vc


# ----------------------------------------------------------------------------------------
# step 2: block-table gather -- Spyre PR, "Description", step 2
# ----------------------------------------------------------------------------------------

def gather_sequence(cache: np.ndarray, table_row: np.ndarray, seq_len: int, block_size: int):
    """Logical rows 0..L-1 of one sequence: row p lives in block table_row[p // B], slot p % B."""
    out = np.empty((seq_len,) + cache.shape[2:], cache.dtype)
    for p in range(seq_len):
        out[p] = cache[int(table_row[p // block_size]), p % block_size]
    return out


# ----------------------------------------------------------------------------------------
# steps 3-6: masked, scaled, stable-softmax attention per sequence
# ----------------------------------------------------------------------------------------

def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Query head h reads the kv head that repeat_interleave would have copied into slot h
    (Spyre PR, "Description": GQA by repeat_interleave on the KV heads)."""
    group = num_heads // num_kv_heads
    return h // group


def is_visible(p: int, a: int, seq_len: int, mask: int, span_len: int) -> bool:
    """Key position p is visible to the query at absolute position a.

    CAUSAL is bottom-right aligned (vllm-omni piecewise PR: rightDownCausal contract,
    Sq <= Skv); BLOCK_CAUSAL is the dense `(q >= kv) or same block` rule of that PR's
    reference, with blocks tiling absolute positions from 0 in steps of span_len.
    """
    if p >= seq_len:
        return False
    if mask == MASK_NONE:
        return True
    if mask == MASK_CAUSAL:
        return p <= a
    if mask == MASK_BLOCK_CAUSAL:
        return p <= a or (p // span_len) == (a // span_len)
    raise ValueError(mask)


def full_span_of(pos: int, full_spans) -> Optional[int]:
    """Index of the full span [start, end) of the list that holds position pos, else None."""
    for i, (s, e) in enumerate(full_spans):
        if s <= pos < e:
            return i
    return None


def span_visible(p: int, a: int, seq_len: int, full_spans) -> bool:
    """SPANS mask: general span lists (the `full_attn_spans` metadata of the vllm-omni
    piecewise PR).  Key p is visible to the query at absolute position a when p < L and
    either p <= a, or p and a lie in the same full (image) span; positions outside every
    full span form causal text runs.  This is that PR's dense reference,
    `(q >= kv) or same_image_block`, with the image blocks given by the list."""
    if p >= seq_len:
        return False
    if p <= a:
        return True
    i = full_span_of(a, full_spans)
    return i is not None and i == full_span_of(p, full_spans)


def visibility_matrix(positions: np.ndarray, seq_len: int, mask: int, span_len: int,
                      full_spans=None):
    """Boolean [len(positions), seq_len] matrix of is_visible (or, for SPANS, of
    span_visible over this sequence's full spans).

    The same rules as is_visible / span_visible, written over whole index grids (query
    position a down the rows, key position p across the columns) so that long sequences
    are feasible: NONE every p < L; CAUSAL p <= a; BLOCK_CAUSAL p <= a or p // span ==
    a // span (the piecewise PR's dense reference); SPANS p <= a, or p and a inside the
    same full span.  tests/test_oracle_pins.py holds it equal to the scalar rules entry
    by entry."""
    a = np.asarray(positions, np.int64).reshape(-1, 1)
    p = np.arange(seq_len, dtype=np.int64).reshape(1, -1)
    if mask == MASK_NONE:
        return np.ones((a.shape[0], seq_len), bool)
    if mask == MASK_CAUSAL:
        return p <= a
    if mask == MASK_BLOCK_CAUSAL:
        return (p <= a) | ((p // span_len) == (a // span_len))
    if mask == MASK_SPANS:
        vis = p <= a
        for (b, e) in (full_spans or []):
            vis |= ((a >= b) & (a < e)) & ((p >= b) & (p < e))
        return vis
    raise ValueError(mask)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray, scale: float):
    """One sequence, one query head: q [n, D], k/v [L, D], vis [n, L] -> out [n, D], lse [n].

    Only the keys some row sees and the rows that see some key take part (a key no row
    sees is dropped whatever it holds).  z = scale * q k^T over them (a matmul as a
    library step); a key a row cannot see gets -inf, so its weight below is exactly 0;
    then the stable softmax row by row: subtract the row max over the visible keys,
    exponentiate, normalise, and the weighted sum of the value rows (a matmul).  A row
    with no visible key gives zeros and lse = -inf (reading A6).
    """
    n, D = q.shape
    out = np.zeros((n, v.shape[1]), np.float64)
    lse = np.full(n, -np.inf)
    if n == 0 or k.shape[0] == 0:
        return out, lse
    rows = vis.any(axis=1)
    cols = vis.any(axis=0)
    if not rows.any():
        return out, lse
    sub = vis[rows][:, cols]
    z = np.where(sub, scale * (q[rows] @ k[cols].T), -np.inf)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)                 # exp(-inf) = 0: keys the row cannot see weigh nothing
    l = w.sum(axis=1)
    out[rows] = (w @ v[cols]) / l[:, None]
    lse[rows] = m[:, 0] + np.log(l)
    return out, lse


def paged_attention(query: np.ndarray, keys: Sequence[np.ndarray], values: Sequence[np.ndarray],
                    cu_seqlens_q: np.ndarray, seq_lens: np.ndarray, num_kv_heads: int,
                    scale: float, mask: int, span_len: int = 0,
                    rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
                    spans: Optional[Sequence] = None):
    """Attention of a flat (THD) query batch over per-sequence logical K/V.

    query [T, H, D] float64; keys[s], values[s] [L_s, Hkv, D] float64.  Sequence s owns
    query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, which are its newest tokens, so
    row i of the chunk sits at absolute position a = L_s - q_s + i (chunked prefill;
    decode is the case q_s = 1).  Returns out [T, H, D] and lse [T, H]; with `rows`
    (flat row indices) / `heads` given, only those entries are computed (the rest stay
    zero / -inf) so that large batches can be sampled.  For the SPANS mask, spans[s]
    lists the (start, end) full spans of sequence s in absolute positions.
    """
    T, H, D = query.shape
    out = np.zeros((T, H, values[0].shape[-1] if len(values) else D), np.float64)
    lse = np.full((T, H), -np.inf)
    want_rows = None if rows is None else set(int(r) for r in rows)
    head_list = range(H) if heads is None else [int(h) for h in heads]
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        r0, r1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        q_s = r1 - r0
        ctx = L - q_s
        assert ctx >= 0, "a query chunk longer than its sequence"
        row_ids = [r for r in range(r0, r1) if want_rows is None or r in want_rows]
        if not row_ids:
            continue
        positions = np.array([ctx + (r - r0) for r in row_ids], np.int64)
        vis = visibility_matrix(positions, L, mask, span_len,
                                spans[s] if mask == MASK_SPANS else None)
        for h in head_list:
            kvh = kv_head_of(h, H, num_kv_heads)
            o, l = attend(query[row_ids, h, :], keys[s][:, kvh, :], values[s][:, kvh, :], vis, scale)
            out[row_ids, h, :] = o
            lse[row_ids, h] = l
    return out, lse


def split_logical(rows: np.ndarray, cu_seq_lens: np.ndarray):
    """Per-sequence views of a sequence-major row array [sum L, ...]."""
    return [rows[cu_seq_lens[s]:cu_seq_lens[s + 1]] for s in range(len(cu_seq_lens) - 1)]


def workload_kv(w):
    """Logical K and V rows of a workload as float64: the drawn values, or, for an FP8
    cache, what the cache holds: the quantised codes times the scales."""
    k, v = widen(w.key, w.dtype), widen(w.value, w.dtype)
    if getattr(w, "kv_dtype", None) == "fp8":
        k = dequantize_e4m3(quantize_e4m3(k, np.float32(1) / np.float32(w.k_scale)), np.float32(w.k_scale))
        v = dequantize_e4m3(quantize_e4m3(v, np.float32(1) / np.float32(w.v_scale)), np.float32(w.v_scale))
    return k, v


def workload_attention(w, rows=None, heads=None):
    """Oracle output for a generated workload (float64), from its logical K/V."""
    q = widen(w.query, w.dtype)
    kk, vv = workload_kv(w)
    k = split_logical(kk, w.cu_seq_lens)
    v = split_logical(vv, w.cu_seq_lens)
    return paged_attention(q, k, v, w.cu_seqlens_q, w.seq_lens, w.num_kv_heads, w.scale,
                           w.mask, w.span_len, rows=rows, heads=heads,
                           spans=getattr(w, "spans", None))


# ----------------------------------------------------------------------------------------
# small-seq training path: attention weights and the backward pass (ROCm TransformerEngine
# small-seq PR, description: the forward writes the attention weights for s_q = 1 and
# s_kv <= 16, the backward reads them and computes grad_V, grad_attn, the softmax backward
# and grad_Q / grad_K).  The backward is the gradient of sum(d_out * out).
# ----------------------------------------------------------------------------------------

def smallseq_forward(q: np.ndarray, keys: Sequence[np.ndarray], values: Sequence[np.ndarray],
                     num_kv_heads: int, scale: float, max_kv: Optional[int] = None):
    """One query row per sequence.  q [S, H, D]; keys[s], values[s] [L_s, Hkv, D].

    Returns out [S, H, D] and the attention weights P [S, H, max_kv]:
    P[s, h, k] = softmax over k < L_s of scale <q[s, h], K_s[k, h // g]>, zero for
    k >= L_s (an empty sequence has an all-zero row and a zero output)."""
    S, H, D = q.shape
    if max_kv is None:
        max_kv = max([int(k.shape[0]) for k in keys] + [1])
    out = np.zeros((S, H, values[0].shape[-1] if len(values) else D), np.float64)
    P = np.zeros((S, H, max_kv), np.float64)
    for s in range(S):
        L = int(keys[s].shape[0])
        if L == 0:
            continue
        for h in range(H):
            kvh = kv_head_of(h, H, num_kv_heads)
            z = scale * (keys[s][:, kvh, :] @ q[s, h])
            w = np.exp(z - z.max())
            P[s, h, :L] = w / w.sum()
            out[s, h] = P[s, h, :L] @ values[s][:, kvh, :]
    return out, P


def smallseq_backward(q: np.ndarray, keys: Sequence[np.ndarray], values: Sequence[np.ndarray],
                      d_out: np.ndarray, num_kv_heads: int, scale: float):
    """Gradients of sum(d_out * out) for smallseq_forward, in the pages' four steps, from
    the exact attention weights P (query head h of kv head j = h // g):
      grad_V      dV[k, j] = sum over h of j of P[h, k] dO[h]
      grad_attn   dP[h, k] = <dO[h], V[k, j]>
      softmax bwd dS[h, k] = P[h, k] (dP[h, k] - sum_k' P[h, k'] dP[h, k'])
      grad_Q      dQ[h]    = scale sum_k dS[h, k] K[k, j]
      grad_K      dK[k, j] = scale sum over h of j of dS[h, k] q[h]
    Returns dq [S, H, D] and per-sequence dk[s], dv[s] [L_s, Hkv, D]."""
    S, H, D = q.shape
    _, P = smallseq_forward(q, keys, values, num_kv_heads, scale)
    dq = np.zeros_like(q, dtype=np.float64)
    dk = [np.zeros(k.shape, np.float64) for k in keys]
    dv = [np.zeros(v.shape, np.float64) for v in values]
    for s in range(S):
        L = int(keys[s].shape[0])
        if L == 0:
            continue
        for h in range(H):
            kvh = kv_head_of(h, H, num_kv_heads)
            p = P[s, h, :L]
            dv[s][:, kvh, :] += np.outer(p, d_out[s, h])                       # grad_V
            dp = values[s][:, kvh, :] @ d_out[s, h]                            # grad_attn
            ds = p * (dp - p @ dp)                                             # softmax bwd
            dq[s, h] = scale * (ds @ keys[s][:, kvh, :])                       # grad_Q
            dk[s][:, kvh, :] += scale * np.outer(ds, q[s, h])                  # grad_K
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# cross-split merge by log-sum-exp (the flash-decoding combine)
# ----------------------------------------------------------------------------------------

def lse_merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine attention results over disjoint key subsets: weights exp(lse_j - max lse)."""
    lses = np.stack(lses)            # [J, ...]
    outs = np.stack(outs)            # [J, ..., D]
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Msafe), 0.0)
    tot = w.sum(axis=0)
    num = (w[..., None] * outs).sum(axis=0)
    out = np.where(tot[..., None] > 0, num / np.where(tot > 0, tot, 1.0)[..., None], 0.0)
    lse = np.where(tot > 0, Msafe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return out, lse


# ----------------------------------------------------------------------------------------
# second formulations and the brute-force twin (used as pins)
# ----------------------------------------------------------------------------------------

def brute_force(query, keys, values, cu_seqlens_q, seq_lens, num_kv_heads, scale, mask, span_len=0,
                spans=None):
    """Scalar triple loops with math.exp, no numpy arithmetic: tiny inputs only.

    Independent of the helpers above on purpose: the head map, the chunk positions and
    the mask rules are written out again here from the definition, in a different form
    (the block-causal rule as "key's block no later than the query's block"; the span
    rule as "a later key is visible only up to the end of the query's full span").
    """
    T, H, D = query.shape
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        r0, r1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        for r in range(r0, r1):
            a = L - (r1 - r0) + (r - r0)
            for h in range(H):
                kvh = h // (H // num_kv_heads)
                zs = []
                for p in range(L):
                    if mask == MASK_CAUSAL and p > a:
                        continue
                    if mask == MASK_BLOCK_CAUSAL and (p // span_len) > (a // span_len):
                        continue
                    if mask == MASK_SPANS and p > a:
                        end = a + 1
                        for (ss, se) in spans[s]:
                            if ss <= a < se:
                                end = se
                        if p >= end:
                            continue
                    acc = 0.0
                    for d in range(D):
                        acc += float(query[r, h, d]) * float(keys[s][p, kvh, d])
                    zs.append((p, scale * acc))
                if not zs:
                    continue
                m = max(z for _, z in zs)
                den = 0.0
                num = [0.0] * D
                for p, z in zs:
                    e = math.exp(z - m)
                    den += e
                    for d in range(D):
                        num[d] += e * float(values[s][p, kvh, d])
                for d in range(D):
                    out[r][h][d] = num[d] / den
    return np.array(out, np.float64).reshape(T, H, D)


def fused_head_attention(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray,
                         scale: float, num_kv_heads: int):
    """The block-diagonal fused-head form of the Spyre PR ("Description"): all heads in one
    2D product.  K (after repeat_interleave) is stacked to [H*L, D], Q^T to [D, H*n];
    kq = K Q^T is [H*L, H*n]; cross-head entries are excluded by a block-diagonal mask and
    semantic exclusions by `vis`; softmax runs over the KV axis (axis 0) and the weights
    multiply the stacked V.  q_rows [n, H, D], k/v [L, Hkv, D] -> [n, H, D]."""
    n, H, D = q_rows.shape
    L = k.shape[0]
    g = H // num_kv_heads
    ke = np.repeat(k, g, axis=1)                     # [L, H, D]
    ve = np.repeat(v, g, axis=1)
    kst = ke.transpose(1, 0, 2).reshape(H * L, D)    # head-major stack
    vst = ve.transpose(1, 0, 2).reshape(H * L, -1)
    qt = q_rows.transpose(1, 0, 2).reshape(H * n, D).T
    kq = scale * (kst @ qt)                          # [H*L, H*n]
    allowed = np.zeros((H * L, H * n), bool)
    for h in range(H):
        allowed[h * L:(h + 1) * L, h * n:(h + 1) * n] = vis.T
    kq = np.where(allowed, kq, -np.inf)
    col_max = kq.max(axis=0)
    col_max = np.where(np.isfinite(col_max), col_max, 0.0)
    w = np.exp(kq - col_max)                         # exp(-inf) = 0 off the diagonal blocks
    den = w.sum(axis=0)
    o = (w.T @ vst) / np.where(den > 0, den, 1.0)[:, None]   # [H*n, D]
    o = np.where((den > 0)[:, None], o, 0.0)
    return o.reshape(H, n, -1).transpose(1, 0, 2)


def piecewise_segments(spans: Sequence[tuple], seq_len: int):
    """Segment plan of the vllm-omni piecewise PR for one sequence.

    `spans` lists (start, end, kind) covering [0, seq_len), kind 'causal' or 'full'.  Each
    span becomes one segment (q_start, q_end, kv_end, causal): a causal segment attends
    K[:q_end] bottom-right causally (kv_end == q_end), a full segment attends the whole
    prefix K[:q_end] without a mask.
    """
    segs = []
    for (s, e, kind) in spans:
        e = min(e, seq_len)
        if s >= e:
            continue
        segs.append((s, e, e, kind == "causal"))
    return segs


def uniform_spans(seq_len: int, span_len: int):
    """BLOCK_CAUSAL as a span list: full spans of span_len tiling [0, L) (last one partial)."""
    return [(s, min(s + span_len, seq_len), "full") for s in range(0, seq_len, span_len)]
