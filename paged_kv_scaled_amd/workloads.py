"""Seeded synthetic inputs for paged-KV attention.

This module only *draws* inputs: sequence lengths, a shuffled block pool, block
tables, the slot of every logical token, and Q/K/V values rounded to the storage
dtype.  It computes no attention, softmax, mask or gather; both the fp64 oracle
(test infrastructure) and the HIP path consume what it returns.

Workload shapes follow the pages:
  * tiny prefill with a shuffled, partly unmapped block table (CSA2 Vanilla
    golden PR, "Test Coverage": shuffled and partly unmapped pages);
  * decode batches over a paged cache (Spyre paged-attention PR, "Description",
    steps 1-2: scatter through slot_mapping, gather from scattered blocks);
  * chunked prefill (Spyre PR, example runner forcing many chunked prefills);
  * s_q = 1, s_kv <= 16 varlen cross attention with b = 30720 (ROCm
    TransformerEngine CK small-seq PR, test description and dispatch condition);
  * long block-causal prefill with 2048-token spans (vllm-omni piecewise
    block-causal PR, the shared compressed (2048, 2048) mask).

Draw order for every config (fixed, so one seed fixes every array):
  1. lengths, 2. block permutation, 3. Q, K, V as float32 N(0, 1),
  4. rounding to the storage dtype (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_BLOCK_CAUSAL, MASK_SPANS = 0, 1, 2, 3
MASK_NAMES = {MASK_NONE: "none", MASK_CAUSAL: "causal", MASK_BLOCK_CAUSAL: "block_causal",
              MASK_SPANS: "spans"}

# Storage dtypes: name -> (numpy storage dtype of the raw bits, bytes per element)
DTYPES = {"f32": (np.uint32, 4), "f16": (np.uint16, 2), "bf16": (np.uint16, 2)}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> raw storage bits of `dtype` (RNE).  Input generation only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # round-to-nearest-even on the 16 dropped bits (inputs are finite normals)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(dtype)


def nan_bits(dtype: str):
    """A quiet-NaN bit pattern of the storage dtype (sentinel for untouched memory)."""
    return {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}[dtype]


@dataclasses.dataclass
class Workload:
    """One batch.  All arrays are host numpy arrays of raw storage bits / ints."""
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    mask: int
    span_len: int
    scale: float
    seq_lens: np.ndarray          # int32 [S]   L_s = cached context + new tokens
    q_lens: np.ndarray            # int32 [S]   new (query) tokens of this call
    cu_seqlens_q: np.ndarray      # int32 [S+1]
    cu_seq_lens: np.ndarray       # int32 [S+1] prefix sums of seq_lens (logical K/V rows)
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq]
    slots: np.ndarray             # int64 [sum L]  cache slot of every logical K/V row
    query: np.ndarray             # bits [T, H, D]
    key: np.ndarray               # bits [sum L, Hkv, D] logical keys, sequence-major
    value: np.ndarray             # bits [sum L, Hkv, D]
    decode: bool = False          # one query token per sequence
    spans: Optional[list] = None  # SPANS mask: per sequence, the (start, end) full spans
    kv_dtype: Optional[str] = None  # "fp8": the cache holds E4M3 codes of key/value
    k_scale: float = 1.0            # FP8 cache: value = code * scale
    v_scale: float = 1.0
    num_ctx_seqs: Optional[int] = None   # mixed batch: context sequences first, then
                                         # one-row generation sequences
    d_out: Optional[np.ndarray] = None   # small-seq backward: gradient of the output
                                         # [S, H, D], storage bits of `dtype`

    def span_arrays(self):
        """The span lists flattened for the library: int32 [num_spans, 2] (start, end)
        pairs, sequence by sequence, and int32 [S+1] offsets into them."""
        lists = self.spans or [[] for _ in range(self.num_seqs)]
        flat = [pair for seq in lists for pair in seq]
        cu = np.zeros(self.num_seqs + 1, np.int32)
        cu[1:] = np.cumsum([len(x) for x in lists])
        arr = np.array(flat, np.int32).reshape(-1, 2) if flat else np.zeros((0, 2), np.int32)
        return arr, cu

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    def new_token_rows(self) -> np.ndarray:
        """Indices into key/value of the rows written by this call (last q_s of each seq)."""
        idx = [np.arange(self.cu_seq_lens[s + 1] - self.q_lens[s], self.cu_seq_lens[s + 1])
               for s in range(self.num_seqs)]
        return np.concatenate(idx).astype(np.int64) if idx else np.zeros(0, np.int64)

    def context_rows(self) -> np.ndarray:
        idx = [np.arange(self.cu_seq_lens[s], self.cu_seq_lens[s + 1] - self.q_lens[s])
               for s in range(self.num_seqs)]
        return np.concatenate(idx).astype(np.int64) if idx else np.zeros(0, np.int64)


def _standard_normal(rng: np.random.Generator, shape, chunk=1 << 26) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        out[i:j] = rng.standard_normal(j - i, dtype=np.float32)
    return out.reshape(shape)


def _draw_values(rng, shape, dtype, chunk_rows=None):
    """N(0,1) float32 rounded to `dtype`, drawn in row chunks to bound host memory."""
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    chunk_rows = chunk_rows or max(1, (1 << 25) // max(per_row, 1))
    out = np.empty(shape, DTYPES[dtype][0])
    for i in range(0, rows, chunk_rows):
        j = min(rows, i + chunk_rows)
        out[i:j] = round_to_storage(_standard_normal(rng, (j - i,) + tuple(shape[1:])), dtype)
    return out


def build(name: str, seed: int, dtype: str, seq_lens, q_lens, num_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, mask: int, span_len: int = 0, scale: Optional[float] = None,
          spare_blocks: int = 1, max_blocks_per_seq: Optional[int] = None, decode: bool = False,
          rng: Optional[np.random.Generator] = None) -> Workload:
    """Lay out a batch over a shuffled block pool and draw its Q/K/V.

    Each sequence owns ceil(L_s / block_size) blocks taken, in order, from one
    random permutation of the pool; `spare_blocks` extra blocks stay unmapped
    (callers fill them with NaN sentinels).  Table entries past a sequence's
    last block point at the first unmapped block when there is one, else at 0.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int32)
    q_lens = np.asarray(q_lens, np.int32)
    S = seq_lens.shape[0]
    assert q_lens.shape == (S,) and np.all(q_lens <= seq_lens) and np.all(q_lens >= 0)
    nblk = (seq_lens.astype(np.int64) + block_size - 1) // block_size
    used = int(nblk.sum())
    num_blocks = used + spare_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)          # draw 2: block permutation
    mb = max_blocks_per_seq or max(1, int(nblk.max()) if S else 1)
    assert mb >= (int(nblk.max()) if S else 0)
    filler = perm[used] if spare_blocks > 0 else 0
    tables = np.full((S, mb), filler, np.int32)
    off = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += int(nblk[s])
    cu_k = np.zeros(S + 1, np.int32)
    cu_k[1:] = np.cumsum(seq_lens)
    cu_q = np.zeros(S + 1, np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    # slot of every logical row: caller-side layout of the cache (block id * B + offset)
    slots = np.empty(int(cu_k[-1]), np.int64)
    for s in range(S):
        p = np.arange(seq_lens[s], dtype=np.int64)
        slots[cu_k[s]:cu_k[s + 1]] = tables[s, p // block_size].astype(np.int64) * block_size + p % block_size
    T = int(cu_q[-1])
    q = _draw_values(rng, (T, num_heads, head_dim), dtype)               # draw 3: Q, K, V
    k = _draw_values(rng, (int(cu_k[-1]), num_kv_heads, head_dim), dtype)
    v = _draw_values(rng, (int(cu_k[-1]), num_kv_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / float(np.sqrt(head_dim))
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, num_blocks=num_blocks, mask=mask,
                    span_len=span_len, scale=float(scale), seq_lens=seq_lens, q_lens=q_lens,
                    cu_seqlens_q=cu_q, cu_seq_lens=cu_k, block_tables=tables, slots=slots,
                    query=q, key=k, value=v, decode=decode)


# --------------------------------------------------------------------------------------
# The five workload shapes.  `scale_down` shrinks the batch for parity tests that the
# oracle must finish in seconds, keeping every other parameter.
# --------------------------------------------------------------------------------------

def tiny_prefill(seed: int = 0) -> Workload:
    """2 sequences (5, 9), 4 q heads / 2 kv heads, D 16, B 4, 8 blocks shuffled, fp32, causal.

    The 8-block pool holds 5 mapped blocks; 3 stay unmapped.
    """
    rng = np.random.default_rng(seed)
    lens = np.array([5, 9], np.int32)
    return build("tiny_prefill", seed, "f32", lens, lens, 4, 2, 16, 4, MASK_CAUSAL,
                 scale=0.25, spare_blocks=3, rng=rng)


def decode_batch(seed: int = 1, num_seqs: int = 64, lo: int = 256, hi: int = 4096,
                 dtype: str = "bf16", spare_blocks: int = 1) -> Workload:
    """64 sequences, one new token each, context uniform in [lo, hi] (incl. the new token)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)     # draw 1
    return build("decode_batch", seed, dtype, lens, np.ones(num_seqs, np.int32), 32, 8, 128, 16,
                 MASK_NONE, spare_blocks=spare_blocks, decode=True, rng=rng)


def chunked_prefill(seed: int = 2, num_seqs: int = 8, ctx_hi: int = 2048, q_lo: int = 32,
                    q_hi: int = 512, dtype: str = "bf16", spare_blocks: int = 1) -> Workload:
    """8 sequences: cached context U{0..2048} plus a new chunk U{32..512}; causal."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, ctx_hi + 1, size=num_seqs).astype(np.int32)   # draw 1
    ql = rng.integers(q_lo, q_hi + 1, size=num_seqs).astype(np.int32)
    return build("chunked_prefill", seed, dtype, ctx + ql, ql, 32, 8, 128, 16, MASK_CAUSAL,
                 spare_blocks=spare_blocks, rng=rng)


SMALLSEQ_KV = (2, 4, 6, 8, 12, 16)


def smallseq_varlen(seed: int = 3, num_seqs: int = 30720, dtype: str = "bf16",
                    spare_blocks: int = 1) -> Workload:
    """s_q = 1, s_kv uniform over {2,4,6,8,12,16}, 16 heads (MHA), D 128, B 16: one block per seq."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(SMALLSEQ_KV, np.int32)[rng.integers(0, len(SMALLSEQ_KV), size=num_seqs)]
    return build("smallseq_varlen", seed, dtype, lens, np.ones(num_seqs, np.int32), 16, 16, 128, 16,
                 MASK_NONE, spare_blocks=spare_blocks, decode=True, rng=rng)


def smallseq_train(seed: int = 7, num_seqs: int = 30720, dtype: str = "bf16",
                   num_heads: int = 16, num_kv_heads: int = 16, head_dim: int = 128,
                   kv_choices=SMALLSEQ_KV) -> Workload:
    """The small-seq shape for the training path: s_q = 1, s_kv uniform over
    {2,4,6,8,12,16}, 16 heads (MHA), D 128, B 16, plus the output gradient d_out ~ N(0,1)
    (drawn after Q, K and V)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(kv_choices, np.int32)[rng.integers(0, len(kv_choices), size=num_seqs)]
    w = build("smallseq_train", seed, dtype, lens, np.ones(num_seqs, np.int32), num_heads,
              num_kv_heads, head_dim, 16, MASK_NONE, decode=True, rng=rng)
    w.d_out = _draw_values(rng, (num_seqs, num_heads, head_dim), dtype)     # draw 4
    return w


def long_block_causal(seed: int = 4, num_seqs: int = 4, seq_len: int = 8192, dtype: str = "bf16",
                      num_heads: int = 64, spare_blocks: int = 1, num_kv_heads: int = 8) -> Workload:
    """4 x 8192 tokens, 64 q heads / 8 kv heads, D 128, B 16, block-causal spans of 2048.
    (num_heads = 8, num_kv_heads = 1 is one GPU's share when the kv heads are split over
    eight GPUs.)"""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, seq_len, np.int32)
    return build("long_block_causal", seed, dtype, lens, lens, num_heads, num_kv_heads, 128, 16,
                 MASK_BLOCK_CAUSAL, span_len=2048, spare_blocks=spare_blocks, rng=rng)


def span_layout(rng: np.random.Generator, seq_len: int, text=(16, 256), image=(256, 1024)):
    """A text/image layout of one sequence: alternating causal text runs and full image
    blocks with lengths drawn uniformly from the given ranges, starting with text.
    Returns the full spans as (start, end) pairs (the text runs are what lies between)."""
    spans, pos, is_text = [], 0, True
    while pos < seq_len:
        lo, hi = text if is_text else image
        n = int(rng.integers(lo, hi + 1))
        if not is_text:
            spans.append((pos, min(pos + n, seq_len)))
        pos += n
        is_text = not is_text
    return spans


def mixed_spans(seed: int = 5, num_seqs: int = 4, seq_len: int = 4096, dtype: str = "bf16",
                num_heads: int = 32, q_len: Optional[int] = None, spare_blocks: int = 1,
                text=(16, 256), image=(256, 1024), head_dim: int = 128) -> Workload:
    """General span lists (the next row after the five shapes): per sequence, text runs of
    U{16..256} tokens (causal) alternating with image blocks of U{256..1024} tokens (full),
    32 q / 8 kv heads, D 128, B 16.  q_len < seq_len makes it a chunked prefill."""
    rng = np.random.default_rng(seed)
    lens = np.full(num_seqs, seq_len, np.int32)                       # draw 1 (fixed)
    layouts = [span_layout(rng, seq_len, text, image) for _ in range(num_seqs)]   # draw 1b
    ql = np.full(num_seqs, q_len or seq_len, np.int32)
    w = build("mixed_spans", seed, dtype, lens, ql, num_heads, 8, head_dim, 16, MASK_SPANS,
              spare_blocks=spare_blocks, rng=rng)
    w.spans = layouts
    return w


def with_fp8_cache(w: Workload, k_scale: float = 0.0173, v_scale: float = 0.0211) -> Workload:
    """The same batch over an FP8 (E4M3) cache: kv_cache_write quantises the drawn K/V rows
    with one scale per tensor (N(0, 1) rows reach about +-5, well inside 448 * scale)."""
    w.kv_dtype, w.k_scale, w.v_scale = "fp8", float(np.float32(k_scale)), float(np.float32(v_scale))
    w.name = w.name + "_fp8"
    return w


def decode_long_seq(seed: int = 7, length: int = 32768, dtype: str = "bf16",
                    spare_blocks: int = 1) -> Workload:
    """One sequence of 32768 keys decoding its next token (long-context batch-1 serving),
    32 q / 8 kv heads, D 128, B 16."""
    rng = np.random.default_rng(seed)
    return build("decode_long_seq", seed, dtype, np.array([length], np.int32),
                 np.ones(1, np.int32), 32, 8, 128, 16, MASK_NONE, spare_blocks=spare_blocks,
                 decode=True, rng=rng)


def decode_batch_fp8(seed: int = 1, **kw) -> Workload:
    """The decode batch (64 sequences, contexts U[256, 4096], 32 q / 8 kv heads, D 128,
    B 16) over an FP8 cache."""
    return with_fp8_cache(decode_batch(seed=seed, **kw))


def mixed_batch(seed: int = 6, num_ctx: int = 8, num_gen: int = 64, ctx_hi: int = 2048,
                q_lo: int = 32, q_hi: int = 512, lo: int = 256, hi: int = 4096,
                dtype: str = "bf16", num_heads: int = 32, num_kv_heads: int = 8,
                head_dim: int = 128, block_size: int = 16, mask: int = MASK_CAUSAL,
                span_len: int = 0) -> Workload:
    """One serving step: the chunked-prefill shape (8 sequences, context U{0..2048} plus a
    chunk U{32..512}) followed by the decode-batch shape (64 one-token sequences with
    contexts U[256, 4096]), 32 q / 8 kv heads, D 128, B 16, causal."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, ctx_hi + 1, size=num_ctx).astype(np.int32)     # draw 1
    ql = rng.integers(q_lo, q_hi + 1, size=num_ctx).astype(np.int32)
    gl = rng.integers(lo, hi + 1, size=num_gen).astype(np.int32)
    lens = np.concatenate([ctx + ql, gl])
    qls = np.concatenate([ql, np.ones(num_gen, np.int32)])
    w = build("mixed_batch", seed, dtype, lens, qls, num_heads, num_kv_heads, head_dim,
              block_size, mask, span_len=span_len, rng=rng)
    w.num_ctx_seqs = num_ctx
    return w


def long_block_causal_fp8(seed: int = 4, **kw) -> Workload:
    """The long block-causal prefill (4 x 8192 tokens, 64 q / 8 kv heads, spans of 2048)
    over an FP8 cache."""
    return with_fp8_cache(long_block_causal(seed=seed, **kw))


CONFIGS = {
    "tiny_prefill": tiny_prefill,
    "decode_batch": decode_batch,
    "chunked_prefill": chunked_prefill,
    "smallseq_varlen": smallseq_varlen,
    "long_block_causal": long_block_causal,
    "mixed_spans": mixed_spans,
    "decode_batch_fp8": decode_batch_fp8,
    "decode_long_seq": decode_long_seq,
    "long_block_causal_fp8": long_block_causal_fp8,
    "mixed_batch": mixed_batch,
    "smallseq_train": smallseq_train,
}


def random_small(seed: int, dtype: str = "f32", max_seqs: int = 3, max_len: int = 12,
                 head_dim: int = 8, mask: Optional[int] = None, decode: bool = False,
                 block_size: Optional[int] = None) -> Workload:
    """Tiny random batches for brute-force checks: S <= 3, L <= 12, D <= 8."""
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, max_seqs + 1))
    L = rng.integers(1, max_len + 1, size=S).astype(np.int32)
    if decode:
        ql = np.ones(S, np.int32)
    else:
        ql = np.array([rng.integers(1, l + 1) for l in L], np.int32)
    hkv = int(rng.integers(1, 3))
    g = int(rng.integers(1, 4))
    bs = block_size or int(2 ** rng.integers(0, 3))
    m = int(rng.integers(0, 3)) if mask is None else mask
    span = int(rng.integers(1, 6))
    return build(f"random_small_{seed}", seed, dtype, L, ql, hkv * g, hkv, head_dim, bs, m,
                 span_len=span, scale=float(rng.uniform(0.1, 0.6)), spare_blocks=1, decode=decode,
                 rng=rng)
