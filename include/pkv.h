/*
 * pkv.h -- C ABI of libpkv: scaled dot-product attention over a paged KV cache
 * (variable-length batches) for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument named for a tensor is a DEVICE pointer owned by the
 *   caller.  The library allocates no device memory and keeps no state apart
 *   from a thread-local error string (pkv_last_error), two device words of the
 *   device-side checks, and the fixed scratch array of
 *   pkv_paged_attention_decode_noalloc (one copy per GPU, part of the loaded
 *   code object, held until the process ends).
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Every call only enqueues work on that stream: it never synchronises and
 *   never copies device memory to the host, so device-resident lengths and
 *   tables are trusted, and host "hints" (max_seq_len, max_q_len) size grids.
 *   (Spyre paged-attention PR, "Description"/review: no .item() host syncs in
 *   the forward; ROCm TransformerEngine small-seq PR: host max_seqlen sizes
 *   work on shape queries.)
 * - Everything that can be checked on the host is checked BEFORE anything is
 *   enqueued; a rejected call returns a negative pkv_status, writes nothing and
 *   leaves a message in pkv_last_error() (CSA2 Vanilla golden PR,
 *   "Description": unsupported modes are rejected before anything is written;
 *   review thread: a retry must not fail on stale state).
 * - Element types: dtype applies to query, key, value, caches and output alike,
 *   except in the FP8-cache entry points (*_fp8), whose caches hold E4M3 codes.
 * - Alignment: the attention calls read rows in 16-byte vectors, so out, query
 *   and both caches must be 16-byte aligned and cache_block_stride a multiple
 *   of 16 bytes (INVALID_ARG otherwise).
 * - Cache layout: key_cache and value_cache are each [num_blocks, block_size,
 *   num_kv_heads, head_dim] with the first dimension strided by
 *   cache_block_stride ELEMENTS; inside a block the layout is dense.  A combined
 *   (num_blocks, 2, block_size, num_kv_heads, head_dim) tensor (the final
 *   layout of the Spyre paged-attention PR) is passed as two views with
 *   cache_block_stride = 2*block_size*num_kv_heads*head_dim.
 * - Slot encoding: slot = block_id * block_size + offset_in_block (int64);
 *   a negative slot marks a padding token that is skipped.
 * - GQA: query head h reads kv head h / (num_heads / num_kv_heads), the mapping
 *   repeat_interleave produces (Spyre PR, "Description").
 * - Masks: query row i of a sequence with L tokens and q new tokens sits at
 *   absolute position a = L - q + i and sees key p < L when
 *     PKV_MASK_NONE         always (padding / length only)
 *     PKV_MASK_CAUSAL       p <= a  (bottom-right aligned, vllm-omni piecewise
 *                           block-causal PR: rightDownCausal contract)
 *     PKV_MASK_BLOCK_CAUSAL p <= a or p / span_len == a / span_len (that PR's
 *                           dense "(q >= kv) or same block" reference, blocks
 *                           tiling absolute positions from 0)
 *   A row with no visible key produces zeros.
 * - Precision: bf16/fp16 inputs, fp32 scores, softmax statistics and
 *   accumulators; probabilities are rounded to the input type for the
 *   probability-times-V products; output rounded to nearest even.
 * - Non-finite inputs: cache slots a row cannot see (masked keys, unmapped
 *   blocks, table tails, in-block tails) never enter its arithmetic, so they
 *   may hold anything, NaN included.  A NaN or infinity in a query row or in a
 *   key or value row that a query row does see gives that output row undefined
 *   values on the MFMA prefill kernel, which the prefill, span-list, FP8
 *   prefill and mixed-batch calls use (it is compiled to assume finite
 *   operands); the decode kernels give a NaN row.
 *
 * Device-content preconditions (not checked by default, undefined behaviour if
 * violated; pkv_set_device_checks(1) checks them on the GPU, slot uniqueness
 * through pkv_check_slots_unique):
 *   slots in [0, num_blocks*block_size) or negative, unique within one call;
 *   block_tables entries in [0, num_blocks) for the blocks a sequence uses;
 *   seq_lens[s] <= max_blocks_per_seq*block_size and <= max_seq_len;
 *   cu_seq_lens (gather, small-seq backward) prefix sums from 0 to the total,
 *   equal to the differences of seq_lens where both are given;
 *   cu_seqlens_q non-decreasing with q_s = cu[s+1]-cu[s] <= min(seq_lens[s], max_q_len);
 *   cu_seqlens_q[num_seqs] == num_tokens.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes          */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not compiled: head_dim, dtype              */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the size query     */
  PKV_ERR_LAUNCH = -4       /* the HIP runtime rejected a kernel launch             */
} pkv_status;

/* PKV_FP8_E4M3 (one-byte OCP E4M3 codes) names an FP8 cache; only
 * pkv_kv_cache_gather takes it as its dtype (a raw byte copy).  The FP8 entry
 * points below take the caches as codes and dtype for the other tensors. */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

typedef enum { PKV_MASK_NONE = 0, PKV_MASK_CAUSAL = 1, PKV_MASK_BLOCK_CAUSAL = 2 } pkv_mask_mode;

/* Supported head_dim values (compiled kernel set). */
#define PKV_HEAD_DIM_SUPPORTED(d) ((d) == 16 || (d) == 64 || (d) == 128)

/*
 * pkv_kv_cache_write -- step 1 of the Spyre paged-attention PR ("Description":
 * write new key/value tokens into the paged cache by vectorised scatter through
 * slot_mapping).
 *
 * key, value      [num_tokens, num_kv_heads, head_dim]; token t starts at
 *                 t*kv_token_stride elements (heads and dims dense inside a token).
 * slot_mapping    int64 [num_tokens]; slot < 0 skips the token.
 * key_cache,
 * value_cache     written at block slot/block_size, offset slot%block_size.
 * The copy is a raw bit copy (bit-exact).  num_tokens == 0 is a successful no-op.
 * Errors: INVALID_ARG for null pointers, block_size not a power of two in
 * [1, 256], non-positive sizes, kv_token_stride < num_kv_heads*head_dim, or
 * cache_block_stride < block_size*num_kv_heads*head_dim; UNSUPPORTED for dtype.
 */
int pkv_kv_cache_write(const void* key, const void* value, int64_t kv_token_stride,
                       const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                       void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                       pkv_dtype dtype, void* stream);

/*
 * FP8 KV cache (E4M3).  The pages accept FP8 staging of cache rows (CSA2
 * Vanilla golden PR, "Description") and name FP8 paths (vllm-omni piecewise
 * block-causal PR, review thread) but give no scale convention; the one here:
 * one float scale per cache tensor (k_scale for keys, v_scale for values),
 *   code  = E4M3_RNE(clamp(float32(x * float32(1 / scale)), -448, 448))
 *   value = e4m3(code) * scale
 * with OCP E4M3 (bias 7, max 448, 0x7F / 0xFF NaN, no infinities), ties to
 * even, subnormals kept; a NaN input gives a NaN code.  Attention over such a
 * cache computes softmax(scale * q . (e4m3(k_code) * k_scale)) . (e4m3(v_code)
 * * v_scale) with the precision rules above (the widening to bf16 / fp16 is
 * exact).  Scales must be positive and finite with finite reciprocals.
 *
 * pkv_kv_cache_write_fp8 -- pkv_kv_cache_write that quantises: key and value
 * are dtype (F32, F16 or BF16) rows as in pkv_kv_cache_write; the caches are
 * byte arrays of the same [num_blocks, block_size, num_kv_heads, head_dim]
 * layout (cache_block_stride in bytes).  kv_token_stride and
 * cache_block_stride must be multiples of 4 and the pointers 4-element aligned.
 * Errors as pkv_kv_cache_write, plus INVALID_ARG for scales or alignment.
 */
int pkv_kv_cache_write_fp8(const void* key, const void* value, int64_t kv_token_stride,
                           const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                           void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           float k_scale, float v_scale, pkv_dtype dtype, void* stream);

/*
 * pkv_kv_cache_gather -- step 2 of the Spyre PR ("Description"): the rows a
 * sequence needs are read out of the scattered cache blocks through its block
 * table and laid out contiguously.  Test and debugging aid: the attention
 * kernels fuse this gather into their loads and never materialise it.
 *
 * cu_seq_lens     int32 [num_seqs+1], prefix sums of the sequence lengths.
 * key_out,
 * value_out       [total_tokens, num_kv_heads, head_dim] dense; sequence s fills
 *                 rows cu_seq_lens[s] .. cu_seq_lens[s+1]-1 with its logical
 *                 positions 0..L_s-1.  total_tokens == cu_seq_lens[num_seqs].
 * Errors as pkv_kv_cache_write, plus INVALID_ARG for max_seq_len < 0.
 */
int pkv_kv_cache_gather(void* key_out, void* value_out, const int32_t* cu_seq_lens,
                        const void* key_cache, const void* value_cache,
                        int64_t cache_block_stride, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_tokens,
                        int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_seq_len, pkv_dtype dtype, void* stream);

/*
 * pkv_decode_workspace_size -- bytes of device workspace pkv_paged_attention_decode
 * needs for these sizes (0 when every sequence fits one split): fp32 partial
 * (output, max, sum) slots of (head_dim + 2) * 4 bytes each, plus, beyond 256
 * sequences, the tables a planning kernel writes (8 bytes per sequence, 8 more,
 * and 12 per key range).  The caller
 * allocates it ahead of time (ROCm TransformerEngine small-seq PR: workspace
 * and aux buffers are pre-allocated from host max sequence lengths).
 * Returns 0 for invalid sizes as well; the decode call then validates.
 */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len);

/*
 * pkv_paged_attention_decode -- single-token decode: one query token per
 * sequence attending all L_s cached tokens (the new token already written
 * by pkv_kv_cache_write).  Flash decoding: the keys of a sequence are cut into
 * splits, each split reduces to (partial output, max, sum) in the workspace,
 * and a log-sum-exp merge combines them.  Scores, running max and sums are
 * fp32; the probabilities are rounded to the query type for the P.V products,
 * which run on MFMA or on the vector ALU depending on the shape (bf16/fp16 with
 * several query heads per kv head mostly take MFMA; fp32 and head_dim 16 never
 * do).  The small-seq varlen
 * cross-attention case of the ROCm TransformerEngine PR (s_q = 1, s_kv <= 16,
 * one sequence per query token) is this call with num_seqs = number of query
 * tokens.
 *
 * out, query      [num_seqs, num_heads, head_dim] dense.
 * block_tables    int32 [num_seqs, max_blocks_per_seq] (row stride max_blocks_per_seq).
 * seq_lens        int32 [num_seqs]; 0 yields a zero output row.
 * max_seq_len     host hint >= every seq_lens[s]; sizes the split grid.
 * workspace       device buffer of at least pkv_decode_workspace_size(...) bytes,
 *                 16-byte aligned (may be NULL when that size is 0).  Contents
 *                 need no initialisation; calls sharing one workspace must be
 *                 ordered.
 * Errors: INVALID_ARG (null pointers, num_heads % num_kv_heads != 0, sizes, a
 * misaligned workspace), UNSUPPORTED (head_dim, dtype), WORKSPACE (too small).
 */
int pkv_paged_attention_decode(void* out, const void* query, const void* key_cache,
                               const void* value_cache, int64_t cache_block_stride,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               int32_t block_size, float scale, int32_t max_seq_len,
                               void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                               void* stream);

/*
 * pkv_paged_attention_decode_noalloc -- pkv_paged_attention_decode for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, results
 * and kernels, without the workspace arguments.  The workspace is the
 * library's own scratch array of PKV_DECODE_NOALLOC_MAX_WORKSPACE bytes, one per
 * GPU (its address is looked up once per device, on the first call there); the
 * call allocates and frees nothing.  Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (concurrent streams, threads)
 * race and give undefined results: order them.  Its contents need no
 * clearing between calls (every partial is written before it is read).
 * Errors: as pkv_paged_attention_decode, plus WORKSPACE when
 * pkv_decode_workspace_size(...) for these sizes exceeds
 * PKV_DECODE_NOALLOC_MAX_WORKSPACE, and LAUNCH when the array's device
 * address cannot be obtained.
 */
#define PKV_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, int64_t cache_block_stride,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t num_blocks, int32_t block_size, float scale,
                                       int32_t max_seq_len, pkv_dtype dtype, void* stream);

/*
 * pkv_paged_attention_decode_fp8 -- pkv_paged_attention_decode over FP8 caches
 * written by pkv_kv_cache_write_fp8 (conventions above).  query and out are
 * dtype (PKV_BF16 or PKV_F16); the caches are byte arrays with
 * cache_block_stride in bytes (a multiple of 16).  Same workspace size as
 * pkv_paged_attention_decode.  Errors as pkv_paged_attention_decode, plus
 * UNSUPPORTED for a dtype other than BF16 / F16 and INVALID_ARG for scales.
 */
int pkv_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, int64_t cache_block_stride,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                   int32_t block_size, float scale, float k_scale, float v_scale,
                                   int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                                   pkv_dtype dtype, void* stream);

/*
 * pkv_paged_attention_prefill -- prefill and chunked prefill over a flat (THD)
 * query batch: sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1,
 * which are its newest q_s tokens, so row i sits at position L_s - q_s + i
 * (Spyre PR "Description" steps 3-6 without padding: rows are addressed in
 * place and written back in query order).
 *
 * out, query      [num_tokens, num_heads, head_dim] dense.
 * cu_seqlens_q    int32 [num_seqs+1].
 * seq_lens        int32 [num_seqs], total keys per sequence including the new ones.
 * mask, span_len  see the mask rules above; span_len > 0 required for BLOCK_CAUSAL.
 * max_q_len,
 * max_seq_len     host hints >= every q_s and L_s; they size the grid.
 * bf16/fp16 with head_dim 64 or 128 run on MFMA; fp32 and head_dim 16 run on a
 * vector-ALU kernel with fp32 probabilities.
 * Errors: INVALID_ARG (null pointers, num_heads % num_kv_heads, sizes, mask,
 * span_len), UNSUPPORTED (head_dim, dtype).
 */
int pkv_paged_attention_prefill(void* out, const void* query, const int32_t* cu_seqlens_q,
                                const int32_t* seq_lens, const void* key_cache,
                                const void* value_cache, int64_t cache_block_stride,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                int32_t block_size, float scale, pkv_mask_mode mask,
                                int32_t span_len, int32_t max_q_len, int32_t max_seq_len,
                                pkv_dtype dtype, void* stream);

/*
 * pkv_paged_attention_prefill_fp8 -- pkv_paged_attention_prefill over FP8
 * caches written by pkv_kv_cache_write_fp8 (conventions above); query and out
 * are dtype (PKV_BF16 or PKV_F16), the caches byte arrays with
 * cache_block_stride in bytes (a multiple of 16).  Masks NONE, CAUSAL and
 * BLOCK_CAUSAL; there is no FP8 form of the span-list call (the quantised path
 * of the vllm-omni piecewise block-causal PR rejects span metadata).  Errors as
 * pkv_paged_attention_prefill, plus UNSUPPORTED for a dtype other than BF16 /
 * F16 and INVALID_ARG for scales.
 */
int pkv_paged_attention_prefill_fp8(void* out, const void* query, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens, const void* key_cache,
                                    const void* value_cache, int64_t cache_block_stride,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                    int32_t block_size, float scale, float k_scale, float v_scale,
                                    pkv_mask_mode mask, int32_t span_len, int32_t max_q_len,
                                    int32_t max_seq_len, pkv_dtype dtype, void* stream);

/*
 * Mixed batch -- one step's context rows (prefill / chunked prefill) and
 * generation rows (single-token decode) in one call: the prefill kernel over
 * the context rows, then the decode kernels over the generation rows, enqueued
 * on `stream` in that order (results and speed equal to the two calls
 * pkv_paged_attention_prefill + pkv_paged_attention_decode on the two parts).
 * The Spyre paged-attention PR ("Description") sends the prefill and decode
 * sequences of a step through one attention call; the CSA2 Vanilla golden PR
 * ("Description") orders a batch context first, generation after, and keeps
 * query tiles from crossing that boundary.
 *
 * Sequences 0 .. num_ctx_seqs-1 are context sequences: query rows
 * cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (cu_seqlens_q int32 [num_ctx_seqs+1],
 * cu_seqlens_q[num_ctx_seqs] == num_ctx_tokens), the mask rules of
 * pkv_paged_attention_prefill.  Sequences num_ctx_seqs .. num_seqs-1 are
 * generation sequences with one query row each, row num_ctx_tokens + (s -
 * num_ctx_seqs), which attends all seq_lens[s] keys (the last row of any mask).
 * num_tokens - num_ctx_tokens must equal num_seqs - num_ctx_seqs.
 * out, query      [num_tokens, num_heads, head_dim] dense (THD).
 * seq_lens        int32 [num_seqs]; block_tables int32 [num_seqs, max_blocks_per_seq].
 * max_q_len       host hint >= every context chunk length (0 without context rows).
 * workspace       device buffer of pkv_mixed_workspace_size(num_seqs -
 *                 num_ctx_seqs, ...) bytes (the decode workspace of the
 *                 generation rows, pkv_decode_workspace_size of the same
 *                 arguments), 16-byte aligned (may be NULL when that is 0).
 *                 Contents need no initialisation; calls sharing one workspace
 *                 must be ordered.
 * Errors: as pkv_paged_attention_prefill and
 * pkv_paged_attention_decode, plus INVALID_ARG for an inconsistent boundary.
 */
size_t pkv_mixed_workspace_size(int32_t num_gen_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_seq_len);

int pkv_paged_attention_mixed(void* out, const void* query, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens, const void* key_cache,
                              const void* value_cache, int64_t cache_block_stride,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              int32_t num_seqs, int32_t num_tokens, int32_t num_ctx_seqs,
                              int32_t num_ctx_tokens, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t block_size,
                              float scale, pkv_mask_mode mask, int32_t span_len,
                              int32_t max_q_len, int32_t max_seq_len, void* workspace,
                              size_t workspace_bytes, pkv_dtype dtype, void* stream);

/*
 * Small-seq training path (ROCm TransformerEngine small-seq PR, description:
 * varlen cross attention with one query token per sequence and s_kv <= 16; the
 * forward writes the attention weights, the backward reads them and computes
 * grad_V, grad_attn, the softmax backward and grad_Q / grad_K).  Keys and
 * values come from the paged cache through the block table, as in decode.
 *
 * pkv_smallseq_attention_fwd -- out[s, h] = sum_k P[s, h, k] V_s[k, h / g] with
 *   P[s, h, k] = softmax over k < seq_lens[s] of scale <q[s, h], K_s[k, h / g]>.
 * out, query      [num_seqs, num_heads, head_dim] dense.
 * weights         [num_seqs, num_heads, max_seq_len] in dtype: P rounded to
 *                 nearest even, zero for k >= seq_lens[s] (a sequence with no
 *                 keys gets a zero row and a zero output).
 * max_seq_len     1..16, >= every seq_lens[s]; the row length of weights.
 * dtype           PKV_BF16 or PKV_F16; head_dim 16, 64 or 128.
 * Errors: INVALID_ARG (null pointers, max_seq_len outside [1, 16], sizes,
 * alignment), UNSUPPORTED (dtype, head_dim).
 */
int pkv_smallseq_attention_fwd(void* out, void* weights, const void* query,
                               const void* key_cache, const void* value_cache,
                               int64_t cache_block_stride, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks, int32_t block_size,
                               float scale, int32_t max_seq_len, pkv_dtype dtype, void* stream);

/*
 * pkv_smallseq_attention_bwd -- gradients of sum(d_out * out) for the forward
 * above, from the weights it saved (P as stored, not recomputed):
 *   dV[k, j] = sum over the heads h of kv head j of P[h, k] dO[h]
 *   dP[h, k] = <dO[h], V[k, j]>;  dS = P (dP - sum_k P dP)
 *   dQ[h]    = scale sum_k dS[h, k] K[k, j]
 *   dK[k, j] = scale sum over the heads h of kv head j of dS[h, k] q[h]
 * d_query, d_out, query  [num_seqs, num_heads, head_dim].
 * d_key, d_value  [total_kv, num_kv_heads, head_dim]: key k of sequence s at row
 *                 cu_seq_lens[s] + k (THD, the layout of the packed K/V inputs).
 * cu_seq_lens     int32 [num_seqs+1], prefix sums of seq_lens, ending at total_kv.
 * Scalars and errors as pkv_smallseq_attention_fwd.  Accumulation is fp32;
 * results are rounded to nearest even.
 */
int pkv_smallseq_attention_bwd(void* d_query, void* d_key, void* d_value, const void* d_out,
                               const void* query, const void* weights, const void* key_cache,
                               const void* value_cache, int64_t cache_block_stride,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, const int32_t* cu_seq_lens,
                               int32_t num_seqs, int32_t total_kv, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               int32_t block_size, float scale, int32_t max_seq_len,
                               pkv_dtype dtype, void* stream);

/* Prefill with general span lists (vllm-omni piecewise block-causal PR: the
 * `full_attn_spans` metadata -- image blocks attend bidirectionally, text runs
 * causally; its dense reference "(q >= kv) or same_image_block").
 *
 * Same arguments and layouts as pkv_paged_attention_prefill, except the mask:
 * the query at absolute position a of sequence s sees key p < seq_lens[s] when
 * p <= a, or when a lies in a full span [start, end) of s and p < end.  Rows
 * outside every full span are causal (text).  The full spans of sequence s are
 * the pairs full_spans[2*i], full_spans[2*i+1] for i in [cu_spans[s],
 * cu_spans[s+1]), in absolute positions, sorted by start and disjoint (a span
 * may reach past seq_lens[s]; keys past it do not exist).  full_spans is int32
 * [num_spans][2], cu_spans int32 [num_seqs+1], both device memory owned by the
 * caller.  num_spans == 0 is plain CAUSAL (full_spans and cu_spans may then be
 * NULL).  Errors: as pkv_paged_attention_prefill, plus num_spans < 0 or a NULL
 * span array with num_spans > 0 -> PKV_ERR_INVALID_ARG. */
int pkv_paged_attention_prefill_spans(void* out, const void* query, const int32_t* cu_seqlens_q,
                                      const int32_t* seq_lens, const void* key_cache,
                                      const void* value_cache, int64_t cache_block_stride,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                      int32_t block_size, float scale, const int32_t* full_spans,
                                      const int32_t* cu_spans, int32_t num_spans,
                                      int32_t max_q_len, int32_t max_seq_len, pkv_dtype dtype,
                                      void* stream);

/* ---- device-side precondition checks -------------------------------------------
 * The preconditions on device memory above cannot be seen by the host without a
 * copy, which the calls never make.  With checks on, each call first runs a
 * check kernel on its stream that ORs one bit per violated precondition into a
 * per-device error word, and every kernel of the library returns at once while
 * that word is non-zero, so a violating call (and every later call on that
 * device) writes nothing and reads no memory outside its arguments' true
 * extents.  The word stays set until pkv_check_device_error reads it.
 * (Spyre paged-attention PR: no host syncs in the forward, hence the checks run
 * on the device; CSA2 Vanilla golden PR: a failed call writes nothing.)
 * Duplicate slots within one kv_cache_write call are detected by
 * pkv_check_slots_unique (below), which needs a caller-owned bitmap. */
typedef enum {
  PKV_CHECK_SLOT_RANGE = 1,  /* a slot >= num_blocks * block_size                    */
  PKV_CHECK_SEQ_LEN = 2,     /* seq_lens[s] < 0, > max_seq_len, or > max_blocks*B;   */
                             /* for the gather: cu_seq_lens not non-decreasing from 0 */
                             /* or not ending at total_tokens                        */
  PKV_CHECK_TABLE = 4,       /* a used block_tables entry outside [0, num_blocks)    */
  PKV_CHECK_CU_Q = 8,        /* cu_seqlens_q: not from 0, decreasing, not ending at  */
                             /* num_tokens, or q_s > min(seq_lens[s], max_q_len)     */
  PKV_CHECK_SPANS = 16,      /* span lists: cu_spans not from 0 / decreasing / not   */
                             /* ending at num_spans, or a sequence's spans unsorted, */
                             /* overlapping, empty or starting below 0               */
  PKV_CHECK_DUP_SLOT = 32    /* two tokens of one slot_mapping share a slot          */
} pkv_check_bits;

/* pkv_check_slots_unique -- the uniqueness precondition of pkv_kv_cache_write
 * (two tokens of one call with the same slot race; the Spyre paged-attention PR,
 * "Description", step 1, scatters each new token to its own slot).  Enqueues, on
 * `stream`, a pass that sets one bit per valid slot of slot_mapping in `marks` and
 * ORs PKV_CHECK_DUP_SLOT into the device error word when a bit was already set, then
 * a pass that clears those bits again.  Run it before the kv_cache_write call it
 * checks, on the same stream: with device checks on (pkv_set_device_checks) that
 * write and every later call then write nothing until pkv_check_device_error reads
 * the word; with checks off the bit still waits there for pkv_check_device_error.
 *
 * slot_mapping    int64 [num_tokens], as given to pkv_kv_cache_write; negative and
 *                 out-of-range slots are skipped (the range check reports the latter).
 * marks           device bitmap of at least ((num_blocks*block_size + 31) / 32) uint32
 *                 words, 4-byte aligned, owned by the caller, ALL ZERO before the first
 *                 call (for instance from hipMemset once); every call leaves it all zero.
 *                 Calls sharing one bitmap must be ordered.
 * Errors: INVALID_ARG for null pointers, num_tokens < 0, num_blocks or block_size out
 * of range, or a bitmap that is too small or misaligned; LAUNCH if the device error
 * word is unavailable.  num_tokens == 0 is a successful no-op. */
int pkv_check_slots_unique(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, void* marks, size_t marks_bytes, void* stream);

/* Turn the device-side checks on (enable != 0) or off for every later call in
 * this process.  Checks cost one small kernel per call.  Returns PKV_OK. */
int pkv_set_device_checks(int enable);

/* Wait for `stream`, read and clear the error word of the current device.
 * Returns PKV_OK when no check failed since the last read, else
 * PKV_ERR_INVALID_ARG with the violated checks named in pkv_last_error() and
 * the pkv_check_bits in *bits (when bits is not NULL); PKV_ERR_LAUNCH if the
 * HIP runtime fails.  This call synchronises: it is for tests and debugging. */
int pkv_check_device_error(void* stream, uint32_t* bits);

/* Launch log: with it on, every kernel launch prints one line to stderr naming the
 * kernel, its grid and block and the variant chosen (decode mode, heads per wave,
 * prefill tiling, ...).  Initially on when PKV_LOG is set to a value other than 0 in the
 * environment; pkv_set_log(enable) switches it for every later call.  Returns PKV_OK. */
int pkv_set_log(int enable);

/* Message of the last failed call on this thread ("" if none).  Valid until the
 * next pkv_* call on the same thread. */
const char* pkv_last_error(void);

/* ABI version: (major << 16) | minor. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
