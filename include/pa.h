/*
 * pa.h -- C ABI of libpa: paged grouped-query attention for LLM decoding on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the attention step of a decoding engine with a paged KV
 * cache, as the page "From 183 ms to 19 ms per decode step" (mini-engine)
 * describes it in section "Four changes, one profile at a time":
 *   - change 2: the cache is head-major, [kv_heads, num_blocks, block_size,
 *     head_dim], so one index over the slots of a head returns a sequence's
 *     context in order;
 *   - change 3: the kernel walks each sequence's block table and reads K and V
 *     in place, one program per (sequence, KV head) serving every query head
 *     of its group, with an fp32 online softmax (running max and sum,
 *     rescaled per tile);
 *   - change 4: each step hands the kernels fixed buffers of cache slots,
 *     block tables and lengths;
 * and in section "Then speculative decoding got slower": a kernel for a few
 * query tokens per sequence (k+1 speculative tokens) with a causal mask
 * among the new tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory: every pointer argument is DEVICE memory owned by the caller,
 *   contiguous and row-major in the shape given.  The library never
 *   allocates, frees or synchronises, and never reads device memory on the
 *   host.  Pointers to 16-bit or wider data must be 16-byte aligned.
 * Streams: `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues kernels on it and returns; results are valid once the stream has
 *   reached that point.  No call records or waits on events, so calls can be
 *   captured into a hipGraph.
 * Dtypes: q / cache / out combinations supported:
 *   PA_F32 / PA_F32 / fp32, PA_BF16 / PA_BF16 / bf16, PA_BF16 / PA_INT8 / bf16.
 *   bf16 values are raw bfloat16 bit patterns; outputs are rounded to nearest
 *   even.  Accumulation is fp32.
 * int8 caches: signed codes in [-127, 127]; the value of a cached element is
 *   code * scale[kv_head, physical_block] (one fp32 scale per block and KV
 *   head, separately for K and V).
 * Lengths: context_lens[b] is the number of cached positions sequence b
 *   attends to, INCLUDING the token(s) being decoded -- write the new token's
 *   K/V with pa_reshape_and_cache first, then attend (the decode loop of
 *   "Anatomy of a Decode-Step Stall", section "Full Source", engine.py, writes
 *   at the token's position and then attends over everything up to it).
 *   A context length of 0 yields a zero output row.
 * Block tables: block_tables[b, i] is the physical block of logical block i
 *   of sequence b (positions 16*i .. 16*i+15).  Only the first
 *   ceil(context_lens[b] / block_size) entries are read; the rest may hold
 *   anything (e.g. -1).  Positions >= context_lens[b] are never read, so stale
 *   or poisoned slots in a sequence's last block do not matter.
 * Head mapping: query head h reads KV head h / (q_heads / kv_heads).
 * Errors: each call returns a pa_status.  Argument errors are detected on the
 *   host before anything is enqueued; a failed launch returns PA_ERR_HIP.
 *   pa_last_error() returns a message for the calling thread's last failure.
 *   Device-side preconditions (the host cannot read device memory):
 *   block-table entries that are read lie in [0, num_blocks), 0 <=
 *   context_lens[b] <= min(max_context_len, max_blocks_per_seq * block_size),
 *   slots are < num_blocks * block_size (or negative: skipped), and
 *   query_start offsets are non-decreasing within [0, total_query_tokens].
 *   The kernels clamp every index they form, so a violation gives an
 *   unspecified result (e.g. positions past max_context_len are not attended
 *   to) but never an access outside the buffers.  The release library does
 *   not report violations; the debug library (libpa_debug.so, built with
 *   PA_DEVICE_CHECKS=1, same ABI) records each kind in a per-GPU status word
 *   that pa_device_check_status reads.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, inconsistent sizes, bad enum   */
  PA_ERR_UNSUPPORTED = -2,  /* valid but not built: dtype triple, head_dim, */
                            /* group size or block size                     */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or too small               */
  PA_ERR_HIP = -4           /* the HIP runtime reported a launch failure    */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_INT8 = 2 } pa_dtype;

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * Device-side precondition checks (debug library only).  Bits of the status
 * word: a block-table entry read outside [0, num_blocks); a context length
 * below 0 or past max_blocks_per_seq * block_size; a context length past
 * max_context_len (its positions beyond the pieces the grid covers are not
 * attended to); a cache slot >= num_blocks * block_size; query_start offsets
 * decreasing, past total_query_tokens or a sequence with more than
 * max_query_tokens tokens.
 */
#define PA_CHECK_TABLE_ENTRY   1u
#define PA_CHECK_CONTEXT_TABLE 2u
#define PA_CHECK_CONTEXT_MAX   4u
#define PA_CHECK_SLOT          8u
#define PA_CHECK_QUERY_START   16u

/*
 * pa_device_check_status -- the current GPU's check status word: the OR of the
 * PA_CHECK_* bits of every violation the library's kernels met since it was
 * last cleared (clear != 0 clears it after the read).  Synchronises the
 * device (hipDeviceSynchronize) and copies 4 bytes to the host: a debugging
 * aid, not for a step loop.  The release library has no checks: it sets
 * *flags = 0 and returns PA_ERR_UNSUPPORTED.
 */
int pa_device_check_status(unsigned* flags, int clear);

/* Message describing the calling thread's most recent non-OK status. */
const char* pa_last_error(void);

/*
 * pa_reshape_and_cache -- write new tokens' K and V into their cache slots.
 *
 * For each token i with slot_mapping[i] >= 0 and every KV head g:
 *   k_cache[g, slot / block_size, slot % block_size, :] = key[i, g, :]
 *   v_cache[g, slot / block_size, slot % block_size, :] = value[i, g, :]
 * Tokens with a negative slot are skipped (padding rows).  Bits are copied
 * unchanged; no other byte of either cache is touched.  Slots follow "From
 * 183 ms to 19 ms per decode step", "Four changes", changes 2 and 4: a flat
 * index over the (block, offset) slots of one head.
 *
 * key, value    [num_tokens, kv_heads, head_dim], dtype kv_dtype
 * k_cache, v_cache [kv_heads, num_blocks, block_size, head_dim], kv_dtype
 * slot_mapping  [num_tokens] int64
 * kv_dtype      PA_F32, PA_BF16 or PA_INT8.  For an int8 cache the codes are
 *               copied as given: quantising them with the block's scale
 *               (k_scale / v_scale, which this call does not touch) is the
 *               caller's part.
 * head_dim      64 or 128; block_size 16.  num_tokens == 0 is a no-op.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int kv_heads,
                         int head_dim, int num_blocks, int block_size, int kv_dtype,
                         void* stream);

/*
 * pa_reshape_and_cache_quant -- write new tokens into an int8 cache,
 * requantizing each target block ("A Rust inference server for Qwen2 on Apple
 * Silicon", "Day 4 measurements -- int8 KV", "Partial blocks").
 *
 * For each token i with slot_mapping[i] >= 0, in index order, and every KV
 * head g, with block p = slot / block_size and offset o = slot % block_size:
 *   X = k_cache[g, p] * k_scale[g, p]         (fp32, the 16 rows of the block)
 *   X[o, :] = key[i, g, :]
 *   k_scale[g, p] = max|X| / 127               (1 when X is all zero)
 *   k_cache[g, p] = clip(rint(X / k_scale[g, p]), -127, 127)
 * and the same for value / v_cache / v_scale.  Every step is an fp32
 * operation (rint rounds half to even), so the codes are exact functions of
 * the inputs.  Unwritten slots hold code 0 and never raise the maximum; a
 * value on the grid comes back unchanged while the scale does not change.
 * Tokens aimed at the same block in one call act as consecutive calls.
 *
 * key, value    [num_tokens, kv_heads, head_dim], in_dtype PA_BF16 or PA_F32
 * k_cache, v_cache [kv_heads, num_blocks, block_size, head_dim] int8
 * k_scale, v_scale [kv_heads, num_blocks] fp32, read and written
 * slot_mapping  [num_tokens] int64; negative = skip
 * head_dim 64 or 128; block_size 16; num_blocks * block_size < 2^31.
 */
int pa_reshape_and_cache_quant(const void* key, const void* value, int8_t* k_cache,
                               int8_t* v_cache, float* k_scale, float* v_scale,
                               const int64_t* slot_mapping, int num_tokens, int kv_heads,
                               int head_dim, int num_blocks, int block_size, int in_dtype,
                               void* stream);

/*
 * Split-K over context.  A sequence's context is cut into consecutive pieces
 * of `split_tokens` positions (a multiple of block_size); each piece is
 * reduced to a partial (normalised output, log-sum-exp) pair in fp32, and a
 * second launch merges each row's pieces in piece order: with
 * M = max_s lse_s and w_s = exp(lse_s - M), out = sum_s w_s o_s / sum_s w_s.  This is the online-softmax rescaling
 * applied across pieces instead of across tiles.  The piece length depends
 * only on the arguments given here, never on the lengths in the batch, so a
 * sequence's result does not depend on what it is batched with.
 *
 * pa_default_split_tokens returns the piece length used when a call passes
 * split_tokens = 0 (num_query_tokens is 1 for pa_decode): 1024 * kv_heads
 * clamped to [2048, 4096] for calls that run on the matrix cores (pa_verify;
 * pa_decode over an int8 cache or with bf16 groups of 4 or more query heads
 * per KV head), else 64 * kv_heads clamped to [128, 512].
 */
int pa_default_split_tokens(int num_query_tokens, int q_heads, int kv_heads, int head_dim,
                            int kv_dtype);

/*
 * Workspace bytes pa_decode / pa_verify need for these sizes (0 when one
 * piece covers max_context_len).  num_query_tokens is 1 for pa_decode.
 * Returns 0 and sets pa_last_error on invalid sizes.
 */
size_t pa_workspace_size(int num_seqs, int num_query_tokens, int q_heads, int kv_heads,
                         int head_dim, int max_context_len, int kv_dtype, int split_tokens);

/*
 * pa_decode -- one query token per sequence over the paged cache.
 *
 * out[b, h, :] = softmax_j(scale * <q[b, h, :], K_b[j, :]>) @ V_b[j, :]
 * over positions j < context_lens[b], with K_b / V_b read in place through
 * block_tables from KV head h / G.  ("From 183 ms to 19 ms per decode step",
 * "Four changes", change 3; the per-row formula of "Anatomy of a Decode-Step
 * Stall", "Full Source", engine.py.)
 *
 * out           [num_seqs, q_heads, head_dim], dtype q_dtype
 * q             [num_seqs, q_heads, head_dim], dtype q_dtype
 * k_cache, v_cache [kv_heads, num_blocks, block_size, head_dim], kv_dtype
 * k_scale, v_scale [kv_heads, num_blocks] fp32; required for PA_INT8, else
 *               ignored (may be NULL)
 * block_tables  [num_seqs, max_blocks_per_seq] int32
 * context_lens  [num_seqs] int32
 * max_context_len  host-side upper bound of context_lens (sizes the grid and
 *               the workspace; does not change the arithmetic)
 * scale         softmax scale (typically 1/sqrt(head_dim))
 * split_tokens  piece length, a multiple of block_size in [16, 4096], or 0
 *               for pa_default_split_tokens()
 * workspace     device scratch of at least pa_workspace_size(...) bytes,
 *               256-byte aligned (may be NULL when that size is 0); it holds
 *               the pieces' partial outputs.  Its contents on entry are
 *               ignored.  Calls sharing one workspace must be ordered on one
 *               stream.
 * Supported: head_dim 64 or 128; block_size 16; q_heads / kv_heads in 1..8
 * or 16; the dtype triples listed at the top.
 * Precision: scores, softmax and the weighted sum accumulate in fp32.  Over a
 * bf16 cache the softmax weights are rounded to bf16 (to nearest even) for the
 * weighted sum of V and the row's sum of weights adds those rounded weights,
 * so each output row is a weighted mean of V rows whose weights sum to 1; over
 * an fp32 cache the weights stay fp32; over an int8 cache see pa_verify.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
              int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
              int max_context_len, float scale, int q_dtype, int kv_dtype, int split_tokens,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same call without a workspace argument.
 *
 * The split-K partials go to a fixed array of PA_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on, from the first such call on
 * that GPU until the process ends.  Nothing is allocated or freed per call.
 * Results are those of pa_decode with the same arguments, bit for bit (same
 * kernels).  Sizes whose partials exceed the array (pa_workspace_size(...) >
 * PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU uses that GPU's single array: calls that
 * may overlap on one GPU (different streams without ordering between them)
 * race and give unspecified results; calls ordered on one stream are safe.
 * The array's contents between calls are not part of the result (each call
 * writes every partial it reads).  Other arguments as pa_decode.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
                      int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int q_dtype, int kv_dtype,
                      int split_tokens, void* stream);

/*
 * pa_decode_append -- pa_reshape_and_cache of one new token per sequence
 * followed by pa_decode, in one launch (the kernel pa_decode would run for
 * the shape: vector ALUs for fp32 and bf16 groups below 4 query heads per KV
 * head, matrix cores for larger bf16 groups), with pa_decode's result bit for
 * bit.
 *
 * key, value     [num_seqs, kv_heads, head_dim], kv_dtype: the new token of
 *                each sequence, written to slot_mapping[b] (skipped when
 *                negative) exactly as pa_reshape_and_cache writes it.
 * The attention covers positions 0 .. context_lens[b] - 1, where position
 * context_lens[b] - 1 is the new token: its K/V are taken from key/value
 * directly.  The result equals pa_reshape_and_cache followed by pa_decode
 * whenever slot_mapping[b] is the slot of position context_lens[b] - 1, which
 * is what a decode step passes (the write-then-attend order of "Anatomy of a
 * Decode-Step Stall", "Full Source", engine.py).  For a padding row (negative
 * slot) nothing is written and the row's output is unspecified.
 * Other arguments as pa_decode.  Caches: PA_F32 or PA_BF16 (an int8 cache
 * returns PA_ERR_UNSUPPORTED: pa_decode_append_quant writes int8 caches).
 */
int pa_decode_append(void* out, const void* q, const void* key, const void* value,
                     void* k_cache, void* v_cache, const int64_t* slot_mapping,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                     int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pa_decode_append_quant -- pa_reshape_and_cache_quant of one new token per
 * sequence followed by pa_decode over the int8 cache, in one launch of the
 * matrix-core kernel, with the two calls' results bit for bit: the same codes
 * and scales in the cache, the same output.  The workgroup that reads the
 * block holding position context_lens[b] - 1 requantizes it as the write does
 * ("A Rust inference server for Qwen2 on Apple Silicon", "Day 4 measurements
 * -- int8 KV", "Partial blocks": the 16 rows dequantized with the old scale,
 * the new row put in, the scale recomputed as max|x| / 127, every value
 * requantized), attends over the new codes and scale, and stores them.
 *
 * key, value     [num_seqs, kv_heads, head_dim], in_dtype (PA_BF16 or PA_F32).
 * k_cache, v_cache  int8 [kv_heads, num_blocks, block_size, head_dim];
 * k_scale, v_scale  fp32 [kv_heads, num_blocks], read and written.
 * slot_mapping   [num_seqs] int64: the slot of position context_lens[b] - 1
 *                (negative: nothing is written and the row's output is
 *                unspecified; slots past the pool are ignored).
 * q, out         bf16 [num_seqs, q_heads, head_dim].
 * Other arguments as pa_decode; groups of at most 16 query heads per KV head.
 * The results equal pa_reshape_and_cache_quant followed by pa_decode whenever
 * each slot is the slot of its sequence's position context_lens[b] - 1 and no
 * two sequences share a block (what a decode step passes).
 */
int pa_decode_append_quant(void* out, const void* q, const void* key, const void* value,
                           int in_dtype, int8_t* k_cache, int8_t* v_cache, float* k_scale,
                           float* v_scale, const int64_t* slot_mapping,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int q_heads, int kv_heads, int head_dim, int block_size,
                           int num_blocks, int max_blocks_per_seq, int max_context_len,
                           float scale, int split_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * pa_verify -- T = num_query_tokens new tokens per sequence (a speculative
 * verify step of k+1 tokens), causal among themselves.
 *
 * context_lens[b] counts the cached positions INCLUDING the T new tokens,
 * whose K/V must already be in the cache.  Query token t (0-based) sits at
 * position context_lens[b] - T + t and attends to positions
 * 0 .. context_lens[b] - T + t.  ("From 183 ms to 19 ms per decode step",
 * section "Then speculative decoding got slower"; causal slicing as in the
 * prefill code of "Anatomy of a Decode-Step Stall", "Full Source".)
 * A sequence with context_lens[b] < T has no position for its earliest
 * tokens; those rows see positions 0 .. context_lens[b] - T + t only, and a
 * row that sees none returns zeros.
 *
 * out, q        [num_seqs, num_query_tokens, q_heads, head_dim], q_dtype
 * other arguments as pa_decode.  Any num_query_tokens and group size: the
 * num_query_tokens * (q_heads / kv_heads) query rows of a (sequence, KV head)
 * take one to three 16-row matrix-core tiles that share every K and V read
 * (up to 48 rows, with split-K pieces as pa_decode); beyond 48 rows the call
 * runs on the prefill kernel (pa_prefill's definition, which is this one; no
 * pieces, the workspace and a work plan are then not used).
 * Supported dtypes: PA_BF16 q with a PA_BF16 or PA_INT8 cache (bf16 output;
 * int8 needs k_scale / v_scale); head_dim 64 or 128.  Scores and the output
 * accumulate in fp32 on the matrix cores.  The softmax weights are rounded to
 * bf16 (to nearest even) for the weighted sum of V -- over an int8 cache each
 * weight times its block's V scale, against the exact codes -- and the row's
 * sum of weights adds the rounded weights (an int8 block's divided by its V
 * scale again), so numerator and denominator use one set of weights.
 * int8 caches: the scores are fp16 products: q is converted to fp16 (to
 * nearest even; exact for bf16 values of magnitude 6.1e-5 .. 65504, infinite
 * past it), the codes exactly.  The V scales of the blocks read must be
 * positive and finite.
 */
int pa_verify(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int num_query_tokens, int q_heads,
              int kv_heads, int head_dim, int block_size, int num_blocks,
              int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
              int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Work plans -- the order in which a call's work is started.
 *
 * pa_decode and pa_verify split their work into one unit per (sequence, piece
 * of context, KV head) and start the units in a fixed natural order.  Each
 * unit's arithmetic depends on the unit alone, so the order changes no bit of
 * any result; it changes how evenly the GPU is loaded.  With lengths that
 * differ, a long unit that happens to start late finishes the launch alone;
 * started longest first, the long units overlap the short ones.  A plan is
 * that order, computed on the device from the step's lengths.  The decode
 * step of "From 183 ms to 19 ms per decode step" ("Four changes, one profile
 * at a time", change 4) hands every layer the same block tables and lengths,
 * so one pa_plan per step serves the attention calls of all its layers.
 *
 * pa_plan_size -- bytes of a plan for these sizes (arguments as
 *   pa_workspace_size; num_query_tokens is 1 for decode, T for verify, and
 *   split_tokens 0 resolves as in the attention calls).  Returns 0 and sets
 *   pa_last_error on invalid sizes or when num_seqs * ceil(max_context_len /
 *   split_tokens) exceeds 8192 units.
 *
 * pa_plan -- writes the plan: the (sequence, piece) units sorted by their
 *   tile count, longest first (units of equal length in any order), each with
 *   its sequence, piece, context length and a COPY of the piece's block-table
 *   entries.  block_tables and context_lens as for pa_decode (device memory,
 *   read by the plan kernel on `stream`); plan: device memory of at least
 *   pa_plan_size(...) bytes, 16-byte aligned, written entirely by this call.
 *   The other arguments must be those of the attention calls that use it.
 *
 * pa_decode_planned, pa_decode_append_planned, pa_decode_append_quant_planned,
 * pa_verify_planned -- pa_decode, pa_decode_append, pa_decode_append_quant
 *   and pa_verify, started in the plan's order, with results
 *   identical bit for bit to the unplanned calls.  plan / plan_bytes: a plan
 *   from pa_plan (plan_bytes >= pa_plan_size(...) for the call's sizes, else
 *   PA_ERR_INVALID_ARG).  The call takes each unit's length and block-table
 *   entries from the plan, not from block_tables / context_lens: the plan must
 *   be made again whenever the tables or lengths change (in a decode step:
 *   once, after the step's tables and lengths are written, before the first
 *   layer).  A plan made for other sizes (sequences, piece length, table
 *   width) is detected on the device and ignored: the call then runs in the
 *   natural order.  Calls that use one plan may run concurrently; pa_plan
 *   must not overwrite it while they run.
 */
size_t pa_plan_size(int num_seqs, int num_query_tokens, int q_heads, int kv_heads,
                    int head_dim, int max_context_len, int kv_dtype, int split_tokens);

int pa_plan(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
            int num_query_tokens, int q_heads, int kv_heads, int head_dim,
            int max_blocks_per_seq, int max_context_len, int kv_dtype, int split_tokens,
            void* plan, size_t plan_bytes, void* stream);

int pa_decode_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
                      int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int q_dtype, int kv_dtype,
                      int split_tokens, void* workspace, size_t workspace_bytes,
                      const void* plan, size_t plan_bytes, void* stream);

int pa_decode_append_planned(void* out, const void* q, const void* key, const void* value,
                             void* k_cache, void* v_cache, const int64_t* slot_mapping,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int q_heads, int kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_blocks_per_seq,
                             int max_context_len, float scale, int q_dtype, int kv_dtype,
                             int split_tokens, void* workspace, size_t workspace_bytes,
                             const void* plan, size_t plan_bytes, void* stream);
int pa_decode_append_quant_planned(void* out, const void* q, const void* key,
                                   const void* value, int in_dtype, int8_t* k_cache,
                                   int8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, const int32_t* block_tables,
                                   const int32_t* context_lens, int num_seqs, int q_heads,
                                   int kv_heads, int head_dim, int block_size, int num_blocks,
                                   int max_blocks_per_seq, int max_context_len, float scale,
                                   int split_tokens, void* workspace, size_t workspace_bytes,
                                   const void* plan, size_t plan_bytes, void* stream);

int pa_verify_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int num_query_tokens,
                      int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                      int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                      const void* plan, size_t plan_bytes, void* stream);

/*
 * pa_verify_varlen -- pa_verify with a number of new tokens per sequence:
 * T_b = query_start[b + 1] - query_start[b] (0 .. max_query_tokens), where
 * the pages pad every sequence to k+1 ("From 183 ms to 19 ms per decode
 * step", "Then speculative decoding got slower").  Each sequence is exactly
 * the pa_verify of that sequence with T = T_b: query token t attends to
 * positions 0 .. context_lens[b] - T_b + t.
 *
 * out, q        [total_query_tokens, q_heads, head_dim], bf16; sequence b's
 *               tokens are rows query_start[b] .. query_start[b + 1] - 1.
 * query_start   [num_seqs + 1] int32, non-decreasing, query_start[0] = 0,
 *               query_start[num_seqs] = total_query_tokens (device memory,
 *               not checked by the host; out-of-range offsets are clamped so
 *               that nothing outside q / out is touched).  Rows of out that
 *               belong to no sequence are not written.
 * total_query_tokens  <= num_seqs * max_query_tokens, else PA_ERR_INVALID_ARG;
 *               0: nothing is read or written (out and q may be NULL).
 * max_query_tokens    the largest T_b (beyond 48 rows per (sequence, KV
 *               head) the call runs on the prefill kernel, as pa_verify).
 * split_tokens  0 = the matrix-core default (pa_default_split_tokens with
 *               num_query_tokens >= 2), so a sequence's result does not depend
 *               on the other sequences of the call.
 * workspace     pa_workspace_size(num_seqs, max_query_tokens, ...) bytes
 *               suffice.
 * Other arguments, dtypes and limits as pa_verify.
 */
int pa_verify_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const float* k_scale, const float* v_scale, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                     int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                     int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                     int max_context_len, float scale, int q_dtype, int kv_dtype,
                     int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill -- chunked prefill over the paged cache: many new tokens per
 * sequence, causal among themselves (the next kernel on the roadmap of "From
 * 183 ms to 19 ms per decode step", section "Limits").  The result is the one
 * pa_verify_varlen defines -- sequence b's T_b = query_start[b + 1] -
 * query_start[b] new tokens are its last T_b positions (their K/V already in
 * the cache, e.g. by pa_reshape_and_cache), query token t attends to positions
 * 0 .. context_lens[b] - T_b + t -- without its limit on rows: any
 * max_query_tokens, any group size.  Each workgroup covers 128 query rows
 * (token, head) of one (sequence, KV head) over their whole visible context,
 * so there are no pieces and no workspace.
 *
 * out, q        [total_query_tokens, q_heads, head_dim], bf16, packed by
 *               sequence as in pa_verify_varlen (rows of out belonging to no
 *               sequence are not written).
 * query_start   [num_seqs + 1] int32 device offsets (clamped on the device to
 *               [0, total_query_tokens] and to max_query_tokens per sequence).
 * total_query_tokens  <= num_seqs * max_query_tokens, else PA_ERR_INVALID_ARG;
 *               0: nothing is read or written (out and q may be NULL).
 * max_query_tokens  the largest T_b (sets the grid).
 * Supported: PA_BF16 q with a PA_BF16 or PA_INT8 cache (k_scale / v_scale
 * for int8); head_dim 64 or 128; block_size 16.  Other arguments as
 * pa_decode; max_context_len is only checked against the table width.
 * Precision: products on the matrix cores with fp32 accumulation; weights
 * rounded and summed as pa_verify describes (the same ranges hold for int8
 * caches).
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const float* k_scale, const float* v_scale, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
               int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
               int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
               int max_context_len, float scale, int q_dtype, int kv_dtype, void* stream);

/*
 * Prefill work plans -- pa_prefill's (sequence, tile of query rows) units in
 * the order they are started, longest first.
 *
 * A prefill tile's work is the number of cached positions its last query row
 * sees (causal); with chunks on top of prior contexts of different lengths the
 * tiles differ many times over, and in the natural order (later tiles of every
 * sequence first) the longest can end the launch alone.  A plan orders the
 * tiles by that length (in 256 buckets of equal width).  Each tile's
 * arithmetic does not depend on the order: pa_prefill_planned gives the bits
 * pa_prefill gives.
 *
 * pa_prefill_plan_size -- bytes of a plan (0 and pa_last_error on invalid
 *   sizes or more than 8192 units; units = num_seqs * ceil(max_query_tokens *
 *   (q_heads / kv_heads) / rows per workgroup)).
 * pa_prefill_plan -- writes the plan from context_lens and query_start (the
 *   pa_prefill arguments; device memory read on `stream`).  It holds copies of
 *   the offsets and lengths: make it again whenever they change.
 * pa_prefill_planned -- pa_prefill started in the plan's order.  plan_bytes
 *   must be at least pa_prefill_plan_size(...) for the call's sizes, else
 *   PA_ERR_INVALID_ARG; a plan made for other sizes is detected on the device
 *   and ignored (natural order).
 */
size_t pa_prefill_plan_size(int num_seqs, int max_query_tokens, int q_heads, int kv_heads);

int pa_prefill_plan(const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                    int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                    int max_blocks_per_seq, void* plan, size_t plan_bytes, void* stream);

int pa_prefill_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                       int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                       int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                       int max_context_len, float scale, int q_dtype, int kv_dtype,
                       const void* plan, size_t plan_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
