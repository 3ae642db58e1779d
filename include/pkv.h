/*
 * pkv.h - attention over a block-paged KV cache on AMD MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Every kernel entry point takes plain pointers and sizes,
 * enqueues its kernels on the caller's HIP stream and returns at once.  The
 * library allocates no device memory and its kernel entry points keep no state
 * between calls; they are safe to call from several threads on distinct
 * buffers.  The one exception is paged_decode_attention_noalloc, whose
 * workspace is a static device array of the library (one per GPU).  The block manager (pkv_bm_*) is host-only state in a handle the
 * caller creates and destroys.
 *
 * Common conventions
 *   - "device" pointers are HIP device (or managed) memory; every tensor is
 *     contiguous and row-major in the shape given; every data pointer must be
 *     16-byte aligned.
 *   - dtype: PKV_F32 or PKV_BF16.  q, out, k_new, v_new and both pools share it.
 *     All arithmetic accumulates in fp32; bf16 results are rounded to nearest even.
 *   - KV pool (one per layer; the caller picks the layer by pointer):
 *       k_cache, v_cache : [n_blocks, h_kv, 16, d_h]
 *     A physical block holds 16 consecutive tokens of one sequence; inside a
 *     block the layout is head-major, token, then channel.  This is the paged
 *     pool of fixed 16-token blocks reached through a per-sequence block table
 *     that the LLM Inference Server page describes (Optional Stretch
 *     Challenges, "Paged KV-Cache Block Allocator"), and the "block table /
 *     paged KV slots" box of the pipeline figure on the "LLM Inference Server
 *     From Scratch" page (How it works).
 *   - block_tables : int32 [n_seqs, max_blocks_per_seq]; token t of sequence s
 *     lives in block block_tables[s][t / 16] at offset t % 16.  Entries past
 *     ceil(context_len / 16) are never read.
 *   - context_len counts every token of the sequence including the ones
 *     appended this step (the cache is written first, then attended, as in the
 *     LayerKVCache reference class of the LLM Inference Server page, Starter &
 *     Verification Code Examples).
 *   - Grouped-query attention (the "GQA" of the Attention Kernel box, pipeline
 *     figure, From Scratch page): query head h reads KV head h / (h_q / h_kv).
 *   - stream: the HIP stream the work is enqueued on; NULL is the null stream.
 *
 * Errors: every call returns a pkv_status.  Host-checkable argument errors are
 * reported before any HIP call is made and nothing is enqueued.  Values that
 * live in device memory (slots, table entries, lengths) are the caller's
 * contract and are not read on the host unless the environment variable
 * PKV_DEBUG=1 is set, in which case they are copied to the host (synchronising
 * the stream) and checked; an out-of-range value then returns
 * PKV_ERR_INVALID_ARG.  Without PKV_DEBUG the kernels still never touch memory
 * outside the buffers described by the size arguments: an out-of-range slot is
 * not written, an out-of-range block-table entry is read as block 0 and a
 * context length is clamped to max_blocks_per_seq * 16; the results are then
 * unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared exactly as HIP's runtime header declares it
 * (an identical typedef may be repeated in C11 and C++), so that this header
 * needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

/* PKV_INT8 names the INT8 cache (int8 codes with a float32 scale per token
 * head row, read by bf16 queries); it is accepted by pkv_decode_num_splits and
 * pkv_decode_workspace_bytes_split only. */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_INT8 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad device value (PKV_DEBUG) */
  PKV_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (d_h, dtype), or beyond the
                              size limits: block tables wider than 2^27 - 1 blocks (2^31
                              tokens), decode lines of more than 2^40 block reads */
  PKV_ERR_WORKSPACE = 3,   /* decode workspace missing or too small */
  PKV_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  PKV_ERR_NO_BLOCKS = 5    /* block manager: not enough free blocks; nothing changed */
} pkv_status;

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(int status);

/*
 * kv_append - write the K and V rows of T new tokens into their pool slots, in
 * place.
 *
 * Defined by the pre-allocated cache that is updated in place at the current
 * write position instead of being re-concatenated (LLM Inference Server page,
 * Stage 1 "KV-Cache Engine", pre-allocation task, and its LayerKVCache class),
 * with the write position given as a paged slot ("paged KV slots", pipeline
 * figure of the From Scratch page).
 *
 *   k_new, v_new : device [T, h_kv, d_h]; row i is token i's K (resp. V).
 *   slot_mapping : device int64 [T]; slot = physical_block * 16 + offset.  A
 *                  negative slot skips that token (padding).  Two tokens with
 *                  the same non-negative slot in one call is a caller error (the
 *                  stored row is then one of them, unspecified which).
 *   k_cache, v_cache : device pools, written in place; nothing else changes.
 *   T >= 0 (T == 0 enqueues nothing), h_kv >= 1, d_h in {64, 128}, n_blocks >= 1.
 * The copy is bit-exact.
 */
int kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
              void* k_cache, void* v_cache,
              int T, int h_kv, int d_h, int n_blocks, int dtype, hipStream_t stream);

/*
 * paged_decode_attention - one query token per sequence attends to its whole
 * paged context.
 *
 * out[b, h, :] = sum_t softmax_t(scale * <q[b, h, :], K_b[t, h / g, :]>) V_b[t, h / g, :]
 * over t < context_lens[b], g = h_q / h_kv.  This is the single-token decode
 * step over the cached context of the LLM Inference Server page (Stage 1,
 * prefill/decode task: a decode step feeds only the new token at start_pos =
 * current length) for a continuous batch of variable-length sequences (From
 * Scratch page, What you build).
 *
 *   out : device [B, h_q, d_h];  q : device [B, h_q, d_h]
 *   k_cache, v_cache : device pools [n_blocks, h_kv, 16, d_h]
 *   block_tables : device int32 [B, max_blocks_per_seq]
 *   context_lens : device int32 [B], 0 <= context_lens[b] <= max_context_len.
 *                  A context of length 0 gives an all-zero output row.
 *   max_context_len : host int, an upper bound of context_lens,
 *                  0 <= max_context_len <= max_blocks_per_seq * 16.
 *   scale : the softmax scale (1/sqrt(d_h) for standard attention).
 *   workspace : device scratch of at least
 *                  pkv_decode_workspace_bytes(B, h_q, d_h, max_context_len)
 *                  bytes, 16-byte aligned.  Its contents on entry do not
 *                  matter.  The caller owns it and must not use it
 *                  concurrently with the call.
 * The blocks of all (sequence, KV head) pairs, laid end to end, are cut into
 * one range per wavefront the device holds at once, or fewer where the line
 * is short (at most one range per two blocks of the longest line the
 * arguments allow); ranges of wavefronts on even XCDs are 11/10 the size of
 * those on odd XCDs, which run slower.  Results do not depend on the cut
 * beyond fp32 rounding.  B == 0 enqueues nothing.
 * Requires h_q % h_kv == 0, d_h in {64, 128}; returns PKV_ERR_UNSUPPORTED
 * when B * h_kv * ceil(max_context_len / 16) exceeds 2^40 block reads.
 */
int paged_decode_attention(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int B, int h_q, int h_kv, int d_h, int n_blocks,
                           int max_blocks_per_seq, int max_context_len,
                           float scale, int dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes paged_decode_attention needs for these arguments, whatever
 * h_kv (dividing h_q) and the pool dtype (bf16, fp32 or INT8): an upper bound.
 * Host-only, no HIP call.  0 for B <= 0 or other invalid arguments. */
size_t pkv_decode_workspace_bytes(int B, int h_q, int d_h, int max_context_len);

/*
 * paged_decode_attention_split - paged_decode_attention with the number of
 * ranges set by the caller (for tuning and for tests of the merge):
 *   num_splits : 0 picks the split automatically (as paged_decode_attention);
 *                  otherwise 1 .. 65536 ranges, weighted as in
 *                  paged_decode_attention (one range: the whole line).
 *   workspace : at least pkv_decode_workspace_bytes_split(B, h_q, h_kv, d_h,
 *                  max_context_len, dtype, num_splits) bytes.
 */
int paged_decode_attention_split(void* out, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int B, int h_q, int h_kv, int d_h, int n_blocks,
                                 int max_blocks_per_seq, int max_context_len,
                                 float scale, int dtype, int num_splits,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Exact workspace bytes of a decode call with these arguments (dtype PKV_F32,
 * PKV_BF16 or PKV_INT8; num_splits as for paged_decode_attention_split, 0 =
 * enough for the largest automatic split).  Host-only, no HIP call.  Returns 0
 * for invalid arguments; the call itself then reports the error. */
size_t pkv_decode_workspace_bytes_split(int B, int h_q, int h_kv, int d_h, int max_context_len,
                                        int dtype, int num_splits);

/*
 * paged_decode_attention_noalloc - paged_decode_attention without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The decode workspace is a static device array of
 * 32 MiB inside the library; each GPU the library runs on holds its own copy
 * from the first call on that device until the process ends.  The other
 * arguments, the result and the errors are those of paged_decode_attention,
 * with these differences:
 *   - a call whose workspace would exceed 32 MiB returns PKV_ERR_WORKSPACE
 *     (the size is pkv_decode_workspace_bytes_split(..., num_splits) at the
 *     automatic split count, pkv_decode_num_splits(..., 0); for example
 *     B = 64, h_q = 32, h_kv = 8, d_h = 128, bf16 at 2048 splits needs 8.5 MB);
 *   - stream must belong to the current device (else PKV_ERR_INVALID_ARG);
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (two streams, two threads) race and give undefined results.  Calls
 *     ordered on one stream are safe; nothing in the array needs clearing.
 */
int paged_decode_attention_noalloc(void* out, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int B, int h_q, int h_kv, int d_h, int n_blocks,
                                   int max_blocks_per_seq, int max_context_len,
                                   float scale, int dtype, hipStream_t stream);

/*
 * INT8 KV cache.  The cached K and V are quantised dynamically to int8 per
 * token head (LLM Inference Server page, Optional Stretch Challenges, "INT8
 * KV-Cache Quantization") with the symmetric absmax rule of the same page
 * (Required Mathematical Concepts): for each row x of d_h values that one token
 * holds for one KV head, s = max(max|x|, 1e-8) / 127 and x_q = round(x / s),
 * computed in float32 with a true division and rounding half to even, as in the
 * page's reference INT8 layer (Starter & Verification Code Examples).  The
 * cache holds x_hat = s * x_q.
 *
 *   k_cache, v_cache : device int8 [n_blocks, h_kv, 16, d_h] (codes, laid out
 *                      like the bf16 pools)
 *   k_scale, v_scale : device float32 [n_blocks, h_kv, 16] (s of each row),
 *                      16-byte aligned (kv_append_int8 needs 4)
 */

/*
 * kv_append_int8 - quantise the K and V rows of T new tokens and write codes
 * and scales to their pool slots, in place.  Arguments as for kv_append;
 * dtype (PKV_F32 or PKV_BF16) is that of k_new and v_new.  The codes and
 * scales are bit-exact against the rule above.
 */
int kv_append_int8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                   int T, int h_kv, int d_h, int n_blocks, int dtype, hipStream_t stream);

/*
 * paged_decode_attention_int8 - paged_decode_attention over an INT8 cache:
 * the same result with K and V replaced by x_hat = s * x_q.  q and out are
 * bf16; the codes are widened exactly in registers, the K scale multiplies the
 * score and the V scale the softmax weight (weights rounded to bf16 as in the
 * bf16 decode; accumulation in fp32).  Other arguments are as for
 * paged_decode_attention_split; the workspace is sized by
 * pkv_decode_workspace_bytes (any num_splits == 0 call) or
 * pkv_decode_workspace_bytes_split with dtype PKV_INT8.
 */
int paged_decode_attention_int8(void* out, const void* q,
                                const int8_t* k_cache, const int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int B, int h_q, int h_kv, int d_h, int n_blocks,
                                int max_blocks_per_seq, int max_context_len, float scale,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Inspection of the decode's cut (host-only, no HIP call; the kernels use the
 * same code).  The blocks of all (sequence, KV head, head chunk) segments,
 * laid end to end, form a line of `total` blocks, cut into `splits` ranges;
 * wave w of the decode grid streams positions
 * [pkv_decode_line_start(total, splits, w), ...start(total, splits, w + 1)).
 * Waves 4k .. 4k + 3 run on XCD k mod 8, and a wave of an even XCD takes 11
 * blocks for every 10 of a wave of an odd XCD (odd XCDs stream slower).
 *   pkv_decode_line_start : 0 <= w <= splits; returns -1 on invalid arguments
 *                           (total in 0 .. 2^40, splits in 1 .. 65536).
 *   pkv_decode_line_wave_of : the wave whose range holds position p,
 *                           0 <= p < total; -1 on invalid arguments. */
int64_t pkv_decode_line_start(int64_t total, int splits, int w);
int pkv_decode_line_wave_of(int64_t total, int splits, int64_t p);

/* Number of splits a decode call uses for these arguments; -1 on invalid
 * arguments.  With num_splits == 0 it queries the current device's occupancy
 * for the decode kernel (2048 wavefronts are assumed when no device can be
 * queried). */
int pkv_decode_num_splits(int B, int h_q, int h_kv, int d_h, int max_context_len, int dtype,
                          int num_splits);

/*
 * paged_prefill_attention - causal attention of the new prompt tokens of S
 * sequences over their paged contexts (chunked prefill).
 *
 * The prompt is processed in parallel (LLM Inference Server page, Stage 1,
 * prefill/decode task: q_len = prompt length) with causal masking (Attention
 * Kernel box of the pipeline figure and "What you build", From Scratch page).
 * Query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 are the n_s newest tokens
 * of sequence s, at positions context_lens[s] - n_s .. context_lens[s] - 1; the
 * query at position p attends to keys 0..p inclusive.  Their K/V must already
 * be in the pool (kv_append first, on the same stream).
 *
 *   out, q : device [T_q, h_q, d_h], rows packed by sequence.
 *   cu_seqlens_q : device int32 [S + 1], cu_seqlens_q[0] = 0,
 *                  cu_seqlens_q[S] = T_q, n_s <= context_lens[s].
 *   k_cache, v_cache, block_tables [S, max_blocks_per_seq], context_lens [S]:
 *                  as for decode.
 *   max_q_len : host int, an upper bound of every n_s.
 * S == 0 or T_q == 0 enqueues nothing.  bf16 only (the QK^T and PV
 * contractions run on bf16 matrix cores); PKV_F32 returns PKV_ERR_UNSUPPORTED.
 */
int paged_prefill_attention(void* out, const void* q, const int32_t* cu_seqlens_q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int S, int T_q, int max_q_len, int h_q, int h_kv, int d_h,
                            int n_blocks, int max_blocks_per_seq, float scale, int dtype,
                            hipStream_t stream);

/*
 * paged_prefill_attention_int8 - paged_prefill_attention over an INT8 cache:
 * the same causal chunked prefill with K and V replaced by x_hat = s * x_q,
 * for chunked prefill, prefill after a prefix-cache hit and multi-token
 * decode over a cache quantised as above.  q and out are bf16 [T_q, h_q, d_h];
 * k_cache, v_cache, k_scale, v_scale as for paged_decode_attention_int8
 * (scale pools 16-byte aligned); the other arguments as for
 * paged_prefill_attention.  The codes are widened exactly to bf16 for the
 * matrix products; the K scale multiplies each score and the V scale each
 * softmax weight, which is rounded to bf16 as in the bf16 prefill;
 * accumulation is in fp32.  Slots past a sequence's context are never used,
 * whatever they hold.
 */
int paged_prefill_attention_int8(void* out, const void* q, const int32_t* cu_seqlens_q,
                                 const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int S, int T_q, int max_q_len, int h_q, int h_kv, int d_h,
                                 int n_blocks, int max_blocks_per_seq, float scale,
                                 hipStream_t stream);

/*
 * Block copies between KV pools.
 *
 * A pool set is the pools of one layer that share one block numbering: the K
 * and V pools, plus k_scale and v_scale for the INT8 cache.  Block b of a pool
 * whose blocks are block_bytes long is bytes [b * block_bytes, (b + 1) *
 * block_bytes) from its base; the copies are whole blocks, bit for bit.
 *
 *   pools, src_pools, dst_pools, block_bytes : HOST arrays of n_pools entries,
 *       1 <= n_pools <= 8.  Each pool pointer is 16-byte aligned memory the GPU
 *       can reach: device memory, or (swap_blocks) pinned host memory from
 *       hipHostMalloc, which the kernel reads or writes through its device
 *       mapping over PCIe.  Pageable host memory returns PKV_ERR_INVALID_ARG.
 *       block_bytes[i] > 0, a multiple of 16, the same for source and
 *       destination pool i.
 *   pairs : int32 [n_pairs, 2] of (source block, destination block), device
 *       memory or pinned host memory.  n_pairs == 0 enqueues nothing.  A pair
 *       with an index outside [0, n_blocks) is skipped (and rejected under
 *       PKV_DEBUG=1, as is a destination named twice).
 * The pointer checks query the runtime (hipPointerGetAttributes) but enqueue
 * nothing; the copy is one kernel on stream.
 */

/*
 * copy_blocks - within one pool set, block dst of every pool becomes a copy of
 * block src: the copy on write of a shared, partly filled block before a
 * sequence appends into it (LLM Inference Server page, Stage 1 "KV-Cache
 * Engine", prefix-cache task: sequences with the same system prompt share its
 * blocks).  n_blocks: blocks of each pool.  No block may be both a source and
 * a destination in one call (the copies run in parallel).
 */
int copy_blocks(void* const* pools, const int64_t* block_bytes, int n_pools, int n_blocks,
                const int32_t* pairs, int n_pairs, hipStream_t stream);

/*
 * swap_blocks - between two pool sets (device and pinned host, either way, or
 * two device sets): block dst of dst_pools[i] becomes a copy of block src of
 * src_pools[i].  This moves a preempted sequence's blocks out of HBM and back
 * in (the scheduler's preemption in the pipeline figure of the From Scratch
 * page, How it works).  n_src_blocks, n_dst_blocks: blocks of each source and
 * destination pool.  src_pools[i] == dst_pools[i] returns PKV_ERR_INVALID_ARG
 * (use copy_blocks within one set); the two sets must not overlap.
 */
int swap_blocks(const void* const* src_pools, void* const* dst_pools, const int64_t* block_bytes,
                int n_pools, int n_src_blocks, int n_dst_blocks, const int32_t* pairs,
                int n_pairs, hipStream_t stream);

/*
 * Block manager (host-only; no HIP call).  It decides which physical block of a
 * pool holds each token of each sequence: the block tables and slots that the
 * calls above take.  It is the block pool with per-sequence block tables of
 * the LLM Inference Server page (Optional Stretch Challenges, "Paged KV-Cache
 * Block Allocator"), with blocks shared across requests (Mini inference engine
 * page, section 2), the prefix cache with hit/miss counts (hash-keyed there, exact here) whose
 * second request sharing a system prompt skips prefill on it (LLM Inference
 * Server page, Stage 1 "KV-Cache Engine", prefix-cache task; From Scratch page,
 * "Take it further"), a fixed budget that rejects what does not fit so the
 * caller can queue it (Stage 1, footprint-calculator task), and swapping of
 * preempted sequences (the preempt/swap of the Scheduler box, pipeline figure,
 * From Scratch page).  The device memory itself stays the caller's: the
 * manager returns the copies to make, and the caller runs copy_blocks /
 * swap_blocks BEFORE the kv_append of the same step.
 *
 * Policy:
 *   - Free blocks form one FIFO queue, initially 0..n_blocks-1.  Allocation
 *     takes the head; a block whose last holder lets go joins the tail; a freed
 *     sequence lets go of its blocks last block first.
 *   - With prefix_cache != 0, every block that holds tokens stays indexed by
 *     (the tokens before it, the tokens it holds) until it is reallocated, held
 *     or not.  A new prompt is matched block by block: among the indexed
 *     blocks with the same preceding tokens, the one sharing the longest run of
 *     leading tokens with the prompt's block (ties: the lowest id).  A whole
 *     16-token match continues with the next block, a shorter one ends the
 *     match; the matched tokens are reported as cached.  The match stops
 *     before the prompt's last token, which is always left to the prefill (its
 *     query row gives the next token's logits), so a prompt resubmitted
 *     exactly hits all but that token.  The preceding tokens are keyed
 *     exactly, not by a hash: each run of whole 16-token blocks is interned
 *     once as a node of a trie (parent node, 16 token ids), and a block's key
 *     is the node of the whole blocks before it, so two different prefixes
 *     never share a key.
 *   - Writing a token at offset o of a block another sequence also holds
 *     copies it first to a new block (copy on write: one (src, dst) pair).  A
 *     block held alone that holds more than o tokens drops them and is written
 *     in place.  A copy's source is always still held, so the pairs of one step
 *     never name a block both as a source and as a destination.
 *   - Operations are all or nothing: one that needs more free blocks than
 *     there are returns PKV_ERR_NO_BLOCKS and changes nothing.
 *   - Swap out copies every block of a sequence to host blocks (a FIFO queue
 *     of n_host_blocks of its own) and lets go of the device blocks; swap in
 *     allocates new device blocks and frees the host blocks.
 * A manager is not thread-safe; calls on one handle must not overlap.
 * Sequence ids are the caller's (any int64); an unknown, swapped (where not
 * allowed) or duplicate id returns PKV_ERR_INVALID_ARG.
 */
typedef struct pkv_block_manager pkv_block_manager;

typedef struct {
  int32_t n_blocks, free_blocks;
  int32_t cached_blocks;       /* blocks indexed by the prefix cache, held or free */
  int32_t cached_free_blocks;  /* of those, the ones no sequence holds */
  int32_t n_host_blocks, host_free_blocks, n_sequences;
  int64_t hit_tokens, query_tokens;   /* prompt tokens served from the cache / looked up */
  int64_t hit_requests, requests;     /* prompts with at least one cached token / all */
} pkv_bm_stats;

/* A manager of n_blocks >= 1 device blocks and n_host_blocks >= 0 host blocks;
 * NULL on invalid sizes or out of memory.  Destroy frees it (NULL is a no-op). */
pkv_block_manager* pkv_bm_create(int n_blocks, int n_host_blocks, int prefix_cache);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Admit a prompt of n_tokens token ids (host int32).  Outputs (host):
 *   slots[n_tokens] : the slot of each token, -1 for the *n_cached leading
 *                     tokens already in the pool (kv_append skips negative
 *                     slots, and the prefill runs the last n_tokens - *n_cached
 *                     tokens as a chunked prefill);
 *   cow_pairs[2], *n_cow : at most one copy on write to run first.
 * PKV_ERR_NO_BLOCKS when the pool cannot hold it (nothing changes). */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                        int n_tokens, int64_t* slots, int32_t* cow_pairs, int* n_cow,
                        int* n_cached);

/* Append n_tokens tokens (a decode step: one; a verify step: a few) to a
 * sequence; slots[n_tokens] and at most one copy on write as above. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int n_tokens,
                  int64_t* slots, int32_t* cow_pairs, int* n_cow);

/* One decode step of a batch: token tokens[i] is appended to sequence
 * seq_ids[i] (distinct, resident) for i < n, in that order, as by n calls of
 * pkv_bm_append; slots[n] receives their slots (the step's slot_mapping) and
 * cow_pairs (room for n pairs) the copies on write to run first.  All or
 * nothing: PKV_ERR_NO_BLOCKS if the free queue cannot supply the whole step. */
int pkv_bm_append_batch(pkv_block_manager* bm, int n, const int64_t* seq_ids,
                        const int32_t* tokens, int64_t* slots, int32_t* cow_pairs, int* n_cow);

/* Block tables and context lengths of n resident sequences, laid out as the
 * attention calls take them: tables [n, max_blocks] (host int32, row i holds
 * sequence seq_ids[i]'s blocks, then zeros) and context_lens [n].
 * PKV_ERR_INVALID_ARG if a sequence is unknown, swapped out or has more than
 * max_blocks blocks (nothing written). */
int pkv_bm_block_tables(const pkv_block_manager* bm, int n, const int64_t* seq_ids,
                        int32_t* tables, int max_blocks, int32_t* context_lens);

/* child shares every block of parent (parallel sampling); later writes copy on
 * write. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Lets go of a sequence's blocks (device or host). */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id);

/* Swap a sequence out (pairs = (device block, host block)) or in (pairs =
 * (host block, device block)); pairs has room for max_pairs pairs, one per
 * block of the sequence.  Run swap_blocks on them before the next step. */
int pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs, int max_pairs,
                    int* n_pairs);
int pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs, int max_pairs,
                   int* n_pairs);

/* A resident sequence's block table (host int32, room for max_blocks) and its
 * length.  *n_blocks and *seq_len are set for any known sequence, also when
 * max_blocks is too small or the sequence is swapped out (both return
 * PKV_ERR_INVALID_ARG). */
int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table,
                       int max_blocks, int* n_blocks, int* seq_len);

int pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out);

/* KV-cache bytes of batch sequences of seq_len tokens: the footprint
 * 2 * n_layers * n_kv_heads * d_head * seq_len * bytes_per_elem of the LLM
 * Inference Server page (Required Mathematical Concepts; its
 * compute_kv_cache_bytes task), times batch.  dtype PKV_F32 / PKV_BF16, or
 * PKV_INT8 (one byte per element plus one float32 scale per token head row).
 * paged != 0 rounds each sequence up to whole 16-token blocks.  -1 on invalid
 * arguments. */
int64_t pkv_kv_cache_bytes(int n_layers, int h_kv, int d_h, int64_t batch, int64_t seq_len,
                           int dtype, int paged);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
