/*
 * pagedattn.h -- C ABI of libpagedattn: attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950, CDNA4), with the cache write and block copy
 * that go with it.
 *
 * The method: a sequence's keys and values live in fixed-size blocks of
 * block_size tokens that need not be adjacent in memory; a per-sequence block
 * table maps logical block i (positions i*B .. i*B+B-1) to a physical block.
 * Attention of a query over the sequence is ordinary softmax attention over
 * exactly its context_len valid positions, computed by visiting the blocks
 * where they lie (paper notes "PagedAttention: Efficient Memory Management for
 * Large Language Model Serving with PagedAttention", unpurerationalist.github.io,
 * section 3.1 and its block-wise attention equation; Korean review
 * mz-moonzoo.tistory.com/116, section 4.1).  The three fused kernels of that
 * design -- block write, block read + attention, batched block copy -- are the
 * entry points below (review section 5.1; notes section 4.1).
 *
 * Conventions for every call
 *  - All data pointers are DEVICE pointers allocated by the caller (e.g. by
 *    PyTorch), except where a call says otherwise (host pointer arrays of
 *    pa_copy_blocks and pa_swap_blocks, pinned host pools of pa_swap_blocks,
 *    the host-only block manager).  The library keeps no pointer after a
 *    call returns, allocates no device memory, and holds no mutable global
 *    state: calls are re-entrant (a block manager is an object of its own,
 *    created and destroyed by the caller).  The one exception is
 *    pa_paged_attention_decode_noalloc, whose workspace is a fixed array
 *    the library holds on each device.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns without synchronising.
 *  - Layouts are C-contiguous:
 *      caches      [num_blocks][num_heads][block_size][head_dim]
 *      q, out      [rows][num_heads][head_dim]
 *      block_tables[num_seqs][max_blocks_per_seq]   int32
 *      context_lens[num_seqs]                       int32
 *  - Positions, logical blocks and slots count from 0.  The flat slot of
 *    position p of a sequence is block_tables[s][p / B] * B + p % B
 *    ("KV 캐시 관리와 PagedAttention", llm-systems-engineering.pages.dev,
 *    section on linking token order to storage).
 *  - Supported shapes: head_dim 64 or 128; block_size 4, 8, 16, 32 or 64;
 *    dtype fp32, fp16 or bf16 (the shared-prefix decode: block_size 16 to
 *    64).  All data pointers must be 16-byte aligned.
 *  - Errors are found by synchronous host checks on the scalar arguments and
 *    pointers (never on device data).  On any error the call returns a
 *    non-zero status, enqueues nothing and writes nothing; pa_last_error()
 *    then describes the problem.  PA_ERR_HIP means a launch failed.
 *  - Data-dependent preconditions cannot be checked without a device sync and
 *    are the caller's: table entries of valid positions in [0, num_blocks);
 *    context_lens[s] <= max_context_len <= max_blocks_per_seq * block_size;
 *    slots of one reshape call distinct; copy destinations distinct and not
 *    sources.  The kernels never read or write outside the buffers whatever
 *    the device data holds: a table entry outside [0, num_blocks) makes its
 *    block contribute nothing; a slot outside the pool is skipped; a copy
 *    pair outside the pool is skipped; context lengths are clipped to
 *    [0, min(max_context_len, max_blocks_per_seq * block_size)].
 *  - Debug validation: with PA_DEBUG_VALIDATE=1 in the environment, every
 *    call that reads device index arrays (reshape_and_cache, the decode
 *    calls but the reduce, decode_shared, copy_blocks, swap_blocks,
 *    prefill_chunk) first synchronises `stream`, copies those arrays to the
 *    host and checks the preconditions above -- and for decode_shared that
 *    the groups match the tables, for prefill_chunk that cu_q_lens runs from
 *    0 to total_q with every q_len within max_q_len and its context, for
 *    swap_blocks that pairs lie in their pools with distinct destinations.
 *    At the first violation it returns PA_ERR_INVALID_ARG, pa_last_error()
 *    naming it, and enqueues nothing.  For debugging only: it blocks the
 *    host and cannot run under stream capture (PA_ERR_HIP there).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 3

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, misalignment, inconsistent sizes */
  PA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block_size or dtype */
  PA_ERR_WORKSPACE = 3,   /* decode workspace missing or too small */
  PA_ERR_HIP = 4,         /* a kernel launch failed */
  PA_ERR_NO_BLOCKS = 5    /* block manager: the free pool cannot cover the request */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* PA_ABI_VERSION of the built library. */
int pa_abi_version(void);

/* Static text for a status code. */
const char *pa_status_string(pa_status status);

/* Detail of the last failed call on this thread ("" if none). */
const char *pa_last_error(void);

/*
 * pa_slot_mapping -- the cache slot of each token a step writes.
 *
 * The address translation of "KV 캐시 관리와 PagedAttention"
 * (llm-systems-engineering.pages.dev, section on linking token order to
 * storage): position p of a sequence lies at offset p % B of its logical
 * block p / B, the sequence's block table maps that logical block to a
 * physical one, and the flat slot is physical * B + p % B -- the slot
 * numbering pa_reshape_and_cache takes.  For every token t:
 *     s = seq_ids[t], p = positions[t]
 *     slot_mapping[t] = block_tables[s][p / B] * B + p % B
 * or -1 (a token pa_reshape_and_cache skips) when s is outside
 * [0, num_seqs), p < 0, p / B >= max_blocks_per_seq, or the table entry is
 * outside [0, num_blocks).
 *
 *  block_tables   device int32 [num_seqs][max_blocks_per_seq].
 *  seq_ids        device int32 [num_tokens]: the token's sequence.
 *  positions      device int32 [num_tokens]: its position, from 0 (e.g. the
 *                 newest token of a decode step is at context_len - 1).
 *  slot_mapping   device int64 [num_tokens], written.
 *  num_tokens     >= 0 (0 is a no-op).
 * Errors: PA_ERR_INVALID_ARG for a null pointer with num_tokens > 0 or a
 * non-positive size.  Runs on the device, so it may be enqueued under
 * stream capture between the steps that produce the tables and the cache
 * write that consumes the slots.
 */
pa_status pa_slot_mapping(const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                          const int32_t *seq_ids, const int32_t *positions, int64_t num_tokens,
                          int32_t block_size, int64_t num_blocks, int64_t *slot_mapping, void *stream);

/*
 * pa_reshape_and_cache -- write new K/V rows into their cache slots.
 *
 * The fused reshape-and-block-write kernel (review section 5.1, item 1; notes
 * section 4.1): for every token t with slot = slot_mapping[t] >= 0 and every
 * head h, the head_dim elements key[t][h][:] are copied bit for bit into
 * k_cache[slot / B][h][slot % B][:], and value[t][h][:] into v_cache
 * likewise.  Nothing else is written.  A negative slot means "no write" (a
 * padding token).
 *
 *  key, value         device [num_tokens][num_heads][head_dim]; consecutive
 *                     tokens are key_token_stride / value_token_stride
 *                     ELEMENTS apart (>= num_heads*head_dim, and a multiple of
 *                     16 bytes), heads are contiguous within a token, so a
 *                     slice of a fused QKV tensor can be passed directly.
 *  k_cache, v_cache   device caches, num_blocks blocks.
 *  slot_mapping       device int64 [num_tokens].
 *  num_tokens         >= 0 (0 is a no-op).
 */
pa_status pa_reshape_and_cache(const void *key, const void *value, int64_t key_token_stride,
                               int64_t value_token_stride, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int64_t num_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               pa_dtype dtype, void *stream);

/*
 * Decode attention runs as a partition pass and a reduce pass.  Attention
 * over a context splits by block (review section 4.1): any run of
 * consecutive positions can be attended on its own, giving a running max m,
 * a running sum l and an unnormalised weighted value sum, and such pieces
 * merge exactly by rescaling to a common max.  The partition pass cuts the
 * whole batch -- every (sequence, head, 16-token tile) -- into equal
 * contiguous ranges, one per worker wave, so that every wave reads the same
 * number of K/V bytes whatever the mix of context lengths.  A (sequence,
 * head) pair that lies inside one range is finished by its wave; a pair cut
 * by range boundaries leaves partial results that the reduce pass merges.
 *
 * split_workers: 0 lets the library use as many worker waves as the device
 * holds at once (pa_decode_default_workers); a positive value uses at most
 * that many.  The result does not depend on it beyond floating-point
 * rounding; tests use it to move the cut points.
 */
int32_t pa_decode_default_workers(pa_dtype dtype, int32_t head_dim, int32_t block_size);

/* Workspace bytes pa_paged_attention_decode needs for up to split_workers
 * worker waves (0: an upper bound for the current device); 0 only for
 * num_seqs 0.  Layout: the work plan (uint32: 4 header words plus three per
 * worker, padded to 256 bytes), then two fp32 partial results of head_dim + 2
 * floats per worker.  Its contents need no initialisation; calls that share
 * one workspace must be ordered on one stream. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t block_size,
                                 int32_t split_workers);

/*
 * pa_paged_attention_decode -- one query per sequence over its paged KV.
 *
 * For each sequence s (n = context_lens[s], which counts the current token,
 * written beforehand by pa_reshape_and_cache: "KV 캐시 관리와 PagedAttention",
 * section on attention over scattered KV) and head h:
 *     out[s][h][:] = sum_p softmax_p(scale * q[s][h][:] . k_p) * v_p
 * over positions p = 0..n-1, k_p / v_p read from the physical block
 * block_tables[s][p / B] at offset p % B.  n = 0 gives a zero output.
 * Arithmetic: inputs in `dtype`, products, sums and softmax in fp32, the
 * output rounded to `dtype` (nearest even).
 *
 *  out              device [num_seqs][num_heads][head_dim], `dtype`.
 *  q                device [num_seqs][num_heads][head_dim], `dtype`.
 *  max_context_len  host upper bound of context_lens (sizes the grid).
 *  scale            softmax scale, normally 1/sqrt(head_dim).
 *  workspace        device, >= pa_decode_workspace_bytes(...) bytes, 16-byte
 *                   aligned; may be NULL only when num_seqs is 0.
 */
pa_status pa_paged_attention_decode(void *out, const void *q, const void *k_cache,
                                    const void *v_cache, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                    int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                    float scale, pa_dtype dtype, int32_t split_workers,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_paged_attention_decode_ex -- pa_paged_attention_decode with flags that
 * choose how the kernels read the cache; the output bytes do not depend on
 * them.
 *
 * PA_DECODE_REUSED_BLOCKS: the batch's sequences point at some of the same
 * physical blocks (samples forked from one prompt, beams of one search:
 * paper notes "PagedAttention: Efficient Memory Management for Large
 * Language Model Serving", sections 3.4.1 Parallel sampling and 3.4.2 Beam
 * search), so a block is read once per sequence that holds it.  K/V are
 * then read with ordinary loads, which leave them in the caches for the next
 * reader; without the flag they are read with non-temporal loads, the faster
 * choice when every block is read once.  When the sharing is a common prompt
 * prefix of known groups, pa_paged_attention_decode_shared reads each shared
 * block only once.
 *
 *  flags  0 or PA_DECODE_REUSED_BLOCKS; any other bit gives
 *         PA_ERR_INVALID_ARG.  All other arguments, the workspace and the
 *         result are as for pa_paged_attention_decode.
 */
#define PA_DECODE_REUSED_BLOCKS 1u
pa_status pa_paged_attention_decode_ex(void *out, const void *q, const void *k_cache,
                                       const void *v_cache, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                                       int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       float scale, pa_dtype dtype, int32_t split_workers,
                                       uint32_t flags, void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * pa_paged_attention_decode_noalloc -- pa_paged_attention_decode without a
 * caller workspace, for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, same kernels and the same output bytes as
 * pa_paged_attention_decode with the same split_workers; the plan and the
 * partial results live instead in a fixed array of PA_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every device it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks the array's address up.
 *
 * The array needs no initialisation and keeps the last call's contents.
 * Every call on one device shares it: calls that may overlap on a device
 * (two streams, two threads) race and give wrong results -- order them on
 * one stream.  A decode whose workspace (pa_decode_workspace_bytes with the
 * same arguments) exceeds PA_NOALLOC_SCRATCH_BYTES is refused with
 * PA_ERR_WORKSPACE before anything is enqueued; head_dim <= 128 at up to 32
 * worker waves per compute unit on 256 compute units fits.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status pa_paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache,
                                            const void *v_cache, const int32_t *block_tables,
                                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                                            int32_t max_context_len, int32_t num_seqs,
                                            int32_t num_heads, int32_t head_dim, int32_t block_size,
                                            int64_t num_blocks, float scale, pa_dtype dtype,
                                            int32_t split_workers, void *stream);

/*
 * pa_paged_attention_decode_append -- the decode step's cache write and its
 * attention in two launches instead of three.  A decode step first stores
 * the new token's K and V in its slot, then attends over a context that
 * includes it ("KV 캐시 관리와 PagedAttention", section on attention over
 * scattered KV).  The pages fuse the write's steps into one kernel to save
 * launches (review section 5.1, item 1; notes section 4.1); this call goes
 * one launch further: the partition pass reads the newest token from
 * key/value instead of the cache, and the reduce pass, which runs after
 * every read of the partition pass, stores it into the cache.
 *
 * For each sequence s with n = context_lens[s] >= 1 (clipped to
 * max_context_len as in pa_paged_attention_decode), key[s] and value[s]
 * ([num_heads][head_dim] each) are the K and V of position n - 1.  The call
 * leaves the caches and `out` byte for byte as
 *     pa_reshape_and_cache(key, value, ..., slot_mapping) with
 *         slot_mapping[s] = block_tables[s][(n-1)/B] * B + (n-1) % B,
 *     then pa_paged_attention_decode(...)
 * would.  A sequence with n = 0 writes nothing; a table entry for position
 * n - 1 outside [0, num_blocks) is neither read nor written (as both calls
 * skip it).
 *
 *  key, value        device, sequence s's rows at key + s*key_seq_stride
 *                    (elements; >= num_heads*head_dim, whole 16-byte units),
 *                    heads contiguous; a fused QKV tensor's slices work.
 *  k_cache, v_cache  written at each sequence's slot of position n - 1.
 *  others            as for pa_paged_attention_decode (same workspace size).
 *
 * Beyond pa_paged_attention_decode's preconditions: the block holding
 * position n - 1 of a sequence is not read by another sequence of the batch
 * (true of any copy-on-write table: a block written to has one owner), and
 * key/value do not overlap the caches.  Under PA_DEBUG_VALIDATE the table
 * and length checks of pa_paged_attention_decode apply, and the written
 * slots must be distinct and lie in blocks no other sequence of the batch
 * reads (a shared block the caller forgot to copy is refused).
 */
pa_status pa_paged_attention_decode_append(void *out, const void *q, const void *key,
                                           const void *value, int64_t key_seq_stride,
                                           int64_t value_seq_stride, void *k_cache, void *v_cache,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, int32_t max_context_len,
                                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                           int32_t block_size, int64_t num_blocks, float scale,
                                           pa_dtype dtype, int32_t split_workers, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* The two passes of pa_paged_attention_decode_append, separately (same
 * arguments each).  The partition pass reads the newest tokens from
 * key/value and writes nothing to the caches;
 * pa_paged_attention_decode_append_reduce then merges the cut pairs into
 * `out` and stores the newest tokens into the caches.  Together they leave
 * the same bytes as pa_paged_attention_decode_append; between the two calls
 * the caches do not yet hold the new tokens. */
pa_status pa_paged_attention_decode_append_partitions(
    void *out, const void *q, const void *key, const void *value, int64_t key_seq_stride,
    int64_t value_seq_stride, void *k_cache, void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    float scale, pa_dtype dtype, int32_t split_workers, void *workspace, size_t workspace_bytes,
    void *stream);
pa_status pa_paged_attention_decode_append_reduce(
    void *out, const void *q, const void *key, const void *value, int64_t key_seq_stride,
    int64_t value_seq_stride, void *k_cache, void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    float scale, pa_dtype dtype, int32_t split_workers, void *workspace, size_t workspace_bytes,
    void *stream);

/* The partition pass alone (same arguments).  Writes `out` for every pair
 * that one worker wave finished and the workspace (plan and partial
 * results) for the others. */
pa_status pa_paged_attention_decode_partitions(
    void *out, const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    float scale, pa_dtype dtype, int32_t split_workers, void *workspace, size_t workspace_bytes,
    void *stream);

/* The reduce pass alone: merges the partial results of the pairs the
 * partition pass left cut into `out`.  Arguments as for
 * pa_paged_attention_decode; it must see the same split_workers and the
 * workspace the partition pass wrote. */
pa_status pa_paged_attention_decode_reduce(void *out, const int32_t *context_lens,
                                           int32_t max_context_len, int32_t max_blocks_per_seq,
                                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                           int32_t block_size, pa_dtype dtype,
                                           int32_t split_workers, const void *workspace,
                                           size_t workspace_bytes, void *stream);

/*
 * pa_paged_attention_decode_shared -- decode for groups of sequences that
 * share a prompt (parallel sampling), reading the shared blocks once per
 * group instead of once per sequence.  Same result as
 * pa_paged_attention_decode, up to floating-point summation order.
 *
 * Samples forked from one prompt point their block tables at the same
 * physical blocks for it (paper notes "PagedAttention: Efficient Memory
 * Management for Large Language Model Serving", section 3.4.1 Parallel
 * sampling; "KV 캐시 관리와 PagedAttention", section on sharing the common KV
 * of several responses).  Attention splits by position range (review
 * section 4.1), so the call computes, per (sequence, head): the shared
 * prefix [0, P) for all members of a group at once, each member's own
 * positions [P, n) with the stream-K pass, and their merge.  The first two
 * share one launch whose worker waves split both the prefix tiles and the
 * own tiles evenly; the own positions' cut pairs and the merge are two more
 * launches.
 *
 *  group_members  device int32 [num_groups][PA_MAX_GROUP_MEMBERS]: the
 *                 members of each group, a leading run of sequence ids,
 *                 padded with -1.  A sequence is in at most one group.
 *  group_prefix   device int32 [num_groups]: P, the tokens whose blocks all
 *                 members share (same physical block ids at the same table
 *                 entries), a multiple of 16 and of block_size, at most
 *                 every member's context length.  pa_shared_prefix_groups
 *                 derives these three arrays from the tables.
 *  seq_starts     device int32 [num_seqs]: P of the sequence's group, 0 for
 *                 a sequence in no group (decoded as usual).
 *  max_prefix_len host upper bound of group_prefix.
 *  workspace      >= pa_decode_shared_workspace_bytes(...) bytes, 16-byte
 *                 aligned; needs no initialisation.
 *  phases         which of the three steps this call enqueues: PA_SHARED_OWN
 *                 (each sequence's own positions: the stream-K pass and its
 *                 fix-up), PA_SHARED_PREFIX (the groups' shared prefixes),
 *                 PA_SHARED_COMBINE (the merge into out); PA_SHARED_ALL runs
 *                 them on `stream`, OWN and PREFIX in one launch.  OWN and
 *                 PREFIX read disjoint data and write disjoint parts of the
 *                 workspace, so a caller may also enqueue them as separate
 *                 calls on two streams; COMBINE must follow both (e.g. after
 *                 an event join).  Every call of one decode passes the same
 *                 arguments, split_workers and workspace; the results are
 *                 then the same bits however the steps are enqueued.
 * Other arguments as for pa_paged_attention_decode.  block_size 16, 32 or
 * 64 (PA_ERR_UNSUPPORTED otherwise).  The group description is checked
 * against the tables only under PA_DEBUG_VALIDATE=1 (that needs device
 * data); an inconsistent one gives wrong results, never an access outside
 * the given arrays.
 */
#define PA_MAX_GROUP_MEMBERS 8

/*
 * pa_shared_prefix_groups -- the sharing description that
 * pa_paged_attention_decode_shared takes, derived from the block tables.
 * Host only: all arrays are host memory, no GPU call.
 *
 * The caller names which sequences were forked from one prompt (paper notes,
 * section 3.4.1 Parallel sampling: the samples point at the prompt's
 * physical blocks).  For each such group the call finds P, the tokens of
 * the leading table entries that every member holds identically (the same
 * physical block at the same logical index) and has filled (every position
 * of the block is below every member's context length), rounded down to a
 * multiple of 16 (the decode's tile).  A group of more than
 * PA_MAX_GROUP_MEMBERS sequences is split, in order, into groups of at most
 * that many with the same P.
 *
 *  block_tables   [num_seqs][max_blocks_per_seq] int32; context_lens
 *                 [num_seqs] int32 (negative lengths count as 0).
 *  group_offsets  [num_groups + 1] int32, non-decreasing from 0: group g's
 *                 members are group_seqs[group_offsets[g] ..
 *                 group_offsets[g + 1]); an empty group is skipped.
 *  group_seqs     int32 sequence ids in [0, num_seqs), each in at most one
 *                 group.
 *  max_out_groups capacity of the outputs below; num_groups +
 *                 group_offsets[num_groups] / PA_MAX_GROUP_MEMBERS always
 *                 suffices.
 *  group_members  written: [*num_out_groups][PA_MAX_GROUP_MEMBERS], each row
 *                 a leading run of sequence ids padded with -1.
 *  group_prefix   written: [*num_out_groups], P of each output group.
 *  seq_starts     written: [num_seqs], P of the sequence's group, 0 for a
 *                 sequence in no group.
 *  num_out_groups, max_prefix_len  written: the output group count and the
 *                 largest P (0 without groups).
 * Errors (nothing written): PA_ERR_INVALID_ARG for a null pointer, bad
 * offsets, a sequence id out of range or in two groups, or too small a
 * max_out_groups (the message gives the count needed).
 */
pa_status pa_shared_prefix_groups(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  const int32_t *group_offsets, int32_t num_groups,
                                  const int32_t *group_seqs, int32_t block_size,
                                  int32_t max_out_groups, int32_t *group_members,
                                  int32_t *group_prefix, int32_t *seq_starts,
                                  int32_t *num_out_groups, int32_t *max_prefix_len);

#define PA_SHARED_OWN 1
#define PA_SHARED_PREFIX 2
#define PA_SHARED_COMBINE 4
#define PA_SHARED_ALL 7
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t block_size,
                                        int32_t num_groups, int32_t max_prefix_len,
                                        int32_t split_workers);
pa_status pa_paged_attention_decode_shared(
    void *out, const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    float scale, pa_dtype dtype, const int32_t *group_members, const int32_t *group_prefix,
    const int32_t *seq_starts, int32_t num_groups, int32_t max_prefix_len, int32_t split_workers,
    int32_t phases, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_copy_blocks -- batched whole-block copy for copy-on-write.
 *
 * The fused block-copy kernel (review section 5.1, item 3; notes section
 * 4.1): one launch copies, for every layer l < num_layers and every pair
 * (src, dst) = (block_mapping[2i], block_mapping[2i+1]), the block_bytes
 * bytes of physical block src onto block dst, in k_caches[l] and in
 * v_caches[l] -- every head and every slot, filled or not ("KV 캐시 관리와
 * PagedAttention", copy-on-write section: the copy keeps the K/V already in
 * the block).
 *
 *  k_caches, v_caches  HOST arrays of num_layers DEVICE pointers; each cache
 *                      holds num_blocks blocks of block_bytes bytes.  The
 *                      host arrays are read during the call only.
 *  block_mapping       DEVICE int64 [num_pairs][2].
 *  block_bytes         num_heads*block_size*head_dim*element size; a
 *                      positive multiple of 16.
 *  num_pairs           >= 0 (0 is a no-op); num_layers >= 1.
 */
pa_status pa_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                         const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                         int64_t num_blocks, void *stream);

/*
 * pa_paged_attention_prefill_chunk -- causal attention of a chunk of queries
 * over a paged cache (chunked prefill; teardown of vLLM's scheduler on
 * arcyou.ai, continuous-batching section, where long prompts are split into
 * chunks).  The chunk's own K/V must already be in the cache
 * (pa_reshape_and_cache).
 *
 * Sequence s owns query rows cu_q_lens[s] .. cu_q_lens[s+1]-1 (q_len rows);
 * context_lens[s] counts its cached tokens plus the chunk, so the chunk
 * starts at c = context_lens[s] - q_len and query j attends, with the same
 * softmax as decode, to positions 0 .. c+j.
 *
 * fp16 and bf16 at head_dim 128 run on the matrix cores (MFMA); fp32, and
 * head_dim 64, run on the vector ALU (8 queries per wave, each K/V tile read
 * once for them).  The matrix kernel forms the weighted sum of V in fp16
 * (for a bf16 cache it converts the V rows to fp16 on chip); a group of 16
 * queries whose sums come out non-finite (a V value beyond fp16's range, or
 * an inf/NaN in a row it must not see) is recomputed in fp32, so the result
 * is within the attention tolerance for any finite input.
 *
 *  out, q          device [total_q][num_heads][head_dim], `dtype`.
 *  cu_q_lens       device int32 [num_seqs + 1], non-decreasing, from 0 to
 *                  total_q.
 *  max_q_len       host bound of the per-sequence q_len.
 *  max_context_len host bound of context_lens.
 *  scale           multiplies q.k before the softmax; positive and finite
 *                  (PA_ERR_INVALID_ARG otherwise).
 */
pa_status pa_paged_attention_prefill_chunk(void *out, const void *q, const int32_t *cu_q_lens,
                                           const void *k_cache, const void *v_cache,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t total_q, int32_t max_q_len,
                                           int32_t max_context_len, int32_t num_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, float scale, pa_dtype dtype,
                                           void *stream);

/*
 * pa_paged_attention_prefill_chunk_append -- the chunk's cache write and its
 * attention in one launch.  The pages store a chunk's new K/V with the fused
 * reshape-and-write kernel before attending to them (review section 5.1,
 * item 1; notes section 4.1).  This call instead reads the chunk's keys from
 * key/value and writes them into the cache from the same kernel.
 *
 * Token t = cu_q_lens[s] + j of sequence s (position c + j, c as above) has
 * its K and V rows at key + t*key_token_stride and value +
 * t*value_token_stride ([num_heads][head_dim] each; strides in elements,
 * >= num_heads*head_dim and whole 16-byte units, so slices of a fused QKV
 * tensor work).  The call leaves the caches and `out` byte for byte as
 *     pa_reshape_and_cache(key, value, ..., slot_mapping) with
 *         slot_mapping[t] = block_tables[s][(c+j)/B] * B + (c+j) % B,
 *     then pa_paged_attention_prefill_chunk(...)
 * would.  Tokens whose table entry lies outside [0, num_blocks) are not
 * written (the two calls skip them too).
 *
 * fp16 and bf16 at head_dim 128 only (the matrix-core kernel);
 * PA_ERR_UNSUPPORTED otherwise.  Beyond pa_paged_attention_prefill_chunk's
 * preconditions: the blocks the chunk writes are not read by another
 * sequence of the batch, and key/value do not overlap the caches.  Under
 * PA_DEBUG_VALIDATE the checks of pa_paged_attention_prefill_chunk apply,
 * and the written slots must be distinct and lie in blocks no other
 * sequence of the batch reads.
 */
pa_status pa_paged_attention_prefill_chunk_append(void *out, const void *q, const void *key,
                                                  const void *value, int64_t key_token_stride,
                                                  int64_t value_token_stride,
                                                  const int32_t *cu_q_lens, void *k_cache,
                                                  void *v_cache, const int32_t *block_tables,
                                                  int32_t max_blocks_per_seq,
                                                  const int32_t *context_lens, int32_t num_seqs,
                                                  int32_t total_q, int32_t max_q_len,
                                                  int32_t max_context_len, int32_t num_heads,
                                                  int32_t head_dim, int32_t block_size,
                                                  int64_t num_blocks, float scale, pa_dtype dtype,
                                                  void *stream);

/*
 * pa_swap_blocks -- batched whole-block copy between two pools, for swapping
 * blocks out to host memory and back in (paper notes "PagedAttention:
 * Efficient Memory Management for Large Language Model Serving", sections
 * 3.5 Scheduling and Preemption and 4.1 Kernel-level Optimization: blocks
 * of preempted requests move to CPU memory and are copied in many small
 * pieces, which one launch replaces).  For every cache c < num_caches and
 * every pair (src, dst) = (block_mapping[2i], block_mapping[2i+1]) it copies
 * block src of src_caches[c] (a pool of src_num_blocks blocks) onto block dst
 * of dst_caches[c] (dst_num_blocks blocks): block_bytes bytes, every head
 * and slot.
 *
 *  src_caches, dst_caches  HOST arrays of num_caches pointers, e.g. the K
 *                      and V caches of every layer; each is device memory
 *                      or pinned host memory (hipHostMalloc, torch's
 *                      pin_memory), checked with hipPointerGetAttributes --
 *                      pageable memory is refused (PA_ERR_INVALID_ARG).
 *  block_mapping       int64 [num_pairs][2], device or pinned host memory.
 *                      Destinations must be distinct within a call; pairs
 *                      with an index outside its pool are skipped.
 *  block_bytes         a positive multiple of 16.
 * Enqueued on `stream`; the caller keeps both pools alive until it ends.
 */
pa_status pa_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                         const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                         int64_t src_num_blocks, int64_t dst_num_blocks, void *stream);

/*
 * pa_stream_read -- measurement helper, not a step of the attention path.
 *
 * Reads `bytes` bytes of device memory once, with 16-byte non-temporal
 * loads, in `workgroups` workgroups of 256 lanes that sweep the buffer
 * together in grid-stride order; the kernel does nothing else.  Its rate is the plain streaming
 * read bandwidth of the device the cache kernels run on, the same-device
 * reference beside the vendor's HBM figure for memory-bound kernels
 * (decode reads every valid K/V row once: "Efficient Memory Management for
 * Large Language Model Serving with PagedAttention", evaluation section).
 *
 *  src         device buffer, 16-byte aligned; bytes a positive multiple of
 *              16.  Read only.
 *  sink        device uint32 [4 * workgroups]; receives one XOR of the data
 *              per wave (so the loads cannot be elided).  Caller-owned.
 *  workgroups  1 .. 2^31-1.
 *
 * Errors: PA_ERR_INVALID_ARG for a null or misaligned pointer or a bad size;
 * PA_ERR_HIP if the launch fails.
 */
pa_status pa_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                         void *stream);

/* ------------------------------------------------------------------------
 * Block manager (host only; no device memory, no GPU calls).
 *
 * The bookkeeping that feeds the kernels above: a pool of num_blocks
 * physical blocks of block_size tokens, one block table per sequence, one
 * reference count per block.  It follows the paper notes' KV cache manager
 * and its three operations ("PagedAttention: Efficient Memory Management for
 * Large Language Model Serving", sections 3.2, 3.4.1, 3.4.2 and 4.2: fork,
 * append, free) and the copy-on-write and block-return walk-throughs of
 * "KV 캐시 관리와 PagedAttention" (sections on splitting a shared block that
 * must be written and on returning blocks after a request ends):
 *  - blocks come from a first-in first-out queue of free blocks (the vLLM
 *    teardown on arcyou.ai, section on paging the KV cache) whose initial
 *    order is free_order (NULL: 0, 1, 2, ...); freed blocks join its back;
 *  - a sequence takes a new block only when its last block is full;
 *  - fork shares every block of the parent (each gains one reference);
 *  - appending to a sequence whose partly filled last block is shared moves
 *    the sequence onto a fresh block and reports (src, dst): the caller must
 *    copy the block on the device (pa_copy_blocks) before writing the token
 *    (pa_reshape_and_cache at the returned slot);
 *  - free drops one reference per block; blocks reaching zero are queued.
 * Slots are block * block_size + offset, positions count from 0.  A manager
 * is not thread-safe; every call on it must come from one thread at a time.
 * Errors change nothing: PA_ERR_INVALID_ARG (null pointer, dead or repeated
 * sequence id, a table row that would overflow), PA_ERR_NO_BLOCKS.
 * ------------------------------------------------------------------------ */
typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks blocks (< 2^31); free_order, if not NULL, is a
 * host array listing every block id once.  *out is NULL on error. */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t *free_order, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);

/* Free blocks (-1 for a NULL manager) and a block's reference count (-1 if
 * out of range). */
int64_t pa_bm_num_free(const pa_block_manager *bm);
int32_t pa_bm_refcount(const pa_block_manager *bm, int64_t block);

/* A new sequence holding num_tokens tokens (a prompt): ceil(num_tokens /
 * block_size) blocks at once.  Ids count up from 0 and are never reused. */
pa_status pa_bm_add_sequence(pa_block_manager *bm, int32_t num_tokens, int32_t *seq_id);

/* A new sequence sharing every block (and the length) of `parent`. */
pa_status pa_bm_fork(pa_block_manager *bm, int32_t parent, int32_t *child);

/* One more token for each of the num_seqs distinct sequences seqs[i],
 * handled in order: slots[i] receives the slot of sequence i's new token,
 * copies[2k], copies[2k+1] the k-th (src, dst) block copy the writes need
 * first (at most num_seqs), *num_copies their number.  All host arrays.
 * Either every sequence gets its token or (PA_ERR_NO_BLOCKS when the pool
 * is short) nothing changes. */
pa_status pa_bm_append_slots(pa_block_manager *bm, const int32_t *seqs, int32_t num_seqs,
                             int64_t *slots, int64_t *copies, int32_t *num_copies);

/* End a sequence; blocks no longer referenced return to the free queue. */
pa_status pa_bm_free_sequence(pa_block_manager *bm, int32_t seq);

/* Length (tokens) and blocks of a live sequence. */
pa_status pa_bm_sequence(const pa_block_manager *bm, int32_t seq, int32_t *length,
                         int32_t *num_blocks);

/* The decode inputs of a batch: tables (host int32 [num_seqs][
 * max_blocks_per_seq], rows padded with -1) and context_lens (host int32
 * [num_seqs]). */
pa_status pa_bm_block_tables(const pa_block_manager *bm, const int32_t *seqs, int32_t num_seqs,
                             int32_t *tables, int32_t *context_lens);

/* Slots (host int64 [count]) of positions first .. first+count-1 of a live
 * sequence, e.g. its prompt for pa_reshape_and_cache. */
pa_status pa_bm_slots(const pa_block_manager *bm, int32_t seq, int32_t first, int32_t count,
                      int64_t *slots);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
