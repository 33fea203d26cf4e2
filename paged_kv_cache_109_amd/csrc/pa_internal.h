// Host-side interface between the C-ABI layer (pa_api.cpp) and the kernel
// launchers (pa_decode.hip, pa_cache.hip, pa_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedattn.h"

namespace pa {

enum class Dt : int;

// Set (or clear) the message pa_last_error returns; return `st` (PA_OK).
pa_status record_error(pa_status st, const char *msg);
pa_status record_ok();

// Arguments of the decode passes.  Pointers are device pointers.
struct DecodeArgs {
  void *out;            // [S][H][D] dtype
  uint32_t *plan;       // [kPlanHeader + kPlanWords*workers]: total tiles, workers used, per-worker start
  float *frags;         // [workers][2][D + 2]: fragment value sums, then m (log2 units), l
  const void *q;        // [S][H][D]
  const void *k_cache;  // [N][H][B][D]
  const void *v_cache;
  const int32_t *block_tables;  // [S][max_blocks]
  const int32_t *context_lens;  // [S]
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_heads;
  int32_t block_size;     // tokens per cache block
  int32_t ctx_cap;        // context lengths are clipped to [0, ctx_cap]
  int32_t workers;        // worker waves launched (the split of the tile stream)
  int32_t out_row_words;  // 32-bit words of one sequence's output rows (H*D*elt/4)
  float scale_log2;       // softmax scale * log2(e)
  int32_t reused_blocks;  // nonzero: the sequences share K/V blocks, read them with ordinary loads
  // Shared-prefix decode only (both null otherwise): starts[s] is the first
  // position the pass covers for sequence s (a multiple of kDecodeTile);
  // for s with starts[s] > 0 the pass leaves fp32 partials in suffix_out
  // ([S][H][D + 2]: the normalised output, then log2 of its softmax
  // denominator in the scale*log2(e) domain) instead of writing out.
  const int32_t *starts;
  float *suffix_out;
  int32_t suffix_row;  // floats of suffix_out per sequence: num_heads * (head_dim + 2)
  // Fused append only (both null otherwise): the K and V rows ([H][D]) of
  // each sequence's newest token, position n - 1, new_*_stride bytes apart.
  // The partition pass reads that position from them instead of the cache;
  // the reduce pass writes them into the cache (k_cache / v_cache are then
  // writable).
  const void *new_key;
  const void *new_value;
  int64_t new_key_stride;
  int64_t new_value_stride;
};

// 32-bit words before the per-worker starts in the plan, and words per
// worker: (s | h << 16, t) of its first tile and the tiles of that pair.
constexpr int kPlanHeader = 4;
constexpr int kPlanWords = 3;
// Tokens a decode wave processes per step (one tile).
constexpr int kDecodeTile = 16;
// Independent worker waves packed into one workgroup.
constexpr int kDecodeWavesPerGroup = 4;
// Upper bound of resident waves per CU used to size workspaces.
constexpr int kMaxWavesPerCu = 32;

// Resident worker waves per CU of the decode instantiation (0 if unsupported).
int decode_waves_per_cu(int dtype, int head_dim, int block_size);
bool decode_supported(int dtype, int head_dim, int block_size);
// Launches the fused-append instantiation when a.new_key is set.
hipError_t launch_decode_partitions(const DecodeArgs &a, int dtype, int head_dim, int block_size,
                                    hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream);
// The one-workgroup plan of the partition pass (batches above the size the
// workers plan for themselves).
hipError_t launch_decode_plan(const DecodeArgs &a, hipStream_t stream);

// The allocation-free decode's workspace: a fixed device array of
// PA_NOALLOC_SCRATCH_BYTES per device (pa_decode.hip).  Sets *ptr to the
// current device's copy, looked up once per device.
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_slot_mapping(const int32_t *block_tables, int32_t max_blocks, int32_t num_seqs,
                               const int32_t *seq_ids, const int32_t *positions, int64_t num_tokens,
                               int32_t block_size, int64_t num_blocks, int64_t *slot_mapping, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void *key, const void *value, int64_t key_stride_bytes,
                                    int64_t value_stride_bytes, void *k_cache, void *v_cache,
                                    const int64_t *slot_mapping, int64_t num_tokens, int32_t num_heads,
                                    int32_t row_bytes, int32_t block_size, int64_t num_blocks,
                                    hipStream_t stream);

// Most layers one copy launch covers (pointer pairs travel as kernel arguments).
constexpr int kCopyMaxLayers = 64;
hipError_t launch_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                              const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream);

// Most caches one swap launch covers (pointer pairs travel as kernel arguments).
constexpr int kSwapMaxCaches = 64;
hipError_t launch_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                              const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                              int64_t src_blocks, int64_t dst_blocks, hipStream_t stream);

// Sink words the streaming-read kernel stores per workgroup (one per wave).
constexpr int kStreamSinkWordsPerGroup = 4;
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                              hipStream_t stream);

struct PrefillArgs {
  void *out;                    // [total_q][H][D]
  const void *q;                // [total_q][H][D]
  const int32_t *cu_q_lens;     // [S+1]
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;  // [S][max_blocks]
  const int32_t *context_lens;  // [S]
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t max_blocks;
  int32_t num_heads;
  int32_t ctx_cap;
  float scale_log2;
  // Fused cache write only (both null otherwise): the chunk's K and V rows
  // ([total_q][H][D], new_*_stride bytes apart).  The kernel reads the
  // chunk's keys from them instead of the cache, and each workgroup writes
  // the rows of its own queries' tokens into the cache (k_cache / v_cache
  // are then writable).
  const void *new_key;
  const void *new_value;
  int64_t new_key_stride;
  int64_t new_value_stride;
};

// Shared-prefix decode (pa_shared.hip): members per group.
constexpr int kSharedMaxMembers = 8;
static_assert(kSharedMaxMembers == PA_MAX_GROUP_MEMBERS, "group width of the C ABI");
// Shortest range of prefix tiles a worker takes (bounds the pieces of a pair).
constexpr int kPrefixMinTiles = 8;
// 32-bit words before the per-group entries of the prefix plan.
constexpr int kPrefixPlanHeader = 4;

struct SharedArgs {
  void *out;                    // [S][H][D]
  const void *q;                // [S][H][D]
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;  // [S][max_blocks]
  const int32_t *context_lens;  // [S]
  const int32_t *starts;        // [S] first position of each sequence's own part (0: not in a group)
  const int32_t *members;       // [G][kSharedMaxMembers] sequence ids, -1 past the last member
  const int32_t *prefix;        // [G] shared prefix tokens
  float *partials;              // [G][chunks][H][kSharedMaxMembers][D + 2]: value sums, max, sum per piece
  uint32_t *pplan;              // [kPrefixPlanHeader + 2G]: prefix tiles, workers used; per group offset, tiles
  const float *suffix;          // [S][H][D + 2]: the decode pass's partials of the own parts
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t num_groups;
  int32_t chunks;               // piece slots per (group, head): the most pieces a prefix pair can be cut into
  int32_t max_prefix_tiles;     // prefixes are clamped to this many tiles
  int32_t ctx_cap;
  int32_t suffix_row;           // H * (D + 2)
  float scale_log2;
};

bool shared_supported(int dtype, int head_dim, int block_size);
// Resident waves per CU of the shared-prefix pass (its worker count per CU).
int shared_waves_per_cu(int dtype, int head_dim, int block_size);
// The own positions (own: partitions into d, with d.starts / d.suffix_out set)
// and the shared prefixes (prefix: pieces into s.partials) in one launch of
// d.workers worker waves; the reduce and the combine follow.
hipError_t launch_shared_pass(const DecodeArgs &d, const SharedArgs &s, int dtype, int head_dim, int block_size,
                              bool own, bool prefix, hipStream_t stream);
hipError_t launch_shared_combine(const SharedArgs &a, int dtype, int head_dim, hipStream_t stream);

bool prefill_supported(int dtype, int head_dim, int block_size);
// Shapes whose prefill runs on the matrix-core kernel (the only one with the
// fused chunk write).
bool prefill_append_supported(int dtype, int head_dim, int block_size);
// fp32 and head_dim 64 prefill (pa_prefill_general.hip).
bool prefill_general_supported(int dtype, int head_dim, int block_size);
hipError_t launch_prefill_general(const PrefillArgs &a, int dtype, int head_dim, int block_size, hipStream_t stream);

// Debug validation of the data-dependent preconditions (pa_validate.cpp):
// active when PA_DEBUG_VALIDATE=1; each synchronises `stream`, reads the
// index arrays to the host and returns PA_ERR_INVALID_ARG (with the
// last-error record set) at the first violation.  `append`: the call also
// writes each sequence's new tokens (fused decode append, fused chunk
// write), whose slots must be distinct and in blocks no other sequence
// reads.
bool debug_validate();
pa_status validate_slots(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                         hipStream_t stream);
pa_status validate_decode(const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t block_size, int64_t num_blocks,
                          bool append, hipStream_t stream);
pa_status validate_shared(const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t block_size, int64_t num_blocks,
                          const int32_t *group_members, const int32_t *group_prefix, const int32_t *seq_starts,
                          int32_t num_groups, int32_t max_prefix_len, hipStream_t stream);
pa_status validate_copy_pairs(const int64_t *block_mapping, int64_t num_pairs, int64_t num_blocks, hipStream_t stream);
pa_status validate_swap_pairs(const int64_t *block_mapping, int64_t num_pairs, int64_t src_num_blocks,
                              int64_t dst_num_blocks, hipStream_t stream);
pa_status validate_prefill(const int32_t *cu_q_lens, const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *context_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                           int32_t max_context_len, int32_t block_size, int64_t num_blocks, bool append,
                           hipStream_t stream);
hipError_t launch_prefill_chunk(const PrefillArgs &a, int dtype, int head_dim, int block_size,
                                hipStream_t stream);

}  // namespace pa
