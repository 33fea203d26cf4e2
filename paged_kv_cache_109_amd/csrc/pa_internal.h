// Host-side interface between the C-ABI layer (pa_api.cpp) and the kernel
// launchers (pa_decode.hip, pa_cache.hip, pa_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Dt : int;

// Arguments of the decode partition pass.  Pointers are device pointers.
struct DecodeArgs {
  void *out;            // [S][H][D] dtype
  float *ws_ml;         // [S][H][max_parts][2]   (m in log2 units, l)
  float *ws_acc;        // [S][H][max_parts][D]
  const void *q;        // [S][H][D]
  const void *k_cache;  // [N][H][B][D]
  const void *v_cache;
  const int32_t *block_tables;  // [S][max_blocks]
  const int32_t *context_lens;  // [S]
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_heads;
  int32_t ctx_cap;      // context lengths are clipped to [0, ctx_cap]
  int32_t part_tokens;  // tokens per partition
  int32_t max_parts;    // ceil(ctx_cap / part_tokens)
  float scale_log2;     // softmax scale * log2(e)
};

// Tokens a decode wave processes per step; partitions are whole tiles.
constexpr int kDecodeTile = 16;
// Most table entries one partition may span (one per lane of a wave).
constexpr int kMaxPartitionBlocks = 64;

bool decode_supported(int dtype, int head_dim, int block_size);
hipError_t launch_decode_partitions(const DecodeArgs &a, int dtype, int head_dim, int block_size,
                                    hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream);

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
};

bool prefill_supported(int dtype, int head_dim, int block_size);
hipError_t launch_prefill_chunk(const PrefillArgs &a, int dtype, int head_dim, int block_size,
                                hipStream_t stream);

}  // namespace pa
