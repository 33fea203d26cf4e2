// Slot translation, cache write through a slot mapping, and batched
// whole-block copy.
//
// The write and the copies are pure byte moves (no arithmetic, no
// conversion), so they are bit-exact for every dtype.  They are the fused
// single-launch kernels the
// Korean review of the vLLM paper (mz-moonzoo.tistory.com/116, section 5.1,
// items 1 and 3) describes: the write replaces a split/reshape/scatter
// sequence, and the copy replaces one small memcpy per block.
//
// gfx950 mapping: every lane moves 16 bytes per instruction
// (global_load_dwordx4 / global_store_dwordx4); consecutive lanes touch
// consecutive 16-byte chunks of a row or block, so every wave access is a
// contiguous 1 KB run (or a whole 256 B token row per 16 lanes).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kCacheThreads = 256;

// Grid (token, part): workgroup (t, y) copies 16-byte chunks y*256 ..
// y*256+255 of token t's K rows then V rows (num_heads rows of row_bytes
// each, a multiple of 16) into (slot / B, h, slot % B).  Each lane moves at
// most one chunk, so a token's copy is one load and one store deep however
// many heads it has, and a batch of a few tokens still spreads over many
// workgroups; the slot is read once per workgroup, as a scalar load.
__global__ __launch_bounds__(kCacheThreads) void reshape_and_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, int64_t key_stride_bytes,
    int64_t value_stride_bytes, char *__restrict__ k_cache, char *__restrict__ v_cache,
    const int64_t *__restrict__ slot_mapping, int32_t num_heads, int32_t row_bytes, int32_t block_size,
    int64_t num_slots) {
  const int64_t t = blockIdx.x;
  const int64_t slot = load_uniform(slot_mapping, t);
  if (slot < 0 || slot >= num_slots) return;
  const int chunks_per_row = row_bytes >> 4;
  const int per_tensor = num_heads * chunks_per_row;
  const int idx = blockIdx.y * kCacheThreads + threadIdx.x;
  if (idx >= 2 * per_tensor) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot % block_size;
  const bool is_v = idx >= per_tensor;
  const int r = is_v ? idx - per_tensor : idx;
  const int h = r / chunks_per_row;
  const int c = r - h * chunks_per_row;
  const char *src = (is_v ? value + t * value_stride_bytes : key + t * key_stride_bytes) + (int64_t)h * row_bytes +
                    c * 16;
  char *dst = (is_v ? v_cache : k_cache) + ((blk * num_heads + h) * block_size + off) * row_bytes + c * 16;
  *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}

hipError_t launch_reshape_and_cache(const void *key, const void *value, int64_t key_stride_bytes,
                                    int64_t value_stride_bytes, void *k_cache, void *v_cache,
                                    const int64_t *slot_mapping, int64_t num_tokens, int32_t num_heads,
                                    int32_t row_bytes, int32_t block_size, int64_t num_blocks,
                                    hipStream_t stream) {
  // Chunks of one token's K and V rows, in workgroups of kCacheThreads lanes
  // (the host bounds 2 * num_heads * row_bytes / 16 below 2^31).
  const int64_t chunks = 2 * (int64_t)num_heads * (row_bytes / 16);
  const int64_t parts = (chunks + kCacheThreads - 1) / kCacheThreads;
  if (parts > 65535) return hipErrorInvalidValue;
  // grid.x is at most 2^31-1; split very long mappings into several launches.
  const int64_t kMaxGrid = 0x7fffffff;
  for (int64_t first = 0; first < num_tokens; first += kMaxGrid) {
    const int64_t count = num_tokens - first < kMaxGrid ? num_tokens - first : kMaxGrid;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)count, (unsigned)parts), dim3(kCacheThreads), 0,
                       stream, reinterpret_cast<const char *>(key) + first * key_stride_bytes,
                       reinterpret_cast<const char *>(value) + first * value_stride_bytes, key_stride_bytes,
                       value_stride_bytes, reinterpret_cast<char *>(k_cache), reinterpret_cast<char *>(v_cache),
                       slot_mapping + first, num_heads, row_bytes, block_size, num_blocks * block_size);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------------- slot mapping
//
// Address translation of the tokens a step writes ("KV 캐시 관리와
// PagedAttention", section on linking token order to storage): position p
// of a sequence lies at offset p % B of its logical block p / B, which the
// sequence's block table maps to a physical block; the flat slot is
// physical * B + offset.  One lane per token; -1 marks a token that names no
// valid slot (sequence or position out of range, table entry outside the
// pool), which the cache write then skips.

constexpr int kSlotMapGroups = 4096;

__global__ __launch_bounds__(kCacheThreads) void slot_mapping_kernel(
    const int32_t *__restrict__ block_tables, int32_t max_blocks, int32_t num_seqs,
    const int32_t *__restrict__ seq_ids, const int32_t *__restrict__ positions, int64_t num_tokens,
    int32_t block_size, int64_t num_blocks, int64_t *__restrict__ slot_mapping) {
  for (int64_t t = (int64_t)blockIdx.x * kCacheThreads + threadIdx.x; t < num_tokens;
       t += (int64_t)gridDim.x * kCacheThreads) {
    const int32_t s = seq_ids[t], p = positions[t];
    int64_t slot = -1;
    if (s >= 0 && s < num_seqs && p >= 0) {
      const int32_t logical = p / block_size;
      if (logical < max_blocks) {
        const int32_t phys = block_tables[(int64_t)s * max_blocks + logical];
        if (phys >= 0 && phys < num_blocks) slot = (int64_t)phys * block_size + p % block_size;
      }
    }
    slot_mapping[t] = slot;
  }
}

hipError_t launch_slot_mapping(const int32_t *block_tables, int32_t max_blocks, int32_t num_seqs,
                               const int32_t *seq_ids, const int32_t *positions, int64_t num_tokens,
                               int32_t block_size, int64_t num_blocks, int64_t *slot_mapping, hipStream_t stream) {
  const int64_t need = (num_tokens + kCacheThreads - 1) / kCacheThreads;
  const unsigned groups = (unsigned)(need < kSlotMapGroups ? need : kSlotMapGroups);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(groups), dim3(kCacheThreads), 0, stream, block_tables, max_blocks,
                     num_seqs, seq_ids, positions, num_tokens, block_size, num_blocks, slot_mapping);
  return hipGetLastError();
}

// ---------------------------------------------------------------- copy_blocks

struct LayerPtrs {
  char *k[kCopyMaxLayers];
  char *v[kCopyMaxLayers];
};

// 16-byte chunks per lane: a copy-on-write copy within the pool, and a swap
// between two pools (whose other side is reached over the host link, so it
// keeps more requests in flight per lane).
constexpr int kCopyUnroll = 2;
constexpr int kSwapUnroll = 4;
template <int kUnroll>
constexpr int64_t chunk_bytes() { return (int64_t)kCacheThreads * 16 * kUnroll; }  // bytes per workgroup

// One workgroup's part of a whole-block copy: chunk `chunk` (kUnroll * 4 KB)
// of the block_bytes at `from` onto `to`.  Each lane has all its loads in
// flight before its first store.  kStreamStores: the stores are
// non-temporal, so the copied blocks do not push out of the caches the
// blocks that are read again next -- the source block, which the copies of
// several forks read in turn, and the shared prompt blocks the decode that
// follows reads once per sample.
template <int kUnroll, bool kStreamStores>
__device__ __forceinline__ void copy_block_chunk(const char *from, char *to, int64_t block_bytes, int64_t chunk) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t begin = chunk * chunk_bytes<kUnroll>();
  u32x4 r[kUnroll];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t o = begin + ((int64_t)u * kCacheThreads + threadIdx.x) * 16;
    live[u] = o < block_bytes;
    if (live[u]) r[u] = *reinterpret_cast<const u32x4 *>(from + o);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t o = begin + ((int64_t)u * kCacheThreads + threadIdx.x) * 16;
    if (!live[u]) continue;
    if constexpr (kStreamStores) __builtin_nontemporal_store(r[u], reinterpret_cast<u32x4 *>(to + o));
    else *reinterpret_cast<u32x4 *>(to + o) = r[u];
  }
}

// grid.x = pair * chunks_per_block + chunk, grid.y = 2 * layer + (K=0 / V=1).
__global__ __launch_bounds__(kCacheThreads) void copy_blocks_kernel(LayerPtrs ptrs,
                                                                    const int64_t *__restrict__ mapping,
                                                                    int64_t block_bytes, int64_t num_blocks,
                                                                    int32_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t chunk = blockIdx.x - pair * chunks_per_block;
  const int layer = blockIdx.y >> 1;
  char *base = (blockIdx.y & 1) ? ptrs.v[layer] : ptrs.k[layer];
  const int64_t src = mapping[2 * pair];
  const int64_t dst = mapping[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  copy_block_chunk<kCopyUnroll, true>(base + src * block_bytes, base + dst * block_bytes, block_bytes, chunk);
}

hipError_t launch_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                              const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream) {
  const int64_t chunks = (block_bytes + chunk_bytes<kCopyUnroll>() - 1) / chunk_bytes<kCopyUnroll>();
  const int64_t max_pairs = 0x7fffffff / chunks;
  for (int32_t l0 = 0; l0 < num_layers; l0 += kCopyMaxLayers) {
    const int32_t nl = num_layers - l0 < kCopyMaxLayers ? num_layers - l0 : kCopyMaxLayers;
    LayerPtrs p = {};
    for (int32_t i = 0; i < nl; ++i) {
      p.k[i] = reinterpret_cast<char *>(k_caches[l0 + i]);
      p.v[i] = reinterpret_cast<char *>(v_caches[l0 + i]);
    }
    for (int64_t first = 0; first < num_pairs; first += max_pairs) {
      const int64_t np = num_pairs - first < max_pairs ? num_pairs - first : max_pairs;
      dim3 grid((unsigned)(np * chunks), (unsigned)(2 * nl));
      hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCacheThreads), 0, stream, p, block_mapping + 2 * first,
                         block_bytes, num_blocks, (int32_t)chunks);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ------------------------------------------------------------- swap_blocks
//
// Whole-block copies from one pool to another (HBM to pinned host memory to
// swap blocks out, or back): every (src, dst) pair of the mapping, for every
// cache listed (e.g. the K and V caches of each layer), in one launch.  The
// host side is reached through the host link, so loads are issued four per
// lane at once to keep many requests in flight.

struct SwapPtrs {
  const char *src[kSwapMaxCaches];
  char *dst[kSwapMaxCaches];
};

// grid.x = pair * chunks_per_block + chunk, grid.y = cache.
__global__ __launch_bounds__(kCacheThreads) void swap_blocks_kernel(SwapPtrs ptrs, const int64_t *__restrict__ mapping,
                                                                    int64_t block_bytes, int64_t src_blocks,
                                                                    int64_t dst_blocks, int32_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t chunk = blockIdx.x - pair * chunks_per_block;
  const int64_t src = mapping[2 * pair];
  const int64_t dst = mapping[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  copy_block_chunk<kSwapUnroll, false>(ptrs.src[blockIdx.y] + src * block_bytes,
                                       ptrs.dst[blockIdx.y] + dst * block_bytes, block_bytes, chunk);
}

hipError_t launch_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                              const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                              int64_t src_blocks, int64_t dst_blocks, hipStream_t stream) {
  const int64_t chunks = (block_bytes + chunk_bytes<kSwapUnroll>() - 1) / chunk_bytes<kSwapUnroll>();
  const int64_t max_pairs = 0x7fffffff / chunks;
  for (int32_t c0 = 0; c0 < num_caches; c0 += kSwapMaxCaches) {
    const int32_t nc = num_caches - c0 < kSwapMaxCaches ? num_caches - c0 : kSwapMaxCaches;
    SwapPtrs p = {};
    for (int32_t i = 0; i < nc; ++i) {
      p.src[i] = reinterpret_cast<const char *>(src_caches[c0 + i]);
      p.dst[i] = reinterpret_cast<char *>(dst_caches[c0 + i]);
    }
    for (int64_t first = 0; first < num_pairs; first += max_pairs) {
      const int64_t np = num_pairs - first < max_pairs ? num_pairs - first : max_pairs;
      hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)(np * chunks), (unsigned)nc), dim3(kCacheThreads), 0,
                         stream, p, block_mapping + 2 * first, block_bytes, src_blocks, dst_blocks, (int32_t)chunks);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ---------------------------------------------------------- streaming read
//
// The bandwidth reference the cache kernels are compared with on the same
// device: a read of one contiguous buffer with 16-byte non-temporal loads and
// nothing else.  The workgroups sweep the buffer together in grid-stride
// order, each lane with four loads in flight.  Every lane XORs what it read
// and each wave stores the XOR of its lanes, so no load can be dropped.

constexpr int kStreamUnroll = 4;
static_assert(kStreamSinkWordsPerGroup == kCacheThreads / 64, "one sink word per wave");
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCacheThreads) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                                    uint32_t *__restrict__ sink) {
  constexpr int64_t kSpan = (int64_t)kCacheThreads * kStreamUnroll;
  const int64_t stride = (int64_t)gridDim.x * kSpan;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t base = (int64_t)blockIdx.x * kSpan + threadIdx.x;
  for (; base + (kStreamUnroll - 1) * kCacheThreads < n16; base += stride) {
    u32x4 r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) r[u] = __builtin_nontemporal_load(src + base + u * kCacheThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= r[u];
  }
  // The last, partial span of the sweep: at most kStreamUnroll - 1 loads.
  for (; base < n16; base += kCacheThreads) acc ^= __builtin_nontemporal_load(src + base);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * kStreamSinkWordsPerGroup + threadIdx.x / 64] = x;
}

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kCacheThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
