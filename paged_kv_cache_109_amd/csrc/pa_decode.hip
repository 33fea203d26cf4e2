// Paged decode attention for gfx950: plan, stream-K partition pass, fix-up.
//
// What is computed (paper notes "PagedAttention: Efficient Memory Management
// for Large Language Model Serving with PagedAttention", unpurerationalist
// .github.io, section 3.1 and its block-wise attention equation): for one
// query q of a sequence, the softmax over every valid key of every block of
// scale*q.k, then the weight-sum of the values.  The Korean review
// (mz-moonzoo.tistory.com/116, section 4.1) points out that the sum splits
// by block: each block's contribution can be formed on its own and the
// pieces added at the end.  Here a piece is any run of consecutive 16-token
// tiles of one (sequence, head) pair, carrying (running max m, running sum
// l, unnormalised value sum); pieces are merged by rescaling to a common max.
//
// Work decomposition (stream-K).  Decode is bound by HBM reads, and context
// lengths vary, so the batch is treated as one stream of tiles: every
// (sequence s, head h, tile t) in the order s, h, t gets a global index g in
// [0, T_total).  The G resident waves (as many as fit on the chip) each take
// an equal contiguous range [floor(w*T/G), floor((w+1)*T/G)) and walk it
// without pause across pair boundaries.  A pair that lies inside one range
// is finished by that wave, which writes the output; a pair cut by range
// boundaries leaves one fragment per wave involved (at most two per wave),
// and a small fix-up kernel merges them.  A one-workgroup plan kernel
// prefix-sums the tile counts, writes every wave's start (s, h, t) and
// zeroes the outputs of empty sequences; for batches of up to 1024
// sequences the worker waves do that themselves (each reads all lengths),
// which saves a launch.
//
// Mapping to CDNA4.  A wave is an independent worker (no LDS, no barriers).
// The K (or V) row of one token and head is D*elt bytes contiguous inside its
// block (256 B for fp16/bf16 D=128), so a token row is covered by LPT =
// row/16 lanes doing one 16-byte load each, and one global_load_dwordx4 of
// the wave covers 64/LPT consecutive tokens: fully coalesced 1 KB reads
// chased through the block table (entries fetched with scalar loads), issued
// non-temporal since every byte is read once.  PA_DECODE_DEPTH tiles are in
// flight per wave; the issue cursor runs that far ahead of the consume
// cursor, across pair boundaries.  q.k is 4 packed dot2 instructions per lane
// (fp16/bf16) followed by a DPP all-reduce over the LPT lanes of the token;
// each lane group keeps its own online-softmax state and fp32 value
// accumulator, merged with lane swaps when a pair ends.

#include <algorithm>
#include <mutex>

#include "pa_stream.h"

namespace pa {

constexpr int kPlanThreads = 1024;

// ----------------------------------------------------------------------- plan

// Plan for batches of more than kSelfPlanSeqs sequences (smaller batches are
// planned by the worker waves themselves, see self_plan).  One workgroup.
// plan[0] = total tiles T, plan[1] = G = min(launched workers, T), and for
// every worker w < G the (s | h << 16, t) of its first tile and the tiles of
// that pair at plan[kPlanHeader + kPlanWords*w]; zeroes the outputs of empty
// sequences.
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
  __shared__ uint32_t scan[kPlanThreads];
  const int tid = threadIdx.x;
  const int S = a.num_seqs;
  const uint32_t H = (uint32_t)a.num_heads;
  const int per = (S + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  uint32_t mine = 0;
  for (int s = lo; s < hi; ++s) mine += (uint32_t)pass_tiles(a, s, clip_ctx(a.context_lens[s], a.ctx_cap)) * H;
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    const uint32_t v = tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const uint32_t total = scan[kPlanThreads - 1];
  // Never more workers than tiles, so that every worker's range is non-empty.
  const uint32_t G = total < (uint32_t)a.workers ? total : (uint32_t)a.workers;
  uint32_t c = scan[tid] - mine;  // tiles before sequence lo
  if (tid == 0) {
    a.plan[0] = total;
    a.plan[1] = G;
  }
  for (int s = lo; s < hi; ++s) {
    const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
    const uint32_t ts = (uint32_t)pass_tiles(a, s, n);
    const uint32_t c_next = c + ts * H;
    if (ts > 0) {
      // Workers whose first tile falls in [c, c_next): w in [ceil(c*G/T), ceil(c_next*G/T)).
      const uint64_t w_lo = ((uint64_t)c * G + total - 1) / total;
      const uint64_t w_hi = ((uint64_t)c_next * G + total - 1) / total;
      for (uint64_t w = w_lo; w < w_hi; ++w) {
        const uint32_t local = range_begin((uint32_t)w, total, G) - c;
        a.plan[kPlanHeader + kPlanWords * w] = (uint32_t)s | ((local / ts) << 16);
        a.plan[kPlanHeader + kPlanWords * w + 1] = local % ts;
        a.plan[kPlanHeader + kPlanWords * w + 2] = ts;
      }
    } else {
      empty_rows(a, s, 0, 1);
    }
    c = c_next;
  }
}


// Fragments a merge reads in one batch (a pair usually spans a few
// workers); longer runs take the loop below.
constexpr uint32_t kMergeBatch = 8;

// Merge the fragments workers wa..wb left for pair (s, h) and write its
// output row: wa's is in its back slot (1), every later worker's in its front
// slot (0).  One wave; lanes stride over the head dimension.  The sums run
// over the fragments in order either way, so both paths give the same bits.
template <Dt T, int D>
__device__ __forceinline__ void merge_fragments(const DecodeArgs &a, uint32_t wa, uint32_t wb, int s, int h) {
  const int lane = threadIdx.x % kWave;
  auto frag = [&](uint32_t v) -> const float * {
    return a.frags + ((int64_t)v * 2 + (v == wa ? 1 : 0)) * (D + 2);
  };
  constexpr int kPer = (D + kWave - 1) / kWave;  // head dimensions per lane
  const uint32_t cnt = wb - wa + 1;
  float M = -INFINITY, L = 0.f, A[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) A[j] = 0.f;
  if (cnt <= kMergeBatch) {
    // Every load first, so they are in flight together: lane v reads
    // fragment wa+v's max and sum, and every lane its dimensions of each
    // fragment (indices past wb repeat wb's and are not summed).
    const float *fl = frag(wa + min((uint32_t)lane, cnt - 1));
    const float mv = fl[D], lv = fl[D + 1];
    float x[kMergeBatch][kPer];
#pragma unroll
    for (uint32_t v = 0; v < kMergeBatch; ++v) {
      const float *f = frag(wa + min(v, cnt - 1));
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[v][j] = (lane + kWave * j < D) ? f[lane + kWave * j] : 0.f;
    }
#pragma unroll
    for (uint32_t v = 0; v < kMergeBatch; ++v)
      if (v < cnt) M = fmaxf(M, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), v)));
    const float mu = (M == -INFINITY) ? 0.f : M;
#pragma unroll
    for (uint32_t v = 0; v < kMergeBatch; ++v) {
      if (v < cnt) {
        const float e = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), v)) - mu);
        L += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), v)) * e;
#pragma unroll
        for (int j = 0; j < kPer; ++j) A[j] += x[v][j] * e;
      }
    }
    M = mu;
  } else {
    for (uint32_t v = wa; v <= wb; ++v) M = fmaxf(M, frag(v)[D]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    for (uint32_t v = wa; v <= wb; ++v) L += frag(v)[D + 1] * fast_exp2(frag(v)[D] - mu);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int d = lane + kWave * j;
      if (d < D)
        for (uint32_t v = wa; v <= wb; ++v) A[j] += frag(v)[d] * fast_exp2(frag(v)[D] - mu);
    }
    M = mu;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float *part = nullptr;
  if (a.starts && to_partial(a, start_of(a.starts[s], clip_ctx(a.context_lens[s], a.ctx_cap))))
    part = a.suffix_out + (int64_t)s * a.suffix_row + (int64_t)h * (D + 2);
  const int64_t out_row = ((int64_t)s * a.num_heads + h) * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = lane + kWave * j;
    if (d < D) {
      if (part) part[d] = A[j] * inv;
      else store_out_elem<T, D>(a.out, out_row + d, A[j] * inv);
    }
  }
  if (part && lane == 0) {
    part[D] = L > 0.f ? M + __builtin_amdgcn_logf(L) : -INFINITY;
    part[D + 1] = 0.f;
  }
}

// The partition pass: every wave of the grid is one stream-K worker.
template <Dt T, int D, int B, bool kAppend, bool kStream = kStreamLoads>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_partition_kernel(DecodeArgs a) {
  partition_worker<T, D, B, kAppend, kDepth, kStream>(a, blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform());
}

// Merge the fragments of every pair cut by range boundaries.  Worker wave w
// handles the pair holding its first tile when that pair started before its
// range and ends inside it (so every fragment of the pair exists).
//
// Append (a.new_key set): first, every lane of the grid stores 16-byte
// chunks of the newest tokens' K and V rows (position n - 1 of each
// sequence, read by the partition pass from the new rows) into their cache
// slots.  The partition pass has ended, so no read of the caches races with
// these stores.  A sequence with n = 0, or whose table entry for position
// n - 1 lies outside the pool, stores nothing.
// Workgroups of the reduce pass that merge cut pairs (none when no pair was
// cut); any further ones store the new tokens of an append step.
__host__ __device__ inline uint32_t reduce_merge_groups(const DecodeArgs &a) {
  return a.workers > 1 ? (uint32_t)((a.workers + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup) : 0u;
}

template <Dt T, int D>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_reduce_kernel(DecodeArgs a) {
  // The first reduce_merge_groups(a) workgroups merge cut pairs; the rest
  // (append only) store the new tokens, so that the two chains of
  // dependent loads run side by side.
  const uint32_t merge_groups = reduce_merge_groups(a);
  if (blockIdx.x >= merge_groups) {
    using R = RowShape<T, D, kDecodeTile>;
    const int64_t row_chunks = (int64_t)a.num_heads * R::kLPT;  // chunks of one token's K (or V) rows
    const int64_t total = (int64_t)a.num_seqs * 2 * row_chunks;
    const int64_t block_stride = (int64_t)a.num_heads * a.block_size * R::kRowBytes;
    const int64_t step = (int64_t)(gridDim.x - merge_groups) * blockDim.x;
    for (int64_t c = (int64_t)(blockIdx.x - merge_groups) * blockDim.x + threadIdx.x; c < total; c += step) {
      const int s = (int)(c / (2 * row_chunks));
      const int64_t r = c - (int64_t)s * 2 * row_chunks;
      const bool is_v = r >= row_chunks;
      const int64_t rc = is_v ? r - row_chunks : r;
      const int h = (int)(rc / R::kLPT), col = (int)(rc % R::kLPT);
      const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
      if (n < 1) continue;
      const int p = n - 1;
      const int32_t e = a.block_tables[(int64_t)s * a.max_blocks + p / a.block_size];
      if (e < 0 || (int64_t)e >= a.num_blocks) continue;
      const char *src = reinterpret_cast<const char *>(is_v ? a.new_value : a.new_key) +
                        (int64_t)s * (is_v ? a.new_value_stride : a.new_key_stride) + h * R::kRowBytes + col * 16;
      char *dst = reinterpret_cast<char *>(const_cast<void *>(is_v ? a.v_cache : a.k_cache)) +
                  (int64_t)e * block_stride + ((int64_t)h * a.block_size + p % a.block_size) * R::kRowBytes + col * 16;
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }
    return;
  }
  // Every worker wave v that the loop below visits has a non-empty range
  // (the plan never uses more workers than tiles) and wrote its fragment.
  // This wave's plan words are read together with G, at an index clamped to
  // the plan (the grid may hold a few waves more than workers).
  const uint32_t w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  const uint32_t wc = w < (uint32_t)a.workers ? w : (uint32_t)a.workers - 1u;
  const uint32_t G = load_uniform(a.plan, 1), total = load_uniform(a.plan, 0);
  const uint32_t sh = load_uniform(a.plan, kPlanHeader + kPlanWords * wc);
  const uint32_t t = load_uniform(a.plan, kPlanHeader + kPlanWords * wc + 1);
  const uint32_t nt = load_uniform(a.plan, kPlanHeader + kPlanWords * wc + 2);
  if (w >= G) return;
  const uint32_t g0 = range_begin(w, total, G), g1 = range_begin(w + 1, total, G);
  const int s = (int)(sh & 0xffffu), h = (int)(sh >> 16);
  if (t == 0) return;  // the pair starts at g0: not cut at the front of this range
  const uint32_t pair_start = g0 - t;
  if (pair_start + nt > g1) return;  // continues past this range: a later worker merges it
  merge_fragments<T, D>(a, first_worker(pair_start, total, G), w, s, h);
}

// ------------------------------------------------------------------ dispatch

// Both variants launch this many workers per CU (the plain kernel's
// occupancy), so the workspace layout and the reduce pass do not depend on
// the variant; where the append variant holds fewer waves at once, the
// extra workers simply start later.
template <Dt T, int D, int B>
static int waves_per_cu() {
  static const int v = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_partition_kernel<T, D, B, false>,
                                                     kDecodeWavesPerGroup * kWave, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb * kDecodeWavesPerGroup;
  }();
  return v;
}

hipError_t launch_decode_plan(const DecodeArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

template <Dt T, int D, int B>
static hipError_t launch_part(const DecodeArgs &a, hipStream_t st) {
  if (a.num_seqs > kSelfPlanSeqs) {
    const hipError_t e = launch_decode_plan(a, st);
    if (e != hipSuccess) return e;
  }
  const unsigned groups = (unsigned)((a.workers + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup);
  if (a.new_key)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, B, true>), dim3(groups), dim3(kDecodeWavesPerGroup * kWave), 0,
                       st, a);
  else if (a.reused_blocks)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, B, false, false>), dim3(groups),
                       dim3(kDecodeWavesPerGroup * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((decode_partition_kernel<T, D, B, false>), dim3(groups), dim3(kDecodeWavesPerGroup * kWave), 0,
                       st, a);
  return hipGetLastError();
}

#define PA_DISPATCH_B(B, FN, ...)                  \
  switch (B) {                                     \
    case 4: return FN<T, D, 4>(__VA_ARGS__);       \
    case 8: return FN<T, D, 8>(__VA_ARGS__);       \
    case 16: return FN<T, D, 16>(__VA_ARGS__);     \
    case 32: return FN<T, D, 32>(__VA_ARGS__);     \
    case 64: return FN<T, D, 64>(__VA_ARGS__);     \
  }

template <Dt T, int D>
static hipError_t launch_part_b(const DecodeArgs &a, int B, hipStream_t st) {
  PA_DISPATCH_B(B, launch_part, a, st)
  return hipErrorInvalidValue;
}

template <Dt T, int D>
static int waves_b(int B) {
  PA_DISPATCH_B(B, waves_per_cu)
  return 0;
}

template <Dt T>
static hipError_t launch_part_d(const DecodeArgs &a, int D, int B, hipStream_t st) {
  switch (D) {
    case 64: return launch_part_b<T, 64>(a, B, st);
    case 128: return launch_part_b<T, 128>(a, B, st);
  }
  return hipErrorInvalidValue;
}

template <Dt T>
static int waves_d(int D, int B) {
  switch (D) {
    case 64: return waves_b<T, 64>(B);
    case 128: return waves_b<T, 128>(B);
  }
  return 0;
}

bool decode_supported(int dtype, int head_dim, int block_size) {
  const bool dt = dtype >= 0 && dtype <= 2;
  const bool d = head_dim == 64 || head_dim == 128;
  const bool b = block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
  return dt && d && b;
}

int decode_waves_per_cu(int dtype, int head_dim, int block_size) {
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return waves_d<Dt::F32>(head_dim, block_size);
    case Dt::F16: return waves_d<Dt::F16>(head_dim, block_size);
    case Dt::BF16: return waves_d<Dt::BF16>(head_dim, block_size);
  }
  return 0;
}

hipError_t launch_decode_partitions(const DecodeArgs &a, int dtype, int head_dim, int block_size,
                                    hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_part_d<Dt::F32>(a, head_dim, block_size, stream);
    case Dt::F16: return launch_part_d<Dt::F16>(a, head_dim, block_size, stream);
    case Dt::BF16: return launch_part_d<Dt::BF16>(a, head_dim, block_size, stream);
  }
  return hipErrorInvalidValue;
}

// Store workgroups: one 16-byte chunk per thread, at most kReduceStoreGroups
// of them (grid-stride beyond).
constexpr int64_t kReduceStoreGroups = 4096;

template <Dt T>
static hipError_t launch_red(const DecodeArgs &a, int D, hipStream_t st) {
  int64_t store_groups = 0;
  if (a.new_key) {
    const int64_t chunks = (int64_t)a.num_seqs * 2 * a.num_heads * (D * (int64_t)EltBytes<T>::value / 16);
    const int64_t threads = kDecodeWavesPerGroup * kWave;
    store_groups = std::min<int64_t>((chunks + threads - 1) / threads, kReduceStoreGroups);
  }
  const dim3 grid((unsigned)(reduce_merge_groups(a) + store_groups));
  if (grid.x == 0) return hipSuccess;
  switch (D) {
    case 64:
      hipLaunchKernelGGL((decode_reduce_kernel<T, 64>), grid, dim3(kDecodeWavesPerGroup * kWave), 0, st, a);
      break;
    case 128:
      hipLaunchKernelGGL((decode_reduce_kernel<T, 128>), grid, dim3(kDecodeWavesPerGroup * kWave), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream) {
  if (a.num_seqs == 0 || (a.workers <= 1 && !a.new_key)) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_red<Dt::F32>(a, head_dim, stream);
    case Dt::F16: return launch_red<Dt::F16>(a, head_dim, stream);
    case Dt::BF16: return launch_red<Dt::BF16>(a, head_dim, stream);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------- workspace of the no-alloc call

// The plan and partial results of pa_paged_attention_decode_noalloc, for
// callers that cannot allocate.  Each device holds its own copy of this
// array from the library's load until the process ends.  In host code the
// name is only a stand-in for it, never a device address: the address is
// asked of the runtime once per device, with that device current, and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace pa
