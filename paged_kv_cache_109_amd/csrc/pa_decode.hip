// Paged decode attention for gfx950: a split-KV partition pass and a reduce
// pass.
//
// What is computed (paper notes "PagedAttention: Efficient Memory Management
// for Large Language Model Serving with PagedAttention", unpurerationalist
// .github.io, section 3.1 and its block-wise attention equation): for one
// query q of a sequence, the softmax over every valid key of every block of
// scale*q.k, then the weight-sum of the values.  The Korean review
// (mz-moonzoo.tistory.com/116, section 4.1) points out that the sum splits
// by block: each block's contribution can be formed on its own and the
// pieces added at the end.  Here the pieces are partitions of up to
// part_tokens positions, each carrying (running max m, running sum l,
// unnormalised value sum), merged by rescaling to a common max.
//
// Mapping to CDNA4.  One workgroup = 4 wave64s = one (sequence, head,
// partition).  The K (or V) row of one token and head is D*elt bytes
// contiguous inside its block (256 B for fp16/bf16 D=128), so a token row is
// covered by LPT = row/16 lanes doing one 16-byte load each, and one
// global_load_dwordx4 of the wave covers 64/LPT consecutive tokens: fully
// coalesced 1 KB reads chased through the block table.  A wave processes 16
// tokens per step (a tile); the four waves take the partition's tiles
// round-robin.  q.k is 4 packed dot2 instructions per lane (fp16/bf16)
// followed by a DPP all-reduce over the LPT lanes of the token; each lane
// group keeps its own online-softmax state and value accumulator (fp32), so
// the inner loop has no cross-row traffic.  Groups, then waves (through
// LDS), are merged once at the end.  The table entries a partition needs are
// fetched once per wave, one per lane, and broadcast with readlane.
// The next tile's K and V are loaded before the current tile is consumed.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kDecodeWaves = 4;

template <Dt T, int D>
struct RowShape {
  static constexpr int kEB = EltBytes<T>::value;
  static constexpr int kRowBytes = D * kEB;      // one token row of one head
  static constexpr int kLPT = kRowBytes / 16;    // lanes per token row
  static constexpr int kGroups = kWave / kLPT;   // tokens per wave load
  static constexpr int kNI = kDecodeTile / kGroups;  // loads per tile
  static constexpr int kFE = Frag<T>::kElems;    // elements per lane fragment
  static_assert(kRowBytes % 16 == 0 && kLPT >= 1 && kLPT <= kWave, "row must be whole fragments");
  static_assert(kDecodeTile % kGroups == 0, "tile must be whole wave loads");
  static_assert(kLPT * kFE == D, "fragments must tile the head");
};

__device__ __forceinline__ int clip_ctx(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

template <Dt T, int D>
__device__ __forceinline__ void store_out_elem(void *out, int64_t idx, float x) {
  if constexpr (T == Dt::F32) {
    reinterpret_cast<float *>(out)[idx] = x;
  } else if constexpr (T == Dt::F16) {
    reinterpret_cast<uint16_t *>(out)[idx] = (uint16_t)f32_to_f16_bits(x);
  } else {
    reinterpret_cast<uint16_t *>(out)[idx] = (uint16_t)f32_to_bf16_bits(x);
  }
}

template <Dt T, int D, int B>
__global__ __launch_bounds__(kDecodeWaves *kWave) void decode_partition_kernel(DecodeArgs a) {
  using R = RowShape<T, D>;
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id_uniform();

  const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
  const int nparts = (n + a.part_tokens - 1) / a.part_tokens;
  const int64_t out_row = ((int64_t)s * a.num_heads + h) * D;
  if (n == 0) {
    if (part == 0 && threadIdx.x < D) store_out_elem<T, D>(a.out, out_row + threadIdx.x, 0.f);
    return;
  }
  if (part >= nparts) return;

  const int p_begin = part * a.part_tokens;
  const int p_end = min(n, p_begin + a.part_tokens);
  const int tile_begin = p_begin / kDecodeTile;
  const int tile_end = (p_end + kDecodeTile - 1) / kDecodeTile;
  const int blk_begin = p_begin / B;
  const int nblk = (p_end + B - 1) / B - blk_begin;  // <= kMaxPartitionBlocks

  const int grp = lane / R::kLPT;  // token slot within one wave load
  const int col = lane % R::kLPT;  // 16-byte column within the token row

  // One table entry per lane; broadcast later.
  const int32_t *table = a.block_tables + (int64_t)s * a.max_blocks;
  const int32_t my_entry = (lane < nblk) ? table[blk_begin + lane] : -1;

  const char *q_ptr = reinterpret_cast<const char *>(a.q) + out_row * R::kEB + col * 16;
  const uint4 qf = *reinterpret_cast<const uint4 *>(q_ptr);

  const char *kbase = reinterpret_cast<const char *>(a.k_cache);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache);
  const int64_t block_stride = (int64_t)a.num_heads * B * R::kRowBytes;
  const int64_t lane_off = (int64_t)h * B * R::kRowBytes + col * 16;

  // Loads of one tile.  ok[i]: the token of load i exists (position inside
  // the partition, table entry inside the pool); masked fragments are zero.
  auto load_tile = [&](int tile, uint4 *kf, uint4 *vf, bool *ok) {
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const int pos = tile * kDecodeTile + i * R::kGroups + grp;
      int32_t phys;
      if constexpr (B >= kDecodeTile) {
        const int bi = tile * kDecodeTile / B - blk_begin;  // uniform
        phys = __builtin_amdgcn_readlane(my_entry, bi);
      } else {
        phys = __shfl(my_entry, pos / B - blk_begin, kWave);
      }
      ok[i] = (pos < p_end) && (phys >= 0) && ((int64_t)phys < a.num_blocks);
      const int64_t off = (int64_t)phys * block_stride + lane_off + (int64_t)(pos % B) * R::kRowBytes;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (ok[i]) {
        kv = *reinterpret_cast<const uint4 *>(kbase + off);
        vv = *reinterpret_cast<const uint4 *>(vbase + off);
      }
      kf[i] = kv;
      vf[i] = vv;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  float acc[R::kFE];
#pragma unroll
  for (int e = 0; e < R::kFE; ++e) acc[e] = 0.f;

  uint4 kc[R::kNI], vc[R::kNI], kn[R::kNI], vn[R::kNI];
  bool okc[R::kNI], okn[R::kNI];
  int tile = tile_begin + wave;
  if (tile < tile_end) load_tile(tile, kc, vc, okc);
  while (tile < tile_end) {
    const int next = tile + kDecodeWaves;
    if (next < tile_end) load_tile(next, kn, vn, okn);

    float sc[R::kNI];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      float d = group_sum<R::kLPT>(frag_dot<T>(qf, kc[i]));
      sc[i] = okc[i] ? d * a.scale_log2 : -INFINITY;
      mt = fmaxf(mt, sc[i]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < R::kFE; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const float p = fast_exp2(sc[i] - m_use);
      l_run += p;
      frag_axpy<T>(acc, p, vc[i]);
    }
    m_run = m_new;

#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      kc[i] = kn[i];
      vc[i] = vn[i];
      okc[i] = okn[i];
    }
    tile = next;
  }

  // Merge the lane groups of the wave (each saw its own tokens).
#pragma unroll
  for (int x = R::kLPT; x < kWave; x *= 2) {
    const float mo = __shfl_xor(m_run, x, kWave);
    const float lo = __shfl_xor(l_run, x, kWave);
    const float mn = fmaxf(m_run, mo);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float fa = fast_exp2(m_run - mu), fb = fast_exp2(mo - mu);
    l_run = l_run * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < R::kFE; ++e) acc[e] = acc[e] * fa + __shfl_xor(acc[e], x, kWave) * fb;
    m_run = mn;
  }

  // Merge the waves through LDS.
  __shared__ float sh_m[kDecodeWaves], sh_l[kDecodeWaves];
  __shared__ float sh_acc[kDecodeWaves][D];
  if (lane < R::kLPT) {
#pragma unroll
    for (int e = 0; e < R::kFE; ++e) sh_acc[wave][col * R::kFE + e] = acc[e];
  }
  if (lane == 0) {
    sh_m[wave] = m_run;
    sh_l[wave] = l_run;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float M = sh_m[0];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sh_m[w]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = fast_exp2(sh_m[w] - mu);
      L += sh_l[w] * f;
      A += sh_acc[w][d] * f;
    }
    if (nparts == 1) {
      store_out_elem<T, D>(a.out, out_row + d, L > 0.f ? A / L : 0.f);
    } else {
      const int64_t slot = ((int64_t)s * a.num_heads + h) * a.max_parts + part;
      a.ws_acc[slot * D + d] = A;
      if (d == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = L;
      }
    }
  }
}

// Merge the partials of sequences with two or more partitions.
template <Dt T, int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
  const int nparts = (n + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)s * a.num_heads + h) * a.max_parts;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += kWave) M = fmaxf(M, a.ws_ml[2 * (base + p)]);
#pragma unroll
  for (int x = 1; x < kWave; x *= 2) M = fmaxf(M, __shfl_xor(M, x, kWave));
  const float mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  for (int p = lane; p < nparts; p += kWave) L += a.ws_ml[2 * (base + p) + 1] * fast_exp2(a.ws_ml[2 * (base + p)] - mu);
#pragma unroll
  for (int x = 1; x < kWave; x *= 2) L += __shfl_xor(L, x, kWave);
  const float inv = L > 0.f ? 1.f / L : 0.f;

  const int64_t out_row = ((int64_t)s * a.num_heads + h) * D;
#pragma unroll
  for (int d = lane; d < D; d += kWave) {
    float A = 0.f;
    for (int p = 0; p < nparts; ++p) A += a.ws_acc[(base + p) * D + d] * fast_exp2(a.ws_ml[2 * (base + p)] - mu);
    store_out_elem<T, D>(a.out, out_row + d, A * inv);
  }
}

// ------------------------------------------------------------------ dispatch

template <Dt T, int D, int B>
static hipError_t launch_part(const DecodeArgs &a, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, B>), grid, dim3(kDecodeWaves * kWave), 0, st, a);
  return hipGetLastError();
}

template <Dt T, int D>
static hipError_t launch_part_b(const DecodeArgs &a, int B, hipStream_t st) {
  switch (B) {
    case 4: return launch_part<T, D, 4>(a, st);
    case 8: return launch_part<T, D, 8>(a, st);
    case 16: return launch_part<T, D, 16>(a, st);
    case 32: return launch_part<T, D, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

template <Dt T>
static hipError_t launch_part_d(const DecodeArgs &a, int D, int B, hipStream_t st) {
  switch (D) {
    case 64: return launch_part_b<T, 64>(a, B, st);
    case 128: return launch_part_b<T, 128>(a, B, st);
  }
  return hipErrorInvalidValue;
}

bool decode_supported(int dtype, int head_dim, int block_size) {
  const bool dt = dtype >= 0 && dtype <= 2;
  const bool d = head_dim == 64 || head_dim == 128;
  const bool b = block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32;
  return dt && d && b;
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

template <Dt T>
static hipError_t launch_red(const DecodeArgs &a, int D, hipStream_t st) {
  dim3 grid(a.num_heads, a.num_seqs);
  switch (D) {
    case 64: hipLaunchKernelGGL((decode_reduce_kernel<T, 64>), grid, dim3(kWave), 0, st, a); break;
    case 128: hipLaunchKernelGGL((decode_reduce_kernel<T, 128>), grid, dim3(kWave), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_parts <= 1) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_red<Dt::F32>(a, head_dim, stream);
    case Dt::F16: return launch_red<Dt::F16>(a, head_dim, stream);
    case Dt::BF16: return launch_red<Dt::BF16>(a, head_dim, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
