// Chunked-prefill attention over a paged KV cache, on MFMA (gfx950).
//
// What is computed: a sequence's chunk of q_len new queries follows c cached
// tokens; query j sits at position c + j and attends, causally, to positions
// 0 .. c + j of the sequence -- the same softmax attention as decode, with
// the K/V read through the block table (paper notes "PagedAttention:
// Efficient Memory Management for Large Language Model Serving with
// PagedAttention", unpurerationalist.github.io, section 3.1; chunking long
// prompts across steps: the arcyou.ai teardown of vLLM, continuous-batching
// section).  Unlike decode, this IS a dense contraction (128 queries share
// every K/V row), so it runs on the matrix cores.
//
// Mapping to CDNA4.  A workgroup of 8 waves takes up to 256 queries of one
// (sequence, head) -- a whole chunk, so each K/V byte crosses HBM once --
// and each wave owns 32 of them.  K/V stream through LDS in blocks of 32
// keys gathered through the block table (entries read with scalar loads):
// global loads run two blocks ahead into registers and land in a
// triple-buffered LDS ring.  Per block a wave computes S^T = K Q^T with 8
// v_mfma_f32_32x32x16 (bf16 or f16 in, fp32 out) and O^T += V^T P^T with 8
// more (16 for bf16, whose P is split into a high and a low bf16 term to keep
// the weights' precision).  Working transposed keeps one query per lane
// column, so the softmax max/sum need one lane swap and the per-query
// rescale of O stays in-lane.  The K rows are fed to the MFMA in a
// bit-permuted order (bits 2 and 3 of the key index swapped) so that the
// accumulator registers of S^T land exactly where the B operand of the P V
// product wants 8 consecutive keys per lane: P never leaves registers.  V is
// written to LDS transposed (V^T[d][key]) so its operand reads are 16
// contiguous bytes.  A wave skips the key blocks past its causal limit.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPfD = 128;            // head_dim
constexpr int kPfWaves = 8;          // waves per workgroup
constexpr int kPfQ = 32 * kPfWaves;  // queries per workgroup
constexpr int kPfKeys = 32;          // keys per LDS block
constexpr int kKRow = kPfD * 2 + 16;      // bytes per K row in LDS (padded)
constexpr int kVRow = kPfKeys * 2 + 16;   // bytes per V^T row in LDS (padded)
constexpr int kKBuf = kPfKeys * kKRow;    // 8704 B
constexpr int kVBuf = kPfD * kVRow;       // 10240 B
constexpr int kRing = 3;                  // LDS buffers (loads run two blocks ahead)
constexpr int kTableCache = 4096;         // table entries kept in LDS (16 KB)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <Dt T>
__device__ __forceinline__ f32x16 mfma(const uint4 &a, const uint4 &b, const f32x16 &c) {
  if constexpr (T == Dt::BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
  }
}

template <Dt T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return pack_pair<T == Dt::BF16>(lo, hi);
}

// Row of the K block fed to MFMA row r: bits 2 and 3 of r swapped.
__device__ __forceinline__ int k_row_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

}  // namespace

template <Dt T, int B>
__global__ __launch_bounds__(kPfWaves *kWave) void prefill_chunk_kernel(PrefillArgs a, int qtiles) {
  __shared__ __attribute__((aligned(16))) char lds_k[kRing][kKBuf];
  __shared__ __attribute__((aligned(16))) char lds_v[kRing][kVBuf];
  __shared__ int32_t lds_table[kTableCache];
  static_assert(kPfWaves * kWave == 512, "staging maps 512 threads onto a 32-key block");

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = wave_id_uniform();
  const int half = lane / 32;  // which 8 of a 16-wide k step this lane holds
  const int col = lane % 32;   // MFMA column: this lane's query

  // Work item: the q tiles of one (sequence, head) pair get workgroup ids that
  // are equal mod 8, so they run on the same XCD and share its L2 for K/V.
  const int group = blockIdx.x / (8 * qtiles);
  const int rem = blockIdx.x - group * 8 * qtiles;
  const int qt = rem / 8;
  const int pair = group * 8 + rem % 8;
  if (pair >= a.num_seqs * a.num_heads) return;
  const int s = pair / a.num_heads, h = pair - s * a.num_heads;

  const int q0 = a.cu_q_lens[s];
  const int q_len = a.cu_q_lens[s + 1] - q0;
  const int n = min(max(a.context_lens[s], 0), a.ctx_cap);
  const int c = n - q_len;  // cached tokens before the chunk (queries past n are left alone)
  const int qbase = qt * kPfQ;
  if (qbase >= q_len || q_len <= 0) return;

  // ---- this lane's query and its Q fragments (B operand of S^T = K Q^T)
  const int jq = qbase + wave * 32 + col;  // query index in the chunk
  // Valid query: inside the chunk, inside the context, and inside q / out
  // (cu_q_lens is device data, so its rows are checked against total_q).
  const bool q_ok = jq < q_len && c + jq >= 0 && c + jq < n && q0 >= 0 && q0 + jq < a.total_q;
  const int qpos = c + jq;  // its absolute position
  uint4 qf[kPfD / 16];
  {
    const char *qrow =
        reinterpret_cast<const char *>(a.q) + ((int64_t)(q0 + (q_ok ? jq : 0)) * a.num_heads + h) * (kPfD * 2);
#pragma unroll
    for (int st = 0; st < kPfD / 16; ++st)
      qf[st] = q_ok ? *reinterpret_cast<const uint4 *>(qrow + (16 * st + 8 * half) * 2) : make_uint4(0, 0, 0, 0);
  }

  // ---- keys this workgroup and this wave need
  const int kv_end = max(0, min(n, c + qbase + kPfQ));  // keys [0, kv_end) for the tile
  const int nkb = (kv_end + kPfKeys - 1) / kPfKeys;
  const int wave_last = c + qbase + wave * 32 + 31;   // last position any query of the wave sees
  const int wave_nkb = max(0, min(nkb, (min(wave_last, n - 1) + kPfKeys) / kPfKeys));

  const char *kbase = reinterpret_cast<const char *>(a.k_cache);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache);
  const int64_t table_row = (int64_t)s * a.max_blocks;
  const int64_t head_off = (int64_t)h * B * (kPfD * 2);
  const int64_t block_stride = (int64_t)a.num_heads * B * (kPfD * 2);

  // The table entries of the tile's keys, copied once into LDS so the
  // address of every K/V load is one LDS read away (longer contexts read the
  // rest from memory).
  const int nent = (kv_end + B - 1) / B;
  for (int i = tid; i < min(nent, kTableCache); i += kPfWaves * kWave) {
    const int32_t e = a.block_tables[table_row + i];
    lds_table[i] = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  }
  __syncthreads();
  // Physical block of logical block lb, or -1 (outside the tile's keys or the pool).
  auto entry = [&](int lb) -> int32_t {
    if (lb * B >= kv_end) return -1;
    if (lb < kTableCache) return lds_table[lb];
    const int32_t e = a.block_tables[table_row + lb];
    return (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  };

  // Staging of one 32-key block, 16 bytes of K and 16 of V per thread.
  //  K: thread t loads chunk t of the 8 KB block: key t/16 (the 4 keys of a
  //     wave share one paged block), columns 8*(t%16) .. +8.
  //  V: key t%32, columns 8*(t/32) .. +8 (consecutive lanes, consecutive keys).
  // Every call issues both loads; keys outside [0, kv_end) read row 0 of
  // block 0 and are zeroed when stored, so the compiler can count loads.
  struct Stage {
    uint4 k, v;
    bool kok, vok;
  };
  auto load_block = [&](int kb, Stage &st) {
    const int kkey = kb * kPfKeys + wave * 4 + lane / 16;  // wave-uniform block
    const int32_t ke = entry((kb * kPfKeys + wave * 4) / B);
    st.kok = ke >= 0 && kkey < kv_end;
    const int64_t ka = st.kok ? (int64_t)ke * block_stride + head_off + (int64_t)(kkey % B) * (kPfD * 2) : 0;
    st.k = *reinterpret_cast<const uint4 *>(kbase + ka + (lane % 16) * 16);
    const int vkey = kb * kPfKeys + lane % 32;
    int32_t ve = -1;
#pragma unroll
    for (int b = 0; b < kPfKeys / B; ++b)  // the blocks of this 32-key block
      if ((lane % 32) / B == b) ve = entry((kb * kPfKeys) / B + b);
    if constexpr (B > kPfKeys) ve = entry((kb * kPfKeys) / B);
    st.vok = ve >= 0 && vkey < kv_end;
    const int64_t va = st.vok ? (int64_t)ve * block_stride + head_off + (int64_t)(vkey % B) * (kPfD * 2) : 0;
    st.v = *reinterpret_cast<const uint4 *>(vbase + va + (8 * (tid / 32)) * 2);
  };
  auto store_block = [&](int buf, const Stage &st) {
    const uint4 k = st.kok ? st.k : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(&lds_k[buf][(tid / 16) * kKRow + (tid % 16) * 16]) = k;
    const uint4 v = st.vok ? st.v : make_uint4(0, 0, 0, 0);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    const int key = tid % 32, dc = 8 * (tid / 32);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint16_t *>(&lds_v[buf][(dc + e) * kVRow + key * 2]) = (uint16_t)(w4[e / 2] >> (16 * (e % 2)));
  };

  // ---- running softmax state of this lane's query, and O^T accumulators
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[kPfD / 32];
#pragma unroll
  for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;

  // Lowest query position of the wave, and whether all its queries are valid:
  // key blocks entirely at or before it need no causal mask.
  const int wave_first = c + qbase + wave * 32;
  const bool wave_full = __builtin_amdgcn_ballot_w64(q_ok) == ~0ull;

  auto compute = [&](int kb, int buf) {
    // S^T = K Q^T over head_dim: A = K rows (permuted), B = this lane's Q;
    // two independent accumulation chains (even / odd head_dim steps).
    f32x16 s0, s1;
#pragma unroll
    for (int j = 0; j < 16; ++j) s0[j] = s1[j] = 0.f;
    const char *krow = &lds_k[buf][k_row_perm(col) * kKRow];
#pragma unroll
    for (int st = 0; st < kPfD / 16; st += 2) {
      const uint4 ka0 = *reinterpret_cast<const uint4 *>(krow + (16 * st + 8 * half) * 2);
      const uint4 ka1 = *reinterpret_cast<const uint4 *>(krow + (16 * (st + 1) + 8 * half) * 2);
      s0 = mfma<T>(ka0, qf[st], s0);
      s1 = mfma<T>(ka1, qf[st + 1], s1);
    }
    f32x16 sacc;
    // Register j holds key kb*32 + 16*(j/8) + 8*half + j%8 for this lane's query.
    float mloc = -INFINITY;
    if (wave_full && kb * kPfKeys + kPfKeys - 1 <= wave_first) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sacc[j] = (s0[j] + s1[j]) * a.scale_log2;
        mloc = fmaxf(mloc, sacc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int p = kb * kPfKeys + 16 * (j / 8) + 8 * half + (j % 8);
        const bool ok = q_ok && p <= qpos;
        sacc[j] = ok ? (s0[j] + s1[j]) * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, sacc[j]);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    // Lazy max: the reference max moves only when a block exceeds it by more
    // than 8 (log2 units), so weights stay <= 2^8 and O is rarely rescaled.
    // The result is the same softmax; only the common factor differs.
    const bool bump = mloc > m_run + 8.f;
    const float m_new = bump ? mloc : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = bump ? fast_exp2(m_run - m_use) : 1.f;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sacc[j] = fast_exp2(sacc[j] - m_use);
      lsum += sacc[j];
    }
    lsum += __shfl_xor(lsum, 32, kWave);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
      for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
    }
    // P^T as the B operand: k step t holds keys 16t + 8*half .. +8 = registers 8t .. 8t+7.
    // bf16 keeps only 8 significant bits, too few for the weights, so P is
    // carried as P_hi + P_lo (two bf16 terms, about 16 bits) and the product
    // is formed twice; fp16's 11 bits are enough on their own.
    uint4 pb[2], pl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = sacc[8 * t + e];
        float hi;
        if constexpr (T == Dt::BF16) hi = bf16_lo(f32_to_bf16_bits(p));
        else hi = (float)(_Float16)p;
        lo[e] = p - hi;
      }
      pb[t] = make_uint4(pack2<T>(sacc[8 * t + 0], sacc[8 * t + 1]), pack2<T>(sacc[8 * t + 2], sacc[8 * t + 3]),
                         pack2<T>(sacc[8 * t + 4], sacc[8 * t + 5]), pack2<T>(sacc[8 * t + 6], sacc[8 * t + 7]));
      pl[t] = make_uint4(pack2<T>(lo[0], lo[1]), pack2<T>(lo[2], lo[3]), pack2<T>(lo[4], lo[5]), pack2<T>(lo[6], lo[7]));
    }
    // O^T += V^T P^T: A = V^T rows (d = 32*dt + col), 8 keys at 16t + 8*half.
#pragma unroll
    for (int dt = 0; dt < kPfD / 32; ++dt) {
      const char *vrow = &lds_v[buf][(32 * dt + col) * kVRow];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 va = *reinterpret_cast<const uint4 *>(vrow + (16 * t + 8 * half) * 2);
        o[dt] = mfma<T>(va, pb[t], o[dt]);
        if constexpr (T == Dt::BF16) o[dt] = mfma<T>(va, pl[t], o[dt]);
      }
    }
  };

  // Pipeline: stage X holds block kb+1 (loaded during kb-1), stage Y receives
  // block kb+2; block kb is in LDS ring slot kb % 3.
  Stage sx, sy;
  if (nkb > 0) {
    load_block(0, sx);
    load_block(1, sy);  // harmless dummy loads when nkb == 1
    store_block(0, sx);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    // even step: X is free, Y holds kb+1
    load_block(kb + 2, sx);
    if (kb < wave_nkb) compute(kb, kb % kRing);
    if (kb + 1 < nkb) store_block((kb + 1) % kRing, sy);
    __syncthreads();
    if (kb + 1 >= nkb) break;
    // odd step: Y is free, X holds kb+2
    load_block(kb + 3, sy);
    if (kb + 1 < wave_nkb) compute(kb + 1, (kb + 1) % kRing);
    if (kb + 2 < nkb) store_block((kb + 2) % kRing, sx);
    __syncthreads();
  }

  // ---- write this lane's query: O^T register j of tile dt is d = 32*dt + 8*(j/4) + 4*half + j%4.
  if (q_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    char *orow = reinterpret_cast<char *>(a.out) + ((int64_t)(q0 + jq) * a.num_heads + h) * (kPfD * 2);
#pragma unroll
    for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const uint2 w = make_uint2(pack2<T>(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                   pack2<T>(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
        *reinterpret_cast<uint2 *>(orow + d * 2) = w;
      }
  }
}

bool prefill_supported(int dtype, int head_dim, int block_size) {
  const bool dt = dtype == (int)Dt::F16 || dtype == (int)Dt::BF16;
  const bool b = block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32;
  return dt && head_dim == kPfD && b;
}

template <Dt T, int B>
static hipError_t launch_pf(const PrefillArgs &a, hipStream_t st) {
  const int qtiles = (a.max_q_len + kPfQ - 1) / kPfQ;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_heads;
  const int64_t groups = (pairs + 7) / 8;
  const int64_t grid = groups * 8 * qtiles;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_chunk_kernel<T, B>), dim3((unsigned)grid), dim3(kPfWaves * kWave), 0, st, a, qtiles);
  return hipGetLastError();
}

template <Dt T>
static hipError_t launch_pf_b(const PrefillArgs &a, int B, hipStream_t st) {
  switch (B) {
    case 4: return launch_pf<T, 4>(a, st);
    case 8: return launch_pf<T, 8>(a, st);
    case 16: return launch_pf<T, 16>(a, st);
    case 32: return launch_pf<T, 32>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, int dtype, int head_dim, int block_size, hipStream_t stream) {
  if (!prefill_supported(dtype, head_dim, block_size)) return hipErrorInvalidValue;
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  if (dtype == (int)Dt::BF16) return launch_pf_b<Dt::BF16>(a, block_size, stream);
  return launch_pf_b<Dt::F16>(a, block_size, stream);
}

}  // namespace pa
