// Chunked-prefill attention over a paged KV cache, on MFMA (gfx950).
//
// What is computed: a sequence's chunk of q_len new queries follows c cached
// tokens; query j sits at position c + j and attends, causally, to positions
// 0 .. c + j of the sequence -- the same softmax attention as decode, with
// the K/V read through the block table (paper notes "PagedAttention:
// Efficient Memory Management for Large Language Model Serving with
// PagedAttention", unpurerationalist.github.io, section 3.1; chunking long
// prompts across steps: the arcyou.ai teardown of vLLM, continuous-batching
// section).  Unlike decode, this IS a dense contraction (32 queries share
// every K/V row a wave reads), so it runs on the matrix cores.
//
// Mapping to CDNA4.  A workgroup of 4 waves takes 128 queries of one
// (sequence, head); each wave owns 32 of them, one per MFMA column.  Two
// workgroups share a CU, so one's barrier waits are the other's issue slots.
// The q tiles of one (sequence, head) get workgroup ids equal mod 8, so they
// run on one XCD and read its K/V through the same L2.  K/V stream through
// a 3-slot LDS ring in blocks of 32 keys gathered through the block table
// (entries cached in LDS); global loads run two blocks ahead in registers.
//
// Per block a wave computes S^T = K Q^T with 8 v_mfma_f32_32x32x16 (bf16 or
// f16 in, fp32 out) and O^T += V^T P^T with 8 more (16 for bf16, whose P is
// carried as a high and a low bf16 term to keep the weights' precision).
// The loop is software-pipelined: the S^T products of block kb+1 are issued
// before the softmax of block kb, so the matrix core and the vector ALU work
// at the same time.  Working transposed keeps one query per lane column: the
// softmax max needs one lane swap (v_permlane32_swap), the row sum stays
// in-lane until the end, and the rescale of O is per lane.  The K rows are
// fed to the MFMA bit-permuted (bits 2 and 3 of the key index swapped) so
// that the accumulator registers of S^T are exactly the B operand of the
// P V product.  V is written to LDS transposed (V^T[d][key]) so its operand
// reads are 16 contiguous bytes.  A wave skips the key blocks past its
// causal limit; only blocks on a wave's diagonal are masked.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPfD = 128;                // head_dim
constexpr int kPfWaves = 4;              // waves per workgroup
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfQ = 32 * kPfWaves;      // queries per workgroup
constexpr int kPfKeys = 32;              // keys per LDS block
constexpr int kKRow = kPfD * 2 + 16;     // bytes per K row in LDS (padded)
constexpr int kVRow = kPfKeys * 2 + 16;  // bytes per V^T row in LDS (padded)
constexpr int kKBuf = kPfKeys * kKRow;   // 8704 B
constexpr int kVBuf = kPfD * kVRow;      // 10240 B
constexpr int kRing = 3;                 // LDS slots: V of kb, K of kb+1, store of kb+2
constexpr int kTableCache = 4096;        // table entries kept in LDS (16 KB)
constexpr int kSortSeqs = 64;            // batches up to this size run longest first

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

// Row of the K block fed to MFMA row r: bits 2 and 3 of r swapped.
__device__ __forceinline__ int k_row_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// x of lane (lane ^ 32), by v_permlane32_swap (which exchanges the upper
// half of its first operand with the lower half of its second).  Every lane
// of the wave must be active.
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x % kWave < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ uint4 load16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }

}  // namespace

// kLong: contexts longer than kTableCache*B tokens read their table entries
// from global memory instead of the LDS copy.
template <Dt T, int B, bool kLong>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_chunk_kernel(PrefillArgs a, int qtiles) {
  __shared__ __attribute__((aligned(16))) char lds_k[kRing][kKBuf];
  __shared__ __attribute__((aligned(16))) char lds_v[kRing][kVBuf];
  __shared__ int32_t lds_table[kLong ? 1 : kTableCache];
  static_assert(kPfThreads == 256, "staging maps 256 threads onto a 32-key block");

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
  const int rank = pair / a.num_heads, h = pair - rank * a.num_heads;
  // Workgroups start in id order as earlier ones finish, so the longest
  // contexts go first (longest-processing-time order): for up to
  // kSortSeqs sequences, the sequence of rank r is the one with the r-th
  // largest context length (ties by index).
  int s = rank;
  if (a.num_seqs <= kSortSeqs) {
    __shared__ int32_t lds_ctx[kSortSeqs];
    __shared__ int32_t lds_seq;
    if (tid < a.num_seqs) lds_ctx[tid] = a.context_lens[tid];
    __syncthreads();
    if (tid < a.num_seqs) {
      const int32_t mine = lds_ctx[tid];
      int before = 0;
      for (int j = 0; j < a.num_seqs; ++j) {
        const int32_t cj = lds_ctx[j];
        before += (cj > mine || (cj == mine && j < tid)) ? 1 : 0;
      }
      if (before == rank) lds_seq = tid;
    }
    __syncthreads();
    s = lds_seq;
  }

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
        reinterpret_cast<const char *>(a.q) + ((int64_t)(q_ok ? q0 + jq : 0) * a.num_heads + h) * (kPfD * 2);
#pragma unroll
    for (int st = 0; st < kPfD / 16; ++st)
      qf[st] = q_ok ? load16(qrow + (16 * st + 8 * half) * 2) : make_uint4(0, 0, 0, 0);
  }

  // ---- keys this workgroup and this wave need
  const int kv_end = max(0, min(n, c + qbase + kPfQ));  // keys [0, kv_end) for the tile
  const int nkb = (kv_end + kPfKeys - 1) / kPfKeys;
  const int wave_last = c + qbase + wave * 32 + 31;  // last position any query of the wave sees
  const int wave_nkb = max(0, min(nkb, (min(wave_last, n - 1) + kPfKeys) / kPfKeys));

  const int64_t table_row = (int64_t)s * a.max_blocks;
  const uint32_t block_stride = (uint32_t)a.num_heads * B * (kPfD * 2);
  // Base of this head's rows: block e's row r of this head is at
  // e*block_stride + r*256 from here.
  const char *kbase = reinterpret_cast<const char *>(a.k_cache) + (int64_t)h * B * (kPfD * 2);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache) + (int64_t)h * B * (kPfD * 2);

  // The table entries of the tile's keys, copied once into LDS.  An entry
  // outside the pool is replaced by block 0, so every address formed below
  // stays inside the caches; only the keys of a well-formed table matter.
  const int nent = max((kv_end + B - 1) / B, 1);
  if constexpr (!kLong) {
    for (int i = tid; i < nent; i += kPfThreads) {
      const int32_t e = a.block_tables[table_row + i];
      lds_table[i] = (e >= 0 && (int64_t)e < a.num_blocks) ? e : 0;
    }
    __syncthreads();
  }

  // Staging of one 32-key block: per thread two 16-byte K chunks and two V
  // chunks.  K: keys r0 = tid/16 and r0 + 16 of the block, columns
  // 8*(tid%16) .. +8.  V: key tid%32, columns 8*(tid/32) and 64 + 8*(tid/32)
  // (consecutive lanes, consecutive keys, so the transposed LDS writes do not
  // collide).  The in-block part of each address is fixed per lane; only the
  // table entry changes with the block.  Every call issues all four loads
  // (keys past the table end read the last entry's block), and V rows of
  // keys at or past kv_end are zeroed when stored -- their K rows need no
  // zeroing, because those keys are masked out of every query's softmax.
  const int r0 = tid / 16, rv = tid % 32;
  const uint32_t lane_k0 = (uint32_t)((r0 & (B - 1)) * (kPfD * 2) + (tid % 16) * 16);
  const uint32_t lane_k1 = (uint32_t)(((r0 + 16) & (B - 1)) * (kPfD * 2) + (tid % 16) * 16);
  const uint32_t lane_v = (uint32_t)((rv & (B - 1)) * (kPfD * 2) + (tid / 32) * 16);
  auto entry = [&](int lb) __attribute__((always_inline)) -> uint32_t {
    lb = min(lb, nent - 1);
    if constexpr (kLong) {
      const int32_t e = a.block_tables[table_row + lb];
      return (e >= 0 && (int64_t)e < a.num_blocks) ? (uint32_t)e : 0u;
    } else {
      return (uint32_t)lds_table[lb];
    }
  };
  struct Stage {
    uint4 k0, k1, v[2];
    bool vok;
  };
  auto load_block = [&](int kb, Stage &st) __attribute__((always_inline)) {
    const int lb = kb * (kPfKeys / B);
    const char *k0 = kbase + ((uint64_t)entry(lb + r0 / B) * block_stride + lane_k0);
    const char *k1 = kbase + ((uint64_t)entry(lb + (r0 + 16) / B) * block_stride + lane_k1);
    const char *v = vbase + ((uint64_t)entry(lb + rv / B) * block_stride + lane_v);
    st.vok = kb * kPfKeys + rv < kv_end;
    st.k0 = load16(k0);
    st.k1 = load16(k1);
    st.v[0] = load16(v);
    st.v[1] = load16(v + 128);
  };
  auto store_block = [&](int buf, const Stage &st) __attribute__((always_inline)) {
    char *kd = &lds_k[buf][r0 * kKRow + (tid % 16) * 16];
    *reinterpret_cast<uint4 *>(kd) = st.k0;
    *reinterpret_cast<uint4 *>(kd + 16 * kKRow) = st.k1;
    // Masks applied per word (a select between whole vectors would be turned
    // into a select between their addresses, forcing them into memory).
    const uint32_t mv = st.vok ? ~0u : 0u;
    const int dc = 8 * (tid / 32);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const uint32_t w4[4] = {st.v[part].x & mv, st.v[part].y & mv, st.v[part].z & mv, st.v[part].w & mv};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t *>(&lds_v[buf][(dc + 64 * part + e) * kVRow + rv * 2]) =
            (uint16_t)(w4[e / 2] >> (16 * (e % 2)));
    }
  };

  // ---- running softmax state of this lane's query, and O^T accumulators.
  // l_run is this lane's half of the row sum (its 16 keys of every block);
  // both halves share m_run, so the halves are added only at the end.
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
  const float sc = a.scale_log2;  // > 0 (checked by the host)

  // S^T of the block in LDS slot `slot` for this lane's query: register j
  // holds the raw q.k of key 16*(j/8) + 8*half + j%8 of the block.
  auto qk = [&](int slot) __attribute__((always_inline)) -> f32x16 {
    f32x16 sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
    const char *krow = &lds_k[slot][k_row_perm(col) * kKRow];
#pragma unroll
    for (int st = 0; st < kPfD / 16; ++st)
      sacc = mfma<T>(load16(krow + (16 * st + 8 * half) * 2), qf[st], sacc);
    return sacc;
  };

  // One block of a wave: the softmax of block kb (raw scores `scur`) into
  // P^T, O^T += V^T P^T, and -- issued among the softmax instructions so the
  // matrix core is busy meanwhile -- S^T of block kb+1 into `snext`.
  auto compute = [&](int kb, f32x16 &scur, f32x16 &snext) __attribute__((always_inline)) {
    f32x16 &x = scur;
    if (!(wave_full && kb * kPfKeys + kPfKeys - 1 <= wave_first)) {
      // Register j is key kb*32 + 8*half + (16*(j/8) + j%8); it is visible
      // to this lane's query iff that is <= qpos.
      const int lim = q_ok ? qpos - kb * kPfKeys - 8 * half : -1;
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = (16 * (j / 8) + j % 8 <= lim) ? x[j] : -INFINITY;
    }
    snext = qk((kb + 1) % kRing);
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, other_half(mx));
    // Lazy max: the reference max moves only when a block exceeds it by more
    // than 8 (log2 units), so weights stay <= 2^8 and O is rarely rescaled.
    // The result is the same softmax; only the common factor differs.
    const float mblk = mx * sc;
    const bool bump = mblk > m_run + 8.f;
    const float m_new = bump ? mblk : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = bump ? fast_exp2(m_run - m_use) : 1.f;
    float p[16];
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = fast_exp2(fmaf(x[j], sc, -m_use));
      lsum += p[j];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    // P^T as the B operand: k step t holds keys 16t + 8*half .. +8 =
    // registers 8t .. 8t+7.  bf16 keeps only 8 significant bits, too few for
    // the weights, so P is carried as P_hi + P_lo (P_hi the top 16 bits of
    // the float, P_lo the rest rounded to bf16: about 16 bits together) and
    // the product is formed twice; fp16's 11 bits are enough on their own.
    uint4 pb[2], pl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = p[8 * t + 2 * e], p1 = p[8 * t + 2 * e + 1];
        if constexpr (T == Dt::BF16) {
          const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
          hw[e] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // high halves: p1 | p0
          lw[e] = pack_pair<true>(p0 - __uint_as_float(b0 & 0xffff0000u), p1 - __uint_as_float(b1 & 0xffff0000u));
        } else {
          hw[e] = pack_pair<false>(p0, p1);
          lw[e] = 0;
        }
      }
      pb[t] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      pl[t] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
      for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
    }
    // O^T += V^T P^T: A = V^T rows (d = 32*dt + col), 8 keys at 16t + 8*half.
#pragma unroll
    for (int dt = 0; dt < kPfD / 32; ++dt) {
      const char *vrow = &lds_v[kb % kRing][(32 * dt + col) * kVRow];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 va = load16(vrow + (16 * t + 8 * half) * 2);
        o[dt] = mfma<T>(va, pb[t], o[dt]);
        if constexpr (T == Dt::BF16) o[dt] = mfma<T>(va, pl[t], o[dt]);
      }
    }
  };

  // Pipeline.  At the top of a half-step for block kb: blocks kb and kb+1
  // are in LDS (slots kb%3, (kb+1)%3), one staging set holds block kb+2
  // (loaded during the previous half-step), and the wave holds S^T of block
  // kb.  The half-step loads block kb+3 into the other set, computes block kb
  // (and S^T of kb+1), stores kb+2 into the slot block kb-1 used, and ends at
  // a barrier.  The loop runs whole pairs of half-steps (an odd block count
  // ends with an idle half-step), so the two staging sets and the two score
  // tiles keep fixed registers.
  Stage sx, sy;
  f32x16 sa, sb;
#pragma unroll
  for (int j = 0; j < 16; ++j) sa[j] = sb[j] = 0.f;
  if (nkb > 0) {
    load_block(0, sx);
    load_block(1, sy);
    store_block(0, sx);
    store_block(1, sy);
    load_block(2, sx);
  }
  __syncthreads();
  if (0 < wave_nkb) sa = qk(0);
  for (int kb = 0; kb < nkb; kb += 2) {
    load_block(kb + 3, sy);
    if (kb < wave_nkb) compute(kb, sa, sb);
    if (kb + 2 < nkb) store_block((kb + 2) % kRing, sx);
    __syncthreads();
    load_block(kb + 4, sx);
    if (kb + 1 < wave_nkb) compute(kb + 1, sb, sa);
    if (kb + 3 < nkb) store_block((kb + 3) % kRing, sy);
    __syncthreads();
  }

  // ---- write this lane's query: O^T register j of tile dt is d = 32*dt + 8*(j/4) + 4*half + j%4.
  const float l = l_run + other_half(l_run);
  if (q_ok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    char *orow = reinterpret_cast<char *>(a.out) + ((int64_t)(q0 + jq) * a.num_heads + h) * (kPfD * 2);
#pragma unroll
    for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const uint2 w = make_uint2(pack_pair<T == Dt::BF16>(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                   pack_pair<T == Dt::BF16>(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
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
  // The LDS copy of the table covers every tile whose context fits it.
  if ((int64_t)a.ctx_cap > (int64_t)kTableCache * B)
    hipLaunchKernelGGL((prefill_chunk_kernel<T, B, true>), dim3((unsigned)grid), dim3(kPfThreads), 0, st, a, qtiles);
  else
    hipLaunchKernelGGL((prefill_chunk_kernel<T, B, false>), dim3((unsigned)grid), dim3(kPfThreads), 0, st, a,
                       qtiles);
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
