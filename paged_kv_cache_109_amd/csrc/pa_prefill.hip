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
// run on one XCD and read its K/V through the same L2, and the sequences are
// taken longest first.  K/V blocks of 32 keys are gathered through the block
// table (entries cached in LDS) straight from HBM into a 4-slot LDS ring by
// global_load_lds_dwordx4, three blocks ahead, with no register staging; the
// rows are stored as they are in memory, with the 16-byte chunks of each row
// XOR-swizzled so the operand reads below do not collide in the LDS banks.
//
// Per block a wave computes S^T = K Q^T with 8 v_mfma_f32_32x32x16 (bf16 or
// f16 in, fp32 out) and O^T += V^T P^T with 8 more (16 for bf16, whose P is
// carried as a high and a low bf16 term to keep the weights' precision).
// V^T operands come from the row-major V with ds_read_b64_tr_b16, the LDS
// read that transposes 16-bit elements across each group of 16 lanes.  The
// loop is software-pipelined: the S^T products of block kb+1 are issued
// before the softmax of block kb, so the matrix core and the vector ALU work
// at the same time.  Working transposed keeps one query per lane column: the
// softmax max needs one lane swap (v_permlane32_swap), the row sum stays
// in-lane until the end, and the rescale of O is per lane.  The K rows are
// fed to the MFMA bit-permuted (bits 2 and 3 of the key index swapped) so
// that the accumulator registers of S^T are exactly the B operand of the
// P V product.  A wave skips the key blocks past its causal limit; only
// blocks on a wave's diagonal are masked.

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPfD = 128;                // head_dim
constexpr int kPfWaves = 4;              // waves per workgroup
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfQ = 32 * kPfWaves;      // queries per workgroup
constexpr int kPfKeys = 32;              // keys per LDS block
constexpr int kRow = kPfD * 2;           // bytes of one K or V row
constexpr int kSlot = kPfKeys * kRow;    // bytes of one block of K (or V) in LDS
constexpr int kTableCache = 3072;        // table entries kept in LDS (12 KB)
constexpr int kSortSeqs = 64;            // batches up to this size run longest first

typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Position of 16-byte chunk c of LDS row r is c ^ swz(r), with swz(r) the
// two low bits of r over the next two (a bijection of r mod 16).  LDS serves
// 256 bytes per cycle: the 16 lanes of a K operand read hit 16 distinct rows
// mod 16 at one chunk, so 16 distinct positions; a transposing V read covers
// 4 aligned rows x 4 chunks per 32 lanes, and the row's low bits move the
// chunk by whole groups of 4, so again 16 distinct positions.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// s_waitcnt immediates (vmcnt in bits 3:0, expcnt 6:4, lgkmcnt 11:8; the
// other counters left at their maximum, i.e. not waited for).
constexpr int kWaitVm4 = 0x0F74;
constexpr int kWaitVm0 = 0x0F70;

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
  // The LDS ring: one array per slot, so the compiler can tell the slot a
  // read uses from the slots the in-flight loads write.
  __shared__ __attribute__((aligned(1024))) char k_0[kSlot], k_1[kSlot], k_2[kSlot], k_3[kSlot];
  __shared__ __attribute__((aligned(1024))) char v_0[kSlot], v_1[kSlot], v_2[kSlot], v_3[kSlot];
  __shared__ int32_t lds_table[kLong ? 1 : kTableCache];
  static_assert(kPfThreads == 256, "loads map 256 threads onto a 32-key block");

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

  auto entry = [&](int lb) __attribute__((always_inline)) -> uint32_t {
    if constexpr (kLong) {
      const int32_t e = a.block_tables[table_row + lb];
      return (e >= 0 && (int64_t)e < a.num_blocks) ? (uint32_t)e : 0u;
    } else {
      return (uint32_t)lds_table[lb];
    }
  };
  auto kslot = [&](auto sc) __attribute__((always_inline)) -> char * {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return k_0;
    else if constexpr (S == 1) return k_1;
    else if constexpr (S == 2) return k_2;
    else return k_3;
  };
  auto vslot = [&](auto sc) __attribute__((always_inline)) -> char * {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return v_0;
    else if constexpr (S == 1) return v_1;
    else if constexpr (S == 2) return v_2;
    else return v_3;
  };

  // Loading one 32-key block: each wave moves 4 rows of K and 4 of V per
  // instruction (64 lanes x 16 bytes land contiguously in LDS), rows
  // 4*wave .. +3 and 16 + 4*wave .. +3.  Lane l fills position l%16 of its
  // row with chunk (l%16) ^ swz(row) of the K/V row.  Keys at or past kv_end
  // read the row of key kv_end-1 instead: their scores are masked and their
  // weights are 0, and a real (finite) V row keeps 0 * V finite.
  const int r0 = 4 * wave + lane / 16;  // swz(r0 + 16) == swz(r0)
  const uint32_t chunk_off = (uint32_t)(16 * ((lane % 16) ^ swz(r0)));
  // A block's load in two steps, so the table lookup can run well ahead of
  // the loads: the two table entries of this thread's rows, then the four
  // loads into ring slot `sc`.
  struct Rows {
    uint32_t e0, e1;
    int key0, key1;
  };
  auto rows = [&](int kb) __attribute__((always_inline)) -> Rows {
    Rows r;
    r.key0 = min(kb * kPfKeys + r0, kv_end - 1);
    r.key1 = min(kb * kPfKeys + r0 + 16, kv_end - 1);
    r.e0 = entry(r.key0 / B);
    r.e1 = entry(r.key1 / B);
    return r;
  };
  auto issue_half = [&](const Rows &r, int part, auto sc) __attribute__((always_inline)) {
    const uint32_t e = part ? r.e1 : r.e0;
    const int key = part ? r.key1 : r.key0;
    const uint64_t off = (uint64_t)e * block_stride + (uint32_t)((key & (B - 1)) * kRow) + chunk_off;
    const int dst = 1024 * (wave + 4 * part);
    __builtin_amdgcn_global_load_lds(kbase + off, (lds_char *)(kslot(sc) + dst), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vbase + off, (lds_char *)(vslot(sc) + dst), 16, 0, 0);
  };
  auto load_block = [&](int kb, auto sc) __attribute__((always_inline)) {
    const Rows r = rows(kb);
    issue_half(r, 0, sc);
    issue_half(r, 1, sc);
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

  // Per-lane LDS offsets of the MFMA operands.  K: row R = k_row_perm(col),
  // chunk 2*st + half, at its swizzled position.  V^T (transposing reads):
  // for rows d = 32*dt + col and keys 16*t + 8*half + 4*i .. +3, lane j of
  // each 16-lane group points at 4 elements of key 16*t + 8*half + 4*i +
  // j/4, columns 32*dt + 16*(lane/16 % 2) + 4*(j%4) .. +3; the read hands
  // lane j element e of the lane 4*e + j/4 that pointed there.  The offset
  // of read (dt, i) is fixed per lane; t adds 16 rows.
  uint32_t k_off[kPfD / 16];
  {
    const int R = k_row_perm(col);
#pragma unroll
    for (int st = 0; st < kPfD / 16; ++st) k_off[st] = (uint32_t)(R * kRow + 16 * ((2 * st + half) ^ swz(R)));
  }
  uint32_t v_off[kPfD / 32][2];
  {
    const int j = lane % 16, gm = (lane / 16) % 2;
#pragma unroll
    for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int key = 8 * half + 4 * i + j / 4;
        const int chunk = 4 * dt + 2 * gm + (j % 4) / 2;
        v_off[dt][i] = (uint32_t)(key * kRow + 16 * (chunk ^ swz(key)) + 8 * (j % 2));
      }
  }

  // ---- operand reads and products.
  // K operand st of the block in slot `sc` (A of S^T = K Q^T).
  auto kread = [&](auto sc, int st) __attribute__((always_inline)) -> uint4 {
    return load16(kslot(sc) + k_off[st]);
  };
  // V^T operand (t, dt) of the block in slot `sc` (A of O^T += V^T P^T).
  auto vread = [&](auto sc, int t, int dt) __attribute__((always_inline)) -> uint4 {
    const lds_char *vb_ = (const lds_char *)vslot(sc);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3))) *)(vb_ + v_off[dt][0] + 16 * kRow * t));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3))) *)(vb_ + v_off[dt][1] + 16 * kRow * t));
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3)));
  };
  // S^T of the block in slot `sc` in one go (used before the loop).
  auto qk = [&](auto sc) __attribute__((always_inline)) -> f32x16 {
    f32x16 sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
    for (int st = 0; st < kPfD / 16; ++st) sacc = mfma<T>(kread(sc, st), qf[st], sacc);
    return sacc;
  };

  // PV MFMA n of a block: t = n / (kPV/2), then the four accumulators in
  // turn (P_hi first, then P_lo for bf16), so consecutive MFMAs never depend
  // on each other.
  constexpr int kPV = (T == Dt::BF16) ? 16 : 8;
  auto pv = [&](int n, const uint4 (&va)[2][kPfD / 32], const uint4 (&pb)[2], const uint4 (&pl)[2])
                __attribute__((always_inline)) {
    const int t = n / (kPV / 2), r = n % (kPV / 2), dt = r % 4;
    o[dt] = mfma<T>(va[t][dt], r < 4 ? pb[t] : pl[t], o[dt]);
  };

  // Weights of one block from its masked scores x against the reference m:
  // p = 2^(x*scale_log2 - m), their sum, and P^T packed as the B operand (k
  // step t holds keys 16t + 8*half .. +8 = registers 8t .. 8t+7).  bf16
  // keeps only 8 significant bits, too few for the weights, so P is carried
  // as P_hi + P_lo (P_hi the top 16 bits of the float, P_lo the rest rounded
  // to bf16: about 16 bits together) and the product is formed twice; fp16's
  // 11 bits are enough on their own.

  // One half-step of a wave that still has block h to do (raw S^T of block
  // h in `scur`).  First the lazy-max check: the reference max m_run moves
  // only when a block exceeds it by more than 8 (log2 units), so weights
  // stay <= 2^8 and O is rarely rescaled; the result is the same softmax,
  // only the common factor differs.  Each half of the wave judges its own 16
  // keys of the query, and only if some query's max moves do the halves
  // agree on it and rescale O (which holds blocks up to h-1).  Then one
  // fenced region of 8 + kPV MFMA slots fixes the issue order so the
  // matrix core and the vector ALU work at once:
  //  - slots 0..7: S^T of block h+1 (K from slot KS, into `snext`), with the
  //    weights of keys 0..15 of block h and the reads of block h's V^T
  //    operands (slot VS) under them;
  //  - the first half of the P V products (keys 0..15), with the weights of
  //    keys 16..31 under them;
  //  - the second half, with block h+3's loads (into slot DS) under them.
  auto compute = [&](int h, f32x16 &scur, f32x16 &snext, auto vs, auto ks, auto ds)
                     __attribute__((always_inline)) {
    f32x16 &x = scur;
    if (!(wave_full && h * kPfKeys + kPfKeys - 1 <= wave_first)) {
      // Register j is key h*32 + 8*half + (16*(j/8) + j%8); it is visible
      // to this lane's query iff that is <= qpos.
      const int lim = q_ok ? qpos - h * kPfKeys - 8 * half : -1;
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = (16 * (j / 8) + j % 8 <= lim) ? x[j] : -INFINITY;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) mx = fmaxf(mx, x[j]);
    if (__builtin_amdgcn_ballot_w64(mx * sc > m_run + 8.f) != 0) {
      mx = fmaxf(mx, other_half(mx));
      const float mblk = mx * sc;
      const bool bump = mblk > m_run + 8.f;
      const float m_new = bump ? mblk : m_run;
      const float alpha = bump ? fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new)) : 1.f;
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < kPfD / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
    }
    const float m = (m_run == -INFINITY) ? 0.f : m_run;
    const Rows nr = rows(h + 3);
    const bool more = h + 3 < nkb;  // block h+3 exists: load it
    uint4 ka[kPfD / 16], va[2][kPfD / 32], pb[2], pl[2];
    float p[16], lsum = 0.f;
    // Pair q (registers 2q, 2q+1): the two weights, then their packing.
    auto exps = [&](int q) __attribute__((always_inline)) {
      p[2 * q] = fast_exp2(fmaf(x[2 * q], sc, -m));
      p[2 * q + 1] = fast_exp2(fmaf(x[2 * q + 1], sc, -m));
      lsum += p[2 * q];
      lsum += p[2 * q + 1];
    };
    auto pack = [&](int q) __attribute__((always_inline)) {
      const float p0 = p[2 * q], p1 = p[2 * q + 1];
      uint32_t hw, lw = 0;
      if constexpr (T == Dt::BF16) {
        const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
        hw = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // high halves: p1 | p0
        lw = pack_pair<true>(p0 - __uint_as_float(b0 & 0xffff0000u), p1 - __uint_as_float(b1 & 0xffff0000u));
      } else {
        hw = pack_pair<false>(p0, p1);
      }
      const int t = q / 4, e = q % 4;
      if (e == 0) { pb[t].x = hw; pl[t].x = lw; }
      else if (e == 1) { pb[t].y = hw; pl[t].y = lw; }
      else if (e == 2) { pb[t].z = hw; pl[t].z = lw; }
      else { pb[t].w = hw; pl[t].w = lw; }
    };
    constexpr int kHalf = kPV / 2;       // PV MFMAs per key half
    constexpr int kPer = kHalf / 4;      // slots per pair while the first half runs
    ka[0] = kread(ks, 0);
    ka[1] = kread(ks, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < 8 + kPV; ++sl) {
      if (sl < 8) {
        snext = mfma<T>(ka[sl], qf[sl], sl == 0 ? f32x16{} : snext);
        if (sl + 2 < 8) ka[sl + 2] = kread(ks, sl + 2);
        va[sl / 4][sl % 4] = vread(vs, sl / 4, sl % 4);
        if (sl % 2 == 0) exps(sl / 2);
        else pack(sl / 2);
      } else {
        pv(sl - 8, va, pb, pl);
        if (sl < 8 + kHalf) {
          const int local = sl - 8, q = 4 + local / kPer;
          if (kPer == 1 || local % kPer == 0) exps(q);
          if (kPer == 1 || local % kPer == 1) pack(q);
        }
        if (more && sl == 8 + kHalf) issue_half(nr, 0, ds);
        if (more && sl == 8 + kHalf + 2) issue_half(nr, 1, ds);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lsum;
  };
  auto step = [&](int h, f32x16 &scur, f32x16 &snext, auto vs, auto ks, auto ds) __attribute__((always_inline)) {
    if (h < wave_nkb) compute(h, scur, snext, vs, ks, ds);
    else if (h + 3 < nkb) load_block(h + 3, ds);
  };

  // Wait until at most `kWait` of this wave's loads are in flight, then
  // meet the other waves.  The loads write LDS directly, so a barrier with
  // the usual memory fence would wait for all of them; this one waits only
  // for the older blocks (the empty asm statements keep the compiler from
  // moving LDS accesses across it).
  auto sync_blocks = [&](auto wait) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(decltype(wait)::value);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Pipeline.  Half-step h starts with blocks h and h+1 in the ring (slots
  // h%4, (h+1)%4) and block h+2's loads in flight; it issues block h+3's
  // loads into the slot block h-1 used, computes, waits for block h+2 and
  // ends at a barrier.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using Wait4 = std::integral_constant<int, kWaitVm4>;
  using Wait0 = std::integral_constant<int, kWaitVm0>;
  // End of half-step h: while blocks are still being loaded, the four loads
  // of block h+3 may stay in flight; past the last block none were issued.
  auto end_step = [&](int h) __attribute__((always_inline)) {
    if (h + 3 < nkb) sync_blocks(Wait4{});
    else sync_blocks(Wait0{});
  };
  f32x16 sa, sb;
#pragma unroll
  for (int j = 0; j < 16; ++j) sa[j] = sb[j] = 0.f;
  if (nkb > 0) {
    // The Q fragments are in registers before any block load is issued (so
    // no later wait for them has to count the block loads).
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    load_block(0, S0{});
    if (nkb > 1) load_block(1, S1{});
    if (nkb > 2) {
      load_block(2, S2{});
      sync_blocks(Wait4{});  // blocks 0 and 1 are in
    } else {
      sync_blocks(Wait0{});
    }
    if (0 < wave_nkb) sa = qk(S0{});
    for (int h = 0;; h += 4) {
      step(h, sa, sb, S0{}, S1{}, S3{});
      end_step(h);
      if (h + 1 >= nkb) break;
      step(h + 1, sb, sa, S1{}, S2{}, S0{});
      end_step(h + 1);
      if (h + 2 >= nkb) break;
      step(h + 2, sa, sb, S2{}, S3{}, S1{});
      end_step(h + 2);
      if (h + 3 >= nkb) break;
      step(h + 3, sb, sa, S3{}, S0{}, S2{});
      end_step(h + 3);
      if (h + 4 >= nkb) break;
    }
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

static bool prefill_mfma_supported(int dtype, int head_dim, int block_size) {
  const bool dt = dtype == (int)Dt::F16 || dtype == (int)Dt::BF16;
  const bool b = block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
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
    case 64: return launch_pf<T, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(int dtype, int head_dim, int block_size) {
  return prefill_mfma_supported(dtype, head_dim, block_size) || prefill_general_supported(dtype, head_dim, block_size);
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, int dtype, int head_dim, int block_size, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  if (prefill_mfma_supported(dtype, head_dim, block_size)) {
    if (dtype == (int)Dt::BF16) return launch_pf_b<Dt::BF16>(a, block_size, stream);
    return launch_pf_b<Dt::F16>(a, block_size, stream);
  }
  // fp32, or head_dim 64: the vector-ALU kernel.
  if (prefill_general_supported(dtype, head_dim, block_size))
    return launch_prefill_general(a, dtype, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
