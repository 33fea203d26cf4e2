// Chunked-prefill attention over a paged KV cache, on MFMA (gfx950).
//
// What is computed: a sequence's chunk of q_len new queries follows c cached
// tokens; query j sits at position c + j and attends, causally, to positions
// 0 .. c + j of the sequence -- the same softmax attention as decode, with
// the K/V read through the block table (paper notes "PagedAttention:
// Efficient Memory Management for Large Language Model Serving with
// PagedAttention", unpurerationalist.github.io, section 3.1; chunking long
// prompts across steps: the arcyou.ai teardown of vLLM, continuous-batching
// section).  Unlike decode, this IS a dense contraction (16 queries share
// every K/V row a wave reads), so it runs on the matrix cores.
//
// Mapping to CDNA4.  A workgroup of 8 waves takes 128 queries of one
// (sequence, head); each wave owns 16 of them, one per column of a 16x16
// MFMA tile.  A wave needs at most 128 VGPRs, so two workgroups share a CU at
// four waves per SIMD: while one wave waits on LDS, an exp chain or the
// matrix core, another issues.  The q tiles of one (sequence, head) get
// workgroup ids equal mod 8, so they run on one XCD and read its K/V
// through the same L2, and the heaviest tiles are taken first (longest
// context, then the last q tile).  K/V blocks of 32 keys are gathered
// through the block table straight from HBM into a 4-slot LDS ring by
// global_load_lds_dwordx4, three blocks ahead, with no register staging; the
// rows are stored as they are in memory, with the 16-byte chunks of each row
// XOR-swizzled so the operand reads below do not collide in the LDS banks.
//
// Per block a wave computes S^T = K Q^T with 8 v_mfma_f32_16x16x32 (two
// 16-key tiles x four 32-wide steps of the head dimension; bf16 or f16 in,
// fp32 out) and O^T += V^T P^T with 8 more, always in f16: bf16 keeps too
// few bits for the weights P, so for bf16 caches each wave rewrites the V
// rows it loaded into the ring as f16 once (exact inside f16's range; below
// 2^-14 the error is under 2^-25 absolute) and P goes in as f16.  A V value
// beyond f16's range turns into inf there, which leaves the accumulators of
// every wave that reads it non-finite; such a wave (as any wave whose
// accumulators end non-finite, e.g. 0 * NaN from a key it must not see)
// recomputes its queries key by key in fp32 straight from the cache, so
// the result is exact for any input and the fast path pays nothing.  Working
// transposed keeps one query per lane column: lane (g, n) holds query n's
// scores of keys 16*mt + 4g + j (tile mt, register j), and those eight
// registers, packed, are exactly its B operand of the P V product -- the
// contraction index 8g + 4mt + j is mapped to that key, and the V^T operand
// is read with the same map.  V^T comes from the row-major V with
// ds_read_b64_tr_b16, the LDS read that transposes 16-bit elements across
// each group of 16 lanes.  A wave skips the key blocks past its causal
// limit; only blocks on a wave's diagonal are masked.

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPfD = 128;                     // head_dim
constexpr int kPfWaves = 8;                   // waves per workgroup
constexpr int kPfRing = 4;                    // LDS ring slots (blocks)
constexpr int kPfOcc = 2;                     // workgroups per CU
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfWaveQ = 16;                  // queries per wave
constexpr int kPfQ = kPfWaveQ * kPfWaves;     // queries per workgroup
constexpr int kPfKeys = 32;                   // keys per LDS block
constexpr int kRow = kPfD * 2;                // bytes of one K or V row
constexpr int kSlot = kPfKeys * kRow;         // bytes of one block of K (or V) in LDS
constexpr int kLoads = kSlot / (kPfThreads * 16);  // K (and V) loads per wave per block
constexpr int kSortSeqs = 64;                 // batches up to this size run longest first
constexpr int kWavesPerEu = kPfOcc * kPfWaves / 4;
static_assert(kLoads >= 1 && kLoads * kPfThreads * 16 == kSlot, "a block splits evenly over the waves");
static_assert(kPfWaves >= 4, "load rows 16 apart share their swizzle");
static_assert(kPfOcc * (2 * kPfRing * kSlot + 4 * kSortSeqs + 16) <= 160 * 1024,
              "kPfOcc workgroups fit the LDS of a CU");

typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Position of 16-byte chunk c of LDS row r is c ^ swz(r), swz a bijection
// of r mod 16 (bits r1 r0, r2^r3, r3 from the top).  LDS serves 64 banks of
// 4 bytes.  A K operand read has the 16 lanes of a quarter-wave on rows
// 0..15 of a tile at one chunk: 16 distinct positions.  A transposing V read
// has lane group g on rows 4g .. 4g+3, 32 bytes (an aligned chunk pair) of
// each; swz(r) / 2 differs across any two groups' rows, so groups served
// together (g with g+1, or g with g+2) land in distinct banks.
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 3) & 1);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are in flight (n < 64; expcnt and lgkmcnt not waited for).
template <int N>
struct WaitVm : std::integral_constant<int, 0x0F70 | (N & 15) | ((N >> 4) << 14)> {
  static_assert(N >= 0 && N < 64, "vmcnt range");
};
// s_waitcnt immediate that waits for this wave's LDS (and scalar) operations.
struct WaitLgkm0 : std::integral_constant<int, 0xC07F> {};

template <Dt T>
__device__ __forceinline__ f32x4 mfma(const uint4 &a, const uint4 &b, const f32x4 &c) {
  if constexpr (T == Dt::BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
  }
}

__device__ __forceinline__ uint4 load16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }

// Eight 16-bit values of dtype T (one 16-byte chunk) as floats.
template <Dt T>
__device__ __forceinline__ void widen8(const uint4 &w, float (&f)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (T == Dt::BF16) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    } else {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
    }
  }
}

// 16 bytes per lane from global memory straight into LDS (lane i writes
// dst + 16*i; dst must be wave-uniform; M0 holds the LDS address).  Issued
// as inline assembly so the compiler does not track it: its own tracking of
// these loads loses the ring slots apart at loop joins and drains every
// load in flight before some operand reads (the compiler builtin for this
// load measured 5% slower for that reason).  Every read of the ring is
// ordered after its load by this kernel's own s_waitcnt vmcnt and barrier.
// M0 is a register the compiler reserves: it does not honour the clobber
// (it warns so) and keeps no value of its own in M0 across these
// statements -- this kernel's code has no other use of M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const char *src, const lds_char *dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"((uint32_t)(uintptr_t)dst)
               : "m0");
}
#pragma clang diagnostic pop

}  // namespace

// kAppend: the chunk's own K/V come from a.new_key / a.new_value.  Every
// workgroup of a (sequence, head) reads the chunk's keys from those rows
// (never from the cache), and after its main loop each workgroup copies the
// rows of its own queries' tokens into their cache slots, so each token is
// written once and no workgroup reads a cache row another one writes.
template <Dt T, int B, bool kAppend>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu, kWavesPerEu))) void
prefill_chunk_kernel(PrefillArgs a, int qtiles) {
  // The LDS ring: one array per slot, so the compiler can tell the slot a
  // read uses from the slots the in-flight loads write.
  __shared__ __attribute__((aligned(1024))) char k_0[kSlot], k_1[kSlot], k_2[kSlot], k_3[kSlot];
  __shared__ __attribute__((aligned(1024))) char v_0[kSlot], v_1[kSlot], v_2[kSlot], v_3[kSlot];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = wave_id_uniform();
  const int g = lane / 16;   // lane group: which 8 of a 32-wide k step this lane holds
  const int col = lane % 16;  // MFMA column: this lane's query

  // Work item: the q tiles of one (sequence, head) pair get workgroup ids that
  // are equal mod 8, so they run on the same XCD and share its L2 for K/V.
  const int group = blockIdx.x / (8 * qtiles);
  const int rem = blockIdx.x - group * 8 * qtiles;
  const int qt = qtiles - 1 - rem / 8;  // the tile with the most keys first
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

  // ---- this lane's query and its Q fragments (B operand of S^T = K Q^T:
  // step st holds dimensions 32*st + 8*g .. +7)
  const int jq = qbase + wave * kPfWaveQ + col;  // query index in the chunk
  // Valid query: inside the chunk, inside the context, and inside q / out
  // (cu_q_lens is device data, so its rows are checked against total_q).
  const bool q_ok = jq < q_len && c + jq >= 0 && c + jq < n && q0 >= 0 && q0 + jq < a.total_q;
  const int qpos = c + jq;  // its absolute position
  uint4 qf[kPfD / 32];
  {
    const char *qrow =
        reinterpret_cast<const char *>(a.q) + ((int64_t)(q_ok ? q0 + jq : 0) * a.num_heads + h) * (kPfD * 2);
#pragma unroll
    for (int st = 0; st < kPfD / 32; ++st) qf[st] = q_ok ? load16(qrow + 16 * (4 * st + g)) : make_uint4(0, 0, 0, 0);
  }

  // ---- keys this workgroup and this wave need
  const int kv_end = max(0, min(n, c + qbase + kPfQ));  // keys [0, kv_end) for the tile
  const int nkb = (kv_end + kPfKeys - 1) / kPfKeys;
  const bool any_q = __builtin_amdgcn_ballot_w64(q_ok) != 0;
  const int wave_last = c + qbase + wave * kPfWaveQ + kPfWaveQ - 1;  // last position any query of the wave sees
  const int wave_nkb = any_q ? max(0, min(nkb, (min(wave_last, n - 1) + kPfKeys) / kPfKeys)) : 0;

  const int64_t table_row = (int64_t)s * a.max_blocks;
  const uint32_t block_stride = (uint32_t)a.num_heads * B * (kPfD * 2);
  // Base of this head's rows: block e's row r of this head is at
  // e*block_stride + r*256 from here.
  const char *kbase = reinterpret_cast<const char *>(a.k_cache) + (int64_t)h * B * (kPfD * 2);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache) + (int64_t)h * B * (kPfD * 2);

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

  // Loading one 32-key block: each load instruction moves 4 rows (64 lanes x
  // 16 bytes land contiguously in LDS); wave w issues kLoads of them for K
  // and as many for V, rows 4*w + 4*kPfWaves*i .. +3.  Lane l fills position
  // l%16 of its row with chunk (l%16) ^ swz(row) of the K/V row.  Keys at or
  // past kv_end read the row of key kv_end-1 instead: their scores are
  // masked and their weights are 0, and a real (finite) V row keeps 0 * V
  // finite.  The 4 rows of one load are 4-aligned and a block holds at least
  // 4 tokens, so they share one table entry: a scalar load, fetched a step
  // before the block's loads are issued.  An entry outside the pool is
  // replaced by block 0, so every address stays inside the caches; only the
  // keys of a well-formed table matter.
  const int r0 = 4 * wave + lane / 16;  // swz(r0 + 16*i) == swz(r0)
  const uint32_t chunk_off = (uint32_t)(16 * ((lane % 16) ^ swz(r0)));
  auto entries = [&](int kb, uint32_t (&e)[kLoads]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int key0 = min(kb * kPfKeys + 4 * wave + 4 * kPfWaves * i, kv_end - 1);
      const int32_t v = load_uniform(a.block_tables, table_row + key0 / B);
      e[i] = (v >= 0 && (int64_t)v < a.num_blocks) ? (uint32_t)v : 0u;
    }
  };
  // Append: a chunk key (position >= c) is row q0 + key - c of the new rows;
  // its offsets from the cache bases, valid while that row lies in q (the
  // row index comes from device data).
  // Append: this tile's own tokens are keys tok_lo .. tok_hi-1; those at or
  // past ring_lo are still in the ring when the loop ends.
  [[maybe_unused]] const int tok_lo = max(c + qbase, 0), tok_hi = min(c + qbase + kPfQ, n);
  [[maybe_unused]] const int ring_lo = max(nkb - kPfRing, 0) * kPfKeys;
  [[maybe_unused]] const int store_lo = max(tok_lo, ring_lo);
  [[maybe_unused]] const int64_t knew = kAppend ? (int64_t)((uintptr_t)a.new_key - (uintptr_t)kbase) +
                                                      (int64_t)h * (kPfD * 2) + chunk_off : 0;
  [[maybe_unused]] const int64_t vnew = kAppend ? (int64_t)((uintptr_t)a.new_value - (uintptr_t)vbase) +
                                                      (int64_t)h * (kPfD * 2) + chunk_off : 0;
  auto load_block = [&](int kb, const uint32_t (&e)[kLoads], auto sc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int key = min(kb * kPfKeys + r0 + 4 * kPfWaves * i, kv_end - 1);
      const uint64_t blk = (uint64_t)e[i] * block_stride;
      const uint32_t off = (uint32_t)((key & (B - 1)) * kRow) + chunk_off;
      const int dst = 1024 * (wave + kPfWaves * i);
      if constexpr (kAppend) {
        const int row = q0 + key - c;
        const bool fresh = key >= c && q0 >= 0 && row < a.total_q;
        const int64_t ko = fresh ? knew + (int64_t)row * a.new_key_stride : (int64_t)(blk + off);
        const int64_t vo = fresh ? vnew + (int64_t)row * a.new_value_stride : (int64_t)(blk + off);
        load_lds16(kbase + ko, (const lds_char *)(kslot(sc) + dst));
        load_lds16(vbase + vo, (const lds_char *)(vslot(sc) + dst));
      } else {
        load_lds16(kbase + blk + off, (const lds_char *)(kslot(sc) + dst));
        load_lds16(vbase + blk + off, (const lds_char *)(vslot(sc) + dst));
      }
    }
  };

  // ---- running softmax state of this lane's query, and O^T accumulators
  // (tile dt: lane (g, n) register j is dimension 16*dt + 4*g + j of query
  // n).  l_run is this lane's part of the row sum (its 8 keys of every
  // block); the four lane groups of a query share m_run, so the parts are
  // added only at the end.
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[kPfD / 16];
#pragma unroll
  for (int dt = 0; dt < kPfD / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Lowest query position of the wave, and whether all its queries are valid:
  // key blocks entirely at or before it need no causal mask.
  const int wave_first = c + qbase + wave * kPfWaveQ;
  const bool wave_full = __builtin_amdgcn_ballot_w64(q_ok) == ~0ull;
  const float sc = a.scale_log2;  // > 0 (checked by the host)
  // log2 of the factor on the bf16 kernel's weights (see the weights below).
  constexpr float kPScale = T == Dt::BF16 ? 7.f : 0.f;

  // Per-lane LDS offsets of the MFMA operands (tile or half t adds 16 rows).
  //  K (A of S^T, tile mt, step st): row 16*mt + col, chunk 4*st + g.
  //  V^T (A of O^T, tile dt): the half i read covers keys 16*i + 4*g ..
  //  +3; lane j of each 16-lane group points at 4 elements of key 16*i +
  //  4*g + j/4, dimensions 16*dt + 4*(j%4) .. +3, and the read hands lane j
  //  element e of the lane 4*e + j/4 that pointed there: dimension 16*dt + j
  //  of keys 16*i + 4*g + e.
  uint32_t k_off[kPfD / 32];
#pragma unroll
  for (int st = 0; st < kPfD / 32; ++st) k_off[st] = (uint32_t)(col * kRow + 16 * ((4 * st + g) ^ swz(col)));
  uint32_t v_off[kPfD / 16];
  {
    const int row = 4 * g + col / 4;
#pragma unroll
    for (int dt = 0; dt < kPfD / 16; ++dt)
      v_off[dt] = (uint32_t)(row * kRow + 16 * ((2 * dt + (col % 4) / 2) ^ swz(row)) + 8 * (col % 2));
  }
  auto kread = [&](auto sc_, int mt, int st) __attribute__((always_inline)) -> uint4 {
    return load16(kslot(sc_) + k_off[st] + 16 * kRow * mt);
  };
  auto vread = [&](auto sc_, int dt) __attribute__((always_inline)) -> uint4 {
    const lds_char *vb_ = (const lds_char *)vslot(sc_);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3))) *)(vb_ + v_off[dt]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3))) *)(vb_ + v_off[dt] + 16 * kRow));
    return __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One block (index kb, in slot `ks`) for a wave that still needs it.
  auto compute = [&](int kb, auto ks) __attribute__((always_inline)) {
    // S^T: tile mt holds keys kb*32 + 16*mt + (4*g + j) in register j.
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int st = 0; st < kPfD / 32; ++st) {
      s0 = mfma<T>(kread(ks, 0, st), qf[st], s0);
      s1 = mfma<T>(kread(ks, 1, st), qf[st], s1);
    }
    float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    if (!(wave_full && kb * kPfKeys + kPfKeys - 1 <= wave_first)) {
      // x[4*mt + j] is key kb*32 + 16*mt + 4*g + j: visible iff <= qpos.
      const int lim = q_ok ? qpos - kb * kPfKeys - 4 * g : -1;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (16 * (e / 4) + e % 4 <= lim) ? x[e] : -INFINITY;
    }
    // Lazy max: the reference m_run moves only when a block exceeds it by
    // more than 8 (log2 units), so weights stay <= 2^8 and O is rarely
    // rescaled; the result is the same softmax, only the common factor
    // differs.  Each lane judges its own 8 keys of its query; only if some
    // query's max moves do the four lane groups agree on it and rescale.
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int e = 2; e < 8; ++e) mx = fmaxf(mx, x[e]);
    if (__builtin_amdgcn_ballot_w64(mx * sc > m_run + 8.f) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mblk = mx * sc;
      const bool bump = mblk > m_run + 8.f;
      const float m_new = bump ? mblk : m_run;
      const float alpha = bump ? fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new)) : 1.f;
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < kPfD / 16; ++dt) o[dt] *= alpha;
    }
    // Weights p = 2^(x*scale_log2 - m) and P^T packed as the f16 B operand
    // (element e = 4*mt + j).  For bf16 caches the weights are scaled by
    // 2^7 (at most 2^15 under the lazy max, inside f16's range), which
    // keeps small weights out of f16's subnormals; the scale cancels in O/l.
    const float m = (m_run == -INFINITY) ? 0.f : m_run - kPScale;
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(x[e], sc, -m));
      lsum += p[e];
    }
    l_run += lsum;
    uint32_t hw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hw[q] = pack_pair<false>(p[2 * q], p[2 * q + 1]);
    const uint4 pb = make_uint4(hw[0], hw[1], hw[2], hw[3]);
#pragma unroll
    for (int dt = 0; dt < kPfD / 16; ++dt) o[dt] = mfma<Dt::F16>(vread(ks, dt), pb, o[dt]);
  };

  // Wait until at most N of this wave's loads are in flight, then meet the
  // other waves.  The loads write LDS directly, so a barrier with the usual
  // memory fence would wait for all of them; this one waits only for the
  // older blocks (the empty asm statements keep the compiler from moving
  // LDS accesses across it).
  auto sync_blocks = [&](auto wait) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(decltype(wait)::value);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Loads per wave per block (K and V).
  constexpr int kL = 2 * kLoads;
  static_assert(kPfRing == 4, "the pipeline below is written for 4 slots");
  // bf16: the V rows this wave loaded for block kb (slot sc_) rewritten as
  // f16, in place.  The append kernel first stores the rows of this tile's
  // own tokens into their cache slots as loaded (bf16), for the keys still
  // in the ring at the end (the K rows follow from the ring after the loop).
  // Those stores count in vmcnt; the ring's loads complete in order, so a
  // wait for a block's loads stays exact and at most also waits for them.
  auto convert = [&](int kb, auto sc_) __attribute__((always_inline)) {
    if constexpr (T == Dt::BF16) {
      char *p = vslot(sc_) + 1024 * wave + 16 * lane;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        uint4 w = *reinterpret_cast<const uint4 *>(p + 1024 * kPfWaves * i);
        if constexpr (kAppend) {
          const int key = kb * kPfKeys + r0 + 4 * kPfWaves * i;
          if (key >= store_lo && key < tok_hi && q0 >= 0 && q0 + key - c < a.total_q) {
            const int32_t e = a.block_tables[table_row + (kb * kPfKeys + 4 * wave + 4 * kPfWaves * i) / B];
            if (e >= 0 && (int64_t)e < a.num_blocks)
              *reinterpret_cast<uint4 *>(const_cast<char *>(vbase) + (int64_t)e * block_stride +
                                         (int64_t)(key & (B - 1)) * kRow + chunk_off) = w;
          }
        }
        float f[8];
        widen8<Dt::BF16>(w, f);
        w = make_uint4(pack_pair<false>(f[0], f[1]), pack_pair<false>(f[2], f[3]), pack_pair<false>(f[4], f[5]),
                       pack_pair<false>(f[6], f[7]));
        *reinterpret_cast<uint4 *>(p + 1024 * kPfWaves * i) = w;
      }
    }
  };
  // End of step kb: block kb+1 must be in; the blocks issued after it (up
  // to two, fewer near the end) may stay in flight.  For bf16 each wave
  // already waited for its own loads of block kb+1 to convert them, so the
  // barrier only has to follow its LDS writes.
  auto end_step = [&](int kb) __attribute__((always_inline)) {
    if constexpr (T == Dt::BF16) {
      sync_blocks(WaitLgkm0{});
    } else {
      const int after = min(nkb - 1, kb + 3) - (kb + 1);
      if (after >= 2) sync_blocks(WaitVm<2 * kL>{});
      else if (after == 1) sync_blocks(WaitVm<kL>{});
      else sync_blocks(WaitVm<0>{});
    }
  };
  // Step kb: block kb is in slot kb % 4; the load of block kb+3 goes into
  // the slot block kb-1 used, with the table entries fetched a step before.
  // bf16 first converts this wave's part of block kb+1 (slot ns), waiting
  // for its loads with block kb+2's still in flight.
  uint32_t ent[kLoads];  // table entries of the next block to load
  auto step = [&](int kb, auto ks, auto ds, auto ns) __attribute__((always_inline)) {
    if constexpr (T == Dt::BF16) {
      if (kb + 1 < nkb) {
        if (kb + 2 < nkb) __builtin_amdgcn_s_waitcnt(WaitVm<kL>::value);
        else __builtin_amdgcn_s_waitcnt(WaitVm<0>::value);
        asm volatile("" ::: "memory");
        convert(kb + 1, ns);
      }
    }
    if (kb + 3 < nkb) {
      load_block(kb + 3, ent, ds);
      if (kb + 4 < nkb) entries(kb + 4, ent);
    }
    if (kb < wave_nkb) compute(kb, ks);
    end_step(kb);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if (nkb > 0) {
    // The Q fragments are in registers before any block load is issued (so
    // no later wait for them has to count the block loads).
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::value);
    entries(0, ent);
    load_block(0, ent, S0{});
    if (nkb > 1) {
      entries(1, ent);
      load_block(1, ent, S1{});
    }
    if (nkb > 2) {
      entries(2, ent);
      load_block(2, ent, S2{});
    }
    if (nkb > 3) entries(3, ent);
    // Block 0 in (converted, for bf16); blocks 1 and 2 may stay in flight.
    if constexpr (T == Dt::BF16) {
      if (nkb > 2) __builtin_amdgcn_s_waitcnt(WaitVm<2 * kL>::value);
      else if (nkb == 2) __builtin_amdgcn_s_waitcnt(WaitVm<kL>::value);
      else __builtin_amdgcn_s_waitcnt(WaitVm<0>::value);
      asm volatile("" ::: "memory");
      convert(0, S0{});
      sync_blocks(WaitLgkm0{});
    } else {
      if (nkb > 2) sync_blocks(WaitVm<2 * kL>{});
      else if (nkb == 2) sync_blocks(WaitVm<kL>{});
      else sync_blocks(WaitVm<0>{});
    }
    for (int kb = 0;; kb += 4) {
      step(kb, S0{}, S3{}, S1{});
      if (kb + 1 >= nkb) break;
      step(kb + 1, S1{}, S0{}, S2{});
      if (kb + 2 >= nkb) break;
      step(kb + 2, S2{}, S1{}, S3{});
      if (kb + 3 >= nkb) break;
      step(kb + 3, S3{}, S2{}, S0{});
      if (kb + 4 >= nkb) break;
    }
  }

  char *orow = reinterpret_cast<char *>(a.out) + ((int64_t)(q_ok ? q0 + jq : 0) * a.num_heads + h) * (kPfD * 2);
  bool bad = false;
#pragma unroll
  for (int dt = 0; dt < kPfD / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) bad |= !__builtin_isfinite(o[dt][j]);
  if (__builtin_amdgcn_ballot_w64(bad) == 0) {
    // ---- write this lane's query: dimensions 16*dt + 4*g .. +3.
    float l = l_run + __shfl_xor(l_run, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (q_ok) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < kPfD / 16; ++dt) {
        const uint2 w = make_uint2(pack_pair<T == Dt::BF16>(o[dt][0] * inv, o[dt][1] * inv),
                                   pack_pair<T == Dt::BF16>(o[dt][2] * inv, o[dt][3] * inv));
        *reinterpret_cast<uint2 *>(orow + (16 * dt + 4 * g) * 2) = w;
      }
    }
  } else {
    // ---- exact recomputation of the wave's queries, key by key in fp32
    // with an online softmax, K/V read straight from the cache (the chunk's
    // keys from the new rows in the append kernel).  Lane (g, n) keeps
    // dimensions 32*st + 8*g .. +7 of query n, the layout of its Q
    // fragments; the four lane groups add their parts of each score.
    float qv[kPfD / 4], acc[kPfD / 4];
#pragma unroll
    for (int st = 0; st < kPfD / 32; ++st) {
      float f[8];
      widen8<T>(qf[st], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qv[8 * st + i] = f[i];
        acc[8 * st + i] = 0.f;
      }
    }
    float me = -INFINITY, le = 0.f;
    const int last = q_ok ? qpos : -1;
    const int wave_end = min(wave_last, n - 1);
    for (int key = 0; key <= wave_end; ++key) {
      const char *krow, *vrow;
      const int row = q0 + key - c;
      if (kAppend && key >= c && q0 >= 0 && row < a.total_q) {
        krow = reinterpret_cast<const char *>(a.new_key) + (int64_t)row * a.new_key_stride + (int64_t)h * kRow;
        vrow = reinterpret_cast<const char *>(a.new_value) + (int64_t)row * a.new_value_stride + (int64_t)h * kRow;
      } else {
        const int32_t v = load_uniform(a.block_tables, table_row + key / B);
        const uint32_t e = (v >= 0 && (int64_t)v < a.num_blocks) ? (uint32_t)v : 0u;
        const uint64_t off = (uint64_t)e * block_stride + (uint32_t)(key & (B - 1)) * kRow;
        krow = kbase + off;
        vrow = vbase + off;
      }
      float d = 0.f;
#pragma unroll
      for (int st = 0; st < kPfD / 32; ++st) {
        float f[8];
        widen8<T>(load16(krow + 16 * (4 * st + g)), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(qv[8 * st + i], f[i], d);
      }
      d += __shfl_xor(d, 16, kWave);
      d += __shfl_xor(d, 32, kWave);
      if (key <= last) {
        const float s = d * sc;
        const float mn = fmaxf(me, s);
        const float al = fast_exp2(me - mn);
        const float pw = fast_exp2(s - mn);
        le = le * al + pw;
#pragma unroll
        for (int st = 0; st < kPfD / 32; ++st) {
          float f[8];
          widen8<T>(load16(vrow + 16 * (4 * st + g)), f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[8 * st + i] = fmaf(acc[8 * st + i], al, pw * f[i]);
        }
        me = mn;
      }
    }
    if (q_ok) {
      const float inv = le > 0.f ? 1.f / le : 0.f;
#pragma unroll
      for (int st = 0; st < kPfD / 32; ++st) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack_pair<T == Dt::BF16>(acc[8 * st + 2 * i] * inv, acc[8 * st + 2 * i + 1] * inv);
        *reinterpret_cast<uint4 *>(orow + 16 * (4 * st + g)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // ---- append: write the K/V rows of this tile's tokens (chunk indices
  // qbase .. qbase+kPfQ-1, keys tok_lo .. tok_hi-1) into their cache slots.
  // The ring still holds the last four blocks, loaded from the new rows:
  // each lane stores the 16 bytes it loaded there for every such key (for
  // bf16 only the K rows: its V rows were stored before they were
  // converted).  Keys in an older block (at most kPfKeys-1 of them, when the
  // tile does not start on a block) are copied from the new rows.  Tokens
  // outside the context or q, or whose table entry lies outside the pool,
  // are skipped.
  if constexpr (kAppend) {
    auto store_slot = [&](auto sc) __attribute__((always_inline)) {
      constexpr int j = decltype(sc)::value;
      // The block in slot j: the last one below nkb that is j mod 4.
      const int b = nkb - 1 - (((nkb - 1 - j) % kPfRing) + kPfRing) % kPfRing;
      const int key = b * kPfKeys + r0;
      const int key0 = b * kPfKeys + 4 * wave;  // the wave's 4 rows share one table entry
      if (b >= 0 && key >= tok_lo && key < tok_hi && key < kv_end && q0 >= 0 && q0 + key - c < a.total_q) {
        const int32_t e = a.block_tables[table_row + key0 / B];
        if (e >= 0 && (int64_t)e < a.num_blocks) {
          const int64_t d = (int64_t)e * block_stride + (int64_t)(key & (B - 1)) * kRow + chunk_off;
          const int l = 1024 * wave + 16 * lane;
          *reinterpret_cast<uint4 *>(const_cast<char *>(kbase) + d) = *reinterpret_cast<const uint4 *>(kslot(sc) + l);
          if constexpr (T != Dt::BF16)
            *reinterpret_cast<uint4 *>(const_cast<char *>(vbase) + d) = *reinterpret_cast<const uint4 *>(vslot(sc) + l);
        }
      }
    };
    // The ring's loads are ordered before these reads by the waits above;
    // wait for them explicitly too, so that this copy does not depend on
    // how the pipeline ends.
    __builtin_amdgcn_s_waitcnt(WaitVm<0>::value);
    asm volatile("" ::: "memory");
    store_slot(S0{});
    store_slot(S1{});
    store_slot(S2{});
    store_slot(S3{});
    if (tok_lo < min(tok_hi, ring_lo)) {  // workgroup-uniform
      constexpr int kCopyRows = kPfQ * 32 / kPfThreads;
      const int part = tid % 32, is_v = part / 16, ch = part % 16;
      uint4 rowv[kCopyRows];
      int64_t dsto[kCopyRows];
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u) {
        const int j = qbase + tid / 32 + (kPfThreads / 32) * u;  // chunk index of the token
        const int p = c + j;
        const int row = q0 + j;
        const bool live = j < q_len && p >= 0 && p < n && p < ring_lo && q0 >= 0 && row < a.total_q;
        int32_t e = -1;
        if (live) e = a.block_tables[table_row + p / B];
        dsto[u] = (e >= 0 && (int64_t)e < a.num_blocks)
                      ? (int64_t)e * block_stride + (int64_t)(p % B) * (kPfD * 2) + ch * 16
                      : -1;
        rowv[u] = make_uint4(0, 0, 0, 0);
        if (dsto[u] >= 0)
          rowv[u] = load16(reinterpret_cast<const char *>(is_v ? a.new_value : a.new_key) +
                           (int64_t)row * (is_v ? a.new_value_stride : a.new_key_stride) + (int64_t)h * (kPfD * 2) +
                           ch * 16);
      }
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u)
        if (dsto[u] >= 0) *reinterpret_cast<uint4 *>(const_cast<char *>(is_v ? vbase : kbase) + dsto[u]) = rowv[u];
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
  if (a.new_key)
    hipLaunchKernelGGL((prefill_chunk_kernel<T, B, true>), dim3((unsigned)grid), dim3(kPfThreads), 0, st, a, qtiles);
  else
    hipLaunchKernelGGL((prefill_chunk_kernel<T, B, false>), dim3((unsigned)grid), dim3(kPfThreads), 0, st, a, qtiles);
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

bool prefill_append_supported(int dtype, int head_dim, int block_size) {
  return prefill_mfma_supported(dtype, head_dim, block_size);
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
  // fp32, or head_dim 64: the vector-ALU kernel (which has no fused write).
  if (!a.new_key && prefill_general_supported(dtype, head_dim, block_size))
    return launch_prefill_general(a, dtype, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
