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

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 3
#endif
// 1: stream K/V with non-temporal loads (they are read exactly once).
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif

namespace pa {

constexpr int kDepth = PA_DECODE_DEPTH;
constexpr int kPlanThreads = 1024;
// Largest batch whose worker waves plan for themselves (16 chunks of 64).
constexpr int kSelfPlanSeqs = 1024;

__device__ __forceinline__ uint4 load16(const char *p) {
#if PA_DECODE_NT
  return load_nt16(p);
#else
  return *reinterpret_cast<const uint4 *>(p);
#endif
}

__device__ __forceinline__ int clip_ctx(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }
__device__ __forceinline__ int tiles_of(int n) { return (n + kDecodeTile - 1) / kDecodeTile; }

// First position the pass covers for a sequence of n (clipped) tokens: 0,
// or with a shared prefix its start, rounded down to a whole tile and
// clamped to [0, n].
__device__ __forceinline__ int start_of(int raw_start, int n) {
  const int st = raw_start < 0 ? 0 : (raw_start & ~(kDecodeTile - 1));
  return st < n ? st : n;
}
// Tiles of sequence s (n clipped tokens) the pass covers.
__device__ __forceinline__ int pass_tiles(const DecodeArgs &a, int s, int n) {
  return a.starts ? tiles_of(n - start_of(a.starts[s], n)) : tiles_of(n);
}
// Whether the pass leaves partials (not the output) for sequence s.
__device__ __forceinline__ bool to_partial(const DecodeArgs &a, int start) { return a.suffix_out && start > 0; }

// The result of a sequence with no tile in the pass: a zero output row, or
// with a shared prefix an empty partial (zero sum, log2-denominator -inf)
// for every head.  Written by `count` cooperating lanes from `first`.
__device__ __forceinline__ void empty_rows(const DecodeArgs &a, int s, int first, int count) {
  const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
  if (a.starts && to_partial(a, start_of(a.starts[s], n))) {
    float *row = a.suffix_out + (int64_t)s * a.suffix_row;
    const int per_head = a.suffix_row / a.num_heads;  // head_dim + 2
    for (int i = first; i < a.suffix_row; i += count) row[i] = (i % per_head == per_head - 2) ? -INFINITY : 0.f;
  } else {
    uint32_t *row = reinterpret_cast<uint32_t *>(a.out) + (int64_t)s * a.out_row_words;
    for (int i = first; i < a.out_row_words; i += count) row[i] = 0u;  // +0.0 in every dtype
  }
}

// Range [g0, g1) of global tiles owned by worker wave w of G.
__device__ __forceinline__ uint32_t range_begin(uint32_t w, uint32_t total, uint32_t G) {
  return (uint32_t)(((uint64_t)w * total) / G);
}

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

// ----------------------------------------------------------------------- plan

// Plan for batches of more than kSelfPlanSeqs sequences (smaller batches are
// planned by the worker waves themselves, see self_plan).  One workgroup.
// plan[0] = total tiles T, plan[1] = G = min(launched workers, T), and for
// every worker w < G the (s | h << 16, t) of its first tile at
// plan[kPlanHeader + 2w]; zeroes the outputs of empty sequences.
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
        a.plan[kPlanHeader + 2 * w] = (uint32_t)s | ((local / ts) << 16);
        a.plan[kPlanHeader + 2 * w + 1] = local % ts;
      }
    } else {
      empty_rows(a, s, 0, 1);
    }
    c = c_next;
  }
}

// ------------------------------------------------------------ partition pass

// Position of a cursor in the tile stream.  All fields are wave-uniform.
struct Cursor {
  int s, h, t;     // sequence, head, tile within the pair
  int n, nt;       // context length and tiles of sequence s
  int st;          // first position of sequence s in the pass (0 without a shared prefix)
  uint32_t g;      // global tile index
};

// Length, start and tiles of the sequence under the cursor.
__device__ __forceinline__ void cursor_load(Cursor &c, const DecodeArgs &a) {
  c.n = clip_ctx(load_uniform(a.context_lens, c.s), a.ctx_cap);
  c.st = a.starts ? start_of(load_uniform(a.starts, c.s), c.n) : 0;
  c.nt = tiles_of(c.n - c.st);
}

// Step to the next tile; crosses to the next head, then to the next
// non-empty sequence.  Only called while g + 1 < end, so a next tile exists.
__device__ __forceinline__ void cursor_next(Cursor &c, const DecodeArgs &a) {
  ++c.g;
  if (++c.t < c.nt) return;
  c.t = 0;
  if (++c.h < a.num_heads) return;
  c.h = 0;
  do {
    ++c.s;
    cursor_load(c, a);
  } while (c.nt == 0);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

// Batches of at most kSelfPlanSeqs sequences: every worker wave reads all
// context lengths and finds the (s, h, t) of its first tile itself -- no plan
// launch.  Lane l owns the k = ceil(S / 64) consecutive sequences from l*k, so
// one inclusive scan over the lanes' tile counts places every lane's run in
// the stream; the lane whose run holds tile g0 is found with a ballot and its
// k sequences are walked on the scalar unit.  Wave 0 also publishes T and G
// in plan[0..1]; every worker stores its start for the fix-up, and zeroes
// the outputs of the empty sequences s with s % G == w.  Returns false if
// the wave has no work.
__device__ __forceinline__ bool self_plan(const DecodeArgs &a, uint32_t w, uint32_t &total, uint32_t &G,
                                          int &s0, int &h0, int &t0) {
  constexpr int kMaxPerLane = kSelfPlanSeqs / kWave;
  const int lane = threadIdx.x % kWave;
  const uint32_t H = (uint32_t)a.num_heads;
  const int S = a.num_seqs;
  const int k = (S + kWave - 1) / kWave;  // wave-uniform, 1 .. kMaxPerLane
  const int first = lane * k;
  int32_t raw[kMaxPerLane], raw_st[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < k) raw[i] = a.context_lens[min(first + i, S - 1)];
    if (i < k) raw_st[i] = a.starts ? a.starts[min(first + i, S - 1)] : 0;
  }
  uint32_t tiles[kMaxPerLane];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < k && first + i < S) {
      const int n = clip_ctx(raw[i], a.ctx_cap);
      tiles[i] = (uint32_t)tiles_of(n - start_of(raw_st[i], n));
    } else {
      tiles[i] = 0u;
    }
    mine += tiles[i] * H;
  }
  const uint32_t incl = wave_inclusive_scan(mine);
  total = __builtin_amdgcn_readlane(incl, kWave - 1);
  G = total < (uint32_t)a.workers ? total : (uint32_t)a.workers;
  if (w == 0 && lane == 0) {
    a.plan[0] = total;
    a.plan[1] = G;
  }
  // Zero the rows of empty sequences, each row by one whole wave.
  const uint32_t zero_waves = G > 0 ? G : 1u;
  if (w < zero_waves) {
    for (int i = 0; i < k; ++i) {
      const int s = first + i;
      uint64_t todo = __builtin_amdgcn_ballot_w64(s < S && tiles[i] == 0 && (uint32_t)s % zero_waves == w);
      while (todo) {
        const int l = __builtin_ctzll(todo);
        todo &= todo - 1;
        empty_rows(a, l * k + i, lane, kWave);
      }
    }
  }
  if (w >= G) return false;
  const uint32_t g0 = range_begin(w, total, G);
  const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > g0);
  const int l = __builtin_ctzll(hit);  // first lane whose run passes g0 (exists: g0 < total)
  uint32_t start = __builtin_amdgcn_readlane(incl - mine, l);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const uint32_t ts = __builtin_amdgcn_readlane(tiles[i], l);
    if (i < k && g0 < start + ts * H) {
      const uint32_t local = g0 - start;
      s0 = l * k + i;
      h0 = (int)(local / ts);
      t0 = (int)(local % ts);
      if (lane == 0) {
        a.plan[kPlanHeader + 2 * w] = (uint32_t)s0 | ((uint32_t)h0 << 16);
        a.plan[kPlanHeader + 2 * w + 1] = (uint32_t)t0;
      }
      return true;
    }
    start += ts * H;
  }
  return false;  // not reached: lane l's run holds g0
}

// First worker whose range holds tiles of a pair starting at pair_start: the
// last w with range_begin(w) <= pair_start.
__device__ __forceinline__ uint32_t first_worker(uint32_t pair_start, uint32_t total, uint32_t G) {
  return (uint32_t)((((uint64_t)pair_start + 1) * G + total - 1) / total) - 1;
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
  const int n = clip_ctx(a.context_lens[s], a.ctx_cap);
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
  if (a.starts && to_partial(a, start_of(a.starts[s], n)))
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

// kAppend: each sequence's newest token (position n - 1) is read from
// a.new_key / a.new_value instead of the cache.  The pass only reads; the
// rows are stored into the cache by the reduce pass, after every read of
// this launch.
template <Dt T, int D, int B, bool kAppend>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_partition_kernel(DecodeArgs a) {
  using R = RowShape<T, D, kDecodeTile>;
  const int lane = threadIdx.x % kWave;
  const uint32_t w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  uint32_t G, total;
  Cursor ic;  // issue cursor
  if (a.num_seqs <= kSelfPlanSeqs) {
    if (!self_plan(a, w, total, G, ic.s, ic.h, ic.t)) return;
  } else {
    G = load_uniform(a.plan, 1);
    if (w >= G) return;
    total = load_uniform(a.plan, 0);
    const uint32_t sh = load_uniform(a.plan, kPlanHeader + 2 * w);
    ic.s = (int)(sh & 0xffffu);
    ic.h = (int)(sh >> 16);
    ic.t = (int)load_uniform(a.plan, kPlanHeader + 2 * w + 1);
  }
  const uint32_t g0 = range_begin(w, total, G), g1 = range_begin(w + 1, total, G);

  const int grp = lane / R::kLPT;  // token slot within one wave load
  const int col = lane % R::kLPT;  // 16-byte column within the token row
  const char *kbase = reinterpret_cast<const char *>(a.k_cache);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache);
  const int64_t block_stride = (int64_t)a.num_heads * B * R::kRowBytes;

  cursor_load(ic, a);
  ic.g = g0;
  Cursor cc = ic;  // consume cursor

  // Table entry of logical block `blk` of sequence s; -1 when outside the pool.
  auto entry = [&](int s, int blk) -> int32_t {
    const int32_t e = load_uniform(a.block_tables, (int64_t)s * a.max_blocks + blk);
    return (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  };

  // Issue the loads of one tile into a slot: q of its pair, then 4 K and 4 V
  // fragments (for fp16/bf16 D=128).  Every call issues the same loads,
  // whether or not `live` (the issue cursor inside the range) and whatever
  // the mask, so the compiler can count outstanding loads exactly and wait
  // only for the slot being consumed.  Masked and dead loads read row 0 of
  // block 0 -- always inside the pool -- and are discarded on consumption.
  auto issue = [&](uint4 *kf, uint4 *vf, uint4 &qf, uint32_t &okm, bool live) {
    const int s = live ? ic.s : 0, h = live ? ic.h : 0;
    const char *qp = reinterpret_cast<const char *>(a.q) + ((int64_t)s * a.num_heads + h) * R::kRowBytes;
    qf = *reinterpret_cast<const uint4 *>(qp + col * 16);
    const int base = ic.st + ic.t * kDecodeTile;
    const int64_t head_off = (int64_t)ic.h * B * R::kRowBytes + col * 16;
    // A table entry is read only for a block whose first token is < n, so the
    // read stays inside the sequence's row.  With B >= 16 one entry covers
    // the whole tile (base < n always holds for a live tile).
    int32_t tile_phys = -1;
    if constexpr (B >= kDecodeTile) tile_phys = live ? entry(ic.s, base / B) : -1;
    // Append: the last tile of a sequence holds position n - 1.
    [[maybe_unused]] const bool tail = kAppend && live && base + kDecodeTile >= ic.n;
    okm = 0;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const int pos = base + i * R::kGroups + grp;
      const int pos0 = base + i * R::kGroups;  // first token of this load
      int32_t phys;
      if constexpr (B >= kDecodeTile) {
        phys = tile_phys;
      } else if constexpr (B >= R::kGroups) {
        phys = (live && pos0 < ic.n) ? entry(ic.s, pos0 / B) : -1;  // one block for the whole load
      } else {
        static_assert(R::kGroups == 2 * B, "a load spans at most two blocks");
        const int b0 = pos0 / B;
        const int32_t e0 = (live && pos0 < ic.n) ? entry(ic.s, b0) : -1;
        const int32_t e1 = (live && (b0 + 1) * B < ic.n) ? entry(ic.s, b0 + 1) : -1;
        phys = (grp >= B) ? e1 : e0;
      }
      const bool ok = live && (pos < ic.n) && (phys >= 0);
      const int64_t off =
          ok ? (int64_t)phys * block_stride + head_off + (int64_t)(pos % B) * R::kRowBytes : (int64_t)col * 16;
      if constexpr (kAppend) {
        const char *kp = kbase + off, *vp = vbase + off;
        if (tail && ok && pos == ic.n - 1) {
          kp = reinterpret_cast<const char *>(a.new_key) + (int64_t)s * a.new_key_stride + h * R::kRowBytes + col * 16;
          vp = reinterpret_cast<const char *>(a.new_value) + (int64_t)s * a.new_value_stride + h * R::kRowBytes +
               col * 16;
        }
        kf[i] = load16(kp);
        vf[i] = load16(vp);
      } else {
        kf[i] = load16(kbase + off);
        vf[i] = load16(vbase + off);
      }
      okm |= ok ? (1u << i) : 0u;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  float acc[R::kFE];
  uint4 qcur = make_uint4(0, 0, 0, 0);

  // Finish the pair under the consume cursor: merge the lane groups, then
  // write the output (pair inside this range) or a fragment.
  auto finish = [&]() {
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
    const uint32_t pair_start = cc.g - (uint32_t)cc.t;
    const uint32_t pair_end = pair_start + (uint32_t)cc.nt;
    if (pair_start >= g0 && pair_end <= g1) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      if (to_partial(a, cc.st)) {
        float *f = a.suffix_out + (int64_t)cc.s * a.suffix_row + (int64_t)cc.h * (D + 2);
        if (lane < R::kLPT) {
#pragma unroll
          for (int e = 0; e < R::kFE; ++e) f[col * R::kFE + e] = acc[e] * inv;
        }
        if (lane == 0) {
          f[D] = l_run > 0.f ? m_run + __builtin_amdgcn_logf(l_run) : -INFINITY;
          f[D + 1] = 0.f;
        }
      } else if (lane < R::kLPT) {
        float o[R::kFE];
#pragma unroll
        for (int e = 0; e < R::kFE; ++e) o[e] = acc[e] * inv;
        char *op = reinterpret_cast<char *>(a.out) + ((int64_t)cc.s * a.num_heads + cc.h) * R::kRowBytes;
        *reinterpret_cast<uint4 *>(op + col * 16) = frag_pack<T>(o);
      }
    } else {
      const int slot = pair_start < g0 ? 0 : 1;
      float *f = a.frags + ((int64_t)w * 2 + slot) * (D + 2);
      if (lane < R::kLPT) {
#pragma unroll
        for (int e = 0; e < R::kFE; ++e) f[col * R::kFE + e] = acc[e];
      }
      if (lane == 0) {
        f[D] = m_run;
        f[D + 1] = l_run;
      }
    }
  };

  // Fold one tile into the running state of the pair under the consume cursor.
  constexpr uint32_t kAll = (1u << R::kNI) - 1u;
  auto consume = [&](const uint4 *kf, uint4 *vf, const uint4 &qslot, uint32_t okm) {
    if (cc.t == 0 || cc.g == g0) {
      qcur = qslot;
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) acc[e] = 0.f;
    }
    // Masked fragments hold whatever the dummy row holds: zero their values
    // (their weights are 0, but 0 * NaN is not).  Rare: partial tiles only.
    if (__builtin_amdgcn_ballot_w64(okm != kAll) != 0) {
#pragma unroll
      for (int i = 0; i < R::kNI; ++i)
        if (!((okm >> i) & 1u)) vf[i] = make_uint4(0, 0, 0, 0);
    }
    float sc[R::kNI];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const float d = group_sum<R::kLPT>(frag_dot<T>(qcur, kf[i]));
      sc[i] = (okm >> i) & 1u ? d * a.scale_log2 : -INFINITY;
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
      frag_axpy<T>(acc, p, vf[i]);
    }
    m_run = m_new;
    if (cc.t + 1 == cc.nt || cc.g + 1 == g1) finish();
  };

  // Software pipeline over the wave's L tiles with kDepth slots.  Every loop
  // step consumes slot d (if a tile is left) and refills it with the tile
  // kDepth ahead, or with dummy loads past the end.
  const uint32_t L = g1 - g0;
  uint32_t issued = 0;
  uint4 kb[kDepth][R::kNI], vb[kDepth][R::kNI], qb[kDepth];
  uint32_t okb[kDepth];
  auto refill = [&](int d) {
    const bool live = issued < L;
    issue(kb[d], vb[d], qb[d], okb[d], live);
    if (live) {
      ++issued;
      if (issued < L) cursor_next(ic, a);
    }
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) refill(d);
  for (uint32_t it = 0; it < L; it += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (it + d < L) {
        consume(kb[d], vb[d], qb[d], okb[d]);
        if (it + d + 1 < L) cursor_next(cc, a);
      }
      refill(d);
    }
  }

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
  const uint32_t G = a.plan[1];
  const uint32_t w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  if (w >= G) return;
  const uint32_t total = a.plan[0];
  const uint32_t g0 = range_begin(w, total, G), g1 = range_begin(w + 1, total, G);
  const uint32_t sh = a.plan[kPlanHeader + 2 * w];
  const int s = (int)(sh & 0xffffu), h = (int)(sh >> 16);
  const uint32_t t = a.plan[kPlanHeader + 2 * w + 1];
  if (t == 0) return;  // the pair starts at g0: not cut at the front of this range
  const uint32_t nt = (uint32_t)pass_tiles(a, s, clip_ctx(a.context_lens[s], a.ctx_cap));
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

template <Dt T, int D, int B>
static hipError_t launch_part(const DecodeArgs &a, hipStream_t st) {
  if (a.num_seqs > kSelfPlanSeqs) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned groups = (unsigned)((a.workers + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup);
  if (a.new_key)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, B, true>), dim3(groups), dim3(kDecodeWavesPerGroup * kWave), 0,
                       st, a);
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
