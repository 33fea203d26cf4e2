// The stream-K walk of the decode partition pass, as a device function:
// used by the plain partition kernel (pa_decode.hip) and by the
// shared-prefix pass, which runs it beside the prefix work (pa_shared.hip).
//
// A worker wave w of G takes the tiles [floor(w*T/G), floor((w+1)*T/G)) of
// the stream of every (sequence, head, 16-token tile) and walks them with
// kDepth tiles of loads in flight; see pa_decode.hip for the method.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 3
#endif
// 1: by default, stream K/V with non-temporal loads (each is read once).
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif

namespace pa {

constexpr int kDepth = PA_DECODE_DEPTH;
constexpr bool kStreamLoads = PA_DECODE_NT != 0;
// Largest batch whose worker waves plan for themselves (16 chunks of 64).
constexpr int kSelfPlanSeqs = 1024;

// A 16-byte K/V load: non-temporal when every block is read once
// (kStream), ordinary when the batch's sequences share blocks, so that the
// caches can serve the repeated reads.
template <bool kStream>
__device__ __forceinline__ uint4 load_kv16(const char *p) {
  if constexpr (kStream) return load_nt16(p);
  else return *reinterpret_cast<const uint4 *>(p);
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
// in plan[0..1]; every worker stores its start (and the tiles of the pair
// there) for the fix-up, and zeroes
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
        a.plan[kPlanHeader + kPlanWords * w] = (uint32_t)s0 | ((uint32_t)h0 << 16);
        a.plan[kPlanHeader + kPlanWords * w + 1] = (uint32_t)t0;
        a.plan[kPlanHeader + kPlanWords * w + 2] = ts;
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

// One worker wave's share of the partition pass.  kAppend: each sequence's
// newest token (position n - 1) is read from a.new_key / a.new_value instead
// of the cache.  The pass only reads; the rows are stored into the cache by
// the reduce pass, after every read of this launch.  kStream: the K/V loads
// are non-temporal (see load_kv16).
template <Dt T, int D, int B, bool kAppend, int kDepthT, bool kStream = kStreamLoads>
__device__ __forceinline__ void partition_worker(const DecodeArgs &a, uint32_t w) {
  using R = RowShape<T, D, kDecodeTile>;
  const int lane = threadIdx.x % kWave;
  uint32_t G, total;
  Cursor ic;  // issue cursor
  if (a.num_seqs <= kSelfPlanSeqs) {
    if (!self_plan(a, w, total, G, ic.s, ic.h, ic.t)) return;
  } else {
    G = load_uniform(a.plan, 1);
    if (w >= G) return;
    total = load_uniform(a.plan, 0);
    const uint32_t sh = load_uniform(a.plan, kPlanHeader + kPlanWords * w);
    ic.s = (int)(sh & 0xffffu);
    ic.h = (int)(sh >> 16);
    ic.t = (int)load_uniform(a.plan, kPlanHeader + kPlanWords * w + 1);
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
        kf[i] = load_kv16<kStream>(kp);
        vf[i] = load_kv16<kStream>(vp);
      } else {
        kf[i] = load_kv16<kStream>(kbase + off);
        vf[i] = load_kv16<kStream>(vbase + off);
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

  // Software pipeline over the wave's L tiles with kDepthT slots.  Every loop
  // step consumes slot d (if a tile is left) and refills it with the tile
  // kDepthT ahead, or with dummy loads past the end.
  const uint32_t L = g1 - g0;
  uint32_t issued = 0;
  uint4 kb[kDepthT][R::kNI], vb[kDepthT][R::kNI], qb[kDepthT];
  uint32_t okb[kDepthT];
  auto refill = [&](int d) {
    const bool live = issued < L;
    issue(kb[d], vb[d], qb[d], okb[d], live);
    if (live) {
      ++issued;
      if (issued < L) cursor_next(ic, a);
    }
  };
#pragma unroll
  for (int d = 0; d < kDepthT; ++d) refill(d);
  for (uint32_t it = 0; it < L; it += kDepthT) {
#pragma unroll
    for (int d = 0; d < kDepthT; ++d) {
      if (it + d < L) {
        consume(kb[d], vb[d], qb[d], okb[d]);
        if (it + d + 1 < L) cursor_next(cc, a);
      }
      refill(d);
    }
  }
}

}  // namespace pa
