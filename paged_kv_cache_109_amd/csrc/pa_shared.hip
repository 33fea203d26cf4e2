// Decode for groups of sequences that share a prompt (parallel sampling):
// the shared blocks are read from HBM once per group instead of once per
// sample.
//
// Background.  Samples forked from one prompt point their block tables at
// the same physical blocks for the prompt (paper notes "PagedAttention:
// Efficient Memory Management for Large Language Model Serving", section
// 3.4.1; "KV 캐시 관리와 PagedAttention", section on sharing the common KV of
// several responses), but each sample's query still attends over all of
// them, so a plain decode reads each shared block once per sample.  The
// softmax splits by position range (the same fact the split-KV pass rests
// on), so a group's attention is computed as
//   - the shared prefix [0, P): each K/V tile is loaded once and folded into
//     the running state of every member's query;
//   - each member's own positions [P, n): the stream-K decode walk with a
//     per-sequence start, leaving a normalised fp32 partial and its log2
//     softmax denominator (pa_stream.h);
//   - a merge of the two per (sequence, head) into the output
//     (decode_combine_kernel, below).
//
// One launch does the first two (decode_shared_pass_kernel).  Its worker
// waves split both streams evenly: worker w of G takes the w-th G-th of the
// prefix tiles, ordered (group, head, tile), and then the w-th G-th of the
// own positions' tiles (the partition walk), so every worker gets the same
// mix and no launch boundary separates the two.  A (group, head) pair of the
// prefix cut by range boundaries leaves one piece per worker; the combine
// merges the pieces in order.  Ranges of the prefix stream are at least
// kPrefixMinTiles long, which bounds the pieces of a pair.
//
// Mapping.  As in the decode pass, a K/V row of one token and head is
// covered by LPT lanes with one 16-byte load each; one wave load covers
// 64/LPT tokens, a 16-token tile takes kNI loads for K and kNI for V.  The
// prefix tiles are always full (P is a multiple of the tile, within every
// member's context), so no masking is needed there.  Members' states live
// in registers (up to kSharedMaxMembers); the lane groups of a wave hold
// different tokens and are merged at the end of each piece.

#include "pa_stream.h"

namespace pa {

#ifndef PA_SHARED_OWN_DEPTH
#define PA_SHARED_OWN_DEPTH 4
#endif
#ifndef PA_SHARED_PREFIX_DEPTH
#define PA_SHARED_PREFIX_DEPTH 2
#endif
constexpr int kSharedOwnDepth = PA_SHARED_OWN_DEPTH;        // own tiles in flight per wave
constexpr int kSharedPrefixDepth = PA_SHARED_PREFIX_DEPTH;  // prefix tiles in flight per wave

// Tiles (per head) of group g's shared prefix: the prefix clamped to the
// first member's context and to the call's bound, in whole tiles; 0 for a
// group without a valid first member.  Lane-varying g.
__device__ __forceinline__ uint32_t group_tiles(const SharedArgs &a, int g) {
  const int lead = a.members[(int64_t)g * kSharedMaxMembers];
  if (lead < 0 || lead >= a.num_seqs) return 0u;
  const int n0 = clip_ctx(a.context_lens[lead], a.ctx_cap);
  const int p = a.prefix[g];
  const int t = (p < 0 ? 0 : (p > n0 ? n0 : p)) / kDecodeTile;
  return (uint32_t)(t < a.max_prefix_tiles ? t : a.max_prefix_tiles);
}

// The same for a wave-uniform g (scalar loads).
__device__ __forceinline__ uint32_t group_tiles_uniform(const SharedArgs &a, int g) {
  const int lead = load_uniform(a.members, (int64_t)g * kSharedMaxMembers);
  if (lead < 0 || lead >= a.num_seqs) return 0u;
  const int n0 = clip_ctx(load_uniform(a.context_lens, lead), a.ctx_cap);
  const int p = load_uniform(a.prefix, g);
  const int t = (p < 0 ? 0 : (p > n0 ? n0 : p)) / kDecodeTile;
  return (uint32_t)(t < a.max_prefix_tiles ? t : a.max_prefix_tiles);
}

// Fold tiles [t0, t1) of group g's prefix, head h, into the state of every
// member's query and store each member's (value sum, max, sum) as piece c of
// the pair.
template <Dt T, int D, int B, int kDepthP>
__device__ __forceinline__ void prefix_piece(const SharedArgs &a, int g, int h, int t0, int t1, uint32_t c) {
  using R = RowShape<T, D, kDecodeTile>;
  constexpr int kM = kSharedMaxMembers;
  static_assert(B % kDecodeTile == 0, "a prefix tile must lie in one block");
  const int lane = threadIdx.x % kWave;
  const int H = a.num_heads;

  // Members: a leading run of valid sequence ids.
  int sm[kM];
  int nm = 0;
#pragma unroll
  for (int j = 0; j < kM; ++j) {
    const int s = load_uniform(a.members, (int64_t)g * kM + j);
    sm[j] = s;
    if (nm == j && s >= 0 && s < a.num_seqs) nm = j + 1;
  }
  if (nm == 0 || c >= (uint32_t)a.chunks) return;
  float *dst = a.partials + (((int64_t)g * a.chunks + c) * H + h) * kM * (D + 2);
  const int leader = sm[0];

  const int grp = lane / R::kLPT, col = lane % R::kLPT;
  const char *kbase = reinterpret_cast<const char *>(a.k_cache);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache);
  const int64_t block_stride = (int64_t)H * B * R::kRowBytes;
  const int64_t head_off = (int64_t)h * B * R::kRowBytes + col * 16;

  uint4 qf[kM];
#pragma unroll
  for (int j = 0; j < kM; ++j) {
    qf[j] = make_uint4(0, 0, 0, 0);
    if (j < nm)
      qf[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(a.q) +
                                                ((int64_t)sm[j] * H + h) * R::kRowBytes + col * 16);
  }
  float m[kM], l[kM], acc[kM][R::kFE];
#pragma unroll
  for (int j = 0; j < kM; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < R::kFE; ++e) acc[j][e] = 0.f;
  }

  // Loads of tile t into slot d; t past the piece (or a block outside the
  // pool) loads row 0 of block 0 and is marked dead, so that every issue is
  // the same instruction sequence and the waits stay exact.
  uint4 kb[kDepthP][R::kNI], vb[kDepthP][R::kNI];
  bool okb[kDepthP];
  auto issue = [&](int d, int t) {
    int32_t phys = -1;
    if (t < t1) {
      const int32_t e = load_uniform(a.block_tables, (int64_t)leader * a.max_blocks + (t * kDecodeTile) / B);
      phys = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
    }
    okb[d] = phys >= 0;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const int pos = t * kDecodeTile + i * R::kGroups + grp;
      const int64_t off = phys >= 0 ? (int64_t)phys * block_stride + head_off + (int64_t)(pos % B) * R::kRowBytes
                                    : (int64_t)col * 16;
      kb[d][i] = load_nt16(kbase + off);
      vb[d][i] = load_nt16(vbase + off);
    }
  };
  auto consume = [&](int d) {
    if (!okb[d]) return;  // wave-uniform: a table entry outside the pool
#pragma unroll
    for (int j = 0; j < kM; ++j) {
      if (j >= nm) continue;
      float sc[R::kNI];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < R::kNI; ++i) {
        sc[i] = group_sum<R::kLPT>(frag_dot<T>(qf[j], kb[d][i])) * a.scale_log2;
        mt = fmaxf(mt, sc[i]);
      }
      const float mn = fmaxf(m[j], mt);
      const float alpha = fast_exp2(m[j] - mn);  // m[j] = -inf at first: 0
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < R::kNI; ++i) {
        const float p = fast_exp2(sc[i] - mn);
        l[j] += p;
        frag_axpy<T>(acc[j], p, vb[d][i]);
      }
      m[j] = mn;
    }
  };

#pragma unroll
  for (int d = 0; d < kDepthP; ++d) issue(d, t0 + d);
  for (int t = t0; t < t1; t += kDepthP) {
#pragma unroll
    for (int d = 0; d < kDepthP; ++d) {
      if (t + d < t1) consume(d);
      issue(d, t + d + kDepthP);
    }
  }

  // Merge the lane groups (each held different tokens), then store every
  // member's (value sum, max, sum) for the combine step.
#pragma unroll
  for (int j = 0; j < kM; ++j) {
    if (j >= nm) continue;
#pragma unroll
    for (int x = R::kLPT; x < kWave; x *= 2) {
      const float mo = __shfl_xor(m[j], x, kWave);
      const float lo = __shfl_xor(l[j], x, kWave);
      const float mx = fmaxf(m[j], mo);
      const float mu = (mx == -INFINITY) ? 0.f : mx;
      const float fa = fast_exp2(m[j] - mu), fb = fast_exp2(mo - mu);
      l[j] = l[j] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) acc[j][e] = acc[j][e] * fa + __shfl_xor(acc[j][e], x, kWave) * fb;
      m[j] = mx;
    }
    float *f = dst + j * (D + 2);
    if (lane < R::kLPT) {
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) f[col * R::kFE + e] = acc[j][e];
    }
    if (lane == 0) {
      f[D] = m[j];
      f[D + 1] = l[j];
    }
  }
}

// Worker w's share of the prefix stream: every (group g, head h, tile t),
// ordered g, h, t, split over Gp <= G workers in equal ranges of at least
// kPrefixMinTiles tiles.  Worker 0 publishes the stream's size and split and
// every group's offset and tiles in a.pplan for the combine.
template <Dt T, int D, int B, int kDepthP>
__device__ __forceinline__ void prefix_worker(const SharedArgs &a, uint32_t w, uint32_t G) {
  const int lane = threadIdx.x % kWave;
  const int NG = a.num_groups;
  const uint64_t H = (uint64_t)a.num_heads;
  uint32_t per_head = 0;
  for (int c0 = 0; c0 < NG; c0 += kWave) {
    const int g = c0 + lane;
    const uint32_t tg = g < NG ? group_tiles(a, g) : 0u;
    per_head += __builtin_amdgcn_readlane(wave_inclusive_scan(tg), kWave - 1);
  }
  const uint32_t TP = (uint32_t)(per_head * H);
  uint32_t Gp = TP / kPrefixMinTiles;
  Gp = Gp < 1u ? 1u : (Gp > G ? G : Gp);
  const bool writer = w == 0;
  if (writer && lane == 0) {
    a.pplan[0] = TP;
    a.pplan[1] = Gp;
  }
  const bool worker = TP > 0 && w < Gp;
  if (!worker && !writer) return;
  const uint32_t p0 = worker ? range_begin(w, TP, Gp) : 0u, p1 = worker ? range_begin(w + 1, TP, Gp) : 0u;

  // The group holding p0 (the first with tiles whose end passes p0); worker
  // 0 also stores every group's offset and tiles.
  int g_at = -1;
  uint32_t off_at = 0, tg_at = 0, base = 0;
  for (int c0 = 0; c0 < NG; c0 += kWave) {
    const int g = c0 + lane;
    const uint32_t tg = g < NG ? group_tiles(a, g) : 0u;
    const uint32_t incl = wave_inclusive_scan(tg);
    const uint32_t off = base + incl - tg;
    if (writer && g < NG) {
      a.pplan[kPrefixPlanHeader + 2 * g] = off;
      a.pplan[kPrefixPlanHeader + 2 * g + 1] = tg;
    }
    if (worker && g_at < 0) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(tg > 0 && (uint64_t)(off + tg) * H > p0);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        g_at = c0 + l;
        off_at = __builtin_amdgcn_readlane(off, l);
        tg_at = __builtin_amdgcn_readlane(tg, l);
      }
    }
    base += __builtin_amdgcn_readlane(incl, kWave - 1);
    if (!writer && g_at >= 0) break;
  }
  if (!worker || g_at < 0) return;

  int g = g_at;
  uint32_t off = off_at, tg = tg_at;
  const uint32_t local = p0 - (uint32_t)(off * H);
  int h = (int)(local / tg), t = (int)(local % tg);
  uint32_t p = p0;
  for (;;) {
    const uint32_t pair_start = (uint32_t)(off * H) + (uint32_t)h * tg;
    const uint32_t left = p1 - p;
    const int t_end = (uint32_t)(tg - t) < left ? (int)tg : t + (int)left;
    prefix_piece<T, D, B, kDepthP>(a, g, h, t, t_end, w - first_worker(pair_start, TP, Gp));
    p += (uint32_t)(t_end - t);
    if (p >= p1) break;
    t = 0;
    if (++h == a.num_heads) {
      h = 0;
      off += tg;
      do {
        if (++g >= NG) return;  // not reached: p < p1 <= TP
        tg = group_tiles_uniform(a, g);
      } while (tg == 0);
    }
  }
}

constexpr int kPassOwn = 1;
constexpr int kPassPrefix = 2;

// The own positions (what & kPassOwn) and the shared prefixes (what &
// kPassPrefix) of a shared-prefix decode in one launch; every wave of the
// grid is a worker of both streams (a.workers of them).
template <Dt T, int D, int B>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_shared_pass_kernel(DecodeArgs a, SharedArgs s,
                                                                                         int what) {
  const uint32_t w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  if (what & kPassPrefix) prefix_worker<T, D, B, kSharedPrefixDepth>(s, w, (uint32_t)a.workers);
  if (what & kPassOwn) partition_worker<T, D, B, false, kSharedOwnDepth>(a, w);
}

// Members one combine wave merges: j and j + kM/2 of its (group, head), so
// that a launch for the widest groups fits the chip's resident waves at once.
constexpr int kCombineMembers = 2;

// out[s][h] for members j and j + kM/2 of group g: the pieces of the (g, h)
// prefix pair and the pass's partial of s's own positions, rescaled to a
// common max.  One wave per (group, member pair, head); lane l holds
// dimensions l, l+64, ...  The work is a few small reads, so their latency is
// what counts.  The first kU piece slots of both members depend only on (g,
// j, h), so they are loaded together with the prefix plan and the member ids
// (and used only for the pieces the plan says exist), and the members' own
// rows right after them: two round trips to memory in the usual case of at
// most kU pieces.  The sums run over the suffix and then the pieces in order,
// whichever loop a piece's loads are in.
template <Dt T, int D>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_combine_kernel(SharedArgs a) {
  constexpr int kM = kSharedMaxMembers;
  constexpr int kJ = kCombineMembers;
  constexpr int kSpan = kM / kJ;          // member j + kSpan is the wave's second
  constexpr int kU = 4;                   // pieces loaded up front (and per later batch)
  constexpr int kPer = D / kWave;         // dimensions per lane
  static_assert(D % kWave == 0, "head_dim is whole waves");
  static_assert(kM % kJ == 0, "members split evenly over the waves");
  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  const int H = a.num_heads;
  const int h = w % H;
  const int j0 = (w / H) % kSpan;
  const int g = w / (H * kSpan);
  if (g >= a.num_groups) return;
  const int C = a.chunks;
  const int64_t chunk_stride = (int64_t)H * kM * (D + 2);  // floats from piece slot c to c+1
  const uint32_t TP = load_uniform(a.pplan, 0), Gp = load_uniform(a.pplan, 1);
  const uint32_t off = load_uniform(a.pplan, kPrefixPlanHeader + 2 * g);
  const uint32_t tg = load_uniform(a.pplan, kPrefixPlanHeader + 2 * g + 1);
  const float *part0[kJ];
  float mc0[kJ][kU], lc0[kJ][kU], v0[kJ][kU][kPer];
#pragma unroll
  for (int m = 0; m < kJ; ++m) {
    part0[m] = a.partials + (((int64_t)g * C * H + h) * kM + j0 + m * kSpan) * (D + 2);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = u < C;
      mc0[m][u] = in ? load_uniform(part0[m] + u * chunk_stride, D) : -INFINITY;
      lc0[m][u] = in ? load_uniform(part0[m] + u * chunk_stride, D + 1) : 0.f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) v0[m][u][i] = in ? part0[m][u * chunk_stride + lane + kWave * i] : 0.f;
    }
  }
  // Member j exists only inside the leading run of valid ids (as the prefix
  // pieces count them).
  int ids[kM];
#pragma unroll
  for (int i = 0; i < kM; ++i) ids[i] = load_uniform(a.members, (int64_t)g * kM + i);
  bool ok[kJ];
  int sq[kJ];
#pragma unroll
  for (int m = 0; m < kJ; ++m) {
    ok[m] = true;
#pragma unroll
    for (int i = 0; i < kM; ++i)
      if (i <= j0 + m * kSpan && (ids[i] < 0 || ids[i] >= a.num_seqs)) ok[m] = false;
    sq[m] = ok[m] ? ids[j0 + m * kSpan] : 0;
  }
  bool any = false;
#pragma unroll
  for (int m = 0; m < kJ; ++m) any |= ok[m];
  if (!any) return;
  // The members' own rows (a member that does not exist reads sequence 0's
  // and is skipped).
  int n[kJ], raw[kJ];
  float m_sfx[kJ], sv[kJ][kPer];
#pragma unroll
  for (int m = 0; m < kJ; ++m) {
    const float *sfx = a.suffix + (int64_t)sq[m] * a.suffix_row + (int64_t)h * (D + 2);
    n[m] = clip_ctx(load_uniform(a.context_lens, sq[m]), a.ctx_cap);
    raw[m] = load_uniform(a.starts, sq[m]);
    m_sfx[m] = load_uniform(sfx, D);
#pragma unroll
    for (int i = 0; i < kPer; ++i) sv[m][i] = sfx[lane + kWave * i];
  }
  // Pieces of the pair: one per worker whose prefix range meets it.
  int np = 0;
  if (tg > 0) {
    const uint32_t ps = off * (uint32_t)H + (uint32_t)h * tg;
    np = (int)(first_worker(ps + tg - 1, TP, Gp) - first_worker(ps, TP, Gp)) + 1;
    np = np < C ? np : C;
  }
#pragma unroll
  for (int m = 0; m < kJ; ++m) {
    const int st = raw[m] < 0 ? 0 : min(raw[m] & ~(kDecodeTile - 1), n[m]);
    if (!ok[m] || st == 0) continue;  // no member, or no shared prefix: the pass wrote the output
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u >= np) {
        mc0[m][u] = -INFINITY;
        lc0[m][u] = 0.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) v0[m][u][i] = 0.f;
      }
    }
    // The common max over the suffix and every piece, then the sums.
    float M = m_sfx[m];
#pragma unroll
    for (int u = 0; u < kU; ++u) M = fmaxf(M, mc0[m][u]);
    for (int c0 = kU; c0 < np; c0 += kU) {
      float mc[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        mc[u] = c0 + u < np ? load_uniform(part0[m] + (c0 + u) * chunk_stride, D) : -INFINITY;
#pragma unroll
      for (int u = 0; u < kU; ++u) M = fmaxf(M, mc[u]);
    }
    const float mu = (M == -INFINITY) ? 0.f : M;
    const float ws = fast_exp2(m_sfx[m] - mu);  // the suffix partial is normalised: its sum is 1
    float L = ws, A[kPer];
    float e0[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      e0[u] = fast_exp2(mc0[m][u] - mu);
      L += lc0[m][u] * e0[u];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      A[i] = sv[m][i] * ws;
#pragma unroll
      for (int u = 0; u < kU; ++u) A[i] += v0[m][u][i] * e0[u];
    }
    for (int c0 = kU; c0 < np; c0 += kU) {
      float mc[kU], lc[kU], v[kU][kPer];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const bool in = c0 + u < np;
        mc[u] = in ? load_uniform(part0[m] + (c0 + u) * chunk_stride, D) : -INFINITY;
        lc[u] = in ? load_uniform(part0[m] + (c0 + u) * chunk_stride, D + 1) : 0.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) v[u][i] = in ? part0[m][(c0 + u) * chunk_stride + lane + kWave * i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float e = fast_exp2(mc[u] - mu);
        L += lc[u] * e;
#pragma unroll
        for (int i = 0; i < kPer; ++i) A[i] += v[u][i] * e;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float o = A[i] * inv;
      const int64_t idx = ((int64_t)sq[m] * H + h) * D + lane + kWave * i;
      if constexpr (T == Dt::F32) reinterpret_cast<float *>(a.out)[idx] = o;
      else if constexpr (T == Dt::F16) reinterpret_cast<uint16_t *>(a.out)[idx] = (uint16_t)f32_to_f16_bits(o);
      else reinterpret_cast<uint16_t *>(a.out)[idx] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <Dt T, int D, int B>
int pass_waves() {
  static const int v = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_shared_pass_kernel<T, D, B>,
                                                     kDecodeWavesPerGroup * kWave, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb * kDecodeWavesPerGroup;
  }();
  return v;
}

template <Dt T, int D, int B>
hipError_t launch_pass_tdb(const DecodeArgs &a, const SharedArgs &s, int what, hipStream_t st) {
  const unsigned groups = (unsigned)((a.workers + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup);
  hipLaunchKernelGGL((decode_shared_pass_kernel<T, D, B>), dim3(groups), dim3(kDecodeWavesPerGroup * kWave), 0, st,
                     a, s, what);
  return hipGetLastError();
}

#define PA_SHARED_DISPATCH(FN, ...)                                   \
  switch (D) {                                                        \
    case 64:                                                          \
      switch (B) {                                                    \
        case 16: return FN<T, 64, 16>(__VA_ARGS__);                   \
        case 32: return FN<T, 64, 32>(__VA_ARGS__);                   \
        case 64: return FN<T, 64, 64>(__VA_ARGS__);                   \
      }                                                               \
      break;                                                          \
    case 128:                                                         \
      switch (B) {                                                    \
        case 16: return FN<T, 128, 16>(__VA_ARGS__);                  \
        case 32: return FN<T, 128, 32>(__VA_ARGS__);                  \
        case 64: return FN<T, 128, 64>(__VA_ARGS__);                  \
      }                                                               \
      break;                                                          \
  }

template <Dt T>
int pass_waves_t(int D, int B) {
  PA_SHARED_DISPATCH(pass_waves)
  return 0;
}

template <Dt T>
hipError_t launch_pass_t(const DecodeArgs &a, const SharedArgs &s, int D, int B, int what, hipStream_t st) {
  PA_SHARED_DISPATCH(launch_pass_tdb, a, s, what, st)
  return hipErrorInvalidValue;
}

template <Dt T>
hipError_t launch_combine_t(const SharedArgs &a, int D, hipStream_t st) {
  const int64_t items = (int64_t)a.num_groups * (kSharedMaxMembers / kCombineMembers) * a.num_heads;
  const dim3 grid((unsigned)((items + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup));
  const dim3 block(kDecodeWavesPerGroup * kWave);
  if (D == 64) hipLaunchKernelGGL((decode_combine_kernel<T, 64>), grid, block, 0, st, a);
  else if (D == 128) hipLaunchKernelGGL((decode_combine_kernel<T, 128>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool shared_supported(int dtype, int head_dim, int block_size) {
  return dtype >= 0 && dtype <= 2 && (head_dim == 64 || head_dim == 128) &&
         (block_size == 16 || block_size == 32 || block_size == 64);
}

int shared_waves_per_cu(int dtype, int head_dim, int block_size) {
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return pass_waves_t<Dt::F32>(head_dim, block_size);
    case Dt::F16: return pass_waves_t<Dt::F16>(head_dim, block_size);
    case Dt::BF16: return pass_waves_t<Dt::BF16>(head_dim, block_size);
  }
  return 0;
}

hipError_t launch_shared_pass(const DecodeArgs &a, const SharedArgs &s, int dtype, int head_dim, int block_size,
                              bool own, bool prefix, hipStream_t stream) {
  if (!own && !prefix) return hipSuccess;
  if (own && a.num_seqs > kSelfPlanSeqs) {
    const hipError_t e = launch_decode_plan(a, stream);
    if (e != hipSuccess) return e;
  }
  const int what = (own ? kPassOwn : 0) | (prefix ? kPassPrefix : 0);
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_pass_t<Dt::F32>(a, s, head_dim, block_size, what, stream);
    case Dt::F16: return launch_pass_t<Dt::F16>(a, s, head_dim, block_size, what, stream);
    case Dt::BF16: return launch_pass_t<Dt::BF16>(a, s, head_dim, block_size, what, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_shared_combine(const SharedArgs &a, int dtype, int head_dim, hipStream_t stream) {
  if (a.num_groups == 0) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_combine_t<Dt::F32>(a, head_dim, stream);
    case Dt::F16: return launch_combine_t<Dt::F16>(a, head_dim, stream);
    case Dt::BF16: return launch_combine_t<Dt::BF16>(a, head_dim, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
