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
//   - the shared prefix [0, P): one wave per (group, head, chunk of prefix
//     tiles) loads each K/V tile once and folds it into the running state of
//     every member's query (decode_prefix_kernel, below);
//   - each member's own positions [P, n): the stream-K decode pass with a
//     per-sequence start, leaving a normalised fp32 partial and its log2
//     softmax denominator (pa_decode.hip);
//   - a merge of the two per (sequence, head) into the output
//     (decode_combine_kernel, below).
//
// Mapping.  As in the decode pass, a K/V row of one token and head is
// covered by LPT lanes with one 16-byte load each; one wave load covers
// 64/LPT tokens, a 16-token tile takes kNI loads for K and kNI for V.  The
// prefix tiles are always full (P is a multiple of the tile, within every
// member's context), so no masking is needed there.  Members' states live
// in registers (up to kSharedMaxMembers); the lane groups of a wave hold
// different tokens and are merged at the end of the chunk.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

}  // namespace

constexpr int kPrefixDepth = 2;  // tiles in flight per wave

template <Dt T, int D, int B>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_prefix_kernel(SharedArgs a) {
  using R = RowShape<T, D, kDecodeTile>;
  constexpr int kM = kSharedMaxMembers;
  static_assert(B % kDecodeTile == 0, "a prefix tile must lie in one block");
  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  const int H = a.num_heads;
  const int h = w % H;
  const int c = (w / H) % a.chunks;
  const int g = w / (H * a.chunks);
  if (g >= a.num_groups) return;

  // Members (a leading run of valid sequence ids) and the group's prefix
  // tiles, clamped to the first member's context so that every table entry
  // read lies inside its row.
  int sm[kM];
  int nm = 0;
#pragma unroll
  for (int j = 0; j < kM; ++j) {
    const int s = load_uniform(a.members, (int64_t)g * kM + j);
    sm[j] = s;
    if (nm == j && s >= 0 && s < a.num_seqs) nm = j + 1;
  }
  float *dst = a.partials + (((int64_t)g * a.chunks + c) * H + h) * kM * (D + 2);
  if (nm == 0) return;
  const int leader = sm[0];
  int prefix = load_uniform(a.prefix, g);
  const int n0 = clamp_len(load_uniform(a.context_lens, leader), a.ctx_cap);
  prefix = prefix < 0 ? 0 : (prefix > n0 ? n0 : prefix);
  const int tiles = prefix / kDecodeTile;
  const int t0 = c * a.chunk_tiles;
  const int t1 = min(tiles, t0 + a.chunk_tiles);

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

  // Loads of tile t into slot d; t past the range (or a block outside the
  // pool) loads row 0 of block 0 and is marked dead, so that every issue is
  // the same instruction sequence and the waits stay exact.
  uint4 kb[kPrefixDepth][R::kNI], vb[kPrefixDepth][R::kNI];
  bool okb[kPrefixDepth];
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
  for (int d = 0; d < kPrefixDepth; ++d) issue(d, t0 + d);
  for (int t = t0; t < t1; t += kPrefixDepth) {
#pragma unroll
    for (int d = 0; d < kPrefixDepth; ++d) {
      if (t + d < t1) consume(d);
      issue(d, t + d + kPrefixDepth);
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

// out[s][h] for member j of group g: the prefix chunks' partials and the
// pass's partial of s's own positions, rescaled to a common max.  One wave
// per (group, member, head); lane l holds dimensions l, l+64, ...  The work
// is a few small reads, so their latency is what counts.  The partials of
// the first kU chunks depend only on (g, j, h), so they are loaded before
// the member ids, and the member's own row right after them: two round trips
// to memory in the usual case of at most kU chunks.  The sums run over the
// suffix and then the chunks in order, whichever loop a chunk's loads are in.
template <Dt T, int D>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void decode_combine_kernel(SharedArgs a) {
  constexpr int kM = kSharedMaxMembers;
  constexpr int kU = 4;                   // chunks loaded up front (and per later batch)
  constexpr int kPer = D / kWave;         // dimensions per lane
  static_assert(D % kWave == 0, "head_dim is whole waves");
  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  const int H = a.num_heads;
  const int h = w % H;
  const int j = (w / H) % kM;
  const int g = w / (H * kM);
  if (g >= a.num_groups) return;
  const int C = a.chunks;
  const int64_t chunk_stride = (int64_t)H * kM * (D + 2);  // floats from chunk c to c+1
  const float *part0 = a.partials + (((int64_t)g * C * H + h) * kM + j) * (D + 2);
  float mc0[kU], lc0[kU], v0[kU][kPer];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const bool in = u < C;
    mc0[u] = in ? load_uniform(part0 + u * chunk_stride, D) : -INFINITY;
    lc0[u] = in ? load_uniform(part0 + u * chunk_stride, D + 1) : 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) v0[u][i] = in ? part0[u * chunk_stride + lane + kWave * i] : 0.f;
  }
  // Member j exists only inside the leading run of valid ids (as the prefix
  // kernel counts them).
  int ids[kM];
#pragma unroll
  for (int i = 0; i < kM; ++i) ids[i] = load_uniform(a.members, (int64_t)g * kM + i);
#pragma unroll
  for (int i = 0; i < kM; ++i)
    if (i <= j && (ids[i] < 0 || ids[i] >= a.num_seqs)) return;
  const int s = ids[j];
  const float *sfx = a.suffix + (int64_t)s * a.suffix_row + (int64_t)h * (D + 2);
  const int n = clamp_len(load_uniform(a.context_lens, s), a.ctx_cap);
  const int raw = load_uniform(a.starts, s);
  const float m_sfx = load_uniform(sfx, D);
  float sv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) sv[i] = sfx[lane + kWave * i];
  const int st = raw < 0 ? 0 : min(raw & ~(kDecodeTile - 1), n);
  if (st == 0) return;  // no shared prefix for s: the pass wrote its output
  // The common max over the suffix and every chunk, then the sums.
  float M = m_sfx;
#pragma unroll
  for (int u = 0; u < kU; ++u) M = fmaxf(M, mc0[u]);
  for (int c0 = kU; c0 < C; c0 += kU) {
    float mc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) mc[u] = c0 + u < C ? load_uniform(part0 + (c0 + u) * chunk_stride, D) : -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) M = fmaxf(M, mc[u]);
  }
  const float mu = (M == -INFINITY) ? 0.f : M;
  const float ws = fast_exp2(m_sfx - mu);  // the suffix partial is normalised: its sum is 1
  float L = ws, A[kPer];
  float e0[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    e0[u] = fast_exp2(mc0[u] - mu);
    L += lc0[u] * e0[u];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    A[i] = sv[i] * ws;
#pragma unroll
    for (int u = 0; u < kU; ++u) A[i] += v0[u][i] * e0[u];
  }
  for (int c0 = kU; c0 < C; c0 += kU) {
    float mc[kU], lc[kU], v[kU][kPer];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = c0 + u < C;
      mc[u] = in ? load_uniform(part0 + (c0 + u) * chunk_stride, D) : -INFINITY;
      lc[u] = in ? load_uniform(part0 + (c0 + u) * chunk_stride, D + 1) : 0.f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) v[u][i] = in ? part0[(c0 + u) * chunk_stride + lane + kWave * i] : 0.f;
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
    const int64_t idx = ((int64_t)s * H + h) * D + lane + kWave * i;
    if constexpr (T == Dt::F32) reinterpret_cast<float *>(a.out)[idx] = o;
    else if constexpr (T == Dt::F16) reinterpret_cast<uint16_t *>(a.out)[idx] = (uint16_t)f32_to_f16_bits(o);
    else reinterpret_cast<uint16_t *>(a.out)[idx] = (uint16_t)f32_to_bf16_bits(o);
  }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <Dt T, int D, int B>
hipError_t launch_prefix_tdb(const SharedArgs &a, hipStream_t st) {
  const int64_t items = (int64_t)a.num_groups * a.chunks * a.num_heads;
  const unsigned groups = (unsigned)((items + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup);
  hipLaunchKernelGGL((decode_prefix_kernel<T, D, B>), dim3(groups), dim3(kDecodeWavesPerGroup * kWave), 0, st, a);
  return hipGetLastError();
}

template <Dt T, int D>
hipError_t launch_prefix_td(const SharedArgs &a, int B, hipStream_t st) {
  switch (B) {
    case 16: return launch_prefix_tdb<T, D, 16>(a, st);
    case 32: return launch_prefix_tdb<T, D, 32>(a, st);
    case 64: return launch_prefix_tdb<T, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <Dt T>
hipError_t launch_shared_t(const SharedArgs &a, int D, int B, bool prefix, bool combine, hipStream_t st) {
  const int64_t items = (int64_t)a.num_groups * kSharedMaxMembers * a.num_heads;
  const dim3 grid((unsigned)((items + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup));
  const dim3 block(kDecodeWavesPerGroup * kWave);
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  if (prefix) {
    const hipError_t e = D == 64 ? launch_prefix_td<T, 64>(a, B, st) : launch_prefix_td<T, 128>(a, B, st);
    if (e != hipSuccess) return e;
  }
  if (combine) {
    if (D == 64) hipLaunchKernelGGL((decode_combine_kernel<T, 64>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_combine_kernel<T, 128>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

bool shared_supported(int dtype, int head_dim, int block_size) {
  return dtype >= 0 && dtype <= 2 && (head_dim == 64 || head_dim == 128) &&
         (block_size == 16 || block_size == 32 || block_size == 64);
}

hipError_t launch_shared_phases(const SharedArgs &a, int dtype, int head_dim, int block_size, bool prefix,
                                bool combine, hipStream_t stream) {
  if (a.num_groups == 0 || (!prefix && !combine)) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_shared_t<Dt::F32>(a, head_dim, block_size, prefix, combine, stream);
    case Dt::F16: return launch_shared_t<Dt::F16>(a, head_dim, block_size, prefix, combine, stream);
    case Dt::BF16: return launch_shared_t<Dt::BF16>(a, head_dim, block_size, prefix, combine, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
