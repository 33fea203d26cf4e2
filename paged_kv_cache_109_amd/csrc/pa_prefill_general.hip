// Chunked-prefill attention for the shapes the MFMA kernel does not cover
// (fp32, or head_dim 64): the same causal attention over a paged cache,
// computed on the vector ALU.
//
// What is computed is what pa_prefill.hip computes: query j of a sequence's
// chunk sits at position c + j (c cached tokens before the chunk) and
// attends with the softmax of scale * q.k over positions 0 .. c + j, the
// K/V read through the block table (paper notes "PagedAttention: Efficient
// Memory Management for Large Language Model Serving", section 3.1; the
// arcyou.ai teardown of vLLM, continuous-batching section, for chunking).
//
// Mapping.  One wave per (sequence, head, 8 consecutive queries): the K/V
// tiles those queries see are loaded once, and every query's online
// softmax state lives in registers.  As in decode, a K/V row of one token
// is covered by LPT lanes with one 16-byte load each and the lane groups of
// a wave hold different tokens (merged at the end); each group looks its
// token's table entry up itself, so blocks of any size work.  A tile that
// lies wholly before a query's position needs no mask for it; the others
// mask per token.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kGenQueries = 8;  // queries per wave
constexpr int kGenDepth = 2;    // tiles in flight per wave

template <Dt T, int D, int B>
__global__ __launch_bounds__(kDecodeWavesPerGroup *kWave) void prefill_general_kernel(PrefillArgs a, int qgroups) {
  using R = RowShape<T, D, kDecodeTile>;
  constexpr int kQ = kGenQueries;
  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * kDecodeWavesPerGroup + wave_id_uniform();
  const int H = a.num_heads;
  const int qg = w % qgroups;
  const int h = (w / qgroups) % H;
  const int s = w / (qgroups * H);
  if (s >= a.num_seqs) return;
  const int q0 = load_uniform(a.cu_q_lens, s);
  const int q_len = load_uniform(a.cu_q_lens, s + 1) - q0;
  const int n = min(max(load_uniform(a.context_lens, s), 0), a.ctx_cap);
  const int c = n - q_len;
  const int j0 = qg * kQ;
  if (q_len <= 0 || j0 >= q_len) return;
  // Valid queries: inside the chunk and the context, and whose rows lie in
  // q / out (cu_q_lens is device data, so rows are checked against total_q).
  int nq = 0;
  for (int j = 0; j < kQ; ++j) {
    const int jq = j0 + j;
    if (jq < q_len && c + jq >= 0 && c + jq < n && q0 >= 0 && q0 + jq < a.total_q) nq = j + 1;
    else break;
  }
  if (nq == 0) return;
  const int last_pos = c + j0 + nq - 1;  // the last position any of these queries sees
  const int tiles = last_pos / kDecodeTile + 1;

  const int grp = lane / R::kLPT, col = lane % R::kLPT;
  const char *kbase = reinterpret_cast<const char *>(a.k_cache);
  const char *vbase = reinterpret_cast<const char *>(a.v_cache);
  const int64_t block_stride = (int64_t)H * B * R::kRowBytes;
  const int64_t head_off = (int64_t)h * B * R::kRowBytes + col * 16;
  const int64_t table_row = (int64_t)s * a.max_blocks;

  uint4 qf[kQ];
  float m[kQ], l[kQ], acc[kQ][R::kFE];
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    qf[j] = make_uint4(0, 0, 0, 0);
    if (j < nq)
      qf[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(a.q) +
                                                ((int64_t)(q0 + j0 + j) * H + h) * R::kRowBytes + col * 16);
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < R::kFE; ++e) acc[j][e] = 0.f;
  }

  // Loads of tile t into slot d: this lane group's token of each load, its
  // table entry looked up per token (entries outside the pool, and tokens
  // past last_pos, read row 0 of block 0 and are masked at use).
  uint4 kb[kGenDepth][R::kNI], vb[kGenDepth][R::kNI];
  uint32_t okb[kGenDepth];
  auto issue = [&](int d, int t) {
    uint32_t ok = 0;
#pragma unroll
    for (int i = 0; i < R::kNI; ++i) {
      const int pos = t * kDecodeTile + i * R::kGroups + grp;
      int64_t off = (int64_t)col * 16;
      if (t < tiles && pos <= last_pos) {
        const int32_t e = a.block_tables[table_row + pos / B];
        if (e >= 0 && (int64_t)e < a.num_blocks) {
          off = (int64_t)e * block_stride + head_off + (int64_t)(pos % B) * R::kRowBytes;
          ok |= 1u << i;
        }
      }
      kb[d][i] = *reinterpret_cast<const uint4 *>(kbase + off);
      vb[d][i] = *reinterpret_cast<const uint4 *>(vbase + off);
    }
    okb[d] = ok;
  };
  auto consume = [&](int d, int t) {
    // Masked tokens hold the dummy row: zero their values (their weights
    // are 0, but 0 * NaN is not).
#pragma unroll
    for (int i = 0; i < R::kNI; ++i)
      if (!((okb[d] >> i) & 1u)) vb[d][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      if (j >= nq) continue;
      const int qpos = c + j0 + j;
      float sc[R::kNI];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < R::kNI; ++i) {
        const int pos = t * kDecodeTile + i * R::kGroups + grp;
        const float dot = group_sum<R::kLPT>(frag_dot<T>(qf[j], kb[d][i])) * a.scale_log2;
        sc[i] = (((okb[d] >> i) & 1u) && pos <= qpos) ? dot : -INFINITY;
        mt = fmaxf(mt, sc[i]);
      }
      const float mn = fmaxf(m[j], mt);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(m[j] - mu);
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < R::kNI; ++i) {
        const float p = fast_exp2(sc[i] - mu);
        l[j] += p;
        frag_axpy<T>(acc[j], p, vb[d][i]);
      }
      m[j] = mn;
    }
  };

#pragma unroll
  for (int d = 0; d < kGenDepth; ++d) issue(d, d);
  for (int t = 0; t < tiles; t += kGenDepth) {
#pragma unroll
    for (int d = 0; d < kGenDepth; ++d) {
      if (t + d < tiles) consume(d, t + d);
      issue(d, t + d + kGenDepth);
    }
  }

  // Merge the lane groups, then write each query's row.
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    if (j >= nq) continue;
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
    if (lane < R::kLPT) {
      const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
      float o[R::kFE];
#pragma unroll
      for (int e = 0; e < R::kFE; ++e) o[e] = acc[j][e] * inv;
      char *orow = reinterpret_cast<char *>(a.out) + ((int64_t)(q0 + j0 + j) * H + h) * R::kRowBytes;
      *reinterpret_cast<uint4 *>(orow + col * 16) = frag_pack<T>(o);
    }
  }
}

template <Dt T, int D, int B>
hipError_t launch_gen_tdb(const PrefillArgs &a, hipStream_t st) {
  const int qgroups = (a.max_q_len + kGenQueries - 1) / kGenQueries;
  const int64_t items = (int64_t)a.num_seqs * a.num_heads * qgroups;
  const int64_t groups = (items + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_general_kernel<T, D, B>), dim3((unsigned)groups), dim3(kDecodeWavesPerGroup * kWave), 0,
                     st, a, qgroups);
  return hipGetLastError();
}

template <Dt T, int D>
hipError_t launch_gen_td(const PrefillArgs &a, int B, hipStream_t st) {
  switch (B) {
    case 4: return launch_gen_tdb<T, D, 4>(a, st);
    case 8: return launch_gen_tdb<T, D, 8>(a, st);
    case 16: return launch_gen_tdb<T, D, 16>(a, st);
    case 32: return launch_gen_tdb<T, D, 32>(a, st);
    case 64: return launch_gen_tdb<T, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <Dt T>
hipError_t launch_gen_t(const PrefillArgs &a, int D, int B, hipStream_t st) {
  if (D == 64) return launch_gen_td<T, 64>(a, B, st);
  if (D == 128) return launch_gen_td<T, 128>(a, B, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_general_supported(int dtype, int head_dim, int block_size) {
  return dtype >= 0 && dtype <= 2 && (head_dim == 64 || head_dim == 128) &&
         (block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64);
}

hipError_t launch_prefill_general(const PrefillArgs &a, int dtype, int head_dim, int block_size, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  switch (static_cast<Dt>(dtype)) {
    case Dt::F32: return launch_gen_t<Dt::F32>(a, head_dim, block_size, stream);
    case Dt::F16: return launch_gen_t<Dt::F16>(a, head_dim, block_size, stream);
    case Dt::BF16: return launch_gen_t<Dt::BF16>(a, head_dim, block_size, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
