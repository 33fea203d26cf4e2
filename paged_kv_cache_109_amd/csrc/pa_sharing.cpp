// Host-side derivation of the prompt-sharing description that the
// shared-prefix decode takes (pa_shared_prefix_groups).
//
// Samples forked from one prompt point their block tables at the prompt's
// physical blocks (paper notes "PagedAttention: Efficient Memory Management
// for Large Language Model Serving", section 3.4.1 Parallel sampling;
// "KV 캐시 관리와 PagedAttention", section on sharing the common KV of
// several responses).  A group's shared prefix is the run of leading table
// entries identical in every member and filled in every member, in whole
// 16-token tiles; the shared-prefix decode reads those blocks once for the
// whole group.  No GPU call: the tables a scheduler builds live on the host.
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <vector>

#include "pa_internal.h"

namespace {

constexpr int32_t kTile = 16;

}  // namespace

extern "C" pa_status pa_shared_prefix_groups(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                             const int32_t *context_lens, int32_t num_seqs,
                                             const int32_t *group_offsets, int32_t num_groups,
                                             const int32_t *group_seqs, int32_t block_size, int32_t max_out_groups,
                                             int32_t *group_members, int32_t *group_prefix, int32_t *seq_starts,
                                             int32_t *num_out_groups, int32_t *max_prefix_len) {
  char msg[256];
  auto bad = [&](const char *text) { return pa::record_error(PA_ERR_INVALID_ARG, text); };
  if (num_seqs < 0 || num_groups < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || max_out_groups < 0)
    return bad("pa_shared_prefix_groups: sizes must be positive (num_seqs, num_groups, max_out_groups >= 0)");
  if (!group_offsets || !num_out_groups || !max_prefix_len || (num_seqs > 0 && (!block_tables || !context_lens ||
                                                                                  !seq_starts)))
    return bad("pa_shared_prefix_groups: null pointer argument");
  if (group_offsets[0] != 0) return bad("pa_shared_prefix_groups: group_offsets[0] must be 0");
  int64_t needed = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t k = group_offsets[g + 1] - group_offsets[g];
    if (k < 0) return bad("pa_shared_prefix_groups: group_offsets must not decrease");
    needed += (k + PA_MAX_GROUP_MEMBERS - 1) / PA_MAX_GROUP_MEMBERS;
  }
  const int32_t total = group_offsets[num_groups];
  if (total > 0 && !group_seqs) return bad("pa_shared_prefix_groups: null group_seqs");
  if (needed > max_out_groups) {
    snprintf(msg, sizeof msg, "pa_shared_prefix_groups: %lld output groups needed, max_out_groups is %d",
             (long long)needed, max_out_groups);
    return bad(msg);
  }
  if (needed > 0 && (!group_members || !group_prefix)) return bad("pa_shared_prefix_groups: null output pointer");
  std::vector<char> seen(num_seqs, 0);
  for (int32_t i = 0; i < total; ++i) {
    const int32_t s = group_seqs[i];
    if (s < 0 || s >= num_seqs) {
      snprintf(msg, sizeof msg, "pa_shared_prefix_groups: group_seqs[%d] = %d outside [0, %d)", i, s, num_seqs);
      return bad(msg);
    }
    if (seen[s]) {
      snprintf(msg, sizeof msg, "pa_shared_prefix_groups: sequence %d is listed twice", s);
      return bad(msg);
    }
    seen[s] = 1;
  }
  // Every check passed: write the outputs.
  std::fill(seq_starts, seq_starts + num_seqs, 0);
  int32_t out = 0, widest = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t *mem = group_seqs + group_offsets[g];
    const int32_t k = group_offsets[g + 1] - group_offsets[g];
    if (k == 0) continue;
    // Leading entries identical in every member, then blocks every member
    // has filled: a block is filled when the shortest context covers it.
    const int32_t *first = block_tables + (int64_t)mem[0] * max_blocks_per_seq;
    int32_t shared = max_blocks_per_seq;
    int32_t shortest = INT32_MAX;
    for (int32_t i = 0; i < k; ++i) {
      const int32_t *row = block_tables + (int64_t)mem[i] * max_blocks_per_seq;
      int32_t b = 0;
      while (b < shared && row[b] == first[b]) ++b;
      shared = b;
      shortest = std::min(shortest, std::max(context_lens[mem[i]], 0));
    }
    const int32_t filled = shortest / block_size;
    int64_t P = (int64_t)std::min(shared, filled) * block_size;
    P -= P % kTile;
    for (int32_t i0 = 0; i0 < k; i0 += PA_MAX_GROUP_MEMBERS, ++out) {
      int32_t *row = group_members + (int64_t)out * PA_MAX_GROUP_MEMBERS;
      for (int j = 0; j < PA_MAX_GROUP_MEMBERS; ++j) row[j] = i0 + j < k ? mem[i0 + j] : -1;
      group_prefix[out] = (int32_t)P;
    }
    for (int32_t i = 0; i < k; ++i) seq_starts[mem[i]] = (int32_t)P;
    widest = std::max<int32_t>(widest, (int32_t)P);
  }
  *num_out_groups = out;
  *max_prefix_len = widest;
  return pa::record_ok();
}
