// Debug validation of the data-dependent preconditions (PA_DEBUG_VALIDATE=1).
//
// The entry points check only host scalars and pointers; the device data is
// the caller's promise.  With PA_DEBUG_VALIDATE=1 in the environment each
// entry point first calls one of these: it synchronises the stream, copies
// the index arrays the call will read to the host, and checks what the
// method assumes of them -- a table entry of every valid position names a
// block of the pool (the block table of "PagedAttention: Efficient Memory
// Management for Large Language Model Serving", section 4.1), slots of one
// write are distinct, a copy-on-write destination is a fresh block
// ("KV 캐시 관리와 PagedAttention", copy-on-write section), the sharing
// description of a shared-prefix decode matches the tables, and the calls
// that write the new tokens themselves write distinct slots of blocks no
// other sequence reads.  The first
// violation is reported through the last-error record.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <string>
#include <algorithm>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {

template <typename T>
pa_status fetch(const T *src, size_t count, hipStream_t stream, std::vector<T> &dst, const char *what) {
  dst.resize(count);
  if (count == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(dst.data(), src, count * sizeof(T), hipMemcpyDefault, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    const std::string msg = std::string("PA_DEBUG_VALIDATE: reading ") + what + " failed: " + hipGetErrorString(e);
    return record_error(PA_ERR_HIP, msg.c_str());
  }
  return PA_OK;
}

pa_status bad(const std::string &msg) { return record_error(PA_ERR_INVALID_ARG, ("PA_DEBUG_VALIDATE: " + msg).c_str()); }

std::string str(int64_t v) { return std::to_string(v); }

// Entries of positions [0, ctx) of every sequence name blocks of the pool;
// contexts lie in [0, max_context_len] and max_context_len fits a row.
pa_status check_tables(const std::vector<int32_t> &tables, const std::vector<int32_t> &ctx, int32_t max_blocks,
                       int32_t max_context_len, int32_t block_size, int64_t num_blocks) {
  if ((int64_t)max_context_len > (int64_t)max_blocks * block_size)
    return bad("max_context_len " + str(max_context_len) + " exceeds max_blocks_per_seq * block_size = " +
               str((int64_t)max_blocks * block_size));
  for (size_t s = 0; s < ctx.size(); ++s) {
    const int32_t n = ctx[s];
    if (n < 0 || n > max_context_len)
      return bad("context_lens[" + str(s) + "] = " + str(n) + " outside [0, max_context_len = " +
                 str(max_context_len) + "]");
    const int64_t used = ((int64_t)n + block_size - 1) / block_size;
    for (int64_t b = 0; b < used; ++b) {
      const int32_t e = tables[s * (size_t)max_blocks + b];
      if (e < 0 || e >= num_blocks)
        return bad("block_tables[" + str(s) + "][" + str(b) + "] = " + str(e) + " outside [0, " + str(num_blocks) +
                   ") for context length " + str(n));
    }
  }
  return PA_OK;
}

// The fused-write calls store each sequence's new tokens themselves, at
// positions [first[s], ctx[s]) (decode: the newest token only; prefill: the
// chunk).  Their slots must be distinct, and no other sequence of the batch
// may read a block being written: it would race with the store inside one
// launch.  A block written to has one owner under copy-on-write ("KV 캐시
// 관리와 PagedAttention", section on splitting a shared block that must be
// written), so a shared block a caller forgot to copy is refused here.
pa_status check_writes(const std::vector<int32_t> &tables, const std::vector<int32_t> &ctx,
                       const std::vector<int32_t> &first, int32_t max_blocks, int32_t block_size) {
  const size_t S = ctx.size();
  // Up to two distinct readers of every block inside some context.
  std::unordered_map<int32_t, std::pair<int32_t, int32_t>> readers;
  for (size_t s = 0; s < S; ++s) {
    const int64_t used = ((int64_t)ctx[s] + block_size - 1) / block_size;
    for (int64_t b = 0; b < used; ++b) {
      auto it = readers.emplace(tables[s * (size_t)max_blocks + b], std::make_pair((int32_t)s, -1)).first;
      if (it->second.first != (int32_t)s && it->second.second < 0) it->second.second = (int32_t)s;
    }
  }
  std::unordered_set<int64_t> written;
  for (size_t s = 0; s < S; ++s) {
    for (int32_t p = std::max(first[s], 0); p < ctx[s]; ++p) {
      const int32_t blk = tables[s * (size_t)max_blocks + p / block_size];
      const int64_t slot = (int64_t)blk * block_size + p % block_size;
      if (!written.insert(slot).second)
        return bad("slot " + str(slot) + " is written twice (sequence " + str(s) + ", position " + str(p) + ")");
      const auto &r = readers.at(blk);
      const int32_t other = r.first != (int32_t)s ? r.first : r.second;
      if (other >= 0)
        return bad("sequence " + str(s) + " writes position " + str(p) + " into block " + str(blk) +
                   ", which sequence " + str(other) + " also reads (a shared block must be copied before a write)");
    }
  }
  return PA_OK;
}

}  // namespace

bool debug_validate() {
  const char *v = std::getenv("PA_DEBUG_VALIDATE");
  return v && std::strcmp(v, "1") == 0;
}

pa_status validate_slots(const int64_t *slot_mapping, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                         hipStream_t stream) {
  std::vector<int64_t> slots;
  pa_status st = fetch(slot_mapping, (size_t)num_tokens, stream, slots, "slot_mapping");
  if (st != PA_OK) return st;
  const int64_t pool = num_blocks * block_size;
  std::unordered_set<int64_t> seen;
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t v = slots[t];
    if (v < 0) continue;  // a padding token: skipped
    if (v >= pool) return bad("slot_mapping[" + str(t) + "] = " + str(v) + " outside the pool of " + str(pool) + " slots");
    if (!seen.insert(v).second) return bad("slot " + str(v) + " appears twice in slot_mapping (token " + str(t) + ")");
  }
  return PA_OK;
}

pa_status validate_decode(const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t block_size, int64_t num_blocks,
                          bool append, hipStream_t stream) {
  std::vector<int32_t> tables, ctx;
  pa_status st = fetch(block_tables, (size_t)num_seqs * max_blocks, stream, tables, "block_tables");
  if (st == PA_OK) st = fetch(context_lens, (size_t)num_seqs, stream, ctx, "context_lens");
  if (st != PA_OK) return st;
  st = check_tables(tables, ctx, max_blocks, max_context_len, block_size, num_blocks);
  if (st != PA_OK || !append) return st;
  std::vector<int32_t> first(ctx.size());
  for (size_t s = 0; s < ctx.size(); ++s) first[s] = ctx[s] - 1;  // the newest token
  return check_writes(tables, ctx, first, max_blocks, block_size);
}

pa_status validate_shared(const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t block_size, int64_t num_blocks,
                          const int32_t *group_members, const int32_t *group_prefix, const int32_t *seq_starts,
                          int32_t num_groups, int32_t max_prefix_len, hipStream_t stream) {
  std::vector<int32_t> tables, ctx, members, prefix, starts;
  pa_status st = fetch(block_tables, (size_t)num_seqs * max_blocks, stream, tables, "block_tables");
  if (st == PA_OK) st = fetch(context_lens, (size_t)num_seqs, stream, ctx, "context_lens");
  if (st == PA_OK) st = fetch(group_members, (size_t)num_groups * kSharedMaxMembers, stream, members, "group_members");
  if (st == PA_OK) st = fetch(group_prefix, (size_t)num_groups, stream, prefix, "group_prefix");
  if (st == PA_OK) st = fetch(seq_starts, (size_t)num_seqs, stream, starts, "seq_starts");
  if (st != PA_OK) return st;
  st = check_tables(tables, ctx, max_blocks, max_context_len, block_size, num_blocks);
  if (st != PA_OK) return st;
  std::vector<int32_t> start_of(num_seqs, 0);
  std::vector<char> grouped(num_seqs, 0);
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t P = prefix[g];
    if (P < 0 || P > max_prefix_len || P % 16 != 0 || P % block_size != 0)
      return bad("group_prefix[" + str(g) + "] = " + str(P) + " is not a multiple of 16 and of block_size in [0, " +
                 str(max_prefix_len) + "]");
    const int32_t *row = &members[(size_t)g * kSharedMaxMembers];
    int32_t first = -1;
    bool padding = false;
    for (int i = 0; i < kSharedMaxMembers; ++i) {
      const int32_t m = row[i];
      if (m == -1) {
        padding = true;
        continue;
      }
      if (padding || m < 0 || m >= num_seqs)
        return bad("group_members[" + str(g) + "][" + str(i) + "] = " + str(m) +
                   ": members are a leading run of sequence ids padded with -1");
      if (grouped[m]) return bad("sequence " + str(m) + " is in more than one group");
      grouped[m] = 1;
      start_of[m] = P;
      if (P > ctx[m])
        return bad("group " + str(g) + ": prefix " + str(P) + " exceeds context_lens[" + str(m) + "] = " + str(ctx[m]));
      if (first < 0) {
        first = m;
        continue;
      }
      for (int32_t b = 0; b < P / block_size; ++b)
        if (tables[(size_t)m * max_blocks + b] != tables[(size_t)first * max_blocks + b])
          return bad("group " + str(g) + ": sequences " + str(first) + " and " + str(m) + " differ at table entry " +
                     str(b) + " inside the shared prefix of " + str(P) + " tokens");
    }
  }
  for (int32_t s = 0; s < num_seqs; ++s)
    if (starts[s] != start_of[s])
      return bad("seq_starts[" + str(s) + "] = " + str(starts[s]) + " but its group's prefix is " + str(start_of[s]));
  return PA_OK;
}

pa_status validate_copy_pairs(const int64_t *block_mapping, int64_t num_pairs, int64_t num_blocks, hipStream_t stream) {
  std::vector<int64_t> map;
  pa_status st = fetch(block_mapping, (size_t)num_pairs * 2, stream, map, "block_mapping");
  if (st != PA_OK) return st;
  std::unordered_set<int64_t> srcs, dsts;
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t s = map[2 * i], d = map[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
      return bad("pair " + str(i) + " (" + str(s) + ", " + str(d) + ") outside [0, " + str(num_blocks) + ")");
    srcs.insert(s);
    if (!dsts.insert(d).second) return bad("destination block " + str(d) + " appears twice (pair " + str(i) + ")");
  }
  for (int64_t d : dsts)
    if (srcs.count(d)) return bad("block " + str(d) + " is both a source and a destination");
  return PA_OK;
}

pa_status validate_swap_pairs(const int64_t *block_mapping, int64_t num_pairs, int64_t src_num_blocks,
                              int64_t dst_num_blocks, hipStream_t stream) {
  std::vector<int64_t> map;
  pa_status st = fetch(block_mapping, (size_t)num_pairs * 2, stream, map, "block_mapping");
  if (st != PA_OK) return st;
  std::unordered_set<int64_t> dsts;
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t s = map[2 * i], d = map[2 * i + 1];
    if (s < 0 || s >= src_num_blocks)
      return bad("pair " + str(i) + ": source block " + str(s) + " outside [0, " + str(src_num_blocks) + ")");
    if (d < 0 || d >= dst_num_blocks)
      return bad("pair " + str(i) + ": destination block " + str(d) + " outside [0, " + str(dst_num_blocks) + ")");
    if (!dsts.insert(d).second) return bad("destination block " + str(d) + " appears twice (pair " + str(i) + ")");
  }
  return PA_OK;
}

pa_status validate_prefill(const int32_t *cu_q_lens, const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *context_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                           int32_t max_context_len, int32_t block_size, int64_t num_blocks, bool append,
                           hipStream_t stream) {
  std::vector<int32_t> cu, tables, ctx;
  pa_status st = fetch(cu_q_lens, (size_t)num_seqs + 1, stream, cu, "cu_q_lens");
  if (st == PA_OK) st = fetch(block_tables, (size_t)num_seqs * max_blocks, stream, tables, "block_tables");
  if (st == PA_OK) st = fetch(context_lens, (size_t)num_seqs, stream, ctx, "context_lens");
  if (st != PA_OK) return st;
  if (cu[0] != 0 || cu[num_seqs] != total_q)
    return bad("cu_q_lens must run from 0 to total_q = " + str(total_q) + " (got " + str(cu[0]) + " .. " +
               str(cu[num_seqs]) + ")");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q_len = cu[s + 1] - cu[s];
    if (q_len < 0 || q_len > max_q_len)
      return bad("sequence " + str(s) + ": q_len " + str(q_len) + " outside [0, max_q_len = " + str(max_q_len) + "]");
    if (q_len > ctx[s])
      return bad("sequence " + str(s) + ": q_len " + str(q_len) + " exceeds context_lens = " + str(ctx[s]) +
                 " (the chunk is part of the context)");
  }
  st = check_tables(tables, ctx, max_blocks, max_context_len, block_size, num_blocks);
  if (st != PA_OK || !append) return st;
  std::vector<int32_t> first(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) first[s] = ctx[s] - (cu[s + 1] - cu[s]);  // the chunk's first position
  return check_writes(tables, ctx, first, max_blocks, block_size);
}

}  // namespace pa
