// Host-side block manager of the paged KV cache: the pool of physical
// blocks, per-sequence block tables, reference counts, copy-on-write.
//
// What it implements (the C declarations in pagedattn.h cite the passages):
// the pool is a fixed set of blocks handed out from a first-in first-out
// queue of free blocks; a sequence maps its logical blocks in order to
// physical ones and takes a new block only when its last one is full; fork
// shares every block of a sequence (one more reference each); appending a
// token to a sequence whose partly filled last block is shared first moves
// that sequence onto a fresh copy of the block (the old block loses one
// reference) and reports the (src, dst) pair so that the caller copies the
// K/V on the device (pa_copy_blocks) before writing the token
// (pa_reshape_and_cache); freeing a sequence drops one reference from each
// of its blocks and queues those that reach zero.
//
// Layout: reference counts in one int32 array over the pool; the free queue
// a ring buffer of block ids (capacity = pool size, so it never overflows);
// each sequence a small vector of block ids plus its token count.  All
// operations are O(blocks touched); a batched append first counts, without
// changing anything, the blocks it will take, so that it either completes
// for every sequence or returns PA_ERR_NO_BLOCKS having changed nothing.

#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <new>
#include <vector>

#include "pa_internal.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t max_blocks_per_seq = 0;
  std::vector<int32_t> refs;         // [num_blocks] references to each block
  std::vector<int32_t> ring;         // free queue: ring[(head + i) % N], i < free_count
  int32_t head = 0;
  int32_t free_count = 0;
  struct Seq {
    bool live = false;
    int32_t length = 0;              // tokens stored
    std::vector<int32_t> blocks;     // logical block -> physical block
  };
  std::vector<Seq> seqs;             // id -> state; ids are never reused
  std::vector<int32_t> pending;      // [num_blocks] scratch of the append dry run
  std::vector<int32_t> touched;

  int32_t take() {
    const int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --free_count;
    refs[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    int64_t tail = (int64_t)head + free_count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++free_count;
  }
  bool live(int32_t id) const { return id >= 0 && id < (int32_t)seqs.size() && seqs[id].live; }
};

namespace {

pa_status bad(const char *what) { return pa::record_error(PA_ERR_INVALID_ARG, what); }

pa_status short_of_blocks(int64_t need, int32_t free_count) {
  char msg[96];
  snprintf(msg, sizeof msg, "need %lld blocks, %d free", (long long)need, free_count);
  return pa::record_error(PA_ERR_NO_BLOCKS, msg);
}

}  // namespace

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t *free_order, pa_block_manager **out) {
  if (!out) return bad("null output pointer");
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0 || max_blocks_per_seq <= 0)
    return bad("num_blocks must be in [1, 2^31), block_size and max_blocks_per_seq positive");
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return bad("max_blocks_per_seq * block_size must fit 31 bits");
  pa_block_manager *bm = new (std::nothrow) pa_block_manager;
  if (!bm) return bad("out of host memory");
  const int32_t n = (int32_t)num_blocks;
  bm->num_blocks = n;
  bm->block_size = block_size;
  bm->max_blocks_per_seq = max_blocks_per_seq;
  bm->refs.assign(n, 0);
  bm->pending.assign(n, 0);
  bm->ring.resize(n);
  if (free_order) {
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= n || seen[b]) {
        delete bm;
        return bad("free_order must list every block id in [0, num_blocks) exactly once");
      }
      seen[b] = 1;
      bm->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < n; ++i) bm->ring[i] = i;
  }
  bm->free_count = n;
  *out = bm;
  return pa::record_ok();
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int64_t pa_bm_num_free(const pa_block_manager *bm) { return bm ? bm->free_count : -1; }

int32_t pa_bm_refcount(const pa_block_manager *bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refs[(size_t)block];
}

pa_status pa_bm_add_sequence(pa_block_manager *bm, int32_t num_tokens, int32_t *seq_id) {
  if (!bm || !seq_id) return bad("null pointer argument");
  if (num_tokens < 0) return bad("num_tokens must be >= 0");
  const int64_t need = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > bm->max_blocks_per_seq) return bad("sequence longer than a block-table row");
  if (need > bm->free_count) return short_of_blocks(need, bm->free_count);
  if (bm->seqs.size() >= (size_t)INT32_MAX) return bad("sequence ids exhausted");
  pa_block_manager::Seq s;
  s.live = true;
  s.length = num_tokens;
  s.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  bm->seqs.push_back(std::move(s));
  *seq_id = (int32_t)bm->seqs.size() - 1;
  return pa::record_ok();
}

pa_status pa_bm_fork(pa_block_manager *bm, int32_t parent, int32_t *child) {
  if (!bm || !child) return bad("null pointer argument");
  if (!bm->live(parent)) return bad("parent is not a live sequence");
  if (bm->seqs.size() >= (size_t)INT32_MAX) return bad("sequence ids exhausted");
  pa_block_manager::Seq s;
  s.live = true;
  s.length = bm->seqs[parent].length;
  s.blocks = bm->seqs[parent].blocks;
  for (int32_t b : s.blocks) ++bm->refs[b];
  bm->seqs.push_back(std::move(s));
  *child = (int32_t)bm->seqs.size() - 1;
  return pa::record_ok();
}

pa_status pa_bm_append_slots(pa_block_manager *bm, const int32_t *seqs, int32_t num_seqs, int64_t *slots,
                             int64_t *copies, int32_t *num_copies) {
  if (!bm || !num_copies) return bad("null pointer argument");
  *num_copies = 0;
  if (num_seqs < 0) return bad("num_seqs must be >= 0");
  if (num_seqs == 0) return pa::record_ok();
  if (!seqs || !slots || !copies) return bad("null pointer argument");
  const int32_t B = bm->block_size;
  // Validate, and count the blocks the batch takes: a sequence whose last
  // block is full takes one; one whose partly filled last block is still
  // shared when its turn comes takes one for the copy (the pending array
  // plays the references the earlier sequences of the batch give up).
  int64_t need = 0;
  pa_status st = PA_OK;
  for (int32_t i = 0; i < num_seqs && st == PA_OK; ++i) {
    const int32_t id = seqs[i];
    if (!bm->live(id)) {
      st = bad("append to a sequence that is not live");
      break;
    }
    pa_block_manager::Seq &s = bm->seqs[id];
    if (s.length / B >= bm->max_blocks_per_seq) {
      st = bad("sequence would outgrow its block-table row");
      break;
    }
    if (s.length % B == 0) {
      ++need;
      continue;
    }
    const int32_t last = s.blocks[s.length / B];
    if (bm->pending[last] == 0) bm->touched.push_back(last);
    if (bm->refs[last] - bm->pending[last] > 1) {
      ++bm->pending[last];
      ++need;
    }
  }
  // Duplicates: a sequence appears at most once per batch.
  if (st == PA_OK) {
    std::vector<int32_t> ids(seqs, seqs + num_seqs);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) st = bad("a sequence may appear once per batch");
  }
  for (int32_t b : bm->touched) bm->pending[b] = 0;
  bm->touched.clear();
  if (st != PA_OK) return st;
  if (need > bm->free_count) return short_of_blocks(need, bm->free_count);

  int32_t nc = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_block_manager::Seq &s = bm->seqs[seqs[i]];
    const int32_t lb = s.length / B, off = s.length % B;
    if (off == 0) {
      s.blocks.push_back(bm->take());
    } else if (bm->refs[s.blocks[lb]] > 1) {
      const int32_t src = s.blocks[lb];
      const int32_t dst = bm->take();
      --bm->refs[src];
      s.blocks[lb] = dst;
      copies[2 * nc] = src;
      copies[2 * nc + 1] = dst;
      ++nc;
    }
    slots[i] = (int64_t)s.blocks[lb] * B + off;
    ++s.length;
  }
  *num_copies = nc;
  return pa::record_ok();
}

pa_status pa_bm_free_sequence(pa_block_manager *bm, int32_t seq) {
  if (!bm) return bad("null pointer argument");
  if (!bm->live(seq)) return bad("sequence is not live");
  pa_block_manager::Seq &s = bm->seqs[seq];
  for (int32_t b : s.blocks)
    if (--bm->refs[b] == 0) bm->give_back(b);
  s.live = false;
  s.length = 0;
  std::vector<int32_t>().swap(s.blocks);
  return pa::record_ok();
}

pa_status pa_bm_sequence(const pa_block_manager *bm, int32_t seq, int32_t *length, int32_t *num_blocks) {
  if (!bm || !length || !num_blocks) return bad("null pointer argument");
  if (!bm->live(seq)) return bad("sequence is not live");
  *length = bm->seqs[seq].length;
  *num_blocks = (int32_t)bm->seqs[seq].blocks.size();
  return pa::record_ok();
}

pa_status pa_bm_block_tables(const pa_block_manager *bm, const int32_t *seqs, int32_t num_seqs,
                             int32_t *tables, int32_t *context_lens) {
  if (!bm) return bad("null pointer argument");
  if (num_seqs < 0) return bad("num_seqs must be >= 0");
  if (num_seqs == 0) return pa::record_ok();
  if (!seqs || !tables || !context_lens) return bad("null pointer argument");
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!bm->live(seqs[i])) return bad("sequence is not live");
  const int32_t M = bm->max_blocks_per_seq;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq &s = bm->seqs[seqs[i]];
    int32_t *row = tables + (int64_t)i * M;
    const int32_t nb = (int32_t)s.blocks.size();
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + nb, row + M, -1);
    context_lens[i] = s.length;
  }
  return pa::record_ok();
}

pa_status pa_bm_slots(const pa_block_manager *bm, int32_t seq, int32_t first, int32_t count, int64_t *slots) {
  if (!bm) return bad("null pointer argument");
  if (!bm->live(seq)) return bad("sequence is not live");
  const pa_block_manager::Seq &s = bm->seqs[seq];
  if (first < 0 || count < 0 || (int64_t)first + count > s.length)
    return bad("positions outside the sequence");
  if (count > 0 && !slots) return bad("null pointer argument");
  const int32_t B = bm->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = first + i;
    slots[i] = (int64_t)s.blocks[p / B] * B + p % B;
  }
  return pa::record_ok();
}

}  // extern "C"
