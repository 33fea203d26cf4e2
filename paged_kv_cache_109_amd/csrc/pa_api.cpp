// C-ABI entry points of libpagedattn: argument checks, partition sizing and
// dispatch to the kernel launchers.  Every check here is on host scalars and
// pointer values; device data is read only in the debug validation
// (PA_DEBUG_VALIDATE=1, pa_validate.cpp).  On any failed check nothing is
// enqueued.
#include "../../include/pagedattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// The last-error record, for the host-side parts in other files.
namespace pa {
pa_status record_error(pa_status st, const char *msg) { return fail(st, "%s", msg); }
pa_status record_ok() { return ok(); }
}  // namespace pa

namespace {

int elt_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

constexpr float kLog2e = 1.4426950408889634f;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (0 when no device is usable).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// Worker waves the workspace must hold for `split_workers` (0 = device default).
int64_t worker_bound(int32_t split_workers) {
  if (split_workers > 0) return split_workers;
  const int cus = device_cus();
  return (int64_t)(cus > 0 ? cus : 1024) * pa::kMaxWavesPerCu;
}

struct DecodeGeometry {
  int32_t ctx_cap;
  int64_t workers;     // worker waves used by the partition pass
  size_t plan_bytes;   // header + per-worker starts
  size_t ws_bytes;     // plan + two fragments per worker
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

DecodeGeometry geometry(int32_t head_dim, int32_t max_context_len, int32_t max_blocks, int32_t block_size,
                        int64_t workers) {
  DecodeGeometry g;
  int64_t cap = max_context_len;
  if (max_blocks >= 0 && (int64_t)max_blocks * block_size < cap) cap = (int64_t)max_blocks * block_size;
  g.ctx_cap = (int32_t)(cap < 0 ? 0 : cap);
  g.workers = workers;
  g.plan_bytes = round_up(((size_t)pa::kPlanHeader + pa::kPlanWords * (size_t)workers) * sizeof(uint32_t), 256);
  g.ws_bytes = g.plan_bytes + (size_t)workers * 2 * ((size_t)head_dim + 2) * sizeof(float);
  return g;
}

// Worker waves a decode call launches: as many as fit on the device at
// once, or split_workers when that is smaller.
int64_t decode_workers(pa_dtype dtype, int32_t head_dim, int32_t block_size, int32_t split_workers) {
  const int64_t fit = (int64_t)device_cus() * pa::decode_waves_per_cu(dtype, head_dim, block_size);
  int64_t w = fit > 0 ? fit : 1;
  if (split_workers > 0 && split_workers < w) w = split_workers;
  return w;
}

pa_status check_decode_common(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, pa_dtype dtype, int32_t split_workers) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d is not one of PA_F32/PA_F16/PA_BF16", dtype);
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG,
                "sizes must be positive (num_seqs >= 0, max_context_len >= 0): num_seqs=%d num_heads=%d "
                "head_dim=%d block_size=%d num_blocks=%lld max_blocks_per_seq=%d max_context_len=%d",
                num_seqs, num_heads, head_dim, block_size, (long long)num_blocks, max_blocks_per_seq,
                max_context_len);
  if (!pa::decode_supported(dtype, head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED, "decode is built for head_dim 64/128 and block_size 4/8/16/32/64 (got %d, %d)",
                head_dim, block_size);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs %d exceeds 65535", num_seqs);
  if (num_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "num_heads %d exceeds 65535", num_heads);
  if (num_seqs > 0 && (!k_cache || !v_cache || !block_tables || !context_lens))
    return fail(PA_ERR_INVALID_ARG, "null cache, block table or context-length pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(PA_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  if (split_workers < 0) return fail(PA_ERR_INVALID_ARG, "split_workers %d must be >= 0", split_workers);
  // Tile indices of the whole batch must fit 31 bits.
  const int64_t cap = std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  if ((int64_t)num_seqs * num_heads * ((cap + pa::kDecodeTile - 1) / pa::kDecodeTile) >= ((int64_t)1 << 31))
    return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_heads * ceil(context/16) must be below 2^31");
  return PA_OK;
}

pa::DecodeArgs decode_args(void *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                           pa_dtype dtype, int64_t num_blocks, float scale, const DecodeGeometry &g,
                           const void *workspace) {
  pa::DecodeArgs a;
  char *ws = reinterpret_cast<char *>(const_cast<void *>(workspace));
  a.out = out;
  a.plan = reinterpret_cast<uint32_t *>(ws);
  a.frags = reinterpret_cast<float *>(ws + g.plan_bytes);
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.block_size = block_size;
  a.ctx_cap = g.ctx_cap;
  a.workers = (int32_t)g.workers;
  a.out_row_words = (int32_t)((int64_t)num_heads * head_dim * elt_bytes(dtype) / 4);
  a.scale_log2 = scale * kLog2e;
  a.reused_blocks = 0;
  a.starts = nullptr;
  a.suffix_out = nullptr;
  a.suffix_row = num_heads * (head_dim + 2);
  a.new_key = nullptr;
  a.new_value = nullptr;
  a.new_key_stride = 0;
  a.new_value_stride = 0;
  return a;
}

pa_status check_workspace(const DecodeGeometry &g, const void *workspace, size_t workspace_bytes) {
  if (!workspace)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required (%lld worker waves)", g.ws_bytes,
                (long long)g.workers);
  if (workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, g.ws_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  return PA_OK;
}

// The address a kernel uses for p: p itself for device memory, the mapped
// device address for pinned host memory; null for anything else (pageable
// host memory, unknown pointers), which a kernel must never touch.
const void *device_address(const void *p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error the failed query left
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return p;
  if (attr.type != hipMemoryTypeHost) return nullptr;
  void *d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void *>(p), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return d;
}


struct SharedGeometry {
  DecodeGeometry dec;
  int32_t chunks;            // piece slots per (group, head)
  int32_t max_prefix_tiles;  // prefixes are clamped to this many tiles
  size_t suffix_off, partials_off, pplan_off, ws_bytes;
};

// The shared-prefix pass splits the prefix tiles into ranges of at least
// kPrefixMinTiles, so a prefix of T tiles meets at most 1 + ceil((T - 1) /
// kPrefixMinTiles) of them: that many piece slots per (group, head).
SharedGeometry shared_geometry(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                               int32_t max_blocks, int32_t block_size, int64_t workers, int32_t num_groups,
                               int32_t max_prefix_len) {
  SharedGeometry g;
  g.dec = geometry(head_dim, max_context_len, max_blocks, block_size, workers);
  const int64_t prefix_tiles = ceil_div(std::max<int32_t>(max_prefix_len, 0), pa::kDecodeTile);
  g.max_prefix_tiles = (int32_t)prefix_tiles;
  g.chunks = (int32_t)(prefix_tiles <= 1 ? 1 : 1 + ceil_div(prefix_tiles - 1, pa::kPrefixMinTiles));
  const size_t row = (size_t)head_dim + 2;
  g.suffix_off = round_up(g.dec.ws_bytes, 256);
  g.partials_off = round_up(g.suffix_off + (size_t)num_seqs * num_heads * row * sizeof(float), 256);
  g.pplan_off = round_up(g.partials_off + (size_t)num_groups * g.chunks * num_heads * pa::kSharedMaxMembers * row *
                                              sizeof(float),
                         256);
  g.ws_bytes = g.pplan_off + ((size_t)pa::kPrefixPlanHeader + 2 * (size_t)num_groups) * sizeof(uint32_t);
  return g;
}

// Worker waves of a shared-prefix call: as many as the pass kernel holds on
// the device at once, or split_workers when that is smaller.
int64_t shared_workers(pa_dtype dtype, int32_t head_dim, int32_t block_size, int32_t split_workers) {
  const int64_t fit = (int64_t)device_cus() * pa::shared_waves_per_cu(dtype, head_dim, block_size);
  int64_t w = fit > 0 ? fit : 1;
  if (split_workers > 0 && split_workers < w) w = split_workers;
  return w;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char *pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failure";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_slot_mapping(const int32_t *block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                          const int32_t *seq_ids, const int32_t *positions, int64_t num_tokens, int32_t block_size,
                          int64_t num_blocks, int64_t *slot_mapping, void *stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_tokens, num_seqs >= 0): num_tokens=%lld "
                "num_seqs=%d max_blocks_per_seq=%d block_size=%d num_blocks=%lld", (long long)num_tokens, num_seqs,
                max_blocks_per_seq, block_size, (long long)num_blocks);
  if (num_tokens == 0) return ok();
  if (!seq_ids || !positions || !slot_mapping || (num_seqs > 0 && !block_tables))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  return hip_status(pa::launch_slot_mapping(block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions,
                                            num_tokens, block_size, num_blocks, slot_mapping,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "slot_mapping");
}

pa_status pa_reshape_and_cache(const void *key, const void *value, int64_t key_token_stride,
                               int64_t value_token_stride, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int64_t num_tokens, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                               void *stream) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d is not one of PA_F32/PA_F16/PA_BF16", dtype);
  if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_tokens >= 0)");
  const int64_t eb = elt_bytes(dtype);
  const int64_t row_bytes = head_dim * eb;
  if (row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "head_dim * element size (%lld bytes) must be a multiple of 16",
                (long long)row_bytes);
  if (row_bytes > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "head_dim too large");
  if (2 * (int64_t)num_heads * (row_bytes / 16) > 65535LL * 256)
    return fail(PA_ERR_UNSUPPORTED, "num_heads * head_dim too large (a token's K and V exceed 65535 * 256 16-byte "
                "chunks)");
  if (key_token_stride < (int64_t)num_heads * head_dim || value_token_stride < (int64_t)num_heads * head_dim)
    return fail(PA_ERR_INVALID_ARG, "token strides (%lld, %lld) smaller than num_heads*head_dim %lld",
                (long long)key_token_stride, (long long)value_token_stride, (long long)num_heads * head_dim);
  if ((key_token_stride * eb) % 16 != 0 || (value_token_stride * eb) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "token strides must be multiples of 16 bytes");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "key, value and caches must be 16-byte aligned");
  if (pa::debug_validate()) {
    const pa_status vs = pa::validate_slots(slot_mapping, num_tokens, num_blocks, block_size,
                                            reinterpret_cast<hipStream_t>(stream));
    if (vs != PA_OK) return vs;
  }
  return hip_status(pa::launch_reshape_and_cache(key, value, key_token_stride * eb, value_token_stride * eb,
                                                 k_cache, v_cache, slot_mapping, num_tokens, num_heads,
                                                 (int32_t)row_bytes, block_size, num_blocks,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    "reshape_and_cache");
}

int32_t pa_decode_default_workers(pa_dtype dtype, int32_t head_dim, int32_t block_size) {
  if (!valid_dtype(dtype) || !pa::decode_supported(dtype, head_dim, block_size)) return 0;
  return (int32_t)decode_workers(dtype, head_dim, block_size, 0);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                                 int32_t block_size, int32_t split_workers) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_context_len < 0 ||
      split_workers < 0)
    return 0;
  return geometry(head_dim, max_context_len, -1, block_size, worker_bound(split_workers)).ws_bytes;
}

// The newest token's rows for the fused append (decode_impl's `app`).
struct AppendRows {
  const void *key, *value;
  int64_t key_stride, value_stride;  // elements between rows (sequences for decode, tokens for prefill)
};

static pa_status decode_impl(bool run_parts, bool run_reduce, void *out, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                             int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float scale, pa_dtype dtype, int32_t split_workers, void *workspace,
                             size_t workspace_bytes, void *stream, const AppendRows *app = nullptr,
                             bool reused_blocks = false) {
  pa_status st = check_decode_common(k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks,
                                     dtype, split_workers);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (num_seqs > 0 && (!out || !q)) return fail(PA_ERR_INVALID_ARG, "null out or q pointer");
  if (!aligned16(out) || !aligned16(q)) return fail(PA_ERR_INVALID_ARG, "out and q must be 16-byte aligned");
  if (app) {
    const int64_t row = (int64_t)num_heads * head_dim;
    if (num_seqs > 0 && (!app->key || !app->value)) return fail(PA_ERR_INVALID_ARG, "null key or value pointer");
    if (!aligned16(app->key) || !aligned16(app->value))
      return fail(PA_ERR_INVALID_ARG, "key and value must be 16-byte aligned");
    if (app->key_stride < row || app->value_stride < row)
      return fail(PA_ERR_INVALID_ARG, "sequence strides (%lld, %lld) smaller than num_heads*head_dim %lld",
                  (long long)app->key_stride, (long long)app->value_stride, (long long)row);
    if ((app->key_stride * elt_bytes(dtype)) % 16 != 0 || (app->value_stride * elt_bytes(dtype)) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "sequence strides must be whole 16-byte units");
  }
  if (num_seqs == 0) return ok();
  const DecodeGeometry g = geometry(head_dim, max_context_len, max_blocks_per_seq, block_size,
                                    decode_workers(dtype, head_dim, block_size, split_workers));
  st = check_workspace(g, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, num_heads, head_dim, block_size, dtype, num_blocks, scale, g, workspace);
  a.reused_blocks = reused_blocks ? 1 : 0;
  if (app) {
    a.new_key = app->key;
    a.new_value = app->value;
    a.new_key_stride = app->key_stride * elt_bytes(dtype);
    a.new_value_stride = app->value_stride * elt_bytes(dtype);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((run_parts || app) && pa::debug_validate()) {
    st = pa::validate_decode(block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs, block_size,
                             num_blocks, app != nullptr, s);
    if (st != PA_OK) return st;
  }
  if (run_parts) {
    st = hip_status(pa::launch_decode_partitions(a, dtype, head_dim, block_size, s), "decode partitions");
    if (st != PA_OK) return st;
  }
  if (run_reduce) {
    st = hip_status(pa::launch_decode_reduce(a, dtype, head_dim, s), "decode reduce");
    if (st != PA_OK) return st;
  }
  return ok();
}

pa_status pa_paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                    int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                    float scale, pa_dtype dtype, int32_t split_workers, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream);
}

pa_status pa_paged_attention_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                       int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       float scale, pa_dtype dtype, int32_t split_workers, uint32_t flags,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  if (flags & ~(uint32_t)PA_DECODE_REUSED_BLOCKS)
    return fail(PA_ERR_INVALID_ARG, "unknown decode flags 0x%x", flags & ~(uint32_t)PA_DECODE_REUSED_BLOCKS);
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream, nullptr,
                     (flags & PA_DECODE_REUSED_BLOCKS) != 0);
}

pa_status pa_paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                                            const int32_t *context_lens, int32_t max_context_len,
                                            int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                            int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                                            int32_t split_workers, void *stream) {
  pa_status st = check_decode_common(k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks,
                                     dtype, split_workers);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return ok();
  const DecodeGeometry g = geometry(head_dim, max_context_len, max_blocks_per_seq, block_size,
                                    decode_workers(dtype, head_dim, block_size, split_workers));
  if (g.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE,
                "decode_noalloc: the call needs %zu bytes of workspace (%lld worker waves, head_dim %d), more than "
                "the fixed %u-byte device array; pass a smaller split_workers or use pa_paged_attention_decode",
                g.ws_bytes, (long long)g.workers, head_dim, (unsigned)PA_NOALLOC_SCRATCH_BYTES);
  void *scratch = nullptr;
  const hipError_t e = pa::noalloc_scratch(&scratch);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "decode_noalloc: device address of the fixed workspace: %s", hipGetErrorString(e));
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, scratch, PA_NOALLOC_SCRATCH_BYTES, stream);
}

pa_status pa_paged_attention_decode_append(void *out, const void *q, const void *key, const void *value,
                                           int64_t key_seq_stride, int64_t value_seq_stride, void *k_cache,
                                           void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                           int32_t num_heads, int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, float scale, pa_dtype dtype, int32_t split_workers,
                                           void *workspace, size_t workspace_bytes, void *stream) {
  const AppendRows app{key, value, key_seq_stride, value_seq_stride};
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream, &app);
}

pa_status pa_paged_attention_decode_append_partitions(
    void *out, const void *q, const void *key, const void *value, int64_t key_seq_stride, int64_t value_seq_stride,
    void *k_cache, void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype, int32_t split_workers, void *workspace,
    size_t workspace_bytes, void *stream) {
  const AppendRows app{key, value, key_seq_stride, value_seq_stride};
  return decode_impl(true, false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream, &app);
}

pa_status pa_paged_attention_decode_append_reduce(
    void *out, const void *q, const void *key, const void *value, int64_t key_seq_stride, int64_t value_seq_stride,
    void *k_cache, void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype, int32_t split_workers, void *workspace,
    size_t workspace_bytes, void *stream) {
  const AppendRows app{key, value, key_seq_stride, value_seq_stride};
  return decode_impl(false, true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream, &app);
}

pa_status pa_paged_attention_decode_partitions(void *out, const void *q, const void *k_cache, const void *v_cache,
                                               const int32_t *block_tables, int32_t max_blocks_per_seq,
                                               const int32_t *context_lens, int32_t max_context_len,
                                               int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                               int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                                               int32_t split_workers, void *workspace, size_t workspace_bytes,
                                               void *stream) {
  return decode_impl(true, false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                     split_workers, workspace, workspace_bytes, stream);
}

pa_status pa_paged_attention_decode_reduce(void *out, const int32_t *context_lens, int32_t max_context_len,
                                           int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_heads,
                                           int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                           int32_t split_workers, const void *workspace, size_t workspace_bytes,
                                           void *stream) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d is not one of PA_F32/PA_F16/PA_BF16", dtype);
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0 || split_workers < 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_seqs, max_context_len, split_workers >= 0)");
  if (!pa::decode_supported(dtype, head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED, "decode is built for head_dim 64/128 and block_size 4/8/16/32/64");
  if (num_seqs > 65535 || num_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs or num_heads exceeds 65535");
  if (num_seqs == 0) return ok();
  const DecodeGeometry g = geometry(head_dim, max_context_len, max_blocks_per_seq, block_size,
                                    decode_workers(dtype, head_dim, block_size, split_workers));
  pa_status st = check_workspace(g, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARG, "null out or context-length pointer");
  if (!aligned16(out)) return fail(PA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const pa::DecodeArgs a = decode_args(out, nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq, context_lens,
                                       num_seqs, num_heads, head_dim, block_size, dtype, 1, 1.f, g, workspace);
  return hip_status(pa::launch_decode_reduce(a, dtype, head_dim, reinterpret_cast<hipStream_t>(stream)),
                    "decode reduce");
}

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t block_size, int32_t num_groups,
                                        int32_t max_prefix_len, int32_t split_workers) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_context_len < 0 ||
      num_groups < 0 || max_prefix_len < 0 || split_workers < 0)
    return 0;
  return shared_geometry(num_seqs, num_heads, head_dim, max_context_len, -1, block_size,
                         worker_bound(split_workers), num_groups, max_prefix_len)
      .ws_bytes;
}

pa_status pa_paged_attention_decode_shared(void *out, const void *q, const void *k_cache, const void *v_cache,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                           int32_t num_heads, int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, float scale, pa_dtype dtype,
                                           const int32_t *group_members, const int32_t *group_prefix,
                                           const int32_t *seq_starts, int32_t num_groups, int32_t max_prefix_len,
                                           int32_t split_workers, int32_t phases, void *workspace,
                                           size_t workspace_bytes, void *stream) {
  pa_status st = check_decode_common(k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                     max_context_len, num_seqs, num_heads, head_dim, block_size, num_blocks,
                                     dtype, split_workers);
  if (st != PA_OK) return st;
  if (!pa::shared_supported(dtype, head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED, "shared-prefix decode is built for block_size 16/32/64 (got %d)", block_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (num_groups < 0 || max_prefix_len < 0)
    return fail(PA_ERR_INVALID_ARG, "num_groups and max_prefix_len must be >= 0");
  if (phases <= 0 || (phases & ~PA_SHARED_ALL) != 0)
    return fail(PA_ERR_INVALID_ARG, "phases must be a non-empty mask of PA_SHARED_OWN/PREFIX/COMBINE");
  if (num_seqs > 0 && (!out || !q || !seq_starts)) return fail(PA_ERR_INVALID_ARG, "null out, q or seq_starts");
  if (num_groups > 0 && (!group_members || !group_prefix))
    return fail(PA_ERR_INVALID_ARG, "null group_members or group_prefix");
  if (!aligned16(out) || !aligned16(q)) return fail(PA_ERR_INVALID_ARG, "out and q must be 16-byte aligned");
  if (num_seqs == 0) return ok();
  const int64_t workers = shared_workers(dtype, head_dim, block_size, split_workers);
  const SharedGeometry g = shared_geometry(num_seqs, num_heads, head_dim, max_context_len, max_blocks_per_seq,
                                           block_size, workers, num_groups, max_prefix_len);
  if (!workspace || workspace_bytes < g.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", g.ws_bytes, workspace_bytes);
  if (!aligned16(workspace)) return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  char *ws = reinterpret_cast<char *>(workspace);
  pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                 num_heads, head_dim, block_size, dtype, num_blocks, scale, g.dec, workspace);
  a.starts = seq_starts;
  a.suffix_out = reinterpret_cast<float *>(ws + g.suffix_off);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (pa::debug_validate()) {
    st = pa::validate_shared(block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs, block_size,
                             num_blocks, group_members, group_prefix, seq_starts, num_groups, max_prefix_len, s);
    if (st != PA_OK) return st;
  }
  pa::SharedArgs sa;
  sa.out = out;
  sa.q = q;
  sa.k_cache = k_cache;
  sa.v_cache = v_cache;
  sa.block_tables = block_tables;
  sa.context_lens = context_lens;
  sa.starts = seq_starts;
  sa.members = group_members;
  sa.prefix = group_prefix;
  sa.partials = reinterpret_cast<float *>(ws + g.partials_off);
  sa.pplan = reinterpret_cast<uint32_t *>(ws + g.pplan_off);
  sa.suffix = a.suffix_out;
  sa.num_blocks = num_blocks;
  sa.num_seqs = num_seqs;
  sa.num_heads = num_heads;
  sa.max_blocks = max_blocks_per_seq;
  sa.num_groups = num_groups;
  sa.chunks = g.chunks;
  sa.max_prefix_tiles = g.max_prefix_tiles;
  sa.ctx_cap = g.dec.ctx_cap;
  sa.suffix_row = a.suffix_row;
  sa.scale_log2 = a.scale_log2;
  const bool own = (phases & PA_SHARED_OWN) != 0, prefix = (phases & PA_SHARED_PREFIX) != 0;
  st = hip_status(pa::launch_shared_pass(a, sa, dtype, head_dim, block_size, own, prefix, s), "shared-prefix pass");
  if (st != PA_OK) return st;
  if (own) {
    st = hip_status(pa::launch_decode_reduce(a, dtype, head_dim, s), "decode reduce");
    if (st != PA_OK) return st;
  }
  if (phases & PA_SHARED_COMBINE)
    return hip_status(pa::launch_shared_combine(sa, dtype, head_dim, s), "shared-prefix combine");
  return ok();
}

pa_status pa_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers,
                         const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes, int64_t num_blocks,
                         void *stream) {
  if (num_layers <= 0 || num_pairs < 0 || block_bytes <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_layers, block_bytes and num_blocks must be positive, num_pairs >= 0");
  if (block_bytes % 16 != 0) return fail(PA_ERR_INVALID_ARG, "block_bytes %lld is not a multiple of 16",
                                         (long long)block_bytes);
  if (num_pairs == 0) return ok();
  if (!k_caches || !v_caches || !block_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return fail(PA_ERR_INVALID_ARG, "layer %d: null cache pointer", l);
    if (!aligned16(k_caches[l]) || !aligned16(v_caches[l]))
      return fail(PA_ERR_INVALID_ARG, "layer %d: caches must be 16-byte aligned", l);
  }
  if (pa::debug_validate()) {
    const pa_status vs =
        pa::validate_copy_pairs(block_mapping, num_pairs, num_blocks, reinterpret_cast<hipStream_t>(stream));
    if (vs != PA_OK) return vs;
  }
  return hip_status(pa::launch_copy_blocks(k_caches, v_caches, num_layers, block_mapping, num_pairs, block_bytes,
                                           num_blocks, reinterpret_cast<hipStream_t>(stream)),
                    "copy_blocks");
}

static pa_status prefill_impl(void *out, const void *q, const int32_t *cu_q_lens, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                              int32_t max_context_len, int32_t num_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, float scale, pa_dtype dtype, void *stream,
                              const AppendRows *app = nullptr) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d is not one of PA_F32/PA_F16/PA_BF16", dtype);
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0 || num_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_seqs, total_q, max_q_len, max_context_len >= 0)");
  if (!pa::prefill_supported(dtype, head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED, "prefill chunk is built for head_dim 64/128 and block_size 4/8/16/32/64 "
                "(got dtype %d, head_dim %d, block_size %d)", dtype, head_dim, block_size);
  if (app && !pa::prefill_append_supported(dtype, head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED, "the fused chunk write runs on the matrix-core kernel: fp16/bf16, head_dim 128 "
                "(got dtype %d, head_dim %d)", dtype, head_dim);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (num_seqs > 65535 || num_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "grid dimension exceeds 65535");
  if (app) {
    const int64_t row = (int64_t)num_heads * head_dim;
    if (app->key_stride < row || app->value_stride < row)
      return fail(PA_ERR_INVALID_ARG, "token strides (%lld, %lld) smaller than num_heads*head_dim %lld",
                  (long long)app->key_stride, (long long)app->value_stride, (long long)row);
    if ((app->key_stride * elt_bytes(dtype)) % 16 != 0 || (app->value_stride * elt_bytes(dtype)) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "token strides must be whole 16-byte units");
  }
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_tables || !context_lens ||
      (app && (!app->key || !app->value)))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (app && (!aligned16(app->key) || !aligned16(app->value))))
    return fail(PA_ERR_INVALID_ARG, "out, q, caches (and key, value) must be 16-byte aligned");
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.cu_q_lens = cu_q_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_blocks = max_blocks_per_seq;
  a.num_heads = num_heads;
  int64_t cap = max_context_len;
  if ((int64_t)max_blocks_per_seq * block_size < cap) cap = (int64_t)max_blocks_per_seq * block_size;
  a.ctx_cap = (int32_t)cap;
  a.scale_log2 = scale * kLog2e;
  a.new_key = app ? app->key : nullptr;
  a.new_value = app ? app->value : nullptr;
  a.new_key_stride = app ? app->key_stride * elt_bytes(dtype) : 0;
  a.new_value_stride = app ? app->value_stride * elt_bytes(dtype) : 0;
  if (pa::debug_validate()) {
    const pa_status vs = pa::validate_prefill(cu_q_lens, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                              total_q, max_q_len, max_context_len, block_size, num_blocks,
                                              app != nullptr, reinterpret_cast<hipStream_t>(stream));
    if (vs != PA_OK) return vs;
  }
  return hip_status(pa::launch_prefill_chunk(a, dtype, head_dim, block_size, reinterpret_cast<hipStream_t>(stream)),
                    "prefill chunk");
}

pa_status pa_paged_attention_prefill_chunk(void *out, const void *q, const int32_t *cu_q_lens, const void *k_cache,
                                           const void *v_cache, const int32_t *block_tables,
                                           int32_t max_blocks_per_seq, const int32_t *context_lens,
                                           int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                           int32_t max_context_len, int32_t num_heads, int32_t head_dim,
                                           int32_t block_size, int64_t num_blocks, float scale, pa_dtype dtype,
                                           void *stream) {
  return prefill_impl(out, q, cu_q_lens, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      total_q, max_q_len, max_context_len, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                      stream);
}

pa_status pa_paged_attention_prefill_chunk_append(void *out, const void *q, const void *key, const void *value,
                                                  int64_t key_token_stride, int64_t value_token_stride,
                                                  const int32_t *cu_q_lens, void *k_cache, void *v_cache,
                                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                                  const int32_t *context_lens, int32_t num_seqs, int32_t total_q,
                                                  int32_t max_q_len, int32_t max_context_len, int32_t num_heads,
                                                  int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                                  float scale, pa_dtype dtype, void *stream) {
  const AppendRows app{key, value, key_token_stride, value_token_stride};
  return prefill_impl(out, q, cu_q_lens, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      total_q, max_q_len, max_context_len, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                      stream, &app);
}

pa_status pa_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                         const int64_t *block_mapping, int64_t num_pairs, int64_t block_bytes,
                         int64_t src_num_blocks, int64_t dst_num_blocks, void *stream) {
  if (num_caches <= 0 || num_pairs < 0 || block_bytes <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_caches, block_bytes and both pool sizes must be positive, num_pairs >= 0");
  if (block_bytes % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "block_bytes %lld is not a multiple of 16", (long long)block_bytes);
  if (num_pairs == 0) return ok();
  if (!src_caches || !dst_caches || !block_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const int64_t *mapping = static_cast<const int64_t *>(device_address(block_mapping));
  if (!mapping) return fail(PA_ERR_INVALID_ARG, "block_mapping must be device memory or pinned host memory");
  std::vector<const void *> src(num_caches);
  std::vector<void *> dst(num_caches);
  for (int32_t c = 0; c < num_caches; ++c) {
    if (!src_caches[c] || !dst_caches[c]) return fail(PA_ERR_INVALID_ARG, "cache %d: null pointer", c);
    if (!aligned16(src_caches[c]) || !aligned16(dst_caches[c]))
      return fail(PA_ERR_INVALID_ARG, "cache %d: caches must be 16-byte aligned", c);
    src[c] = device_address(src_caches[c]);
    dst[c] = const_cast<void *>(device_address(dst_caches[c]));
    if (!src[c] || !dst[c])
      return fail(PA_ERR_INVALID_ARG, "cache %d: caches must be device memory or pinned host memory", c);
  }
  if (pa::debug_validate()) {
    const pa_status vs = pa::validate_swap_pairs(block_mapping, num_pairs, src_num_blocks, dst_num_blocks,
                                                 reinterpret_cast<hipStream_t>(stream));
    if (vs != PA_OK) return vs;
  }
  return hip_status(pa::launch_swap_blocks(src.data(), dst.data(), num_caches, mapping, num_pairs, block_bytes,
                                           src_num_blocks, dst_num_blocks, reinterpret_cast<hipStream_t>(stream)),
                    "swap_blocks");
}

pa_status pa_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups, void *stream) {
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (bytes <= 0 || bytes % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "bytes %lld is not a positive multiple of 16", (long long)bytes);
  if (workgroups <= 0) return fail(PA_ERR_INVALID_ARG, "workgroups must be positive");
  if (!aligned16(src) || !aligned16(sink)) return fail(PA_ERR_INVALID_ARG, "src and sink must be 16-byte aligned");
  return hip_status(pa::launch_stream_read(src, bytes, sink, workgroups, reinterpret_cast<hipStream_t>(stream)),
                    "stream read");
}

}  // extern "C"
