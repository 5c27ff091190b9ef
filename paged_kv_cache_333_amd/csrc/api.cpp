// C ABI for the device operations: argument validation, the optional
// PA_DEBUG checks of device-side indices, and dispatch to the kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "launch.hpp"
#include "slot_blocks.hpp"
#include "status.hpp"

namespace pa {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev{nullptr, nullptr};
  return ev;
}
}  // namespace pa

namespace {

using pa::fail;

bool debug_mode() {
  static const bool on = [] {
    const char* v = std::getenv("PA_DEBUG");
    return v && std::strcmp(v, "0") != 0 && v[0] != '\0';
  }();
  return on;
}

int elem_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : dt == PA_F16 || dt == PA_BF16 ? 2 : 1; }

bool is_code_type(pa_dtype dt) { return dt == PA_FP8_E4M3 || dt == PA_INT8 || dt == PA_INT8_TOKEN; }

// Bytes of one (block, KV head) tile of a pool of element type dt: its
// elements, then (PA_INT8_TOKEN) a scale area of whole 128-byte lines.
int64_t tile_bytes(pa_dtype dt, int32_t head_dim, int32_t block_size) {
  return static_cast<int64_t>(block_size) * head_dim * elem_bytes(dt) +
         (dt == PA_INT8_TOKEN ? (static_cast<int64_t>(block_size) * 4 + 127) / 128 * 128 : 0);
}

pa_status check_scales(float k_scale, float v_scale) {
  // finite and positive (NaN fails the comparisons)
  if (!(k_scale > 0.0f && k_scale <= 3.4028235e38f) || !(v_scale > 0.0f && v_scale <= 3.4028235e38f))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Form of pa_upload_and_cache's write when every token has a block of its
// own.  The whole-tile form rewrites each written value tile in full lines
// instead of one element per dim row.  What decides is the bytes of one dim
// row of a value tile (block_size * element bytes), measured on full decode
// steps:
//   64 bytes: tiles (16-bit, 32-token blocks: GQA bf16 step 216 -> 200 us, the
//     decode after it running at its clean-cache speed; 8-bit, 64-token blocks:
//     int8 GQA 132.5 -> 117.9 us, FP8 130.7 -> 127.9 us);
//   32 bytes of codes: tiles (8-bit, 32-token blocks: int8 GQA 130 -> 123 us);
//   32 bytes of 16-bit elements, 16 bytes: the same either way (the time the
//     shorter write saves reappears in the decode), so the element-wise form
//     stays, with non-temporal stores for model-type pools (see put in
//     cache_ops.hip);
//   128 bytes (16-bit, 64-token blocks): the element-wise form (tiles made the
//     LLaMA-7B-like step 219 -> 248 us).
// PA_TILE_WRITE=always / never overrides the rule (read on every call); the
// whole-tile form is never used when two tokens share a block.
bool tile_write_wanted(int32_t block_size, int32_t elem_bytes) {
  const char* v = std::getenv("PA_TILE_WRITE");
  if (v && std::strcmp(v, "always") == 0) return true;
  if (v && std::strcmp(v, "never") == 0) return false;
  const int32_t row = block_size * elem_bytes;
  return row == 64 || (elem_bytes == 1 && row == 32);
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

pa_status check_shape(pa_dtype dt, int32_t head_dim, int32_t block_size) {
  if (dt != PA_F32 && dt != PA_F16 && dt != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype");
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size != 16 && block_size != 32 && !(head_dim == 128 && (block_size == 8 || block_size == 64)))
    return fail(PA_ERR_UNSUPPORTED, "block_size must be 16 or 32, or 8 or 64 with head_dim 128");
  return PA_OK;
}

// A decode step over 8-bit codes spans 64 tokens, at most four blocks: no 8-token blocks.
pa_status check_code_block(pa_dtype kv_dtype, int32_t block_size) {
  if (is_code_type(kv_dtype) && block_size == 8)
    return fail(PA_ERR_UNSUPPORTED, "8-bit pools need block_size 16, 32 or 64");
  return PA_OK;
}

// After a launch: report launch errors; in debug mode also wait and report
// execution errors.
pa_status finish(hipError_t launch, hipStream_t st, const char* what) {
  pa::launch_events() = pa::LaunchEvents{nullptr, nullptr};  // they applied to this call only
  if (launch != hipSuccess) return hip_fail(launch, what);
  if (debug_mode()) {
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return PA_OK;
}

template <typename T>
pa_status fetch(std::vector<T>& host, const T* dev, size_t n, hipStream_t st) {
  host.resize(n);
  if (n == 0) return PA_OK;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "PA_DEBUG copy-back");
  return PA_OK;
}

pa_status check_decode_args(const pa::DecodeArgs& a) {
  pa_status s = check_shape(a.dtype, a.head_dim, a.block_size);
  if (s != PA_OK) return s;
  if ((s = check_code_block(a.kv_dtype, a.block_size)) != PA_OK) return s;
  if (a.num_seqs < 0 || a.num_heads <= 0 || a.num_kv_heads <= 0 || a.max_blocks_per_seq < 0 ||
      a.num_blocks < 0 || a.max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if (a.num_heads % a.num_kv_heads) return fail(PA_ERR_INVALID_ARG, "num_heads % num_kv_heads != 0");
  if (a.num_seqs == 0) return PA_OK;
  if (!a.out || !a.query || !a.key_cache || !a.value_cache || !a.block_tables || !a.context_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(a.out) || !aligned16(a.query) || !aligned16(a.key_cache) || !aligned16(a.value_cache))
    return fail(PA_ERR_INVALID_ARG, "query, out and the pools must be 16-byte aligned");
  if (static_cast<int64_t>(a.num_seqs) * a.num_heads > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_seqs * num_heads too large");
  return PA_OK;
}

int64_t len_limit(const pa::DecodeArgs& a) {
  const int64_t cap = static_cast<int64_t>(a.max_blocks_per_seq) * a.block_size;
  return cap < a.max_context_len ? cap : a.max_context_len;
}

pa_status debug_check_tables(const pa::DecodeArgs& a, hipStream_t st) {
  std::vector<int32_t> ctx, tab;
  pa_status s = fetch(ctx, a.context_lens, a.num_seqs, st);
  if (s == PA_OK) s = fetch(tab, a.block_tables, static_cast<size_t>(a.num_seqs) * a.max_blocks_per_seq, st);
  if (s != PA_OK) return s;
  std::vector<int32_t> mlo, mhi;  // masked positions: blocks wholly inside are never read
  if (a.mask_lo) {
    if ((s = fetch(mlo, a.mask_lo, a.num_seqs, st)) != PA_OK) return s;
    if ((s = fetch(mhi, a.mask_hi, a.num_seqs, st)) != PA_OK) return s;
  }
  const int64_t lim = len_limit(a);
  for (int32_t i = 0; i < a.num_seqs; ++i) {
    if (ctx[i] < 0 || ctx[i] > lim)
      return fail(PA_ERR_BAD_TABLE, "context_lens[" + std::to_string(i) + "] = " + std::to_string(ctx[i]) +
                                        " outside [0, " + std::to_string(lim) + "]");
    const int32_t nb = (ctx[i] + a.block_size - 1) / a.block_size;
    for (int32_t j = 0; j < nb; ++j) {
      if (a.mask_lo && mlo[i] < mhi[i]) {
        const int64_t first = static_cast<int64_t>(j) * a.block_size;
        const int64_t stop = std::min<int64_t>(first + a.block_size, ctx[i]);
        if (first >= mlo[i] && stop <= mhi[i]) continue;
      }
      const int32_t b = tab[static_cast<size_t>(i) * a.max_blocks_per_seq + j];
      if (b < 0 || b >= a.num_blocks)
        return fail(PA_ERR_BAD_TABLE, "block_tables[" + std::to_string(i) + "][" + std::to_string(j) +
                                          "] = " + std::to_string(b) + " outside the pool");
    }
  }
  if (a.seq_order) {
    std::vector<int32_t> ord;
    if ((s = fetch(ord, a.seq_order, a.num_seqs, st)) != PA_OK) return s;
    std::vector<char> seen(a.num_seqs, 0);
    for (int32_t i = 0; i < a.num_seqs; ++i) {
      if (ord[i] < 0 || ord[i] >= a.num_seqs || seen[ord[i]])
        return fail(PA_ERR_BAD_TABLE, "seq_order is not a permutation of 0..num_seqs-1");
      seen[ord[i]] = 1;
    }
  }
  return PA_OK;
}

pa_status debug_check_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                            int32_t block_size, hipStream_t st) {
  std::vector<int32_t> slots;
  pa_status s = fetch(slots, slot_mapping, num_tokens, st);
  if (s != PA_OK) return s;
  const int64_t nslots = static_cast<int64_t>(num_blocks) * block_size;
  std::unordered_set<int32_t> seen;
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (slots[i] < 0) continue;
    if (slots[i] >= nslots) return fail(PA_ERR_BAD_TABLE, "slot_mapping[" + std::to_string(i) + "] past the pool");
    if (!seen.insert(slots[i]).second)
      return fail(PA_ERR_BAD_TABLE, "slot " + std::to_string(slots[i]) + " written twice");
  }
  return PA_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct SplitSizes {
  int64_t off_l, off_o, total;
  int32_t parts;
};

// Launch shape of the single pass (max_query_len 0) or of the several-token
// pass: workgroups per sequence and workgroups the device holds at once.  The
// occupancy query behind it costs host time on every decode call, so the
// answer is kept per (device, dtypes, head_dim, block_size, heads, group,
// max_query_len).
hipError_t launch_shape(const pa::DecodeArgs& a, int32_t max_query_len, int64_t* workgroups, int64_t* resident) {
  struct Entry {
    int64_t key[8];
    int64_t per_seq, resident;
  };
  static std::mutex mu;
  static std::vector<Entry> memo;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int64_t key[8] = {dev, a.dtype, a.kv_dtype, a.head_dim, a.block_size, a.num_heads, a.num_kv_heads,
                          max_query_len};
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& en : memo)
      if (std::equal(key, key + 8, en.key)) {
        *workgroups = en.per_seq * a.num_seqs;
        *resident = en.resident;
        return hipSuccess;
      }
  }
  pa::DecodeArgs one = a;
  one.num_seqs = 1;
  int64_t per_seq = 0, res = 0;
  e = max_query_len > 0 ? pa::multi_pass_shape(one, max_query_len, &per_seq, &res)
                        : pa::single_pass_shape(one, &per_seq, &res);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    Entry en{};
    std::copy(key, key + 8, en.key);
    en.per_seq = per_seq;
    en.resident = res;
    if (memo.size() < 256) memo.push_back(en);
  }
  *workgroups = per_seq * a.num_seqs;
  *resident = res;
  return hipSuccess;
}

bool split_sizes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                 int32_t partition_size, SplitSizes* out) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_size <= 0)
    return false;
  const int64_t parts = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
  if (parts > 65535) return false;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_heads * parts;
  out->parts = static_cast<int32_t>(parts);
  out->off_l = align256(units * 4);
  out->off_o = out->off_l + align256(units * 4);
  out->total = out->off_o + units * head_dim * 4;
  return true;
}

pa_status make_layout(void* workspace, size_t workspace_bytes, int32_t num_seqs, int32_t num_heads,
                      int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                      pa::SplitLayout* ws) {
  SplitSizes z;
  if (!split_sizes(num_seqs, num_heads, head_dim, max_context_len, partition_size, &z))
    return fail(PA_ERR_INVALID_ARG, "split sizes (at most 65535 partitions)");
  if (static_cast<int64_t>(workspace_bytes) < z.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "need " + std::to_string(z.total) + " bytes, got " + std::to_string(workspace_bytes));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(PA_ERR_INVALID_ARG, "workspace must be non-null and 256-byte aligned");
  char* base = static_cast<char*>(workspace);
  ws->m = reinterpret_cast<float*>(base);
  ws->l = reinterpret_cast<float*>(base + z.off_l);
  ws->o = reinterpret_cast<float*>(base + z.off_o);
  ws->partition_size = partition_size;
  ws->num_parts = z.parts;
  return PA_OK;
}

// The pa_decode_auto rule: split only when the single pass could not fill the
// device (fewer workgroups than it holds at once, so compute units would sit
// idle while a few workgroups walk very long contexts), the context spans at
// least four partitions and the workspace is large enough.
// PA_SPLIT=never / always overrides the automatic path choice (always: when
// the workspace and partition size allow a split); unset or anything else:
// the rule.  Read on every call, so a process can change it between calls.
int split_override() {
  const char* v = std::getenv("PA_SPLIT");
  if (!v) return 0;
  if (std::strcmp(v, "never") == 0) return -1;
  if (std::strcmp(v, "always") == 0) return 1;
  return 0;
}

bool choose_split(const pa::DecodeArgs& a, int32_t partition_size, const void* workspace, size_t workspace_bytes) {
  const int force = split_override();
  if (force < 0 || !workspace || a.num_seqs <= 0 || partition_size <= 0 || partition_size % a.block_size ||
      partition_size > 4096)
    return false;
  SplitSizes z;
  if (!split_sizes(a.num_seqs, a.num_heads, a.head_dim, a.max_context_len, partition_size, &z) ||
      static_cast<int64_t>(workspace_bytes) < z.total)
    return false;
  if (force > 0) return true;
  if (a.max_context_len < 4 * static_cast<int64_t>(partition_size)) return false;
  int64_t workgroups = 0, resident = 0;
  const bool ok = launch_shape(a, 0, &workgroups, &resident) == hipSuccess;
  (void)hipGetLastError();
  return ok && workgroups < resident;
}

pa::DecodeArgs pack(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                    int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
                    pa_dtype dtype, uint32_t flags) {
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                   num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                   max_context_len, scale, dtype, flags};
  a.kv_dtype = dtype;
  return a;
}

}  // namespace

extern "C" {

pa_status pa_set_launch_events(void* start_event, void* stop_event) {
  pa::launch_events() = pa::LaunchEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return PA_OK;
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                               void* stream) {
  pa_status s = check_shape(dtype, head_dim, block_size);
  if (s != PA_OK) return s;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_slots(slot_mapping, num_tokens, num_blocks, block_size, st)) != PA_OK)
    return s;
  return finish(pa::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                             num_blocks, num_kv_heads, head_dim, elem_bytes(dtype),
                                             block_size, st),
                st, "pa_reshape_and_cache");
}

pa_status pa_reshape_and_cache_quant(const void* key, const void* value, void* key_cache, void* value_cache,
                                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                     pa_dtype kv_dtype, float k_scale, float v_scale, void* stream) {
  pa_status s = check_shape(dtype, head_dim, block_size);
  if (s != PA_OK) return s;
  if (!is_code_type(kv_dtype)) return fail(PA_ERR_UNSUPPORTED, "kv_dtype must be an 8-bit code type");
  if ((s = check_code_block(kv_dtype, block_size)) != PA_OK) return s;
  if (kv_dtype != PA_INT8_TOKEN && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_slots(slot_mapping, num_tokens, num_blocks, block_size, st)) != PA_OK)
    return s;
  if (kv_dtype == PA_INT8_TOKEN)
    return finish(pa::launch_reshape_and_cache_rows(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                                    num_blocks, num_kv_heads, head_dim, block_size, dtype, st),
                  st, "pa_reshape_and_cache_quant");
  return finish(pa::launch_reshape_and_cache_quant(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                                   num_blocks, num_kv_heads, head_dim, block_size, dtype, kv_dtype,
                                                   k_scale, v_scale, st),
                st, "pa_reshape_and_cache_quant");
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void* stream) {
  pa_status s = check_shape(is_code_type(dtype) ? PA_F16 : dtype, head_dim, block_size);
  if (s != PA_OK) return s;
  if (num_pairs < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !pairs) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    std::vector<int32_t> pr;
    s = fetch(pr, pairs, static_cast<size_t>(num_pairs) * 2, st);
    if (s != PA_OK) return s;
    std::unordered_set<int32_t> dsts, srcs;
    for (int32_t p = 0; p < num_pairs; ++p) {
      const int32_t a = pr[2 * p], b = pr[2 * p + 1];
      if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks)
        return fail(PA_ERR_BAD_TABLE, "copy pair " + std::to_string(p) + " outside the pool");
      if (!dsts.insert(b).second) return fail(PA_ERR_BAD_TABLE, "two copies into one block");
      srcs.insert(a);
    }
    for (int32_t b : dsts)
      if (srcs.count(b)) return fail(PA_ERR_BAD_TABLE, "a copy destination is also a source");
  }
  const int64_t block_bytes = num_kv_heads * tile_bytes(dtype, head_dim, block_size);
  return finish(pa::launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, num_blocks, block_bytes, st),
                st, "pa_copy_blocks");
}

namespace {
// Device view of a buffer for a kernel: device memory as it is, page-locked
// host memory through its mapping.  kind: 0 device, 1 host; -1 if neither.
static int device_view(const void* p, const void** view) {
  hipPointerAttribute_t at{};
  const bool ok = hipPointerGetAttributes(&at, p) == hipSuccess;
  (void)hipGetLastError();
  if (!ok) return -1;
  if (at.type == hipMemoryTypeDevice) {
    *view = p;
    return 0;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    *view = at.devicePointer;
    return 1;
  }
  return -1;
}
}  // namespace

pa_status pa_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                         const void* src_value_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_src_blocks, int32_t num_dst_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void* stream) {
  pa_status s = check_shape(is_code_type(dtype) ? PA_F16 : dtype, head_dim, block_size);
  if (s != PA_OK) return s;
  if (num_pairs < 0 || num_src_blocks < 0 || num_dst_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if (num_pairs == 0) return PA_OK;
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !pairs)
    return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(dst_key_cache) || !aligned16(dst_value_cache) || !aligned16(src_key_cache) ||
      !aligned16(src_value_cache))
    return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const void *dk = nullptr, *dv = nullptr, *sk = nullptr, *sv = nullptr, *pv = nullptr;
  const int kdk = device_view(dst_key_cache, &dk), kdv = device_view(dst_value_cache, &dv);
  const int ksk = device_view(src_key_cache, &sk), ksv = device_view(src_value_cache, &sv);
  const int kp = device_view(pairs, &pv);
  if (kdk < 0 || kdv < 0 || ksk < 0 || ksv < 0 || kp < 0)
    return fail(PA_ERR_INVALID_ARG, "pools and pairs must be device memory or page-locked host memory");
  if (kdk != kdv || ksk != ksv) return fail(PA_ERR_INVALID_ARG, "K and V pools of one side must live together");
  const int64_t block_bytes = num_kv_heads * tile_bytes(dtype, head_dim, block_size);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(pa::launch_swap_blocks(const_cast<void*>(dk), const_cast<void*>(dv), sk, sv,
                                       static_cast<const int32_t*>(pv), num_pairs, num_src_blocks, num_dst_blocks,
                                       block_bytes, ksk == 1, st),
                st, "pa_swap_blocks");
}

pa_status pa_upload(void* dst, const void* src, size_t nbytes, void* stream) {
  if (nbytes == 0) return PA_OK;
  if (!dst || !src) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if ((nbytes & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u) || (reinterpret_cast<uintptr_t>(src) & 3u))
    return fail(PA_ERR_INVALID_ARG, "pa_upload moves whole 4-byte words: pointers and nbytes must be 4-aligned");
  // The kernel dereferences the source from the GPU, so both ends of the range
  // must lie in page-locked host memory mapped for the device, contiguously.
  hipPointerAttribute_t first{}, last{}, d{};
  const char* end = static_cast<const char*>(src) + nbytes - 1;
  const bool ok_first = hipPointerGetAttributes(&first, src) == hipSuccess;
  const bool ok_last = ok_first && hipPointerGetAttributes(&last, end) == hipSuccess;
  const bool ok_dst = hipPointerGetAttributes(&d, dst) == hipSuccess;
  (void)hipGetLastError();  // a failed query must not surface as a later launch error
  if (!ok_first || !ok_last || first.type != hipMemoryTypeHost || last.type != hipMemoryTypeHost ||
      !first.devicePointer ||
      static_cast<const char*>(last.devicePointer) - static_cast<const char*>(first.devicePointer) !=
          static_cast<ptrdiff_t>(nbytes - 1))
    return fail(PA_ERR_INVALID_ARG, "pa_upload: src must be page-locked host memory mapped for the device");
  if (!ok_dst || d.type != hipMemoryTypeDevice)
    return fail(PA_ERR_INVALID_ARG, "pa_upload: dst must be device memory");
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(pa::launch_upload(dst, first.devicePointer, static_cast<int64_t>(nbytes), st), st, "pa_upload");
}

pa_status pa_upload_and_cache(void* dst, const void* src, size_t nbytes, const void* key, const void* value,
                              void* key_cache, void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float k_scale, float v_scale, pa_dtype dtype, pa_dtype kv_dtype, void* stream) {
  pa_status s = check_shape(dtype, head_dim, block_size);
  if (s != PA_OK) return s;
  if ((s = check_code_block(kv_dtype, block_size)) != PA_OK) return s;
  const bool quant = is_code_type(kv_dtype);
  if (kv_dtype == PA_INT8_TOKEN)
    return fail(PA_ERR_UNSUPPORTED, "per-row int8 pools are written by pa_reshape_and_cache_quant");
  if (!quant && kv_dtype != dtype)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype must equal dtype, or be an 8-bit code type");
  if (quant && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or zero heads");
  if ((nbytes & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u) || (reinterpret_cast<uintptr_t>(src) & 3u))
    return fail(PA_ERR_INVALID_ARG, "the upload moves whole 4-byte words: pointers and nbytes must be 4-aligned");
  if (nbytes == 0 && num_tokens == 0) return PA_OK;
  const void* src_view = nullptr;
  const void* slots_view = nullptr;
  const void* dst_view = nullptr;
  if (nbytes > 0) {
    if (!dst || !src) return fail(PA_ERR_INVALID_ARG, "null pointer");
    const void* last_view = nullptr;
    if (device_view(src, &src_view) != 1 ||
        device_view(static_cast<const char*>(src) + nbytes - 1, &last_view) != 1 ||
        static_cast<const char*>(last_view) - static_cast<const char*>(src_view) !=
            static_cast<ptrdiff_t>(nbytes - 1))
      return fail(PA_ERR_INVALID_ARG, "src must be page-locked host memory mapped for the device");
    if (device_view(dst, &dst_view) != 0) return fail(PA_ERR_INVALID_ARG, "dst must be device memory");
  }
  if (num_tokens > 0) {
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
      return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
      return fail(PA_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    if (device_view(slot_mapping, &slots_view) != 1)
      return fail(PA_ERR_INVALID_ARG, "slot_mapping must be page-locked host memory");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // when every token has a block of its own (a decode step appending one token per sequence): the
  // whole-tile write, or the element-wise one with non-temporal stores (model-type pools only: the
  // quantising write's one-byte non-temporal stores made the FP8 step slower, 125 -> 130 us); else
  // plain element-wise stores
  const bool own_blocks = num_tokens > 0 && pa::one_token_per_block(slot_mapping, num_tokens, num_blocks, block_size);
  const int32_t elem = quant ? 1 : dtype == PA_F32 ? 4 : 2;
  const int32_t form = !own_blocks ? 0 : tile_write_wanted(block_size, elem) ? 2 : quant ? 0 : 1;
  return finish(pa::launch_upload_and_cache(dst, src_view, static_cast<int64_t>(nbytes), key, value, key_cache,
                                            value_cache, static_cast<const int32_t*>(slots_view), num_tokens,
                                            num_blocks, num_kv_heads, head_dim, block_size, dtype, kv_dtype,
                                            k_scale, v_scale, form, slot_mapping, st),
                st, "pa_upload_and_cache");
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                    int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
                    pa_dtype dtype, uint32_t flags, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  pa_status s = check_decode_args(a);
  if (s != PA_OK || num_seqs == 0) return s;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV)) return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_tables(a, st)) != PA_OK) return s;
  return finish(pa::launch_decode(a, st), st, "pa_decode");
}

size_t pa_decode_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size) {
  SplitSizes z;
  if (!split_sizes(num_seqs, num_heads, head_dim, max_context_len, partition_size, &z)) return 0;
  return static_cast<size_t>(z.total);
}

pa_status pa_decode_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                          int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                          float scale, pa_dtype dtype, uint32_t flags, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV)) return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  if (partition_size <= 0 || partition_size % block_size || partition_size > 4096)
    return fail(PA_ERR_INVALID_ARG, "partition_size must be a multiple of block_size, at most 4096");
  if (num_seqs == 0) return PA_OK;
  pa::SplitLayout ws;
  s = make_layout(workspace, workspace_bytes, num_seqs, num_heads, head_dim, max_context_len,
                  partition_size, &ws);
  if (s != PA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_tables(a, st)) != PA_OK) return s;
  return finish(pa::launch_decode_split(a, ws, st), st, "pa_decode_split");
}

pa_status pa_decode_split_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                                 int32_t partition_size, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV)) return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  if (partition_size <= 0 || partition_size % block_size || partition_size > 4096)
    return fail(PA_ERR_INVALID_ARG, "partition_size must be a multiple of block_size, at most 4096");
  if (num_seqs == 0) return PA_OK;
  SplitSizes z;
  if (!split_sizes(num_seqs, num_heads, head_dim, max_context_len, partition_size, &z))
    return fail(PA_ERR_INVALID_ARG, "split sizes (at most 65535 partitions)");
  if (z.total > static_cast<int64_t>(PA_STATIC_SCRATCH_BYTES))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "the partials need " + std::to_string(z.total) + " bytes, the static workspace holds " +
                    std::to_string(static_cast<int64_t>(PA_STATIC_SCRATCH_BYTES)) +
                    "; pass a workspace to pa_decode_split instead");
  void* scratch = nullptr;
  hipError_t e = pa::static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "pa_decode_split_static: static workspace lookup");
  pa::SplitLayout ws;
  s = make_layout(scratch, PA_STATIC_SCRATCH_BYTES, num_seqs, num_heads, head_dim, max_context_len, partition_size,
                  &ws);
  if (s != PA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_tables(a, st)) != PA_OK) return s;
  return finish(pa::launch_decode_split(a, ws, st), st, "pa_decode_split_static");
}

pa_status pa_decode_auto(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                         int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                         int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* path,
                         void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  const bool split = choose_split(a, partition_size, workspace, workspace_bytes);
  if (path) *path = split ? 1 : 0;
  if (split)
    return pa_decode_split(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                           num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                           max_context_len, scale, dtype, flags, partition_size, workspace, workspace_bytes,
                           stream);
  return pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs, num_heads,
                   num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                   dtype, flags, stream);
}

pa_status pa_decode_append(void* out, const void* query, const void* key, const void* value,
                           const int32_t* slot_mapping, void* key_cache, void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                           int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* path,
                           void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV)) return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  if (num_seqs == 0) {
    if (path) *path = 0;
    return PA_OK;
  }
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(key) || !aligned16(value)) return fail(PA_ERR_INVALID_ARG, "key and value must be 16-byte aligned");
  const bool split = choose_split(a, partition_size, workspace, workspace_bytes);
  if (path) *path = split ? 1 : 0;
  pa::SplitLayout ws;
  if (split && (s = make_layout(workspace, workspace_bytes, num_seqs, num_heads, head_dim, max_context_len,
                                partition_size, &ws)) != PA_OK)
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    if ((s = debug_check_slots(slot_mapping, num_seqs, num_blocks, block_size, st)) != PA_OK) return s;
    if ((s = debug_check_tables(a, st)) != PA_OK) return s;
  }
  return finish(pa::launch_decode_append(a, key, value, slot_mapping, split ? &ws : nullptr, st), st,
                "pa_decode_append");
}

pa_status pa_decode_masked(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* mask_lo,
                           const int32_t* mask_hi, const int32_t* seq_order, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t max_context_len, float scale, float k_scale, float v_scale,
                           pa_dtype dtype, pa_dtype kv_dtype, uint32_t flags, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, int32_t* path, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  a.kv_dtype = kv_dtype;
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (is_code_type(kv_dtype)) {
    if (dtype != PA_F16 && dtype != PA_BF16)
      return fail(PA_ERR_UNSUPPORTED, "8-bit pools decode with PA_F16 or PA_BF16 queries");
    if (kv_dtype != PA_INT8_TOKEN && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
    a.k_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : k_scale;  // per-row scales come from the pools
    a.v_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : v_scale;
  } else if (kv_dtype != dtype) {
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype must equal dtype, or be an 8-bit code type");
  }
  if ((mask_lo == nullptr) != (mask_hi == nullptr))
    return fail(PA_ERR_INVALID_ARG, "mask_lo and mask_hi must both be given or both be NULL");
  a.mask_lo = mask_lo;
  a.mask_hi = mask_hi;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV | PA_DECODE_SPLIT))
    return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  a.flags = flags & PA_DECODE_CACHED_KV;
  bool split = false;
  if (flags & PA_DECODE_SPLIT) {
    if (partition_size <= 0 || partition_size % block_size || partition_size > 4096)
      return fail(PA_ERR_INVALID_ARG, "partition_size must be a multiple of block_size, at most 4096");
    split = true;
  } else {
    split = choose_split(a, partition_size, workspace, workspace_bytes);
  }
  if (path) *path = split ? 1 : 0;
  if (num_seqs == 0) return PA_OK;
  pa::SplitLayout ws;
  if (split && (s = make_layout(workspace, workspace_bytes, num_seqs, num_heads, head_dim, max_context_len,
                                partition_size, &ws)) != PA_OK)
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_tables(a, st)) != PA_OK) return s;
  return finish(split ? pa::launch_decode_split(a, ws, st) : pa::launch_decode(a, st), st, "pa_decode_masked");
}

size_t pa_decode_multi_workspace_bytes(int32_t num_query_tokens, int32_t num_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size) {
  SplitSizes z;
  if (!split_sizes(num_query_tokens, num_heads, head_dim, max_context_len, partition_size, &z)) return 0;
  return static_cast<size_t>(align256(z.total) + static_cast<int64_t>(num_query_tokens) * 4);
}

pa_status pa_decode_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                          const int32_t* seq_order, int32_t num_seqs, int32_t num_query_tokens,
                          int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, float k_scale, float v_scale, pa_dtype dtype,
                          pa_dtype kv_dtype, uint32_t flags, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, int32_t* path, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  a.kv_dtype = kv_dtype;
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (is_code_type(kv_dtype)) {
    if (dtype != PA_F16 && dtype != PA_BF16)
      return fail(PA_ERR_UNSUPPORTED, "8-bit pools decode with PA_F16 or PA_BF16 queries");
    if (kv_dtype != PA_INT8_TOKEN && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
    a.k_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : k_scale;  // per-row scales come from the pools
    a.v_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : v_scale;
  } else if (kv_dtype != dtype) {
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype must equal dtype, or be an 8-bit code type");
  }
  if (num_query_tokens < 0 || max_query_len < 1 || max_query_len > 4096)
    return fail(PA_ERR_INVALID_ARG, "num_query_tokens >= 0 and 1 <= max_query_len <= 4096");
  if (static_cast<int64_t>(num_query_tokens) * num_heads > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_query_tokens * num_heads too large");
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV | PA_DECODE_SPLIT))
    return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  a.flags = flags & PA_DECODE_CACHED_KV;
  if (num_seqs > 0 && !query_start) return fail(PA_ERR_INVALID_ARG, "null query_start");
  // path: as pa_decode_quant, with the workgroup count of the multi-token launch
  SplitSizes z;
  const bool sizes_ok = split_sizes(num_query_tokens, num_heads, head_dim, max_context_len,
                                    partition_size > 0 ? partition_size : 1, &z);
  const int64_t need = sizes_ok ? align256(z.total) + static_cast<int64_t>(num_query_tokens) * 4 : -1;
  bool split = false;
  if (flags & PA_DECODE_SPLIT) {
    if (partition_size <= 0 || partition_size % block_size || partition_size > 4096)
      return fail(PA_ERR_INVALID_ARG, "partition_size must be a multiple of block_size, at most 4096");
    split = true;
  } else if (split_override() >= 0 && workspace && num_seqs > 0 && partition_size > 0 &&
             partition_size % block_size == 0 && partition_size <= 4096 && sizes_ok &&
             static_cast<int64_t>(workspace_bytes) >= need) {
    if (split_override() > 0) {
      split = true;
    } else if (a.max_context_len >= 4 * static_cast<int64_t>(partition_size)) {
      int64_t workgroups = 0, resident = 0;
      const bool ok = launch_shape(a, max_query_len, &workgroups, &resident) == hipSuccess;
      (void)hipGetLastError();
      split = ok && workgroups < resident;
    }
  }
  if (path) *path = split ? 1 : 0;
  if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
  if (!aligned16(out) || !aligned16(query)) return fail(PA_ERR_INVALID_ARG, "query and out must be 16-byte aligned");
  pa::SplitLayout ws;
  int32_t* ws_len = nullptr;
  if (split) {
    if (!sizes_ok) return fail(PA_ERR_INVALID_ARG, "split sizes (at most 65535 partitions)");
    if (static_cast<int64_t>(workspace_bytes) < need)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                  "need " + std::to_string(need) + " bytes, got " + std::to_string(workspace_bytes));
    if ((s = make_layout(workspace, workspace_bytes, num_query_tokens, num_heads, head_dim, max_context_len,
                         partition_size, &ws)) != PA_OK)
      return s;
    ws.rows = num_query_tokens;
    ws_len = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256(z.total));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    if ((s = debug_check_tables(a, st)) != PA_OK) return s;
    std::vector<int32_t> qsv, ctx;
    if ((s = fetch(qsv, query_start, static_cast<size_t>(num_seqs) + 1, st)) != PA_OK) return s;
    if ((s = fetch(ctx, context_lens, num_seqs, st)) != PA_OK) return s;
    if (qsv[0] != 0 || qsv[num_seqs] != num_query_tokens)
      return fail(PA_ERR_BAD_TABLE, "query_start must run from 0 to num_query_tokens");
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t span = qsv[i + 1] - qsv[i];
      if (span < 0 || span > max_query_len || span > ctx[i])
        return fail(PA_ERR_BAD_TABLE, "query span of sequence " + std::to_string(i) +
                                          " negative, above max_query_len or above its context length");
    }
  }
  return finish(pa::launch_decode_multi(a, query_start, num_query_tokens, max_query_len, split ? &ws : nullptr,
                                        ws_len, st),
                st,
                "pa_decode_multi");
}

namespace {

// Partition of the longest context into `parts` pieces, rounded up to 64
// tokens (a multiple of every step and block size).
static int32_t partition_of(int32_t max_context_len, int32_t parts) {
  const int64_t piece = (static_cast<int64_t>(max_context_len) + parts - 1) / parts;
  const int64_t p = (piece + 63) / 64 * 64;
  return static_cast<int32_t>(p < 64 ? 64 : p);
}

// The smallest partition of the prefixes pa_decode_shared uses (8 pieces of
// the longest context): the workspace is sized for it.
static int32_t shared_partition_min(int32_t max_context_len) { return partition_of(max_context_len, 8); }

// A piece of the longest context for P shared-prefix partitions: 15 % longer
// than an even cut (then rounded up to 64 tokens), so the last partition is
// the shortest.  The launch places partitions in order (partition-major: the
// k-th workgroup a compute unit receives takes partition k), and the last
// workgroup on a compute unit is served last.  On the parallel-sampling
// workload (P = 3) pieces of 832 (even), 896, 960, 1024 and 1088 tokens gave
// calls of 202.7, 200.6, 200.2, 202.8 and 207.0 us flushed.
static int32_t shared_piece(int32_t max_context_len, int32_t parts) {
  const int64_t piece = (static_cast<int64_t>(max_context_len) * 23 + 20 * parts - 1) / (20 * parts);
  const int64_t p = (piece + 63) / 64 * 64;
  return static_cast<int32_t>(p < 64 ? 64 : p);
}

// Partition of the shared prefixes.  Each prefix unit of the launch (a
// group and head tile) cuts the longest context into P pieces
// (shared_piece), one wave each, and the launch packs the waves four to a
// workgroup across units, so no P leaves a wave idle.  P in 1..8 minimises
// the estimated time: the rounds of resident workgroups the launch needs,
// times the tokens of one wave plus 64 for its fixed costs.  On the
// parallel-sampling workload (1024 units, 768 workgroups resident) that is
// P = 3, one round; the earlier fixed P = 8 needed 2048 workgroups, and its
// third round ran two thirds empty.  PA_SHARED_PARTS=1..8 overrides the rule
// (read on every call).  Every piece is at least shared_partition_min's.
static int32_t shared_partition(const pa::DecodeArgs& a, int32_t num_groups, int32_t max_group_size) {
  const char* v = std::getenv("PA_SHARED_PARTS");
  if (v) {
    const int forced = std::atoi(v);
    if (forced >= 1 && forced <= 8) return shared_piece(a.max_context_len, forced);
  }
  pa::DecodeArgs g = a;
  g.num_seqs = num_groups;
  int64_t units = 0, resident = 0;
  if (launch_shape(g, max_group_size, &units, &resident) != hipSuccess || units <= 0 || resident <= 0) {
    (void)hipGetLastError();
    return shared_partition_min(a.max_context_len);
  }
  int32_t best = 8;
  int64_t best_cost = -1;
  for (int32_t parts = 1; parts <= 8; ++parts) {
    const int64_t piece = shared_piece(a.max_context_len, parts);
    const int64_t used = (static_cast<int64_t>(a.max_context_len) + piece - 1) / piece;  // pieces with tokens
    const int64_t workgroups = (units * used + 3) / 4;
    const int64_t rounds = (workgroups + resident - 1) / resident;
    const int64_t cost = rounds * (piece + 64);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = parts;
    }
  }
  return shared_piece(a.max_context_len, best);
}

// Workspace of the shared-prefix decode: the prefix partials (sized for the
// smallest partition, whatever partition a call takes), the own-token partials
// m, l [S x H] and o [S x H x D], then the prefix length each sequence's
// partials covered, one int per sequence, at the end.
struct SharedSizes {
  int64_t own_m, own_l, own_o, len_off, total;
};
static bool shared_sizes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                  SharedSizes* out) {
  SplitSizes z;
  if (!split_sizes(num_seqs, num_heads, head_dim, max_context_len, shared_partition_min(max_context_len), &z))
    return false;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads;
  out->own_m = align256(z.total);
  out->own_l = align256(out->own_m + rows * 4);
  out->own_o = align256(out->own_l + rows * 4);
  out->len_off = align256(out->own_o + rows * head_dim * 4);
  out->total = out->len_off + static_cast<int64_t>(num_seqs) * 4;
  return true;
}

}  // namespace

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len) {
  SharedSizes z;
  if (!shared_sizes(num_seqs, num_heads, head_dim, max_context_len, &z)) return 0;
  return static_cast<size_t>(z.total);
}

pa_status pa_decode_shared(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_start,
                           const int32_t* prefix_len, int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
                           float k_scale, float v_scale, pa_dtype dtype, pa_dtype kv_dtype, uint32_t flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, nullptr, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  a.kv_dtype = kv_dtype;
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (is_code_type(kv_dtype)) {
    if (dtype != PA_F16 && dtype != PA_BF16)
      return fail(PA_ERR_UNSUPPORTED, "8-bit pools decode with PA_F16 or PA_BF16 queries");
    if (kv_dtype != PA_INT8_TOKEN && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
    a.k_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : k_scale;  // per-row scales come from the pools
    a.v_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : v_scale;
  } else if (kv_dtype != dtype) {
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype must equal dtype, or be an 8-bit code type");
  }
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV)) return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  if (max_group_size < 1 || max_group_size > 4096)
    return fail(PA_ERR_INVALID_ARG, "1 <= max_group_size <= 4096");
  if (num_seqs == 0) return PA_OK;
  if (num_groups < 1 || num_groups > num_seqs)
    return fail(PA_ERR_INVALID_ARG, "the groups must partition the sequences: 1 <= num_groups <= num_seqs");
  if (!group_start || !prefix_len) return fail(PA_ERR_INVALID_ARG, "null group_start or prefix_len");
  SharedSizes zs;
  // the workspace is checked against the size pa_decode_shared_workspace_bytes
  // returns (the smallest partition), whatever partition this call uses
  if (!shared_sizes(num_seqs, num_heads, head_dim, max_context_len, &zs))
    return fail(PA_ERR_INVALID_ARG, "workspace sizes");
  const int64_t need = zs.total;
  if (static_cast<int64_t>(workspace_bytes) < need)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "need " + std::to_string(need) + " bytes, got " + std::to_string(workspace_bytes));
  const int32_t part = shared_partition(a, num_groups, max_group_size);
  pa::SplitLayout ws;
  if ((s = make_layout(workspace, workspace_bytes, num_seqs, num_heads, head_dim, max_context_len, part, &ws)) !=
      PA_OK)
    return s;
  ws.rows = num_seqs;
  char* base = static_cast<char*>(workspace);
  ws.own_m = reinterpret_cast<float*>(base + zs.own_m);
  ws.own_l = reinterpret_cast<float*>(base + zs.own_l);
  ws.own_o = reinterpret_cast<float*>(base + zs.own_o);
  int32_t* ws_len = reinterpret_cast<int32_t*>(base + zs.len_off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    if ((s = debug_check_tables(a, st)) != PA_OK) return s;
    std::vector<int32_t> gs, pl, ctx, tab;
    if ((s = fetch(gs, group_start, static_cast<size_t>(num_groups) + 1, st)) != PA_OK) return s;
    if ((s = fetch(pl, prefix_len, num_seqs, st)) != PA_OK) return s;
    if ((s = fetch(ctx, context_lens, num_seqs, st)) != PA_OK) return s;
    if ((s = fetch(tab, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, st)) != PA_OK) return s;
    if (gs[0] != 0 || gs[num_groups] != num_seqs)
      return fail(PA_ERR_BAD_TABLE, "group_start must run from 0 to num_seqs");
    for (int32_t g = 0; g < num_groups; ++g) {
      const int32_t lead = gs[g], stop = gs[g + 1];
      if (stop <= lead || stop - lead > max_group_size)
        return fail(PA_ERR_BAD_TABLE, "group " + std::to_string(g) + " empty or above max_group_size");
      int32_t r = lead;  // the group's row: the member with the largest prefix_len, the first of them
      for (int32_t i = lead + 1; i < stop; ++i)
        if (pl[i] > pl[r]) r = i;
      for (int32_t i = lead; i < stop; ++i) {
        if (pl[i] < 0 || pl[i] > ctx[i])
          return fail(PA_ERR_BAD_TABLE, "prefix_len of sequence " + std::to_string(i) + " lies outside [0, its context]");
        const int32_t nb = (pl[i] + block_size - 1) / block_size;
        for (int32_t j = 0; j < nb; ++j)
          if (tab[static_cast<size_t>(i) * max_blocks_per_seq + j] !=
              tab[static_cast<size_t>(r) * max_blocks_per_seq + j])
            return fail(PA_ERR_BAD_TABLE, "sequence " + std::to_string(i) + " does not share block " +
                                              std::to_string(j) + " with its group's row");
      }
    }
  }
  return finish(pa::launch_decode_shared(a, group_start, num_groups, max_group_size, prefix_len, ws, ws_len, st),
                st, "pa_decode_shared");
}

pa_status pa_decode_quant(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, float k_scale, float v_scale, pa_dtype dtype,
                          pa_dtype kv_dtype, uint32_t flags, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, int32_t* path, void* stream) {
  pa::DecodeArgs a = pack(out, query, key_cache, value_cache, block_tables, context_lens, seq_order, num_seqs,
                          num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                          max_context_len, scale, dtype, flags);
  a.kv_dtype = kv_dtype;
  a.k_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : k_scale;  // per-row scales come from the pools
  a.v_scale = kv_dtype == PA_INT8_TOKEN ? 1.0f : v_scale;
  pa_status s = check_decode_args(a);
  if (s != PA_OK) return s;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "8-bit pools decode with PA_F16 or PA_BF16 queries");
  if (!is_code_type(kv_dtype)) return fail(PA_ERR_UNSUPPORTED, "kv_dtype must be an 8-bit code type");
  if (kv_dtype != PA_INT8_TOKEN && (s = check_scales(k_scale, v_scale)) != PA_OK) return s;
  if (flags & ~uint32_t(PA_DECODE_CACHED_KV | PA_DECODE_SPLIT))
    return fail(PA_ERR_INVALID_ARG, "unknown flag bits");
  a.flags = flags & PA_DECODE_CACHED_KV;
  bool split = false;
  if (flags & PA_DECODE_SPLIT) {
    if (partition_size <= 0 || partition_size % block_size || partition_size > 4096)
      return fail(PA_ERR_INVALID_ARG, "partition_size must be a multiple of block_size, at most 4096");
    split = true;
  } else {
    split = choose_split(a, partition_size, workspace, workspace_bytes);
  }
  if (path) *path = split ? 1 : 0;
  if (num_seqs == 0) return PA_OK;
  pa::SplitLayout ws;
  if (split && (s = make_layout(workspace, workspace_bytes, num_seqs, num_heads, head_dim, max_context_len,
                                partition_size, &ws)) != PA_OK)
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode() && (s = debug_check_tables(a, st)) != PA_OK) return s;
  return finish(split ? pa::launch_decode_split(a, ws, st) : pa::launch_decode(a, st), st, "pa_decode_quant");
}

pa_status pa_lse_reduce(void* out, const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                        int32_t partition_size, pa_dtype dtype, void* stream) {
  pa_status s = check_shape(dtype, head_dim, 16);
  if (s != PA_OK) return s;
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0 || partition_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs == 0) return PA_OK;
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARG, "null pointer");
  if (static_cast<int64_t>(num_seqs) * num_heads > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_seqs * num_heads too large");
  pa::SplitLayout ws;
  s = make_layout(const_cast<void*>(workspace), workspace_bytes, num_seqs, num_heads, head_dim,
                  max_context_len, partition_size, &ws);
  if (s != PA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_mode()) {
    std::vector<int32_t> ctx;
    if ((s = fetch(ctx, context_lens, num_seqs, st)) != PA_OK) return s;
    for (int32_t i = 0; i < num_seqs; ++i)
      if (ctx[i] < 0 || ctx[i] > max_context_len)
        return fail(PA_ERR_BAD_TABLE, "context_lens[" + std::to_string(i) + "] outside [0, max_context_len]");
  }
  return finish(pa::launch_lse_reduce(out, ws, context_lens, nullptr, num_seqs, num_heads, head_dim,
                                      max_context_len, dtype, st),
                st, "pa_lse_reduce");
}

}  // extern "C"
