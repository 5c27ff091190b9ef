// Internal interface between the C ABI layer (api.cpp) and the kernel
// launchers.  Arguments reaching these functions have been validated.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Measurement hook (pa_set_launch_events): events to attach to the kernels of
// the next library call made on this thread.  launch_kernel takes them: the
// first kernel of the call records `start` when it starts, and every kernel
// records `stop` when it ends, so the last one's end remains
// (hipExtLaunchKernel).  The call's finish clears them.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchEvents& launch_events();  // this thread's

template <typename F, typename... Args>
void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start || ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
    ev.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  }
}

struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* seq_order;  // optional, may be null
  int32_t num_seqs, num_heads, num_kv_heads, head_dim, block_size;
  int32_t max_blocks_per_seq, num_blocks, max_context_len;
  float scale;
  pa_dtype dtype;  // query / output type
  uint32_t flags;  // PA_DECODE_* bits
  // pools: kv_dtype == dtype, or an 8-bit code type with per-pool scales
  pa_dtype kv_dtype = PA_F32;
  float k_scale = 1.0f;
  float v_scale = 1.0f;
  // optional per-sequence masked positions [mask_lo, mask_hi)
  const int32_t* mask_lo = nullptr;
  const int32_t* mask_hi = nullptr;
};

// The three fp32 arrays of the split workspace (see pa_decode_split_workspace_bytes).
struct SplitLayout {
  float* m;
  float* l;
  float* o;
  int32_t partition_size;
  int32_t num_parts;
  int32_t rows = 0;  // rows of the partials (sequences; query rows for several query tokens)
  // the shared-prefix decode's own-token partials, one per (row, head): m, l [rows x heads],
  // o [rows x heads x head_dim]
  float* own_m = nullptr;
  float* own_l = nullptr;
  float* own_o = nullptr;
};

// One more partial per (row, head) for the log-sum-exp merge, and the context
// length each row's partitions must have covered (see lse_reduce_kernel).
struct ExtraPartial {
  const float* m = nullptr;
  const float* l = nullptr;
  const float* o = nullptr;
  const int32_t* expect = nullptr;
};

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t elem_bytes, int32_t block_size, hipStream_t stream);
// The quantising slot-mapping write: rows of `dtype` -> codes of `kv_dtype`.
hipError_t launch_reshape_and_cache_quant(const void* key, const void* value, void* key_cache, void* value_cache,
                                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pa_dtype dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                                          hipStream_t stream);
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                              hipStream_t stream);
hipError_t launch_upload(void* dst, const void* src_device_view, int64_t nbytes, hipStream_t stream);
// The quantising write into int8 pools with a scale per (token, KV head)
// (PA_INT8_TOKEN): each row's scale computed from the row, stored in its tile.
hipError_t launch_reshape_and_cache_rows(const void* key, const void* value, void* key_cache, void* value_cache,
                                         const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                         hipStream_t stream);
// pa_upload and the slot-mapping write (plain or quantising) in one launch; the
// slots are read from page-locked host memory (its device view).
hipError_t launch_upload_and_cache(void* dst, const void* src_device_view, int64_t nbytes, const void* key,
                                   const void* value, void* key_cache, void* value_cache,
                                   const int32_t* slot_mapping_device_view, int32_t num_tokens,
                                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   pa_dtype dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                                   int32_t write_form, const int32_t* host_slots, hipStream_t stream);
// write_form: 0 element-wise; 1 element-wise with non-temporal stores; 2 whole
// value tiles (host_slots: the host-readable slot mapping).  Forms 1 and 2
// need a call in which no two tokens share a block.
// Whole-block copies between two pools (device views of host pools allowed).
hipError_t launch_swap_blocks(void* dst_key, void* dst_value, const void* src_key, const void* src_value,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_src_blocks,
                              int32_t num_dst_blocks, int64_t block_bytes, bool src_host, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, const SplitLayout& ws, hipStream_t stream);
// Slot-mapping write of one new token per sequence fused into the decode
// (single pass when ws is null, else split + merge).
hipError_t launch_decode_append(const DecodeArgs& a, const void* new_k, const void* new_v, const int32_t* slots,
                                const SplitLayout* ws, hipStream_t stream);
// Workgroups the single-pass launch would start, and how many of them the
// current device holds at once.
hipError_t single_pass_shape(const DecodeArgs& a, int64_t* workgroups, int64_t* resident);
// Several causal query tokens per sequence: rows query_start[s] .. query_start[s+1]-1
// of query/out (single pass when ws is null, else split + merge; ws_len: one int per
// query row in the workspace, the merge's context lengths).
hipError_t launch_decode_multi(const DecodeArgs& a, const int32_t* query_start, int32_t num_query_tokens,
                               int32_t max_query_len, const SplitLayout* ws, int32_t* ws_len, hipStream_t stream);
hipError_t multi_pass_shape(const DecodeArgs& a, int32_t max_query_len, int64_t* workgroups, int64_t* resident);
// Groups of sequences sharing their first prefix_len tokens' blocks: sequences
// group_start[g] .. group_start[g+1]-1, prefix_len per sequence (equal within a
// group).  One flat launch reads each group's prefix once into per-member
// partials (ws, one int per sequence in ws_len) and each sequence's own tokens
// into one more partial (ws.own_*); the merge combines them.
hipError_t launch_decode_shared(const DecodeArgs& a, const int32_t* group_start, int32_t num_groups,
                                int32_t max_group, const int32_t* prefix_len, const SplitLayout& ws, int32_t* ws_len,
                                hipStream_t stream);
// Device address of the library's static split workspace on the current device
// (PA_STATIC_SCRATCH_BYTES bytes, 256-byte aligned), looked up on the first
// call per device.
hipError_t static_scratch(void** ptr);
hipError_t launch_lse_reduce(void* out, const SplitLayout& ws, const int32_t* context_lens,
                             const int32_t* seq_order, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t len_limit, pa_dtype dtype, hipStream_t stream, ExtraPartial extra = {});

}  // namespace pa
