// Host-side launchers of the paged decode kernels (decode_kernel.hpp): the
// single pass, the split pass plus its log-sum-exp merge, the fused
// slot-mapping write, and the occupancy query behind pa_decode_auto.
#include <algorithm>

#include "decode_kernel.hpp"

namespace pa {

// ---------------------------------------------------------------------------
// host-side dispatch

namespace {

hipError_t by_dtype(const LaunchOp& op, pa_dtype dt, pa_dtype kv, bool split, bool append, int d, int bs, int gt) {
  if (kv == dt) {
    switch (dt) {
      case PA_F32: return dispatch_f32(op, split, append, d, bs, gt);
      case PA_F16: return dispatch_f16(op, split, append, d, bs, gt);
      case PA_BF16: return dispatch_bf16(op, split, append, d, bs, gt);
      default: return hipErrorInvalidValue;
    }
  }
  if (kv == PA_FP8_E4M3 && dt == PA_F16) return dispatch_e4m3_f16(op, split, append, d, bs, gt);
  if (kv == PA_FP8_E4M3 && dt == PA_BF16) return dispatch_e4m3_bf16(op, split, append, d, bs, gt);
  if (kv == PA_INT8 && dt == PA_F16) return dispatch_i8_f16(op, split, append, d, bs, gt);
  if (kv == PA_INT8 && dt == PA_BF16) return dispatch_i8_bf16(op, split, append, d, bs, gt);
  if (kv == PA_INT8_TOKEN && dt == PA_F16) return dispatch_i8t_f16(op, split, append, d, bs, gt);
  if (kv == PA_INT8_TOKEN && dt == PA_BF16) return dispatch_i8t_bf16(op, split, append, d, bs, gt);
  return hipErrorInvalidValue;
}

hipError_t occupancy_by_dtype(int* per_cu, pa_dtype dt, pa_dtype kv, int d, int bs, int gt) {
  if (kv == dt) {
    switch (dt) {
      case PA_F32: return occupancy_f32(per_cu, d, bs, gt);
      case PA_F16: return occupancy_f16(per_cu, d, bs, gt);
      case PA_BF16: return occupancy_bf16(per_cu, d, bs, gt);
      default: return hipErrorInvalidValue;
    }
  }
  if (kv == PA_FP8_E4M3 && dt == PA_F16) return occupancy_e4m3_f16(per_cu, d, bs, gt);
  if (kv == PA_FP8_E4M3 && dt == PA_BF16) return occupancy_e4m3_bf16(per_cu, d, bs, gt);
  if (kv == PA_INT8 && dt == PA_F16) return occupancy_i8_f16(per_cu, d, bs, gt);
  if (kv == PA_INT8 && dt == PA_BF16) return occupancy_i8_bf16(per_cu, d, bs, gt);
  if (kv == PA_INT8_TOKEN && dt == PA_F16) return occupancy_i8t_f16(per_cu, d, bs, gt);
  if (kv == PA_INT8_TOKEN && dt == PA_BF16) return occupancy_i8t_bf16(per_cu, d, bs, gt);
  return hipErrorInvalidValue;
}

// Heads per workgroup: the largest of {16, 8, 4, 2, 1} dividing the group size
// (16 fills the 16 columns of a q.K tile without replication).
int group_tile(int group) {
  for (int gt : {16, 8, 4, 2}) if (group % gt == 0) return gt;
  return 1;
}

int log2_of(int x) {
  int l = 0;
  while ((1 << (l + 1)) <= x) ++l;
  return l;
}

DecodeParams make_params(const DecodeArgs& x) {
  DecodeParams p{};
  p.col_heads_log2 = log2_of(group_tile(x.num_heads / x.num_kv_heads));
  p.q_chunks = 1;
  p.out = x.out;
  p.q = static_cast<const char*>(x.query);
  p.kc = static_cast<const char*>(x.key_cache);
  p.vc = static_cast<const char*>(x.value_cache);
  p.tables = x.block_tables;
  p.ctx = x.context_lens;
  p.order = x.seq_order;
  p.mask_lo = x.mask_lo;
  p.mask_hi = x.mask_hi;
  p.num_seqs = x.num_seqs;
  p.num_heads = x.num_heads;
  p.num_kv_heads = x.num_kv_heads;
  p.max_blocks = x.max_blocks_per_seq;
  p.num_blocks = x.num_blocks;
  const int64_t cap = static_cast<int64_t>(x.max_blocks_per_seq) * x.block_size;
  p.len_limit = static_cast<int32_t>(cap < x.max_context_len ? cap : x.max_context_len);
  // 8-bit pools: the key scale folds into the logit scale, the value scale
  // into the output (both 1 for model-type pools)
  p.scale_log2 = x.scale * x.k_scale * 1.4426950408889634f;
  p.v_scale = x.v_scale;
  return p;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& x, hipStream_t stream) {
  DecodeParams p = make_params(x);
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  return by_dtype(LaunchOp{p, x.num_seqs, (x.flags & PA_DECODE_CACHED_KV) != 0, stream}, x.dtype, x.kv_dtype,
                  false, false, x.head_dim, x.block_size, gt);
}

hipError_t launch_decode_split(const DecodeArgs& x, const SplitLayout& ws, hipStream_t stream) {
  DecodeParams p = make_params(x);
  p.ws_m = ws.m;
  p.ws_l = ws.l;
  p.ws_o = ws.o;
  p.part_size = ws.partition_size;
  p.num_parts = ws.num_parts;
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  hipError_t e = by_dtype(LaunchOp{p, x.num_seqs, (x.flags & PA_DECODE_CACHED_KV) != 0, stream}, x.dtype,
                           x.kv_dtype, true, false, x.head_dim, x.block_size, gt);
  if (e != hipSuccess) return e;
  return launch_lse_reduce(x.out, ws, x.context_lens, x.seq_order, x.num_seqs, x.num_heads, x.head_dim,
                           p.len_limit, x.dtype, stream);
}

hipError_t launch_decode_append(const DecodeArgs& x, const void* new_k, const void* new_v, const int32_t* slots,
                                const SplitLayout* ws, hipStream_t stream) {
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  DecodeParams p = make_params(x);
  p.new_k = static_cast<const char*>(new_k);
  p.new_v = static_cast<const char*>(new_v);
  p.slots = slots;
  // one (sequence, KV head) pair per writing wave, at most 1024 workgroups (then several each)
  const int64_t pairs = static_cast<int64_t>(x.num_seqs) * x.num_kv_heads;
  p.append_wgs = static_cast<int32_t>(std::min<int64_t>((pairs + kWaves - 1) / kWaves, 1024));
  if (ws) {
    p.ws_m = ws->m;
    p.ws_l = ws->l;
    p.ws_o = ws->o;
    p.part_size = ws->partition_size;
    p.num_parts = ws->num_parts;
  }
  hipError_t e = by_dtype(LaunchOp{p, x.num_seqs, (x.flags & PA_DECODE_CACHED_KV) != 0, stream}, x.dtype,
                          x.kv_dtype, ws != nullptr, true, x.head_dim, x.block_size, gt);
  if (e != hipSuccess || !ws) return e;
  return launch_lse_reduce(x.out, *ws, x.context_lens, x.seq_order, x.num_seqs, x.num_heads, x.head_dim,
                           p.len_limit, x.dtype, stream);
}

// Columns of a tile for several query tokens per sequence: 2^lg heads x the
// rest tokens, NC <= 16; the choice minimises the workgroups per (sequence, KV
// head) (each reads that KV head once), then prefers fewer padding columns.
void multi_tile(int group, int max_q, int* nc, int* lg_heads, int* chunks) {
  int best = -1;
  for (int gh = 1; gh <= 16 && gh <= group; gh *= 2) {
    if (group % gh) continue;
    int nq = 1;
    while (nq * 2 * gh <= 16 && nq < max_q) nq *= 2;
    const int wgs = (group / gh) * ((max_q + nq - 1) / nq);
    const int cols = gh * nq;
    const int cost = wgs * 64 + cols;  // workgroups first, then tile width
    if (best < 0 || cost < best) {
      best = cost;
      *nc = cols;
      *lg_heads = log2_of(gh);
      *chunks = (max_q + nq - 1) / nq;
    }
  }
}

hipError_t launch_decode_multi(const DecodeArgs& x, const int32_t* query_start, int32_t num_query_tokens,
                               int32_t max_query_len, const SplitLayout* ws, int32_t* ws_len, hipStream_t stream) {
  DecodeParams p = make_params(x);
  p.num_q_rows = num_query_tokens;
  int nc = 1, lg = 0, chunks = 1;
  multi_tile(x.num_heads / x.num_kv_heads, max_query_len, &nc, &lg, &chunks);
  p.q_start = query_start;
  p.col_heads_log2 = lg;
  p.q_chunks = chunks;
  if (ws) {
    p.ws_m = ws->m;
    p.ws_l = ws->l;
    p.ws_o = ws->o;
    p.part_size = ws->partition_size;
    p.num_parts = ws->num_parts;
    p.ws_len = ws_len;
  }
  hipError_t e = by_dtype(LaunchOp{p, x.num_seqs, (x.flags & PA_DECODE_CACHED_KV) != 0, stream}, x.dtype,
                          x.kv_dtype, ws != nullptr, false, x.head_dim, x.block_size, nc);
  if (e != hipSuccess || !ws) return e;
  // one merge row per (query row, head); each row's context length was written by the partials pass
  return launch_lse_reduce(x.out, *ws, ws_len, nullptr, ws->rows, x.num_heads, x.head_dim, p.len_limit, x.dtype,
                           stream);
}

hipError_t launch_decode_shared(const DecodeArgs& x, const int32_t* group_start, int32_t num_groups,
                                int32_t max_group, const int32_t* prefix_len, const SplitLayout& ws, int32_t* ws_len,
                                hipStream_t stream) {
  const bool cached = (x.flags & PA_DECODE_CACHED_KV) != 0;
  // One flat launch.  Its first wave items read each group's shared prefix once for all
  // its members (their queries are the columns of the tile) into per-member partials; the
  // rest read each sequence's own tokens after its prefix, one wave per (sequence, head
  // tile), into one more partial.  Short own items fill in behind the long prefix items.
  DecodeArgs g = x;
  g.num_seqs = num_groups;
  g.context_lens = prefix_len;  // read at each group's first member
  g.seq_order = nullptr;
  g.mask_lo = g.mask_hi = nullptr;
  DecodeParams p = make_params(g);
  p.shared = 1;
  p.q_start = group_start;
  p.num_q_rows = x.num_seqs;
  int nc = 1, lg = 0, chunks = 1;
  multi_tile(x.num_heads / x.num_kv_heads, max_group, &nc, &lg, &chunks);
  p.col_heads_log2 = lg;
  p.q_chunks = chunks;
  p.ws_m = ws.m;
  p.ws_l = ws.l;
  p.ws_o = ws.o;
  p.part_size = ws.partition_size;
  p.num_parts = ws.num_parts;
  p.flat = 1;  // the partition count need not be a multiple of the waves per workgroup
  p.ws_len = ws_len;
  const int64_t tiles = x.num_heads >> lg;
  p.n_lead = static_cast<int32_t>(static_cast<int64_t>(num_groups) * tiles * chunks * ws.num_parts);
  p.n_own = static_cast<int32_t>(static_cast<int64_t>(x.num_seqs) * tiles);
  p.own_ctx = x.context_lens;
  p.own_lo = prefix_len;
  p.own_m = ws.own_m;
  p.own_l = ws.own_l;
  p.own_o = ws.own_o;
  hipError_t e = by_dtype(LaunchOp{p, num_groups, cached, stream}, x.dtype, x.kv_dtype, true, false, x.head_dim,
                          x.block_size, nc);
  if (e != hipSuccess) return e;
  // per (sequence, head): the prefix's partitions, then the own tokens' partial; a sequence
  // whose prefix length differs from the one its group's partitions covered gets NaN
  return launch_lse_reduce(x.out, ws, ws_len, nullptr, x.num_seqs, x.num_heads, x.head_dim, p.len_limit, x.dtype,
                           stream, ExtraPartial{ws.own_m, ws.own_l, ws.own_o, prefix_len});
}

hipError_t multi_pass_shape(const DecodeArgs& x, int32_t max_query_len, int64_t* workgroups, int64_t* resident) {
  int nc = 1, lg = 0, chunks = 1;
  multi_tile(x.num_heads / x.num_kv_heads, max_query_len, &nc, &lg, &chunks);
  *workgroups = static_cast<int64_t>(x.num_seqs) * (x.num_heads >> lg) * chunks;
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = occupancy_by_dtype(&per_cu, x.dtype, x.kv_dtype, x.head_dim, x.block_size, nc);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  *resident = static_cast<int64_t>(per_cu) * cus;
  return e;
}

hipError_t single_pass_shape(const DecodeArgs& x, int64_t* workgroups, int64_t* resident) {
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  *workgroups = static_cast<int64_t>(x.num_seqs) * (x.num_heads / gt);
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = occupancy_by_dtype(&per_cu, x.dtype, x.kv_dtype, x.head_dim, x.block_size, gt);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  *resident = static_cast<int64_t>(per_cu) * cus;
  return e;
}

hipError_t launch_lse_reduce(void* out, const SplitLayout& ws, const int32_t* ctx, const int32_t* order,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t len_limit,
                             pa_dtype dt, hipStream_t stream, ExtraPartial extra) {
  if (ws.num_parts + (extra.m ? 1 : 0) <= kSmallParts) {
    // few partials per row: one wave per (row, head)
    const dim3 grid(static_cast<uint32_t>((static_cast<int64_t>(num_seqs) * num_heads + 3) / 4));
#define PA_MERGE(T, D)                                                                                   \
  launch_kernel(lse_merge_small_kernel<T, D>, grid, dim3(256), stream, out, ws.m, ws.l, ws.o, ctx, order, \
                num_seqs, num_heads, len_limit, ws.partition_size, ws.num_parts, extra)
    if (head_dim == 64) {
      if (dt == PA_F32) PA_MERGE(TF32, 64);
      else if (dt == PA_F16) PA_MERGE(TF16, 64);
      else PA_MERGE(TBF16, 64);
    } else {
      if (dt == PA_F32) PA_MERGE(TF32, 128);
      else if (dt == PA_F16) PA_MERGE(TF16, 128);
      else PA_MERGE(TBF16, 128);
    }
#undef PA_MERGE
    return hipGetLastError();
  }
  if (extra.m) return hipErrorInvalidValue;  // the extra partial comes with few partitions only
  const dim3 grid(static_cast<uint32_t>(num_seqs) * num_heads, static_cast<uint32_t>(head_dim / 32));
#define PA_REDUCE(T, D)                                                                          \
  launch_kernel(lse_reduce_kernel<T, D>, grid, dim3(256), stream, out, ws.m, ws.l, ws.o, \
                     ctx, order, num_seqs, num_heads, len_limit, ws.partition_size, ws.num_parts)
  if (head_dim == 64) {
    if (dt == PA_F32) PA_REDUCE(TF32, 64);
    else if (dt == PA_F16) PA_REDUCE(TF16, 64);
    else PA_REDUCE(TBF16, 64);
  } else {
    if (dt == PA_F32) PA_REDUCE(TF32, 128);
    else if (dt == PA_F16) PA_REDUCE(TF16, 128);
    else PA_REDUCE(TBF16, 128);
  }
#undef PA_REDUCE
  return hipGetLastError();
}

}  // namespace pa
