// Pool writes: the slot-mapping scatter of new K/V rows, and whole-block copies
// for copy-on-write.  Both are pure copies, bit-exact.  Every lane reads one
// 16-byte chunk of a row and consecutive lanes take consecutive chunks; key
// rows are stored as whole chunks, value rows element by element down a
// column of the dim-major value tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

// Slot-mapping write ("Ascend C算子开发高阶实战…" §3.1: slot_mapping maps a
// token to block slot / bs, offset slot % bs; "PagedAttention 实现细节" §3.4:
// the new K/V of each step goes into its block).  One thread per 16-byte chunk
// of one (token, KV head) row.  The key chunk is stored whole (keys are token
// rows, [NB, H_kv, bs, D]); the value chunk's EPL elements go down column
// `offset` of the value tile ([NB, H_kv, D, bs]), one element per dim.  Slots
// outside [0, num_blocks * block_size) write nothing.
template <int E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char* __restrict__ key, const char* __restrict__ value, char* __restrict__ key_cache,
    char* __restrict__ value_cache, const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
    int64_t num_slots, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
  constexpr int EPL = 16 / E;
  const int32_t cpr = head_dim / EPL;  // chunks per row
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(num_kv_heads) * cpr;
  if (idx >= per_token * num_tokens) return;
  const int64_t tok = idx / per_token;
  const int64_t rem = idx - tok * per_token;  // = h * cpr + c
  const int32_t h = static_cast<int32_t>(rem / cpr);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * cpr);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t tile = blk * num_kv_heads + h;  // (block, KV head) tile
  const int64_t src = idx * 16;
  store16(key_cache + ((tile * block_size + off) * head_dim + static_cast<int64_t>(c) * EPL) * E,
          load16(key + src));
  const u32x4 v = load16(value + src);
  char* vcol = value_cache + ((tile * head_dim + static_cast<int64_t>(c) * EPL) * block_size + off) * E;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const uint32_t w = word(v, e * E / 4);
    if constexpr (E == 4)
      *reinterpret_cast<uint32_t*>(vcol + static_cast<int64_t>(e) * block_size * E) = w;
    else
      *reinterpret_cast<uint16_t*>(vcol + static_cast<int64_t>(e) * block_size * E) =
          static_cast<uint16_t>(e & 1 ? w >> 16 : w);
  }
}

// The slot-mapping write into 8-bit pools (the quantised cache of the xdnf.cn
// article, §2.3 and §6.3: KV values stored as 8-bit codes).  Same thread
// layout as above: one thread per 16-byte chunk of one (token, KV head) input
// row, EPL elements of the model type T.  Each element becomes the code of
// x / scale (fp32 quotient, round to nearest even; to_code); the EPL key codes
// are stored as one EPL-byte piece of the key row, the value codes one byte
// each down column `offset` of the value tile.
template <typename T, typename C>
__global__ __launch_bounds__(256) void reshape_and_cache_quant_kernel(
    const char* __restrict__ key, const char* __restrict__ value, uint8_t* __restrict__ key_cache,
    uint8_t* __restrict__ value_cache, const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
    int64_t num_slots, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float k_scale,
    float v_scale) {
  constexpr int EPL = T::kEPL;
  constexpr int NW = EPL / 4;  // 32-bit words of codes per chunk
  const int32_t cpr = head_dim / EPL;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(num_kv_heads) * cpr;
  if (idx >= per_token * num_tokens) return;
  const int64_t tok = idx / per_token;
  const int64_t rem = idx - tok * per_token;
  const int32_t h = static_cast<int32_t>(rem / cpr);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * cpr);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t tile = blk * num_kv_heads + h;
  const u32x4 kx = load16(key + idx * 16);
  const u32x4 vx = load16(value + idx * 16);
  uint32_t kw[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) kw[w] = 0;
  uint8_t* vcol = value_cache + (tile * head_dim + static_cast<int64_t>(c) * EPL) * block_size + off;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    kw[e / 4] |= to_code(C{}, elem_to_float(T{}, kx, e) / k_scale) << (8 * (e % 4));
    vcol[static_cast<int64_t>(e) * block_size] =
        static_cast<uint8_t>(to_code(C{}, elem_to_float(T{}, vx, e) / v_scale));
  }
  uint32_t* krow = reinterpret_cast<uint32_t*>(key_cache + (tile * block_size + off) * head_dim +
                                               static_cast<int64_t>(c) * EPL);
#pragma unroll
  for (int w = 0; w < NW; ++w) krow[w] = kw[w];
}

// Whole-block copy ("PagedAttention 实现细节" §3.3: the full contents of the
// original block go to the new one).  grid.x = pair * groups_per_pair + group,
// grid.y = pool (K or V); each workgroup copies a stretch of the block's
// 16-byte chunks.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ key_cache,
                                                          char* __restrict__ value_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t chunks_per_block,
                                                          int32_t groups_per_pair) {
  const int32_t p = blockIdx.x / groups_per_pair;
  const int32_t grp = blockIdx.x - p * groups_per_pair;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* pool = blockIdx.y == 0 ? key_cache : value_cache;
  const char* s = pool + static_cast<int64_t>(src) * chunks_per_block * 16;
  char* d = pool + static_cast<int64_t>(dst) * chunks_per_block * 16;
  constexpr int kUnroll = 4;
  const int64_t stride = static_cast<int64_t>(groups_per_pair) * blockDim.x;
  int64_t i = static_cast<int64_t>(grp) * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < chunks_per_block; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load16(s + (i + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) store16(d + (i + u * stride) * 16, v[u]);
  }
  for (; i < chunks_per_block; i += stride) store16(d + i * 16, load16(s + i * 16));
}

// Swap copies ("PagedAttention 实现细节" §3.4: blocks move between the GPU
// pool and the CPU pool): block pairs[2p] of the source pools -> block
// pairs[2p+1] of the destination pools, K and V, whole blocks.  One side is
// page-locked host memory mapped for the device (either side may be).  Reads
// of host memory, and of the pairs, are system-scope loads, so the copy sees
// what the host (or an earlier swap) wrote whatever the mapping's caching;
// writes to host memory are visible to the host once the stream has finished.
// grid.x = pair * groups_per_pair + group, grid.y = pool (K or V).
template <bool SRC_HOST>
__global__ __launch_bounds__(256) void swap_blocks_kernel(char* __restrict__ dst_key, char* __restrict__ dst_value,
                                                          const char* src_key, const char* src_value,
                                                          const int32_t* pairs, int32_t num_src_blocks,
                                                          int32_t num_dst_blocks, int64_t chunks_per_block,
                                                          int32_t groups_per_pair) {
  const int32_t p = blockIdx.x / groups_per_pair;
  const int32_t grp = blockIdx.x - p * groups_per_pair;
  const int32_t src = __hip_atomic_load(pairs + 2 * p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const int32_t dst = __hip_atomic_load(pairs + 2 * p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (src < 0 || src >= num_src_blocks || dst < 0 || dst >= num_dst_blocks) return;
  const char* s = (blockIdx.y == 0 ? src_key : src_value) + static_cast<int64_t>(src) * chunks_per_block * 16;
  char* d = (blockIdx.y == 0 ? dst_key : dst_value) + static_cast<int64_t>(dst) * chunks_per_block * 16;
  const int64_t stride = static_cast<int64_t>(groups_per_pair) * blockDim.x;
  int64_t i = static_cast<int64_t>(grp) * blockDim.x + threadIdx.x;
  if constexpr (SRC_HOST) {
    // 16-byte loads at system scope (the sc0 sc1 bits of a system-scope load),
    // four in flight per lane: each is one host-link read.  The waitcnt takes
    // the four registers as operands, so nothing uses them before the data is in.
    for (; i < chunks_per_block; i += 4 * stride) {
      u32x4 v0{}, v1{}, v2{}, v3{};
      const bool ok1 = i + stride < chunks_per_block, ok2 = i + 2 * stride < chunks_per_block,
                 ok3 = i + 3 * stride < chunks_per_block;
      asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v0) : "v"(s + i * 16) : "memory");
      if (ok1) asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v1) : "v"(s + (i + stride) * 16) : "memory");
      if (ok2)
        asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v2) : "v"(s + (i + 2 * stride) * 16) : "memory");
      if (ok3)
        asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v3) : "v"(s + (i + 3 * stride) * 16) : "memory");
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3) : : "memory");
      store16(d + i * 16, v0);
      if (ok1) store16(d + (i + stride) * 16, v1);
      if (ok2) store16(d + (i + 2 * stride) * 16, v2);
      if (ok3) store16(d + (i + 3 * stride) * 16, v3);
    }
  } else {
    for (; i < chunks_per_block; i += stride) store16(d + i * 16, load16(s + i * 16));
  }
}

hipError_t launch_swap_blocks(void* dst_key, void* dst_value, const void* src_key, const void* src_value,
                              const int32_t* pairs, int32_t num_pairs, int32_t num_src_blocks,
                              int32_t num_dst_blocks, int64_t block_bytes, bool src_host, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  int64_t gx = (chunks + 1023) / 1024;
  if (gx < 1) gx = 1;
  const dim3 grid(static_cast<uint32_t>(gx * num_pairs), 2);
#define PA_SWAP(H)                                                                                           \
  hipLaunchKernelGGL(swap_blocks_kernel<H>, grid, dim3(256), 0, stream, static_cast<char*>(dst_key),         \
                     static_cast<char*>(dst_value), static_cast<const char*>(src_key),                      \
                     static_cast<const char*>(src_value), pairs, num_src_blocks, num_dst_blocks, chunks,      \
                     static_cast<int32_t>(gx))
  if (src_host)
    PA_SWAP(true);
  else
    PA_SWAP(false);
#undef PA_SWAP
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t elem_bytes, int32_t block_size, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim * elem_bytes / 16);
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
#define PA_RESHAPE(E)                                                                                      \
  hipLaunchKernelGGL(reshape_and_cache_kernel<E>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, \
                     static_cast<const char*>(key), static_cast<const char*>(value),                      \
                     static_cast<char*>(key_cache), static_cast<char*>(value_cache), slot_mapping,          \
                     num_tokens, num_slots, num_kv_heads, head_dim, block_size)
  if (elem_bytes == 4)
    PA_RESHAPE(4);
  else
    PA_RESHAPE(2);
#undef PA_RESHAPE
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_quant(const void* key, const void* value, void* key_cache, void* value_cache,
                                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pa_dtype dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                                          hipStream_t stream) {
  const int32_t elem = dtype == PA_F32 ? 4 : 2;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim * elem / 16);
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((total + 255) / 256));
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
#define PA_QWRITE(T, C)                                                                                    \
  hipLaunchKernelGGL((reshape_and_cache_quant_kernel<T, C>), grid, dim3(256), 0, stream,                   \
                     static_cast<const char*>(key), static_cast<const char*>(value),                      \
                     static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache), slot_mapping,    \
                     num_tokens, num_slots, num_kv_heads, head_dim, block_size, k_scale, v_scale)
  if (kv_dtype == PA_FP8_E4M3) {
    if (dtype == PA_F32) PA_QWRITE(TF32, TE4M3);
    else if (dtype == PA_F16) PA_QWRITE(TF16, TE4M3);
    else PA_QWRITE(TBF16, TE4M3);
  } else {
    if (dtype == PA_F32) PA_QWRITE(TF32, TI8);
    else if (dtype == PA_F16) PA_QWRITE(TF16, TI8);
    else PA_QWRITE(TBF16, TI8);
  }
#undef PA_QWRITE
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  // about 4 chunks per thread per workgroup pass; at least one workgroup
  int64_t gx = (chunks + 1023) / 1024;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(gx * num_pairs), 2), dim3(256), 0,
                     stream, static_cast<char*>(key_cache), static_cast<char*>(value_cache), pairs,
                     num_blocks, chunks, static_cast<int32_t>(gx));
  return hipGetLastError();
}

}  // namespace pa
