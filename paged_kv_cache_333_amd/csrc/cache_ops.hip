// Pool writes: the slot-mapping scatter of new K/V rows, and whole-block copies
// for copy-on-write.  Both are pure copies, bit-exact.  Every lane reads one
// 16-byte chunk of a row and consecutive lanes take consecutive chunks; key
// rows are stored as whole chunks, value rows element by element down a
// column of the dim-major value tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

// Arguments of the slot-mapping write (both forms below).
struct WriteArgs {
  const char* key;
  const char* value;
  char* key_cache;
  char* value_cache;
  const int32_t* slots;
  int32_t num_tokens;
  int64_t num_slots;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  float k_scale, v_scale;  // 8-bit pools only
};

// Store of the element-wise writes: plain, or (NT) non-temporal.  A decode
// step that appends one token per sequence writes each cache line of a value
// tile once; non-temporal stores then leave no partly written line in the L2
// for the kernels that follow (measured: the LLaMA-7B-like step 206 -> 203
// us, its decode 190 -> 186.5 us).  Where several tokens of a call share a
// block, plain stores let the L2 merge their writes to one line (with
// non-temporal stores the 4-token verification step took 256 instead of
// 232 us).  The host picks non-temporal stores for model-type pools only:
// the quantising write's one-byte stores made the FP8 step slower with them.
template <bool NT, typename U>
__device__ __forceinline__ void put(U* p, U v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// Slot of token `tok`: from device memory, or (HOST_SLOTS) from the
// workgroup's LDS copy of its tokens' slots (staged from host memory once per
// workgroup, see upload_and_cache_kernel; tok_first is its first token).
struct HostSlots {
  const int32_t* lds;
  int64_t tok_first;
};
template <bool HOST_SLOTS>
__device__ __forceinline__ int64_t slot_of(const int32_t* slots, const HostSlots& hs, int64_t tok) {
  if constexpr (HOST_SLOTS)
    return hs.lds[tok - hs.tok_first];
  else
    return slots[tok];
}

// Slot-mapping write ("Ascend C算子开发高阶实战…" §3.1: slot_mapping maps a
// token to block slot / bs, offset slot % bs; "PagedAttention 实现细节" §3.4:
// the new K/V of each step goes into its block).  Thread `idx` handles one
// 16-byte chunk of one (token, KV head) row.  The key chunk is stored whole
// (keys are token rows, [NB, H_kv, bs, D]); the value chunk's EPL elements go
// down column `offset` of the value tile ([NB, H_kv, D, bs]), one element per
// dim.  Slots outside [0, num_blocks * block_size) write nothing.
template <int E, bool HOST_SLOTS, bool NT>
__device__ __forceinline__ void write_chunk(const WriteArgs& a, int64_t idx, const HostSlots& hs) {
  constexpr int EPL = 16 / E;
  const int32_t cpr = a.head_dim / EPL;  // chunks per row
  const int64_t per_token = static_cast<int64_t>(a.num_kv_heads) * cpr;
  if (idx >= per_token * a.num_tokens) return;
  const int64_t tok = idx / per_token;
  const int64_t rem = idx - tok * per_token;  // = h * cpr + c
  const int32_t h = static_cast<int32_t>(rem / cpr);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * cpr);
  const int64_t slot = slot_of<HOST_SLOTS>(a.slots, hs, tok);
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t tile = blk * a.num_kv_heads + h;  // (block, KV head) tile
  const int64_t src = idx * 16;
  put<NT>(reinterpret_cast<u32x4*>(a.key_cache +
                                   ((tile * a.block_size + off) * a.head_dim + static_cast<int64_t>(c) * EPL) * E),
          load16(a.key + src));
  const u32x4 v = load16(a.value + src);
  char* vcol = a.value_cache + ((tile * a.head_dim + static_cast<int64_t>(c) * EPL) * a.block_size + off) * E;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const uint32_t w = word(v, e * E / 4);
    if constexpr (E == 4)
      put<NT>(reinterpret_cast<uint32_t*>(vcol + static_cast<int64_t>(e) * a.block_size * E), w);
    else
      put<NT>(reinterpret_cast<uint16_t*>(vcol + static_cast<int64_t>(e) * a.block_size * E),
              static_cast<uint16_t>(e & 1 ? w >> 16 : w));
  }
}

// Element `e` of a 16-byte chunk of E-byte elements replaced by the low 8*E
// bits of x (selects over the four words, no indexed register access).
template <int E>
__device__ __forceinline__ u32x4 with_element(u32x4 v, int e, uint32_t x) {
  const int w = e * E / 4;
  const int sh = (e * E % 4) * 8;
  uint32_t mask;
  if constexpr (E == 4)
    mask = 0xffffffffu;
  else
    mask = ((1u << (8 * E)) - 1u) << sh;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t vi = word(v, i);
    r[i] = i == w ? (vi & ~mask) | ((x << sh) & mask) : vi;
  }
  return r;
}

// Whole-tile form of the write, used when no two tokens of a call fall in
// one block (a decode step that appends one token per sequence: the block a
// sequence writes has that sequence as its only owner).  A token's value
// column crosses every cache line of its dim-major value tile, so the
// element-wise stores above leave each line of the tile partly written, and
// the kernel that next reads those lines pays far beyond their byte count
// (with 32-token blocks, a decode right after such a write ran 16 us slower
// than after a write of whole lines).  Here one workgroup owns the tiles of
// KV heads h0..h1-1 of one token: it stores the key rows in 16-byte chunks,
// reads the value tiles chunk by chunk, puts the new element into the chunk
// of each dim row that holds column `offset`, and stores every chunk back, so
// every line of the tiles is written whole and only the new column changes.
// Bit-exact, like the element-wise form.
template <int E>
__device__ __forceinline__ void write_tile(const WriteArgs& a, int64_t tok, int32_t h0, int32_t h1, int64_t slot) {
  constexpr int EPL = 16 / E;
  const int64_t blk = slot / a.block_size;
  const int32_t off = static_cast<int32_t>(slot - blk * a.block_size);
  const int32_t cpr = a.head_dim / EPL;
  for (int32_t j = threadIdx.x; j < (h1 - h0) * cpr; j += blockDim.x) {
    const int32_t h = h0 + j / cpr;
    const int32_t c = j - (h - h0) * cpr;
    const int64_t tile = blk * a.num_kv_heads + h;
    store16(a.key_cache + ((tile * a.block_size + off) * a.head_dim + static_cast<int64_t>(c) * EPL) * E,
            load16(a.key + ((tok * a.num_kv_heads + h) * a.head_dim + static_cast<int64_t>(c) * EPL) * E));
  }
  // the value tiles of heads h0..h1-1 are contiguous: [h, d, chunk of the row]
  const int32_t rc = a.block_size / EPL;  // chunks per dim row of the value tile
  const int32_t oc = off / EPL;           // the chunk of a row holding column `off`
  const int32_t oe = off - oc * EPL;      // and its element there
  char* vt = a.value_cache + (blk * a.num_kv_heads + h0) * a.head_dim * a.block_size * E;
  const char* vin = a.value + (tok * a.num_kv_heads + h0) * a.head_dim * E;  // rows of heads h0.. of the token
  const int32_t n = (h1 - h0) * a.head_dim * rc;
  for (int32_t i = threadIdx.x; i < n; i += blockDim.x) {
    u32x4 v = load16(vt + static_cast<int64_t>(i) * 16);
    const int32_t r = i / rc;  // (head - h0) * head_dim + d
    if (i - r * rc == oc) {
      uint32_t x;
      if constexpr (E == 4)
        x = *reinterpret_cast<const uint32_t*>(vin + static_cast<int64_t>(r) * 4);
      else
        x = *reinterpret_cast<const uint16_t*>(vin + static_cast<int64_t>(r) * 2);
      v = with_element<E>(v, oe, x);
    }
    store16(vt + static_cast<int64_t>(i) * 16, v);
  }
}

// The codes of the EPL key elements of input chunk `kx` (x / k_scale, see
// write_chunk_quant), stored as EPL bytes at `dst`.
template <typename T, typename C, bool NT = false>
__device__ __forceinline__ void store_key_codes(const WriteArgs& a, u32x4 kx, char* dst) {
  constexpr int EPL = T::kEPL;
  constexpr int NW = EPL / 4;  // 32-bit words of codes per chunk
  uint32_t kw[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) kw[w] = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) kw[e / 4] |= to_code(C{}, elem_to_float(T{}, kx, e) / a.k_scale) << (8 * (e % 4));
  uint32_t* krow = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
  for (int w = 0; w < NW; ++w) put<NT>(krow + w, kw[w]);
}

// The slot-mapping write into 8-bit pools (the quantised cache of the xdnf.cn
// article, §2.3 and §6.3: KV values stored as 8-bit codes).  Same thread
// layout: one thread per 16-byte chunk of one (token, KV head) input row, EPL
// elements of the model type T.  Each element becomes the code of x / scale
// (fp32 quotient, round to nearest even; to_code); the EPL key codes are
// stored as one EPL-byte piece of the key row, the value codes one byte each
// down column `offset` of the value tile.
template <typename T, typename C, bool HOST_SLOTS, bool NT>
__device__ __forceinline__ void write_chunk_quant(const WriteArgs& a, int64_t idx, const HostSlots& hs) {
  constexpr int EPL = T::kEPL;
  const int32_t cpr = a.head_dim / EPL;
  const int64_t per_token = static_cast<int64_t>(a.num_kv_heads) * cpr;
  if (idx >= per_token * a.num_tokens) return;
  const int64_t tok = idx / per_token;
  const int64_t rem = idx - tok * per_token;
  const int32_t h = static_cast<int32_t>(rem / cpr);
  const int32_t c = static_cast<int32_t>(rem - static_cast<int64_t>(h) * cpr);
  const int64_t slot = slot_of<HOST_SLOTS>(a.slots, hs, tok);
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t tile = blk * a.num_kv_heads + h;
  store_key_codes<T, C, NT>(a, load16(a.key + idx * 16),
                            a.key_cache + (tile * a.block_size + off) * a.head_dim + static_cast<int64_t>(c) * EPL);
  const u32x4 vx = load16(a.value + idx * 16);
  uint8_t* vcol = reinterpret_cast<uint8_t*>(a.value_cache) +
                  (tile * a.head_dim + static_cast<int64_t>(c) * EPL) * a.block_size + off;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    put<NT>(vcol + static_cast<int64_t>(e) * a.block_size,
            static_cast<uint8_t>(to_code(C{}, elem_to_float(T{}, vx, e) / a.v_scale)));
}

// Whole-tile form of the quantising write (see write_tile): the key codes of
// the token's rows, then the value tiles [D, bs] of one-byte codes read and
// stored back in 16-byte chunks with the new column's codes put in.
template <typename T, typename C>
__device__ __forceinline__ void write_tile_quant(const WriteArgs& a, int64_t tok, int32_t h0, int32_t h1,
                                                 int64_t slot) {
  constexpr int EPL = T::kEPL;
  constexpr int EB = T::kBytes;
  const int64_t blk = slot / a.block_size;
  const int32_t off = static_cast<int32_t>(slot - blk * a.block_size);
  const int32_t cpr = a.head_dim / EPL;
  for (int32_t j = threadIdx.x; j < (h1 - h0) * cpr; j += blockDim.x) {
    const int32_t h = h0 + j / cpr;
    const int32_t c = j - (h - h0) * cpr;
    const int64_t tile = blk * a.num_kv_heads + h;
    store_key_codes<T, C>(a, load16(a.key + ((tok * a.num_kv_heads + h) * a.head_dim +
                                             static_cast<int64_t>(c) * EPL) * EB),
                          a.key_cache + (tile * a.block_size + off) * a.head_dim + static_cast<int64_t>(c) * EPL);
  }
  const int32_t rc = a.block_size / 16;  // 16-byte chunks per dim row of codes
  const int32_t oc = off / 16;
  const int32_t oe = off - oc * 16;
  char* vt = a.value_cache + (blk * a.num_kv_heads + h0) * a.head_dim * a.block_size;
  const char* vin = a.value + (tok * a.num_kv_heads + h0) * a.head_dim * EB;
  const int32_t n = (h1 - h0) * a.head_dim * rc;
  for (int32_t i = threadIdx.x; i < n; i += blockDim.x) {
    u32x4 v = load16(vt + static_cast<int64_t>(i) * 16);
    const int32_t r = i / rc;
    if (i - r * rc == oc) {
      uint32_t x;
      if constexpr (EB == 4)
        x = *reinterpret_cast<const uint32_t*>(vin + static_cast<int64_t>(r) * 4);
      else
        x = *reinterpret_cast<const uint16_t*>(vin + static_cast<int64_t>(r) * 2);
      const u32x4 xin = {x, 0u, 0u, 0u};  // the element as element 0 of a chunk
      v = with_element<1>(v, oe, to_code(C{}, elem_to_float(T{}, xin, 0) / a.v_scale));
    }
    store16(vt + static_cast<int64_t>(i) * 16, v);
  }
}

// One model-type element at p, as fp32 (exact).
__device__ __forceinline__ float element_at(TF32, const char* p) {
  return __builtin_bit_cast(float, *reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float element_at(TF16, const char* p) {
  return static_cast<float>(__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(p)));
}
__device__ __forceinline__ float element_at(TBF16, const char* p) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

// The slot-mapping write into int8 pools with one scale per (token, KV head)
// (the per-token int8 form of the xdnf.cn article's §2.3/§6.3).  One wave per
// (token, KV head): its key row and its value row each get s = max |x| / 127
// (fp32 division) and codes to_code(x / s) (nearest, ties to even,
// saturating at +-127); a row of zeros gets s = 0 and codes 0.  Lane l holds
// elements EL l .. EL l + EL - 1; the row's max comes from a butterfly of lane
// exchanges.  The key codes go to the token's row of the key tile, the value
// codes one byte each down column `offset` of the value tile, the key scale to
// byte BS * D + 4 offset of the key tile, and the value scale to byte
// BS * D + 4 BS + 4 offset of the key tile when the block's scales are paired
// there (token_scales_paired), else to byte BS * D + 4 offset of the value
// tile.  Slots outside the pool write nothing.
template <typename T, int D>
__global__ __launch_bounds__(256) void reshape_and_cache_rows_kernel(WriteArgs a) {
  constexpr int EL = D / 64;
  constexpr int E = T::kBytes;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // token * H_kv + head
  if (row >= static_cast<int64_t>(a.num_tokens) * a.num_kv_heads) return;
  const int64_t tok = row / a.num_kv_heads;
  const int32_t h = static_cast<int32_t>(row - tok * a.num_kv_heads);
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  // bytes per tile: the codes, then the scale area
  const int64_t tb = static_cast<int64_t>(a.block_size) * D + token_scale_area(a.block_size);
  char* kt = a.key_cache + (blk * a.num_kv_heads + h) * tb;
  char* vt = a.value_cache + (blk * a.num_kv_heads + h) * tb;
  float xk[EL], xv[EL];
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int i = 0; i < EL; ++i) {
    const int64_t src = (row * D + EL * lane + i) * E;
    xk[i] = element_at(T{}, a.key + src);
    xv[i] = element_at(T{}, a.value + src);
    mk = fmaxf(mk, fabsf(xk[i]));
    mv = fmaxf(mv, fabsf(xv[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, o));
    mv = fmaxf(mv, __shfl_xor(mv, o));
  }
  const float sk = mk / 127.0f;
  const float sv = mv / 127.0f;
#pragma unroll
  for (int i = 0; i < EL; ++i) {
    const int d = EL * lane + i;
    const uint32_t ck = sk > 0.f ? to_code(TI8{}, xk[i] / sk) : 0u;
    const uint32_t cv = sv > 0.f ? to_code(TI8{}, xv[i] / sv) : 0u;
    reinterpret_cast<uint8_t*>(kt)[off * D + d] = static_cast<uint8_t>(ck);
    reinterpret_cast<uint8_t*>(vt)[static_cast<int64_t>(d) * a.block_size + off] = static_cast<uint8_t>(cv);
  }
  if (lane == 0) {
    const int64_t area = static_cast<int64_t>(a.block_size) * D;
    *reinterpret_cast<float*>(kt + area + 4 * off) = sk;
    char* vs = token_scales_paired(a.block_size) ? kt + area + 4 * a.block_size : vt + area;
    *reinterpret_cast<float*>(vs + 4 * off) = sv;
  }
}

// W::template run<HOST_SLOTS, NT>(a, idx, hs) is one of the two element-wise writes above,
// W::run_tile(a, tok, h0, h1, slot) the matching whole-tile write.
template <int E>
struct PlainWrite {
  static constexpr int kEPL = 16 / E;
  template <bool H, bool NT>
  __device__ static void run(const WriteArgs& a, int64_t idx, const HostSlots& hs) {
    write_chunk<E, H, NT>(a, idx, hs);
  }
  __device__ static void run_tile(const WriteArgs& a, int64_t tok, int32_t h0, int32_t h1, int64_t slot) {
    write_tile<E>(a, tok, h0, h1, slot);
  }
};
template <typename T, typename C>
struct QuantWrite {
  static constexpr int kEPL = T::kEPL;
  template <bool H, bool NT>
  __device__ static void run(const WriteArgs& a, int64_t idx, const HostSlots& hs) {
    write_chunk_quant<T, C, H, NT>(a, idx, hs);
  }
  __device__ static void run_tile(const WriteArgs& a, int64_t tok, int32_t h0, int32_t h1, int64_t slot) {
    write_tile_quant<T, C>(a, tok, h0, h1, slot);
  }
};

template <typename W>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(WriteArgs a) {
  W::template run<false, false>(a, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                                HostSlots{nullptr, 0});
}

// One launch for the two small transfers of a decode step: the first
// `up_blocks` workgroups copy the step's index block from page-locked host
// memory to the device (as pa_upload), the others do the slot-mapping write,
// with the slots read from the host copy.  Two launches would cost a
// dependent-dispatch gap between them.  A host read is a round trip over the
// host link, so a writing workgroup fetches the slots of its few tokens once
// (one lane each, system-scope loads) into LDS and its threads read them there.
// The upload part: workgroups 0..up_blocks-1 copy `words` words from host memory.
__device__ __forceinline__ void upload_words(uint32_t* __restrict__ dst, const uint32_t* src, int64_t words,
                                             int32_t up_blocks) {
  const int64_t stride = static_cast<int64_t>(up_blocks) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += stride)
    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The slots of a call of at most kArgSlots tokens, passed with the launch
// (ARG): the writing workgroups then wait on no host read before their
// stores.  Used where no two tokens share a block (the host has read the
// slots to check that); with the element-wise form and non-temporal stores
// it shortened the LLaMA-7B-like step by 2 us (202 -> 200 us).
constexpr int32_t kArgSlots = 256;
struct ArgSlots {
  int32_t v[kArgSlots];
};

template <typename W, bool NT, bool ARG>
__global__ __launch_bounds__(256) void upload_and_cache_kernel(WriteArgs a, uint32_t* __restrict__ dst,
                                                               const uint32_t* src, int64_t words,
                                                               int32_t up_blocks, ArgSlots arg) {
  if (static_cast<int32_t>(blockIdx.x) < up_blocks) {
    upload_words(dst, src, words, up_blocks);
    return;
  }
  __shared__ int32_t slots_lds[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x - up_blocks) * blockDim.x;
  const int64_t per_token = static_cast<int64_t>(a.num_kv_heads) * (a.head_dim / W::kEPL);
  const int64_t tok_first = base / per_token;
  // tokens of this workgroup's 256 chunks: at most 256 (a row has at least one chunk)
  const int64_t tok_stop = min((base + blockDim.x - 1) / per_token + 1, static_cast<int64_t>(a.num_tokens));
  if (tok_first + threadIdx.x < tok_stop) {
    if constexpr (ARG)
      slots_lds[threadIdx.x] = arg.v[tok_first + threadIdx.x];
    else
      slots_lds[threadIdx.x] = __hip_atomic_load(a.slots + tok_first + threadIdx.x, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __syncthreads();
  W::template run<true, NT>(a, base + threadIdx.x, HostSlots{slots_lds, tok_first});
}

// The same launch with the whole-tile write (write_tile), for calls in which
// no two tokens share a block.  Slots come from the kernel arguments when the
// call has at most kArgSlots tokens: workgroup up_blocks + tok * num_kv_heads
// + h then writes token tok's tile of KV head h.  Larger calls read each slot
// from host memory once, and workgroup up_blocks + tok writes all the token's
// tiles (host reads of one line by many workgroups queue behind each other).

template <typename W, bool ARG_SLOTS>
__global__ __launch_bounds__(256) void upload_and_cache_tiles_kernel(WriteArgs a, uint32_t* __restrict__ dst,
                                                                     const uint32_t* src, int64_t words,
                                                                     int32_t up_blocks, ArgSlots arg) {
  if (static_cast<int32_t>(blockIdx.x) < up_blocks) {
    upload_words(dst, src, words, up_blocks);
    return;
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) - up_blocks;
  if constexpr (ARG_SLOTS) {
    const int32_t tok = static_cast<int32_t>(t / a.num_kv_heads);
    const int32_t h = static_cast<int32_t>(t - static_cast<int64_t>(tok) * a.num_kv_heads);
    const int64_t slot = arg.v[tok];
    if (slot < 0 || slot >= a.num_slots) return;
    W::run_tile(a, tok, h, h + 1, slot);
  } else {
    __shared__ int32_t slot_lds;
    if (threadIdx.x == 0) slot_lds = __hip_atomic_load(a.slots + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    const int64_t slot = slot_lds;
    if (slot < 0 || slot >= a.num_slots) return;
    W::run_tile(a, t, 0, a.num_kv_heads, slot);
  }
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
  launch_kernel(swap_blocks_kernel<H>, grid, dim3(256), stream, static_cast<char*>(dst_key),         \
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

namespace {

WriteArgs write_args(const void* key, const void* value, void* key_cache, void* value_cache,
                     const int32_t* slots, int32_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, float k_scale, float v_scale) {
  return WriteArgs{static_cast<const char*>(key), static_cast<const char*>(value), static_cast<char*>(key_cache),
                   static_cast<char*>(value_cache), slots, num_tokens,
                   static_cast<int64_t>(num_blocks) * block_size, num_kv_heads, head_dim, block_size, k_scale,
                   v_scale};
}

// Launch `Op` (reshape alone, or upload + reshape) with the write for
// (dtype, kv_dtype); `chunks` write threads.
template <typename Op>
hipError_t by_write(const Op& op, pa_dtype dtype, pa_dtype kv_dtype) {
  if (kv_dtype == PA_FP8_E4M3) {
    if (dtype == PA_F32) return op.template run<QuantWrite<TF32, TE4M3>>();
    if (dtype == PA_F16) return op.template run<QuantWrite<TF16, TE4M3>>();
    return op.template run<QuantWrite<TBF16, TE4M3>>();
  }
  if (kv_dtype == PA_INT8) {
    if (dtype == PA_F32) return op.template run<QuantWrite<TF32, TI8>>();
    if (dtype == PA_F16) return op.template run<QuantWrite<TF16, TI8>>();
    return op.template run<QuantWrite<TBF16, TI8>>();
  }
  if (dtype == PA_F32) return op.template run<PlainWrite<4>>();
  return op.template run<PlainWrite<2>>();
}

struct ReshapeOp {
  WriteArgs a;
  int64_t chunks;
  hipStream_t stream;
  template <typename W>
  hipError_t run() const {
    launch_kernel(reshape_and_cache_kernel<W>, dim3(static_cast<uint32_t>((chunks + 255) / 256)), dim3(256),
                       stream, a);
    return hipGetLastError();
  }
};

struct UploadAndWriteOp {
  WriteArgs a;
  int64_t chunks;
  uint32_t* dst;
  const uint32_t* src;
  int64_t words;
  hipStream_t stream;
  const int32_t* host_slots;  // the slot mapping readable here (no two tokens in one block), or null
  bool nt;                    // element-wise write with non-temporal stores (no two tokens in one block)
  bool tile;                  // whole-tile write (no two tokens in one block; host_slots set)
  template <typename W>
  hipError_t run() const {
    int64_t up = (words + 255) / 256;
    if (up > 64) up = 64;  // the index block is a few KB to a few hundred KB
    if (up < 1) up = 1;
    if (tile && a.num_tokens <= kArgSlots) {
      ArgSlots arg;
      for (int32_t i = 0; i < kArgSlots; ++i) arg.v[i] = i < a.num_tokens ? host_slots[i] : -1;
      const int64_t wr = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads;
      launch_kernel(upload_and_cache_tiles_kernel<W, true>, dim3(static_cast<uint32_t>(up + wr)), dim3(256), stream,
                    a, dst, src, words, static_cast<int32_t>(up), arg);
    } else if (tile) {
      launch_kernel(upload_and_cache_tiles_kernel<W, false>, dim3(static_cast<uint32_t>(up + a.num_tokens)),
                         dim3(256), stream, a, dst, src, words, static_cast<int32_t>(up), ArgSlots{});
    } else {
      const int64_t wr = (chunks + 255) / 256;
      if (nt && host_slots && a.num_tokens <= kArgSlots) {
        ArgSlots arg;
        for (int32_t i = 0; i < kArgSlots; ++i) arg.v[i] = i < a.num_tokens ? host_slots[i] : -1;
        launch_kernel(upload_and_cache_kernel<W, true, true>, dim3(static_cast<uint32_t>(up + wr)), dim3(256),
                      stream, a, dst, src, words, static_cast<int32_t>(up), arg);
      } else if (nt) {
        launch_kernel(upload_and_cache_kernel<W, true, false>, dim3(static_cast<uint32_t>(up + wr)),
                           dim3(256), stream, a, dst, src, words, static_cast<int32_t>(up), ArgSlots{});
      } else {
        launch_kernel(upload_and_cache_kernel<W, false, false>, dim3(static_cast<uint32_t>(up + wr)),
                           dim3(256), stream, a, dst, src, words, static_cast<int32_t>(up), ArgSlots{});
      }
    }
    return hipGetLastError();
  }
};

int64_t write_chunks(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype) {
  const int32_t e = dtype == PA_F32 ? 4 : 2;
  return static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim * e / 16);
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t elem_bytes, int32_t block_size, hipStream_t stream) {
  const pa_dtype dt = elem_bytes == 4 ? PA_F32 : PA_F16;
  const int64_t chunks = write_chunks(num_tokens, num_kv_heads, head_dim, dt);
  if (chunks == 0) return hipSuccess;
  return by_write(ReshapeOp{write_args(key, value, key_cache, value_cache, slot_mapping, num_tokens, num_blocks,
                                       num_kv_heads, head_dim, block_size, 1.f, 1.f),
                            chunks, stream},
                  dt, dt);
}

hipError_t launch_reshape_and_cache_quant(const void* key, const void* value, void* key_cache, void* value_cache,
                                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pa_dtype dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                                          hipStream_t stream) {
  const int64_t chunks = write_chunks(num_tokens, num_kv_heads, head_dim, dtype);
  if (chunks == 0) return hipSuccess;
  return by_write(ReshapeOp{write_args(key, value, key_cache, value_cache, slot_mapping, num_tokens, num_blocks,
                                       num_kv_heads, head_dim, block_size, k_scale, v_scale),
                            chunks, stream},
                  dtype, kv_dtype);
}

hipError_t launch_reshape_and_cache_rows(const void* key, const void* value, void* key_cache, void* value_cache,
                                         const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                         hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
  if (rows == 0) return hipSuccess;
  const WriteArgs a = write_args(key, value, key_cache, value_cache, slot_mapping, num_tokens, num_blocks,
                                 num_kv_heads, head_dim, block_size, 1.f, 1.f);
  const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
#define PA_ROWS(T, D) launch_kernel(reshape_and_cache_rows_kernel<T, D>, grid, dim3(256), stream, a)
  if (head_dim == 64) {
    if (dtype == PA_F32) PA_ROWS(TF32, 64);
    else if (dtype == PA_F16) PA_ROWS(TF16, 64);
    else PA_ROWS(TBF16, 64);
  } else {
    if (dtype == PA_F32) PA_ROWS(TF32, 128);
    else if (dtype == PA_F16) PA_ROWS(TF16, 128);
    else PA_ROWS(TBF16, 128);
  }
#undef PA_ROWS
  return hipGetLastError();
}

hipError_t launch_upload_and_cache(void* dst, const void* src_device_view, int64_t nbytes, const void* key,
                                   const void* value, void* key_cache, void* value_cache,
                                   const int32_t* slot_mapping_device_view, int32_t num_tokens,
                                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   pa_dtype dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                                   int32_t write_form, const int32_t* host_slots, hipStream_t stream) {
  const int64_t chunks = write_chunks(num_tokens, num_kv_heads, head_dim, dtype);
  const int64_t words = nbytes / 4;
  if (chunks == 0 && words == 0) return hipSuccess;
  const int32_t* tiles = num_tokens > 0 && write_form == 2 ? host_slots : nullptr;
  const bool nt = write_form == 1;
  const int32_t* arg_slots = nt ? host_slots : nullptr;
  return by_write(UploadAndWriteOp{write_args(key, value, key_cache, value_cache, slot_mapping_device_view,
                                              num_tokens, num_blocks, num_kv_heads, head_dim, block_size, k_scale,
                                              v_scale),
                                   chunks, static_cast<uint32_t*>(dst), static_cast<const uint32_t*>(src_device_view),
                                   words, stream, tiles ? tiles : arg_slots, nt, tiles != nullptr},
                  dtype, kv_dtype);
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  // about 4 chunks per thread per workgroup pass; at least one workgroup
  int64_t gx = (chunks + 1023) / 1024;
  if (gx < 1) gx = 1;
  launch_kernel(copy_blocks_kernel, dim3(static_cast<uint32_t>(gx * num_pairs), 2), dim3(256),
                     stream, static_cast<char*>(key_cache), static_cast<char*>(value_cache), pairs,
                     num_blocks, chunks, static_cast<int32_t>(gx));
  return hipGetLastError();
}

}  // namespace pa
