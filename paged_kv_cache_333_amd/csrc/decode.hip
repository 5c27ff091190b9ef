// Paged decode attention for gfx950: single pass, split partials, and the
// log-sum-exp merge of partials.
//
// What is computed ("PagedAttention 实现细节" §3.1 index-based kernel: token t
// of a sequence lives in block table[t / bs] at row t % bs, read in place;
// "Ascend C算子开发高阶实战…" §三/§四: gather, QK^T, softmax and OV fused in one
// pass with an online softmax and fp32 accumulation):
//   out[s,h] = sum_t softmax_t(scale * <q[s,h], K_t>) V_t over t < ctx[s],
// with K_t, V_t taken from KV head h / (H / H_kv).
//
// Work decomposition.  A workgroup of kWaves waves owns one (sequence, group
// of GT query heads that share a KV head, token range).  The range is the
// whole context (single pass) or one partition (split).  Wave w takes blocks
// w, w + kWaves, ... of the range.  Inside a wave, a token row of the K/V tile
// (head_dim elements) is spread over LPR lanes, 16 bytes per lane, so one
// load instruction reads RPL = 64 / LPR consecutive rows of a block, fully
// coalesced.  Each row position keeps its own online-softmax state (running
// max m, running sum l, fp32 accumulator), so the hot loop needs no cross-row
// traffic: q.K is a per-lane packed dot plus a DPP sum inside the row.  The
// per-row states are merged at the end (lane shuffles inside the wave, then
// LDS across waves) with the same rescaling rule as the split merge.  The GT
// query heads of a group reuse every K/V element loaded, so a KV element is
// read from HBM once per group.
//
// Logits are kept in base-2 units (scale folded with log2 e) so the hardware
// exp2 is used; the running max and sum are rescaled together with the
// accumulator whenever the max grows (the page's own loop rescales only the
// sum; the correct rule rescales both).
//
// Invalid device data never leads to an out-of-bounds access: a block id
// outside the pool is not read and turns the affected outputs into NaN; a
// context length outside its bound does the same.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

constexpr int kWaves = 4;

struct DecodeParams {
  void* out;
  const char* q;
  const char* kc;
  const char* vc;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* order;  // optional launch order of the sequences (a permutation), or null
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t len_limit;   // largest valid context length
  int32_t part_size;   // split only
  int32_t num_parts;   // split only
  float scale_log2;    // scale * log2(e)
};

template <typename T, int D, int BS, int GT, bool SPLIT, bool CACHED>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeParams a) {
  constexpr int EPL = T::kEPL;
  constexpr int LPR = D / EPL;   // lanes per token row
  constexpr int RPL = 64 / LPR;  // rows per wave load
  constexpr int NJ = BS / RPL;   // loads per block per pool
  constexpr int JB0 = GT >= 8 ? 2 : 8;
  constexpr int JB = NJ < JB0 ? NJ : JB0;  // loads consumed per inner step
  static_assert(NJ % JB == 0, "block rows");
  constexpr float kNegInf = -__builtin_huge_valf();

  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps the block loop and the table lookups in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane - r * LPR;
  const int groups = a.num_heads / GT;
  const int slot = blockIdx.x / groups;
  const int h0 = (blockIdx.x - slot * groups) * GT;
  // Workgroups start in blockIdx order; with a longest-first order the long
  // sequences start first and the short ones fill in behind them.
  const int s = a.order ? a.order[slot] : slot;
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(a.num_seqs)) return;
  const int kvh = h0 / (a.num_heads / a.num_kv_heads);
  const int n = a.ctx[s];
  const bool bad_len = n < 0 || n > a.len_limit;

  int t_begin = 0, t_end = bad_len ? 0 : n;
  if constexpr (SPLIT) {
    t_begin = blockIdx.y * a.part_size;
    if (bad_len || t_begin >= n) return;  // nothing to write for this partition
    t_end = min(t_begin + a.part_size, n);
  }
  const int b_begin = t_begin / BS;
  const int b_end = (t_end + BS - 1) / BS;
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.max_blocks;

  u32x4 qv[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g)
    qv[g] = load16(a.q + ((static_cast<int64_t>(s) * a.num_heads + h0 + g) * D + c * EPL) * T::kBytes);

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }
  int bad = 0;

  for (int b = b_begin + wave; b < b_end; b += kWaves) {
    const int32_t phys = trow[b];
    if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_blocks)) {
      bad = 1;
      continue;
    }
    const int64_t row0 = (static_cast<int64_t>(phys) * a.num_kv_heads + kvh) * BS + r;
    const char* kp = a.kc + (row0 * D + c * EPL) * T::kBytes;
    const char* vp = a.vc + (row0 * D + c * EPL) * T::kBytes;
    const int tok0 = b * BS + r;
#pragma unroll
    for (int j0 = 0; j0 < NJ; j0 += JB) {
      u32x4 kv[JB], vv[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int64_t off = static_cast<int64_t>((j0 + jj) * RPL) * D * T::kBytes;
        if constexpr (CACHED) {
          kv[jj] = load16(kp + off);
          vv[jj] = load16(vp + off);
        } else {
          kv[jj] = load16_stream(kp + off);
          vv[jj] = load16_stream(vp + off);
        }
      }
      bool valid[JB];
      float vf[JB][EPL];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        valid[jj] = tok0 + (j0 + jj) * RPL < t_end;
        // masked rows may hold anything (even NaN): zero them before use
        const u32x4 zero = {0u, 0u, 0u, 0u};
        to_float(T{}, valid[jj] ? vv[jj] : zero, vf[jj]);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float z[JB];
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          const float d = row_sum<LPR>(dot16(T{}, qv[g], kv[jj])) * a.scale_log2;
          z[jj] = valid[jj] ? d : kNegInf;
          mx = fmaxf(mx, z[jj]);
        }
        const float m_new = fmaxf(m[g], mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m[g] - m_use);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          const float p = fast_exp2(z[jj] - m_use);
          l[g] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = __builtin_fmaf(p, vf[jj][e], acc[g][e]);
        }
        m[g] = m_new;
      }
    }
  }

  // merge the RPL row states of this wave (partners differ only in the row)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float M = fmaxf(m[g], mo);
      const float Mu = M == kNegInf ? 0.f : M;
      const float w1 = fast_exp2(m[g] - Mu);
      const float w2 = fast_exp2(mo - Mu);
      l[g] = l[g] * w1 + lo * w2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * w1 + __shfl_xor(acc[g][e], off) * w2;
      m[g] = M;
    }
  }

  __shared__ float sm_m[kWaves][GT];
  __shared__ float sm_l[kWaves][GT];
  __shared__ float sm_acc[kWaves][GT][D];
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][g][c * EPL + e] = acc[g][e];
      if (c == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  const int any_bad = __syncthreads_or(bad);

  for (int i = threadIdx.x; i < GT * D; i += kWaves * 64) {
    const int g = i / D;
    const int d = i - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    const float Mu = M == kNegInf ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - Mu);
      L = __builtin_fmaf(sm_l[w][g], wt, L);
      A = __builtin_fmaf(sm_acc[w][g][d], wt, A);
    }
    const int64_t sh = static_cast<int64_t>(s) * a.num_heads + h0 + g;
    if constexpr (SPLIT) {
      const int64_t idx = sh * a.num_parts + blockIdx.y;
      const float qnan = __builtin_nanf("");
      if (d == 0) {
        a.ws_m[idx] = M * 0.6931471805599453f;  // back to natural-log units
        a.ws_l[idx] = any_bad ? qnan : L;
      }
      a.ws_o[idx * D + d] = any_bad ? qnan : A / L;
    } else {
      const float val = any_bad || bad_len ? __builtin_nanf("") : (L > 0.f ? A / L : 0.f);
      store_elem(T{}, a.out, sh * D + d, val);
    }
  }
}

// Log-sum-exp merge of split partials: M = max_p m_p, w_p = l_p exp(m_p - M),
// out = sum_p w_p o_p / sum_p w_p.  One workgroup per (sequence, head), one
// lane per output element.
template <typename T, int D>
__global__ __launch_bounds__(D) void lse_reduce_kernel(void* out, const float* __restrict__ ws_m,
                                                       const float* __restrict__ ws_l,
                                                       const float* __restrict__ ws_o,
                                                       const int32_t* __restrict__ ctx,
                                                       const int32_t* __restrict__ order, int32_t num_seqs,
                                                       int32_t num_heads, int32_t len_limit,
                                                       int32_t part_size, int32_t num_parts) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int slot = blockIdx.x / num_heads;
  const int h = blockIdx.x - slot * num_heads;
  const int s = order ? order[slot] : slot;  // same sequence set as the partials pass
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(num_seqs)) return;
  const int64_t sh = static_cast<int64_t>(s) * num_heads + h;
  const int d = threadIdx.x;
  const int n = ctx[s];
  if (n < 0 || n > len_limit) {
    store_elem(T{}, out, sh * D + d, __builtin_nanf(""));
    return;
  }
  const int np = (n + part_size - 1) / part_size;
  const float* mp = ws_m + sh * num_parts;
  const float* lp = ws_l + sh * num_parts;
  const float* op = ws_o + sh * num_parts * D + d;
  float M = -__builtin_huge_valf();
  for (int p = 0; p < np; ++p) M = fmaxf(M, mp[p]);
  float L = 0.f, A = 0.f;
  for (int p = 0; p < np; ++p) {
    const float w = lp[p] * fast_exp2((mp[p] - M) * kLog2e);
    L += w;
    A = __builtin_fmaf(w, op[static_cast<int64_t>(p) * D], A);
  }
  store_elem(T{}, out, sh * D + d, np == 0 ? 0.f : A / L);
}

// ---------------------------------------------------------------------------
// host-side dispatch

namespace {

template <typename T, int D, int BS, int GT, bool SPLIT>
hipError_t launch_t(const DecodeParams& p, int32_t num_seqs, bool cached, hipStream_t stream) {
  const uint32_t gx = static_cast<uint32_t>(num_seqs) * (p.num_heads / GT);
  const uint32_t gy = SPLIT ? static_cast<uint32_t>(p.num_parts) : 1u;
  if (cached)
    hipLaunchKernelGGL((decode_kernel<T, D, BS, GT, SPLIT, true>), dim3(gx, gy), dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, BS, GT, SPLIT, false>), dim3(gx, gy), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, int BS, bool SPLIT>
hipError_t by_group(const DecodeParams& p, int32_t num_seqs, int gt, bool cached, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_t<T, D, BS, 1, SPLIT>(p, num_seqs, cached, stream);
    case 2: return launch_t<T, D, BS, 2, SPLIT>(p, num_seqs, cached, stream);
    case 4: return launch_t<T, D, BS, 4, SPLIT>(p, num_seqs, cached, stream);
    case 8: return launch_t<T, D, BS, 8, SPLIT>(p, num_seqs, cached, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, bool SPLIT>
hipError_t by_shape(const DecodeParams& p, int32_t num_seqs, int d, int bs, int gt, bool cached,
                    hipStream_t stream) {
  if (d == 64 && bs == 16) return by_group<T, 64, 16, SPLIT>(p, num_seqs, gt, cached, stream);
  if (d == 64 && bs == 32) return by_group<T, 64, 32, SPLIT>(p, num_seqs, gt, cached, stream);
  if (d == 128 && bs == 16) return by_group<T, 128, 16, SPLIT>(p, num_seqs, gt, cached, stream);
  if (d == 128 && bs == 32) return by_group<T, 128, 32, SPLIT>(p, num_seqs, gt, cached, stream);
  return hipErrorInvalidValue;
}

template <bool SPLIT>
hipError_t by_dtype(const DecodeParams& p, int32_t num_seqs, pa_dtype dt, int d, int bs, int gt, bool cached,
                    hipStream_t stream) {
  switch (dt) {
    case PA_F32: return by_shape<TF32, SPLIT>(p, num_seqs, d, bs, gt, cached, stream);
    case PA_F16: return by_shape<TF16, SPLIT>(p, num_seqs, d, bs, gt, cached, stream);
    case PA_BF16: return by_shape<TBF16, SPLIT>(p, num_seqs, d, bs, gt, cached, stream);
  }
  return hipErrorInvalidValue;
}

// Largest head-group tile in {8, 4, 2, 1} dividing the group size.
int group_tile(int group) {
  for (int gt : {8, 4, 2}) if (group % gt == 0) return gt;
  return 1;
}

DecodeParams make_params(const DecodeArgs& x) {
  DecodeParams p{};
  p.out = x.out;
  p.q = static_cast<const char*>(x.query);
  p.kc = static_cast<const char*>(x.key_cache);
  p.vc = static_cast<const char*>(x.value_cache);
  p.tables = x.block_tables;
  p.ctx = x.context_lens;
  p.order = x.seq_order;
  p.num_seqs = x.num_seqs;
  p.num_heads = x.num_heads;
  p.num_kv_heads = x.num_kv_heads;
  p.max_blocks = x.max_blocks_per_seq;
  p.num_blocks = x.num_blocks;
  const int64_t cap = static_cast<int64_t>(x.max_blocks_per_seq) * x.block_size;
  p.len_limit = static_cast<int32_t>(cap < x.max_context_len ? cap : x.max_context_len);
  p.scale_log2 = x.scale * 1.4426950408889634f;
  return p;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& x, hipStream_t stream) {
  DecodeParams p = make_params(x);
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  return by_dtype<false>(p, x.num_seqs, x.dtype, x.head_dim, x.block_size, gt, x.flags & PA_DECODE_CACHED_KV,
                         stream);
}

hipError_t launch_decode_split(const DecodeArgs& x, const SplitLayout& ws, hipStream_t stream) {
  DecodeParams p = make_params(x);
  p.ws_m = ws.m;
  p.ws_l = ws.l;
  p.ws_o = ws.o;
  p.part_size = ws.partition_size;
  p.num_parts = ws.num_parts;
  const int gt = group_tile(x.num_heads / x.num_kv_heads);
  hipError_t e = by_dtype<true>(p, x.num_seqs, x.dtype, x.head_dim, x.block_size, gt,
                                x.flags & PA_DECODE_CACHED_KV, stream);
  if (e != hipSuccess) return e;
  return launch_lse_reduce(x.out, ws, x.context_lens, x.seq_order, x.num_seqs, x.num_heads, x.head_dim,
                           p.len_limit, x.dtype, stream);
}

hipError_t launch_lse_reduce(void* out, const SplitLayout& ws, const int32_t* ctx, const int32_t* order,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t len_limit,
                             pa_dtype dt, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(num_seqs) * num_heads);
#define PA_REDUCE(T, D)                                                                          \
  hipLaunchKernelGGL((lse_reduce_kernel<T, D>), grid, dim3(D), 0, stream, out, ws.m, ws.l, ws.o, \
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
