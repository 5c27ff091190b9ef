// Paged decode attention for gfx950 on the matrix cores: single pass, split
// partials, and the log-sum-exp merge of partials (kernel templates and the
// compile-time dispatch; host launchers in decode.hip).
//
// What is computed ("PagedAttention 实现细节" §3.1 index-based kernel: token t
// of a sequence lives in block table[t / bs] at row t % bs, read in place;
// "Ascend C算子开发高阶实战…" §三/§四: gather, QK^T, softmax and OV fused in one
// pass with an online softmax and fp32 accumulation):
//   out[s,h] = sum_t softmax_t(scale * <q[s,h], K_t>) V_t over t < ctx[s],
// with K_t, V_t taken from KV head h / (H / H_kv).
//
// Pools.  Keys are stored token-major, [NB, H_kv, bs, D]; values dim-major,
// [NB, H_kv, D, bs] (block size innermost, the arrangement of "Ascend C算子
// 开发高阶实战…" §3.1/§5.2).  Each 16-byte load then holds 8 (4 for fp32)
// consecutive elements along the contraction axis of its product: head_dim
// for q.K, tokens for P.V, which is what a matrix-core operand wants.
//
// Work decomposition.  A workgroup of kWaves waves serves one (sequence, NC
// columns that share a KV head: query heads, or with several query tokens per
// sequence, (query token, head) pairs).  Single pass: the waves share the whole
// context, wave w taking steps w, w + kWaves, ... of TS tokens (32 for
// fp16/bf16, 16 for fp32), and merge through LDS at the end.  Split: each wave
// owns one partition outright and writes its partial (m, l, o) itself, so a
// workgroup covers kWaves consecutive partitions with no barrier.  In a step,
// with lane = 16 q + n:
//   * q.K: one 16x16 tile per 16 tokens, C[m][n'] = sum_d K[tok(m)][d] Q[n'][d]
//     on v_mfma_f32_16x16x32_{f16,bf16} (fp32: 16x16x4).  Column n' of Q is
//     column n' % NC, so the NC columns are replicated to fill the 16 and
//     every lane ends up holding logits of one column.  Token rows
//     are permuted so that lane (q, n) receives tokens EPL q .. EPL q + EPL-1
//     of the step, exactly the slice it supplies to P.V.
//   * online softmax per head on those EPL logits per lane: running max (made
//     common to the four lanes of a column with two cross-row max steps),
//     running sum, rescale of the accumulator when the max grows.
//   * P.V: out^T tile C[m][d'] = sum_t P[m][t] V[t][d'], one product per 16
//     output dims; P never leaves the registers that computed it.  For bf16,
//     P is split into a bf16 high part and a bf16 residual (two products) so
//     the weights keep ~16 significant bits; fp16 P keeps 11, and over
//     row-scaled pools an fp16 high part and residual (~22 bits).
// Each KV element is loaded once per workgroup; the NC columns share it.
//
// Several query tokens per sequence (speculative verification): query token i
// of a span of L sits at position n - L + i and sees positions up to it.  The
// columns of a tile are heads x consecutive query tokens; each lane applies its
// column's causal limit in the last steps, and value rows are zeroed only past
// the tile's furthest limit.
//
// int8 pools with a scale per (token, KV head) (storage type TI8T): each tile
// holds its codes, then a scale area of whole 128-byte lines (an unpadded
// 16-row tile would leave half of all code rows straddling two lines: back to
// back, the decode measured 117 instead of 110 us); with 16-token blocks the
// key and value scales of a block share the key tile's one scale line
// (device_common.hpp, TI8T).  With the
// step's other loads, lane i loads the key scale and the value scale of the
// step's token i; lane (q, n) takes those of its tokens 16 q + e from lane e
// of its row (a DPP row broadcast), so the scales cost two registers in
// flight.  The key scale multiplies the lane's logit of that token, and the
// value scale its weight p before P.V (the running sum l stays unscaled), so
// the codes still go to the matrix cores widened as they are.
//
// Logits are kept in base-2 units (scale folded with log2 e) so the hardware
// exp2 is used.  Tokens past the context are masked by select (never by
// multiplying by 0), and their value columns are zeroed before the product,
// so NaN garbage in unused rows cannot leak.  The merge of the waves (LDS) and
// of the split partials uses the same rescaling rule.  Reduction order depends
// only on logical token positions, so relabelling physical blocks gives
// bit-identical results.
//
// Masked positions.  With mask arrays, positions mask_lo[s] <= t < mask_hi[s]
// are left out: their logits are -inf and their value rows are zeroed, a step
// wholly inside the interval is not visited (nor its block ids checked), and
// when the interval covers the start of the range the walk starts at the first
// step that reaches past it (a sliding window skips everything before it).
// A block wholly inside the interval is never read, so its table entry may be
// anything (a window's dropped blocks).  No token left: a zero row.
//
// Invalid device data never leads to an out-of-bounds access: a block id
// outside the pool is not read and turns the affected outputs into NaN; a
// context length outside its bound does the same.
#pragma once

#include <math.h>

#include <type_traits>

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
  // optional per-sequence masked positions [mask_lo, mask_hi) (a prefix hole, or the
  // tokens before a sliding window), or null; not used by the fused write
  const int32_t* mask_lo;
  const int32_t* mask_hi;
  // query tokens: rows q_start[s] .. q_start[s+1]-1 of q/out belong to sequence s
  // (several causal query tokens, pa_decode_multi); null: row s, one token.  The
  // NC columns of a q.K tile carry 2^col_heads_log2 heads x NC / 2^col_heads_log2
  // query tokens; q_chunks workgroups cover one (sequence, head group) along the
  // tokens.  ws_len (split with q_start): per query row, its causal context length.
  const int32_t* q_start;
  int32_t num_q_rows;  // rows of q/out when q_start is set
  // Shared-prefix pass (with q_start, split): "sequence" s is a group of
  // sequences q_start[s] .. q_start[s+1]-1; member i's first ctx[i] tokens sit
  // in the same blocks as those of the member with the largest ctx (its prefix
  // length); a tile of members reads up to its longest prefix through that
  // member's table row, each member's query seeing its own ctx[i] tokens, and
  // the partials land in the members' rows.
  int32_t shared;
  int32_t col_heads_log2;
  int32_t q_chunks;
  int32_t* ws_len;
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
  // Split only, nonzero: a flat launch.  Wave item blockIdx.x * kWaves + wave
  // below n_lead is partition item / units of unit item % units (units =
  // n_lead / num_parts, the launch's (sequence, head group, query chunk)
  // units, what blockIdx.x is otherwise), so a partition count that kWaves
  // does not divide leaves no wave idle.  The items go partition by partition:
  // with one resident round, the k-th workgroup a compute unit receives takes
  // partition k, and the last (the shortest, and the youngest, which the
  // memory system serves last) ends sooner than in unit order.  (With n_lead
  // 0, item is partition item % num_parts of unit item / num_parts.)  Never
  // with the fused write.
  int32_t flat;
  // Flat launch of the shared-prefix decode, nonzero: wave items n_lead .. n_lead + n_own - 1
  // (after the groups' prefix partitions) are each query row's own tokens: item n_lead + u
  // takes row u / tiles (tiles = num_heads / 2^col_heads_log2) and its head tile u % tiles,
  // reads [own_lo[row], own_ctx[row]) of the row's own table, and writes its partial (m, l,
  // o) to own_m / own_l [row x heads] and own_o [row x heads x D].
  int32_t n_lead;
  int32_t n_own;
  const int32_t* own_ctx;
  const int32_t* own_lo;
  float* own_m;
  float* own_l;
  float* own_o;
  float scale_log2;    // scale * k_scale * log2(e)
  float v_scale;       // multiplies the output (8-bit value pools; 1 otherwise)
  // fused slot-mapping write (pa_decode_append): new K/V rows [num_seqs, H_kv, D],
  // the slot of each sequence's new token, and the workgroups after the decode's
  // own that store them
  const char* new_k;
  const char* new_v;
  const int32_t* slots;
  int32_t append_wgs;
};

// The fused slot-mapping write of pa_decode_append.  The decode does not wait
// for the new tokens to reach the pools: the wave whose step holds position
// p = ctx - 1 of a sequence takes that token's key row and value column from
// the new rows themselves (a lane's key row is loaded from the new row instead
// of the pool; the value element of p is put into the lane's value chunk after
// its load), so its products see exactly what the pools will hold.  The
// stores are made by append_wgs extra workgroups at the end of the grid, which
// start as the decode's last workgroups drain.  A decode wave may load the
// lines they write at the same time: every byte it keeps there is unchanged by
// the write, and the byte of p it replaces.  A slot outside the pool (or
// negative) writes nothing and the decode then reads the pool at p, as
// pa_reshape_and_cache followed by the decode would.
//
// Wave i of the writers stores (sequence, KV head) pairs i, i + waves, ...:
// the key row as one contiguous run, the value column element by element,
// both non-temporal (no partly written line stays in the L2 for the next
// reader to pay for).
template <typename T, int D, int BS>
__device__ __forceinline__ void write_new_rows(const DecodeParams& a, int wg) {
  typedef typename std::conditional<T::kBytes == 4, uint32_t, uint16_t>::type word_t;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t pairs = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int64_t pool_slots = static_cast<int64_t>(a.num_blocks) * BS;
  const word_t* nk = reinterpret_cast<const word_t*>(a.new_k);
  const word_t* nv = reinterpret_cast<const word_t*>(a.new_v);
  word_t* kc = reinterpret_cast<word_t*>(const_cast<char*>(a.kc));
  word_t* vc = reinterpret_cast<word_t*>(const_cast<char*>(a.vc));
  for (int64_t i = static_cast<int64_t>(wg) * kWaves + wave; i < pairs;
       i += static_cast<int64_t>(a.append_wgs) * kWaves) {
    const int s = static_cast<int>(i / a.num_kv_heads);
    const int h = static_cast<int>(i - static_cast<int64_t>(s) * a.num_kv_heads);
    const int64_t slot = a.slots[s];
    if (slot < 0 || slot >= pool_slots) continue;
    const int64_t blk = slot / BS, off = slot - blk * BS;
    const int64_t tile = blk * a.num_kv_heads + h;
#pragma unroll
    for (int d = lane; d < D; d += 64) {
      __builtin_nontemporal_store(nk[i * D + d], kc + (tile * BS + off) * D + d);
      __builtin_nontemporal_store(nv[i * D + d], vc + (tile * D + d) * BS + off);
    }
  }
}

// T is the query/output type and the type the matrix cores compute in; S is
// the pools' storage type: T itself, or an 8-bit code type (TE4M3, TI8) whose
// chunks are widened exactly to T in registers after the load.
// GT is NC, the number of distinct columns of a q.K tile: query heads that
// share a KV head times query tokens of the same sequence (one token: heads).
template <typename T, typename S, int D, int BS, int GT, bool SPLIT, bool CACHED, bool APPEND>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void decode_kernel(DecodeParams a) {
  constexpr int NC = GT;
  constexpr bool Q8 = S::kBytes == 1;  // 8-bit codes
  constexpr bool ROWS = row_scaled<S>::value;  // a scale per (token, KV head) in each tile
  constexpr int EPL = T::kEPL;       // compute elements per 16-byte chunk
  constexpr int E = T::kBytes;
  constexpr int SE = S::kEPL;        // stored elements per 16-byte load
  constexpr int SB = S::kBytes;
  constexpr int KV = D / EPL / 4;    // q.K products per 16-token tile
  constexpr int KL = D / SE / 4;     // key loads per 16-token tile and lane (chunks 4l + q of a row)
  constexpr int NT = SE / 4;         // 16-token q.K tiles per step
  constexpr int TPL = SE;            // tokens per lane in P.V (= 4 NT)
  constexpr int TS = 16 * NT;        // tokens per step
  constexpr int NV = D / 16;         // value loads per step, 16 output dims each
  constexpr int PV = TPL / EPL;      // P.V products per 16 output dims (2 for 8-bit codes)
  constexpr int NBS = TS > BS ? TS / BS : 1;  // blocks touched by one step
  // bytes of one (block, KV head) tile: its codes or elements, then (ROWS) the scale area
  // (whole 128-byte lines, so every tile's rows stay line-aligned); PAIRED: the key tile's
  // area holds the value scales too (TI8T)
  constexpr int64_t KT = static_cast<int64_t>(BS) * D * SB + (ROWS ? token_scale_area(BS) : 0);
  constexpr bool PAIRED = ROWS && token_scales_paired(BS);
  // P.V runs in TP: the query type, except over 8-bit pools, whose codes are
  // exact in fp16 (and P is in [0, 1]): fp16 there, one product per chunk
  // instead of bf16's high part + residual, and the cheaper fp16 widening.
  using TP = typename std::conditional<Q8, TF16, T>::type;
  // Weights enter P.V as a high part plus a residual (two products) for bf16, whose 8
  // bits would cost accuracy everywhere, and for row-scaled pools, whose weights carry
  // each token's value scale: in one fp16 product even a token holding all the weight
  // would be off by up to 2^-12 of its value.
  constexpr bool SPLIT_P = std::is_same<TP, TBF16>::value || ROWS;
  constexpr float kNegInf = -__builtin_huge_valf();
  static_assert(NC >= 1 && NC <= 16 && (NC & (NC - 1)) == 0, "columns per tile");
  static_assert(Q8 ? T::kBytes == 2 : std::is_same<T, S>::value, "8-bit pools decode in fp16/bf16");
  static_assert(!(Q8 && APPEND), "the fused write stores model-type rows");
  static_assert(NBS <= 4 && KL * SE * 4 == D && KV * EPL * 4 == D, "step shape");
  static_assert(TPL % BS == 0 || BS % TPL == 0, "a lane's tokens never straddle a block boundary");
  static_assert(!ROWS || (TPL == 16 && TS == 64), "row scales: one token of the step per lane, 16 per row");

  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps the step loop and the table lookups in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int n = lane & 15;
  // Columns: column c = n % NC is head h0 + (c & (col_heads - 1)) for query
  // token tok0 + (c >> log2 col_heads) of the sequence.
  const int lg_h = a.col_heads_log2;
  const int col_heads = 1 << lg_h;
  const int col_toks = NC >> lg_h;
  const int groups = a.num_heads >> lg_h;
  const int per_slot = groups * a.q_chunks;
  if constexpr (APPEND) {  // the workgroups after the decode's own store the new rows
    const int64_t n_units = static_cast<int64_t>(a.num_seqs) * per_slot;
    if (static_cast<int64_t>(blockIdx.x) >= n_units) {
      if (blockIdx.y + 1 == gridDim.y) write_new_rows<T, D, BS>(a, static_cast<int>(blockIdx.x - n_units));
      return;
    }
  }
  int unit = static_cast<int>(blockIdx.x);
  int flat_part = 0;
  bool own = false;  // a query row's own tokens after the shared prefixes (DecodeParams::n_lead)
  if constexpr (SPLIT && !APPEND) {
    if (a.flat) {  // see DecodeParams::flat
      const int item = static_cast<int>(blockIdx.x) * kWaves + wave;
      if (a.n_lead > 0 && item >= a.n_lead) {
        own = true;
        unit = item - a.n_lead;
      } else if (a.n_lead > 0) {
        const int units = a.n_lead / a.num_parts;  // n_lead = units x num_parts
        flat_part = item / units;
        unit = item - flat_part * units;
      } else {
        unit = item / a.num_parts;
        flat_part = item - unit * a.num_parts;
      }
    }
  }
  // an own item's "sequence" is a query row of the batch, its unit (row, head tile)
  const int slot = own ? unit / groups : unit / per_slot;
  const int rows = own ? a.num_q_rows : a.num_seqs;
  if (slot >= rows) return;  // a flat launch's last workgroup: waves past the last unit
  const int grp = own ? unit - slot * groups : (unit - slot * per_slot) / a.q_chunks;
  const int chunk = own ? 0 : unit - slot * per_slot - grp * a.q_chunks;
  const int h0 = grp << lg_h;
  // Workgroups start in blockIdx order; with a longest-first order the long
  // sequences start first and the short ones fill in behind them.
  const int s = a.order && !own ? a.order[slot] : slot;
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(rows)) return;
  int qs = s, L = 1;  // the sequence's query rows qs .. qs + L - 1
  if (a.q_start && !own) {
    qs = a.q_start[s];
    L = a.q_start[s + 1] - qs;
    if (qs < 0 || L < 0 || qs > a.num_q_rows - L) return;  // a span outside the rows: no output
  }
  const int tok0 = chunk * col_toks;
  if (tok0 >= L) return;  // no query token for this workgroup
  const int kvh = h0 / (a.num_heads / a.num_kv_heads);
  const bool shared = a.shared != 0 && !own;  // a group's shared prefix (see DecodeParams)
  // A shared tile's members each read their own first ctx[member] tokens (their prefix
  // lengths differ); the tile reads up to the longest of them from the table row of the
  // member that has it (the first such), whose blocks hold every member's prefix.
  int sh_lo = 0, sh_hi = 0, sh_row = qs;
  if (shared) {
    sh_lo = 0x7fffffff;
    sh_hi = -1;
    const int i_end = min(tok0 + col_toks, L);
    for (int i = tok0; i < i_end; ++i) {  // wave-uniform: scalar loads
      const int e = a.ctx[qs + i];
      if (e > sh_hi) {
        sh_hi = e;
        sh_row = qs + i;
      }
      sh_lo = min(sh_lo, e);
    }
  }
  const int nctx = own ? a.own_ctx[s] : shared ? sh_hi : a.ctx[s];
  // (an empty context is valid for plain decode: a zero row; a span of query
  // tokens must lie inside the context)
  // (a group with more members than the launch's tiles cover is invalid as a
  // whole: its members get no partials, and the merge sees a -1 length)
  const bool bad_len = nctx < 0 || nctx > a.len_limit || (a.q_start && !shared && !own && L > nctx) ||
                       (shared && (sh_lo < 0 || L > a.q_chunks * col_toks)) ||
                       (own && (a.own_lo[s] < 0 || a.own_lo[s] > nctx));
  // Causal limits: query token i sits at position nctx - L + i and sees the
  // positions before nctx - L + i + 1.  This lane's column, and the tile's
  // nearest and furthest limits (all nctx for one token per sequence; each
  // member's own prefix length for the members of a shared tile).
  const int my_tok = tok0 + ((n % NC) >> lg_h);
  const int lim_base = shared ? nctx : nctx - L + 1;
  const int lane_lim = shared ? a.ctx[qs + min(my_tok, L - 1)] : lim_base + min(my_tok, L - 1);
  const int tile_lim_lo = shared ? sh_lo : lim_base + tok0;
  const int tile_lim_hi = shared ? sh_hi : lim_base + min(tok0 + col_toks, L) - 1;
  int mlo = 0, mhi = 0;  // masked positions; empty unless mask_lo < mask_hi (mask_lo null: 0)
  if (!APPEND && a.mask_hi) {
    mlo = a.mask_lo ? a.mask_lo[s] : 0;
    mhi = a.mask_hi[s];
    if (mhi <= mlo) mlo = mhi = 0;
  }
  if (own) {  // the row's shared prefix is masked: its tokens come from the group's partitions
    mlo = 0;
    mhi = bad_len ? 0 : a.own_lo[s];
  }

  // Single pass: the workgroup's waves share the context, wave w taking steps
  // w, w + kWaves, ...  Split: each wave owns one partition outright (partition
  // blockIdx.y * kWaves + wave) and writes its partial itself.
  constexpr int WSTEP = SPLIT ? 1 : kWaves;
  const int t_all = bad_len ? 0 : tile_lim_hi;  // the tile's range is [0, t_all)
  int t_begin = 0, t_end = t_all, part = 0;
  if constexpr (SPLIT) {
    // an own item reads its whole range [own_lo, nctx) in one wave
    part = own ? 0 : !APPEND && a.flat ? flat_part : static_cast<int>(blockIdx.y) * kWaves + wave;
    t_begin = own ? 0 : part * a.part_size;
    t_end = own ? t_end : min(t_begin + a.part_size, t_end);
    // the merge needs each query row's context length (any head group writes the same)
    if (!own && a.ws_len && part == 0 && grp == 0 && q == 0 && n < NC && (n & (col_heads - 1)) == 0 && my_tok < L)
      a.ws_len[qs + my_tok] = bad_len ? -1 : (shared ? lane_lim : lim_base + my_tok);
    if (shared && a.ws_len && part == 0 && grp == 0 && chunk == 0) {
      // members past the last tile of the launch: no workgroup computes them
      for (int i = a.q_chunks * col_toks + lane; i < L; i += 64) a.ws_len[qs + i] = -1;
    }
  }
  // pa_decode_append: position p = nctx - 1 is taken from the new rows (write_new_rows)
  // when the new token has a slot in the pool; -1 otherwise
  int fresh_p = -1;
  if constexpr (APPEND) {
    const int64_t slot = a.slots[s];
    if (!bad_len && nctx > 0 && slot >= 0 && slot < static_cast<int64_t>(a.num_blocks) * BS) fresh_p = nctx - 1;
  }
  if constexpr (SPLIT) {
    // nothing to read in this partition (no barrier follows); an own item always writes its
    // partial (no token: m = -inf, l = 0; an invalid row: NaN)
    if (!own && (bad_len || t_begin >= t_all)) return;
  }
  // steps wholly inside a mask that covers the start of the range are skipped
  const int st_skip = mlo <= t_begin && mhi > t_begin ? (min(mhi, t_end) - t_begin) / TS : 0;
  const int st_first = st_skip + (SPLIT ? 0 : wave);
  const int b_end = (t_end + BS - 1) / BS;
  const int32_t* trow = a.tables + static_cast<int64_t>(shared ? sh_row : s) * a.max_blocks;

  // Q operand of q.K: lane (q, n) holds column n % NC (a padding column past
  // the last query token repeats it), the dims its key chunks hold: chunk
  // 4v + q; with 8-bit keys, key load l = v / 2 holds dims 16 (4l + q) .. + 15
  // and widens into chunks 2 (4l + q) and 2 (4l + q) + 1.
  u32x4 qv[KV];
  {
    const int64_t row = static_cast<int64_t>(qs + min(my_tok, L - 1)) * a.num_heads + h0 + (n & (col_heads - 1));
    const char* qrow = a.q + row * D * E;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int c = Q8 ? 2 * (4 * (v >> 1) + q) + (v & 1) : 4 * v + q;
      qv[v] = load16(qrow + c * 16);
    }
  }

  // Online-softmax state of this lane's column (n % NC), and the P.V
  // accumulator: acc[v][j] is out^T row 4q + j (column (4q + j) % NC), dim 16v + n.
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  int bad = own && bad_len ? 1 : 0;

  const int n_steps = (t_end - t_begin + TS - 1) / TS;
  const int64_t hkv = a.num_kv_heads;
  // Block ids.  The first step's come through the scalar path, which a new
  // workgroup reaches without queueing behind the streaming loads the other
  // workgroups on its CU have in flight.  Later steps' ids are prefetched with
  // one vector load per wave: lane i holds the id of block i % NBS of the
  // wave's step k + i / NBS, for the next IDS_PER steps, so no step waits for
  // a table lookup.  Indices are clamped into the table row; an id is used
  // (and validated) only below b_end.
  constexpr int IDS_PER = 64 / NBS;  // steps covered by one prefetch
  const int mb_last = a.max_blocks - 1;
  const int lane_step = lane / NBS, lane_blk = lane - lane_step * NBS;
  auto fetch_ids = [&](int first_step) {
    const int st_l = first_step + WSTEP * lane_step;
    const int b = (t_begin + st_l * TS) / BS + lane_blk;
    return trow[min(b, mb_last)];
  };
  int32_t ph_first[NBS];
  int32_t ids = 0;
  if (mb_last >= 0) {  // needs only s, not the context length
    const int b = (t_begin + st_first * TS) / BS;
#pragma unroll
    for (int i = 0; i < NBS; ++i) ph_first[i] = trow[min(b + i, mb_last)];
    ids = fetch_ids(st_first + WSTEP);
  }
  int k_ids = -1;  // steps consumed from `ids`; -1: the first step uses ph_first
  for (int st = st_first; st < n_steps; st += WSTEP) {
    const int t0 = t_begin + st * TS;
    const int b0 = t0 / BS;
    const int off0 = t0 - b0 * BS;  // nonzero only when a step is shorter than a block
    if (k_ids == IDS_PER) {
      ids = fetch_ids(st);
      k_ids = 0;
    }
    // the step meets the masked interval / lies wholly inside it (wave-uniform)
    const int t_stop = min(t0 + TS, t_end);
    const bool meets = t0 < mhi && t_stop > mlo;
    const bool inside = t0 >= mlo && t_stop <= mhi;
    int32_t ph[NBS];
    bool skip = false;
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      ph[i] = k_ids < 0 ? ph_first[i] : __builtin_amdgcn_readlane(ids, NBS * k_ids + i);
      const int blk = b0 + i;
      const bool dead = blk >= b_end || (meets && blk * BS >= mlo && min((blk + 1) * BS, t_end) <= mhi);
      if (!dead) {
        if (static_cast<uint32_t>(ph[i]) >= static_cast<uint32_t>(a.num_blocks)) skip = true;
      } else {
        ph[i] = -1;  // no token of this block is used: masked below, read from a live block
      }
    }
    ++k_ids;
    if (inside) continue;
    if (skip) {
      bad = 1;
      continue;
    }
    {
      int32_t live = ph[0];
#pragma unroll
      for (int i = 1; i < NBS; ++i) live = live < 0 ? ph[i] : live;
#pragma unroll
      for (int i = 0; i < NBS; ++i) ph[i] = ph[i] < 0 ? live : ph[i];
    }
    // Physical block of step block bi (lane-dependent), by selects on the bits
    // of bi (a compare chain would be turned into an indexed load from a
    // stack copy of ph).
    auto pick = [&](int bi) -> int64_t {
      if constexpr (NBS == 1) {
        return ph[0];
      } else if constexpr (NBS == 2) {
        return bi ? ph[1] : ph[0];
      } else {
        const int32_t lo = bi & 1 ? ph[1] : ph[0];
        const int32_t hi = bi & 1 ? ph[3] : ph[2];
        return bi & 2 ? hi : lo;
      }
    };

    // K rows: in tile tau, lane (q, n) supplies row n = token
    // TPL (n / 4) + 4 tau + n % 4 of the step, chunks 4l + q.  The 4 tau +
    // n % 4 part stays below TPL, and TPL and BS divide one another (off0 is
    // nonzero only when NBS == 1), so the row's block does not depend on tau.
    const int bik = NBS == 1 ? 0 : (off0 + TPL * (n >> 2)) / BS;
    const int64_t kblk = pick(bik);
    // (pa_decode_append) the step holds the new token p (wave-uniform)
    const bool has_fresh = APPEND && fresh_p >= t0 && fresh_p < t0 + TS;
    const int64_t fresh_row = (static_cast<int64_t>(s) * hkv + kvh) * D;  // of the new rows, in elements
    u32x4 kr[NT][KL];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      const int x = off0 + TPL * (n >> 2) + 4 * tau + (n & 3);
      const char* kp = has_fresh && t0 + (x - off0) == fresh_p
                           ? a.new_k + fresh_row * E + q * 16
                           : a.kc + (kblk * hkv + kvh) * KT + ((x - bik * BS) * D) * SB + q * 16;
#pragma unroll
      for (int l = 0; l < KL; ++l) kr[tau][l] = CACHED ? load16(kp + l * 64) : load16_stream(kp + l * 64);
    }
    // V columns: lane (q, n) supplies dim 16v + n of tokens TPL q .. TPL q + TPL-1.
    // A block longer than a step (16-bit and fp32 elements with 64-token blocks)
    // spreads each 128-byte line of a value row over several steps, which other
    // waves read at about the same time: those loads keep the line in the L2 for
    // them (64-token fp16 blocks, decode inside the step 207 instead of 224 us;
    // after a cache flush, though, 245 instead of 222 us).
    constexpr bool V_CACHED = CACHED || BS > TS;
    u32x4 vr[NV];
    float ks1 = 1.f, vs1 = 1.f;  // (ROWS) the key and value scales of the step's token `lane`
    if constexpr (ROWS) {
      const int x = off0 + lane;
      const int bi = NBS == 1 ? 0 : x / BS;
      const int64_t sc = (pick(bi) * hkv + kvh) * KT + static_cast<int64_t>(BS) * D + (x - bi * BS) * 4;
      // streaming like the codes (plain loads that miss allocate L2 lines: measured 140 instead
      // of 108 us for the row-scaled LLaMA-7B-like decode after a cache flush)
      const float* kp1 = reinterpret_cast<const float*>(a.kc + sc);
      const float* vp1 = reinterpret_cast<const float*>(PAIRED ? a.kc + sc + 4 * BS : a.vc + sc);
      ks1 = CACHED ? *kp1 : __builtin_nontemporal_load(kp1);
      vs1 = CACHED ? *vp1 : __builtin_nontemporal_load(vp1);
    }
    {
      const int x = off0 + TPL * q;
      const int bi = NBS == 1 ? 0 : x / BS;
      const int64_t phys = pick(bi);  // bi < NBS: TPL q < TS
      const char* vp = a.vc + (phys * hkv + kvh) * KT + (n * BS + (x - bi * BS)) * SB;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        vr[v] = V_CACHED ? load16(vp + v * 16 * BS * SB) : load16_stream(vp + v * 16 * BS * SB);
    }
    // (pa_decode_append) dims 16 v + n of the new token's value row, for the lanes whose
    // tokens hold p; loaded with the step's other loads, except for fp32 (there they are
    // loaded where they are put in, since holding them through the loads spills registers)
    typedef typename std::conditional<E == 4, uint32_t, uint16_t>::type word_t;
    constexpr bool EARLY_FRESH = E != 4;
    word_t fv[APPEND ? NV : 1];
    if constexpr (APPEND && EARLY_FRESH) {
      if (has_fresh) {
        const word_t* nv = reinterpret_cast<const word_t*>(a.new_v) + fresh_row + n;
#pragma unroll
        for (int v = 0; v < NV; ++v) fv[v] = nv[16 * v];
      }
    }
    // All of the step's loads are issued before any of them is consumed.
    __builtin_amdgcn_sched_barrier(0);

    f32x4 c[NT];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      c[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (Q8) {
#pragma unroll
        for (int l = 0; l < KL; ++l) {
          u32x4 lo, hi;
          widen(S{}, T{}, kr[tau][l], lo, hi);
          c[tau] = mma(T{}, lo, qv[2 * l], c[tau]);
          c[tau] = mma(T{}, hi, qv[2 * l + 1], c[tau]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < KV; ++v) c[tau] = mma(T{}, kr[tau][v], qv[v], c[tau]);
      }
    }
    // c[tau][j]: logit of token t0 + TPL q + 4 tau + j for column n % NC.  In
    // a ragged step (the context or a query token's causal limit ends, or the
    // masked interval starts or ends, inside it) bit e of `use` says whether
    // the lane's token TPL q + e counts for its column, and bit e of `vuse`
    // whether it counts for any column (the value rows to keep).
    const bool ragged = t0 + TS > min(t_end, tile_lim_lo) || meets;
    uint32_t use = ~0u, vuse = ~0u;
    if (ragged) {
      const int base = t0 + TPL * q;
      const uint32_t hole = low_bits(mhi - base) & ~low_bits(mlo - base);
      use = low_bits(min(t_end, lane_lim) - base) & ~hole;
      vuse = low_bits(t_end - base) & ~hole;
    }
    float z[TPL];
    float mx = kNegInf;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = c[tau][j] * a.scale_log2;
        if constexpr (ROWS) v *= row_bcast(ks1, 4 * tau + j);  // the scale of token TPL q + 4 tau + j
        const bool ok = !ragged || ((use >> (4 * tau + j)) & 1u);
        z[4 * tau + j] = ok ? v : kNegInf;
        mx = fmaxf(mx, z[4 * tau + j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float p[TPL];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < TPL; ++e) {
      p[e] = fast_exp2(z[e] - m_use);
      ps += p[e];
    }
    l_run = l_run * alpha + ps;
    if constexpr (ROWS) {
      // weights of the value codes: p times the value row's scale; a token no column
      // uses (its scale may be anything) weighs exactly 0
#pragma unroll
      for (int e = 0; e < TPL; ++e) {
        const float sv = row_bcast(vs1, e);
        p[e] = !ragged || ((vuse >> e) & 1u) ? p[e] * sv : 0.f;
      }
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
      // acc[.][j] belongs to column (4q + j) % NC; its factor sits in a lane
      // of the same row whose column is that one.
      float al[4];
      if constexpr (4 % NC == 0) {
        al[0] = quad_bcast<0>(alpha);
        al[1] = quad_bcast<1>(alpha);
        al[2] = quad_bcast<2>(alpha);
        al[3] = quad_bcast<3>(alpha);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 16 * q + (4 * q + j) % NC);
      }
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[v][j] *= al[j];
    }
    // P in chunks of the compute type: chunk u holds tokens TPL q + EPL u ..
    u32x4 phi[PV], plo[PV];
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      if constexpr (SPLIT_P)
        pack_p_split(TP{}, p + EPL * u, phi[u], plo[u]);
      else
        pack_p(TP{}, p + EPL * u, phi[u], plo[u]);
    }
    if constexpr (APPEND) {
      const int e = fresh_p - t0 - TPL * q;  // the lane's element holding p, if any
      if (has_fresh && e >= 0 && e < TPL) {
        if constexpr (!EARLY_FRESH) {
          const word_t* nv = reinterpret_cast<const word_t*>(a.new_v) + fresh_row + n;
#pragma unroll
          for (int v = 0; v < NV; ++v) fv[v] = nv[16 * v];
        }
        const int wi = E == 4 ? e : e >> 1;
        const uint32_t sh = E == 4 ? 0u : static_cast<uint32_t>(e & 1) * 16u;
        const uint32_t hole = E == 4 ? 0u : ~(0xFFFFu << sh);
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i == wi) vr[v][i] = (vr[v][i] & hole) | (static_cast<uint32_t>(fv[v]) << sh);
      }
    }
    if (ragged) {
      const u32x4 keep = bits_mask(S{}, vuse);
#pragma unroll
      for (int v = 0; v < NV; ++v) vr[v] &= keep;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      u32x4 vc[PV];
      if constexpr (Q8)
        widen(S{}, TP{}, vr[v], vc[0], vc[PV - 1]);
      else
        vc[0] = vr[v];
#pragma unroll
      for (int u = 0; u < PV; ++u) {
        acc[v] = mma(TP{}, phi[u], vc[u], acc[v]);
        if constexpr (SPLIT_P) acc[v] = mma(TP{}, plo[u], vc[u], acc[v]);
      }
    }
  }

  // the four lanes of a column summed disjoint tokens with a common max
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  if constexpr (SPLIT) {
    // This wave's partition: (m_p in natural-log units, l_p, o_p = acc / l_p)
    // for each of the NC columns.  acc[.][j] belongs to column (4q + j) % NC,
    // whose l sits in a lane of the same row (see the rescale above).
    float lg[4];
    if constexpr (4 % NC == 0) {
      lg[0] = quad_bcast<0>(l_run);
      lg[1] = quad_bcast<1>(l_run);
      lg[2] = quad_bcast<2>(l_run);
      lg[3] = quad_bcast<3>(l_run);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) lg[j] = __shfl(l_run, 16 * q + (4 * q + j) % NC);
    }
    const float qnan = __builtin_nanf("");
    // output row of column c (query row x heads + head), or -1 for a padding column
    auto out_row = [&](int c) -> int64_t {
      const int tok = tok0 + (c >> lg_h);
      return tok < L ? static_cast<int64_t>(qs + tok) * a.num_heads + h0 + (c & (col_heads - 1)) : -1;
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * q + j;  // first replica of each column
      const int64_t r = g < NC ? out_row(g) : -1;
      if (r >= 0) {
        float* o = own ? a.own_o + r * D + n : a.ws_o + (r * a.num_parts + part) * D + n;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          o[16 * v] = bad ? qnan : (lg[j] == 0.f ? 0.f : acc[v][j] / lg[j] * a.v_scale);  // 0: all masked
      }
    }
    const int64_t rn = q == 0 && n < NC ? out_row(n) : -1;
    if (rn >= 0) {
      const int64_t idx = own ? rn : rn * a.num_parts + part;
      (own ? a.own_m : a.ws_m)[idx] = m_run * 0.6931471805599453f;  // back to natural-log units
      (own ? a.own_l : a.ws_l)[idx] = bad ? qnan : l_run;
    }
    return;
  }

  __shared__ float sm_m[kWaves][NC];
  __shared__ float sm_l[kWaves][NC];
  __shared__ float sm_acc[kWaves][NC][D];
  if (q == 0 && n < NC) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_run;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * q + j;  // first replica of each column
    if (g < NC) {
#pragma unroll
      for (int v = 0; v < NV; ++v) sm_acc[wave][g][16 * v + n] = acc[v][j];
    }
  }
  const int any_bad = __syncthreads_or(bad);

  for (int i = threadIdx.x; i < NC * D; i += kWaves * 64) {
    const int g = i / D;
    const int d = i - g * D;
    const int tok = tok0 + (g >> lg_h);
    if (tok >= L) continue;  // a padding column
    const int64_t sh = static_cast<int64_t>(qs + tok) * a.num_heads + h0 + (g & (col_heads - 1));
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    const float Mu = M == kNegInf ? 0.f : M;
    float Lsum = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - Mu);
      Lsum = __builtin_fmaf(sm_l[w][g], wt, Lsum);
      A = __builtin_fmaf(sm_acc[w][g][d], wt, A);
    }
    const float val = any_bad || bad_len ? __builtin_nanf("") : (Lsum > 0.f ? A / Lsum * a.v_scale : 0.f);
    store_elem(T{}, a.out, sh * D + d, val);
  }
}

// Log-sum-exp merge of split partials: M = max_p m_p, w_p = l_p exp(m_p - M),
// out = sum_p w_p o_p / sum_p w_p.  A workgroup owns 32 output dims (slice
// blockIdx.y) of one (row, head): thread t takes dims 4 (t % 8) .. +3 of the
// slice and partitions t / 8, t / 8 + 32, ...  A round issues all of a thread's
// loads of 8 partitions (8 x 16 bytes of o, and their m and l) before the first
// is used, so a whole 256-partition context is in flight at once.  Each thread
// keeps its own running max and rescales its sums when it grows; the 32
// partition rows are then brought to the common max and summed across lanes
// and, for the four waves, through LDS.  The summation order depends only on
// the partition count, not on timing.
template <typename T, int D>
__global__ __launch_bounds__(256) void lse_reduce_kernel(void* out, const float* __restrict__ ws_m,
                                                         const float* __restrict__ ws_l,
                                                         const float* __restrict__ ws_o,
                                                         const int32_t* __restrict__ ctx,
                                                         const int32_t* __restrict__ order, int32_t num_seqs,
                                                         int32_t num_heads, int32_t len_limit,
                                                         int32_t part_size, int32_t num_parts) {
  static_assert(D % 32 == 0, "dims in slices of 32");
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kNegInf = -__builtin_huge_valf();
  constexpr int kRows = 32;   // partition rows of a workgroup
  constexpr int kRound = 8;   // partitions per thread per round
  const int slot = blockIdx.x / num_heads;
  const int h = blockIdx.x - slot * num_heads;
  const int s = order ? order[slot] : slot;  // same sequence set as the partials pass
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(num_seqs)) return;
  const int64_t sh = static_cast<int64_t>(s) * num_heads + h;
  const int d_lo = 32 * static_cast<int>(blockIdx.y);
  const int n = ctx[s];
  if (n < 0 || n > len_limit) {
    if (threadIdx.x < 32) store_elem(T{}, out, sh * D + d_lo + threadIdx.x, __builtin_nanf(""));
    return;
  }
  const int np = (n + part_size - 1) / part_size;
  const float* mp = ws_m + sh * num_parts;
  const float* lp = ws_l + sh * num_parts;
  const float* op = ws_o + sh * num_parts * D + d_lo + 4 * (threadIdx.x & 7);
  const int row = threadIdx.x >> 3;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  float m = kNegInf, L = 0.f, A[4] = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < np; base += kRows * kRound) {
    float mv[kRound], lv[kRound];
    float4 ov[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int p = base + row + kRows * u;
      if (p < np) {
        mv[u] = mp[p];
        lv[u] = lp[p];
        ov[u] = *reinterpret_cast<const float4*>(op + static_cast<int64_t>(p) * D);
      } else {
        mv[u] = kNegInf;
        lv[u] = 0.f;
        ov[u] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < kRound; ++u) mc = fmaxf(mc, mv[u]);
    // sums so far are re-based to the new max (nothing to re-base while L is 0)
    const float r = L == 0.f ? 0.f : fast_exp2((m - mc) * kLog2e);
    L *= r;
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] *= r;
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      // a partition with no token (l = 0, m = -inf: all masked) has no weight
      const float w = lv[u] == 0.f ? 0.f : lv[u] * fast_exp2((mv[u] - mc) * kLog2e);
      L += w;
      A[0] = __builtin_fmaf(w, ov[u].x, A[0]);
      A[1] = __builtin_fmaf(w, ov[u].y, A[1]);
      A[2] = __builtin_fmaf(w, ov[u].z, A[2]);
      A[3] = __builtin_fmaf(w, ov[u].w, A[3]);
    }
    m = mc;
  }

  // common max of the 32 rows: lanes 8 apart hold other rows of the wave
  __shared__ float sm_max[4];
  __shared__ float sm_l[4];
  __shared__ float sm_a[4][32];
  float M = m;
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) sm_max[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sm_max[0], sm_max[1]), fmaxf(sm_max[2], sm_max[3]));
  const float f = L == 0.f ? 0.f : fast_exp2((m - M) * kLog2e);
  L *= f;
#pragma unroll
  for (int k = 0; k < 4; ++k) A[k] *= f;
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    L += __shfl_xor(L, off);
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] += __shfl_xor(A[k], off);
  }
  if (lane == 0) sm_l[wave] = L;
  if (lane < 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sm_a[wave][4 * lane + k] = A[k];
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const int d = threadIdx.x;
    const float Ls = (sm_l[0] + sm_l[1]) + (sm_l[2] + sm_l[3]);
    const float As = (sm_a[0][d] + sm_a[1][d]) + (sm_a[2][d] + sm_a[3][d]);
    store_elem(T{}, out, sh * D + d_lo + d, Ls == 0.f ? 0.f : As / Ls);
  }
}


// The same merge for rows of few partials (at most kSmallParts, the extra one
// included): one wave per (row, head), lane l holding dims EL l .. EL l + EL - 1
// (EL = D / 64), every partial's loads issued at once.  The rule and the
// handling of empty and invalid partials are those of lse_reduce_kernel; the
// summation runs in partition order.
//
// With an extra partial (x, the shared-prefix decode's own tokens), row (s, h)
// merges its partitions and then (x.m, x.l, x.o)[s, h], as one more partition;
// and x.expect[s] must equal ctx[s] (the prefix the partitions covered), else
// the row is NaN.  Every slot a row can hold (num_parts of them, and the extra
// partial) is loaded together with the row's length, which then only selects
// among them: one round trip per row, not two.
constexpr int kSmallParts = 16;
template <typename T, int D>
__global__ __launch_bounds__(256) void lse_merge_small_kernel(void* out, const float* __restrict__ ws_m,
                                                              const float* __restrict__ ws_l,
                                                              const float* __restrict__ ws_o,
                                                              const int32_t* __restrict__ ctx,
                                                              const int32_t* __restrict__ order, int32_t num_seqs,
                                                              int32_t num_heads, int32_t len_limit, int32_t part_size,
                                                              int32_t num_parts, ExtraPartial x) {
  constexpr int EL = D / 64;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kNegInf = -__builtin_huge_valf();
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(num_seqs) * num_heads) return;
  const int slot = static_cast<int>(item / num_heads);
  const int h = static_cast<int>(item - static_cast<int64_t>(slot) * num_heads);
  const int s = order ? order[slot] : slot;
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(num_seqs)) return;
  const int64_t sh = static_cast<int64_t>(s) * num_heads + h;
  // the slots, loaded before the length is known (num_parts is uniform; a slot past the
  // row's partitions is in the workspace and is left out of the sums below)
  const int slots = min(num_parts, kSmallParts);
  float mv[kSmallParts], lv[kSmallParts], ov[kSmallParts][EL];
#pragma unroll
  for (int p = 0; p < kSmallParts; ++p) {
    mv[p] = kNegInf;
    lv[p] = 0.f;
#pragma unroll
    for (int i = 0; i < EL; ++i) ov[p][i] = 0.f;
    if (p < slots) {
      mv[p] = ws_m[sh * num_parts + p];
      lv[p] = ws_l[sh * num_parts + p];
#pragma unroll
      for (int i = 0; i < EL; ++i) ov[p][i] = ws_o[(sh * num_parts + p) * D + EL * lane + i];
    }
  }
  float xm = kNegInf, xl = 0.f, xo[EL];
#pragma unroll
  for (int i = 0; i < EL; ++i) xo[i] = 0.f;
  if (x.m) {
    xm = x.m[sh];
    xl = x.l[sh];
#pragma unroll
    for (int i = 0; i < EL; ++i) xo[i] = x.o[sh * D + EL * lane + i];
  }
  const int n = ctx[s];
  const int np = n >= 0 && n <= len_limit ? (n + part_size - 1) / part_size : 0;
  const int nt = np + (x.m ? 1 : 0);
  if (n < 0 || n > len_limit || (x.expect && x.expect[s] != n) || nt > kSmallParts || np > slots) {
#pragma unroll
    for (int i = 0; i < EL; ++i) store_elem(T{}, out, sh * D + EL * lane + i, __builtin_nanf(""));
    return;
  }
  // partitions 0 .. np-1, then the extra partial
  float M = xm;
#pragma unroll
  for (int p = 0; p < kSmallParts; ++p) M = p < np ? fmaxf(M, mv[p]) : M;
  float L = 0.f, A[EL];
#pragma unroll
  for (int i = 0; i < EL; ++i) A[i] = 0.f;
#pragma unroll
  for (int p = 0; p < kSmallParts; ++p) {
    if (p < np) {  // (wave-uniform) a slot past the row's partitions may hold anything, NaN included
      // a partition with no token (l = 0, m = -inf: all masked) has no weight
      const float w = lv[p] == 0.f ? 0.f : lv[p] * fast_exp2((mv[p] - M) * kLog2e);
      L += w;
#pragma unroll
      for (int i = 0; i < EL; ++i) A[i] = __builtin_fmaf(w, ov[p][i], A[i]);
    }
  }
  {
    const float w = xl == 0.f ? 0.f : xl * fast_exp2((xm - M) * kLog2e);
    L += w;
#pragma unroll
    for (int i = 0; i < EL; ++i) A[i] = __builtin_fmaf(w, xo[i], A[i]);
  }
#pragma unroll
  for (int i = 0; i < EL; ++i) store_elem(T{}, out, sh * D + EL * lane + i, L == 0.f ? 0.f : A[i] / L);
}

// The kernel instance for (dtype, head_dim, block_size, heads per workgroup)
// is chosen at run time; Op::run<T, D, BS, GT, SPLIT>() does the work with it.
struct LaunchOp {
  const DecodeParams& p;
  int32_t num_seqs;
  bool cached;
  hipStream_t stream;
  template <typename T, typename S, int D, int BS, int GT, bool SPLIT, bool APPEND>
  hipError_t run() const {
    const int64_t units = static_cast<int64_t>(num_seqs) * (p.num_heads >> p.col_heads_log2) * p.q_chunks;
    const bool flat = SPLIT && !APPEND && p.flat;
    const uint32_t gx = static_cast<uint32_t>(flat ? (units * p.num_parts + p.n_own + kWaves - 1) / kWaves
                                                   : units + (APPEND ? p.append_wgs : 0));
    const uint32_t gy = SPLIT && !flat ? static_cast<uint32_t>((p.num_parts + kWaves - 1) / kWaves) : 1u;
    if (cached)
      launch_kernel(decode_kernel<T, S, D, BS, GT, SPLIT, true, APPEND>, dim3(gx, gy), dim3(kWaves * 64), stream, p);
    else
      launch_kernel(decode_kernel<T, S, D, BS, GT, SPLIT, false, APPEND>, dim3(gx, gy), dim3(kWaves * 64), stream,
                    p);
    return hipGetLastError();
  }
};

// Workgroups of the instance that one compute unit holds at once.
struct OccupancyOp {
  int* per_cu;
  template <typename T, typename S, int D, int BS, int GT, bool SPLIT, bool APPEND>
  hipError_t run() const {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        per_cu, decode_kernel<T, S, D, BS, GT, SPLIT, false, APPEND>, kWaves * 64, 0);
  }
};

template <typename T, typename S, int D, int BS, bool SPLIT, bool APPEND, typename Op>
hipError_t by_group(const Op& op, int gt) {
  switch (gt) {
    case 1: return op.template run<T, S, D, BS, 1, SPLIT, APPEND>();
    case 2: return op.template run<T, S, D, BS, 2, SPLIT, APPEND>();
    case 4: return op.template run<T, S, D, BS, 4, SPLIT, APPEND>();
    case 8: return op.template run<T, S, D, BS, 8, SPLIT, APPEND>();
    case 16: return op.template run<T, S, D, BS, 16, SPLIT, APPEND>();
  }
  return hipErrorInvalidValue;
}

template <typename T, typename S, bool SPLIT, bool APPEND, typename Op>
hipError_t by_shape(const Op& op, int d, int bs, int gt) {
  if (d == 64 && bs == 16) return by_group<T, S, 64, 16, SPLIT, APPEND>(op, gt);
  if (d == 64 && bs == 32) return by_group<T, S, 64, 32, SPLIT, APPEND>(op, gt);
  if (d == 128 && bs == 16) return by_group<T, S, 128, 16, SPLIT, APPEND>(op, gt);
  if (d == 128 && bs == 32) return by_group<T, S, 128, 32, SPLIT, APPEND>(op, gt);
  if (d == 128 && bs == 64) return by_group<T, S, 128, 64, SPLIT, APPEND>(op, gt);
  if constexpr (S::kBytes != 1) {  // a step of 8-bit codes (64 tokens) would span eight 8-token blocks
    if (d == 128 && bs == 8) return by_group<T, S, 128, 8, SPLIT, APPEND>(op, gt);
  }
  return hipErrorInvalidValue;
}

// One translation unit per (query type, storage type) instantiates its
// kernels (they build in parallel): decode_f32.hip, decode_f16.hip,
// decode_bf16.hip, and decode_{e4m3,i8}_{f16,bf16}.hip for 8-bit pools.
hipError_t dispatch_f32(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_f16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_e4m3_f16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_e4m3_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_i8_f16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_i8_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_i8t_f16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t dispatch_i8t_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt);
hipError_t occupancy_f32(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_f16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_bf16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_e4m3_f16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_e4m3_bf16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_i8_f16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_i8_bf16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_i8t_f16(int* per_cu, int d, int bs, int gt);
hipError_t occupancy_i8t_bf16(int* per_cu, int d, int bs, int gt);

template <typename T, typename S = T>
hipError_t dispatch_t(const LaunchOp& op, bool split, bool append, int d, int bs, int gt) {
  if constexpr (S::kBytes == 1) {  // no fused write into 8-bit pools
    if (append) return hipErrorInvalidValue;
    return split ? by_shape<T, S, true, false>(op, d, bs, gt) : by_shape<T, S, false, false>(op, d, bs, gt);
  } else {
    if (split)
      return append ? by_shape<T, S, true, true>(op, d, bs, gt) : by_shape<T, S, true, false>(op, d, bs, gt);
    return append ? by_shape<T, S, false, true>(op, d, bs, gt) : by_shape<T, S, false, false>(op, d, bs, gt);
  }
}
template <typename T, typename S = T>
hipError_t occupancy_t(int* per_cu, int d, int bs, int gt) {
  return by_shape<T, S, false, false>(OccupancyOp{per_cu}, d, bs, gt);
}


}  // namespace pa
