"""Oracle for paged decode attention, in float64 (test infrastructure only).

What is computed, and where the pages define it:

* Gather, then attend.  "PagedAttention 实现细节" §3.1 first collects a
  sequence's K/V rows from its physical blocks (block `table[j]` holds logical
  tokens j*bs .. j*bs+bs-1; only the first `n` tokens are valid) into a
  contiguous tensor, then runs exactly the same math as a contiguous cache.
* The math is single-query scaled-dot-product attention,
  out = softmax(scale * K q) V, with scale = 1/sqrt(head_dim): "PagedAttention
  源码解析：KV Cache 怎么管理" §四 (standard_attention), "Ascend C算子开发高阶实战…"
  §1.3, "PagedAttention 实现细节" §3.1.  The pages' own per-block and online
  loops are not followed where they differ from this definition (one page
  normalises each block separately, another never rescales its accumulator);
  the oracle is the definition they all aim at.
* Pool layouts.  Keys: [num_blocks, num_kv_heads, block_size, head_dim], one
  token row after another ("PagedAttention 实现细节" §3.1 index-based kernel
  signature, §3.4 PagedAttention.forward).  Values: [num_blocks, num_kv_heads,
  head_dim, block_size], the block-size-innermost arrangement of
  "Ascend C算子开发高阶实战…" §3.1/§5.2, so value row t of a block is the
  column [:, t % block_size] of its (block, KV head) tile.
* Query heads share KV heads in contiguous groups: query head h reads KV head
  h // (num_heads // num_kv_heads).  The pages name grouped-query attention
  only as future work ("Ascend C算子开发高阶实战…" §十); contiguous grouping is
  the plain reading.
* Split partials and merge: the pages only say a second kernel exists for few,
  very long sequences ("Ascend平台下的PageAttention优化实践" §2.3).  The oracle
  cuts the context into partitions of `partition_size` tokens, keeps
  (m_p = max logit, l_p = sum exp(z - m_p), o_p = normalised partial output)
  per partition, and merges with the log-sum-exp rule.

* Masked positions (masks = (lo, hi) per sequence): positions lo <= t < hi
  hold no token and are left out of the softmax.  This serves a sequence
  built on a cached prefix, whose own tokens start at the next block boundary
  ("PagedAttention 实现细节" §3.2; the allocator's hole), and a sliding window
  of the last W tokens ([0, n - W) masked; the window itself is the
  "滑动窗口" of "PagedAttention 源码解析：KV Cache 怎么管理" §六, which lists it
  as partly supported on Ascend).  A sequence with every token masked gives a
  zero row, like an empty context.
* Several query tokens per sequence (paged_decode_multi): the query rows of
  sequence s are query_start[s] .. query_start[s+1] - 1, its last L tokens,
  whose K/V are already in the cache; query token i of the span sits at
  position n - L + i and attends to positions 0 .. n - L + i (causal).  This
  is the verification pass of speculative decoding, which the xdnf.cn article
  (§6.3) combines with paging; one query token per sequence is plain decode.
* 8-bit pools (quant = (fmt, k_scale, v_scale)): the pools hold codes and
  stand for decode(code) * scale (oracle/quant.py); the attention over those
  values is the same definition.  With quant = ("int8_token", k_scales,
  v_scales) the pools hold int8 codes and each (token, KV head) row has its
  own scale: k_scales / v_scales [NB, H_kv, bs] float32, the scale of the row
  at block b, KV head g, offset o being k_scales[b, g, o].

Inputs are NumPy arrays in storage type: float32, float16, or bf16 given as
uint16 bit patterns (8-bit pools: uint8 codes).  Everything is upcast exactly
to float64; the scales are taken as the float32 values the kernels receive.
"""
from __future__ import annotations

import numpy as np

from . import quant as Q


def to_f64(x, dtype: str) -> np.ndarray:
    """Exact upcast of a storage array to float64 (bf16: bits << 16 -> float32)."""
    x = np.asarray(x)
    if dtype == "bf16":
        bits = x.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f16"):
        return x.astype(np.float64)
    raise ValueError(dtype)


def scale_f64(scale: float) -> float:
    """The float32 value of `scale`, as float64."""
    return float(np.float32(scale))


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of `num_tokens` occupies: ceil(n / bs)."""
    return (num_tokens + block_size - 1) // block_size


def gather_rows(key_cache, value_cache, table_row, num_tokens: int, kv_head: int):
    """Collect the first `num_tokens` K and V rows of one sequence and KV head, as stored.

    Logical block j of the sequence lives in physical block table_row[j]; its
    rows are tokens j*bs .. j*bs + bs - 1, of which only those below
    `num_tokens` are valid ("PagedAttention 实现细节" §3.1, the gather step).
    key_cache is [NB, H_kv, bs, D] and value_cache [NB, H_kv, D, bs].
    Returns storage-typed arrays K, V of shape [num_tokens, head_dim].
    """
    num_blocks, _, block_size, head_dim = key_cache.shape
    ks, vs = [], []
    for j in range(blocks_for(num_tokens, block_size)):
        phys = int(table_row[j])
        if not 0 <= phys < num_blocks:
            raise IndexError(f"block table entry {phys} outside the pool of {num_blocks}")
        valid = min(block_size, num_tokens - j * block_size)
        ks.append(key_cache[phys, kv_head, :valid, :])
        vs.append(value_cache[phys, kv_head, :, :valid].T)
    if not ks:
        empty = np.zeros((0, head_dim), dtype=key_cache.dtype)
        return empty, empty.copy()
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def gather_kv(key_cache, value_cache, table_row, num_tokens: int, kv_head: int, dtype: str):
    """gather_rows, upcast exactly to float64 [num_tokens, head_dim]."""
    K, V = gather_rows(key_cache, value_cache, table_row, num_tokens, kv_head)
    return to_f64(K, dtype), to_f64(V, dtype)


def kv_head_of(head: int, num_heads: int, num_kv_heads: int) -> int:
    """The KV head query head `head` reads: contiguous groups of G = H / H_kv query heads
    share one KV head, so head h reads KV head h // G (the plain reading of grouped-query
    attention, which the pages name only as future work)."""
    if num_kv_heads <= 0 or num_heads % num_kv_heads:
        raise ValueError("num_heads must be a positive multiple of num_kv_heads")
    if not 0 <= head < num_heads:
        raise IndexError(f"query head {head} outside 0..{num_heads - 1}")
    return head // (num_heads // num_kv_heads)


def keep_positions(num_tokens: int, lo: int, hi: int) -> np.ndarray:
    """Positions t < num_tokens outside [lo, hi)."""
    t = np.arange(num_tokens)
    return t[(t < lo) | (t >= hi)]


def gather_positions(key_cache, value_cache, table_row, positions: np.ndarray, kv_head: int):
    """K and V rows (as stored) of the given token positions of one sequence and KV head:
    position t is row t % bs of block table_row[t // bs].  Blocks holding none of the
    positions are not looked at.  Returns arrays [len(positions), head_dim]."""
    num_blocks, _, block_size, head_dim = key_cache.shape
    positions = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    if np.any((phys < 0) | (phys >= num_blocks)):
        raise IndexError("block table entry outside the pool")
    off = positions % block_size
    return key_cache[phys, kv_head, off, :], value_cache[phys, kv_head, :, off]


def gather_row_scales(scale_pool, table_row, positions, kv_head: int) -> np.ndarray:
    """The per-row scales of the given token positions of one sequence and KV head:
    position t's row sits at block table_row[t // bs], offset t % bs of scale_pool
    [NB, H_kv, bs]."""
    num_blocks, _, block_size = scale_pool.shape
    positions = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    if np.any((phys < 0) | (phys >= num_blocks)):
        raise IndexError("block table entry outside the pool")
    return scale_pool[phys, kv_head, positions % block_size]


def kv_for(key_cache, value_cache, table_row, num_tokens: int, kv_head: int, dtype: str, quant=None,
           mask=None):
    """float64 K, V of one sequence and KV head, one row per position that holds a token:
    all t < num_tokens, or with mask = (lo, hi) those outside [lo, hi) (keep_positions).
    With quant = (fmt, k_scale, v_scale) the pools hold 8-bit codes and stand for
    decode(code) * scale (oracle/quant.py); with quant = ("int8_token", k_scales,
    v_scales) each row has its own scale (decode(code) * the row's scale); otherwise they
    hold `dtype` values."""
    if quant is not None and quant[0] == Q.INT8_TOKEN:
        _, k_scales, v_scales = quant
        pos = np.arange(num_tokens) if mask is None else keep_positions(num_tokens, int(mask[0]), int(mask[1]))
        K, V = gather_positions(key_cache, value_cache, table_row, pos, kv_head)
        return (Q.dequantize_rows_int8(K, gather_row_scales(k_scales, table_row, pos, kv_head)),
                Q.dequantize_rows_int8(V, gather_row_scales(v_scales, table_row, pos, kv_head)))
    if mask is None:
        if quant is None:
            return gather_kv(key_cache, value_cache, table_row, num_tokens, kv_head, dtype)
        K, V = gather_rows(key_cache, value_cache, table_row, num_tokens, kv_head)
    else:
        K, V = gather_positions(key_cache, value_cache, table_row,
                                keep_positions(num_tokens, int(mask[0]), int(mask[1])), kv_head)
    if quant is None:
        return to_f64(K, dtype), to_f64(V, dtype)
    fmt, k_scale, v_scale = quant
    return Q.dequantize(K, k_scale, fmt), Q.dequantize(V, v_scale, fmt)


def logits(q64: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """z_t = scale * <q, K_t> for every cached token t."""
    return scale * (K @ q64)


def softmax_weights(z: np.ndarray) -> np.ndarray:
    """p_t = exp(z_t - max z) / sum_u exp(z_u - max z)."""
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def attend(q64: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Standard single-query attention softmax(scale*K q)^T V.  No tokens -> zeros."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    return softmax_weights(logits(q64, K, scale)) @ V


def paged_decode(query, key_cache, value_cache, block_tables, context_lens, scale: float,
                 dtype: str, quant=None, masks=None) -> np.ndarray:
    """out[s, h] = attention of query[s, h] over the first context_lens[s] tokens of
    sequence s, gathered through block_tables[s] from KV head kv_head_of(h, H, H_kv).

    query [S, H, D]; key_cache [NB, H_kv, bs, D]; value_cache [NB, H_kv, D, bs];
    block_tables [S, MB]; context_lens [S].  Returns float64 [S, H, D].
    quant = (fmt, k_scale, v_scale) when the pools hold 8-bit codes with per-pool scales,
    ("int8_token", k_scales, v_scales) for int8 codes with per-row scales; masks = (lo, hi)
    per-sequence lists of masked positions.
    """
    S, H, D = query.shape
    H_kv = key_cache.shape[1]
    sig = scale_f64(scale)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        n = int(context_lens[s])
        mask = None if masks is None else (masks[0][s], masks[1][s])
        kv = {}
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            if g not in kv:
                kv[g] = kv_for(key_cache, value_cache, block_tables[s], n, g, dtype, quant, mask)
            K, V = kv[g]
            out[s, h] = attend(to_f64(query[s, h], dtype), K, V, sig)
    return out


def decode_one(query, key_cache, value_cache, table_row, num_tokens: int, head: int,
               num_heads: int, scale: float, dtype: str, quant=None, mask=None) -> np.ndarray:
    """One output row: out[s, head] of paged_decode, for query = query[s] ([num_heads, D])
    and table_row = block_tables[s].  The pools may hold every KV head, or only the one
    this head reads (key_cache.shape[1] == 1, as when a caller fetched just that head's
    blocks): then query head `head` of `num_heads` still names its row of `query`, and the
    single stored KV head stands for kv_head_of(head, num_heads, H_kv) of the full pool."""
    if query.shape[0] != num_heads:
        raise ValueError("query must hold the sequence's num_heads rows")
    H_kv = key_cache.shape[1]
    g = 0 if H_kv == 1 else kv_head_of(head, num_heads, H_kv)
    K, V = kv_for(key_cache, value_cache, table_row, num_tokens, g, dtype, quant, mask)
    return attend(to_f64(query[head], dtype), K, V, scale_f64(scale))


# ----------------------------------------------------------------------------
# split-context partials and their merge


def partition_partials(q64: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       partition_size: int, positions=None, num_tokens=None):
    """Per partition p = positions [p*PS, min((p+1)*PS, n)):
    m_p = max z, l_p = sum exp(z - m_p), o_p = sum exp(z - m_p) V / l_p over its tokens.
    Row i of K, V is the token at positions[i] (default: row i is position i, n = rows);
    num_tokens = n sets the partition count P = ceil(n / PS).  A partition holding no
    token (all its positions masked) has m_p = -inf, l_p = 0, o_p = 0: the merge gives it
    no weight.  Returns float64 arrays m [P], l [P], o [P, D].
    """
    pos = np.arange(K.shape[0]) if positions is None else np.asarray(positions)
    n = K.shape[0] if num_tokens is None else num_tokens
    P = (n + partition_size - 1) // partition_size
    D = V.shape[1]
    m = np.zeros(P)
    l = np.zeros(P)
    o = np.zeros((P, D))
    for p in range(P):
        rows = np.nonzero((pos >= p * partition_size) & (pos < (p + 1) * partition_size))[0]
        if rows.size == 0:
            m[p], l[p] = -np.inf, 0.0
            continue
        z = logits(q64, K[rows], scale)
        m[p] = np.max(z)
        e = np.exp(z - m[p])
        l[p] = np.sum(e)
        o[p] = (e @ V[rows]) / l[p]
    return m, l, o


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Merge partition partials: M = max m_p, w_p = l_p exp(m_p - M),
    out = sum_p w_p o_p / sum_p w_p.  No partitions, or none with a token -> zeros."""
    if m.shape[0] == 0 or not np.any(l > 0):
        return np.zeros(o.shape[1], dtype=np.float64)
    M = np.max(m)
    w = np.where(l > 0, l * np.exp(m - M), 0.0)
    return (w @ o) / np.sum(w)


# ----------------------------------------------------------------------------
# several query tokens per sequence


def paged_decode_multi(query, key_cache, value_cache, block_tables, context_lens, query_start, scale: float,
                       dtype: str, quant=None) -> np.ndarray:
    """out[r, h] for every query row r = query_start[s] + i (i < L = query_start[s+1] -
    query_start[s]): attention of query[r, h] over positions 0 .. n - L + i of sequence s
    (n = context_lens[s]).  query [T, H, D]; returns float64 [T, H, D]."""
    T, H, D = query.shape
    H_kv = key_cache.shape[1]
    sig = scale_f64(scale)
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        L = r1 - r0
        if L > n:
            raise ValueError("a sequence has more query tokens than cached tokens")
        kv = {}
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            if g not in kv:
                kv[g] = kv_for(key_cache, value_cache, block_tables[s], n, g, dtype, quant)
            K, V = kv[g]
            for i in range(L):
                lim = n - L + i + 1
                out[r0 + i, h] = attend(to_f64(query[r0 + i, h], dtype), K[:lim], V[:lim], sig)
    return out
