"""PagedAttention as an object: a pool, its allocator and one decode step per call.

"PagedAttention 源码解析：KV Cache 怎么管理" §六 shows the interface a caller sees:
PagedAttention(num_heads, head_dim, block_size, num_blocks), allocate(request_id, seq_len),
forward(query, key, value, ...) and free(request_id).  This class gives that interface over
the library's calls and adds nothing to what they compute:
  - the host allocator (Allocator: FIFO free list, reference counts, fork, append with
    copy-on-write; "PagedAttention 实现细节" §3.3);
  - key/value pools on the device, keys [num_blocks, num_kv_heads, block_size, head_dim],
    values [num_blocks, num_kv_heads, head_dim, block_size];
  - per forward(): the allocator's append, pa_upload of the step's index data, pa_copy_blocks
    for copy-on-write pairs, pa_reshape_and_cache of the new tokens' K/V, and the decode:
    pa_decode_masked when a request has positions without a token (a cached prefix's hole, or
    a sliding window's dropped tokens), else pa_decode_shared when requests forked from one
    parent sit side by side in the batch (their common blocks then read once for all of them),
    else pa_decode_auto;
  - prefix caching ("PagedAttention 实现细节" §3.2: requests with the same prompt prefix share
    its blocks) and a sliding window (the "滑动窗口" of the §六 feature list), through the
    allocator's prefix entries and window release;
  - swapping requests to a pinned host pool and back ("PagedAttention 实现细节" §3.4: the cache
    engine's CPU-side pool), through the allocator's swap and pa_swap_blocks;
  - 8-bit pools (the int8 KV cache beside paging of the xdnf.cn article, §2.3 and §6.3): FP8
    E4M3 or int8 codes with one scale per pool, or int8 with a scale per (token, KV head),
    written by pa_reshape_and_cache_quant and decoded by the calls above or pa_decode_quant.
Calls are enqueued on torch's current stream, as every call of the binding.  One instance
is used from one host thread.
"""
from __future__ import annotations

import math

import numpy as np

from . import (Allocator, pa_copy_blocks, pa_decode_auto, pa_decode_masked, pa_decode_quant, pa_decode_shared,
               pa_decode_shared_workspace_bytes, pa_decode_split_workspace_bytes, pa_order_longest_first,
               pa_reshape_and_cache, pa_reshape_and_cache_quant, pa_shared_prefix_groups, pa_swap_blocks,
               pa_upload, token_tile_bytes)

KV_FORMATS = (None, "fp8_e4m3", "int8", "int8_token")


class PagedAttention:
    """A pool of KV blocks, its allocator, and decode steps over it.

    num_kv_heads defaults to num_heads (multi-head); query head h reads KV head
    h // (num_heads // num_kv_heads).  scale defaults to float32(1 / sqrt(head_dim)).
    partition_size is the split path's partition, used when pa_decode_auto takes it.
    num_host_blocks > 0 adds a pinned host pool of that many blocks for swap_out / swap_in.
    kv_format "fp8_e4m3" or "int8" stores codes of K / k_scale and V / v_scale (uint8 pools of
    the same shapes); "int8_token" stores int8 codes with a scale per (token, KV head) in each
    tile (uint8 [num_blocks, num_kv_heads, token_tile_bytes(block_size, head_dim)] pools, the
    scale arguments unused).  8-bit pools take fp16 or bf16 queries and blocks of 16, 32 or 64."""

    def __init__(self, num_heads: int, head_dim: int, block_size: int = 16, num_blocks: int = 1024,
                 num_kv_heads: int | None = None, dtype=None, device="cuda", scale: float | None = None,
                 partition_size: int = 512, num_host_blocks: int = 0, kv_format: str | None = None,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        import torch
        self._torch = torch
        self.num_heads = num_heads
        self.num_kv_heads = num_kv_heads or num_heads
        if num_heads % self.num_kv_heads:
            raise ValueError("num_heads must be a multiple of num_kv_heads")
        self.head_dim = head_dim
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.dtype = dtype or torch.float16
        self.device = torch.device(device)
        self.scale = float(np.float32(1.0 / math.sqrt(head_dim))) if scale is None else float(scale)
        self.partition_size = partition_size
        if kv_format not in KV_FORMATS:
            raise ValueError(f"kv_format must be one of {KV_FORMATS}")
        if kv_format and (self.dtype not in (torch.float16, torch.bfloat16) or block_size not in (16, 32, 64)):
            raise ValueError("8-bit pools take fp16 or bf16 queries and blocks of 16, 32 or 64 tokens")
        self.kv_format = kv_format
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.key_cache, self.value_cache = self._pools(num_blocks, device=self.device)
        self.allocator = Allocator(num_blocks, block_size)
        self.host_key_cache = self.host_value_cache = None
        if num_host_blocks > 0:
            self.host_key_cache, self.host_value_cache = self._pools(num_host_blocks, pin_memory=True)
            self.allocator.set_host_pool(num_host_blocks)
        self._staging = None   # pinned int32 host buffer of the last step's index data
        self._staged = None    # event after that buffer's upload
        self._workspace = None
        self._prefix_of = {}   # request -> the cached prefix it took a use of

    def _pools(self, n: int, **where):
        """Zeroed key and value pools of n blocks (on the device, or pinned on the host)."""
        torch = self._torch
        Hkv, bs, D = self.num_kv_heads, self.block_size, self.head_dim
        if self.kv_format == "int8_token":
            shape = (n, Hkv, token_tile_bytes(bs, D))
            return torch.zeros(shape, dtype=torch.uint8, **where), torch.zeros(shape, dtype=torch.uint8, **where)
        dt = torch.uint8 if self.kv_format else self.dtype
        return (torch.zeros((n, Hkv, bs, D), dtype=dt, **where), torch.zeros((n, Hkv, D, bs), dtype=dt, **where))

    def _write(self, key, value, slots):
        """The slot-mapping write of K/V rows [n, num_kv_heads, head_dim] (quantising into 8-bit pools)."""
        if self.kv_format:
            pa_reshape_and_cache_quant(key.contiguous(), value.contiguous(), self.key_cache, self.value_cache, slots,
                                       self.k_scale, self.v_scale, kv_format=self.kv_format)
        else:
            pa_reshape_and_cache(key.contiguous(), value.contiguous(), self.key_cache, self.value_cache, slots)

    # -- requests ------------------------------------------------------------------
    def allocate(self, request_id: int, seq_len: int):
        """Take the blocks of a request whose first seq_len tokens (its prompt) will be stored."""
        self.allocator.seq_create(request_id, seq_len)

    def fork(self, parent_id: int, child_id: int):
        """A new request sharing all of the parent's blocks (parallel sampling, beam search)."""
        self.allocator.seq_fork(parent_id, child_id)

    def free(self, request_id: int):
        """Release the request's blocks, and its use of a cached prefix (the prefix's blocks
        return to the pool when its last user is freed)."""
        self.allocator.seq_free(request_id)
        pid = self._prefix_of.pop(request_id, None)
        if pid is not None:
            self.allocator.prefix_release(pid)

    def context_len(self, request_id: int) -> int:
        return self.allocator.seq_len(request_id)

    def block_table(self, request_id: int) -> list:
        return self.allocator.block_table(request_id)

    # -- prefix caching and sliding window -------------------------------------------
    def allocate_with_prefix(self, request_id: int, prefix_tokens, own_len: int):
        """A request whose prompt starts with `prefix_tokens` (token ids), cached by content: the
        first request with this prefix takes its blocks (hit False: store its K/V once with
        store_prefix), later ones share them (hit True).  The request's own own_len prompt
        tokens start at the block boundary after the prefix; the positions in between hold no
        token and decode skips them.  The request holds a use of the prefix until free().
        Returns (prefix_id, hit, position of the first own token)."""
        pid, hit = self.allocator.prefix_get_or_create(prefix_tokens)
        try:
            self.allocator.seq_create_with_prefix(request_id, pid, own_len)
        except Exception:
            self.allocator.prefix_release(pid)
            raise
        self._prefix_of[request_id] = pid
        start = -(-len(prefix_tokens) // self.block_size) * self.block_size
        return pid, hit, start

    def store_prefix(self, prefix_id: int, key, value):
        """Write a cached prefix's K/V rows [prefix length, num_kv_heads, head_dim] into its blocks."""
        torch = self._torch
        blocks, n, _ = self.allocator.prefix_info(prefix_id)
        if key.shape[0] != n or value.shape[0] != n:
            raise ValueError(f"the prefix holds {n} tokens")
        bs = self.block_size
        slots = torch.tensor([blocks[p // bs] * bs + p % bs for p in range(n)], dtype=torch.int32,
                             device=self.device)
        self._write(key, value, slots)

    def set_window(self, request_id: int, window: int):
        """Attend over the request's last `window` tokens from now on; the blocks wholly before
        them return to the pool."""
        self.allocator.seq_set_window(request_id, window)

    # -- swap -------------------------------------------------------------------------
    def swap_out(self, request_ids):
        """Move the requests (forks of one parent move together) to the host pool; their device
        blocks return to the pool.  A swapped request can be swapped in or freed."""
        self._swap(self.allocator.seq_swap_out, request_ids, to_host=True)

    def swap_in(self, request_ids):
        """Bring swapped requests back into device blocks."""
        self._swap(self.allocator.seq_swap_in, request_ids, to_host=False)

    def _swap(self, move, request_ids, to_host: bool):
        torch = self._torch
        if self.host_key_cache is None:
            raise ValueError("no host pool: construct with num_host_blocks > 0")
        pairs = move([int(r) for r in request_ids])
        if not pairs:
            return
        pairs_d = torch.tensor(pairs, dtype=torch.int32, device=self.device)
        D = self.head_dim
        if to_host:
            pa_swap_blocks(self.host_key_cache, self.host_value_cache, self.key_cache, self.value_cache, pairs_d,
                           head_dim=D)
        else:
            pa_swap_blocks(self.key_cache, self.value_cache, self.host_key_cache, self.host_value_cache, pairs_d,
                           head_dim=D)

    # -- K/V of stored tokens --------------------------------------------------------
    def store(self, request_id: int, key, value, start: int = 0):
        """Write the K/V rows [n, num_kv_heads, head_dim] of positions start .. start + n - 1 of
        the request (its prompt) into their slots.  Those blocks must not be shared."""
        torch = self._torch
        n = key.shape[0]
        if value.shape[0] != n or start < 0 or start + n > self.context_len(request_id):
            raise ValueError("positions outside the request's context")
        table = self.block_table(request_id)
        bs = self.block_size
        for j in range(start // bs, -(-(start + n) // bs)):
            if self.allocator.ref_count(table[j]) != 1:
                raise ValueError(f"block {table[j]} of request {request_id} is shared: it cannot be written")
        slots = torch.tensor([table[p // bs] * bs + p % bs for p in range(start, start + n)], dtype=torch.int32,
                             device=self.device)
        self._write(key, value, slots)

    # -- one decode step ---------------------------------------------------------------
    def forward(self, request_ids, query, key, value):
        """One decode step.  For every request a slot is appended (a shared, partly filled last
        block is first copied), the new token's K/V rows key/value [S, num_kv_heads, head_dim]
        are written there, and query [S, num_heads, head_dim] attends over the request's
        context including that token (positions without a token, a cached prefix's hole or
        what a sliding window dropped, left out).  Returns out [S, num_heads, head_dim].
        Requests that share their leading blocks (forks of one parent) and are passed next to
        each other are decoded with those blocks read once."""
        torch = self._torch
        ids = [int(r) for r in request_ids]
        S = len(ids)
        if query.shape != (S, self.num_heads, self.head_dim) or key.shape != (S, self.num_kv_heads, self.head_dim) \
                or value.shape != key.shape:
            raise ValueError("query [S, num_heads, head_dim], key and value [S, num_kv_heads, head_dim] expected")
        out = torch.empty_like(query)
        if S == 0:
            return out
        slots, pairs = self.allocator.seq_append_slots(ids)
        lens_now = [self.context_len(r) for r in ids]
        bs = self.block_size
        max_blocks = max(-(-n // bs) for n in lens_now) + 1
        tables, lens = self.allocator.build_block_tables(ids, max_blocks)
        lo, hi = self.allocator.masks(ids)
        masked = any(h > l for l, h in zip(lo, hi))
        group_start, prefix_len, num_groups, widest = pa_shared_prefix_groups(tables, lens, bs)
        shared = widest > 1 and not masked
        # shared prefixes keep the batch order (groups are runs of neighbours); else longest first
        order = list(range(S)) if shared else pa_order_longest_first(lens)
        # one pinned buffer, one upload: slots | pairs | tables | lengths | launch order | groups
        P = len(pairs)
        parts = [np.asarray(slots, dtype=np.int32), np.asarray(pairs, dtype=np.int32).reshape(-1),
                 np.asarray(tables, dtype=np.int32).reshape(-1), np.asarray(lens, dtype=np.int32),
                 np.asarray(order, dtype=np.int32)]
        if shared:
            parts += [np.asarray(group_start, dtype=np.int32), np.asarray(prefix_len, dtype=np.int32)]
        if masked:
            parts += [np.asarray(lo, dtype=np.int32), np.asarray(hi, dtype=np.int32)]
        host = np.concatenate(parts)
        staging = self._stage(host)
        dev = torch.empty(host.size, dtype=torch.int32, device=self.device)
        pa_upload(dev, staging)
        self._staged = torch.cuda.Event()
        self._staged.record()
        o = 0
        slots_d = dev[o:o + S]
        o += S
        pairs_d = dev[o:o + 2 * P].view(P, 2)
        o += 2 * P
        tables_d = dev[o:o + S * max_blocks].view(S, max_blocks)
        o += S * max_blocks
        lens_d = dev[o:o + S]
        o += S
        order_d = dev[o:o + S]
        o += S
        if shared:
            gs_d = dev[o:o + num_groups + 1]
            o += num_groups + 1
            pl_d = dev[o:o + S]
            o += S
        if masked:
            lo_d = dev[o:o + S]
            hi_d = dev[o + S:o + 2 * S]
        if P:
            pa_copy_blocks(self.key_cache, self.value_cache, pairs_d, head_dim=self.head_dim)
        self._write(key, value, slots_d)
        max_ctx = max_blocks * bs
        if shared:
            need = pa_decode_shared_workspace_bytes(S, self.num_heads, self.head_dim, max_ctx)
        else:
            need = pa_decode_split_workspace_bytes(S, self.num_heads, self.head_dim, max_ctx, self.partition_size)
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        q = query.contiguous()
        kc, vc, fmt, ks, vs = self.key_cache, self.value_cache, self.kv_format, self.k_scale, self.v_scale
        if masked:
            pa_decode_masked(out, q, kc, vc, tables_d, lens_d, lo_d, hi_d, max_ctx, self.scale, ks, vs,
                             kv_format=fmt, partition_size=self.partition_size, workspace=self._workspace,
                             seq_order=order_d)
        elif shared:
            pa_decode_shared(out, q, kc, vc, tables_d, lens_d, gs_d, pl_d, num_groups, widest, max_ctx, self.scale,
                             self._workspace, ks, vs, kv_format=fmt)
        elif fmt:  # the pa_decode_auto rule over 8-bit pools
            pa_decode_quant(out, q, kc, vc, tables_d, lens_d, max_ctx, self.scale, ks, vs, kv_format=fmt,
                            partition_size=self.partition_size, workspace=self._workspace, seq_order=order_d)
        else:
            pa_decode_auto(out, q, kc, vc, tables_d, lens_d, max_ctx, self.scale, self.partition_size,
                           self._workspace, seq_order=order_d)
        self.last_path = "masked" if masked else "shared" if shared else "auto"
        return out

    def _stage(self, host: np.ndarray):
        """A pinned host tensor holding `host`; the previous step's buffer is reused once its
        upload has run."""
        torch = self._torch
        if self._staging is None or self._staging.numel() < host.size:
            if self._staged is not None:
                self._staged.synchronize()
            self._staging = torch.empty(max(host.size, 1024), dtype=torch.int32).pin_memory()
        elif self._staged is not None:
            self._staged.synchronize()
        self._staging[:host.size].copy_(torch.from_numpy(host))
        return self._staging[:host.size]
