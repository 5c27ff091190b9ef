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
    for copy-on-write pairs, pa_reshape_and_cache of the new tokens' K/V, and pa_decode_auto,
    or pa_decode_shared when requests forked from one parent sit side by side in the batch
    (their common blocks are then read once for all of them).
Calls are enqueued on torch's current stream, as every call of the binding.  One instance
is used from one host thread.
"""
from __future__ import annotations

import math

import numpy as np

from . import (Allocator, pa_copy_blocks, pa_decode_auto, pa_decode_shared, pa_decode_shared_workspace_bytes,
               pa_decode_split_workspace_bytes, pa_order_longest_first, pa_reshape_and_cache,
               pa_shared_prefix_groups, pa_upload)


class PagedAttention:
    """A pool of KV blocks, its allocator, and decode steps over it.

    num_kv_heads defaults to num_heads (multi-head); query head h reads KV head
    h // (num_heads // num_kv_heads).  scale defaults to float32(1 / sqrt(head_dim)).
    partition_size is the split path's partition, used when pa_decode_auto takes it."""

    def __init__(self, num_heads: int, head_dim: int, block_size: int = 16, num_blocks: int = 1024,
                 num_kv_heads: int | None = None, dtype=None, device="cuda", scale: float | None = None,
                 partition_size: int = 512):
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
        self.key_cache = torch.zeros((num_blocks, self.num_kv_heads, block_size, head_dim), dtype=self.dtype,
                                     device=self.device)
        self.value_cache = torch.zeros((num_blocks, self.num_kv_heads, head_dim, block_size), dtype=self.dtype,
                                       device=self.device)
        self.allocator = Allocator(num_blocks, block_size)
        self._staging = None   # pinned int32 host buffer of the last step's index data
        self._staged = None    # event after that buffer's upload
        self._workspace = None

    # -- requests ------------------------------------------------------------------
    def allocate(self, request_id: int, seq_len: int):
        """Take the blocks of a request whose first seq_len tokens (its prompt) will be stored."""
        self.allocator.seq_create(request_id, seq_len)

    def fork(self, parent_id: int, child_id: int):
        """A new request sharing all of the parent's blocks (parallel sampling, beam search)."""
        self.allocator.seq_fork(parent_id, child_id)

    def free(self, request_id: int):
        self.allocator.seq_free(request_id)

    def context_len(self, request_id: int) -> int:
        return self.allocator.seq_len(request_id)

    def block_table(self, request_id: int) -> list:
        return self.allocator.block_table(request_id)

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
        pa_reshape_and_cache(key.contiguous(), value.contiguous(), self.key_cache, self.value_cache, slots)

    # -- one decode step ---------------------------------------------------------------
    def forward(self, request_ids, query, key, value):
        """One decode step.  For every request a slot is appended (a shared, partly filled last
        block is first copied), the new token's K/V rows key/value [S, num_kv_heads, head_dim]
        are written there, and query [S, num_heads, head_dim] attends over the request's
        context including that token.  Returns out [S, num_heads, head_dim].  Requests that
        share their leading blocks (forks of one parent) and are passed next to each other are
        decoded with those blocks read once."""
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
        group_start, prefix_len, num_groups, widest = pa_shared_prefix_groups(tables, lens, bs)
        shared = widest > 1
        # shared prefixes keep the batch order (groups are runs of neighbours); else longest first
        order = list(range(S)) if shared else pa_order_longest_first(lens)
        # one pinned buffer, one upload: slots | pairs | tables | lengths | launch order | groups
        P = len(pairs)
        parts = [np.asarray(slots, dtype=np.int32), np.asarray(pairs, dtype=np.int32).reshape(-1),
                 np.asarray(tables, dtype=np.int32).reshape(-1), np.asarray(lens, dtype=np.int32),
                 np.asarray(order, dtype=np.int32)]
        if shared:
            parts += [np.asarray(group_start, dtype=np.int32), np.asarray(prefix_len, dtype=np.int32)]
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
        if P:
            pa_copy_blocks(self.key_cache, self.value_cache, pairs_d)
        pa_reshape_and_cache(key.contiguous(), value.contiguous(), self.key_cache, self.value_cache, slots_d)
        max_ctx = max_blocks * bs
        if shared:
            need = pa_decode_shared_workspace_bytes(S, self.num_heads, self.head_dim, max_ctx)
        else:
            need = pa_decode_split_workspace_bytes(S, self.num_heads, self.head_dim, max_ctx, self.partition_size)
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        if shared:
            pa_decode_shared(out, query.contiguous(), self.key_cache, self.value_cache, tables_d, lens_d, gs_d, pl_d,
                             num_groups, widest, max_ctx, self.scale, self._workspace)
        else:
            pa_decode_auto(out, query.contiguous(), self.key_cache, self.value_cache, tables_d, lens_d, max_ctx,
                           self.scale, self.partition_size, self._workspace, seq_order=order_d)
        self.last_path = "shared" if shared else "auto"
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
