"""Oracle for the host block allocator (test infrastructure only).

Policy, and where the pages fix it:

* The pool starts as a queue of free block ids (0..NB-1, or a given
  permutation).  Allocation takes the head of the queue ("PagedAttention
  源码解析：KV Cache 怎么管理" §二/§三: `free_blocks.pop(0)`; its worked example
  gives requests of 32, 16 and 48 tokens the blocks [0,1], [2], [3,4,5] and
  leaves [6,7,8,...] free, which only first-in-first-out order produces).
* A sequence of n tokens holds ceil(n / bs) blocks (same page §三; "Ascend C
  算子开发高阶实战…" §1.2: 45 tokens -> 3 blocks, 100 -> 7).
* Every block carries a reference count: 1 when allocated, +1 per extra
  sharer, -1 when a sharer lets go; at 0 it returns to the tail of the free
  queue (xdnf.cn PagedAttention article §3.4 and its §4.2 PhysicalBlockPool;
  "PagedAttention 实现细节" §3.3).  A freed sequence releases its blocks in
  block-table order.
* Appending a token at position L (xdnf.cn article §4.2 append_token_kv):
  if L % bs == 0 a fresh block is appended to the table; otherwise the token
  goes to the last block at offset L % bs.  Copy-on-write is decided before
  the write (xdnf.cn article §3.4; "PagedAttention 实现细节" §3.3): a last
  block with refcount > 1 is replaced by a fresh block, the pair (old, new) is
  emitted for a whole-block copy, the old count drops by one and the new one
  is 1; a block with refcount 1 is written in place.  The slot is
  table[L // bs] * bs + L % bs (xdnf.cn article §3.1 addressing).
* Fork (parallel sampling, beam search: xdnf.cn article §3.4) gives the child
  the parent's first ceil(n / bs) blocks and adds one reference to each.
* Running out of blocks is an error that leaves the state unchanged
  ("PagedAttention 源码解析…" §三 raises, xdnf.cn §4.2 asserts, "PagedAttention
  实现细节" §3.3 fails the copy-on-write).
* A batch of appends is processed in the order given, and all-or-nothing.

Prefix caching ("PagedAttention 实现细节" §3.2, CachedPrefix and
PrefixCacheManager):
* An entry maps a prompt prefix (its tokens) to the blocks that hold its KV,
  with a count of the requests using it and its token count.  get_or_create
  on a known prefix adds one user and returns the same blocks; on a new one it
  takes ceil(n / bs) blocks from the pool (the caller then computes and writes
  their KV) with one user.  release drops one user; at zero the entry lets go
  of its blocks.  Reading taken: the key is the token sequence itself (the
  page hashes its text to 12 hex digits; comparing the tokens in full keeps two
  different prompts from ever sharing blocks).  Entry ids count up from 1.
* The entry holds one reference on each of its blocks; a sequence built on it
  holds another (so blocks outlive a released entry while sequences use them).
* A sequence built on a prefix of n_p tokens (seq_create_with_prefix) has the
  prefix's P = ceil(n_p / bs) blocks first and its own tokens from position
  P * bs on, in fresh blocks: the page's demo counts the request's own tokens
  in blocks of their own (9-token prompt, 1 block; 30 own tokens, 2 blocks).
  Positions n_p .. P*bs - 1 are then a hole in the sequence: they hold no
  token and decode must skip them (`masks`).  A sequence's length counts
  positions, hole included; fork keeps the hole and may not end inside it.

Swap ("PagedAttention 实现细节" §3.4: its cache engine holds a device-side pool
and a host-side pool used for swapping):
* A second, host-side pool of block ids with its own first-in-first-out free
  queue and counts.  swap_out(group) moves the sequences of a group to it: every
  distinct device block of their tables (table order, first appearance) gets a
  host block, a (device, host) pair is emitted for the copy, each reference the
  group held moves from the device block to the host block (the device block
  returns to the free queue when nothing else holds it).  swap_in is the
  mirror image with (host, device) pairs.  A group is moved whole, so blocks
  shared inside it stay shared.  A swapped sequence can only be swapped in or
  freed.  All-or-nothing.

Sliding window (the feature "PagedAttention 源码解析：KV Cache 怎么管理" §六
lists): set_window(seq, W) keeps only the last W positions live.  Every block
whose positions all lie before len - W is released and its table entry
becomes -1 (decode never reads it); appends keep releasing as the window moves.
masks() gives [0, len - W).  Not combined with a prefix hole.  A fork of a
windowed sequence keeps the window and must still hold the blocks its own
window needs.
"""
from __future__ import annotations

import copy
from collections import deque


class AllocatorError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}" if msg else code)
        self.code = code


NO_FREE_BLOCKS = "NO_FREE_BLOCKS"
UNKNOWN_SEQ = "UNKNOWN_SEQ"
UNKNOWN_PREFIX = "UNKNOWN_PREFIX"
SEQ_EXISTS = "SEQ_EXISTS"
INVALID_ARG = "INVALID_ARG"


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise AllocatorError(INVALID_ARG, "num_blocks >= 0 and block_size > 0")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocatorError(INVALID_ARG, "initial free order must be a permutation of 0..NB-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refs = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.stats = {"blocks_allocated": 0, "blocks_freed": 0, "cow_copies": 0}
        self.holes: dict[int, tuple[int, int]] = {}      # seq -> (lo, hi) positions with no token
        self.prefixes: dict[tuple, int] = {}             # prefix tokens -> entry id
        self.entries: dict[int, dict] = {}               # entry id -> blocks, users, length, key
        self.next_prefix_id = 1
        self.host_free: deque = deque()                  # host pool (swap)
        self.host_refs: list[int] = []
        self.swapped: set = set()
        self.windows: dict[int, int] = {}

    # -- helpers -------------------------------------------------------------
    def _blocks_for(self, n: int) -> int:
        return (n + self.block_size - 1) // self.block_size

    def _take(self) -> int:
        if not self.free:
            raise AllocatorError(NO_FREE_BLOCKS)
        b = self.free.popleft()
        self.refs[b] = 1
        self.stats["blocks_allocated"] += 1
        return b

    def _release(self, b: int):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free.append(b)
            self.stats["blocks_freed"] += 1

    def _need(self, seq_id: int):
        if seq_id not in self.tables:
            raise AllocatorError(UNKNOWN_SEQ, str(seq_id))

    # -- public verbs ----------------------------------------------------------
    def clone(self) -> "BlockAllocator":
        return copy.deepcopy(self)

    def seq_create(self, seq_id: int, num_tokens: int):
        if seq_id in self.tables:
            raise AllocatorError(SEQ_EXISTS, str(seq_id))
        if num_tokens < 0:
            raise AllocatorError(INVALID_ARG, "num_tokens < 0")
        nb = self._blocks_for(num_tokens)
        if nb > len(self.free):
            raise AllocatorError(NO_FREE_BLOCKS)
        self.tables[seq_id] = [self._take() for _ in range(nb)]
        self.lens[seq_id] = num_tokens

    def seq_fork(self, parent: int, child: int, num_tokens: int = -1):
        self._need(parent)
        if child in self.tables:
            raise AllocatorError(SEQ_EXISTS, str(child))
        if parent in self.swapped:
            raise AllocatorError(INVALID_ARG, "parent is swapped out")
        n = self.lens[parent] if num_tokens < 0 else num_tokens
        if n > self.lens[parent]:
            raise AllocatorError(INVALID_ARG, "fork length beyond the parent")
        hole = self.holes.get(parent)
        if hole and hole[0] < n < hole[1]:
            raise AllocatorError(INVALID_ARG, "fork length inside the prefix hole")
        shared = self.tables[parent][: self._blocks_for(n)]
        W = self.windows.get(parent)
        if W is not None:
            first_live = max(0, n - W) // self.block_size
            if any(b < 0 for b in shared[first_live:]):
                raise AllocatorError(INVALID_ARG, "the child's window needs blocks the parent dropped")
        for b in shared:
            if b >= 0:
                self.refs[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = n
        if hole and n >= hole[1]:
            self.holes[child] = hole
        if W is not None:
            self.windows[child] = W
            self._drop_behind_window(child)

    def seq_append_slot(self, seq_id: int):
        """Reserve the slot of the next token; returns (slot, cow_src, cow_dst), -1s when no copy."""
        self._need(seq_id)
        if seq_id in self.swapped:
            raise AllocatorError(INVALID_ARG, "sequence is swapped out")
        table = self.tables[seq_id]
        L = self.lens[seq_id]
        src = dst = -1
        if L % self.block_size == 0:
            table.append(self._take())
        else:
            last = table[L // self.block_size]
            if self.refs[last] > 1:
                new = self._take()
                self.refs[last] -= 1
                table[L // self.block_size] = new
                src, dst = last, new
                self.stats["cow_copies"] += 1
        slot = table[L // self.block_size] * self.block_size + L % self.block_size
        self.lens[seq_id] = L + 1
        if seq_id in self.windows:
            self._drop_behind_window(seq_id)
        return slot, src, dst

    def seq_append_slots(self, seq_ids):
        """Append one token to each sequence, in order.  Returns (slots, pairs).  All-or-nothing."""
        for s in seq_ids:
            self._need(s)
        for s in seq_ids:
            if s in self.swapped:
                raise AllocatorError(INVALID_ARG, "a sequence in the batch is swapped out")
        saved = copy.deepcopy((self.free, self.refs, self.tables, self.lens, self.stats))
        try:
            slots, pairs = [], []
            for s in seq_ids:
                slot, src, dst = self.seq_append_slot(s)
                slots.append(slot)
                if src >= 0:
                    pairs.append((src, dst))
            return slots, pairs
        except AllocatorError:
            self.free, self.refs, self.tables, self.lens, self.stats = saved
            raise

    def seq_free(self, seq_id: int):
        self._need(seq_id)
        if seq_id in self.swapped:
            for h in self.tables[seq_id]:
                if h >= 0:
                    self._release_host(h)
            self.swapped.discard(seq_id)
        else:
            for b in self.tables[seq_id]:
                if b >= 0:
                    self._release(b)
        del self.tables[seq_id]
        del self.lens[seq_id]
        self.holes.pop(seq_id, None)
        self.windows.pop(seq_id, None)

    def can_allocate(self, num_blocks: int) -> bool:
        return num_blocks <= len(self.free)

    def num_free_blocks(self) -> int:
        return len(self.free)

    def ref_count(self, block: int) -> int:
        return self.refs[block] if 0 <= block < self.num_blocks else -1

    def seq_len(self, seq_id: int) -> int:
        self._need(seq_id)
        return self.lens[seq_id]

    def block_table(self, seq_id: int) -> list:
        self._need(seq_id)
        return list(self.tables[seq_id])

    def free_list(self) -> list:
        return list(self.free)

    def build_block_tables(self, seq_ids, max_blocks: int):
        """Rows of physical block ids, padded with -1 to `max_blocks`, and the context lengths."""
        tables, lens = [], []
        for s in seq_ids:
            self._need(s)
            if s in self.swapped:
                raise AllocatorError(INVALID_ARG, "sequence is swapped out")
            t = self.tables[s]
            if len(t) > max_blocks:
                raise AllocatorError(INVALID_ARG, "block table longer than max_blocks")
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return tables, lens

    # -- prefix caching ------------------------------------------------------
    def prefix_get_or_create(self, tokens):
        """Entry for this prompt prefix: (entry id, hit).  A hit adds a user; a miss takes
        ceil(n / bs) blocks (one reference each, held by the entry) with one user."""
        key = tuple(int(t) for t in tokens)
        if key in self.prefixes:
            pid = self.prefixes[key]
            self.entries[pid]["users"] += 1
            return pid, True
        nb = self._blocks_for(len(key))
        if nb > len(self.free):
            raise AllocatorError(NO_FREE_BLOCKS)
        pid = self.next_prefix_id
        self.next_prefix_id += 1
        self.entries[pid] = {"blocks": [self._take() for _ in range(nb)], "users": 1, "length": len(key),
                             "key": key}
        self.prefixes[key] = pid
        return pid, False

    def _entry(self, pid):
        if pid not in self.entries:
            raise AllocatorError(UNKNOWN_PREFIX, f"prefix {pid}")
        return self.entries[pid]

    def prefix_release(self, pid):
        """Drop one user; at zero the entry releases its blocks (table order) and is removed."""
        e = self._entry(pid)
        e["users"] -= 1
        if e["users"] <= 0:
            for b in e["blocks"]:
                self._release(b)
            del self.prefixes[e["key"]]
            del self.entries[pid]

    def prefix_info(self, pid):
        """(blocks, token count, users) of an entry."""
        e = self._entry(pid)
        return list(e["blocks"]), e["length"], e["users"]

    def seq_create_with_prefix(self, seq_id, pid, own_tokens: int):
        """Sequence = the entry's blocks (one more reference each), then ceil(own / bs) fresh
        blocks for its own tokens at positions P*bs ..; positions n_p .. P*bs - 1 are a hole."""
        if seq_id in self.tables:
            raise AllocatorError(SEQ_EXISTS, str(seq_id))
        if own_tokens < 0:
            raise AllocatorError(INVALID_ARG, "own_tokens < 0")
        e = self._entry(pid)
        nb = self._blocks_for(own_tokens)
        if nb > len(self.free):
            raise AllocatorError(NO_FREE_BLOCKS)
        for b in e["blocks"]:
            self.refs[b] += 1
        P = len(e["blocks"])
        self.tables[seq_id] = list(e["blocks"]) + [self._take() for _ in range(nb)]
        self.lens[seq_id] = P * self.block_size + own_tokens
        if e["length"] < P * self.block_size:
            self.holes[seq_id] = (e["length"], P * self.block_size)

    def masks(self, seq_ids):
        """Per sequence the positions [lo, hi) that hold no token (lo = hi = 0: none)."""
        lo, hi = [], []
        for s in seq_ids:
            self._need(s)
            a, b = self.holes.get(s, (0, 0))
            if s in self.windows:
                a, b = 0, max(0, self.lens[s] - self.windows[s])
            lo.append(a)
            hi.append(b)
        return lo, hi

    # -- sliding window --------------------------------------------------------
    def _drop_behind_window(self, seq_id):
        start = self.lens[seq_id] - self.windows[seq_id]
        t = self.tables[seq_id]
        for j in range(len(t)):
            if (j + 1) * self.block_size > start:
                break
            if t[j] >= 0:
                self._release(t[j])
                t[j] = -1

    def seq_set_window(self, seq_id, window: int):
        """Keep only the last `window` positions live; release the blocks wholly before them."""
        self._need(seq_id)
        if window < 1:
            raise AllocatorError(INVALID_ARG, "window < 1")
        if seq_id in self.swapped or seq_id in self.holes:
            raise AllocatorError(INVALID_ARG, "window on a swapped sequence or one with a prefix hole")
        self.windows[seq_id] = window
        self._drop_behind_window(seq_id)

    # -- swap to the host pool -------------------------------------------------
    def set_host_pool(self, num_host_blocks: int):
        """(Re)create the host pool of num_host_blocks blocks, ids 0.. in order; only while empty."""
        if num_host_blocks < 0:
            raise AllocatorError(INVALID_ARG, "num_host_blocks < 0")
        if self.swapped:
            raise AllocatorError(INVALID_ARG, "sequences are swapped out")
        self.host_free = deque(range(num_host_blocks))
        self.host_refs = [0] * num_host_blocks

    def _release_host(self, h):
        self.host_refs[h] -= 1
        if self.host_refs[h] == 0:
            self.host_free.append(h)

    def _group(self, seq_ids, swapped: bool):
        ids = list(dict.fromkeys(seq_ids))
        for s in ids:
            self._need(s)
            if (s in self.swapped) != swapped:
                raise AllocatorError(INVALID_ARG, "sequence already swapped out" if not swapped else
                                     "sequence is not swapped out")
        distinct = list(dict.fromkeys(b for s in ids for b in self.tables[s] if b >= 0))
        return ids, distinct

    def seq_swap_out(self, seq_ids):
        """Move a group to the host pool; returns the (device, host) copy pairs."""
        ids, distinct = self._group(seq_ids, False)
        if len(distinct) > len(self.host_free):
            raise AllocatorError(NO_FREE_BLOCKS, "host pool")
        where = {}
        for b in distinct:
            h = self.host_free.popleft()
            self.host_refs[h] = 0
            where[b] = h
        for s in ids:
            t = self.tables[s]
            for j, b in enumerate(t):
                if b >= 0:
                    t[j] = where[b]
                    self.host_refs[where[b]] += 1
                    self._release(b)
            self.swapped.add(s)
        return [(b, where[b]) for b in distinct]

    def seq_swap_in(self, seq_ids):
        """Move a swapped group back to the device pool; returns the (host, device) copy pairs."""
        ids, distinct = self._group(seq_ids, True)
        if len(distinct) > len(self.free):
            raise AllocatorError(NO_FREE_BLOCKS)
        where = {}
        for h in distinct:
            d = self.free.popleft()
            self.refs[d] = 0
            self.stats["blocks_allocated"] += 1
            where[h] = d
        for s in ids:
            t = self.tables[s]
            for j, h in enumerate(t):
                if h >= 0:
                    t[j] = where[h]
                    self.refs[where[h]] += 1
                    self._release_host(h)
            self.swapped.discard(s)
        return [(h, where[h]) for h in distinct]

    def host_free_list(self) -> list:
        return list(self.host_free)
