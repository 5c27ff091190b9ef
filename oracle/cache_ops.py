"""Oracle for the two pool-writing operations (test infrastructure only).

* Slot-mapping write: token i's new K/V rows go to slot = slot_mapping[i],
  i.e. physical block slot // bs at offset slot % bs ("Ascend C算子开发高阶实战…"
  §3.1 params: slot_mapping maps a token to (block id, offset in block);
  "PagedAttention 实现细节" §3.4, writing the new KV into its block after each
  step).  A negative slot means "no write" (the pages are silent; plain
  reading: padding tokens are skipped).
* Block copy for copy-on-write: the whole source block, K and V, every KV head,
  every row, is copied to the destination block ("PagedAttention 实现细节"
  §3.3: copy the full contents of the original block to the new one).  Pairs
  are applied in list order.
* Block swap between the device pool and a host pool: the same whole-block copy,
  from block src of one pool pair to block dst of another (the CPU-side cache of
  "PagedAttention 实现细节" §3.4's cache engine, swapping blocks out to host
  memory and back).

Pools: key_cache [NB, H_kv, bs, D] (token rows), value_cache [NB, H_kv, D, bs]
(block size innermost, "Ascend C算子开发高阶实战…" §3.1/§5.2), so a token's
value vector is written down column `offset` of its tile.  Arrays are NumPy
storage arrays (bf16 as uint16 bits), so the results are bit patterns and
compare bit-exactly.  8-bit pools hold uint8 codes; their write quantises
first (reshape_and_cache_quant), their block copy is the same byte copy.  The
int8 form with a scale per (token, KV head) keeps those scales in arrays
[NB, H_kv, bs] beside the code pools (reshape_and_cache_int8_token); a block
copy copies them with the same copy_blocks.
"""
from __future__ import annotations

import numpy as np

from . import quant as Q


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Return copies of the pools with key[i], value[i] ([H_kv, D]) written at slot_mapping[i]."""
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    block_size = kc.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        kc[block, :, offset, :] = key[i]
        vc[block, :, :, offset] = value[i]
    return kc, vc


def reshape_and_cache_quant(key, value, key_cache, value_cache, slot_mapping, dtype: str, fmt: str,
                            k_scale: float, v_scale: float):
    """The slot-mapping write into 8-bit pools: each new row is quantised
    (code = Q(x / scale), oracle/quant.py; keys with k_scale, values with
    v_scale), then written exactly like reshape_and_cache."""
    return reshape_and_cache(Q.quantize(key, dtype, k_scale, fmt), Q.quantize(value, dtype, v_scale, fmt),
                             key_cache, value_cache, slot_mapping)


def reshape_and_cache_int8_token(key, value, key_cache, value_cache, k_scales, v_scales, slot_mapping,
                                 dtype: str):
    """The slot-mapping write into int8 pools with per-(token, KV head) scales: each new
    key and value row is quantised on its own (oracle/quant.py quantize_rows_int8), its
    codes written like reshape_and_cache, its scale at k_scales / v_scales [block, KV head,
    offset].  Returns copies of the four pools."""
    kcodes, ksc = Q.quantize_rows_int8(key, dtype)
    vcodes, vsc = Q.quantize_rows_int8(value, dtype)
    kc, vc = reshape_and_cache(kcodes, vcodes, key_cache, value_cache, slot_mapping)
    ks = np.array(k_scales, copy=True)
    vs = np.array(v_scales, copy=True)
    block_size = ks.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        ks[block, :, offset] = ksc[i]
        vs[block, :, offset] = vsc[i]
    return kc, vc, ks, vs


def copy_blocks(key_cache, value_cache, pairs):
    """Return copies of the pools after copying block src -> dst for each (src, dst) pair."""
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc


def swap_blocks(dst_key, dst_value, src_key, src_value, pairs):
    """Return copies of the destination pools after copying block src of the source pools to
    block dst of the destination pools, for each (src, dst) pair in list order."""
    kd = np.array(dst_key, copy=True)
    vd = np.array(dst_value, copy=True)
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        kd[dst] = src_key[src]
        vd[dst] = src_value[src]
    return kd, vd
