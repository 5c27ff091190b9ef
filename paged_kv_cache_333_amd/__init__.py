"""PagedAttention decode for MI355X (gfx950): Python binding of libpa.so.

Argument marshalling only.  Every step runs in the C++ allocator or the HIP
kernels of libpa.so; torch tensors supply device memory and the current
stream.  Importing this package fails loudly when libpa.so has not been
built (python paged_kv_cache_333_amd/build.py): there is no fallback.

Names follow the C ABI in include/pa.h:
  pa_reshape_and_cache, pa_copy_blocks, pa_upload, pa_decode, pa_decode_split, pa_decode_split_static,
  pa_decode_auto,
  pa_decode_append, pa_reshape_and_cache_quant, pa_decode_quant, pa_decode_masked, pa_decode_multi,
  pa_decode_multi_workspace_bytes, pa_swap_blocks, pa_upload_and_cache,
  pa_decode_split_workspace_bytes, pa_lse_reduce, and the allocator verbs as
  methods of `Allocator` (pa_seq_create -> Allocator.seq_create, ...).
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_333_amd/build.py`")

# torch ships its own HIP runtime.  Loading torch first makes the dynamic
# linker satisfy libpa.so's libamdhip64.so.7 / libhsa-runtime64.so.1 with the
# copies torch already mapped (same sonames), so torch's device memory and
# streams and libpa.so's kernels live in one runtime.
try:
    import torch as _torch_runtime  # noqa: F401
except ImportError:  # plain C use: libpa.so binds to the system runtime
    _torch_runtime = None
lib = C.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps", encoding="utf-8") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return sorted(paths)


_RUNTIMES = _hip_runtimes_mapped()
if len(_RUNTIMES) > 1:
    raise ImportError("two HIP runtimes are mapped in this process (" + ", ".join(_RUNTIMES) + "); "
                      "import torch before anything that loads another libamdhip64")

PA_OK = 0
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_NO_FREE_BLOCKS", 3: "PA_ERR_UNKNOWN_SEQ",
          4: "PA_ERR_SEQ_EXISTS", 5: "PA_ERR_UNSUPPORTED", 6: "PA_ERR_BAD_TABLE",
          7: "PA_ERR_WORKSPACE_TOO_SMALL", 8: "PA_ERR_HIP", 9: "PA_ERR_UNKNOWN_PREFIX"}
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PA_INT8, PA_INT8_TOKEN = 0, 1, 2, 3, 4, 5
PA_DECODE_CACHED_KV = 1
PA_DECODE_SPLIT = 2
DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16}
KV_FORMATS = {"fp8_e4m3": PA_FP8_E4M3, "int8": PA_INT8, "int8_token": PA_INT8_TOKEN}

_i32, _u32, _i64, _f32, _vp, _sz = C.c_int32, C.c_uint32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
_pi32, _pi64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)


class pa_allocator_stats(C.Structure):
    _fields_ = [("blocks_allocated", C.c_int64), ("blocks_freed", C.c_int64), ("cow_copies", C.c_int64)]


_PROTOS = {
    "pa_allocator_create": (_i32, [_i32, _i32, _pi32, C.POINTER(_vp)]),
    "pa_allocator_destroy": (None, [_vp]),
    "pa_allocator_clone": (_i32, [_vp, C.POINTER(_vp)]),
    "pa_seq_create": (_i32, [_vp, _i64, _i32]),
    "pa_seq_fork": (_i32, [_vp, _i64, _i64, _i32]),
    "pa_seq_append_slot": (_i32, [_vp, _i64, _pi32, _pi32, _pi32]),
    "pa_seq_append_slots": (_i32, [_vp, _pi64, _i32, _pi32, _pi32, _pi32]),
    "pa_seq_free": (_i32, [_vp, _i64]),
    "pa_can_allocate": (_i32, [_vp, _i32, _pi32]),
    "pa_num_free_blocks": (_i32, [_vp]),
    "pa_ref_count": (_i32, [_vp, _i32]),
    "pa_seq_len": (_i32, [_vp, _i64, _pi32]),
    "pa_seq_block_table": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pa_free_list": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_build_block_tables": (_i32, [_vp, _pi64, _i32, _i32, _pi32, _pi32]),
    "pa_allocator_get_stats": (_i32, [_vp, C.POINTER(pa_allocator_stats)]),
    "pa_prefix_get_or_create": (_i32, [_vp, _pi32, _i32, _pi64, _pi32]),
    "pa_prefix_release": (_i32, [_vp, _i64]),
    "pa_prefix_info": (_i32, [_vp, _i64, _pi32, _i32, _pi32, _pi32, _pi32]),
    "pa_seq_create_with_prefix": (_i32, [_vp, _i64, _i64, _i32]),
    "pa_build_masks": (_i32, [_vp, _pi64, _i32, _pi32, _pi32]),
    "pa_allocator_set_host_pool": (_i32, [_vp, _i32]),
    "pa_seq_swap_out": (_i32, [_vp, _pi64, _i32, _pi32, _i32, _pi32]),
    "pa_seq_swap_in": (_i32, [_vp, _pi64, _i32, _pi32, _i32, _pi32]),
    "pa_host_free_list": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_host_ref_count": (_i32, [_vp, _i32]),
    "pa_seq_set_window": (_i32, [_vp, _i64, _i32]),
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_order_longest_first": (_i32, [_pi32, _i32, _pi32]),
    "pa_upload": (_i32, [_vp, _vp, _sz, _vp]),
    "pa_set_launch_events": (_i32, [_vp, _vp]),
    "pa_upload_and_cache": (_i32, [_vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                   _f32, _i32, _i32, _vp]),
    "pa_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                         _f32, _i32, _u32, _vp]),
    "pa_decode_split_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_split": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _f32, _i32, _u32, _i32, _vp, _sz, _vp]),
    "pa_decode_auto": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                              _i32, _f32, _i32, _u32, _i32, _vp, _sz, _pi32, _vp]),
    "pa_decode_split_static": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _f32, _i32, _u32, _i32, _vp]),
    "pa_decode_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _f32, _i32, _u32, _i32, _vp, _sz, _pi32, _vp]),
    "pa_lse_reduce": (_i32, [_vp, _vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_reshape_and_cache_quant": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _f32, _f32, _vp]),
    "pa_decode_masked": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _f32, _f32, _f32, _i32, _i32, _u32, _i32, _vp, _sz, _pi32, _vp]),
    "pa_decode_multi_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_multi": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, _f32, _f32, _f32, _i32, _i32, _u32, _i32, _vp, _sz, _pi32, _vp]),
    "pa_decode_shared_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pa_decode_shared": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _f32, _f32, _f32, _i32, _i32, _u32, _vp, _sz, _vp]),
    "pa_shared_prefix_groups": (_i32, [_pi32, _pi32, _i32, _i32, _i32, _pi32, _pi32, _pi32, _pi32]),
    "pa_decode_quant": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _f32, _f32, _f32, _i32, _i32, _u32, _i32, _vp, _sz, _pi32, _vp]),
    "pa_status_string": (C.c_char_p, [_i32]),
    "pa_last_error": (C.c_char_p, []),
    "pa_abi_version": (_i32, []),
}
for _name, (_res, _args) in _PROTOS.items():
    try:
        _fn = getattr(lib, _name)
    except AttributeError as _e:
        raise ImportError(f"{LIB_PATH} lacks {_name}: it is out of date, rebuild it with "
                          "`python paged_kv_cache_333_amd/build.py`") from _e
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_PROTOS)


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        detail = lib.pa_last_error().decode()
        super().__init__(f"{where}: {self.code} ({detail})")


def _check(status: int, where: str):
    if status != PA_OK:
        raise PAError(status, where)


# ---------------------------------------------------------------------------
# device operations (torch tensors in, nothing computed here)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t) -> int:
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpa must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    return _torch().cuda.current_stream().cuda_stream


def _pool_dims(key_cache, value_cache, head_dim=None):
    """(NB, H_kv, bs, D) from key_cache [NB, H_kv, bs, D]; value_cache must be [NB, H_kv, D, bs].
    Pools of int8 codes with a scale per (token, KV head) are uint8 [NB, H_kv, tile] (see
    token_pool): their head_dim must be given, bs follows from it."""
    if key_cache.dim() == 3:
        NB, H_kv, tile = key_cache.shape
        if head_dim is None:
            raise ValueError("pools of int8 codes with row scales need head_dim")
        bs = next((b for b in (16, 32, 64) if token_tile_bytes(b, head_dim) == tile), None)
        if bs is None or tuple(value_cache.shape) != tuple(key_cache.shape) or \
                key_cache.element_size() != 1 or value_cache.element_size() != 1:
            raise ValueError(f"row-scaled int8 pools must both be uint8 [num_blocks, num_kv_heads, "
                             f"token_tile_bytes(block_size, {head_dim})]; got {tuple(key_cache.shape)} and "
                             f"{tuple(value_cache.shape)}")
        return NB, H_kv, bs, head_dim
    NB, H_kv, bs, D = key_cache.shape
    if tuple(value_cache.shape) != (NB, H_kv, D, bs) or value_cache.dtype != key_cache.dtype:
        raise ValueError(f"value_cache must be [num_blocks, num_kv_heads, head_dim, block_size] = "
                         f"{(NB, H_kv, D, bs)} of {key_cache.dtype}, got {tuple(value_cache.shape)} "
                         f"of {value_cache.dtype}")
    return NB, H_kv, bs, D


def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """key, value [T, H_kv, D]; key_cache [NB, H_kv, bs, D]; value_cache [NB, H_kv, D, bs];
    slot_mapping int32 [T]."""
    NB, H_kv, bs, D = _pool_dims(key_cache, value_cache)
    _check(lib.pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                    _ptr(slot_mapping), slot_mapping.numel(), NB, H_kv, D, bs,
                                    _dtype_code(key_cache), _stream(stream)), "pa_reshape_and_cache")


def token_tile_bytes(block_size: int, head_dim: int) -> int:
    """Bytes of one (block, KV head) tile of a row-scaled int8 pool (PA_TOKEN_TILE_BYTES): the
    block_size * head_dim codes, then a scale area of whole 128-byte lines."""
    return block_size * head_dim + (block_size * 4 + 127) // 128 * 128


def token_scale_offsets(block_size: int, head_dim: int):
    """Where a row-scaled int8 block keeps its scales: (byte of the key scales in the key tile,
    byte of the value scales, True if those sit in the key tile).  With 16-token blocks both
    sets share the key tile's one scale line; otherwise each tile holds its own."""
    area = block_size * head_dim
    paired = 8 * block_size <= (block_size * 4 + 127) // 128 * 128
    return area, (area + 4 * block_size if paired else area), paired


def token_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, device="cuda"):
    """A zeroed pool of int8 codes with a scale per (token, KV head) (kv_format "int8_token"):
    uint8 [num_blocks, num_kv_heads, token_tile_bytes(block_size, head_dim)], each (block, KV
    head) tile its codes (keys [block_size, head_dim], values [head_dim, block_size]) followed
    by its scale area (token_scale_offsets)."""
    torch = _torch()
    return torch.zeros((num_blocks, num_kv_heads, token_tile_bytes(block_size, head_dim)), dtype=torch.uint8,
                       device=device)


def pack_token_pools(k_codes, k_scales, v_codes, v_scales):
    """Row-scaled int8 key and value pools from their parts: codes uint8 [NB, H_kv, bs, D]
    (keys) and [NB, H_kv, D, bs] (values), scales float32 [NB, H_kv, bs]; unused bytes zero."""
    torch = _torch()
    NB, H_kv, bs, D = k_codes.shape
    ko, vo, paired = token_scale_offsets(bs, D)
    kp = torch.zeros((NB, H_kv, token_tile_bytes(bs, D)), dtype=torch.uint8, device=k_codes.device)
    vp = torch.zeros_like(kp)
    kp[:, :, :bs * D] = k_codes.reshape(NB, H_kv, -1)
    vp[:, :, :bs * D] = v_codes.reshape(NB, H_kv, -1)
    kp[:, :, ko:ko + 4 * bs] = k_scales.contiguous().view(torch.uint8).reshape(NB, H_kv, -1)
    (kp if paired else vp)[:, :, vo:vo + 4 * bs] = v_scales.contiguous().view(torch.uint8).reshape(NB, H_kv, -1)
    return kp, vp


def unpack_token_pools(key_pool, value_pool, block_size: int, head_dim: int):
    """(key codes [NB, H_kv, bs, D], key scales [NB, H_kv, bs], value codes [NB, H_kv, D, bs],
    value scales [NB, H_kv, bs]) of a pair of row-scaled int8 pools."""
    NB, H_kv, tile = key_pool.shape
    bs, D = block_size, head_dim
    if tile != token_tile_bytes(bs, D) or tuple(value_pool.shape) != tuple(key_pool.shape):
        raise ValueError("not a pair of row-scaled int8 pools of this block size and head_dim")
    ko, vo, paired = token_scale_offsets(bs, D)
    f32 = _torch().float32
    kc = key_pool[:, :, :bs * D].reshape(NB, H_kv, bs, D)
    vc = value_pool[:, :, :bs * D].reshape(NB, H_kv, D, bs)
    ks = key_pool[:, :, ko:ko + 4 * bs].contiguous().view(f32)
    vs = (key_pool if paired else value_pool)[:, :, vo:vo + 4 * bs].contiguous().view(f32)
    return kc, ks, vc, vs


def pa_copy_blocks(key_cache, value_cache, pairs, stream=None, num_pairs=None, head_dim=None):
    """pairs int32 [P, 2] (src, dst) on the device; num_pairs may cover a prefix of it.
    8-bit pools (one-byte elements) are copied as such; row-scaled int8 pools (3-D, see
    token_pool) need head_dim and are copied with their scales."""
    NB, H_kv, bs, D = _pool_dims(key_cache, value_cache, head_dim)
    P = pairs.shape[0] if num_pairs is None else num_pairs
    code = (PA_INT8_TOKEN if key_cache.dim() == 3 else PA_FP8_E4M3) if key_cache.element_size() == 1 \
        else _dtype_code(key_cache)
    _check(lib.pa_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(pairs), P, NB, H_kv, D, bs,
                              code, _stream(stream)), "pa_copy_blocks")


def _kv_format(key_cache, kv_format):
    """Code type of 8-bit pools: `kv_format` ("fp8_e4m3" or "int8"), else from the pool dtype
    (torch.float8_e4m3fn or torch.int8); uint8 pools need kv_format."""
    torch = _torch()
    if key_cache.element_size() != 1:
        raise TypeError(f"8-bit pools expected, got {key_cache.dtype}")
    if key_cache.dim() == 3:  # the row-scaled int8 layout
        if kv_format not in (None, "int8_token"):
            raise ValueError("3-D pools hold int8 codes with row scales (kv_format 'int8_token')")
        return PA_INT8_TOKEN
    if kv_format is None:
        kv_format = {torch.float8_e4m3fn: "fp8_e4m3", torch.int8: "int8"}.get(key_cache.dtype)
        if kv_format is None:
            raise TypeError("uint8 pools need kv_format='fp8_e4m3' or 'int8'")
    return KV_FORMATS[kv_format]


def pa_reshape_and_cache_quant(key, value, key_cache, value_cache, slot_mapping, k_scale: float, v_scale: float,
                               kv_format=None, stream=None):
    """The slot-mapping write into 8-bit pools: key, value [T, H_kv, D] (f32/f16/bf16) are
    stored as codes of x / k_scale and x / v_scale (row-scaled int8 pools: each row with its
    own scale, k_scale and v_scale unused)."""
    NB, H_kv, bs, D = _pool_dims(key_cache, value_cache, key.shape[-1])
    _check(lib.pa_reshape_and_cache_quant(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                          _ptr(slot_mapping), slot_mapping.numel(), NB, H_kv, D, bs,
                                          _dtype_code(key), _kv_format(key_cache, kv_format), k_scale, v_scale,
                                          _stream(stream)), "pa_reshape_and_cache_quant")


def pa_upload_and_cache(dst, src, key, value, key_cache, value_cache, slot_mapping_host, k_scale: float = 1.0,
                        v_scale: float = 1.0, kv_format=None, stream=None):
    """pa_upload(dst, src) and the slot-mapping write of key, value [T, H_kv, D] in one launch;
    slot_mapping_host: int32 [T] in pinned host memory (e.g. a view into src).  8-bit pools
    take the quantising write with k_scale, v_scale."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("pa_upload_and_cache: dst and src differ in size")
    NB, H_kv, bs, D = _pool_dims(key_cache, value_cache, key.shape[-1])
    kv = _kv_format(key_cache, kv_format) if key_cache.element_size() == 1 else _dtype_code(key_cache)
    _check(lib.pa_upload_and_cache(_ptr(dst), _ptr(src), nbytes, _ptr(key), _ptr(value), _ptr(key_cache),
                                   _ptr(value_cache), _ptr(slot_mapping_host), slot_mapping_host.numel(), NB, H_kv,
                                   D, bs, k_scale, v_scale, _dtype_code(key), kv, _stream(stream)),
           "pa_upload_and_cache")


def pa_swap_blocks(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache, pairs, stream=None,
                   num_pairs=None, head_dim=None):
    """Whole-block copies pairs[p] = (src id, dst id) between two pools of the same block shape,
    each on the device or in pinned host memory (swap out: device -> host; swap in: host ->
    device).  pairs: int32 [P, 2] on the device or pinned."""
    NB_d, H_kv, bs, D = _pool_dims(dst_key_cache, dst_value_cache, head_dim)
    NB_s = _pool_dims(src_key_cache, src_value_cache, head_dim)[0]
    if tuple(src_key_cache.shape[1:]) != tuple(dst_key_cache.shape[1:]) or src_key_cache.dtype != dst_key_cache.dtype:
        raise ValueError("source and destination pools differ in block shape or dtype")
    P = pairs.shape[0] if num_pairs is None else num_pairs
    code = (PA_INT8_TOKEN if dst_key_cache.dim() == 3 else PA_FP8_E4M3) if dst_key_cache.element_size() == 1 \
        else _dtype_code(dst_key_cache)
    _check(lib.pa_swap_blocks(_ptr(dst_key_cache), _ptr(dst_value_cache), _ptr(src_key_cache),
                              _ptr(src_value_cache), _ptr(pairs), P, NB_s, NB_d, H_kv, D, bs, code,
                              _stream(stream)), "pa_swap_blocks")


def pa_set_launch_events(start_event, stop_event):
    """Time the next decode call on this thread by events riding on its kernels' own dispatches
    (no marker packet between kernels): start_event records the start of its first kernel,
    stop_event the end of its last.  Events are torch.cuda.Event(enable_timing=True) objects that
    have been recorded once (so that they exist), or None."""
    def raw(ev):
        if ev is None:
            return None
        h = ev.cuda_event
        if not h:
            raise ValueError("pa_set_launch_events: record the event once first, so that it exists")
        return h
    _check(lib.pa_set_launch_events(raw(start_event), raw(stop_event)), "pa_set_launch_events")


def pa_upload(dst, src, stream=None):
    """Copy the pinned host tensor `src` into the device tensor `dst` (same byte size) with a
    kernel on the stream: no copy engine, no cross-engine synchronisation."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("pa_upload: dst and src differ in size")
    if not src.is_pinned():
        raise ValueError("pa_upload: src must be a pinned host tensor (pin_memory())")
    _check(lib.pa_upload(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "pa_upload")


def _opt(t):
    return None if t is None else _ptr(t)


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
              scale: float, stream=None, seq_order=None, cached_kv: bool = False):
    """out, query [S, H, D]; key_cache [NB, H_kv, bs, D]; value_cache [NB, H_kv, D, bs];
    block_tables [S, MB]; context_lens [S];
    seq_order: optional device int32 [S] launch order (see pa_order_longest_first);
    cached_kv: read K/V with the default cache policy (pools with shared blocks)."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    _check(lib.pa_decode(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                         _ptr(context_lens), _opt(seq_order), S, H, H_kv, D, bs, block_tables.shape[1], NB,
                         max_context_len, scale, _dtype_code(query), PA_DECODE_CACHED_KV if cached_kv else 0,
                         _stream(stream)), "pa_decode")


def pa_decode_split_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                                    partition_size: int) -> int:
    return lib.pa_decode_split_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size)


def pa_decode_split(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
                    scale: float, partition_size: int, workspace, stream=None, seq_order=None,
                    cached_kv: bool = False):
    """As pa_decode; workspace is a device tensor of at least pa_decode_split_workspace_bytes bytes."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.pa_decode_split(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                               _ptr(block_tables), _ptr(context_lens), _opt(seq_order), S, H, H_kv, D, bs,
                               block_tables.shape[1], NB, max_context_len, scale, _dtype_code(query),
                               PA_DECODE_CACHED_KV if cached_kv else 0, partition_size, _ptr(workspace), nbytes,
                               _stream(stream)), "pa_decode_split")


PA_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024


def pa_decode_split_static(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
                           scale: float, partition_size: int, stream=None, seq_order=None, cached_kv: bool = False):
    """As pa_decode_split, with the partials in the library's static per-device workspace
    (PA_STATIC_SCRATCH_BYTES): no workspace argument, no allocation."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    _check(lib.pa_decode_split_static(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                      _ptr(block_tables), _ptr(context_lens), _opt(seq_order), S, H, H_kv, D, bs,
                                      block_tables.shape[1], NB, max_context_len, scale, _dtype_code(query),
                                      PA_DECODE_CACHED_KV if cached_kv else 0, partition_size, _stream(stream)),
           "pa_decode_split_static")


def pa_decode_auto(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
                   scale: float, partition_size: int = 512, workspace=None, stream=None, seq_order=None,
                   cached_kv: bool = False) -> str:
    """pa_decode or pa_decode_split, chosen by the library for this launch; returns
    "single" or "split"."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    path = C.c_int32(-1)
    _check(lib.pa_decode_auto(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                              _ptr(context_lens), _opt(seq_order), S, H, H_kv, D, bs, block_tables.shape[1], NB,
                              max_context_len, scale, _dtype_code(query), PA_DECODE_CACHED_KV if cached_kv else 0,
                              partition_size, _opt(workspace), nbytes, C.byref(path), _stream(stream)),
           "pa_decode_auto")
    return "split" if path.value == 1 else "single"


def pa_decode_append(out, query, key, value, slot_mapping, key_cache, value_cache, block_tables, context_lens,
                     max_context_len: int, scale: float, partition_size: int = 512, workspace=None, stream=None,
                     seq_order=None, cached_kv: bool = False) -> str:
    """pa_reshape_and_cache of one new token per sequence (key, value [S, H_kv, D] at
    slot_mapping [S]) fused into pa_decode_auto; returns "single" or "split"."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    if tuple(key.shape) != (S, H_kv, D) or tuple(value.shape) != (S, H_kv, D) or slot_mapping.numel() != S:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim] and slot_mapping [num_seqs]")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    path = C.c_int32(-1)
    _check(lib.pa_decode_append(_ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(slot_mapping),
                                _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(context_lens),
                                _opt(seq_order), S, H, H_kv, D, bs, block_tables.shape[1], NB, max_context_len,
                                scale, _dtype_code(query), PA_DECODE_CACHED_KV if cached_kv else 0, partition_size,
                                _opt(workspace), nbytes, C.byref(path), _stream(stream)), "pa_decode_append")
    return "split" if path.value == 1 else "single"


def pa_decode_quant(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len: int,
                    scale: float, k_scale: float, v_scale: float, kv_format=None, partition_size: int = 512,
                    workspace=None, split: bool = False, stream=None, seq_order=None,
                    cached_kv: bool = False) -> str:
    """Decode over 8-bit pools (K = code * k_scale, V = code * v_scale) with f16/bf16 query and
    output.  Single pass without a workspace; split with split=True; else the pa_decode_auto
    rule.  Returns "single" or "split"."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (PA_DECODE_CACHED_KV if cached_kv else 0) | (PA_DECODE_SPLIT if split else 0)
    path = C.c_int32(-1)
    _check(lib.pa_decode_quant(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                               _ptr(context_lens), _opt(seq_order), S, H, H_kv, D, bs, block_tables.shape[1], NB,
                               max_context_len, scale, k_scale, v_scale, _dtype_code(query),
                               _kv_format(key_cache, kv_format), flags, partition_size, _opt(workspace), nbytes,
                               C.byref(path), _stream(stream)), "pa_decode_quant")
    return "split" if path.value == 1 else "single"


def pa_decode_masked(out, query, key_cache, value_cache, block_tables, context_lens, mask_lo, mask_hi,
                     max_context_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                     kv_format=None, partition_size: int = 512, workspace=None, split: bool = False, stream=None,
                     seq_order=None, cached_kv: bool = False) -> str:
    """Decode leaving out positions mask_lo[s] <= t < mask_hi[s] (device int32 [S] each, or both
    None): a prefix hole or the tokens before a sliding window.  Pools of the query's dtype, or
    8-bit pools (K = code * k_scale, V = code * v_scale).  Single pass without a workspace; split
    with split=True; else the pa_decode_auto rule.  Returns "single" or "split"."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    kv = _kv_format(key_cache, kv_format) if key_cache.element_size() == 1 else _dtype_code(key_cache)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (PA_DECODE_CACHED_KV if cached_kv else 0) | (PA_DECODE_SPLIT if split else 0)
    path = C.c_int32(-1)
    _check(lib.pa_decode_masked(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                _ptr(context_lens), _opt(mask_lo), _opt(mask_hi), _opt(seq_order), S, H, H_kv, D,
                                bs, block_tables.shape[1], NB, max_context_len, scale, k_scale, v_scale,
                                _dtype_code(query), kv, flags, partition_size, _opt(workspace), nbytes,
                                C.byref(path), _stream(stream)), "pa_decode_masked")
    return "split" if path.value == 1 else "single"


def pa_decode_multi_workspace_bytes(num_query_tokens: int, num_heads: int, head_dim: int, max_context_len: int,
                                    partition_size: int) -> int:
    return lib.pa_decode_multi_workspace_bytes(num_query_tokens, num_heads, head_dim, max_context_len,
                                               partition_size)


def pa_decode_multi(out, query, key_cache, value_cache, block_tables, context_lens, query_start, max_query_len: int,
                    max_context_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0, kv_format=None,
                    partition_size: int = 512, workspace=None, split: bool = False, stream=None, seq_order=None,
                    cached_kv: bool = False) -> str:
    """Several causal query tokens per sequence: query/out [T, H, D], query_start int32 [S + 1]
    (rows of sequence s: query_start[s] .. query_start[s+1]-1, its last tokens).  Returns
    "single" or "split"."""
    T, H, D = query.shape
    S = context_lens.numel()
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    if query_start.numel() != S + 1:
        raise ValueError("query_start must hold num_seqs + 1 offsets")
    kv = _kv_format(key_cache, kv_format) if key_cache.element_size() == 1 else _dtype_code(key_cache)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (PA_DECODE_CACHED_KV if cached_kv else 0) | (PA_DECODE_SPLIT if split else 0)
    path = C.c_int32(-1)
    _check(lib.pa_decode_multi(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                               _ptr(context_lens), _ptr(query_start), _opt(seq_order), S, T, max_query_len, H, H_kv,
                               D, bs, block_tables.shape[1], NB, max_context_len, scale, k_scale, v_scale,
                               _dtype_code(query), kv, flags, partition_size, _opt(workspace), nbytes,
                               C.byref(path), _stream(stream)), "pa_decode_multi")
    return "split" if path.value == 1 else "single"


def pa_lse_reduce(out, workspace, context_lens, max_context_len: int, partition_size: int, stream=None):
    """out [S, H, D]; workspace holds the split partials for the same S, H, D."""
    S, H, D = out.shape
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.pa_lse_reduce(_ptr(out), _ptr(workspace), nbytes, _ptr(context_lens), S, H, D,
                             max_context_len, partition_size, _dtype_code(out), _stream(stream)),
           "pa_lse_reduce")


def pa_decode_shared_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int) -> int:
    return lib.pa_decode_shared_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len)


def pa_decode_shared(out, query, key_cache, value_cache, block_tables, context_lens, group_start, prefix_len,
                     num_groups: int, max_group_size: int, max_context_len: int, scale: float, workspace,
                     k_scale: float = 1.0, v_scale: float = 1.0, kv_format=None, stream=None,
                     cached_kv: bool = False):
    """Decode of sequences that share their leading blocks in groups (device int32
    group_start [num_groups + 1] and prefix_len [S], e.g. from pa_shared_prefix_groups):
    each group's shared prefix is read once for all its members, then each sequence's own
    tokens, merged.  Same result as pa_decode; workspace of pa_decode_shared_workspace_bytes."""
    S, H, D = query.shape
    NB, H_kv, bs, _ = _pool_dims(key_cache, value_cache, query.shape[-1])
    kv = _kv_format(key_cache, kv_format) if key_cache.element_size() == 1 else _dtype_code(key_cache)
    nbytes = workspace.numel() * workspace.element_size()
    flags = PA_DECODE_CACHED_KV if cached_kv else 0
    _check(lib.pa_decode_shared(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                _ptr(context_lens), _ptr(group_start), _ptr(prefix_len), S, num_groups,
                                max_group_size, H, H_kv, D, bs, block_tables.shape[1], NB, max_context_len, scale,
                                k_scale, v_scale, _dtype_code(query), kv, flags, _ptr(workspace), nbytes,
                                _stream(stream)), "pa_decode_shared")


def pa_shared_prefix_groups(tables, context_lens, block_size: int):
    """Host helper: (group_start list [G + 1], prefix_len list [S], num_groups, max_group_size)
    from host block tables (S rows of max_blocks ids) and context lengths [S]: sequences that
    share their leading blocks with their neighbours form a group."""
    n = len(context_lens)
    rows = [list(r) for r in tables]
    mb = len(rows[0]) if rows else 0
    if any(len(r) != mb for r in rows) or len(rows) != n:
        raise ValueError("tables must have one row of max_blocks ids per sequence")
    tab = (C.c_int32 * max(n * mb, 1))(*[int(x) for r in rows for x in r])
    lens = (C.c_int32 * max(n, 1))(*[int(x) for x in context_lens])
    gs = (C.c_int32 * (n + 1))()
    pl = (C.c_int32 * max(n, 1))()
    ng, mg = C.c_int32(0), C.c_int32(0)
    _check(lib.pa_shared_prefix_groups(tab, lens, n, mb, block_size, gs, pl, C.byref(ng), C.byref(mg)),
           "pa_shared_prefix_groups")
    return list(gs[:ng.value + 1]), list(pl[:n]), ng.value, mg.value


def pa_shared_prefix_groups_into(tables_ptr: int, lens_ptr: int, n: int, max_blocks: int, block_size: int,
                                 group_start_ptr: int, prefix_len_ptr: int):
    """Raw form for pinned host buffers (int32 pointers); returns (num_groups, max_group_size)."""
    ng, mg = C.c_int32(0), C.c_int32(0)
    _check(lib.pa_shared_prefix_groups(C.cast(tables_ptr, _pi32), C.cast(lens_ptr, _pi32), n, max_blocks,
                                       block_size, C.cast(group_start_ptr, _pi32), C.cast(prefix_len_ptr, _pi32),
                                       C.byref(ng), C.byref(mg)), "pa_shared_prefix_groups")
    return ng.value, mg.value


def pa_order_longest_first(context_lens) -> list:
    """Indices of the sequences from the longest context to the shortest (ties in index order)."""
    n = len(context_lens)
    lens = (C.c_int32 * max(n, 1))(*[int(x) for x in context_lens])
    order = (C.c_int32 * max(n, 1))()
    _check(lib.pa_order_longest_first(lens, n, order), "pa_order_longest_first")
    return list(order[:n])


def pa_order_longest_first_into(lens_ptr: int, n: int, order_ptr: int):
    """Raw form for pinned host buffers (int32 pointers)."""
    _check(lib.pa_order_longest_first(C.cast(lens_ptr, _pi32), n, C.cast(order_ptr, _pi32)),
           "pa_order_longest_first")


def split_layout(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int, partition_size: int):
    """Byte offsets and partition count of the split workspace, as documented in include/pa.h."""
    P = -(-max_context_len // partition_size)
    units = num_seqs * num_heads * P
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    off_l = a256(units * 4)
    off_o = off_l + a256(units * 4)
    return {"parts": P, "off_m": 0, "off_l": off_l, "off_o": off_o, "total": off_o + units * head_dim * 4}


# ---------------------------------------------------------------------------
# host allocator


class Allocator:
    """Host block allocator (pa_allocator_* / pa_seq_* in include/pa.h)."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None, _handle=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        if _handle is not None:
            self._h = _handle
            return
        h = _vp()
        order = None
        if initial_free_order is not None:
            arr = (C.c_int32 * num_blocks)(*[int(x) for x in initial_free_order])
            order = C.cast(arr, _pi32)
        _check(lib.pa_allocator_create(num_blocks, block_size, order, C.byref(h)), "pa_allocator_create")
        self._h = h

    _destroy = lib.pa_allocator_destroy  # kept on the class: module globals may be gone at exit

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    def clone(self) -> "Allocator":
        h = _vp()
        _check(lib.pa_allocator_clone(self._h, C.byref(h)), "pa_allocator_clone")
        return Allocator(self.num_blocks, self.block_size, _handle=h)

    def seq_create(self, seq_id: int, num_tokens: int):
        _check(lib.pa_seq_create(self._h, seq_id, num_tokens), "pa_seq_create")

    def seq_fork(self, parent: int, child: int, num_tokens: int = -1):
        _check(lib.pa_seq_fork(self._h, parent, child, num_tokens), "pa_seq_fork")

    def seq_append_slot(self, seq_id: int):
        slot, src, dst = C.c_int32(), C.c_int32(), C.c_int32()
        _check(lib.pa_seq_append_slot(self._h, seq_id, C.byref(slot), C.byref(src), C.byref(dst)),
               "pa_seq_append_slot")
        return slot.value, src.value, dst.value

    def seq_append_slots_into(self, seq_ids_ptr: int, n: int, slots_ptr: int, pairs_ptr: int) -> int:
        """Raw form for pinned host buffers: pointers to int64 ids, int32 slots, int32 pairs."""
        np_ = C.c_int32()
        _check(lib.pa_seq_append_slots(self._h, C.cast(seq_ids_ptr, _pi64), n, C.cast(slots_ptr, _pi32),
                                       C.cast(pairs_ptr, _pi32), C.byref(np_)), "pa_seq_append_slots")
        return np_.value

    def seq_append_slots(self, seq_ids):
        n = len(seq_ids)
        ids = (C.c_int64 * max(n, 1))(*seq_ids)
        slots = (C.c_int32 * max(n, 1))()
        pairs = (C.c_int32 * max(2 * n, 2))()
        np_ = C.c_int32()
        _check(lib.pa_seq_append_slots(self._h, ids, n, slots, pairs, C.byref(np_)), "pa_seq_append_slots")
        return list(slots[:n]), [(pairs[2 * i], pairs[2 * i + 1]) for i in range(np_.value)]

    def seq_free(self, seq_id: int):
        _check(lib.pa_seq_free(self._h, seq_id), "pa_seq_free")

    def can_allocate(self, num_blocks: int) -> bool:
        ok = C.c_int32()
        _check(lib.pa_can_allocate(self._h, num_blocks, C.byref(ok)), "pa_can_allocate")
        return bool(ok.value)

    def num_free_blocks(self) -> int:
        return lib.pa_num_free_blocks(self._h)

    def ref_count(self, block: int) -> int:
        return lib.pa_ref_count(self._h, block)

    def seq_len(self, seq_id: int) -> int:
        n = C.c_int32()
        _check(lib.pa_seq_len(self._h, seq_id, C.byref(n)), "pa_seq_len")
        return n.value

    def block_table(self, seq_id: int) -> list:
        cap = self.num_blocks + 1
        buf = (C.c_int32 * cap)()
        n = C.c_int32()
        _check(lib.pa_seq_block_table(self._h, seq_id, buf, cap, C.byref(n)), "pa_seq_block_table")
        return list(buf[: n.value])

    def free_list(self) -> list:
        cap = max(self.num_blocks, 1)
        buf = (C.c_int32 * cap)()
        n = C.c_int32()
        _check(lib.pa_free_list(self._h, buf, cap, C.byref(n)), "pa_free_list")
        return list(buf[: n.value])

    def build_block_tables(self, seq_ids, max_blocks: int):
        n = len(seq_ids)
        ids = (C.c_int64 * max(n, 1))(*seq_ids)
        tabs = (C.c_int32 * max(n * max_blocks, 1))()
        lens = (C.c_int32 * max(n, 1))()
        _check(lib.pa_build_block_tables(self._h, ids, n, max_blocks, tabs, lens), "pa_build_block_tables")
        return ([list(tabs[i * max_blocks:(i + 1) * max_blocks]) for i in range(n)], list(lens[:n]))

    def build_block_tables_into(self, seq_ids_ptr: int, n: int, max_blocks: int, tables_ptr: int,
                                lens_ptr: int):
        """Raw form for pinned host buffers."""
        _check(lib.pa_build_block_tables(self._h, C.cast(seq_ids_ptr, _pi64), n, max_blocks,
                                         C.cast(tables_ptr, _pi32), C.cast(lens_ptr, _pi32)),
               "pa_build_block_tables")

    # -- prefix caching --------------------------------------------------------
    def prefix_get_or_create(self, tokens):
        """(entry id, hit) for this prompt prefix; a miss takes ceil(n / bs) blocks."""
        n = len(tokens)
        arr = (C.c_int32 * max(n, 1))(*[int(t) for t in tokens])
        pid, hit = C.c_int64(), C.c_int32()
        _check(lib.pa_prefix_get_or_create(self._h, arr, n, C.byref(pid), C.byref(hit)), "pa_prefix_get_or_create")
        return pid.value, bool(hit.value)

    def prefix_release(self, prefix_id: int):
        _check(lib.pa_prefix_release(self._h, prefix_id), "pa_prefix_release")

    def prefix_info(self, prefix_id: int):
        """(blocks, token count, users) of an entry."""
        nb, nt, users = C.c_int32(), C.c_int32(), C.c_int32()
        _check(lib.pa_prefix_info(self._h, prefix_id, None, 0, C.byref(nb), None, None), "pa_prefix_info")
        buf = (C.c_int32 * max(nb.value, 1))()
        _check(lib.pa_prefix_info(self._h, prefix_id, buf, nb.value, C.byref(nb), C.byref(nt), C.byref(users)),
               "pa_prefix_info")
        return list(buf[:nb.value]), nt.value, users.value

    def seq_create_with_prefix(self, seq_id: int, prefix_id: int, own_tokens: int):
        _check(lib.pa_seq_create_with_prefix(self._h, seq_id, prefix_id, own_tokens), "pa_seq_create_with_prefix")

    def masks(self, seq_ids):
        """Per sequence the positions [lo, hi) with no token: (lo list, hi list)."""
        n = len(seq_ids)
        ids = (C.c_int64 * max(n, 1))(*seq_ids)
        lo, hi = (C.c_int32 * max(n, 1))(), (C.c_int32 * max(n, 1))()
        _check(lib.pa_build_masks(self._h, ids, n, lo, hi), "pa_build_masks")
        return list(lo[:n]), list(hi[:n])

    # -- swap and sliding window ------------------------------------------------
    def set_host_pool(self, num_host_blocks: int):
        _check(lib.pa_allocator_set_host_pool(self._h, num_host_blocks), "pa_allocator_set_host_pool")

    def _swap(self, fn, seq_ids, where):
        n = len(seq_ids)
        ids = (C.c_int64 * max(n, 1))(*seq_ids)
        cap = 0
        for s in set(seq_ids):
            try:
                cap += len(self.block_table(s))
            except PAError:
                pass
        buf = (C.c_int32 * max(2 * cap, 2))()
        k = C.c_int32()
        _check(fn(self._h, ids, n, buf, cap, C.byref(k)), where)
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(k.value)]

    def seq_swap_out(self, seq_ids):
        """Move a group to the host pool; returns the (device, host) copy pairs."""
        return self._swap(lib.pa_seq_swap_out, seq_ids, "pa_seq_swap_out")

    def seq_swap_in(self, seq_ids):
        """Move a swapped group back; returns the (host, device) copy pairs."""
        return self._swap(lib.pa_seq_swap_in, seq_ids, "pa_seq_swap_in")

    def host_free_list(self) -> list:
        n = C.c_int32()
        cap = 1 << 20
        buf = (C.c_int32 * cap)()
        _check(lib.pa_host_free_list(self._h, buf, cap, C.byref(n)), "pa_host_free_list")
        return list(buf[:n.value])

    def host_ref_count(self, block: int) -> int:
        return lib.pa_host_ref_count(self._h, block)

    def seq_set_window(self, seq_id: int, window: int):
        _check(lib.pa_seq_set_window(self._h, seq_id, window), "pa_seq_set_window")

    def stats(self) -> dict:
        st = pa_allocator_stats()
        _check(lib.pa_allocator_get_stats(self._h, C.byref(st)), "pa_allocator_get_stats")
        return {"blocks_allocated": st.blocks_allocated, "blocks_freed": st.blocks_freed,
                "cow_copies": st.cow_copies}


from .cache import PagedAttention  # noqa: E402  (the object interface over the calls above)
