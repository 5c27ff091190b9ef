"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and fixes workload shapes.  It holds none
of the arithmetic of the method: no block counts, no address translation, no
attention, no allocation.  Both the CPU oracle and the HIP path read their
inputs from here, so the two sides start from identical bytes.

Workloads (shapes follow the LLaMA-7B-style layer the pages use: 32 heads of
dimension 128, blocks of 16 or 32 tokens, contexts up to 2048 and beyond):

  1 tiny-fp32      fp32, 4 seqs, 4/4 heads, D 64,  bs 16, ctx {1,16,17,45}, pool 16
  2 llama7b-fp16   fp16, 64 seqs, 32/32 heads, D 128, bs 16, ctx U{256..2048}, pool 8192
  3 gqa-bf16       bf16, 256 seqs, 32/8 heads, D 128, bs 32, ctx round(exp U(ln128, ln4096)),
                   pool ceil(1.1 x blocks needed)
  4 long-fp16      fp16, 4 seqs, 32/32 heads, D 128, bs 16, ctx {32768,65536,100000,131072},
                   pool 22645, split into 512-token partitions
  5 cow-fp16       fp16, 32 groups x 5 branches, 32/32 heads, D 128, bs 16, a 2048-token shared
                   prefix plus a per-branch suffix U{0..256}
  6 llama7b-fp8kv  workload 2's shapes (own draw of lengths and free order) with 8-bit FP8 E4M3
                   pools, fp16 query/output, k_scale 0.0165, v_scale 0.0145
  7 gqa-bf16-int8kv  workload 3's shapes (own draw) with int8 pools, bf16 query/output,
                   k_scale 0.031, v_scale 0.029
  8 llama7b-fp16-verify4  workload 2's shapes (own draw) with 4 query tokens per sequence
                   (a speculative verification pass of 4 draft tokens)
  9 llama7b-int8tok  workload 2's shapes (own draw) with int8 pools holding one float32
                   scale per (token, KV head), fp16 query/output

Draw order for workload k (numpy PCG64, seed 1000+k): context lengths, then the
pool's initial free order (a permutation), then (workload 5) the suffix
lengths.  Tensor contents (pools, q, new K/V) come from `normal_host` (numpy,
small cases) or `normal_device` (torch's device generator, full-size pools),
each with its own derived seed.  Normals are drawn in float32 and rounded to
nearest-even into fp16/bf16.  8-bit pools hold codes drawn the same way at a
code scale of CODE_SIGMA (N(0, CODE_SIGMA^2) in code units) and rounded onto
the code grid: torch's float8_e4m3fn cast after clamping to +-448, or the
nearest integer clamped to +-127; `normal_codes_host` / `normal_codes_device`.
With scale ~ 1 / CODE_SIGMA the values they stand for are about N(0, 1).
Pools with a scale per (token, KV head) take their scales from `row_scales_host` /
`row_scales_device`: uniform in [0.75, 1.25] / CODE_SIGMA, one per row.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
KV_FORMATS = ("fp8_e4m3", "int8", "int8_token")
CODE_SIGMA = {"fp8_e4m3": 64.0, "int8": 32.0, "int8_token": 32.0}


@dataclass
class Workload:
    key: int
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: list = field(default_factory=list)
    num_blocks: int = 0
    free_order: np.ndarray | None = None
    partition_size: int = 0
    # workload 5 only: groups, branches per group, prefix and parent lengths, suffixes
    groups: int = 0
    branches: int = 0
    prefix_len: int = 0
    parent_len: int = 0
    suffix_lens: list = field(default_factory=list)
    # 8-bit pools (workloads 6, 7): code format and per-pool scales
    kv_format: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0
    # query tokens per sequence per step (workload 8: 4, a verification pass)
    query_len: int = 1

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def seed(self) -> int:
        return 1000 + self.key


def rng_for(key: int) -> np.random.Generator:
    return np.random.default_rng(1000 + key)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def workload(key: int) -> Workload:
    """Shapes, context lengths and pool free order of workload `key` (1..9)."""
    rng = rng_for(key)
    if key == 1:
        w = Workload(1, "tiny-fp32-mha", "f32", 4, 4, 4, 64, 16)
        w.context_lens = [1, 16, 17, 45]
        w.num_blocks = 16
        w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
        return w
    if key == 2:
        w = Workload(2, "llama7b-fp16-mha", "f16", 64, 32, 32, 128, 16)
        w.context_lens = [int(x) for x in rng.integers(256, 2048, size=64, endpoint=True)]
        w.num_blocks = 8192
        w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
        return w
    if key == 3:
        w = Workload(3, "gqa-bf16", "bf16", 256, 32, 8, 128, 32)
        u = rng.uniform(math.log(128), math.log(4096), size=256)
        w.context_lens = [int(min(4096, max(128, round(math.exp(x))))) for x in u]
        # Pool sizing is a shape parameter of the workload (1.1x the blocks
        # the contexts occupy), stated by the workload itself.
        need = sum(_ceil_div(c, 32) for c in w.context_lens)
        w.num_blocks = _ceil_div(11 * need, 10)
        w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
        return w
    if key == 4:
        w = Workload(4, "long-fp16-split", "f16", 4, 32, 32, 128, 16)
        w.context_lens = [32768, 65536, 100000, 131072]
        need = sum(_ceil_div(c, 16) for c in w.context_lens)
        w.num_blocks = _ceil_div(11 * need, 10)
        w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
        w.partition_size = 512
        return w
    if key == 5:
        w = Workload(5, "cow-fp16-parallel-sampling", "f16", 160, 32, 32, 128, 16)
        w.groups, w.branches = 32, 5
        w.prefix_len, w.parent_len = 2048, 2048 + 256
        parent_blocks = _ceil_div(w.parent_len, 16)
        # room for every parent, one fresh block and one copy per branch, x1.1
        w.num_blocks = _ceil_div(11 * (w.groups * parent_blocks + 2 * w.num_seqs), 10)
        w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
        w.suffix_lens = [int(x) for x in rng.integers(0, 256, size=w.num_seqs, endpoint=True)]
        w.context_lens = [w.prefix_len + s for s in w.suffix_lens]
        return w
    if key == 6:
        w = workload_shapes_like(2, key, rng)
        w.name, w.kv_format = "llama7b-fp8kv", "fp8_e4m3"
        w.k_scale, w.v_scale = float(np.float32(0.0165)), float(np.float32(0.0145))
        return w
    if key == 7:
        w = workload_shapes_like(3, key, rng)
        w.name, w.kv_format = "gqa-bf16-int8kv", "int8"
        w.k_scale, w.v_scale = float(np.float32(0.031)), float(np.float32(0.029))
        return w
    if key == 8:
        w = workload_shapes_like(2, key, rng)
        w.name, w.query_len = "llama7b-fp16-verify4", 4
        return w
    if key == 9:
        w = workload_shapes_like(2, key, rng)
        w.name, w.kv_format = "llama7b-int8tok", "int8_token"
        return w
    raise ValueError(f"unknown workload {key}")


def workload_shapes_like(base: int, key: int, rng: np.random.Generator) -> Workload:
    """Workload `base`'s shapes and length distribution, drawn again from `rng`."""
    if base == 2:
        w = Workload(key, "", "f16", 64, 32, 32, 128, 16)
        w.context_lens = [int(x) for x in rng.integers(256, 2048, size=64, endpoint=True)]
        w.num_blocks = 8192
    else:
        w = Workload(key, "", "bf16", 256, 32, 8, 128, 32)
        u = rng.uniform(math.log(128), math.log(4096), size=256)
        w.context_lens = [int(min(4096, max(128, round(math.exp(x))))) for x in u]
        need = sum(_ceil_div(c, 32) for c in w.context_lens)
        w.num_blocks = _ceil_div(11 * need, 10)
    w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
    return w


def with_block_size(w: Workload, block_size: int) -> Workload:
    """Workload w with another block size: the same contexts, a pool of the same token capacity
    (num_blocks * block_size kept, rounded up) and a free order drawn again, from a seed of
    the workload and the block size."""
    import dataclasses
    v = dataclasses.replace(w)
    v.block_size = block_size
    v.num_blocks = _ceil_div(w.num_blocks * w.block_size, block_size)
    v.free_order = np.random.default_rng(
        np.random.SeedSequence([1000 + w.key, block_size])).permutation(v.num_blocks).astype(np.int32)
    if w.partition_size:
        v.partition_size = max(w.partition_size, block_size)
    return v


def pool_shapes(w: Workload):
    """Shapes of the key pool [NB, H_kv, bs, D] and the value pool [NB, H_kv, D, bs]."""
    return ((w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim),
            (w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size))


# ----------------------------------------------------------------------------
# tensor contents


def _round_to(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type.

    Returns float32 / float16 arrays, and for bf16 the raw uint16 bit patterns
    (numpy has no bfloat16); torch's float32 -> bfloat16 conversion rounds to
    nearest-even.
    """
    if dtype == "f32":
        return x32.astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def normal_host(shape, seed: int, dtype: str) -> np.ndarray:
    """N(0,1) draws in float32 from numpy PCG64(seed), rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return _round_to(x, dtype)


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def normal_device(shape, seed: int, dtype: str, device="cuda"):
    """N(0,1) draws from torch's generator on `device`, rounded to `dtype`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch_dtype(dtype))


def to_torch(arr: np.ndarray, dtype: str):
    """numpy storage array (bf16 as uint16 bits) -> CPU torch tensor of `dtype`."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr))


def to_numpy(t, dtype: str) -> np.ndarray:
    """torch tensor of `dtype` (any device) -> numpy storage array (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def normal_codes_host(shape, seed: int, fmt: str) -> np.ndarray:
    """8-bit codes (uint8) of N(0, CODE_SIGMA^2) float32 draws from numpy PCG64(seed)."""
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(CODE_SIGMA[fmt])
    return _codes(torch.from_numpy(x), fmt).numpy()


def normal_codes_device(shape, seed: int, fmt: str, device="cuda"):
    """8-bit codes (torch.uint8 on `device`) of N(0, CODE_SIGMA^2) draws from torch's generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * CODE_SIGMA[fmt]
    return _codes(x, fmt)


def row_scales_host(shape, seed: int) -> np.ndarray:
    """float32 scales, one per (block, KV head, token row): uniform in [0.75, 1.25] / 32,
    from numpy PCG64(seed)."""
    rng = np.random.default_rng(seed)
    return ((np.float32(0.75) + np.float32(0.5) * rng.random(size=shape, dtype=np.float32))
            / np.float32(CODE_SIGMA["int8_token"])).astype(np.float32)


def row_scales_device(shape, seed: int, device="cuda"):
    """The same distribution from torch's generator on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return (0.75 + 0.5 * u) / CODE_SIGMA["int8_token"]


def _codes(x, fmt: str):
    import torch
    if fmt == "fp8_e4m3":
        return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    if fmt in ("int8", "int8_token"):
        return x.round().clamp(-127.0, 127.0).to(torch.int8).view(torch.uint8)
    raise ValueError(fmt)


def tensor_seeds(key: int) -> dict:
    """Derived seeds for the tensor contents of workload `key`."""
    base = 1000 + key
    return {"key_cache": base * 16 + 1, "value_cache": base * 16 + 2, "query": base * 16 + 3,
            "new_key": base * 16 + 4, "new_value": base * 16 + 5, "key_scales": base * 16 + 6,
            "value_scales": base * 16 + 7}
