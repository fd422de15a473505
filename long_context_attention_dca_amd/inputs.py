"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers; it holds none of the attention
arithmetic.  Recipe (fixed so that any consumer can regenerate the exact same
values): a CPU ``torch.Generator`` seeded with ``seed`` draws Q, then K, then V
with ``torch.randn`` in fp32 at their full shapes, each is multiplied by its
scale (default 1/sqrt(D)), then cast to the requested dtype (round to nearest
even for bf16).

"Discriminating" inputs use the same recipe with q and k scaled by 2 (logits
with a standard deviation of about 4), so that a wrong position map moves the
output far beyond bf16 rounding; v keeps the 1/sqrt(D) scale.
"""
from __future__ import annotations

import math

import torch

_DTYPES = {"f32": torch.float32, "fp32": torch.float32, "float32": torch.float32,
           "bf16": torch.bfloat16, "bfloat16": torch.bfloat16}


def torch_dtype(dtype) -> torch.dtype:
    if isinstance(dtype, torch.dtype):
        return dtype
    return _DTYPES[str(dtype)]


def _draw(gen, shape, scale, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    x.mul_(scale)
    return x.to(torch_dtype(dtype))


def prefill_inputs(B, L, Hq, Hkv, D, dtype="bf16", seed=0, qk_scale=None, v_scale=None):
    """Q [B, L, Hq, D], K and V [B, L, Hkv, D] on the CPU."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    a = 1.0 / math.sqrt(D) if qk_scale is None else float(qk_scale)
    av = 1.0 / math.sqrt(D) if v_scale is None else float(v_scale)
    q = _draw(g, (B, L, Hq, D), a, dtype)
    k = _draw(g, (B, L, Hkv, D), a, dtype)
    v = _draw(g, (B, L, Hkv, D), av, dtype)
    return q, k, v


def decode_inputs(B, kv_len, Hq, Hkv, D, dtype="bf16", seed=0, qk_scale=None, v_scale=None):
    """q [B, Hq, D] (the new token), raw K and V caches [B, kv_len, Hkv, D] on the CPU."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    a = 1.0 / math.sqrt(D) if qk_scale is None else float(qk_scale)
    av = 1.0 / math.sqrt(D) if v_scale is None else float(v_scale)
    q = _draw(g, (B, Hq, D), a, dtype)
    k = _draw(g, (B, kv_len, Hkv, D), a, dtype)
    v = _draw(g, (B, kv_len, Hkv, D), av, dtype)
    return q, k, v


# The workloads the pages' long-context setting is measured on, as synthetic
# stand-ins (Llama2-7B / 70B attention shapes, 16k-128k tokens).  Seeds are the
# workload's index in this table.
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", dtype="f32", B=1, L=512, Hq=1, Hkv=1, D=64,
                     c=128, w=32, base=10000.0, seed=0),
    "llama2_7b_16k": dict(kind="prefill", dtype="bf16", B=1, L=16384, Hq=32, Hkv=32, D=128,
                          c=4096, w=1024, base=10000.0, seed=1),
    "llama2_70b_32k": dict(kind="prefill", dtype="bf16", B=1, L=32768, Hq=64, Hkv=8, D=128,
                           c=4096, w=1024, base=10000.0, seed=2),
    "decode_100k": dict(kind="decode", dtype="bf16", B=16, kv_len=100001, Hq=64, Hkv=8, D=128,
                        c=4096, w=1024, base=10000.0, seed=3),
    "llama2_70b_128k": dict(kind="prefill", dtype="bf16", B=1, L=131072, Hq=64, Hkv=8, D=128,
                            c=4096, w=1024, base=10000.0, seed=4),
    # SelfExtend grouped / neighbor attention on the 70B 32k shape.  The group
    # size and neighbor window are not given by the pages: G = 8 and W = 1024
    # (the same local window as the DCA workloads).
    "selfextend_70b_32k": dict(kind="selfextend", dtype="bf16", B=1, L=32768, Hq=64, Hkv=8, D=128,
                               group=8, window=1024, base=10000.0, seed=5),
    # The DCA guide's coarse / fine map with its own parameters (chunk 512,
    # trained length 4096, target 32768) on the 70B 32k shape.
    "coarse_fine_70b_32k": dict(kind="coarse_fine", dtype="bf16", B=1, L=32768, Hq=64, Hkv=8, D=128,
                                chunk=512, train_len=4096, target_len=32768, base=10000.0, seed=6),
    # The 70B 32k shape with a local window of 1000, so that the chunk size
    # s = c - w = 3096 is not a multiple of the key tiles (every chunk boundary
    # falls inside a tile).
    "llama2_70b_32k_s3096": dict(kind="prefill", dtype="bf16", B=1, L=32768, Hq=64, Hkv=8, D=128,
                                 c=4096, w=1000, base=10000.0, seed=7),
}
