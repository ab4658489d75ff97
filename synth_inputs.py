"""Seeded synthetic inputs for the five workloads.

Shared by the tests, the bench and the smoke check.  This module holds no
attention arithmetic: it only draws random numbers with torch's CPU
generator (fp32 standard normal) and rounds them to the storage dtype with
round-to-nearest-even.  Both the CPU oracle and the GPU library read the
same bytes.

Workloads (sizes as named by the pages' examples):

1. fp32 demo: the Ultralytics glossary's PyTorch demo exactly -- seed 0,
   ``randn(3, 1, 8, 1000, 64)`` split into q, k, v; chunk 256.
2. GQA bf16: 4000-token prompt, 32 query / 8 KV heads, head dim 128,
   cache capacity 8192, chunk width 512 (ONNX GenAI Wiki "Chunked
   Prefill", section 1).
3. Padding ladder: same shapes, five prompt lengths uniform in [100, 5500]
   plus 1137 and 1200 (same page, section 3).
4. Rolling fp16: 16 heads, head dim 128, C = 2048, c = 256, L = 4096
   (Horizon developer blog "Chunk Prefill").
5. Mixed step: 64 decode sequences with contexts uniform in [512, 16384]
   plus a 20,000-token prompt, budgets 2048 and 8192 (Ultralytics glossary
   "Chunked Prefill", sections on generation stalls and the token budget).
"""
from __future__ import annotations

import numpy as np
import torch

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

SEEDS = {"demo": 0, "gqa": 1, "ladder": 2, "rolling": 3, "mixed": 4}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def randn(shape, dtype: str, gen: torch.Generator) -> torch.Tensor:
    """fp32 standard normal draw rounded (RNE) to the storage dtype, on CPU."""
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    return x.to(TORCH_DTYPE[dtype]).contiguous()


def storage(t: torch.Tensor) -> np.ndarray:
    """Raw storage view as numpy: fp32 values, or fp16/bf16 bit patterns as
    uint16 (numpy has no bfloat16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def demo_qkv():
    """The demo's tensors: seed 0, randn(3, 1, 8, 1000, 64).unbind(0), each
    [1, 8, 1000, 64].  Returned both as the demo's own head-major tensors
    and as token-major [1000, 8, 64] tensors for the library's layout."""
    g = generator(SEEDS["demo"])
    q, k, v = torch.randn(3, 1, 8, 1000, 64, generator=g).unbind(0)
    tm = [x[0].permute(1, 0, 2).contiguous() for x in (q, k, v)]
    return (q, k, v), tuple(tm)


def gqa_prompt(L=4000, Hq=32, Hkv=8, D=128, dtype="bf16", seed=None):
    """Token-major q [L, Hq, D], k and v [L, Hkv, D]."""
    g = generator(SEEDS["gqa"] if seed is None else seed)
    q = randn((L, Hq, D), dtype, g)
    k = randn((L, Hkv, D), dtype, g)
    v = randn((L, Hkv, D), dtype, g)
    return q, k, v


def ladder_prompt_lengths(seed=None):
    """Five lengths uniform in [100, 5500], then 1137 and 1200."""
    g = generator(SEEDS["ladder"] if seed is None else seed)
    drawn = torch.randint(100, 5501, (5,), generator=g).tolist()
    return [int(x) for x in drawn] + [1137, 1200]


def rolling_inputs(L=4096, H=16, D=128, dtype="f16", seed=None):
    g = generator(SEEDS["rolling"] if seed is None else seed)
    q = randn((L, H, D), dtype, g)
    k = randn((L, H, D), dtype, g)
    v = randn((L, H, D), dtype, g)
    return q, k, v


def mixed_contexts(n_decode=64, lo=512, hi=16384, seed=None):
    """Context lengths of the running decode sequences, uniform in [lo, hi]."""
    g = generator(SEEDS["mixed"] if seed is None else seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n_decode,), generator=g)]


def fill_seeded(t: torch.Tensor, seed: int) -> torch.Tensor:
    """Fill an existing (possibly device) tensor in place with a seeded fp32
    standard normal draw rounded to its dtype.  Drawn on the tensor's device
    in slabs so that multi-GB caches need no host copy."""
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    n = flat.numel()
    slab = 1 << 26
    for s in range(0, n, slab):
        e = min(n, s + slab)
        flat[s:e] = torch.randn(e - s, generator=g, device=t.device,
                                dtype=torch.float32).to(t.dtype)
    return t
