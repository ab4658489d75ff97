"""The no-allocation packed mixed step (cpk_varlen_step_noalloc) through the
C ABI: the same outputs, cache bytes and lengths as cpk_varlen_step with a
caller workspace, bit for bit, on two calls in a row (the second with a
smaller step, so it must not depend on what the first left in the library's
scratch), and a step whose decode partials exceed the scratch is refused
without touching the cache."""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunked_prefill_causal_kv_amd as cpk  # noqa: E402


def _bitwise(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _step(n_dec, ctx_lo, ctx_hi, prompt_rows, prompt_past, Hq, Hkv, D, seed):
    """Two identical caches and one packed step's inputs: n_dec decode rows
    with contexts in [ctx_lo, ctx_hi] and one prompt chunk."""
    ctxs = si.mixed_contexts(n_dec, ctx_lo, ctx_hi, seed=seed)
    cap = max(max(ctxs) + 1, prompt_past + prompt_rows) + 8
    caches = []
    for _ in range(2):
        c = cpk.KVCache(n_dec + 1, Hkv, cap, D, torch.bfloat16)
        si.fill_seeded(c.k, seed + 1)
        si.fill_seeded(c.v, seed + 2)
        c.seqlens_k.copy_(torch.tensor(ctxs + [prompt_past], dtype=torch.int32))
        c.lens = ctxs + [prompt_past]
        caches.append(c)
    g = si.generator(seed + 3)
    total = n_dec + prompt_rows
    q = si.randn((total, Hq, D), "bf16", g).cuda()
    kn = si.randn((total, Hkv, D), "bf16", g).cuda()
    vn = si.randn((total, Hkv, D), "bf16", g).cuda()
    slots = list(range(n_dec + 1))
    cu = list(range(n_dec + 1)) + [total]
    past = ctxs + [prompt_past]
    return caches, q, kn, vn, slots, cu, past


@pytest.mark.parametrize("shape", [
    # (n_dec, ctx_lo, ctx_hi, prompt_rows, prompt_past, Hq, Hkv, D): a large
    # step, then a smaller one on the same scratch
    [(48, 2000, 9000, 700, 300, 32, 8, 128), (5, 20, 600, 90, 40, 8, 2, 64)],
])
def test_noalloc_step_equals_workspace_step_twice(shape):
    for i, (n_dec, lo, hi, rows, ppast, Hq, Hkv, D) in enumerate(shape):
        print(f"case: no-alloc step {i}: {n_dec} decodes ctx {lo}..{hi}, prompt {rows} rows "
              f"at {ppast}, heads {Hq}/{Hkv} D={D}", flush=True)
        caches, q, kn, vn, slots, cu, past = _step(n_dec, lo, hi, rows, ppast, Hq, Hkv, D,
                                                   seed=700 + 10 * i)
        ref = cpk.cpk_varlen_step(q, kn, vn, caches[0], slots, cu, past)
        got = cpk.cpk_varlen_step_noalloc(q, kn, vn, caches[1], slots, cu, past)
        torch.cuda.synchronize()
        assert _bitwise(ref, got), f"step {i}: outputs differ"
        assert _bitwise(caches[0].k, caches[1].k) and _bitwise(caches[0].v, caches[1].v)
        assert torch.equal(caches[0].seqlens_k, caches[1].seqlens_k)


def test_noalloc_refuses_a_step_beyond_the_scratch():
    """32 decode rows of 8 query heads (one KV head) at context 200,000 need
    32 * 8 * 782 * 132 * 4 bytes of decode partials (105.7 MB), beyond the
    96 MiB scratch: the call fails with CPK_EWORKSPACE before any launch, so
    neither the cache nor its lengths change."""
    n, Hq, Hkv, D, ctx = 32, 8, 1, 128, 200000
    need = cpk.cpk_varlen_workspace_size(n, Hq, ctx + 1, D)
    assert need > cpk.NOALLOC_SCRATCH_BYTES
    print(f"case: no-alloc refusal: {n} decodes at ctx {ctx}, partials {need} bytes", flush=True)
    cache = cpk.KVCache(n, Hkv, ctx + 8, D, torch.bfloat16)
    cache.seqlens_k.fill_(ctx)
    cache.lens = [ctx] * n
    cache.k[:, :, ctx - 4:ctx + 8].fill_(1.0)
    q = torch.zeros((n, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((n, Hkv, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cpk.CpkError) as e:
        cpk.cpk_varlen_step_noalloc(q, kn, kn, cache, list(range(n)), list(range(n + 1)),
                                    [ctx] * n)
    assert e.value.status == cpk.CPK_EWORKSPACE, e.value
    torch.cuda.synchronize()
    assert bool((cache.k[:, :, ctx - 4:ctx + 8] == 1.0).all()), "cache written"
    assert bool((cache.seqlens_k == ctx).all())
