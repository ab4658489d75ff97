"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Cache contents are compared byte for byte; outputs element by element
within the stated tolerances (fp32 max-abs 1e-5, bf16 2e-2, fp16 8.4e-3,
derived below), at sizes the oracle finishes in seconds and, at the workloads' full
sizes, on sampled rows.  Bitwise self-checks of the GPU path (chunked ==
one-shot, padded == unpadded, explicit mask == computed mask) guard the
properties the pages state exactly.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import chunked_prefill_causal_kv_amd as cpk  # noqa: E402

# Output tolerances (max-abs against the fp64 oracle).  fp32: the demo's
# allclose bound.  bf16: the stated 2e-2.  fp16 (fp32 accumulation, P and
# the output rounded to fp16, unit roundoff u = 2^-11): the output is a
# convex combination of V rows, so rounding it costs at most u*|o| <= u*Vmax,
# and rounding each weight by a relative u moves the combination by at most
# u * sum_j w_j |v_j - o| <= 2u*Vmax; with Vmax <= 5.7 (the largest |v| of
# the fp16 inputs, 5.65 for the 4096x16x128 rolling workload) the bound is
# 3 * 2^-11 * 5.7 = 8.4e-3.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 8.4e-3}
ODT = {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16, torch.float16: oracle.F16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check(gpu: torch.Tensor, ref: np.ndarray, tol: float, what: str):
    g = f64(gpu)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    say(f"  {what}: max-abs err {err:.3e} (tol {tol:g})")
    assert err <= tol, f"{what}: max-abs {err} > {tol}"


def bitwise(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                       b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))


def sample_rows(L, chunks, every=13):
    rows = set(range(0, L, every))
    for past, r in chunks:
        rows.update(range(past, min(past + 4, L)))
        rows.update(range(max(past, past + r - 4), past + r))
    return np.array(sorted(rows))


def oracle_rows(q, k, v, rows_idx, dtype):
    """One-shot causal oracle at selected absolute rows (token-major raw
    storage arrays of the whole prompt)."""
    L, Hq, D = q.shape
    n_keys = int(rows_idx.max()) + 1
    qq = oracle.widen(np.ascontiguousarray(q[rows_idx]), dtype)
    kk = oracle.widen(np.ascontiguousarray(k[:n_keys].transpose(1, 0, 2)), dtype)
    vv = oracle.widen(np.ascontiguousarray(v[:n_keys].transpose(1, 0, 2)), dtype)
    lo = np.zeros(len(rows_idx), np.int32)
    return oracle.attention(qq, kk, vv, lo, rows_idx.astype(np.int32), 1.0 / math.sqrt(D))


def poison(cache: cpk.KVCache):
    """Fill every cache byte with NaN (valid positions get written by
    appends; a read past the valid length would surface as NaN)."""
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))


# -------------------------------------------------------------- append

def test_kv_append_bit_exact():
    say("case: kv_append bf16 [2,8,1024,128], 700 rows in 3 chunks at b=1")
    q, k, v = si.gqa_prompt(L=700, Hq=32, Hkv=8, D=128, seed=101)
    cache = cpk.KVCache(2, 8, 1024, 128, torch.bfloat16)
    poison(cache)
    ref = oracle.Cache(oracle.BF16, 2, 8, 1024, 128)
    kd, vd = k.cuda(), v.cuda()
    ks, vs = si.storage(k), si.storage(v)
    for past, rows in cpk.cpk_split_chunks(700, 256):
        cpk.cpk_kv_append(cache, 1, kd[past:past + rows], vd[past:past + rows], past)
        ref.append(1, ks[past:past + rows], vs[past:past + rows], past)
    torch.cuda.synchronize()
    assert int(cache.seqlens_k[1]) == 700 and int(cache.seqlens_k[0]) == 0
    gk = si.storage(cache.k[1, :, :700])
    gv = si.storage(cache.v[1, :, :700])
    assert np.array_equal(gk, ref.k[1, :, :700]) and np.array_equal(gv, ref.v[1, :, :700])
    # the other sequence was not touched (still the NaN poison)
    assert torch.isnan(cache.k[0]).all()


# ------------------------------------------------------ workload 1: fp32 demo

def test_fp32_demo_chunked_and_one_shot():
    say("case: fp32 demo L=1000 H=8 D=64 chunk 256, cap 1024")
    _, (qt, kt, vt) = si.demo_qkv()
    qs, ks, vs = (si.storage(x) for x in (qt, kt, vt))
    ref = oracle.prefill_one_shot(oracle.Cache(oracle.F32, 1, 8, 1024, 64), 0, qs, ks, vs)
    q, k, v = qt.cuda(), kt.cuda(), vt.cuda()
    c1 = cpk.KVCache(1, 8, 1024, 64, torch.float32)
    poison(c1)
    out_c, widths = cpk.prefill_chunked(c1, 0, q, k, v, 256, pad=False)
    assert widths == [256, 256, 256, 232]
    c2 = cpk.KVCache(1, 8, 1024, 64, torch.float32)
    cpk.cpk_kv_append(c2, 0, k, v, 0)
    out_1 = cpk.cpk_chunk_attention(q, c2, 0, 0)
    c3 = cpk.KVCache(1, 8, 1024, 64, torch.float32)
    out_p, widths_p = cpk.prefill_chunked(c3, 0, q, k, v, 256, pad=True)
    torch.cuda.synchronize()
    assert widths_p == [256, 256, 256, 256]
    check(out_c, ref, 1e-5, "chunked vs oracle")
    check(out_1, ref, 1e-5, "one-shot vs oracle")
    assert bitwise(out_c, out_1), "chunked != one-shot (bitwise)"
    assert bitwise(out_c, out_p), "padded != unpadded (bitwise)"
    assert int(c3.seqlens_k[0]) == 1000
    assert np.array_equal(si.storage(c1.k[0, :, :1000]), ks.transpose(1, 0, 2))


# ----------------------------------------------- GQA shapes, full compare

# narrow: the 64-column kernel (its latency-scheduled form wherever the launch
# reads a contiguous cache), wide: the 128-column kernel, general: the
# 64-column kernel's general form everywhere
KERNELS = {"narrow": 1, "wide": 2, "general": 3}


@pytest.mark.parametrize("dtype,Hq,Hkv,D,past,real,W,pad", [
    (torch.bfloat16, 32, 8, 128, 3584, 416, 512, True),    # workload 2's last chunk
    (torch.bfloat16, 32, 8, 128, 0, 512, 512, True),       # its first chunk
    (torch.float16, 8, 2, 64, 300, 77, 128, True),
    (torch.bfloat16, 12, 4, 128, 129, 200, 256, False),    # tiles straddle the new rows
    (torch.bfloat16, 16, 16, 128, 64, 1, 171, True),
])
def test_scheduled_form_bit_equal_to_general(dtype, Hq, Hkv, D, past, real, W, pad):
    """The latency-scheduled form of the 64-column kernel gives the general
    form's bits (same arithmetic in the same order): outputs, every cache
    byte written (padded rows included) and seqlens_k, for one fused prefill
    chunk after a cached prefix; both match the oracle."""
    dn = {torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    say(f"case: scheduled vs general {dn} heads {Hq}/{Hkv} D={D} past={past} real={real} W={W}")
    g = si.generator(610 + past + real)
    pre = [si.randn((past, Hkv, D), dn, g).cuda() for _ in range(2)]
    q, k, v = (si.randn((real, h, D), dn, g).cuda() for h in (Hq, Hkv, Hkv))
    res = []
    for kind in ("general", "narrow"):
        cache = cpk.KVCache(1, Hkv, past + W + 8, D, dtype)
        poison(cache)
        if past:
            cpk.cpk_kv_append(cache, 0, pre[0], pre[1], 0)
        with cpk.attention_kernel(KERNELS[kind]):
            out, width = cpk.cpk_prefill_chunk(q, k, v, cache, 0, past, W, pad=pad)
        torch.cuda.synchronize()
        res.append((out, width, cache))
    (o1, w1, c1), (o2, w2, c2) = res
    assert w1 == w2
    assert bitwise(o1, o2), "outputs differ"
    n = past + w1
    assert bitwise(c1.k[:, :, :n], c2.k[:, :, :n]) and bitwise(c1.v[:, :, :n], c2.v[:, :, :n])
    assert torch.equal(c1.seqlens_k, c2.seqlens_k)
    odt = ODT[dtype]
    kk = oracle.widen(si.storage(c1.k[0, :, :past + real]), odt)
    vv = oracle.widen(si.storage(c1.v[0, :, :past + real]), odt)
    qq = oracle.widen(si.storage(q), odt)
    lim = (past + np.arange(real)).astype(np.int32)
    ref = oracle.attention(qq, kk, vv, np.zeros(real, np.int32), lim, 1.0 / math.sqrt(D))
    check(o2, ref, TOL[dtype], "scheduled form vs oracle")


@pytest.mark.parametrize("kernel", ["narrow", "wide", "general"])
@pytest.mark.parametrize("dtype,Hq,Hkv,D,L,W", [
    (torch.bfloat16, 8, 2, 128, 700, 256),
    (torch.bfloat16, 16, 2, 64, 333, 128),
    (torch.bfloat16, 4, 4, 128, 300, 200),
    (torch.float16, 8, 2, 128, 450, 256),
    (torch.bfloat16, 24, 8, 128, 260, 100),
    (torch.bfloat16, 12, 4, 128, 290, 97),
    (torch.bfloat16, 32, 2, 64, 200, 64),
    (torch.float16, 16, 4, 64, 520, 128),
    (torch.bfloat16, 32, 4, 128, 400, 256),
])
def test_chunked_prefill_full_compare(kernel, dtype, Hq, Hkv, D, L, W):
    say(f"case: chunked prefill [{kernel}] {dtype} Hq={Hq} Hkv={Hkv} D={D} L={L} W={W}")
    with cpk.attention_kernel(KERNELS[kernel]):
        _chunked_prefill_full_compare(dtype, Hq, Hkv, D, L, W)


def _chunked_prefill_full_compare(dtype, Hq, Hkv, D, L, W):
    dn = {torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    q, k, v = si.gqa_prompt(L=L, Hq=Hq, Hkv=Hkv, D=D, dtype=dn, seed=7 + L)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    cap = L + W   # room for the padded tail chunk
    ref = oracle.prefill_one_shot(oracle.Cache(ODT[dtype], 1, Hkv, cap, D), 0, qs, ks, vs)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    c1 = cpk.KVCache(1, Hkv, cap, D, dtype)
    poison(c1)
    out_c, widths = cpk.prefill_chunked(c1, 0, qd, kd, vd, W, pad=True)
    c2 = cpk.KVCache(1, Hkv, cap, D, dtype)
    poison(c2)
    cpk.cpk_kv_append(c2, 0, kd, vd, 0)
    out_1 = cpk.cpk_chunk_attention(qd, c2, 0, 0)
    torch.cuda.synchronize()
    say(f"  widths {widths}")
    check(out_c, ref, TOL[dtype], "chunked vs oracle")
    check(out_1, ref, TOL[dtype], "one-shot vs oracle")
    same = bitwise(out_c, out_1)
    say(f"  chunked == one-shot bitwise: {same}")
    assert same
    assert np.array_equal(si.storage(c1.k[0, :, :L]), ks.transpose(1, 0, 2))
    assert np.array_equal(si.storage(c1.v[0, :, :L]), vs.transpose(1, 0, 2))


@pytest.mark.parametrize("kernel", ["narrow", "wide", "general"])
@pytest.mark.parametrize("dtype,Hq,Hkv,D,past,real,W", [
    (torch.bfloat16, 32, 8, 128, 512, 416, 512),
    (torch.bfloat16, 12, 4, 128, 77, 150, 512),
    (torch.float16, 8, 2, 64, 300, 1, 96),
    (torch.bfloat16, 16, 16, 128, 0, 200, 256),
])
def test_fused_append_matches_two_launches(kernel, dtype, Hq, Hkv, D, past, real, W):
    """cpk_prefill_chunk appends inside the attention kernel: output bits,
    every cache byte it writes (padded rows included) and seqlens_k equal
    the separate append (padded width) + attention launches."""
    say(f"case: fused append [{kernel}] {dtype} Hq={Hq} Hkv={Hkv} D={D} past={past} "
        f"real={real} W={W}")
    dn = {torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    q, k, v = si.gqa_prompt(L=past + real, Hq=Hq, Hkv=Hkv, D=D, dtype=dn, seed=900 + past)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    width = cpk.cpk_ladder_width(W, real)
    cap = past + width + 64
    with cpk.attention_kernel(KERNELS[kernel]):
        caches, outs = [], []
        for fused in (True, False):
            c = cpk.KVCache(1, Hkv, cap, D, dtype)
            poison(c)
            if past:
                cpk.cpk_kv_append(c, 0, kd[:past], vd[:past], 0)
            sl = slice(past, past + real)
            if fused:
                out, w = cpk.cpk_prefill_chunk(qd[sl], kd[sl], vd[sl], c, 0, past, W, pad=True)
                assert w == width
            else:
                cpk.cpk_kv_append(c, 0, kd[sl], vd[sl], past, rows=width)
                out = cpk.cpk_chunk_attention(qd[sl], c, 0, past, rows=width)
                cpk.cpk_rewind(c, 0, past + real)
            torch.cuda.synchronize()
            caches.append(c)
            outs.append(out)
    assert bitwise(outs[0], outs[1]), "fused output differs"
    n = past + width
    assert bitwise(caches[0].k[:, :, :n], caches[1].k[:, :, :n])
    assert bitwise(caches[0].v[:, :, :n], caches[1].v[:, :, :n])
    assert int(caches[0].seqlens_k[0]) == past + real == int(caches[1].seqlens_k[0])
    # padded rows repeat the last real row
    last = si.storage(k[past + real - 1])
    for i in range(past + real, n):
        assert np.array_equal(si.storage(caches[0].k[0, :, i]), last)
    # bytes past the padded width are untouched (still the NaN poison)
    assert torch.isnan(caches[0].k[:, :, n:].float()).all()
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    rows_idx = np.arange(past, past + real)
    ref = oracle_rows(qs, ks, vs, rows_idx, ODT[dtype])
    check(outs[0], ref, TOL[dtype], "fused vs oracle")


def _random_chunk_cases(n=40, seed=4242):
    """Seeded random shapes for a single padded (or unpadded) prefill chunk
    after a cached prefix: dtype, head dim, KV heads, GQA group (3 included),
    past length, chunk width, real rows, padding switch, kernel choice and
    spare capacity past the chunk."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        W = int(rng.choice([64, 128, 171, 256, 512]))
        cases.append(dict(i=i, dn=str(rng.choice(["bf16", "f16"])), D=int(rng.choice([64, 128])),
                          Hkv=int(rng.choice([1, 2, 4])), G=int(rng.choice([1, 2, 3, 4, 8])),
                          past=int(rng.integers(0, 700)), W=W, real=int(rng.integers(1, W + 1)),
                          pad=bool(rng.integers(2)),
                          kernel=str(rng.choice(["auto", "narrow", "wide", "general"])),
                          spare=int(rng.integers(0, 40))))
    return cases


@pytest.mark.parametrize("case", _random_chunk_cases(), ids=lambda c: f"r{c['i']}")
def test_random_prefill_chunk_vs_oracle(case):
    """cpk_prefill_chunk on seeded random shapes (every kernel choice, GQA
    groups 1-8 including 3, head dims 64 and 128, padded and unpadded, tight
    and loose capacity) against the oracle: the real rows' outputs within
    tolerance, the cache's valid rows byte for byte, seqlens_k, and no byte
    written past the issued width."""
    c = case
    Hq, Hkv, D, past, W, real = c["G"] * c["Hkv"], c["Hkv"], c["D"], c["past"], c["W"], c["real"]
    dtype = si.TORCH_DTYPE[c["dn"]]
    say(f"case r{c['i']}: {c['dn']} heads {Hq}/{Hkv} D={D} past={past} real={real} W={W} "
        f"pad={c['pad']} kernel={c['kernel']}")
    q, k, v = si.gqa_prompt(L=past + real, Hq=Hq, Hkv=Hkv, D=D, dtype=c["dn"], seed=5000 + c["i"])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    width = cpk.cpk_ladder_width(W, real) if c["pad"] else real
    cache = cpk.KVCache(1, Hkv, past + width + c["spare"], D, dtype)
    poison(cache)
    with cpk.attention_kernel({"auto": 0, **KERNELS}[c["kernel"]]):
        if past:
            cpk.cpk_kv_append(cache, 0, kd[:past], vd[:past], 0)
        out, w = cpk.cpk_prefill_chunk(qd[past:], kd[past:], vd[past:], cache, 0, past, W,
                                       pad=c["pad"])
        torch.cuda.synchronize()
    assert w == width
    assert int(cache.seqlens_k[0]) == past + real
    ks, vs = si.storage(k), si.storage(v)
    n = past + real
    assert np.array_equal(si.storage(cache.k[0, :, :n]), ks.transpose(1, 0, 2))
    assert np.array_equal(si.storage(cache.v[0, :, :n]), vs.transpose(1, 0, 2))
    assert torch.isnan(cache.k[:, :, past + width:].float()).all()
    ref = oracle_rows(si.storage(q), ks, vs, np.arange(past, n), ODT[dtype])
    check(out, ref, TOL[dtype], "random chunk vs oracle")


def _random_varlen_cases(n=16, seed=777):
    """Seeded random packed steps: 1-6 sequences, each a decode row or a
    prompt chunk of 2-260 rows after 0-1500 cached positions, in random
    slots of a larger cache and a random pack order."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_seqs = int(rng.integers(1, 7))
        seqs = [(int(rng.integers(0, 1500)), 1 if rng.integers(2) else int(rng.integers(2, 261)))
                for _ in range(n_seqs)]
        batch = n_seqs + int(rng.integers(0, 3))
        cases.append(dict(i=i, dn=str(rng.choice(["bf16", "f16"])), D=int(rng.choice([64, 128])),
                          Hkv=int(rng.choice([1, 2, 4])), G=int(rng.choice([1, 2, 3, 4, 8])),
                          kernel=str(rng.choice(["auto", "narrow", "wide", "general"])),
                          seqs=seqs, batch=batch,
                          slots=[int(x) for x in rng.permutation(batch)[:n_seqs]]))
    return cases


@pytest.mark.parametrize("case", _random_varlen_cases(), ids=lambda c: f"v{c['i']}")
def test_random_varlen_step_vs_oracle(case):
    """cpk_varlen_step on seeded random packs (decode rows and prompt chunks
    mixed, random slots and order, GQA groups 1-8 including 3, whose one-row
    sequences take the prompt path) against the oracle over the cached
    prefix and the new rows: every output row within tolerance, the new K/V
    rows in the cache byte for byte, seqlens_k of every slot."""
    c = case
    Hkv, D = c["Hkv"], c["D"]
    Hq = c["G"] * Hkv
    dtype = si.TORCH_DTYPE[c["dn"]]
    say(f"case v{c['i']}: {c['dn']} heads {Hq}/{Hkv} D={D} kernel={c['kernel']} "
        f"seqs (past, rows) {c['seqs']} slots {c['slots']}")
    cap = max(p + r for p, r in c["seqs"]) + 8
    cache = cpk.KVCache(c["batch"], Hkv, cap, D, dtype)
    si.fill_seeded(cache.k, 600 + c["i"])
    si.fill_seeded(cache.v, 700 + c["i"])
    g = si.generator(800 + c["i"])
    new = [tuple(si.randn((r, h, D), c["dn"], g).cuda() for h in (Hq, Hkv, Hkv))
           for _, r in c["seqs"]]
    prefix = [(si.storage(cache.k[sl, :, :p]), si.storage(cache.v[sl, :, :p]))
              for sl, (p, _) in zip(c["slots"], c["seqs"])]
    for sl, (p, _) in zip(c["slots"], c["seqs"]):
        cache.lens[sl] = p
    cu = [0]
    for _, r in c["seqs"]:
        cu.append(cu[-1] + r)
    q = torch.cat([x[0] for x in new])
    kn = torch.cat([x[1] for x in new])
    vn = torch.cat([x[2] for x in new])
    with cpk.attention_kernel({"auto": 0, **KERNELS}[c["kernel"]]):
        out = cpk.cpk_varlen_step(q, kn, vn, cache, c["slots"], cu, [p for p, _ in c["seqs"]])
        torch.cuda.synchronize()
    odt = ODT[dtype]
    for j, (sl, (p, r)) in enumerate(zip(c["slots"], c["seqs"])):
        assert int(cache.seqlens_k[sl]) == p + r, f"seq {j}: seqlens_k"
        ks_new = si.storage(new[j][1]).transpose(1, 0, 2)
        vs_new = si.storage(new[j][2]).transpose(1, 0, 2)
        assert np.array_equal(si.storage(cache.k[sl, :, p:p + r]), ks_new), f"seq {j}: K rows"
        assert np.array_equal(si.storage(cache.v[sl, :, p:p + r]), vs_new), f"seq {j}: V rows"
        kk = oracle.widen(np.ascontiguousarray(np.concatenate([prefix[j][0], ks_new], axis=1)), odt)
        vv = oracle.widen(np.ascontiguousarray(np.concatenate([prefix[j][1], vs_new], axis=1)), odt)
        qq = oracle.widen(si.storage(new[j][0]), odt)
        lim = (p + np.arange(r)).astype(np.int32)
        ref = oracle.attention(qq, kk, vv, np.zeros(r, np.int32), lim, 1.0 / math.sqrt(D))
        check(out[cu[j]:cu[j + 1]], ref, TOL[dtype], f"seq {j} (past {p}, rows {r}) vs oracle")


@pytest.mark.parametrize("case", _random_varlen_cases(n=8, seed=4711), ids=lambda c: f"p{c['i']}")
def test_random_paged_step_vs_oracle(case):
    """The random packed steps over a paged cache (256-position blocks handed
    out in a seeded random order): a first packed step writes every
    sequence's cached prefix as a prompt chunk, the second is the random
    pack; both steps' outputs against the oracle, and the blocks gathered
    back through the table equal the prefix and new rows byte for byte."""
    c = case
    Hkv, D = c["Hkv"], c["D"]
    Hq = c["G"] * Hkv
    dtype = si.TORCH_DTYPE[c["dn"]]
    odt = ODT[dtype]
    say(f"case p{c['i']}: paged {c['dn']} heads {Hq}/{Hkv} D={D} kernel={c['kernel']} "
        f"seqs {c['seqs']} slots {c['slots']}")
    bs = 256
    maxb = (max(p + r for p, r in c["seqs"]) + bs - 1) // bs
    nblk = c["batch"] * maxb + 3
    paged = cpk.PagedKVCache(c["batch"], Hkv, nblk, bs, maxb, D, dtype)
    rng = np.random.default_rng(1000 + c["i"])
    perm = rng.permutation(nblk)[:c["batch"] * maxb].reshape(c["batch"], maxb)
    paged.block_table.copy_(torch.from_numpy(perm.astype(np.int32)))
    g = si.generator(1100 + c["i"])
    pre = [tuple(si.randn((p, h, D), c["dn"], g).cuda() for h in (Hq, Hkv, Hkv))
           for p, _ in c["seqs"]]
    new = [tuple(si.randn((r, h, D), c["dn"], g).cuda() for h in (Hq, Hkv, Hkv))
           for _, r in c["seqs"]]

    def step(parts, pasts, rows):
        use = [j for j in range(len(parts)) if rows[j] > 0]
        cu = [0]
        for j in use:
            cu.append(cu[-1] + rows[j])
        q = torch.cat([parts[j][0] for j in use])
        kn = torch.cat([parts[j][1] for j in use])
        vn = torch.cat([parts[j][2] for j in use])
        out = cpk.cpk_paged_varlen_step(q, kn, vn, paged, [c["slots"][j] for j in use], cu,
                                        [pasts[j] for j in use])
        torch.cuda.synchronize()
        return {j: out[cu[i]:cu[i + 1]] for i, j in enumerate(use)}, use

    def ref_rows(qx, kx, vx, past):
        r = qx.shape[0]
        kk = oracle.widen(np.ascontiguousarray(kx.transpose(1, 0, 2)), odt)
        vv = oracle.widen(np.ascontiguousarray(vx.transpose(1, 0, 2)), odt)
        lim = (past + np.arange(r)).astype(np.int32)
        return oracle.attention(oracle.widen(qx, odt), kk, vv, np.zeros(r, np.int32), lim,
                                1.0 / math.sqrt(D))

    with cpk.attention_kernel({"auto": 0, **KERNELS}[c["kernel"]]):
        pasts0 = [0] * len(c["seqs"])
        out0, use0 = step(pre, pasts0, [p for p, _ in c["seqs"]])
        out1, _ = step(new, [p for p, _ in c["seqs"]], [r for _, r in c["seqs"]])
    for j in use0:
        ps = [si.storage(x) for x in pre[j]]
        check(out0[j], ref_rows(ps[0], ps[1], ps[2], 0), TOL[dtype], f"seq {j} prefix step")
    for j, (sl, (p, r)) in enumerate(zip(c["slots"], c["seqs"])):
        assert int(paged.seqlens_k[sl]) == p + r
        ks = np.concatenate([si.storage(pre[j][1]), si.storage(new[j][1])])
        vs = np.concatenate([si.storage(pre[j][2]), si.storage(new[j][2])])
        gk, gv = paged.gather(sl, p + r)
        assert np.array_equal(si.storage(gk), ks.transpose(1, 0, 2)), f"seq {j}: K blocks"
        assert np.array_equal(si.storage(gv), vs.transpose(1, 0, 2)), f"seq {j}: V blocks"
        ref = ref_rows(si.storage(new[j][0]), ks, vs, p)
        check(out1[j], ref, TOL[dtype], f"seq {j} (past {p}, rows {r}) vs oracle")


@pytest.mark.parametrize("kernel", ["narrow", "wide"])
def test_prefix_reuse(kernel):
    """Prompt-prefix reuse: prompt A = prefix + suffix A is prefilled in slot
    0; prompt B = the same prefix + suffix B reuses A's prefix (copied to
    slot 1) and prefills only its suffix.  B's suffix rows and slot 1's
    cache equal a full chunked prefill of B in slot 2 bit for bit, and the
    oracle within tolerance."""
    say(f"case: prefix reuse [{kernel}]: prefix 700, suffixes 400 / 333, W=256")
    Hq, Hkv, D, W, P = 16, 4, 128, 256, 700
    pre = si.gqa_prompt(L=P, Hq=Hq, Hkv=Hkv, D=D, seed=560)
    sa = si.gqa_prompt(L=400, Hq=Hq, Hkv=Hkv, D=D, seed=561)
    sb = si.gqa_prompt(L=333, Hq=Hq, Hkv=Hkv, D=D, seed=562)
    A = [torch.cat([x, y]).cuda() for x, y in zip(pre, sa)]
    Bt = [torch.cat([x, y]) for x, y in zip(pre, sb)]
    B = [x.cuda() for x in Bt]
    cache = cpk.KVCache(3, Hkv, 2048, D, torch.bfloat16)
    poison(cache)
    with cpk.attention_kernel(KERNELS[kernel]):
        cpk.prefill_chunked(cache, 0, *A, W)
        out_r, _ = cpk.prefill_with_prefix(cache, 1, 0, P, B[0][P:], B[1][P:], B[2][P:], W)
        out_f, _ = cpk.prefill_chunked(cache, 2, *B, W)
        torch.cuda.synchronize()
    n = P + 333
    assert int(cache.seqlens_k[1]) == n == int(cache.seqlens_k[2])
    assert bitwise(out_r, out_f[P:]), "reused-prefix suffix differs from the full prefill"
    assert bitwise(cache.k[1, :, :n], cache.k[2, :, :n])
    assert bitwise(cache.v[1, :, :n], cache.v[2, :, :n])
    qs, ks, vs = (si.storage(x) for x in Bt)
    rows = np.arange(P, n)
    ref = oracle_rows(qs, ks, vs, rows, oracle.BF16)
    check(out_r, ref, 2e-2, "suffix vs oracle")


# ---------------------------------------------- workload 2: GQA bf16 W=512

def test_workload2_gqa_bf16_full_size():
    say("case: workload 2 L=4000 Hq=32 Hkv=8 D=128 cap 8192 W=512 (sampled rows)")
    q, k, v = si.gqa_prompt()
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    chunks = cpk.cpk_split_chunks(4000, 512)
    rows = sample_rows(4000, chunks)
    ref = oracle_rows(qs, ks, vs, rows, oracle.BF16)
    one = cpk.KVCache(1, 8, 8192, 128, torch.bfloat16)
    cpk.cpk_kv_append(one, 0, kd, vd, 0)
    res = {}
    for kind in ("auto", "narrow", "wide"):
        with cpk.attention_kernel({"auto": 0, **KERNELS}[kind]):
            cache = cpk.KVCache(1, 8, 8192, 128, torch.bfloat16)
            poison(cache)
            out_c, widths = cpk.prefill_chunked(cache, 0, qd, kd, vd, 512, pad=True)
            out_1 = cpk.cpk_chunk_attention(qd, one, 0, 0)
            torch.cuda.synchronize()
        assert widths == [512] * 8    # 7 x 512 + 416 padded to 512: eight M=512 forwards
        check(out_c[torch.from_numpy(rows).cuda()], ref, 2e-2,
              f"[{kind}] chunked vs oracle ({len(rows)} rows)")
        check(out_1[torch.from_numpy(rows).cuda()], ref, 2e-2,
              f"[{kind}] one-shot vs oracle ({len(rows)} rows)")
        res[kind] = (out_c, out_1)
    for kind in ("narrow", "wide"):
        assert bitwise(*res[kind]), f"[{kind}] chunked != one-shot"
    # the automatic choice: 512-row chunks fill 128 wide workgroups (fewer
    # than the 256 CUs) and take the narrow kernel; the 4000-row pass fills
    # 1,000 but holds 8.0 x 10^6 visible pairs per head, below the wide
    # kernel's 24 x 2^20, and takes the narrow kernel too
    assert bitwise(res["auto"][0], res["narrow"][0])
    assert bitwise(res["auto"][1], res["narrow"][1])
    assert int(cache.seqlens_k[0]) == 4000
    assert np.array_equal(si.storage(cache.k[0, :, :4000]), ks.transpose(1, 0, 2))
    assert np.array_equal(si.storage(cache.v[0, :, :4000]), vs.transpose(1, 0, 2))
    # the prompt again on the full cache with no length reset in between: the
    # first chunk (past 0) records the slot's new length itself, and the
    # second pass gives the first pass's bits
    again = torch.empty_like(qd)
    for i, (past, n) in enumerate(chunks):
        sl = slice(past, past + n)
        cpk.cpk_prefill_chunk(qd[sl], kd[sl], vd[sl], cache, 0, past, 512, pad=True, out=again[sl])
        if i == 0:
            torch.cuda.synchronize()
            assert int(cache.seqlens_k[0]) == n
    torch.cuda.synchronize()
    assert bitwise(again, res["auto"][0]), "second pass without a reset != first pass"
    assert int(cache.seqlens_k[0]) == 4000


# ------------------------------------------------- workload 3: padding ladder

@pytest.mark.parametrize("past,rows,expect", [
    (4096, 4096, "wide"),     # 1,024 wide workgroups, 25.2 x 10^6 pairs per head
    (0, 4096, "narrow"),      # 1,024 wide workgroups but 8.4 x 10^6 pairs
    (12288, 992, "narrow"),   # 12.7 x 10^6 pairs, but 248 wide workgroups
])
def test_auto_kernel_choice(past, rows, expect):
    """The automatic kernel choice: the 128-column kernel only for launches
    that fill the CUs with its workgroups and hold at least 24 x 2^20
    visible pairs per query head; the output under CPK_ATTN_AUTO has the
    chosen kernel's bits."""
    say(f"case: automatic kernel choice, past {past}, rows {rows}: {expect}")
    Hq, Hkv, D = 32, 8, 128
    cache = cpk.KVCache(1, Hkv, past + rows, D, torch.bfloat16)
    si.fill_seeded(cache.k, 41)
    si.fill_seeded(cache.v, 42)
    q = si.randn((rows, Hq, D), "bf16", si.generator(43)).cuda()
    res = {}
    for kind in ("auto", "narrow", "wide"):
        with cpk.attention_kernel({"auto": 0, **KERNELS}[kind]):
            res[kind] = cpk.cpk_chunk_attention(q, cache, 0, past)
    torch.cuda.synchronize()
    other = "narrow" if expect == "wide" else "wide"
    assert bitwise(res["auto"], res[expect])
    assert not bitwise(res["auto"], res[other]), "the two kernels round differently"


def test_workload3_ladder_twice_on_dirty_cache():
    lengths = si.ladder_prompt_lengths()
    say(f"case: workload 3 ladder prompts {lengths}, each twice, NaN-poisoned tail")
    cache = cpk.KVCache(1, 8, 8192, 128, torch.bfloat16)
    poison(cache)
    plain = cpk.KVCache(1, 8, 8192, 128, torch.bfloat16)
    for i, L in enumerate(lengths):
        q, k, v = si.gqa_prompt(L=L, seed=200 + i)
        qs, ks, vs = (si.storage(x) for x in (q, k, v))
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        outs = []
        for rep in range(2):
            if cache.lens[0]:
                cpk.cpk_rewind(cache, 0, 0)
            out, widths = cpk.prefill_chunked(cache, 0, qd, kd, vd, 512, pad=True)
            outs.append(out)
        if plain.lens[0]:
            cpk.cpk_rewind(plain, 0, 0)
        out_np, _ = cpk.prefill_chunked(plain, 0, qd, kd, vd, 512, pad=False)
        torch.cuda.synchronize()
        tail = L % 512
        exp_tail = cpk.cpk_ladder_width(512, tail) if tail else 512
        assert widths[-1] == exp_tail
        if L == 1137:
            assert widths == [512, 512, 171]
        if L == 1200:
            assert widths == [512, 512, 342]
        assert bitwise(outs[0], outs[1]), "second run differs"
        assert bitwise(outs[0], out_np), "padded != unpadded"
        assert int(cache.seqlens_k[0]) == L
        assert np.array_equal(si.storage(cache.k[0, :, :L]), ks.transpose(1, 0, 2))
        rows = sample_rows(L, cpk.cpk_split_chunks(L, 512), every=97)
        ref = oracle_rows(qs, ks, vs, rows, oracle.BF16)
        check(outs[0][torch.from_numpy(rows).cuda()], ref, 2e-2, f"L={L} widths={widths}")


@pytest.mark.parametrize("kernel", ["narrow", "wide", "general"])
def test_rows_equal_capacity_and_single_row_chunks(kernel):
    say(f"case: [{kernel}] W=1 chunks and a prompt filling the cache exactly")
    with cpk.attention_kernel(KERNELS[kernel]):
        _rows_equal_capacity_and_single_row_chunks()


def _rows_equal_capacity_and_single_row_chunks():
    q, k, v = si.gqa_prompt(L=40, Hq=8, Hkv=2, D=128, seed=300)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    ref = oracle.prefill_one_shot(oracle.Cache(oracle.BF16, 1, 2, 40, 128), 0, qs, ks, vs)
    c = cpk.KVCache(1, 2, 40, 128, torch.bfloat16)
    out, widths = cpk.prefill_chunked(c, 0, q.cuda(), k.cuda(), v.cuda(), 1, pad=True)
    c2 = cpk.KVCache(1, 2, 40, 128, torch.bfloat16)
    out2, widths2 = cpk.prefill_chunked(c2, 0, q.cuda(), k.cuda(), v.cuda(), 40, pad=True)
    torch.cuda.synchronize()
    assert widths == [1] * 40 and widths2 == [40]
    check(out, ref, 2e-2, "W=1")
    check(out2, ref, 2e-2, "W=L=capacity")
    assert bitwise(out, out2)
    with pytest.raises(cpk.CpkError):
        cpk.cpk_kv_append(c2, 0, k[:1].cuda(), v[:1].cuda(), 40)


# -------------------------------------------------- workload 4: rolling fp16

def test_rolling_small_with_left_pad_full_compare():
    L, C, c, H, D = 1000, 512, 128, 4, 128
    say(f"case: rolling fp16 L={L} C={C} c={c} H={H} (24 left-pad rows)")
    q, k, v = si.rolling_inputs(L=L, H=H, D=D, seed=401)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    ref, n_left, rk, rv, masks = oracle.roll_prefill(qs, ks, vs, C, c, oracle.F16)
    assert n_left == 24
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out_a, nl, gk, gv = cpk.roll_prefill(qd, kd, vd, C, c)
    mk = [torch.from_numpy(m.astype(np.float16)).cuda() for m in masks]
    out_m, _, gk2, gv2 = cpk.roll_prefill(qd, kd, vd, C, c, masks=mk)
    torch.cuda.synchronize()
    assert nl == 24
    assert np.array_equal(si.storage(gk), rk) and np.array_equal(si.storage(gv), rv)
    assert np.array_equal(si.storage(gk2), rk)
    check(out_a[n_left:], ref[n_left:], TOL[torch.float16], "computed mask vs oracle (real rows)")
    check(out_m[n_left:], ref[n_left:], TOL[torch.float16], "explicit mask vs oracle (real rows)")
    assert bitwise(out_a[n_left:], out_m[n_left:]), "explicit != computed mask"


def _random_rolling_cases(n=10, seed=991):
    """Seeded random rolling schedules: length, window C, chunk c (c <= C,
    so ring starts wrap mid-tile and C need not be a multiple of the key
    tile), heads, head dim, dtype, GQA group."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        C = int(rng.integers(64, 700))
        c = int(rng.integers(16, C + 1))
        cases.append(dict(i=i, C=C, c=c, L=int(rng.integers(c, 4 * C + 1)),
                          Hkv=int(rng.choice([1, 2, 4])), G=int(rng.choice([1, 2, 4])),
                          D=int(rng.choice([64, 128])), dn=str(rng.choice(["f16", "bf16"]))))
    return cases


@pytest.mark.parametrize("case", _random_rolling_cases(), ids=lambda c: f"roll{c['i']}")
def test_random_rolling_vs_oracle(case):
    """Seeded random rolling schedules through roll_prefill and ring_prefill
    (deferred merges wherever the key range splits) against the oracle's
    literal rolling prefill: real rows within tolerance with computed
    visibility and with the explicit masks, both schedules bit-equal, the
    final caches byte for byte."""
    c_ = case
    C, c, L, Hkv, D = c_["C"], c_["c"], c_["L"], c_["Hkv"], c_["D"]
    Hq = c_["G"] * Hkv
    dtype = si.TORCH_DTYPE[c_["dn"]]
    odt = ODT[dtype]
    say(f"case roll{c_['i']}: {c_['dn']} L={L} C={C} c={c} heads {Hq}/{Hkv} D={D}")
    g = si.generator(900 + c_["i"])
    q = si.randn((L, Hq, D), c_["dn"], g)
    k = si.randn((L, Hkv, D), c_["dn"], g)
    v = si.randn((L, Hkv, D), c_["dn"], g)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    ref, n_left, rk, rv, masks = oracle.roll_prefill(qs, ks, vs, C, c, odt)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mk = [torch.from_numpy(m).to(dtype).cuda() for m in masks]
    for m in (None, mk):
        tag = "explicit mask" if m is not None else "computed visibility"
        out_l, nl, lk, lv = cpk.roll_prefill(qd, kd, vd, C, c, masks=m)
        out_r, nl2, gk, gv, st = cpk.ring_prefill(qd, kd, vd, C, c, masks=m)
        torch.cuda.synchronize()
        assert nl == nl2 == n_left
        assert np.array_equal(si.storage(lk), rk) and np.array_equal(si.storage(lv), rv)
        kview, vview = cpk.cpk_ring_view(gk.unsqueeze(0), gv.unsqueeze(0), st)
        assert np.array_equal(si.storage(kview[0]), rk) and np.array_equal(si.storage(vview[0]), rv)
        assert bitwise(out_l, out_r), f"{tag}: ring != literal shift"
        check(out_l[n_left:], ref[n_left:], TOL[dtype], f"{tag} vs oracle (real rows)")


def test_rolling_split_vs_unsplit():
    """The rolling attention with a workspace (key range split over 4 parts
    of one 128-key tile each, merged in part order) and without one: both
    against the oracle, explicit == computed mask bitwise in each form, and
    the two forms within rounding of each other."""
    L, C, c, H, D = 1000, 512, 128, 4, 128
    assert cpk.cpk_roll_workspace_size(H, H, C, c, D, torch.float16) == 4 * c * H * (D + 4) * 4
    say(f"case: rolling fp16 split vs unsplit L={L} C={C} c={c} H={H}")
    q, k, v = si.rolling_inputs(L=L, H=H, D=D, seed=402)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    ref, n_left, _, _, masks = oracle.roll_prefill(qs, ks, vs, C, c, oracle.F16)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mk = [torch.from_numpy(m.astype(np.float16)).cuda() for m in masks]
    outs = {}
    for split in (True, False):
        out_a, _, _, _ = cpk.roll_prefill(qd, kd, vd, C, c, split=split)
        out_m, _, _, _ = cpk.roll_prefill(qd, kd, vd, C, c, masks=mk, split=split)
        torch.cuda.synchronize()
        check(out_a[n_left:], ref[n_left:], TOL[torch.float16], f"split={split} vs oracle")
        assert bitwise(out_a[n_left:], out_m[n_left:]), f"split={split}: explicit != computed"
        outs[split] = out_a
    d = float((outs[True][n_left:].float() - outs[False][n_left:].float()).abs().max())
    say(f"  split vs unsplit: max-abs {d:.3e}")
    assert d <= 4e-3


def test_workload4_rolling_full_size():
    L, C, c, H, D = 4096, 2048, 256, 16, 128
    say(f"case: workload 4 rolling fp16 L={L} C={C} c={c} H={H} (sampled rows)")
    q, k, v = si.rolling_inputs()
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, nl, gk, gv = cpk.roll_prefill(qd, kd, vd, C, c)
    masks = [torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C).astype(np.float16)).cuda()
             for j in range(L // c)]
    out_m, _, _, _ = cpk.roll_prefill(qd, kd, vd, C, c, masks=masks)
    torch.cuda.synchronize()
    assert nl == 0
    # final cache: the last C positions, right-aligned
    assert np.array_equal(si.storage(gk), ks[L - C:].transpose(1, 0, 2))
    assert np.array_equal(si.storage(gv), vs[L - C:].transpose(1, 0, 2))
    assert bitwise(out, out_m), "explicit != computed mask"
    rows = np.array(sorted(set(range(0, L, 37)) | set(range(L - 8, L)) | {255, 256, 2047, 2048, 2303}))
    qq = oracle.widen(np.ascontiguousarray(qs[rows]), oracle.F16)
    kk = oracle.widen(np.ascontiguousarray(ks.transpose(1, 0, 2)), oracle.F16)
    vv = oracle.widen(np.ascontiguousarray(vs.transpose(1, 0, 2)), oracle.F16)
    lo = np.maximum(0, (rows // c + 1) * c - C).astype(np.int32)
    ref = oracle.attention(qq, kk, vv, lo, rows.astype(np.int32), 1.0 / math.sqrt(D))
    check(out[torch.from_numpy(rows).cuda()], ref, TOL[torch.float16], f"sliding window ({len(rows)} rows)")


@pytest.mark.parametrize("L,C,c,H,D", [
    (1000, 512, 128, 4, 128),    # 24 left-pad rows, start walks 0, 128, 256, 384
    (1000, 300, 96, 2, 64),      # C not a multiple of the key tile, start wraps mid-tile
    (700, 256, 256, 3, 128),     # c == C: every append overwrites the whole ring
])
def test_ring_matches_literal_shift(L, C, c, H, D):
    """The ring-buffer rolling cache: after every chunk its logical view
    equals the literal shift cat(old, chunk)[c:] byte for byte, and ring
    attention equals rolling attention over the literal cache bit for bit
    (both mask forms, split and unsplit), and the oracle within tolerance."""
    say(f"case: ring vs literal shift fp16 L={L} C={C} c={c} H={H} D={D}")
    q, k, v = si.rolling_inputs(L=L, H=H, D=D, seed=410 + C)
    qs, ks, vs = (si.storage(x) for x in (q, k, v))
    ref, n_left, rk, rv, masks = oracle.roll_prefill(qs, ks, vs, C, c, oracle.F16)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mk = [torch.from_numpy(m.astype(np.float16)).cuda() for m in masks]
    # per chunk: literal double buffer against the ring and its view
    z = lambda x: torch.cat([torch.zeros((n_left,) + tuple(x.shape[1:]), dtype=x.dtype,
                                         device=x.device), x])
    qp, kp, vp = z(qd), z(kd), z(vd)
    bufs = [torch.zeros((1, H, C, D), dtype=torch.float16, device="cuda") for _ in range(4)]
    kr = torch.zeros((1, H, C, D), dtype=torch.float16, device="cuda")
    vr = torch.zeros_like(kr)
    start, cur = 0, 0
    for j in range(qp.shape[0] // c):
        sl = slice(j * c, (j + 1) * c)
        ko, vo = bufs[2 * cur], bufs[2 * cur + 1]
        kn, vn = bufs[2 * (1 - cur)], bufs[2 * (1 - cur) + 1]
        cpk.cpk_roll_append(ko, vo, kp[sl].unsqueeze(0), vp[sl].unsqueeze(0), kn, vn)
        cur = 1 - cur
        start = cpk.cpk_ring_append(kp[sl].unsqueeze(0), vp[sl].unsqueeze(0), kr, vr, start)
        assert start == ((j + 1) * c) % C
        kview, vview = cpk.cpk_ring_view(kr, vr, start)
        torch.cuda.synchronize()
        assert bitwise(kview, kn) and bitwise(vview, vn), f"chunk {j}: ring view != literal shift"
        for split in (True, False):
            for m in (None, mk[j]):
                lit = cpk.cpk_roll_attention(qp[sl], kn[0], vn[0], (j + 1) * c, n_left, mask=m,
                                             split=split)
                rng = cpk.cpk_ring_attention(qp[sl], kr[0], vr[0], (j + 1) * c, n_left, start,
                                             mask=m, split=split)
                torch.cuda.synchronize()
                assert bitwise(lit, rng), f"chunk {j} split={split} mask={m is not None}"
    out_r, nl, gk, gv, st = cpk.ring_prefill(qd, kd, vd, C, c)
    torch.cuda.synchronize()
    assert nl == n_left and st == start
    kview, vview = cpk.cpk_ring_view(gk.unsqueeze(0), gv.unsqueeze(0), st)
    assert np.array_equal(si.storage(kview[0]), rk) and np.array_equal(si.storage(vview[0]), rv)
    check(out_r[n_left:], ref[n_left:], TOL[torch.float16], "ring prefill vs oracle (real rows)")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("C,c,Hq,Hkv,D", [
    (512, 128, 4, 4, 128),       # start walks 0, 128, 256, 384 and wraps
    (300, 96, 4, 2, 64),         # C not a multiple of the key tile, GQA
    (256, 256, 2, 2, 128),       # c == C: the chunk replaces the whole ring
])
def test_ring_step_fused_matches_two_calls(dtype, C, c, Hq, Hkv, D):
    """cpk_ring_step (the append fused into the attention launch) equals
    cpk_ring_append followed by cpk_ring_attention bit for bit: the output
    of every chunk and both rings after it, split and unsplit, with the
    computed visibility and with the explicit mask."""
    say(f"case: fused ring step {dtype} C={C} c={c} heads {Hq}/{Hkv} D={D}")
    tdt = si.TORCH_DTYPE[dtype]
    g = si.generator(470 + C)
    n = 5
    q = si.randn((n * c, Hq, D), dtype, g).cuda()
    k = si.randn((n * c, Hkv, D), dtype, g).cuda()
    v = si.randn((n * c, Hkv, D), dtype, g).cuda()
    L = n * c
    for split in (True, False):
        for explicit in (False, True):
            ka = torch.zeros((1, Hkv, C, D), dtype=tdt, device="cuda")
            va = torch.zeros_like(ka)
            kb, vb = ka.clone(), va.clone()
            sa = sb = 0
            for j in range(n):
                sl = slice(j * c, (j + 1) * c)
                m = None
                if explicit:
                    m = torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C)).to(tdt).cuda()
                sa = cpk.cpk_ring_append(k[sl].unsqueeze(0), v[sl].unsqueeze(0), ka, va, sa)
                ref = cpk.cpk_ring_attention(q[sl], ka[0], va[0], (j + 1) * c, 0, sa, mask=m,
                                             split=split)
                got, sb = cpk.cpk_ring_step(q[sl], k[sl], v[sl], kb[0], vb[0], (j + 1) * c, 0,
                                            sb, mask=m, split=split)
                torch.cuda.synchronize()
                assert sb == sa
                tag = f"chunk {j} split={split} mask={explicit}"
                assert bitwise(got, ref), f"{tag}: output differs"
                assert bitwise(kb, ka) and bitwise(vb, va), f"{tag}: rings differ"


@pytest.mark.parametrize("kernel", ["narrow", "general"])
@pytest.mark.parametrize("dtype,C,c,Hq,Hkv,D", [
    ("f16", 512, 128, 4, 4, 128),     # 4 parts of 1 tile; start walks and wraps
    ("bf16", 300, 96, 4, 2, 64),      # 3 parts, tiles that wrap the ring mid-tile, GQA
    ("f16", 2048, 256, 16, 16, 128),  # the rolling workload's shapes: 4 parts of 4 tiles
])
def test_ring_step_deferred_bit_equal(kernel, dtype, C, c, Hq, Hkv, D):
    """A chain of deferred ring steps (each chunk's key-range parts merged
    by the next chunk's launch, the last by the flush; the scheduled form
    merges inside its launch, the general form with a combine launch ahead
    of it) gives cpk_ring_step's bits: the output of every chunk and both
    rings, with computed visibility and with the explicit mask."""
    say(f"case: deferred ring step {kernel} {dtype} C={C} c={c} heads {Hq}/{Hkv} D={D}")
    tdt = si.TORCH_DTYPE[dtype]
    g = si.generator(520 + C)
    n = 5
    q = si.randn((n * c, Hq, D), dtype, g).cuda()
    k = si.randn((n * c, Hkv, D), dtype, g).cuda()
    v = si.randn((n * c, Hkv, D), dtype, g).cuda()
    L = n * c
    nbytes = cpk.cpk_roll_workspace_size(Hq, Hkv, C, c, D, tdt)
    assert nbytes > 0, "the case must split the key range"
    wss = [torch.full((nbytes // 4 + 4,), float("nan"), device="cuda") for _ in range(2)]
    with cpk.attention_kernel(KERNELS[kernel]):
        for explicit in (False, True):
            masks = [torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C)).to(tdt).cuda()
                     if explicit else None for j in range(n)]
            res = []
            for deferred in (False, True):
                kr = torch.zeros((1, Hkv, C, D), dtype=tdt, device="cuda")
                vr = torch.zeros_like(kr)
                out = torch.full((L, Hq, D), float("nan"), dtype=tdt, device="cuda")
                start, pending = 0, None
                for j in range(n):
                    sl = slice(j * c, (j + 1) * c)
                    if deferred:
                        pending, start = cpk.cpk_ring_step_deferred(
                            q[sl], k[sl], v[sl], kr[0], vr[0], (j + 1) * c, 0, start,
                            wss[j % 2], prev=pending, mask=masks[j], out=out[sl])
                    else:
                        _, start = cpk.cpk_ring_step(q[sl], k[sl], v[sl], kr[0], vr[0],
                                                     (j + 1) * c, 0, start, mask=masks[j],
                                                     out=out[sl])
                if pending is not None:
                    cpk.cpk_roll_flush(pending)
                torch.cuda.synchronize()
                res.append((out, kr, vr, start))
            (oa, ka, va, sa), (ob, kb, vb, sb) = res
            tag = f"mask={explicit}"
            assert sa == sb
            assert bitwise(oa, ob), f"{tag}: outputs differ"
            assert bitwise(ka, kb) and bitwise(va, vb), f"{tag}: rings differ"


@pytest.mark.parametrize("kernel", ["narrow", "general"])
@pytest.mark.parametrize("dtype,C,c,Hq,Hkv,D", [
    ("f16", 512, 128, 4, 4, 128),     # 4 parts of 1 tile
    ("bf16", 300, 96, 4, 2, 64),      # 3 parts, GQA, C not a multiple of the key tile
])
def test_roll_attention_deferred_bit_equal(kernel, dtype, C, c, Hq, Hkv, D):
    """The literal-shift schedule with each chunk's split merged by the next
    chunk's attention launch (cpk_roll_attention_deferred, the last chunk by
    cpk_roll_flush) gives cpk_roll_attention's bits for every chunk, with
    computed visibility and with the explicit mask."""
    say(f"case: deferred roll attention {kernel} {dtype} C={C} c={c} heads {Hq}/{Hkv} D={D}")
    tdt = si.TORCH_DTYPE[dtype]
    g = si.generator(560 + C)
    n = 5
    q = si.randn((n * c, Hq, D), dtype, g).cuda()
    k = si.randn((n * c, Hkv, D), dtype, g).cuda()
    v = si.randn((n * c, Hkv, D), dtype, g).cuda()
    L = n * c
    nbytes = cpk.cpk_roll_workspace_size(Hq, Hkv, C, c, D, tdt)
    assert nbytes > 0, "the case must split the key range"
    wss = [torch.full((nbytes // 4 + 4,), float("nan"), device="cuda") for _ in range(2)]
    with cpk.attention_kernel(KERNELS[kernel]):
        for explicit in (False, True):
            masks = [torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C)).to(tdt).cuda()
                     if explicit else None for j in range(n)]
            outs = []
            for deferred in (False, True):
                bufs = [torch.zeros((1, Hkv, C, D), dtype=tdt, device="cuda") for _ in range(4)]
                out = torch.full((L, Hq, D), float("nan"), dtype=tdt, device="cuda")
                cur, pending = 0, None
                for j in range(n):
                    sl = slice(j * c, (j + 1) * c)
                    ko, vo = bufs[2 * cur], bufs[2 * cur + 1]
                    kn, vn = bufs[2 * (1 - cur)], bufs[2 * (1 - cur) + 1]
                    cpk.cpk_roll_append(ko, vo, k[sl].unsqueeze(0), v[sl].unsqueeze(0), kn, vn)
                    cur = 1 - cur
                    if deferred:
                        pending = cpk.cpk_roll_attention_deferred(
                            q[sl], kn[0], vn[0], (j + 1) * c, 0, wss[j % 2], prev=pending,
                            mask=masks[j], out=out[sl])
                    else:
                        cpk.cpk_roll_attention(q[sl], kn[0], vn[0], (j + 1) * c, 0,
                                               mask=masks[j], out=out[sl])
                if pending is not None:
                    cpk.cpk_roll_flush(pending)
                torch.cuda.synchronize()
                outs.append(out)
            assert bitwise(outs[0], outs[1]), f"mask={explicit}: outputs differ"


@pytest.mark.parametrize("dtype,C,c,Hq,Hkv,D", [
    ("f16", 512, 128, 4, 4, 128),     # start walks 0, 128, 256, 384 and wraps
    ("bf16", 300, 96, 4, 2, 64),      # tiles that wrap the ring mid-tile, GQA
    ("f16", 301, 100, 2, 2, 64),      # mask rows of 301 entries: per-element mask loads
])
def test_scheduled_form_bit_equal_to_general_rolling(dtype, C, c, Hq, Hkv, D):
    """Rolling launches (ring buffer, computed visibility and the explicit
    additive mask, split into parts and unsplit, the chunk's append fused
    in) give the same bits in the latency-scheduled and the general form of
    the 64-column kernel: the output of every chunk and both rings after
    it; the scheduled form also matches the oracle's sliding window."""
    say(f"case: scheduled vs general rolling {dtype} C={C} c={c} heads {Hq}/{Hkv} D={D}")
    tdt = si.TORCH_DTYPE[dtype]
    g = si.generator(530 + C)
    n = 5
    q = si.randn((n * c, Hq, D), dtype, g).cuda()
    k = si.randn((n * c, Hkv, D), dtype, g).cuda()
    v = si.randn((n * c, Hkv, D), dtype, g).cuda()
    L = n * c
    masks = [torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C)).to(tdt).cuda() for j in range(n)]
    for split in (True, False):
        for explicit in (False, True):
            res = {}
            for kind in ("narrow", "general"):
                with cpk.attention_kernel(KERNELS[kind]):
                    kr = torch.zeros((1, Hkv, C, D), dtype=tdt, device="cuda")
                    vr = torch.zeros_like(kr)
                    start, outs = 0, []
                    for j in range(n):
                        sl = slice(j * c, (j + 1) * c)
                        o, start = cpk.cpk_ring_step(q[sl], k[sl], v[sl], kr[0], vr[0],
                                                     (j + 1) * c, 0, start, split=split,
                                                     mask=masks[j] if explicit else None)
                        outs.append(o)
                    torch.cuda.synchronize()
                    res[kind] = (torch.cat(outs), kr, vr)
            (oa, ka, va), (ob, kb, vb) = res["narrow"], res["general"]
            tag = f"split={split} mask={explicit}"
            assert bitwise(oa, ob), f"{tag}: outputs differ"
            assert bitwise(ka, kb) and bitwise(va, vb), f"{tag}: rings differ"
    odt = ODT[tdt]
    rows = np.arange(L)
    qq = oracle.widen(si.storage(q), odt)
    kk = oracle.widen(np.ascontiguousarray(si.storage(k).transpose(1, 0, 2)), odt)
    vv = oracle.widen(np.ascontiguousarray(si.storage(v).transpose(1, 0, 2)), odt)
    lo = np.maximum(0, (rows // c + 1) * c - C).astype(np.int32)
    ref = oracle.attention(qq, kk, vv, lo, rows.astype(np.int32), 1.0 / math.sqrt(D))
    check(res["narrow"][0], ref, TOL[tdt], "scheduled rolling vs sliding-window oracle")


def test_workload4_ring_full_size():
    L, C, c, H, D = 4096, 2048, 256, 16, 128
    say(f"case: workload 4 on the ring buffer, L={L} C={C} c={c} H={H}: bit-equal to the shift")
    q, k, v = si.rolling_inputs()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    masks = [torch.from_numpy(oracle.chunk_mask(L, 0, j, c, C).astype(np.float16)).cuda()
             for j in range(L // c)]
    for m in (None, masks):
        lit, _, lk, lv = cpk.roll_prefill(qd, kd, vd, C, c, masks=m)
        rng, _, rk, rv, st = cpk.ring_prefill(qd, kd, vd, C, c, masks=m)
        torch.cuda.synchronize()
        assert st == 0     # 16 chunks of 256 = 2 full turns of the ring
        assert bitwise(lit, rng), f"mask={m is not None}: ring output differs"
        assert bitwise(rk, lk) and bitwise(rv, lv)


# ------------------------------------------------ HIP graph replay

@pytest.mark.parametrize("kernel", ["narrow", "wide", "general"])
def test_graph_replay_of_chunked_prefill(kernel):
    """A chunked prefill (rewind, then cpk_prefill_chunk per chunk with the
    padded tail) captured once as a HIP graph: every replay, with eager work
    between replays, matches the eager run bit for bit (output, cache rows,
    seqlens_k)."""
    say(f"case: HIP graph [{kernel}] of rewind + padded chunked prefill (L=1300, W=512), 3 replays")
    with cpk.attention_kernel(KERNELS[kernel]):
        _graph_replay_of_chunked_prefill()


def test_graph_replay_of_deferred_ring_prefill():
    """ring_prefill with deferred ring steps (each chunk's split merged by
    the next chunk's launch, the last by the flush) captured once as a HIP
    graph: every replay, with eager work between replays, matches the eager
    run bit for bit (outputs and both rings), with the explicit mask and
    with computed visibility."""
    L, C, c, H, D = 1000, 512, 128, 4, 128
    say(f"case: HIP graph of the deferred ring prefill fp16 L={L} C={C} c={c} H={H}, 3 replays")
    q, k, v = (x.cuda() for x in si.rolling_inputs(L=L, H=H, D=D, seed=720))
    assert cpk.cpk_roll_workspace_size(H, H, C, c, D, torch.float16) > 0
    n_left = (-L) % c
    masks = [torch.from_numpy(oracle.chunk_mask(L + n_left, n_left, j, c, C).astype(np.float16))
             .cuda() for j in range((L + n_left) // c)]
    for m in (None, masks):
        res = {}

        def run():
            res["r"] = cpk.ring_prefill(q, k, v, C, c, masks=m)

        run()
        torch.cuda.synchronize()
        ref_out, _, ref_k, ref_v, _ = (x.clone() if torch.is_tensor(x) else x for x in res["r"])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
        out, _, kr, vr, _ = res["r"]
        for rep in range(3):
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            tag = f"mask={m is not None} replay {rep}"
            assert bitwise(out, ref_out), f"{tag}: output differs"
            assert bitwise(kr, ref_k) and bitwise(vr, ref_v), f"{tag}: rings differ"
            cpk.ring_prefill(q, k, v, C, c, masks=m)   # eager work between replays
            torch.cuda.synchronize()


def _graph_replay_of_chunked_prefill():
    L, W, Hq, Hkv, D = 1300, 512, 16, 4, 128
    q, k, v = si.gqa_prompt(L=L, Hq=Hq, Hkv=Hkv, D=D, seed=700)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = cpk.KVCache(1, Hkv, 2048, D, torch.bfloat16)
    out = torch.empty_like(qd)
    chunks = cpk.cpk_split_chunks(L, W)

    def run():
        cpk.cpk_rewind(cache, 0, 0)
        for past, rows in chunks:
            sl = slice(past, past + rows)
            cpk.cpk_prefill_chunk(qd[sl], kd[sl], vd[sl], cache, 0, past, W, pad=True,
                                  out=out[sl])

    run()
    torch.cuda.synchronize()
    ref_out, ref_k, ref_v = out.clone(), cache.k[:, :, :L].clone(), cache.v[:, :, :L].clone()
    assert int(cache.seqlens_k[0]) == L
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        poison(cache)
        cache.seqlens_k.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert bitwise(out, ref_out), f"replay {rep}: output differs"
        assert bitwise(cache.k[:, :, :L], ref_k) and bitwise(cache.v[:, :, :L], ref_v)
        assert int(cache.seqlens_k[0]) == L
        run()   # eager work between replays
        torch.cuda.synchronize()
        assert bitwise(out, ref_out)
    say("  3 replays bit-identical to the eager run")


# ------------------------------------------------ workload 5: mixed varlen

def _run_mixed(n_dec, ctx_lo, ctx_hi, prompt, budget, Hq, Hkv, D, seed, cap, check_steps, every):
    ctxs = si.mixed_contexts(n_dec, ctx_lo, ctx_hi, seed=seed)
    B = n_dec + 1
    cache = cpk.KVCache(B, Hkv, cap, D, torch.bfloat16)
    si.fill_seeded(cache.k, seed + 1)
    si.fill_seeded(cache.v, seed + 2)
    cache.lens = ctxs + [0]
    pq, pk, pv = si.gqa_prompt(L=prompt, Hq=Hq, Hkv=Hkv, D=D, seed=seed + 3)
    pqd, pkd, pvd = pq.cuda(), pk.cuda(), pv.cuda()
    g = si.generator(seed + 4)
    done, step, lens = 0, 0, list(ctxs)
    prompt_out = torch.empty_like(pqd)
    appended = []      # host copies of every step's decode K/V rows
    while done < prompt:
        rows = cpk.cpk_plan_step(budget, n_dec, prompt - done)
        dq = si.randn((n_dec, Hq, D), "bf16", g).cuda()
        dk_h = si.randn((n_dec, Hkv, D), "bf16", g)
        dv_h = si.randn((n_dec, Hkv, D), "bf16", g)
        appended.append((si.storage(dk_h), si.storage(dv_h)))
        dk, dv = dk_h.cuda(), dv_h.cuda()
        q = torch.cat([dq, pqd[done:done + rows]])
        kn = torch.cat([dk, pkd[done:done + rows]])
        vn = torch.cat([dv, pvd[done:done + rows]])
        slots = list(range(B))
        cu = list(range(n_dec + 1)) + [n_dec + rows]
        past = lens + [done]
        out = cpk.cpk_varlen_step(q, kn, vn, cache, slots, cu, past)
        prompt_out[done:done + rows] = out[n_dec:]
        torch.cuda.synchronize()
        if step in check_steps:
            # decode rows: every one, against the oracle over the sequence's cache
            for s in range(n_dec):
                n = lens[s] + 1
                kk = oracle.widen(si.storage(cache.k[s, :, :n]), oracle.BF16)
                vv = oracle.widen(si.storage(cache.v[s, :, :n]), oracle.BF16)
                qq = oracle.widen(si.storage(dq[s:s + 1]), oracle.BF16)
                ref = oracle.attention(qq, kk, vv, np.zeros(1, np.int32),
                                       np.array([n - 1], np.int32), 1.0 / math.sqrt(D))
                # the appended rows are checked before the cache feeds the oracle
                assert np.array_equal(si.storage(cache.k[s, :, n - 1]), si.storage(dk[s]))
                assert np.array_equal(si.storage(cache.v[s, :, n - 1]), si.storage(dv[s]))
                err = float(np.max(np.abs(f64(out[s:s + 1]) - ref)))
                assert err <= 2e-2, f"decode seq {s} ctx {n}: {err}"
            say(f"  step {step}: {n_dec} decode rows ok, prompt rows {done}..{done + rows}")
        lens = [x + 1 for x in lens]
        done += rows
        step += 1
    torch.cuda.synchronize()
    qs, ks, vs = (si.storage(x) for x in (pq, pk, pv))
    rows_idx = sample_rows(prompt, [(0, prompt)], every=every)
    ref = oracle_rows(qs, ks, vs, rows_idx, oracle.BF16)
    check(prompt_out[torch.from_numpy(rows_idx).cuda()], ref, 2e-2,
          f"prompt rows across {step} budgeted steps")
    assert np.array_equal(si.storage(cache.k[n_dec, :, :prompt]), ks.transpose(1, 0, 2))
    assert np.array_equal(si.storage(cache.v[n_dec, :, :prompt]), vs.transpose(1, 0, 2))
    # every step's decode rows (checked steps or not) sit at ctx + step
    ck = si.storage(cache.k[:n_dec])
    cv = si.storage(cache.v[:n_dec])
    for i, (ak, av) in enumerate(appended):
        pos = np.array(ctxs) + i
        got_k = ck[np.arange(n_dec), :, pos]
        got_v = cv[np.arange(n_dec), :, pos]
        assert np.array_equal(got_k, ak) and np.array_equal(got_v, av), f"step {i} append"
    assert cache.seqlens_k.cpu().tolist() == [c + step for c in ctxs] + [prompt]
    return step


@pytest.mark.parametrize("kernel", ["narrow", "wide"])
def test_varlen_interleaved_order(kernel):
    """Prompt and decode sequences interleaved in the pack (prompts first,
    between and after decodes) give, sequence by sequence, the same bits as
    the same step packed decodes-first, and the prompt rows match the
    oracle: the prefill launch covers only the range of prompt sequences
    and skips the decode rows inside it."""
    say(f"case: varlen interleaved order [{kernel}]: 2 prompts, 3 decodes, G=4")
    Hq, Hkv, D, cap = 8, 2, 128, 1024
    # slot: (past, rows)
    seqs = {0: (100, 300), 1: (50, 1), 2: (700, 1), 3: (0, 200), 4: (10, 1)}
    g = si.generator(540)
    data = {}
    for sl, (past, rows) in seqs.items():
        data[sl] = tuple(si.randn((rows, h, D), "bf16", g).cuda() for h in (Hq, Hkv, Hkv))
    caches = []
    for _ in range(2):
        c = cpk.KVCache(5, Hkv, cap, D, torch.bfloat16)
        si.fill_seeded(c.k, 541)
        si.fill_seeded(c.v, 542)
        c.lens = [seqs[s][0] for s in range(5)]
        caches.append(c)
    outs = []
    with cpk.attention_kernel(KERNELS[kernel]):
        for order, cache in zip(([0, 1, 2, 3, 4], [1, 2, 4, 0, 3]), caches):
            q = torch.cat([data[s][0] for s in order])
            kn = torch.cat([data[s][1] for s in order])
            vn = torch.cat([data[s][2] for s in order])
            cu = [0]
            for s in order:
                cu.append(cu[-1] + seqs[s][1])
            out = cpk.cpk_varlen_step(q, kn, vn, cache, order, cu, [seqs[s][0] for s in order])
            torch.cuda.synchronize()
            outs.append({s: out[cu[i]:cu[i + 1]] for i, s in enumerate(order)})
    for s in seqs:
        assert bitwise(outs[0][s], outs[1][s]), f"slot {s}: order changes the output"
    assert bitwise(caches[0].k, caches[1].k) and bitwise(caches[0].v, caches[1].v)
    for s in (0, 3):
        past, rows = seqs[s]
        n = past + rows
        kk = oracle.widen(si.storage(caches[0].k[s, :, :n]), oracle.BF16)
        vv = oracle.widen(si.storage(caches[0].v[s, :, :n]), oracle.BF16)
        qq = oracle.widen(si.storage(data[s][0]), oracle.BF16)
        lim = (past + np.arange(rows)).astype(np.int32)
        ref = oracle.attention(qq, kk, vv, np.zeros(rows, np.int32), lim, 1.0 / math.sqrt(D))
        check(outs[0][s], ref, 2e-2, f"prompt slot {s}")


@pytest.mark.parametrize("kernel", ["narrow", "wide", "general"])
def test_mixed_step_small_full_compare(kernel):
    say(f"case: mixed step small [{kernel}]: 5 decodes ctx 20..300, prompt 700, budget 128, G=4")
    with cpk.attention_kernel(KERNELS[kernel]):
        steps = _run_mixed(5, 20, 300, 700, 128, 8, 2, 128, seed=500, cap=1024,
                           check_steps=set(range(10)), every=1)
    assert steps == 6


def test_mixed_step_two_streams_bit_equal():
    """Decode rows and prompt rows of each packed step on two streams
    (append + decode on the current stream, the prompt attention on a side
    stream after the append): outputs and cache bit-identical to the
    single-stream step, over the budgeted steps of a small mixed workload."""
    say("case: mixed step on two streams vs one: 6 decodes ctx 30..900, prompt 1500, budget 256")
    n_dec, Hq, Hkv, D, cap, prompt, budget = 6, 16, 4, 128, 2048, 1500, 256
    ctxs = si.mixed_contexts(n_dec, 30, 900, seed=520)
    caches = []
    for _ in range(2):
        c = cpk.KVCache(n_dec + 1, Hkv, cap, D, torch.bfloat16)
        si.fill_seeded(c.k, 521)
        si.fill_seeded(c.v, 522)
        caches.append(c)
    pq, pk, pv = (x.cuda() for x in si.gqa_prompt(L=prompt, Hq=Hq, Hkv=Hkv, D=D, seed=523))
    g = si.generator(524)
    side = torch.cuda.Stream()
    done, lens, steps = 0, list(ctxs), 0
    prompt_out = torch.empty_like(pq)
    worst = 0.0
    while done < prompt:
        rows = cpk.cpk_plan_step(budget, n_dec, prompt - done)
        dq = si.randn((n_dec, Hq, D), "bf16", g).cuda()
        dk = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
        dv = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
        q = torch.cat([dq, pq[done:done + rows]])
        kn = torch.cat([dk, pk[done:done + rows]])
        vn = torch.cat([dv, pv[done:done + rows]])
        slots = list(range(n_dec + 1))
        cu = list(range(n_dec + 1)) + [n_dec + rows]
        past = lens + [done]
        o1 = cpk.cpk_varlen_step(q, kn, vn, caches[0], slots, cu, past)
        o2 = cpk.varlen_step_overlapped(q, kn, vn, caches[1], slots, cu, past, side)
        torch.cuda.synchronize()
        assert bitwise(o1, o2), f"step {steps}: two-stream output differs"
        prompt_out[done:done + rows] = o2[n_dec:]
        # every decode row of the two-stream step against the oracle over
        # its sequence's cache (whose new row is checked first)
        for s in range(n_dec):
            n = lens[s] + 1
            assert np.array_equal(si.storage(caches[1].k[s, :, n - 1]), si.storage(dk[s]))
            assert np.array_equal(si.storage(caches[1].v[s, :, n - 1]), si.storage(dv[s]))
            kk = oracle.widen(si.storage(caches[1].k[s, :, :n]), oracle.BF16)
            vv = oracle.widen(si.storage(caches[1].v[s, :, :n]), oracle.BF16)
            qq = oracle.widen(si.storage(dq[s:s + 1]), oracle.BF16)
            ref = oracle.attention(qq, kk, vv, np.zeros(1, np.int32), np.array([n - 1], np.int32),
                                   1.0 / math.sqrt(D))
            err = float(np.max(np.abs(f64(o2[s:s + 1]) - ref)))
            worst = max(worst, err)
            assert err <= TOL[torch.bfloat16], f"step {steps} decode seq {s} ctx {n}: {err}"
        lens = [x + 1 for x in lens]
        done += rows
        steps += 1
    assert bitwise(caches[0].k, caches[1].k) and bitwise(caches[0].v, caches[1].v)
    assert torch.equal(caches[0].seqlens_k, caches[1].seqlens_k)
    say(f"  {steps} steps bit-identical; decode rows vs oracle worst {worst:.3e}")
    qs, ks, vs = (si.storage(x.cpu()) for x in (pq, pk, pv))
    rows_idx = sample_rows(prompt, [(0, prompt)], every=7)
    ref = oracle_rows(qs, ks, vs, rows_idx, oracle.BF16)
    check(prompt_out[torch.from_numpy(rows_idx).cuda()], ref, TOL[torch.bfloat16],
          f"two-stream prompt rows across {steps} steps")


def _to_paged(cont: "cpk.KVCache", paged: "cpk.PagedKVCache", n_pos):
    """Copy positions [0, n_pos[s]) of every slot of a contiguous cache into
    the paged pools through the block table (test plumbing)."""
    bs = paged.block_size
    table = paged.block_table.cpu()
    for s, n in enumerate(n_pos):
        for i in range((n + bs - 1) // bs):
            b = int(table[s, i])
            paged.k[b] = cont.k[s, :, i * bs:(i + 1) * bs]
            paged.v[b] = cont.v[s, :, i * bs:(i + 1) * bs]
        paged.lens[s] = n
    paged.seqlens_k.copy_(cont.seqlens_k)


@pytest.mark.parametrize("kernel", ["narrow", "wide"])
def test_paged_varlen_matches_contiguous(kernel):
    """The packed mixed step over a paged cache (256-position blocks in a
    shuffled order) equals the step over a contiguous cache bit for bit:
    outputs of every step, and every cached position afterwards."""
    say(f"case: paged vs contiguous mixed steps [{kernel}]: 5 decodes ctx 40..1500, prompt 900")
    n_dec, Hq, Hkv, D, cap, prompt, budget, bs = 5, 16, 4, 128, 2048, 900, 300, 256
    ctxs = si.mixed_contexts(n_dec, 40, 1500, seed=530)
    B = n_dec + 1
    cont = cpk.KVCache(B, Hkv, cap, D, torch.bfloat16)
    si.fill_seeded(cont.k, 531)
    si.fill_seeded(cont.v, 532)
    cont.seqlens_k.copy_(torch.tensor(ctxs + [0], dtype=torch.int32))
    cont.lens = ctxs + [0]
    maxb = cap // bs
    paged = cpk.PagedKVCache(B, Hkv, B * maxb + 3, bs, maxb, D, torch.bfloat16)
    perm = torch.randperm(B * maxb + 3, generator=si.generator(533))[:B * maxb]
    paged.block_table.copy_(perm.view(B, maxb).to(torch.int32))
    _to_paged(cont, paged, ctxs + [0])
    pq, pk, pv = (x.cuda() for x in si.gqa_prompt(L=prompt, Hq=Hq, Hkv=Hkv, D=D, seed=534))
    g = si.generator(535)
    done, lens, steps = 0, list(ctxs), 0
    with cpk.attention_kernel(KERNELS[kernel]):
        while done < prompt:
            rows = cpk.cpk_plan_step(budget, n_dec, prompt - done)
            dq = si.randn((n_dec, Hq, D), "bf16", g).cuda()
            dk = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
            dv = si.randn((n_dec, Hkv, D), "bf16", g).cuda()
            q = torch.cat([dq, pq[done:done + rows]])
            kn = torch.cat([dk, pk[done:done + rows]])
            vn = torch.cat([dv, pv[done:done + rows]])
            slots = list(range(B))
            cu = list(range(n_dec + 1)) + [n_dec + rows]
            past = lens + [done]
            o1 = cpk.cpk_varlen_step(q, kn, vn, cont, slots, cu, past)
            o2 = cpk.cpk_paged_varlen_step(q, kn, vn, paged, slots, cu, past)
            torch.cuda.synchronize()
            assert bitwise(o1, o2), f"step {steps}: paged output differs"
            # the paged decode rows (block-table path of the decode kernel)
            # against the oracle over positions gathered through the table
            for s in range(n_dec):
                n = lens[s] + 1
                gk, gv = paged.gather(s, n)
                assert np.array_equal(si.storage(gk[:, n - 1]), si.storage(dk[s]))
                assert np.array_equal(si.storage(gv[:, n - 1]), si.storage(dv[s]))
                kk = oracle.widen(si.storage(gk), oracle.BF16)
                vv = oracle.widen(si.storage(gv), oracle.BF16)
                qq = oracle.widen(si.storage(dq[s:s + 1]), oracle.BF16)
                ref = oracle.attention(qq, kk, vv, np.zeros(1, np.int32),
                                       np.array([n - 1], np.int32), 1.0 / math.sqrt(D))
                err = float(np.max(np.abs(f64(o2[s:s + 1]) - ref)))
                assert err <= TOL[torch.bfloat16], f"paged step {steps} seq {s}: {err}"
            lens = [x + 1 for x in lens]
            done += rows
            steps += 1
    assert torch.equal(cont.seqlens_k, paged.seqlens_k)
    for s, n in enumerate(lens + [prompt]):
        pk_, pv_ = paged.gather(s, n)
        assert bitwise(pk_, cont.k[s, :, :n]) and bitwise(pv_, cont.v[s, :, :n]), f"slot {s}"
    say(f"  {steps} steps bit-identical, cache positions equal")


@pytest.mark.parametrize("kernel", ["narrow", "wide"])
def test_paged_shared_prefix(kernel):
    """Two prompts with a common 512-token prefix stored once (both block
    tables name the same two blocks) prefill their own suffixes in one packed
    step; outputs equal the same step over a contiguous cache holding a copy
    of the prefix in each slot, bit for bit, and the shared blocks are not
    written."""
    say(f"case: paged shared prefix [{kernel}]: prefix 512, suffixes 300 and 177")
    Hq, Hkv, D, bs, P = 16, 4, 128, 256, 512
    suf = [300, 177]
    maxb = 4
    paged = cpk.PagedKVCache(2, Hkv, 8, bs, maxb, D, torch.bfloat16)
    paged.block_table.copy_(torch.tensor([[5, 2, 0, 7], [5, 2, 3, 6]], dtype=torch.int32))
    cont = cpk.KVCache(2, Hkv, maxb * bs, D, torch.bfloat16)
    pre_k = si.randn((Hkv, P, D), "bf16", si.generator(540)).cuda()
    pre_v = si.randn((Hkv, P, D), "bf16", si.generator(541)).cuda()
    for s in range(2):
        cont.k[s, :, :P] = pre_k
        cont.v[s, :, :P] = pre_v
    cont.seqlens_k.fill_(P)
    cont.lens = [P, P]
    _to_paged(cont, paged, [P, P])
    shared_k = paged.k[[5, 2]].clone()
    qs = [si.randn((n, Hq, D), "bf16", si.generator(542 + i)).cuda() for i, n in enumerate(suf)]
    ks = [si.randn((n, Hkv, D), "bf16", si.generator(544 + i)).cuda() for i, n in enumerate(suf)]
    vs = [si.randn((n, Hkv, D), "bf16", si.generator(546 + i)).cuda() for i, n in enumerate(suf)]
    q, kn, vn = torch.cat(qs), torch.cat(ks), torch.cat(vs)
    cu = [0, suf[0], suf[0] + suf[1]]
    with cpk.attention_kernel(KERNELS[kernel]):
        o1 = cpk.cpk_varlen_step(q, kn, vn, cont, [0, 1], cu, [P, P])
        o2 = cpk.cpk_paged_varlen_step(q, kn, vn, paged, [0, 1], cu, [P, P])
        torch.cuda.synchronize()
    assert bitwise(o1, o2), "shared-prefix output differs"
    assert bitwise(paged.k[[5, 2]], shared_k), "shared prefix blocks were written"
    for s in range(2):
        n = P + suf[s]
        pk_, pv_ = paged.gather(s, n)
        assert bitwise(pk_, cont.k[s, :, :n]) and bitwise(pv_, cont.v[s, :, :n])
    # against the oracle: each sequence's rows over prefix + suffix
    for s in range(2):
        kk = oracle.widen(si.storage(cont.k[s, :, :P + suf[s]]), oracle.BF16)
        vv = oracle.widen(si.storage(cont.v[s, :, :P + suf[s]]), oracle.BF16)
        qq = oracle.widen(si.storage(qs[s]), oracle.BF16)
        rows = np.arange(P, P + suf[s], dtype=np.int32)
        ref = oracle.attention(qq, kk, vv, np.zeros(len(rows), np.int32), rows,
                               1.0 / math.sqrt(D))
        check(o2[cu[s]:cu[s + 1]], ref, 2e-2, f"suffix {s} vs oracle")


def test_workload5_mixed_full_size_budget_2048():
    say("case: workload 5: 64 decodes ctx U[512,16384], 20000-token prompt, budget 2048")
    steps = _run_mixed(64, 512, 16384, 20000, 2048, 32, 8, 128, seed=si.SEEDS["mixed"],
                       cap=20480, check_steps={0, 10}, every=211)
    assert steps == 11


def test_workload5_mixed_full_size_budget_8192():
    say("case: workload 5: 64 decodes ctx U[512,16384], 20000-token prompt, budget 8192")
    steps = _run_mixed(64, 512, 16384, 20000, 8192, 32, 8, 128, seed=si.SEEDS["mixed"],
                       cap=20480, check_steps={0, 2}, every=211)
    assert steps == 3    # 8128, 8128 and 3744 prompt rows


# ------------------------------------------------ decode rows, every variant

# past lengths around the decode kernel's boundaries: 16/32-key streaming
# steps, 64-key waves, 256-key work items, and many work items
DECODE_PAST = [0, 1, 14, 15, 16, 31, 32, 255, 256, 511, 1022, 1023, 1024, 2047, 2500, 4095]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_rows_every_variant(dtype, D, G):
    """Decode-only varlen step (one row per sequence) against the oracle for
    every (dtype, head_dim, group) the decode kernel is built for.  The
    cache is NaN past each sequence's length, and every third query is
    scaled by 8 so its scores span far more than the lazy maximum's 2^8
    window (the running reference must be raised mid-stream)."""
    Hkv, n, cap = 2, len(DECODE_PAST), 4096
    Hq = G * Hkv
    sdt = "bf16" if dtype == torch.bfloat16 else "f16"
    odt = ODT[dtype]
    seed = 900 + 10 * D + G + (0 if dtype == torch.bfloat16 else 5)
    say(f"case: decode rows {sdt} D={D} G={G} Hkv={Hkv} past {DECODE_PAST[0]}..{DECODE_PAST[-1]}")
    cache = cpk.KVCache(n, Hkv, cap, D, dtype)
    poison(cache)
    full_k = si.fill_seeded(torch.empty_like(cache.k), seed)
    full_v = si.fill_seeded(torch.empty_like(cache.v), seed + 1)
    for s, p in enumerate(DECODE_PAST):
        cache.k[s, :, :p] = full_k[s, :, :p]
        cache.v[s, :, :p] = full_v[s, :, :p]
    del full_k, full_v
    cache.lens = list(DECODE_PAST)
    g = si.generator(seed + 2)
    q = si.randn((n, Hq, D), sdt, g).cuda()
    q[::3] *= 8
    kn = si.randn((n, Hkv, D), sdt, g).cuda()
    vn = si.randn((n, Hkv, D), sdt, g).cuda()
    out = cpk.cpk_varlen_step(q, kn, vn, cache, list(range(n)), list(range(n + 1)), DECODE_PAST)
    torch.cuda.synchronize()
    # the decode launch appends the new rows itself and records the lengths
    assert cache.seqlens_k.tolist() == [p + 1 for p in DECODE_PAST]
    worst = 0.0
    for s, p in enumerate(DECODE_PAST):
        nk = p + 1
        assert np.array_equal(si.storage(cache.k[s, :, p]), si.storage(kn[s]))
        assert np.array_equal(si.storage(cache.v[s, :, p]), si.storage(vn[s]))
        kk = oracle.widen(si.storage(cache.k[s, :, :nk]), odt)
        vv = oracle.widen(si.storage(cache.v[s, :, :nk]), odt)
        qq = oracle.widen(si.storage(q[s:s + 1]), odt)
        ref = oracle.attention(qq, kk, vv, np.zeros(1, np.int32), np.array([p], np.int32),
                               1.0 / math.sqrt(D))
        g64 = f64(out[s:s + 1])
        assert np.isfinite(g64).all(), f"past {p}: non-finite"
        assert np.abs(vv).max() <= 5.7, "the fp16 tolerance assumes |v| <= 5.7"
        err = float(np.max(np.abs(g64 - ref)))
        worst = max(worst, err)
        assert err <= TOL[dtype], f"past {p}: max-abs {err}"
    say(f"  {n} decode rows: worst max-abs err {worst:.3e} (tol {TOL[dtype]:g})")
