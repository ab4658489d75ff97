"""Pins of the CPU oracle against things other than itself.

Every pin here is independent of the oracle's own code: values the pages
print (tests/golden/pages_values.json), a library routine (torch's
scaled_dot_product_attention, torch.cat, numpy/torch dtype widening),
brute force with exact summation on tiny inputs, closed forms, and the
pages' invariants.  The mutation tests at the end plant plausible mistakes
in the oracle's inputs or bookkeeping (on the CPU) and check that a pin
fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth_inputs as si

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def _causal_oracle(q, k, v, scale=None):
    """q [L,Hq,D], k/v [L,Hkv,D] fp64 token-major -> one-shot causal oracle."""
    L = q.shape[0]
    kk = np.ascontiguousarray(k.transpose(1, 0, 2))
    vv = np.ascontiguousarray(v.transpose(1, 0, 2))
    lo = np.zeros(L, np.int32)
    hi = np.arange(L, dtype=np.int32)
    s = oracle.default_scale(q.shape[2]) if scale is None else scale
    return oracle.attention(q, kk, vv, lo, hi, s)


# --------------------------------------------------------------- widening

def test_widen_f16_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_widen_bf16_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------ the demo (library + golden)

def test_demo_split_matches_printed_chunks():
    g = GOLD["demo_split"]
    chunks = oracle.split_chunks(g["prompt_len"], g["chunk"])
    assert len(chunks) == g["n_chunks"]
    assert [r for _, r in chunks] == g["chunk_rows"]


def _sdpa64(q, k, v, vis=None):
    """Library reference: torch's scaled_dot_product_attention in fp64 on
    token-major arrays q [n_q, Hq, D] and k/v [n_k, Hkv, D] (numpy or torch),
    KV heads repeated to the query heads in contiguous groups.  vis is an
    optional [n_q, n_k] boolean visibility; without it the rows are the
    causal one-shot rows 0..n_q-1 over keys 0..n_k-1."""
    q, k, v = (torch.as_tensor(x).double() for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    tq = q.permute(1, 0, 2)[None]
    tk = k.permute(1, 0, 2)[None].repeat_interleave(G, dim=1)
    tv = v.permute(1, 0, 2)[None].repeat_interleave(G, dim=1)
    if vis is None:
        out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    else:
        out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.as_tensor(vis))
    return out[0].permute(1, 0, 2).numpy()


def test_oracle_entry_points_match_sdpa_on_demo():
    """Library pin of the oracle's own cache-driven entry points on the
    glossary demo (fp32, 8 heads x 64, 1000 tokens, chunk 256): one-shot
    prefill and chunked prefill, each appending into a Cache and attending
    from it, equal torch's causal SDPA in fp64 to rounding and the demo's
    own fp32 SDPA within the page's 1e-5; the chunk split is the printed
    256/256/256/232."""
    g = GOLD["demo_split"]
    (q4, k4, v4), (qt, kt, vt) = si.demo_qkv()
    q, k, v = (si.storage(x) for x in (qt, kt, vt))
    ref64 = _sdpa64(qt, kt, vt)
    ref32 = F.scaled_dot_product_attention(q4, k4, v4, is_causal=True)[0].permute(1, 0, 2)
    ref32 = ref32.double().numpy()
    one = oracle.prefill_one_shot(oracle.Cache(oracle.F32, 1, 8, 1024, 64), 0, q, k, v)
    chunked, chunks = oracle.prefill_chunked(oracle.Cache(oracle.F32, 1, 8, 1024, 64), 0,
                                             q, k, v, g["chunk"])
    assert len(chunks) == g["n_chunks"]
    assert [r for _, r in chunks] == g["chunk_rows"]
    for got in (one, chunked):
        assert np.max(np.abs(got - ref64)) < 1e-12
        assert np.max(np.abs(got - ref32)) < g["allclose_atol"]


@pytest.mark.parametrize("W", [64, 100, 128])
def test_oracle_cache_path_gqa_bf16_matches_sdpa(W):
    """Library pin of the cache path on GQA bf16 storage (8 query heads over
    2 KV heads, head dim 64, 300 tokens): one-shot, chunked and padded
    chunked prefill read K/V back from the oracle's bf16 cache; each equals
    fp64 SDPA over K/V repeated per group (widened by torch, not by the
    oracle) to rounding."""
    qt, kt, vt = si.gqa_prompt(L=300, Hq=8, Hkv=2, D=64, seed=23)
    q, k, v = (si.storage(x) for x in (qt, kt, vt))
    ref = _sdpa64(qt, kt, vt)
    outs = [oracle.prefill_one_shot(oracle.Cache(oracle.BF16, 2, 2, 512, 64), 1, q, k, v)]
    outs.append(oracle.prefill_chunked(oracle.Cache(oracle.BF16, 2, 2, 512, 64), 1,
                                       q, k, v, W)[0])
    outs.append(oracle.prefill_chunked_padded(oracle.Cache(oracle.BF16, 2, 2, 512, 64), 1,
                                              q, k, v, W)[0])
    for got in outs:
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) < 1e-12


def test_oracle_varlen_step_matches_sdpa_with_position_mask():
    """Library pin of the packed step: two decode rows (contexts 37 and 5)
    and a 70-row prompt chunk at past 30, each sequence's rows against fp64
    SDPA with a boolean mask built from absolute positions (key j visible
    to row i when j <= past + i)."""
    Hq, Hkv, D = 4, 2, 32
    gen = si.generator(24)
    ctx = {0: 37, 1: 5, 2: 30}
    rows = {0: 1, 1: 1, 2: 70}
    full = {s: tuple(si.randn((ctx[s] + rows[s], h, D), "bf16", gen) for h in (Hq, Hkv, Hkv))
            for s in ctx}
    cache = oracle.Cache(oracle.BF16, 3, Hkv, 128, D)
    for s in ctx:
        _, kf, vf = full[s]
        if ctx[s]:
            cache.append(s, si.storage(kf[:ctx[s]]), si.storage(vf[:ctx[s]]), 0)
    pack = [torch.cat([full[s][i][ctx[s]:] for s in ctx]) for i in range(3)]
    cu = np.cumsum([0] + [rows[s] for s in ctx])
    outs = oracle.varlen_step(cache, [(s, ctx[s]) for s in ctx],
                              *(si.storage(x) for x in pack), cu)
    for s in ctx:
        qf, kf, vf = full[s]
        n = ctx[s] + rows[s]
        vis = (np.arange(n)[None, :] <= ctx[s] + np.arange(rows[s])[:, None])
        ref = _sdpa64(qf[ctx[s]:], kf, vf, vis)
        assert np.max(np.abs(outs[s] - ref)) < 1e-12


def test_oracle_chunked_equals_one_shot_demo_bitwise():
    _, (qt, kt, vt) = si.demo_qkv()
    q, k, v = (si.storage(x) for x in (qt, kt, vt))
    c1 = oracle.Cache(oracle.F32, 1, 8, 1024, 64)
    one = oracle.prefill_one_shot(c1, 0, q, k, v)
    c2 = oracle.Cache(oracle.F32, 1, 8, 1024, 64)
    chunked, chunks = oracle.prefill_chunked(c2, 0, q, k, v, 256)
    assert [r for _, r in chunks] == [256, 256, 256, 232]
    assert np.array_equal(one, chunked)
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)


# ------------------------------------------------------------ GQA mapping

def test_gqa_mapping_matches_sdpa_with_repeated_kv():
    r = _rng(5)
    L, Hq, Hkv, D = 40, 8, 2, 16
    q = r.standard_normal((L, Hq, D))
    k = r.standard_normal((L, Hkv, D))
    v = r.standard_normal((L, Hkv, D))
    orc = _causal_oracle(q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(orc - ref)) < 1e-12


# ------------------------------------------------- brute force (exact sums)

def _brute(q, k, v, lo, hi, scale, addmask=None):
    """Pure-Python attention with math.fsum (exactly rounded sums)."""
    n_q, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    out = []
    for i in range(n_q):
        row = []
        for h in range(Hq):
            g = h // (Hq // Hkv)
            js = list(range(lo[i], hi[i] + 1))
            s = []
            for j in js:
                dot = math.fsum(q[i][h][d] * k[g][j][d] for d in range(D)) * scale
                if addmask is not None:
                    dot += addmask[i][j]
                s.append(dot)
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = math.fsum(w)
            row.append([math.fsum(w[t] * v[g][js[t]][d] for t in range(len(js))) / den
                        for d in range(D)])
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("D", [1, 2, 4])
@pytest.mark.parametrize("case", ["random", "large", "ties"])
def test_brute_force_tiny(D, case):
    r = _rng(100 + D)
    L, Hq, Hkv = 7, 4, 2
    if case == "random":
        q = r.standard_normal((L, Hq, D))
        k = r.standard_normal((Hkv, L, D))
    elif case == "large":
        q = 30.0 * r.standard_normal((L, Hq, D))
        k = 30.0 * r.standard_normal((Hkv, L, D))
    else:
        q = np.ones((L, Hq, D))
        k = np.ones((Hkv, L, D))
    v = r.standard_normal((Hkv, L, D))
    lo = np.array([0, 0, 1, 0, 2, 0, 3], np.int32)
    hi = np.array([0, 1, 2, 3, 4, 5, 6], np.int32)
    scale = 0.37
    got = oracle.attention(q, k, v, lo, hi, scale)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), lo.tolist(), hi.tolist(), scale)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_brute_force_additive_mask():
    r = _rng(7)
    n_q, n_k, D = 5, 6, 3
    q = r.standard_normal((n_q, 2, D))
    k = r.standard_normal((1, n_k, D))
    v = r.standard_normal((1, n_k, D))
    mask = np.where(r.random((n_q, n_k)) < 0.4, oracle.MASK_FILL, 0.0)
    mask[:, 2] = 0.0
    lo = np.zeros(n_q, np.int32)
    hi = np.full(n_q, n_k - 1, np.int32)
    got = oracle.attention(q, k, v, lo, hi, 0.5, addmask=mask)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), lo.tolist(), hi.tolist(), 0.5, mask.tolist())
    assert np.max(np.abs(got - ref)) < 1e-12


# ------------------------------------------------------------ closed forms

def test_closed_form_zero_query_gives_prefix_means():
    r = _rng(11)
    L, H, D = 50, 2, 8
    q = np.zeros((L, H, D))
    k = r.standard_normal((L, H, D))
    v = r.standard_normal((L, H, D))
    got = _causal_oracle(q, k, v)
    ref = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
    assert np.max(np.abs(got - ref)) < 1e-13


def test_closed_form_first_row_is_first_value_exactly():
    r = _rng(12)
    q = r.standard_normal((10, 4, 8))
    k = r.standard_normal((10, 2, 8))
    v = r.standard_normal((10, 2, 8))
    got = _causal_oracle(q, k, v)
    for h in range(4):
        assert np.array_equal(got[0, h], v[0, h // 2])


def test_closed_form_equal_keys_give_uniform_weights():
    r = _rng(13)
    L, D = 30, 8
    q = r.standard_normal((L, 1, D))
    k = np.repeat(r.standard_normal((1, 1, D)), L, axis=0)
    v = r.standard_normal((L, 1, D))
    got = _causal_oracle(q, k, v)
    ref = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
    assert np.max(np.abs(got - ref)) < 1e-13


def test_closed_form_dominant_score_selects_its_value():
    r = _rng(14)
    L, D = 20, 8
    q = r.standard_normal((L, 1, D))
    k = 0.01 * r.standard_normal((L, 1, D))
    v = r.standard_normal((L, 1, D))
    target = 5
    k[target, 0] = 400.0 * q[L - 1, 0] / np.linalg.norm(q[L - 1, 0])
    got = _causal_oracle(q, k, v)
    assert np.max(np.abs(got[L - 1, 0] - v[target, 0])) < 1e-12


# ----------------------------------------------- cache: append-only, prefix

def test_cache_after_each_chunk_is_prefix_of_one_shot_cache():
    q, k, v = si.gqa_prompt(L=700, Hq=8, Hkv=2, D=64, seed=21)
    q, k, v = (si.storage(x) for x in (q, k, v))
    one = oracle.Cache(oracle.BF16, 1, 2, 1024, 64)
    one.append(0, k, v, 0)
    ch = oracle.Cache(oracle.BF16, 1, 2, 1024, 64)
    for past, rows in oracle.split_chunks(700, 256):
        ch.append(0, k[past:past + rows], v[past:past + rows], past)
        n = past + rows
        assert ch.lens[0] == n
        assert np.array_equal(ch.k[0, :, :n], one.k[0, :, :n])
        assert np.array_equal(ch.v[0, :, :n], one.v[0, :, :n])
    # the cache holds the input bytes verbatim, head-major
    assert np.array_equal(one.k[0, :, :700], k.transpose(1, 0, 2))


def test_chunked_equals_one_shot_gqa_bf16_bitwise():
    q, k, v = si.gqa_prompt(L=600, Hq=8, Hkv=2, D=64, seed=22)
    q, k, v = (si.storage(x) for x in (q, k, v))
    c1 = oracle.Cache(oracle.BF16, 1, 2, 1024, 64)
    one = oracle.prefill_one_shot(c1, 0, q, k, v)
    c2 = oracle.Cache(oracle.BF16, 1, 2, 1024, 64)
    chunked, _ = oracle.prefill_chunked(c2, 0, q, k, v, 128)
    assert np.array_equal(one, chunked)


def test_capacity_is_enforced():
    c = oracle.Cache(oracle.BF16, 1, 1, 8, 4)
    kk = np.zeros((9, 1, 4), np.uint16)
    with pytest.raises(ValueError):
        c.append(0, kk, kk, 0)


# ------------------------------------------------------------------ ladder

def test_ladder_printed_values():
    g = GOLD["ladder"]
    assert oracle.ladder_rungs(g["W"]) == g["rungs"]
    assert oracle.ladder_width(512, 113) == 171
    assert oracle.ladder_width(512, 176) == 342
    assert oracle.ladder_width(512, 311) == 342
    assert oracle.ladder_width(512, 171) == 171
    assert oracle.ladder_width(512, 512) == 512
    waste = max(oracle.ladder_width(512, r) - r for r in range(1, 513))
    assert waste == g["max_extra_rows"]


def test_ladder_top_rung_is_chunk_width_for_all_widths():
    for W in range(1, 8193):
        rungs = oracle.ladder_rungs(W)
        assert rungs[-1] == W
        assert 1 <= len(rungs) <= 3
        assert rungs == sorted(set(rungs))
    # the worst waste is one step minus one row
    for W in list(range(1, 200)) + [256, 511, 512, 513, 1024, 2048]:
        waste = max(oracle.ladder_width(W, r) - r for r in range(1, W + 1))
        assert waste == -(-W // 3) - 1


def test_power_of_two_ladder_penalty_arithmetic():
    g = GOLD["ladder"]["power_of_two_example"]
    rows = g["rows"]
    p2 = 1 << (rows - 1).bit_length()
    assert p2 == g["power_of_two_width"]
    assert round(100 * (p2 - rows) / rows) == g["extra_fraction_pct"]
    assert oracle.ladder_width(512, rows) == 342


# ------------------------------------------------------------------- split

def test_split_printed_examples():
    g = GOLD["split_examples"]
    for L, rows in g["cases"].items():
        assert [r for _, r in oracle.split_chunks(int(L), g["W"])] == rows
    f = GOLD["four_thousand_in_512"]
    ch = oracle.split_chunks(f["L"], f["W"])
    assert len(ch) == f["n_forwards"]
    assert [r for _, r in ch] == [512] * 7 + [416]
    assert [p for p, _ in ch] == [512 * i for i in range(8)]


# ----------------------------------------------------------------- padding

def test_padded_rows_never_change_real_rows():
    q, k, v = si.gqa_prompt(L=1137, Hq=8, Hkv=2, D=64, seed=23)
    q, k, v = (si.storage(x) for x in (q, k, v))
    c1 = oracle.Cache(oracle.BF16, 1, 2, 2048, 64)
    plain, _ = oracle.prefill_chunked(c1, 0, q, k, v, 512)
    c2 = oracle.Cache(oracle.BF16, 1, 2, 2048, 64)
    padded, widths = oracle.prefill_chunked_padded(c2, 0, q, k, v, 512)
    assert widths == [512, 512, 171]
    assert np.array_equal(plain, padded)
    assert c2.lens[0] == 1137
    assert np.array_equal(c1.k[0, :, :1137], c2.k[0, :, :1137])
    assert np.array_equal(c1.v[0, :, :1137], c2.v[0, :, :1137])
    # stale pad entries sit past the logical length, copies of the last row
    assert np.array_equal(c2.k[0, :, 1137:1024 + 171], np.repeat(c2.k[0, :, 1136:1137], 1024 + 171 - 1137, axis=1))


def test_rewind_then_overwrite_matches_clean_run():
    q, k, v = si.gqa_prompt(L=300, Hq=4, Hkv=2, D=64, seed=24)
    q, k, v = (si.storage(x) for x in (q, k, v))
    c = oracle.Cache(oracle.BF16, 1, 2, 512, 64)
    # dirty the cache with a padded run of a different prompt first
    q2, k2, v2 = si.gqa_prompt(L=300, Hq=4, Hkv=2, D=64, seed=25)
    oracle.prefill_chunked_padded(c, 0, si.storage(q2), si.storage(k2), si.storage(v2), 128)
    c.rewind(0, 0)
    out_dirty, _ = oracle.prefill_chunked_padded(c, 0, q, k, v, 128)
    clean = oracle.Cache(oracle.BF16, 1, 2, 512, 64)
    out_clean, _ = oracle.prefill_chunked(clean, 0, q, k, v, 128)
    assert np.array_equal(out_dirty, out_clean)


def test_rewind_rejects_growth():
    c = oracle.Cache(oracle.BF16, 1, 1, 8, 4)
    with pytest.raises(ValueError):
        c.rewind(0, 1)


# ----------------------------------------------------------------- rolling

def test_roll_append_matches_torch_cat():
    r = _rng(31)
    H, C, c, D = 3, 10, 4, 5
    old = r.integers(0, 60000, (H, C, D), dtype=np.uint16)
    chunk = r.integers(0, 60000, (c, H, D), dtype=np.uint16)
    got = oracle.roll_append(old, chunk, oracle.F16)
    t_old = torch.from_numpy(old.astype(np.int32))[None]
    t_new = torch.from_numpy(chunk.astype(np.int32)).permute(1, 0, 2)[None]
    ref = torch.cat([t_old, t_new], dim=2)[:, :, c:][0].numpy().astype(np.uint16)
    assert np.array_equal(got, ref)


def test_rolling_with_room_equals_plain_causal_prefill():
    """C >= L: nothing is evicted, so the real rows equal ordinary causal
    prefill over the real tokens (Horizon blog, section 3)."""
    q, k, v = si.rolling_inputs(L=200, H=2, D=16, seed=32)
    q, k, v = (si.storage(x) for x in (q, k, v))
    out, n_left, _, _, _ = oracle.roll_prefill(q, k, v, C=256, c=64, dtype=oracle.F16)
    assert n_left == 56
    ref = _causal_oracle(oracle.widen(q, oracle.F16), oracle.widen(k, oracle.F16),
                         oracle.widen(v, oracle.F16))
    assert np.array_equal(out[n_left:], ref)
    qt, kt, vt = si.rolling_inputs(L=200, H=2, D=16, seed=32)
    assert np.max(np.abs(out[n_left:] - _sdpa64(qt, kt, vt))) < 1e-12


def test_rolling_past_capacity_is_a_sliding_window():
    """L > C: chunk j's rows see absolute keys [max(0,(j+1)c - C), p]."""
    L, C, c, H, D = 256, 96, 32, 2, 8
    q, k, v = si.rolling_inputs(L=L, H=H, D=D, seed=33)
    q, k, v = (si.storage(x) for x in (q, k, v))
    out, n_left, kc, vc, _ = oracle.roll_prefill(q, k, v, C=C, c=c, dtype=oracle.F16)
    assert n_left == 0
    qd, kd, vd = (oracle.widen(x, oracle.F16) for x in (q, k, v))
    kk = np.ascontiguousarray(kd.transpose(1, 0, 2))
    vv = np.ascontiguousarray(vd.transpose(1, 0, 2))
    p = np.arange(L)
    lo = np.maximum(0, (p // c + 1) * c - C).astype(np.int32)
    ref = oracle.attention(qd, kk, vv, lo, p.astype(np.int32), oracle.default_scale(D))
    assert np.max(np.abs(out - ref)) < 1e-14
    # the same window as a boolean mask for torch's SDPA (library pin)
    qt, kt, vt = si.rolling_inputs(L=L, H=H, D=D, seed=33)
    a = np.arange(L)[None, :]
    vis = (a <= p[:, None]) & (a >= lo[:, None])
    assert np.max(np.abs(out - _sdpa64(qt, kt, vt, vis))) < 1e-12
    # the final cache holds the last C positions, right-aligned
    assert np.array_equal(kc, k[L - C:].transpose(1, 0, 2))


def test_rolling_mask_shape_and_right_alignment():
    m = oracle.chunk_mask(Lp=512, n_leftpad=24, j=0, c=256, C=2048)
    assert m.shape == (256, 2048)
    assert np.all(m[:, :2048 - 256 + 24] == oracle.MASK_FILL)
    # left-pad query rows see nothing; the first real row sees only itself
    assert np.all(m[:24] == oracle.MASK_FILL)
    assert m[24, 2048 - 256 + 24] == 0.0 and m[24, 2048 - 256 + 25] == oracle.MASK_FILL
    assert np.all(m[255, 2048 - 256 + 24:] == 0.0)
    assert GOLD["rolling_mask_fill"]["fill"] == oracle.MASK_FILL


# ----------------------------------------------------------------- planner

def _schedule(budget, n_dec, prompt):
    steps, done = [], 0
    while done < prompt:
        r = oracle.plan_step(budget, n_dec, prompt - done)
        steps.append(r)
        done += r
    return steps


def test_planner_budget_tables():
    assert GOLD["generation_stall_prefill"]["prompt_tokens"] == 20000
    b = GOLD["budget_guidance"]
    assert _schedule(b["latency_budget"], 64, 20000) == [1984] * 10 + [160]
    assert _schedule(b["throughput_budget"], 64, 20000) == [8128, 8128, 3744]
    assert oracle.plan_step(64, 64, 100) == 0
    with pytest.raises(ValueError):
        oracle.plan_step(10, 11, 5)


def test_varlen_budgeted_steps_reproduce_one_shot_prefill():
    """A prompt fed across budgeted mixed steps (decode rows first) produces
    the same prompt outputs as one-shot prefill, and each decode row equals a
    one-row chunk at its context."""
    D, Hq, Hkv = 32, 4, 2
    q, k, v = si.gqa_prompt(L=230, Hq=Hq, Hkv=Hkv, D=D, seed=41)
    q, k, v = (si.storage(x) for x in (q, k, v))
    ctxs = [17, 40, 5]
    rr = _rng(42)
    cache = oracle.Cache(oracle.BF16, 4, Hkv, 512, D)
    ref_cache = oracle.Cache(oracle.BF16, 4, Hkv, 512, D)
    for s, n in enumerate(ctxs):
        kk = rr.integers(0x3c00, 0x4000, (n, Hkv, D), dtype=np.uint16)
        for cc in (cache, ref_cache):
            cc.append(s, kk, kk, 0)
    budget, done, step = 64, 0, 0
    prompt_outs = []
    lens = list(ctxs)
    while done < 230:
        rows = oracle.plan_step(budget, len(ctxs), 230 - done)
        dq = rr.integers(0x3c00, 0x4000, (len(ctxs), Hq, D), dtype=np.uint16)
        dk = rr.integers(0x3c00, 0x4000, (len(ctxs), Hkv, D), dtype=np.uint16)
        pq = np.concatenate([dq, q[done:done + rows]])
        pk = np.concatenate([dk, k[done:done + rows]])
        pv = np.concatenate([dk, v[done:done + rows]])
        cu = list(range(len(ctxs) + 1)) + [len(ctxs) + rows]
        seqs = [(s, lens[s]) for s in range(len(ctxs))] + [(3, done)]
        outs = oracle.varlen_step(cache, seqs, pq, pk, pv, cu)
        for s in range(len(ctxs)):
            ref_cache.append(s, dk[s:s + 1], dk[s:s + 1], lens[s])
            ref = oracle.attend_from_cache(ref_cache, s, dq[s:s + 1], lens[s])
            assert np.array_equal(outs[s], ref)
            lens[s] += 1
        prompt_outs.append(outs[-1])
        done += rows
        step += 1
    assert step == 4
    one = oracle.prefill_one_shot(oracle.Cache(oracle.BF16, 1, Hkv, 512, D), 0, q, k, v)
    assert np.array_equal(np.concatenate(prompt_outs), one)


# --------------------------------------------------- planted mistakes (CPU)

def _demo_small():
    _, (qt, kt, vt) = si.demo_qkv()
    q, k, v = (x[:96].double().numpy() for x in (qt, kt, vt))
    ref = F.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v)), is_causal=True)
    return q, k, v, ref[0].permute(1, 0, 2).numpy()


def _fails(got, ref, tol=1e-5):
    return np.isnan(got).any() or np.max(np.abs(got - ref)) > tol


def test_planted_off_by_one_causal_bound_is_caught():
    q, k, v, ref = _demo_small()
    kk, vv = (np.ascontiguousarray(x.transpose(1, 0, 2)) for x in (k, v))
    L = q.shape[0]
    for hi in (np.arange(L) - 1, np.minimum(np.arange(L) + 1, L - 1)):
        got = oracle.attention(q, kk, vv, np.zeros(L, np.int32), np.maximum(hi, 0).astype(np.int32),
                               oracle.default_scale(64))
        assert _fails(got, ref)


def test_planted_missing_scale_is_caught():
    q, k, v, ref = _demo_small()
    assert _fails(_causal_oracle(q, k, v, scale=1.0), ref)


def test_planted_transposed_operand_is_caught():
    q, k, v, ref = _demo_small()
    assert _fails(_causal_oracle(q, v, k), ref)


def test_planted_wrong_gqa_mapping_is_caught():
    r = _rng(5)
    L, Hq, Hkv, D = 40, 8, 2, 16
    q = r.standard_normal((L, Hq, D))
    k = r.standard_normal((L, Hkv, D))
    v = r.standard_normal((L, Hkv, D))
    # interleaved mapping h % Hkv instead of contiguous groups h // G
    perm = np.array([h % Hkv * (Hq // Hkv) + h // Hkv for h in range(Hq)])
    wrong = _causal_oracle(q[:, perm], k, v)[:, np.argsort(perm)]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2).numpy()
    assert _fails(wrong, ref)


def test_planted_wrong_roll_slice_is_caught():
    r = _rng(31)
    H, C, c, D = 2, 8, 3, 4
    old = r.integers(0, 60000, (H, C, D), dtype=np.uint16)
    chunk = r.integers(0, 60000, (c, H, D), dtype=np.uint16)
    t_old = torch.from_numpy(old.astype(np.int32))[None]
    t_new = torch.from_numpy(chunk.astype(np.int32)).permute(1, 0, 2)[None]
    ref = torch.cat([t_old, t_new], dim=2)[:, :, c:][0].numpy().astype(np.uint16)
    wrong = torch.cat([t_old, t_new], dim=2)[:, :, :C][0].numpy().astype(np.uint16)
    assert not np.array_equal(wrong, ref)
    assert np.array_equal(oracle.roll_append(old, chunk, oracle.F16), ref)


# planted mistakes in the cache-driven entry points (the reference the GPU
# tests compare against): each must break the SDPA pin

def _entry_point_error():
    qt, kt, vt = si.gqa_prompt(L=96, Hq=4, Hkv=2, D=32, seed=25)
    q, k, v = (si.storage(x) for x in (qt, kt, vt))
    ref = _sdpa64(qt, kt, vt)
    outs = [oracle.prefill_one_shot(oracle.Cache(oracle.BF16, 1, 2, 128, 32), 0, q, k, v),
            oracle.prefill_chunked(oracle.Cache(oracle.BF16, 1, 2, 128, 32), 0, q, k, v, 40)[0]]
    return max(float(np.nanmax(np.abs(o - ref))) if not np.isnan(o).any() else np.inf
               for o in outs)


def test_entry_point_pin_is_clean():
    assert _entry_point_error() < 1e-12


def test_planted_cache_path_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "default_scale", lambda D: 1.0 / D)
    assert _entry_point_error() > 1e-5


@pytest.mark.parametrize("shift", [-1, 1])
def test_planted_cache_path_key_bound_is_caught(monkeypatch, shift):
    real = oracle.attention

    def shifted(q, k, v, lo, hi, scale, addmask=None):
        hi = np.clip(np.asarray(hi) + shift, 0, k.shape[1] - 1).astype(np.int32)
        return real(q, k, v, lo, hi, scale, addmask)

    monkeypatch.setattr(oracle, "attention", shifted)
    assert _entry_point_error() > 1e-5


def test_planted_cache_append_swapping_k_and_v_is_caught(monkeypatch):
    real = oracle.Cache.append
    monkeypatch.setattr(oracle.Cache, "append",
                        lambda self, b, k, v, past: real(self, b, v, k, past))
    assert _entry_point_error() > 1e-5


def test_planted_cache_append_one_row_late_is_caught(monkeypatch):
    real = oracle.Cache.append

    def late(self, b, k, v, past):
        real(self, b, k, v, past + 1)
        self.lens[b] = past + k.shape[0]

    monkeypatch.setattr(oracle.Cache, "append", late)
    assert _entry_point_error() > 1e-5
