"""CPU oracle for chunked-prefill causal attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``chunked_prefill_causal_kv_amd``) and never
imports it; the two meet only in the seeded input generator
(``synth_inputs``), which holds no attention arithmetic.

The arithmetic is plain fp64 C (``orc.c``); the drivers here follow the
pages' steps in their order:

* chunk split, append-only cache, causal mask over absolute positions:
  ONNX GenAI Wiki "Chunked Prefill", sections 1 (1.1 append-only cache,
  1.2 causal mask, 1.3 capacity kept apart from length), 2 and 3;
* query-axis padding ladder, pad rows, truncation and rewind: same page,
  sections 4 and 6;
* rolling right-aligned cache and its (c, C) additive mask: Horizon
  developer blog "Chunk Prefill", sections 3, 4 and 5;
* token-budget step planner: Ultralytics glossary "Chunked Prefill",
  section "how chunked prefill works".

Parity status of each function is listed in ``PINS`` below; every entry is
pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")

F32, F16, BF16 = 0, 1, 2
ELEM_SIZE = {F32: 4, F16: 2, BF16: 2}
STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

# The pages' additive mask fill (Horizon blog "Chunk Prefill", sections 4 and
# the follow-up note): masked entries hold -32768 rather than -inf.
MASK_FILL = -32768.0

PINS = {
    "attention": "pinned: torch SDPA (library), brute force with math.fsum, "
                 "closed forms (prefix means, first row, uniform, dominant)",
    "kv_append": "pinned: cache prefix invariant and byte equality with inputs",
    "attend_from_cache / prefill_one_shot": "pinned: torch SDPA in fp64 (library) on the "
                 "fp32 demo and on GQA bf16 storage; planted scale, key-bound, K/V swap "
                 "and late-append mistakes break the pin",
    "prefill_chunked": "pinned: torch SDPA in fp64 (library), equals one-shot (bitwise), "
                       "demo split 256/256/256/232",
    "prefill_chunk_padded": "pinned: torch SDPA in fp64 (library); padded real rows equal "
                            "unpadded rows (bitwise)",
    "ladder": "pinned: printed rungs {171,342,512}, 113->171, 176->342, 311->342",
    "split_chunks": "pinned: printed splits 1137 and 1200 at W=512, demo 1000/256",
    "roll_append": "pinned: torch.cat(...)[:, c:] (library)",
    "roll_prefill": "pinned: C >= L equals plain causal prefill; L > C equals "
                    "a sliding window over absolute positions",
    "plan_step": "pinned: decode-first budget rule, hand-computed step tables",
    "varlen_step": "pinned: torch SDPA with a position mask (library); equals "
                   "per-sequence calls; decode row equals rows=1",
    "fully-masked rows": "parity unpinned (no defined result; excluded)",
}


def build(force: bool = False) -> str:
    """Compile orc.c into liborc.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", _LIB_PATH, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = I
        lib.orc_set_num_threads.argtypes = [I]
        lib.orc_set_num_threads.restype = None
        lib.orc_widen.argtypes = [P, I, I64, P]
        lib.orc_widen.restype = I
        lib.orc_attention.argtypes = [P, I, I, P, P, I, I, I, P, P, P, D, P]
        lib.orc_attention.restype = I
        lib.orc_kv_append.argtypes = [P, P, I, I, I, I, P, P, I, I]
        lib.orc_kv_append.restype = I
        lib.orc_roll_append.argtypes = [P, P, P, I, I, I, I, I]
        lib.orc_roll_append.restype = I
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops use on this host."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's later loops (for timing at one thread)."""
    _load().orc_set_num_threads(int(n))


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- primitives

def widen(raw: np.ndarray, dtype: int) -> np.ndarray:
    """Stored elements (fp32 values, or fp16/bf16 bit patterns as uint16) to
    an fp64 array of the same shape, exactly."""
    raw = np.ascontiguousarray(raw)
    assert raw.dtype == STORAGE[dtype], (raw.dtype, dtype)
    out = np.empty(raw.shape, dtype=np.float64)
    rc = _load().orc_widen(_ptr(raw), dtype, raw.size, _ptr(out))
    if rc != 0:
        raise ValueError("unknown dtype")
    return out


def attention(q, k, v, lo, hi, scale, addmask=None) -> np.ndarray:
    """fp64 attention rows; see orc_attention in orc.c.

    q [n_q, Hq, D], k/v [Hkv, n_k, D] (fp64), lo/hi [n_q] inclusive key
    bounds, optional addmask [n_q, n_k]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    n_q, Hq, D = q.shape
    Hkv, n_k, Dk = k.shape
    assert Dk == D and v.shape == k.shape
    lo = np.ascontiguousarray(lo, dtype=np.int32)
    hi = np.ascontiguousarray(hi, dtype=np.int32)
    assert lo.shape == (n_q,) and hi.shape == (n_q,)
    mask_p = None
    if addmask is not None:
        addmask = np.ascontiguousarray(addmask, dtype=np.float64)
        assert addmask.shape == (n_q, n_k)
        mask_p = _ptr(addmask)
    out = np.empty((n_q, Hq, D), dtype=np.float64)
    rc = _load().orc_attention(_ptr(q), n_q, Hq, _ptr(k), _ptr(v), n_k, Hkv, D,
                               _ptr(lo), _ptr(hi), mask_p, float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("orc_attention: inconsistent sizes")
    return out


def default_scale(D: int) -> float:
    """1/sqrt(D), the scaled-dot-product default the pages' demo relies on."""
    return 1.0 / math.sqrt(D)


# -------------------------------------------------------------- host logic

def split_chunks(L: int, W: int):
    """(past_len, rows) per chunk: full W-row chunks, the last one takes the
    remainder (ONNX GenAI Wiki "Chunked Prefill", sections 2 and 3)."""
    if L < 0 or W < 1:
        raise ValueError("bad split")
    return [(start, min(W, L - start)) for start in range(0, L, W)]


def ladder_rungs(W: int):
    """Three equally spaced query widths at or below the chunk width, the step
    rounded up so that the top rung is the chunk width itself (same page,
    sections 4 and 6).  Duplicates collapse for tiny W."""
    if W < 1:
        raise ValueError("bad chunk width")
    step = -(-W // 3)
    return sorted({min(i * step, W) for i in (1, 2, 3)})


def ladder_width(W: int, rows: int) -> int:
    """Smallest rung that holds `rows` real rows."""
    if rows < 1 or rows > W:
        raise ValueError("rows out of range")
    for r in ladder_rungs(W):
        if r >= rows:
            return r
    raise AssertionError("unreachable: top rung is W")


def plan_step(budget: int, n_decode: int, prompt_remaining: int) -> int:
    """Prompt rows admitted to one step: every running decode gets its one
    token first, the waiting prompt's chunk fills what is left (Ultralytics
    glossary "Chunked Prefill", section "how chunked prefill works")."""
    if budget < 0 or n_decode < 0 or prompt_remaining < 0 or n_decode > budget:
        raise ValueError("bad plan")
    return max(0, min(budget - n_decode, prompt_remaining))


# ---------------------------------------------------------------- the cache

@dataclass
class Cache:
    """Cache bound at physical capacity, true length carried beside it
    (ONNX GenAI Wiki "Chunked Prefill", section 1.3).

    k, v: storage arrays [B, Hkv, cap, D]; lens[b]: number of valid
    positions (not count - 1)."""
    dtype: int
    batch: int
    kv_heads: int
    capacity: int
    head_dim: int
    k: np.ndarray = field(init=False)
    v: np.ndarray = field(init=False)
    lens: np.ndarray = field(init=False)

    def __post_init__(self):
        shape = (self.batch, self.kv_heads, self.capacity, self.head_dim)
        st = STORAGE[self.dtype]
        self.k = np.zeros(shape, dtype=st)
        self.v = np.zeros(shape, dtype=st)
        self.lens = np.zeros(self.batch, dtype=np.int32)

    def append(self, b: int, k_new: np.ndarray, v_new: np.ndarray, past_len: int):
        rows = k_new.shape[0]
        kb = np.ascontiguousarray(self.k[b])
        vb = np.ascontiguousarray(self.v[b])
        rc = _load().orc_kv_append(_ptr(kb), _ptr(vb), self.kv_heads, self.capacity,
                                   self.head_dim, ELEM_SIZE[self.dtype],
                                   _ptr(np.ascontiguousarray(k_new)),
                                   _ptr(np.ascontiguousarray(v_new)), past_len, rows)
        if rc != 0:
            raise ValueError("capacity exceeded")
        self.k[b] = kb
        self.v[b] = vb
        self.lens[b] = past_len + rows

    def rewind(self, b: int, new_len: int):
        """Roll the logical length back; bytes past it stay until overwritten
        (same page, section 4)."""
        if new_len < 0 or new_len > self.lens[b]:
            raise ValueError("bad rewind")
        self.lens[b] = new_len

    def valid_bytes(self, b: int):
        n = int(self.lens[b])
        return self.k[b, :, :n, :].copy(), self.v[b, :, :n, :].copy()


def attend_from_cache(cache: Cache, b: int, q_raw: np.ndarray, past_len: int,
                      rows_idx=None, scale=None) -> np.ndarray:
    """Attention of chunk rows (absolute position past_len + i) over keys
    [0, past_len + i] read from the cache (append first, then attend).

    rows_idx optionally selects a subset of the chunk's rows (sampling);
    the result has one row per selected row."""
    n_rows = q_raw.shape[0]
    if rows_idx is None:
        rows_idx = np.arange(n_rows)
    rows_idx = np.asarray(rows_idx, dtype=np.int64)
    n_keys = past_len + (int(rows_idx.max()) + 1 if len(rows_idx) else 0)
    if n_keys > cache.capacity:
        raise ValueError("keys beyond capacity")
    q = widen(np.ascontiguousarray(q_raw[rows_idx]), cache.dtype)
    k = widen(np.ascontiguousarray(cache.k[b, :, :n_keys, :]), cache.dtype)
    v = widen(np.ascontiguousarray(cache.v[b, :, :n_keys, :]), cache.dtype)
    lo = np.zeros(len(rows_idx), dtype=np.int32)
    hi = (past_len + rows_idx).astype(np.int32)
    s = default_scale(cache.head_dim) if scale is None else scale
    return attention(q, k, v, lo, hi, s)


def prefill_one_shot(cache: Cache, b: int, q, k, v, rows_idx=None, scale=None):
    """The whole prompt as one forward: append all rows, attend all rows."""
    cache.append(b, k, v, 0)
    return attend_from_cache(cache, b, q, 0, rows_idx, scale)


def prefill_chunked(cache: Cache, b: int, q, k, v, W: int, scale=None):
    """Chunk loop: for each chunk, append its K/V at [past, past + rows), then
    attend its rows over [0, past + i].  Returns (out, chunks)."""
    L = q.shape[0]
    outs = []
    chunks = split_chunks(L, W)
    for past, rows in chunks:
        sl = slice(past, past + rows)
        cache.append(b, k[sl], v[sl], past)
        outs.append(attend_from_cache(cache, b, q[sl], past, scale=scale))
    return np.concatenate(outs, axis=0), chunks


def _pad_rows(x: np.ndarray, width: int) -> np.ndarray:
    """Widen a token-major [rows, ...] array to `width` rows by repeating its
    last real row (ONNX GenAI Wiki "Chunked Prefill", section 4)."""
    rows = x.shape[0]
    if width == rows:
        return x
    tail = np.repeat(x[rows - 1:rows], width - rows, axis=0)
    return np.concatenate([x, tail], axis=0)


def prefill_chunk_padded(cache: Cache, b: int, q, k, v, past_len: int, W: int,
                         scale=None):
    """One padded prefill forward, literally: round the rows up the ladder,
    duplicate the last real row into q, k and v, append every padded row,
    attend every padded row, keep only the real rows, then rewind the cache
    to past_len + real rows.  Returns (real-row outputs, padded width)."""
    real = q.shape[0]
    width = ladder_width(W, real)
    qp, kp, vp = _pad_rows(q, width), _pad_rows(k, width), _pad_rows(v, width)
    cache.append(b, kp, vp, past_len)
    out = attend_from_cache(cache, b, qp, past_len, scale=scale)
    cache.rewind(b, past_len + real)
    return out[:real], width


def prefill_chunked_padded(cache: Cache, b: int, q, k, v, W: int, scale=None):
    """Chunk loop with query-axis padding on every prefill forward."""
    outs, widths = [], []
    for past, rows in split_chunks(q.shape[0], W):
        sl = slice(past, past + rows)
        o, w = prefill_chunk_padded(cache, b, q[sl], k[sl], v[sl], past, W, scale)
        outs.append(o)
        widths.append(w)
    return np.concatenate(outs, axis=0), widths


# ------------------------------------------------------------------ rolling

def roll_append(old: np.ndarray, chunk: np.ndarray, dtype: int) -> np.ndarray:
    """new = cat(old, chunk)[c:] for one sequence: old [H, C, D] storage,
    chunk token-major [c, H, D]."""
    H, C, D = old.shape
    c = chunk.shape[0]
    out = np.empty_like(old)
    rc = _load().orc_roll_append(_ptr(np.ascontiguousarray(old)),
                                 _ptr(np.ascontiguousarray(chunk)), _ptr(out),
                                 H, C, c, D, ELEM_SIZE[dtype])
    if rc != 0:
        raise ValueError("chunk longer than the cache")
    return out


def full_additive_mask(Lp: int, n_leftpad: int) -> np.ndarray:
    """[Lp, Lp] additive mask of a left-padded sequence: 0 where query p may
    see key a (a <= p and a is not a pad position), the fill value
    elsewhere."""
    p = np.arange(Lp)[:, None]
    a = np.arange(Lp)[None, :]
    ok = (a <= p) & (a >= n_leftpad)
    return np.where(ok, 0.0, MASK_FILL)


def chunk_mask(Lp: int, n_leftpad: int, j: int, c: int, C: int) -> np.ndarray:
    """The (c, C) mask of chunk j, built as the Horizon blog's section 4
    describes: slice the chunk's c query rows out of the full mask (keys up to
    the chunk's end), then right-align the key axis to C, filling the left
    with the mask fill value (or keeping only the last C keys once the
    sequence is longer than C)."""
    full = full_additive_mask(Lp, n_leftpad)
    end = (j + 1) * c
    rows = full[j * c:end, :end]
    if end >= C:
        return np.ascontiguousarray(rows[:, end - C:])
    pad = np.full((c, C - end), MASK_FILL)
    return np.concatenate([pad, rows], axis=1)


def left_pad_amount(L: int, c: int) -> int:
    """Left padding that brings L up to a multiple of the chunk size (the
    page's alignment step; the cap to the cache size is not applied)."""
    return (-L) % c


def roll_prefill(q, k, v, C: int, c: int, dtype: int, scale=None,
                 explicit_masks=None):
    """Rolling fixed-capacity prefill of one sequence, literally.

    q [L, Hq, D], k/v [L, Hkv, D] storage arrays of the real tokens.  The
    sequence is left-padded with zero rows to a multiple of c; each chunk
    rolls its K/V into the C-slot caches (initially zero) and then attends
    over all C slots with the chunk's additive mask.  Returns
    (out [Lp, Hq, D] fp64 over the padded sequence, n_leftpad, final k, v
    caches [Hkv, C, D], list of per-chunk masks)."""
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    n_left = left_pad_amount(L, c)
    Lp = L + n_left

    def lpad(x):
        z = np.zeros((n_left,) + x.shape[1:], dtype=x.dtype)
        return np.concatenate([z, x], axis=0)

    qp, kp, vp = lpad(q), lpad(k), lpad(v)
    kc = np.zeros((Hkv, C, D), dtype=STORAGE[dtype])
    vc = np.zeros((Hkv, C, D), dtype=STORAGE[dtype])
    s = default_scale(D) if scale is None else scale
    outs, masks = [], []
    for j in range(Lp // c):
        sl = slice(j * c, (j + 1) * c)
        kc = roll_append(kc, kp[sl], dtype)
        vc = roll_append(vc, vp[sl], dtype)
        m = chunk_mask(Lp, n_left, j, c, C)
        masks.append(m)
        qq = widen(np.ascontiguousarray(qp[sl]), dtype)
        lo = np.zeros(c, dtype=np.int32)
        hi = np.full(c, C - 1, dtype=np.int32)
        outs.append(attention(qq, widen(kc, dtype), widen(vc, dtype), lo, hi, s,
                              addmask=m))
    return np.concatenate(outs, axis=0), n_left, kc, vc, masks


# ------------------------------------------------------------------- varlen

def varlen_step(cache: Cache, seqs, q, k_new, v_new, cu_rows, scale=None,
                rows_idx=None):
    """One packed step, sequence by sequence: seqs is a list of
    (slot, past_len); rows cu_rows[s]:cu_rows[s+1] of the packed q/k/v belong
    to sequence s.  Each sequence appends its rows and attends them, exactly
    as a separate call would.  rows_idx optionally maps a sequence index to
    a subset of its rows to evaluate.  Returns a list of per-sequence
    outputs."""
    outs = []
    for s, (slot, past) in enumerate(seqs):
        a, b = int(cu_rows[s]), int(cu_rows[s + 1])
        cache.append(slot, k_new[a:b], v_new[a:b], past)
        sel = None if rows_idx is None else rows_idx.get(s)
        outs.append(attend_from_cache(cache, slot, q[a:b], past, sel, scale))
    return outs
