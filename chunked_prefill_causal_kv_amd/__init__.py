"""Python binding of libcpk: chunked-prefill causal attention over a KV cache
on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the path (append, attention,
rewind, rolling shift, decode, combine) runs in the HIP kernels of
``libcpk.so``; the host logic (ladder, chunk split, step planner) runs in its
C code.  PyTorch provides device memory and the current stream.  There is no
CPU fallback: importing this package fails if the library is not built.

The function names are the C ABI's (``include/cpk.h``).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, NamedTuple, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpk.so")

CPK_OK, CPK_EINVAL, CPK_EDTYPE, CPK_ECAPACITY, CPK_EALIGN, CPK_EWORKSPACE, CPK_EHIP = \
    0, -1, -2, -3, -4, -5, -6
CPK_F32, CPK_F16, CPK_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: CPK_F32, torch.float16: CPK_F16, torch.bfloat16: CPK_BF16}
DECODE_SEGMENT = 256


class CpkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cpk status {status}: {message}")
        self.status = status


class cpk_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class cpk_paged_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python chunked_prefill_causal_kv_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    IP = ctypes.POINTER(ctypes.c_int)
    I32P = ctypes.POINTER(ctypes.c_int32)
    CP = ctypes.POINTER(cpk_kv_cache)
    PCP = ctypes.POINTER(cpk_paged_cache)
    F = ctypes.c_float
    sig = {
        "cpk_version": ([], I),
        "cpk_set_attention_kernel": ([I], I),
        "cpk_kv_copy_prefix": ([CP, I, I, I, P], I),
        "cpk_last_error": ([], ctypes.c_char_p),
        "cpk_device_info": ([ctypes.c_char_p, I, IP], I),
        "cpk_ladder_rungs": ([I, IP, IP], I),
        "cpk_ladder_width": ([I, I, IP], I),
        "cpk_split_chunks": ([I, I, I32P, I32P, I, IP], I),
        "cpk_plan_step": ([I, I, I, IP], I),
        "cpk_kv_append": ([CP, I, P, P, I, I, I, P], I),
        "cpk_chunk_attention": ([P, CP, I, I, I, I, I, F, P, P], I),
        "cpk_rewind": ([CP, I, I, I, P], I),
        "cpk_prefill_chunk": ([P, P, P, CP, I, I, I, I, I, I, F, P, IP, P], I),
        "cpk_varlen_workspace_size": ([I, I, I, I], Z),
        "cpk_varlen_step": ([P, P, P, CP, P, P, P, I32P, I32P, I32P, I, I, I, F, P, P, Z, P], I),
        "cpk_paged_varlen_step": ([P, P, P, PCP, P, P, P, I32P, I32P, I32P, I, I, I, F, P, P, Z, I, P], I),
        "cpk_varlen_step_phases": ([P, P, P, CP, P, P, P, I32P, I32P, I32P, I, I, I, F, P, P, Z, I, P], I),
        "cpk_varlen_step_noalloc": ([P, P, P, CP, P, P, P, I32P, I32P, I32P, I, I, I, F, P, P], I),
        "cpk_roll_append": ([P, P, P, P, P, P, I, I, I, I, I, I, P], I),
        "cpk_roll_attention": ([P, P, P, P, I, I, I, I, I, I, I, I, F, P, P, Z, P], I),
        "cpk_roll_workspace_size": ([I, I, I, I, I, I], Z),
        "cpk_ring_append": ([P, P, P, P, I, I, I, I, I, I, I, P], I),
        "cpk_ring_attention": ([P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, Z, P], I),
        "cpk_ring_step": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, Z, P], I),
        "cpk_ring_step_deferred": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, Z, P,
                                    P, P], I),
        "cpk_roll_flush": ([P, Z, P, I, I, I, I, I, I, P], I),
        "cpk_roll_attention_deferred": ([P, P, P, P, I, I, I, I, I, I, I, I, F, P, P, Z, P, P,
                                         P], I),
        "cpk_ring_view": ([P, P, P, P, I, I, I, I, I, I, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(status: int):
    if status != CPK_OK:
        raise CpkError(status, _lib.cpk_last_error().decode())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcpk must be contiguous")
    return t.data_ptr()


class KVCache:
    """Device cache [batch, kv_heads, capacity, head_dim] bound at physical
    capacity, with seqlens_k on the device and a host mirror `lens`."""

    def __init__(self, batch: int, kv_heads: int, capacity: int, head_dim: int,
                 dtype=torch.bfloat16, device="cuda", k=None, v=None):
        shape = (batch, kv_heads, capacity, head_dim)
        self.k = torch.zeros(shape, dtype=dtype, device=device) if k is None else k
        self.v = torch.zeros(shape, dtype=dtype, device=device) if v is None else v
        self.seqlens_k = torch.zeros(batch, dtype=torch.int32, device=device)
        self.lens = [0] * batch
        self.dtype = dtype
        self.desc = cpk_kv_cache(self.k.data_ptr(), self.v.data_ptr(), self.seqlens_k.data_ptr(),
                                 batch, kv_heads, capacity, head_dim, DTYPE_CODE[dtype])

    @property
    def batch(self):
        return self.desc.batch

    @property
    def kv_heads(self):
        return self.desc.kv_heads

    @property
    def capacity(self):
        return self.desc.capacity

    @property
    def head_dim(self):
        return self.desc.head_dim


class PagedKVCache:
    """Paged cache: K/V pools [n_blocks, kv_heads, block_size, head_dim], a
    device block table [batch, max_blocks] (int32) that the caller fills
    (blocks may be shared between slots), seqlens_k on the device and a host
    mirror `lens`."""

    def __init__(self, batch: int, kv_heads: int, n_blocks: int, block_size: int,
                 max_blocks: int, head_dim: int, dtype=torch.bfloat16, device="cuda"):
        shape = (n_blocks, kv_heads, block_size, head_dim)
        self.k = torch.zeros(shape, dtype=dtype, device=device)
        self.v = torch.zeros(shape, dtype=dtype, device=device)
        self.block_table = torch.zeros((batch, max_blocks), dtype=torch.int32, device=device)
        self.seqlens_k = torch.zeros(batch, dtype=torch.int32, device=device)
        self.lens = [0] * batch
        self.dtype = dtype
        self.desc = cpk_paged_cache(self.k.data_ptr(), self.v.data_ptr(),
                                    self.block_table.data_ptr(), self.seqlens_k.data_ptr(),
                                    batch, kv_heads, block_size, n_blocks, max_blocks, head_dim,
                                    DTYPE_CODE[dtype])

    @property
    def block_size(self):
        return self.desc.block_size

    def gather(self, slot: int, n: int):
        """Positions [0, n) of a slot as contiguous [kv_heads, n, head_dim]
        K and V (a copy, for checks)."""
        bs = self.block_size
        nb = (n + bs - 1) // bs
        ids = self.block_table[slot, :nb].long()
        k = self.k[ids].permute(1, 0, 2, 3).reshape(self.k.shape[1], nb * bs, -1)[:, :n]
        v = self.v[ids].permute(1, 0, 2, 3).reshape(self.v.shape[1], nb * bs, -1)[:, :n]
        return k, v


# ---------------------------------------------------------------- host logic

def cpk_version() -> int:
    return _lib.cpk_version()


ATTN_AUTO, ATTN_NARROW, ATTN_WIDE, ATTN_NARROW_GENERAL = 0, 1, 2, 3


def cpk_set_attention_kernel(kind: int) -> int:
    """Process-wide bf16/fp16 attention kernel choice (ATTN_AUTO, ATTN_NARROW,
    ATTN_WIDE or ATTN_NARROW_GENERAL) for chunk and varlen attention; returns
    the previous one."""
    r = _lib.cpk_set_attention_kernel(int(kind))
    if r < 0:
        _check(r)
    return r


class attention_kernel:
    """Context manager: run a block with the given attention kernel choice."""

    def __init__(self, kind: int):
        self.kind = kind

    def __enter__(self):
        self.prev = cpk_set_attention_kernel(self.kind)
        return self

    def __exit__(self, *exc):
        cpk_set_attention_kernel(self.prev)
        return False


def cpk_last_error() -> str:
    return _lib.cpk_last_error().decode()


def cpk_device_info() -> Tuple[str, int]:
    buf = ctypes.create_string_buffer(128)
    cu = ctypes.c_int(0)
    _check(_lib.cpk_device_info(buf, 128, ctypes.byref(cu)))
    return buf.value.decode(), cu.value


def cpk_ladder_rungs(W: int) -> List[int]:
    out = (ctypes.c_int * 3)()
    n = ctypes.c_int(0)
    _check(_lib.cpk_ladder_rungs(W, out, ctypes.byref(n)))
    return list(out[:n.value])


def cpk_ladder_width(W: int, rows: int) -> int:
    w = ctypes.c_int(0)
    _check(_lib.cpk_ladder_width(W, rows, ctypes.byref(w)))
    return w.value


def cpk_split_chunks(L: int, W: int) -> List[Tuple[int, int]]:
    n = ctypes.c_int(0)
    _lib.cpk_split_chunks(L, W, None, None, 0, ctypes.byref(n))
    cnt = max(n.value, 1)
    past = (ctypes.c_int32 * cnt)()
    rows = (ctypes.c_int32 * cnt)()
    _check(_lib.cpk_split_chunks(L, W, past, rows, cnt, ctypes.byref(n)))
    return [(past[i], rows[i]) for i in range(n.value)]


def cpk_plan_step(budget: int, n_decode: int, prompt_remaining: int) -> int:
    r = ctypes.c_int(0)
    _check(_lib.cpk_plan_step(budget, n_decode, prompt_remaining, ctypes.byref(r)))
    return r.value


# -------------------------------------------------------------- device calls

def cpk_kv_append(cache: KVCache, b: int, k_new: torch.Tensor, v_new: torch.Tensor,
                  past_len: int, rows: Optional[int] = None, stream=None):
    """Append k_new/v_new [real_rows, Hkv, D] at past_len; with rows >
    real_rows the last real row is repeated into the padded positions."""
    real = k_new.shape[0]
    rows = real if rows is None else rows
    _check(_lib.cpk_kv_append(ctypes.byref(cache.desc), b, _ptr(k_new), _ptr(v_new),
                              past_len, rows, real, _stream(stream)))
    cache.lens[b] = past_len + rows


def cpk_chunk_attention(q: torch.Tensor, cache: KVCache, b: int, past_len: int,
                        rows: Optional[int] = None, scale: float = 0.0,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of q [real_rows, Hq, D] at past_len; `rows` >= real_rows
    rows are computed (padding repeats q's last row), real rows written."""
    real, Hq, D = q.shape
    rows = real if rows is None else rows
    if out is None:
        out = torch.empty((real, Hq, D), dtype=q.dtype, device=q.device)
    _check(_lib.cpk_chunk_attention(_ptr(q), ctypes.byref(cache.desc), b, Hq, past_len, rows,
                                    real, float(scale), _ptr(out), _stream(stream)))
    return out


def cpk_kv_copy_prefix(cache: KVCache, src_slot: int, dst_slot: int, length: int,
                       stream=None):
    """Positions [0, length) of src_slot copied to dst_slot; seqlens_k[dst] = length."""
    _check(_lib.cpk_kv_copy_prefix(ctypes.byref(cache.desc), src_slot, dst_slot, length,
                                   _stream(stream)))
    cache.lens[dst_slot] = length


def cpk_rewind(cache: KVCache, b: int, new_len: int, stream=None):
    _check(_lib.cpk_rewind(ctypes.byref(cache.desc), b, new_len, cache.lens[b], _stream(stream)))
    cache.lens[b] = new_len


def cpk_prefill_chunk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cache: KVCache, b: int,
                      past_len: int, W: int, pad: bool = True, scale: float = 0.0,
                      out: Optional[torch.Tensor] = None, stream=None):
    """One padded forward; returns (out [real_rows, Hq, D], issued width)."""
    real, Hq, D = q.shape
    if out is None:
        out = torch.empty((real, Hq, D), dtype=q.dtype, device=q.device)
    width = ctypes.c_int(0)
    _check(_lib.cpk_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(cache.desc), b, Hq,
                                  past_len, real, W, 1 if pad else 0, float(scale), _ptr(out),
                                  ctypes.byref(width), _stream(stream)))
    cache.lens[b] = past_len + real
    return out, width.value


def cpk_varlen_workspace_size(n_seqs: int, q_heads: int, max_ctx: int, head_dim: int) -> int:
    return int(_lib.cpk_varlen_workspace_size(n_seqs, q_heads, max_ctx, head_dim))


PHASE_APPEND, PHASE_DECODE, PHASE_PREFILL, PHASE_ALL = 1, 2, 4, 7


def cpk_varlen_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache,
                    slots: Sequence[int], cu_rows: Sequence[int], past_lens: Sequence[int],
                    scale: float = 0.0, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, dev_meta: Optional[torch.Tensor] = None,
                    stream=None, phases: int = PHASE_ALL) -> torch.Tensor:
    """One packed mixed step (or the given phases of it) over a KVCache or a
    PagedKVCache.  slots/cu_rows/past_lens are host sequences; their device copies go in dev_meta (int32
    [3*n+1], built here if not given)."""
    n = len(slots)
    total, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    h_slots = (ctypes.c_int32 * n)(*slots)
    h_cu = (ctypes.c_int32 * (n + 1))(*cu_rows)
    h_past = (ctypes.c_int32 * n)(*past_lens)
    if dev_meta is None:
        dev_meta = torch.tensor(list(slots) + list(cu_rows) + list(past_lens),
                                dtype=torch.int32).to(q.device)
    base = dev_meta.data_ptr()
    d_slots, d_cu, d_past = base, base + 4 * n, base + 4 * (2 * n + 1)
    max_ctx = max([p + 1 for p, a, b in zip(past_lens, cu_rows[:-1], cu_rows[1:]) if b - a == 1],
                  default=0)
    need = cpk_varlen_workspace_size(n, Hq, max_ctx, D)
    if ws is None:
        ws = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    ws_bytes = ws.numel() * ws.element_size()
    fn = (_lib.cpk_paged_varlen_step if isinstance(cache, PagedKVCache)
          else _lib.cpk_varlen_step_phases)
    _check(fn(_ptr(q), _ptr(k_new), _ptr(v_new), ctypes.byref(cache.desc), d_slots, d_cu,
              d_past, h_slots, h_cu, h_past, n, total, Hq, float(scale), _ptr(out), _ptr(ws),
              ws_bytes, int(phases), _stream(stream)))
    if phases & PHASE_APPEND:
        for s, slot in enumerate(slots):
            cache.lens[slot] = past_lens[s] + cu_rows[s + 1] - cu_rows[s]
    return out


NOALLOC_SCRATCH_BYTES = 96 << 20


def cpk_varlen_step_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            cache: KVCache, slots: Sequence[int], cu_rows: Sequence[int],
                            past_lens: Sequence[int], scale: float = 0.0,
                            out: Optional[torch.Tensor] = None, dev_meta: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """cpk_varlen_step with the decode partials in the library's static
    device scratch (no workspace, no allocation inside the call; out and
    dev_meta, if given, are the caller's)."""
    n = len(slots)
    total, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    h_slots = (ctypes.c_int32 * n)(*slots)
    h_cu = (ctypes.c_int32 * (n + 1))(*cu_rows)
    h_past = (ctypes.c_int32 * n)(*past_lens)
    if dev_meta is None:
        dev_meta = torch.tensor(list(slots) + list(cu_rows) + list(past_lens),
                                dtype=torch.int32).to(q.device)
    base = dev_meta.data_ptr()
    d_slots, d_cu, d_past = base, base + 4 * n, base + 4 * (2 * n + 1)
    _check(_lib.cpk_varlen_step_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), ctypes.byref(cache.desc),
                                        d_slots, d_cu, d_past, h_slots, h_cu, h_past, n, total, Hq,
                                        float(scale), _ptr(out), _stream(stream)))
    for s, slot in enumerate(slots):
        cache.lens[slot] = past_lens[s] + cu_rows[s + 1] - cu_rows[s]
    return out


def cpk_varlen_step_phases(q, k_new, v_new, cache: KVCache, slots, cu_rows, past_lens,
                           phases: int, scale: float = 0.0, out=None, ws=None, dev_meta=None,
                           stream=None):
    """The given phases (PHASE_APPEND | PHASE_DECODE | PHASE_PREFILL) of a
    packed mixed step."""
    return cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, scale, out, ws,
                           dev_meta, stream, phases)


def cpk_paged_varlen_step(q, k_new, v_new, cache: PagedKVCache, slots, cu_rows, past_lens,
                          phases: int = PHASE_ALL, scale: float = 0.0, out=None, ws=None,
                          dev_meta=None, stream=None):
    """A packed mixed step (or the given phases) over a paged cache."""
    assert isinstance(cache, PagedKVCache)
    return cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, scale, out, ws,
                           dev_meta, stream, phases)


def varlen_step_overlapped(q, k_new, v_new, cache: KVCache, slots, cu_rows, past_lens,
                           side_stream, scale: float = 0.0, out=None, ws=None, dev_meta=None):
    """One packed mixed step with the decode rows and the prompt rows on two
    streams: append + decode on the current stream, the prompt attention on
    side_stream after the append; the current stream then waits for it.
    Same outputs as cpk_varlen_step, bit for bit."""
    if out is None:
        out = torch.empty_like(q)
    if dev_meta is None:
        dev_meta = torch.tensor(list(slots) + list(cu_rows) + list(past_lens),
                                dtype=torch.int32).to(q.device)
    main = torch.cuda.current_stream()
    cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, scale, out, ws, dev_meta,
                    phases=PHASE_APPEND)
    side_stream.wait_stream(main)
    with torch.cuda.stream(side_stream):
        cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, scale, out, ws,
                        dev_meta, phases=PHASE_PREFILL)
    cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, scale, out, ws, dev_meta,
                    phases=PHASE_DECODE)
    main.wait_stream(side_stream)
    return out


def cpk_roll_append(k_old, v_old, k_chunk, v_chunk, k_new, v_new, stream=None):
    """new = cat(old, chunk)[c:]; caches [B, H, C, D], chunks [B, c, H, D]."""
    B, H, C, D = k_old.shape
    c = k_chunk.shape[1]
    _check(_lib.cpk_roll_append(_ptr(k_old), _ptr(v_old), _ptr(k_chunk), _ptr(v_chunk),
                                _ptr(k_new), _ptr(v_new), B, H, C, c, D,
                                DTYPE_CODE[k_old.dtype], _stream(stream)))


def cpk_roll_workspace_size(Hq: int, Hkv: int, C: int, c: int, head_dim: int, dtype) -> int:
    return int(_lib.cpk_roll_workspace_size(Hq, Hkv, C, c, head_dim, DTYPE_CODE[dtype]))


_roll_ws = {}


def _roll_workspace(nbytes: int, device, index: int = 0) -> Optional[torch.Tensor]:
    """A reusable device workspace of at least nbytes (None for 0); index
    selects one of several (a deferred ring chain alternates two)."""
    if nbytes == 0:
        return None
    key = (torch.device(device), index)
    ws = _roll_ws.get(key)
    if ws is None or ws.numel() * 4 < nbytes:
        ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=key[0])
        _roll_ws[key] = ws
    return ws


def cpk_roll_attention(q, k, v, abs_end: int, n_leftpad: int, mask=None, scale: float = 0.0,
                       out=None, stream=None, split: bool = True):
    """q [c, Hq, D] over a rolling cache k/v [Hkv, C, D].  split=True passes
    a workspace (the key range is split across workgroups when the shapes
    call for it); split=False runs the unsplit kernel alone."""
    c, Hq, D = q.shape
    Hkv, C, _ = k.shape
    if out is None:
        out = torch.empty_like(q)
    ws = None
    if split:
        ws = _roll_workspace(cpk_roll_workspace_size(Hq, Hkv, C, c, D, q.dtype), q.device)
    ws_bytes = 0 if ws is None else ws.numel() * 4
    _check(_lib.cpk_roll_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), abs_end, n_leftpad,
                                   Hq, Hkv, C, c, D, DTYPE_CODE[q.dtype], float(scale),
                                   _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def cpk_ring_append(k_chunk, v_chunk, k_ring, v_ring, start: int, stream=None) -> int:
    """Write chunk rows [B, c, H, D] over the c oldest slots of rings
    [B, H, C, D] whose logical slot 0 is physical `start`; returns the new
    start (start + c) mod C."""
    B, H, C, D = k_ring.shape
    c = k_chunk.shape[1]
    _check(_lib.cpk_ring_append(_ptr(k_chunk), _ptr(v_chunk), _ptr(k_ring), _ptr(v_ring), B, H,
                                C, c, D, DTYPE_CODE[k_ring.dtype], start, _stream(stream)))
    return (start + c) % C


def cpk_ring_attention(q, k_ring, v_ring, abs_end: int, n_leftpad: int, start: int, mask=None,
                       scale: float = 0.0, out=None, stream=None, split: bool = True):
    """cpk_roll_attention over a ring k/v [Hkv, C, D] with logical slot 0 at
    physical `start`."""
    c, Hq, D = q.shape
    Hkv, C, _ = k_ring.shape
    if out is None:
        out = torch.empty_like(q)
    ws = None
    if split:
        ws = _roll_workspace(cpk_roll_workspace_size(Hq, Hkv, C, c, D, q.dtype), q.device)
    ws_bytes = 0 if ws is None else ws.numel() * 4
    _check(_lib.cpk_ring_attention(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(mask), abs_end,
                                   n_leftpad, Hq, Hkv, C, c, D, DTYPE_CODE[q.dtype],
                                   float(scale), start, _ptr(out), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    return out


def cpk_ring_step(q, k_chunk, v_chunk, k_ring, v_ring, abs_end: int, n_leftpad: int,
                  start: int, mask=None, scale: float = 0.0, out=None, stream=None,
                  split: bool = True):
    """cpk_ring_append then cpk_ring_attention at the advanced start, in one
    launch (bf16/fp16): chunk rows [c, Hkv, D], rings [Hkv, C, D].  Returns
    (out, new start)."""
    c, Hq, D = q.shape
    Hkv, C, _ = k_ring.shape
    if out is None:
        out = torch.empty_like(q)
    ws = None
    if split:
        ws = _roll_workspace(cpk_roll_workspace_size(Hq, Hkv, C, c, D, q.dtype), q.device)
    ws_bytes = 0 if ws is None else ws.numel() * 4
    _check(_lib.cpk_ring_step(_ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(k_ring), _ptr(v_ring),
                              _ptr(mask), abs_end, n_leftpad, Hq, Hkv, C, c, D,
                              DTYPE_CODE[q.dtype], float(scale), start, _ptr(out), _ptr(ws),
                              ws_bytes, _stream(stream)))
    return out, (start + c) % C


class RollPending(NamedTuple):
    """Parts a deferred rolling call left unmerged: merged into `out` by the
    next deferred call (passed as prev) or by cpk_roll_flush."""
    ws: torch.Tensor
    out: torch.Tensor
    Hq: int
    Hkv: int
    C: int
    c: int


def cpk_ring_step_deferred(q, k_chunk, v_chunk, k_ring, v_ring, abs_end: int, n_leftpad: int,
                           start: int, ws, prev: Optional[RollPending] = None, mask=None,
                           scale: float = 0.0, out=None, stream=None):
    """cpk_ring_step whose key-range parts stay in ws (a workspace of
    cpk_roll_workspace_size bytes; the previous call's must be another) and
    are merged into out by the next deferred call or cpk_roll_flush; this
    launch merges prev's parts.  Returns (pending, new start)."""
    c, Hq, D = q.shape
    Hkv, C, _ = k_ring.shape
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.cpk_ring_step_deferred(
        _ptr(q), _ptr(k_chunk), _ptr(v_chunk), _ptr(k_ring), _ptr(v_ring), _ptr(mask), abs_end,
        n_leftpad, Hq, Hkv, C, c, D, DTYPE_CODE[q.dtype], float(scale), start, _ptr(out),
        _ptr(ws), ws.numel() * ws.element_size(), None if prev is None else _ptr(prev.ws),
        None if prev is None else _ptr(prev.out), _stream(stream)))
    return RollPending(ws, out, Hq, Hkv, C, c), (start + c) % C


def cpk_roll_attention_deferred(q, k, v, abs_end: int, n_leftpad: int, ws,
                                prev: Optional[RollPending] = None, mask=None, scale: float = 0.0,
                                out=None, stream=None):
    """cpk_roll_attention over the literal cache k/v [Hkv, C, D] whose
    key-range parts stay in ws (cpk_roll_workspace_size bytes; the previous
    call's must be another) and are merged into out by the next deferred
    call or cpk_roll_flush; this launch merges prev's parts.  Returns the
    pending merge."""
    c, Hq, D = q.shape
    Hkv, C, _ = k.shape
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.cpk_roll_attention_deferred(
        _ptr(q), _ptr(k), _ptr(v), _ptr(mask), abs_end, n_leftpad, Hq, Hkv, C, c, D,
        DTYPE_CODE[q.dtype], float(scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        None if prev is None else _ptr(prev.ws), None if prev is None else _ptr(prev.out),
        _stream(stream)))
    return RollPending(ws, out, Hq, Hkv, C, c)


def cpk_roll_flush(pending: RollPending, stream=None) -> torch.Tensor:
    """Merge the parts a deferred ring step left pending; returns its out."""
    ws, out = pending.ws, pending.out
    _check(_lib.cpk_roll_flush(_ptr(ws), ws.numel() * ws.element_size(), _ptr(out), pending.Hq,
                               pending.Hkv, pending.C, pending.c, out.shape[2],
                               DTYPE_CODE[out.dtype], _stream(stream)))
    return out


def cpk_ring_view(k_ring, v_ring, start: int, k_out=None, v_out=None, stream=None):
    """The logical (literal-shift) view of rings [B, H, C, D]."""
    B, H, C, D = k_ring.shape
    k_out = torch.empty_like(k_ring) if k_out is None else k_out
    v_out = torch.empty_like(v_ring) if v_out is None else v_out
    _check(_lib.cpk_ring_view(_ptr(k_ring), _ptr(v_ring), _ptr(k_out), _ptr(v_out), B, H, C, D,
                              DTYPE_CODE[k_ring.dtype], start, _stream(stream)))
    return k_out, v_out


# ------------------------------------------------------------------- drivers

def prefill_chunked(cache: KVCache, b: int, q, k, v, W: int, pad: bool = True,
                    scale: float = 0.0, out=None, stream=None):
    """Chunked prefill of a whole prompt into sequence b: split by the
    library, one padded forward per chunk.  Returns (out, widths)."""
    L, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    widths = []
    for past, rows in cpk_split_chunks(L, W):
        sl = slice(past, past + rows)
        _, w = cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, b, past, W, pad, scale,
                                 out=out[sl], stream=stream)
        widths.append(w)
    return out, widths


def roll_prefill(q, k, v, C: int, c: int, masks=None, scale: float = 0.0, stream=None,
                 split: bool = True, defer: bool = True):
    """Rolling fixed-capacity prefill of one sequence (batch 1).  q/k/v are
    token-major real tokens; the sequence is left-padded with zero rows to a
    multiple of c.  masks: optional list of per-chunk (c, C) additive masks;
    without it visibility is computed in the kernel.  Where the key range
    splits (split, bf16/fp16) and defer is set, each chunk's attention runs
    cpk_roll_attention_deferred (its parts merged by the next chunk's
    launch, the last by cpk_roll_flush); same outputs, bit for bit.  Returns
    (out over the padded sequence, n_leftpad, k cache, v cache)."""
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    n_left = (-L) % c
    if n_left:
        z = lambda x: torch.cat([torch.zeros((n_left,) + tuple(x.shape[1:]), dtype=x.dtype,
                                             device=x.device), x])
        q, k, v = z(q), z(k), z(v)
    Lp = L + n_left
    bufs = [torch.zeros((1, Hkv, C, D), dtype=q.dtype, device=q.device) for _ in range(4)]
    out = torch.empty_like(q)
    nbytes = cpk_roll_workspace_size(Hq, Hkv, C, c, D, q.dtype) if split and defer else 0
    wss = [_roll_workspace(nbytes, q.device, 1 + i) for i in range(2)] if nbytes else None
    cur, pending = 0, None
    for j in range(Lp // c):
        sl = slice(j * c, (j + 1) * c)
        ko, vo = bufs[2 * cur], bufs[2 * cur + 1]
        kn, vn = bufs[2 * (1 - cur)], bufs[2 * (1 - cur) + 1]
        cpk_roll_append(ko, vo, k[sl].unsqueeze(0), v[sl].unsqueeze(0), kn, vn, stream)
        cur = 1 - cur
        m = None if masks is None else masks[j]
        if wss:
            pending = cpk_roll_attention_deferred(q[sl], kn[0], vn[0], (j + 1) * c, n_left,
                                                  wss[j % 2], prev=pending, mask=m, scale=scale,
                                                  out=out[sl], stream=stream)
            continue
        cpk_roll_attention(q[sl], kn[0], vn[0], (j + 1) * c, n_left, mask=m, scale=scale,
                           out=out[sl], stream=stream, split=split)
    if pending is not None:
        cpk_roll_flush(pending, stream)
    return out, n_left, bufs[2 * cur][0], bufs[2 * cur + 1][0]


def ring_prefill(q, k, v, C: int, c: int, masks=None, scale: float = 0.0, stream=None,
                 split: bool = True, fused: bool = True, defer: bool = True):
    """roll_prefill over a ring buffer: per chunk, cpk_ring_step (append of
    the c rows fused into the attention launch), or with fused=False
    cpk_ring_append then cpk_ring_attention.  Where the key range splits
    (fused, split, bf16/fp16) and defer is set, each chunk runs
    cpk_ring_step_deferred (its parts merged by the next chunk's launch, the
    last by cpk_roll_flush).  Same outputs, bit for bit.  Returns (out over
    the padded sequence, n_leftpad, k ring, v ring, start)."""
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    n_left = (-L) % c
    if n_left:
        z = lambda x: torch.cat([torch.zeros((n_left,) + tuple(x.shape[1:]), dtype=x.dtype,
                                             device=x.device), x])
        q, k, v = z(q), z(k), z(v)
    Lp = L + n_left
    kr = torch.zeros((1, Hkv, C, D), dtype=q.dtype, device=q.device)
    vr = torch.zeros_like(kr)
    out = torch.empty_like(q)
    start = 0
    nbytes = cpk_roll_workspace_size(Hq, Hkv, C, c, D, q.dtype) if fused and split else 0
    if defer and nbytes:
        wss = [_roll_workspace(nbytes, q.device, 1 + i) for i in range(2)]
        pending = None
        for j in range(Lp // c):
            sl = slice(j * c, (j + 1) * c)
            pending, start = cpk_ring_step_deferred(
                q[sl], k[sl], v[sl], kr[0], vr[0], (j + 1) * c, n_left, start, wss[j % 2],
                prev=pending, mask=None if masks is None else masks[j], scale=scale,
                out=out[sl], stream=stream)
        if pending is not None:
            cpk_roll_flush(pending, stream)
        return out, n_left, kr[0], vr[0], start
    for j in range(Lp // c):
        sl = slice(j * c, (j + 1) * c)
        m = None if masks is None else masks[j]
        if fused:
            _, start = cpk_ring_step(q[sl], k[sl], v[sl], kr[0], vr[0], (j + 1) * c, n_left,
                                     start, mask=m, scale=scale, out=out[sl], stream=stream,
                                     split=split)
            continue
        start = cpk_ring_append(k[sl].unsqueeze(0), v[sl].unsqueeze(0), kr, vr, start, stream)
        cpk_ring_attention(q[sl], kr[0], vr[0], (j + 1) * c, n_left, start, mask=m, scale=scale,
                           out=out[sl], stream=stream, split=split)
    return out, n_left, kr[0], vr[0], start


def prefill_with_prefix(cache: KVCache, b: int, src_slot: int, prefix_len: int, q, k, v,
                        W: int, pad: bool = True, scale: float = 0.0, out=None, stream=None):
    """Prompt-prefix reuse: the first prefix_len positions of slot b are
    copied from src_slot (which holds them from an earlier prompt), then only
    the rest of the prompt (q/k/v: its rows past the prefix, token-major) is
    prefilled in W-row chunks starting at past_len = prefix_len.  Returns
    (out for those rows, widths)."""
    L, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    cpk_kv_copy_prefix(cache, src_slot, b, prefix_len, stream)
    widths = []
    for past, rows in cpk_split_chunks(L, W):
        sl = slice(past, past + rows)
        _, w = cpk_prefill_chunk(q[sl], k[sl], v[sl], cache, b, prefix_len + past, W, pad,
                                 scale, out=out[sl], stream=stream)
        widths.append(w)
    return out, widths
