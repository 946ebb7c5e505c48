"""Python binding of libengram, the MI355X (gfx950) Engram forward path.

Argument marshalling only: every function checks the tensors' dtype, device
and contiguity, then calls the C entry point of the same name with raw
pointers and torch's current HIP stream. All computation happens in the HIP
kernels; there is no CPU fallback. Importing this package fails if
libengram.so has not been built (python gram_hashed_embedding_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "EngramError", "HashParams", "lib",
    "engram_check_params", "engram_history_reset", "engram_history_fork",
    "engram_history_append", "engram_hash", "engram_gather_decode", "engram_project",
    "engram_gate", "engram_forward_workspace", "engram_precompute", "engram_gate_precomputed",
    "engram_precompute_buckets", "BucketTable",
    "engram_forward", "engram_forward_noalloc", "engram_gen_table", "engram_pack_wkv",
    "DEAD_TOKEN", "DEAD_IDX", "BUCKETS", "MEM", "STAGE_EVENTS", "PRECOMPUTE_STAGE_ROWS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

DEAD_TOKEN = 0xFFFFFFFF
DEAD_IDX = 0xFFFFFFFF
BUCKETS = 24
MEM = 6144
STAGE_EVENTS = 5
NOALLOC_WORKSPACE_BYTES = 64 << 20
PRECOMPUTE_STAGE_ROWS = 0x1

ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_EHIP, ENGRAM_EUNSUPPORTED = 0, -1, -2, -3


class EngramError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: {_status(status)}: {detail}")
        self.status = status


class BucketTable(ctypes.Structure):
    """Mirror of engram_bucket_table (a table held as one allocation per bucket)."""
    _fields_ = [("codes", ctypes.c_void_p * 24), ("scales", ctypes.c_void_p * 24)]


class HashParams(ctypes.Structure):
    """Mirror of engram_hash_params (one layer's hash tables)."""
    _fields_ = [
        ("mult", (ctypes.c_uint64 * 4) * 24),
        ("prime", ctypes.c_uint32 * 24),
        ("offset", ctypes.c_uint64 * 24),
        ("n_rows", ctypes.c_uint64),
        ("vocab_c", ctypes.c_uint32),
        ("pad_cid", ctypes.c_uint32),
    ]

    @classmethod
    def make(cls, mult, prime, offset, n_rows: int, vocab_c: int, pad_cid: int) -> "HashParams":
        p = cls()
        m = np.asarray(mult, dtype=np.uint64).reshape(24, 4)
        for j in range(24):
            for k in range(4):
                p.mult[j][k] = int(m[j, k])
            p.prime[j] = int(np.asarray(prime)[j])
            p.offset[j] = int(np.asarray(offset)[j])
        p.n_rows, p.vocab_c, p.pad_cid = int(n_rows), int(vocab_c), int(pad_cid)
        return p

    @classmethod
    def from_any(cls, obj) -> "HashParams":
        """Accept a HashParams or any object with mult/prime/offset/n_rows/vocab_c/pad_cid."""
        if isinstance(obj, cls):
            return obj
        return cls.make(obj.mult, obj.prime, obj.offset, obj.n_rows, obj.vocab_c, obj.pad_cid)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python gram_hashed_embedding_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U32, U64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
                                      ctypes.c_size_t)
    sigs = {
        "engram_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "engram_last_error": ([], ctypes.c_char_p),
        "engram_abi_version": ([], ctypes.c_int),
        "engram_check_params": ([P, P, U32], ctypes.c_int),
        "engram_history_reset": ([P, I32, U32, P], ctypes.c_int),
        "engram_history_fork": ([P, P, I32, P], ctypes.c_int),
        "engram_history_append": ([P, P, P, I32, I64, P, U32, U32, P, P], ctypes.c_int),
        "engram_hash": ([P, P, I32, I64, P, P, U32, P, P, P, P], ctypes.c_int),
        "engram_gather_decode": ([P, I64, P, P, U64, P, P, P], ctypes.c_int),
        "engram_project": ([P, I64, P, P, I32, I32, P, P], ctypes.c_int),
        "engram_pack_wkv": ([P, I32, I32, P, P], ctypes.c_int),
        "engram_gate": ([P, P, P, P, I64, I32, I32, F32, F32, P, P], ctypes.c_int),
        "engram_forward_workspace": ([I64, I32, I32], SZ),
        "engram_precompute": ([P, P, I32, I64, P, P, U32, P, P, P, P, P, I32, I32, U32, P, SZ,
                               P, P], ctypes.c_int),
        "engram_gate_precomputed": ([P, P, SZ, P, I32, I64, P, I32, I32, F32, F32, P, P],
                                    ctypes.c_int),
        "engram_precompute_buckets": ([P, P, I32, I64, P, P, U32, P, P, P, P, I32, I32, U32, P,
                                       SZ, P, P], ctypes.c_int),
        "engram_forward": ([P, P, I32, I64, P, P, U32, P, P, P, P, P, P, P, I32, I32, F32,
                            F32, P, SZ, P, P, P, P], ctypes.c_int),
        "engram_gen_table": ([P, P, U64, U64, U64, U64, P], ctypes.c_int),
        "engram_forward_noalloc": ([P, P, I32, I64, P, P, U32, P, P, P, P, P, P, P, I32, I32,
                                    F32, F32, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def _status(s: int) -> str:
    return lib.engram_status_string(s).decode()


def _check(rc: int, fn: str) -> None:
    if rc != ENGRAM_OK:
        raise EngramError(rc, fn, lib.engram_last_error().decode())


# ---------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor", optional=False, host_ok=False):
    """Device pointer of a contiguous CUDA(HIP) tensor (or None -> NULL).
    With host_ok, a pinned host tensor is accepted too: pinned memory is
    mapped into the device's address space at its host address."""
    if t is None:
        if optional:
            return None
        raise TypeError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor" + (" or a pinned host tensor" if host_ok else "")
                         + f" (got {t.device})")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _i32(torch):
    return torch.int32


def _u32(torch):
    return (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _u16(torch):
    return (torch.int16, torch.bfloat16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())


# ---------------------------------------------------------------- entry points
def engram_check_params(params, token_map: Optional[np.ndarray] = None) -> None:
    """Host-only check of one layer's params (and host token map)."""
    p = HashParams.from_any(params)
    if token_map is None:
        rc = lib.engram_check_params(ctypes.byref(p), None, 0)
    else:
        m = np.ascontiguousarray(token_map, dtype=np.uint32)
        rc = lib.engram_check_params(ctypes.byref(p), m.ctypes.data, len(m))
    _check(rc, "engram_check_params")


def _need(t, n: int, name: str) -> None:
    """A device buffer the kernels will touch n elements of must hold them."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, {n} needed")


def _n_seqs(hist, name="hist") -> int:
    """Sequences held by a history tensor of S*3 entries (any shape)."""
    if hist.numel() % 3:
        raise ValueError(f"{name} must hold S*3 entries (got {hist.numel()})")
    return hist.numel() // 3


def engram_history_reset(hist, pad_cid: int, stream=None) -> None:
    torch = _torch()
    S = _n_seqs(hist)
    _check(lib.engram_history_reset(_ptr(hist, _u32(torch), "hist"), S, pad_cid, _stream(stream)),
           "engram_history_reset")


def engram_history_fork(dst, src, stream=None) -> None:
    torch = _torch()
    if dst.numel() != src.numel():
        raise ValueError("dst and src histories differ in size")
    _check(lib.engram_history_fork(_ptr(dst, _u32(torch), "dst"), _ptr(src, _u32(torch), "src"),
                                   _n_seqs(dst, "dst"), _stream(stream)), "engram_history_fork")


def engram_history_append(hist, tok, cu_seqlens, token_map, pad_cid: int, err_flags=None,
                          stream=None) -> None:
    torch = _torch()
    S = cu_seqlens.numel() - 1
    _need(hist, 3 * S, "hist")
    _need(err_flags, 1, "err_flags")
    _check(lib.engram_history_append(
        _ptr(hist, _u32(torch), "hist"), _ptr(tok, _u32(torch), "tok"),
        _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, tok.numel(),
        _ptr(token_map, _u32(torch), "token_map"), token_map.numel(), pad_cid,
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)),
        "engram_history_append")


def engram_hash(tok, cu_seqlens, hist, token_map, params, idx, err_flags=None, stream=None) -> None:
    torch = _torch()
    p = HashParams.from_any(params)
    S = cu_seqlens.numel() - 1
    T = tok.numel()
    if idx.numel() != T * BUCKETS:
        raise ValueError("idx must hold T*24 entries")
    _need(hist, 3 * S, "hist")
    _need(err_flags, 1, "err_flags")
    _check(lib.engram_hash(
        _ptr(tok, _u32(torch), "tok"), _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, T,
        _ptr(hist, _u32(torch), "hist"), _ptr(token_map, _u32(torch), "token_map"),
        token_map.numel(), ctypes.byref(p), _ptr(idx, _u32(torch), "idx"),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)), "engram_hash")


def engram_gather_decode(idx, codes, scales, n_rows: int, mem, err_flags=None, stream=None) -> None:
    torch = _torch()
    T = idx.numel() // BUCKETS
    if idx.numel() % BUCKETS or mem.numel() != T * MEM:
        raise ValueError("idx must hold T*24 entries and mem T*6144")
    _need(codes, n_rows * 256, "codes")
    _need(scales, n_rows * 8, "scales")
    _need(err_flags, 1, "err_flags")
    _check(lib.engram_gather_decode(
        _ptr(idx, _u32(torch), "idx"), T, _ptr(codes, torch.uint8, "codes", host_ok=True),
        _ptr(scales, torch.uint8, "scales", host_ok=True), n_rows, _ptr(mem, _u16(torch), "mem"),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)),
        "engram_gather_decode")


def _check_packed(wkv_packed, wkv) -> None:
    if wkv_packed is not None and wkv_packed.numel() != wkv.numel():
        raise ValueError("wkv_packed must have wkv's size (engram_pack_wkv's output)")


def engram_project(mem, wkv, H: int, hc: int, kv, stream=None, wkv_packed=None) -> None:
    torch = _torch()
    T = mem.numel() // MEM
    if mem.numel() % MEM:
        raise ValueError("mem must hold T*6144 entries")
    if wkv.numel() != (hc + 1) * H * MEM or kv.numel() != T * (hc + 1) * H:
        raise ValueError("wkv must be [(hc+1)*H][6144] and kv [T][(hc+1)*H]")
    _check_packed(wkv_packed, wkv)
    _check(lib.engram_project(_ptr(mem, _u16(torch), "mem"), T, _ptr(wkv, _u16(torch), "wkv"),
                              _ptr(wkv_packed, _u16(torch), "wkv_packed", optional=True),
                              H, hc, _ptr(kv, _u16(torch), "kv"), _stream(stream)),
           "engram_project")


def engram_pack_wkv(wkv, H: int, hc: int, out=None, stream=None):
    """wkv in the decode layout (see include/engram.h); returns `out` (a new
    tensor like wkv if None)."""
    torch = _torch()
    if wkv.numel() != (hc + 1) * H * MEM:
        raise ValueError("wkv must be [(hc+1)*H][6144]")
    if out is None:
        out = torch.empty_like(wkv)
    _check_packed(out, wkv)
    _check(lib.engram_pack_wkv(_ptr(wkv, _u16(torch), "wkv"), H, hc,
                               _ptr(out, _u16(torch), "wkv_packed"), _stream(stream)),
           "engram_pack_wkv")
    return out


def engram_gate(hidden, kv, wqk, tok, H: int, hc: int, eps: float = 1e-6, dot_scale: float = 1.0,
                gate_out=None, stream=None) -> None:
    torch = _torch()
    T = hidden.numel() // (hc * H)
    if hidden.numel() % (hc * H):
        raise ValueError("hidden must hold T*hc*H entries")
    if kv.numel() != T * (hc + 1) * H or wqk.numel() != hc * H:
        raise ValueError("kv must be [T][(hc+1)*H] and wqk [hc][H]")
    _need(tok, T, "tok")
    _need(gate_out, T * hc, "gate_out")
    _check(lib.engram_gate(
        _ptr(hidden, _u16(torch), "hidden"), _ptr(kv, _u16(torch), "kv"),
        _ptr(wqk, torch.float32, "wqk"), _ptr(tok, _u32(torch), "tok", optional=True), T, H, hc,
        eps, dot_scale, _ptr(gate_out, torch.float32, "gate_out", optional=True), _stream(stream)),
        "engram_gate")


def engram_forward_workspace(T: int, H: int, hc: int) -> int:
    return int(lib.engram_forward_workspace(T, H, hc))


def engram_precompute(tok, cu_seqlens, hist, token_map, params, codes, scales, wkv, H: int,
                      hc: int, ws=None, flags: int = 0, err_flags=None, stream=None,
                      wkv_packed=None):
    """The hidden-independent half of one layer (hash, gather + decode,
    projection) into a workspace. Returns the workspace (allocated here when
    None; pass the same one to engram_gate_precomputed)."""
    torch = _torch()
    p = HashParams.from_any(params)
    S = cu_seqlens.numel() - 1
    T = tok.numel()
    if wkv.numel() != (hc + 1) * H * MEM:
        raise ValueError("wkv must be [(hc+1)*H][6144]")
    _check_packed(wkv_packed, wkv)
    _need(hist, 3 * S, "hist")
    _need(codes, p.n_rows * 256, "codes")
    _need(scales, p.n_rows * 8, "scales")
    _need(err_flags, 1, "err_flags")
    need = engram_forward_workspace(T, H, hc)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=wkv.device)
    _need(ws, need, "ws")
    _check(lib.engram_precompute(
        _ptr(tok, _u32(torch), "tok"), _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, T,
        _ptr(hist, _u32(torch), "hist"), _ptr(token_map, _u32(torch), "token_map"),
        token_map.numel(), ctypes.byref(p), _ptr(codes, torch.uint8, "codes", host_ok=True),
        _ptr(scales, torch.uint8, "scales", host_ok=True), _ptr(wkv, _u16(torch), "wkv"),
        _ptr(wkv_packed, _u16(torch), "wkv_packed", optional=True), H, hc, flags,
        _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)),
        "engram_precompute")
    return ws


def _table_ptr(x, name, nbytes):
    """A bucket's address: a device or pinned host tensor (of at least nbytes),
    or an int (the address of nbytes of device memory or of pinned host memory
    mapped at its host address, e.g. from hipHostMalloc)."""
    torch = _torch()
    if isinstance(x, int):
        if x == 0:
            raise ValueError(f"{name} is NULL")
        return x
    _need(x, nbytes, name)
    return _ptr(x, torch.uint8, name, host_ok=True)


def engram_precompute_buckets(tok, cu_seqlens, hist, token_map, params, codes, scales, wkv,
                              H: int, hc: int, ws=None, flags: int = 0, err_flags=None,
                              stream=None, wkv_packed=None):
    """engram_precompute with the table given per bucket: codes[j] / scales[j]
    hold bucket j's prime[j] rows (24 of each). Returns the workspace."""
    torch = _torch()
    p = HashParams.from_any(params)
    if len(codes) != BUCKETS or len(scales) != BUCKETS:
        raise ValueError("codes and scales must list 24 buckets each")
    tbl = BucketTable()
    for j in range(BUCKETS):
        tbl.codes[j] = _table_ptr(codes[j], f"codes[{j}]", int(p.prime[j]) * 256)
        tbl.scales[j] = _table_ptr(scales[j], f"scales[{j}]", int(p.prime[j]) * 8)
    S = cu_seqlens.numel() - 1
    T = tok.numel()
    if wkv.numel() != (hc + 1) * H * MEM:
        raise ValueError("wkv must be [(hc+1)*H][6144]")
    _check_packed(wkv_packed, wkv)
    _need(hist, 3 * S, "hist")
    _need(err_flags, 1, "err_flags")
    need = engram_forward_workspace(T, H, hc)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=wkv.device)
    _need(ws, need, "ws")
    _check(lib.engram_precompute_buckets(
        _ptr(tok, _u32(torch), "tok"), _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, T,
        _ptr(hist, _u32(torch), "hist"), _ptr(token_map, _u32(torch), "token_map"),
        token_map.numel(), ctypes.byref(p), ctypes.byref(tbl), _ptr(wkv, _u16(torch), "wkv"),
        _ptr(wkv_packed, _u16(torch), "wkv_packed", optional=True), H, hc, flags,
        _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)),
        "engram_precompute_buckets")
    return ws


def engram_gate_precomputed(hidden, ws, tok, S: int, wqk, H: int, hc: int, eps: float = 1e-6,
                            dot_scale: float = 1.0, gate_out=None, stream=None) -> None:
    """The gate at layer entry, reading the k/v engram_precompute left in ws
    for the same tokens (S sequences)."""
    torch = _torch()
    T = tok.numel()
    if hidden.numel() != T * hc * H or wqk.numel() != hc * H:
        raise ValueError("hidden must be [T][hc][H] and wqk [hc][H]")
    _need(gate_out, T * hc, "gate_out")
    _need(ws, engram_forward_workspace(T, H, hc), "ws")
    _check(lib.engram_gate_precomputed(
        _ptr(hidden, _u16(torch), "hidden"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _ptr(tok, _u32(torch), "tok"), S, T, _ptr(wqk, torch.float32, "wqk"), H, hc, eps,
        dot_scale, _ptr(gate_out, torch.float32, "gate_out", optional=True), _stream(stream)),
        "engram_gate_precomputed")


def engram_forward(tok, cu_seqlens, hist, token_map, params, codes, scales, wkv, wqk, hidden,
                   H: int, hc: int, eps: float = 1e-6, dot_scale: float = 1.0, ws=None,
                   gate_out=None, err_flags=None, stage_events: Optional[Sequence] = None,
                   stream=None, wkv_packed=None):
    """One Engram layer on the device. Returns the workspace tensor used
    (idx, mem and k/v live in it; pass it back in to reuse it)."""
    torch = _torch()
    p = HashParams.from_any(params)
    S = cu_seqlens.numel() - 1
    T = tok.numel()
    if hidden.numel() != T * hc * H:
        raise ValueError("hidden must be [T][hc][H]")
    if wkv.numel() != (hc + 1) * H * MEM or wqk.numel() != hc * H:
        raise ValueError("wkv must be [(hc+1)*H][6144] and wqk [hc][H]")
    _check_packed(wkv_packed, wkv)
    _need(hist, 3 * S, "hist")
    _need(codes, p.n_rows * 256, "codes")
    _need(scales, p.n_rows * 8, "scales")
    _need(gate_out, T * hc, "gate_out")
    _need(err_flags, 1, "err_flags")
    need = engram_forward_workspace(T, H, hc)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    _need(ws, need, "ws")
    ev = None
    if stage_events is not None:
        if len(stage_events) != STAGE_EVENTS:
            raise ValueError(f"stage_events needs {STAGE_EVENTS} events")
        handles = [e.cuda_event for e in stage_events]
        if not all(handles):
            raise ValueError("stage_events: torch creates an event's HIP handle on its first "
                             "record(); record each event once before passing it")
        ev = (ctypes.c_void_p * STAGE_EVENTS)(*handles)
    _check(lib.engram_forward(
        _ptr(tok, _u32(torch), "tok"), _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, T,
        _ptr(hist, _u32(torch), "hist"), _ptr(token_map, _u32(torch), "token_map"),
        token_map.numel(), ctypes.byref(p), _ptr(codes, torch.uint8, "codes", host_ok=True),
        _ptr(scales, torch.uint8, "scales", host_ok=True), _ptr(wkv, _u16(torch), "wkv"),
        _ptr(wkv_packed, _u16(torch), "wkv_packed", optional=True),
        _ptr(wqk, torch.float32, "wqk"), _ptr(hidden, _u16(torch), "hidden"), H, hc, eps,
        dot_scale, _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _ptr(gate_out, torch.float32, "gate_out", optional=True),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)),
        "engram_forward")
    return ws


def engram_forward_noalloc(tok, cu_seqlens, hist, token_map, params, codes, scales, wkv, wqk,
                           hidden, H: int, hc: int, eps: float = 1e-6, dot_scale: float = 1.0,
                           gate_out=None, err_flags=None, stream=None, wkv_packed=None) -> None:
    """engram_forward with the library's own per-GPU workspace (no
    allocation; batches up to NOALLOC_WORKSPACE_BYTES of workspace)."""
    torch = _torch()
    p = HashParams.from_any(params)
    S = cu_seqlens.numel() - 1
    T = tok.numel()
    if hidden.numel() != T * hc * H:
        raise ValueError("hidden must be [T][hc][H]")
    if wkv.numel() != (hc + 1) * H * MEM or wqk.numel() != hc * H:
        raise ValueError("wkv must be [(hc+1)*H][6144] and wqk [hc][H]")
    _check_packed(wkv_packed, wkv)
    _need(hist, 3 * S, "hist")
    _need(codes, p.n_rows * 256, "codes")
    _need(scales, p.n_rows * 8, "scales")
    _need(gate_out, T * hc, "gate_out")
    _need(err_flags, 1, "err_flags")
    _check(lib.engram_forward_noalloc(
        _ptr(tok, _u32(torch), "tok"), _ptr(cu_seqlens, _i32(torch), "cu_seqlens"), S, T,
        _ptr(hist, _u32(torch), "hist"), _ptr(token_map, _u32(torch), "token_map"),
        token_map.numel(), ctypes.byref(p), _ptr(codes, torch.uint8, "codes", host_ok=True),
        _ptr(scales, torch.uint8, "scales", host_ok=True), _ptr(wkv, _u16(torch), "wkv"),
        _ptr(wkv_packed, _u16(torch), "wkv_packed", optional=True),
        _ptr(wqk, torch.float32, "wqk"), _ptr(hidden, _u16(torch), "hidden"), H, hc, eps,
        dot_scale, _ptr(gate_out, torch.float32, "gate_out", optional=True),
        _ptr(err_flags, _u32(torch), "err_flags", optional=True), _stream(stream)),
        "engram_forward_noalloc")


def engram_gen_table(codes, scales, row_begin: int, n_rows: int, key_data: int, key_scale: int,
                     stream=None) -> None:
    """codes/scales: tensors (device or pinned host) or int addresses (see
    engram_precompute_buckets) of at least n_rows rows."""
    _check(lib.engram_gen_table(_table_ptr(codes, "codes", n_rows * 256),
                                _table_ptr(scales, "scales", n_rows * 8),
                                row_begin, n_rows, key_data, key_scale, _stream(stream)),
           "engram_gen_table")
