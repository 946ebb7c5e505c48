"""Shared helpers of the GPU parity tests: device upload/download of the
seeded inputs, the tolerance checks, and per-config worlds."""
from __future__ import annotations

import dataclasses
import sys
from typing import List

import numpy as np
import torch

import engram_synth as synth
from oracle import engram_oracle as O

DEV = "cuda"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def up32(a: np.ndarray) -> torch.Tensor:
    """uint32/int32 host array -> int32 device tensor (same bits)."""
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a.astype(np.int32)).to(DEV)


def up16(a: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def upf(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def up8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def down32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def down16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, rel: float = 2e-2, what: str = "") -> None:
    """|got - ref| <= rel * max(|ref|, rms(ref row)) elementwise (BF16 bits in,
    rows along the last axis)."""
    g = O.bf16_to_f64(got)
    r = O.bf16_to_f64(ref)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    bound = rel * np.maximum(np.abs(r), rms)
    bad = ~(np.abs(g - r) <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: got {g[tuple(i)]!r} ref {r[tuple(i)]!r}")


def check_gate_rows(got_h, got_g, hidden, got_kv, ref_kv, wqk, dead, H, hc, dot_scale, what):
    """Hidden and gate of the given rows. End to end: hidden against the
    oracle's gate + residual on the oracle's k/v (ref_kv; None to skip).
    On identical inputs: hidden and gate against the oracle's gate +
    residual on the kernel's own k/v (got_kv), the gate at every position.
    (End to end the gate inherits k's BF16 rounding: a key element whose
    float32 and float64 sums round to neighbouring BF16 values moves dot by
    about 1e-2, which near dot = 0 moves sqrt(|dot|), and the gate, by more
    than 1e-3; so the gate bar is applied where its inputs are the same.)"""
    got_kv = np.where(dead[:, None], 0, got_kv)          # DEAD rows have no k/v; their gate is skipped
    new, g, _ = O.gate_residual(hidden, got_kv, wqk, dead, H, hc, 1e-6, dot_scale)
    assert_bf16_close(got_h.reshape(-1, H), new.reshape(-1, H), what=f"{what} hidden (same k/v)")
    assert np.max(np.abs(got_g - g), initial=0.0) <= 1e-3, what
    if ref_kv is not None:
        new_ref, _, _ = O.gate_residual(hidden, ref_kv, wqk, dead, H, hc, 1e-6, dot_scale)
        assert_bf16_close(got_h.reshape(-1, H), new_ref.reshape(-1, H), what=f"{what} hidden (end to end)")
    assert np.array_equal(got_h[dead], hidden[dead])
    assert np.all(got_g[dead] == 0)


@dataclasses.dataclass
class World:
    """Host inputs of one config and layer (small enough to hold on the host)."""
    cfg: synth.Config
    tmap: np.ndarray
    params: List[synth.HashParams]
    keys: List[tuple]

    @classmethod
    def of(cls, name: str) -> "World":
        cfg = synth.CONFIGS[name]
        tmap = synth.make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)
        return cls(cfg, tmap, synth.params_for(cfg),
                   [synth.table_keys(cfg.root, l) for l in cfg.layers])

    def rows(self, li: int):
        kd, ks = self.keys[li]
        return lambda r: synth.table_rows(r, kd, ks)


def device_table(E, n_rows: int, key_data: int, key_scale: int):
    codes = torch.empty(n_rows * 256, dtype=torch.uint8, device=DEV)
    scales = torch.empty(n_rows * 8, dtype=torch.uint8, device=DEV)
    E.engram_gen_table(codes, scales, 0, n_rows, key_data, key_scale)
    return codes, scales


def hidden_device(cfg, layer: int, T: int, first: int = 0, batch: int = 0) -> torch.Tensor:
    """Seeded hidden rows [first, first+T) generated chunk-parallel on the host
    and uploaded as int16 [T][hc][H]."""
    import concurrent.futures as cf
    out = torch.empty((T, cfg.hc, cfg.H), dtype=torch.int16, device=DEV)
    C = synth.HIDDEN_CHUNK
    # chunk-aligned pieces
    pieces, a = [], first
    while a < first + T:
        b = min(first + T, (a // C + 1) * C)
        pieces.append((a, b))
        a = b

    def gen(ab):
        a, b = ab
        return a, synth.hidden_bf16(cfg, layer, b - a, batch=batch, first=a)

    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        for a, h in ex.map(gen, pieces):
            out[a - first:a - first + h.shape[0]].copy_(torch.from_numpy(h.view(np.int16)))
    return out


def hidden_rows(cfg, layer: int, rows, batch: int = 0) -> np.ndarray:
    """Seeded hidden for selected global token rows (regenerating whole chunks once)."""
    rows = np.asarray(rows)
    out = np.empty((len(rows), cfg.hc, cfg.H), dtype=np.uint16)
    C = synth.HIDDEN_CHUNK
    for c in np.unique(rows // C):
        chunk = synth.hidden_bf16(cfg, layer, C, batch=batch, first=int(c) * C)
        sel = rows // C == c
        out[sel] = chunk[rows[sel] - int(c) * C]
    return out


def workspace_views(ws: torch.Tensor, T: int, H: int, hc: int):
    """Device views (idx [T][24], slot [T], mem [T][6144], kv [T][(hc+1)H]) of
    engram_forward's workspace: idx | slot | live counts | mem | kv | live
    positions, each section 256-byte aligned. Batches of more than 1,024 tokens or
    sequences pack the live (non-DEAD) positions' mem and kv rows in position
    order (row slot[t] for position t); smaller ones keep row t for position t."""
    r = lambda x: (x + 255) // 256 * 256
    o_slot = r(T * 96)
    o_mem = o_slot + r(T * 4) + r(4 * (1 + (T + 4095) // 4096))
    o_kv = o_mem + r(T * 12288)
    idx = ws[: T * 96].view(torch.int32)
    slot = ws[o_slot: o_slot + T * 4].view(torch.int32)
    mem = ws[o_mem: o_mem + T * 12288].view(torch.int16)
    kv = ws[o_kv: o_kv + T * (hc + 1) * H * 2].view(torch.int16)
    return idx, slot, mem, kv


def live_positions(ws: torch.Tensor, T: int, H: int, hc: int):
    """Device view of the workspace's last section: the position of each packed
    (live) row, in row order, for batches that pack rows."""
    r = lambda x: (x + 255) // 256 * 256
    kv_section = r(max(T * (hc + 1) * H * 2, T * 24 * 264))   # also holds rows staged from a host table
    o_pos = r(T * 96) + r(T * 4) + r(4 * (1 + (T + 4095) // 4096)) + r(T * 12288) + kv_section
    return ws[o_pos: o_pos + T * 4].view(torch.int32)


def forward_rows(ws: torch.Tensor, T: int, S: int, H: int, hc: int, rows):
    """Host copies of engram_forward's mem and kv rows for the given positions,
    and a mask of the positions that have a row (all of them for small
    batches; the live ones where rows are packed, whose DEAD positions have
    none)."""
    _, slot, mem, kv = workspace_views(ws, T, H, hc)
    rows = np.asarray(rows, dtype=np.int64)
    if T > 1024 or S > 1024:
        sl = slot.cpu().numpy().view(np.uint32)[rows]
        has = sl != 0xFFFFFFFF
        src = np.where(has, sl, 0).astype(np.int64)
    else:
        has = np.ones(len(rows), dtype=bool)
        src = rows
    m = down16(mem).reshape(T, 6144)[src]
    k = down16(kv).reshape(T, (hc + 1) * H)[src]
    return m, k, has
