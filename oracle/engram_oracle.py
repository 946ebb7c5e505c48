"""Engram forward-path oracle: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP library and imports nothing from it; inputs come from engram_synth.

Sources (web pages on Engram):
  [zLLM]    zhuai.tech, "DeepSeek V4.1 Flash 的 Engram：让知识不必每次重新算"
  [Storage] lqnn.cn, "3.84 亿行 Embedding 的存法大揭秘"
  [FlagOS]  gitcode.csdn.net, FlagScale Engram article ("核心可配置参数")
  [vLLM]    data-sketchers.com wiki, "Engram: n-gram 조회를 통한 조건부 메모리"

Steps, in the pages' order:
  1. compress      raw id -> compressed id          [zLLM] 第一步
  2. window        current token + 3 previous slots  [zLLM] 第一步, 第四步
  3. hash          24 multiply-XOR heads mod primes  [vLLM] How it works
  4. gather+decode MXFP8 rows -> BF16 6,144 vector   [zLLM] 第二步, [Storage]
  5. project       wkv (25,600 x 6,144) -> k/v       [zLLM] 第二步, [vLLM]
  6. gate          normalised dot, signed-sqrt sigmoid [zLLM] 第三步
  7. residual      hidden += gate * value; DEAD rows pass through
  8. history       append once per step, fork, reset [zLLM] 第四步

Floating point is float64 throughout; results are rounded to BF16 (round to
nearest even) exactly once where the method stores BF16 (k/v, hidden).

Readings where the pages are silent (each listed in the design notes):
  - orders n = 2, 3, 4 with 8 heads each: bucket j has n = 2 + j // 8;
  - window slot k is the compressed token k positions back; slots before
    the start of the history, or behind a DEAD token, hold pad_cid;
  - each product w_k * m is taken mod 2^64, and the products are XORed;
  - bucket j's row is offset[j] + (x mod prime[j]); memory position
    j*256 + c holds column c of bucket j's row;
  - E4M3 is the OCP "FN" encoding, E8M0 is 2^(s-127) with 255 = NaN,
    scale q covers columns 32q..32q+31;
  - keys are wkv rows [b*H, (b+1)*H) for branch b, the value rows [hc*H, (hc+1)*H);
  - gate normalisation is RMS without bias, eps and dot_scale are arguments.
Parity unpinned: none of the functions below lacks a pin; the synthetic
hash multipliers themselves are inputs and have no page value to match.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

DEAD_TOKEN = 0xFFFFFFFF
DEAD_IDX = 0xFFFFFFFF
HEADS_PER_ORDER = 8
ORDERS = (2, 3, 4)
N_BUCKETS = HEADS_PER_ORDER * len(ORDERS)   # 24 rows per token per layer
ROW = 256                                   # values per row
MEM = N_BUCKETS * ROW                       # 6,144
WINDOW = 4                                  # current token + 3 previous
MASK64 = (1 << 64) - 1


def bucket_order(j: int) -> int:
    """n-gram order of bucket j: buckets 0-7 are 2-grams, 8-15 3-grams,
    16-23 4-grams ([zLLM] 把知识变成可寻址的向量: 3 orders x 8 heads)."""
    return ORDERS[j // HEADS_PER_ORDER]


# --------------------------------------------------------------------------
# 1-2, 8. Compressed ids, windows and the per-sequence history
# --------------------------------------------------------------------------
def history_reset(n_seqs: int, pad_cid: int) -> np.ndarray:
    """A fresh history: every slot PAD ([zLLM] 第四步: reset clears history)."""
    return np.full((n_seqs, WINDOW - 1), pad_cid, dtype=np.uint32)


def history_fork(hist: np.ndarray) -> np.ndarray:
    """A forked session owns a copy of the parent's state ([zLLM] 第四步)."""
    return hist.copy()


def walk(tokens: np.ndarray, cu_seqlens: np.ndarray, hist: np.ndarray,
         token_map: np.ndarray, pad_cid: int
         ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Walk each sequence's tokens in order.

    The window of a text token is [c_t, H0, H1, H2] where c_t is its
    compressed id and H is the history just before it, H0 the most recent
    ([zLLM] 第一步: current token and the three most recent positions).
    After the token, H becomes [c_t, H0, H1]. A DEAD token has no window and
    resets H to PAD, so no n-gram crosses an image span ([zLLM] 第四步).

    Returns (windows uint64[T][4], dead bool[T], history after the batch).
    """
    T = len(tokens)
    win = np.zeros((T, WINDOW), dtype=np.uint64)
    dead = np.zeros(T, dtype=bool)
    new_hist = hist.copy()
    for s in range(len(cu_seqlens) - 1):
        h = [int(x) for x in hist[s]]
        for t in range(int(cu_seqlens[s]), int(cu_seqlens[s + 1])):
            tok = int(tokens[t])
            if tok == DEAD_TOKEN:
                dead[t] = True
                h = [pad_cid] * (WINDOW - 1)
                continue
            c = int(token_map[tok])
            win[t] = [c, h[0], h[1], h[2]]
            h = [c, h[0], h[1]]
        new_hist[s] = h
    return win, dead, new_hist


def history_append(hist: np.ndarray, tokens: np.ndarray, cu_seqlens: np.ndarray,
                   token_map: np.ndarray, pad_cid: int) -> np.ndarray:
    """Append one step's tokens to the history, once ([zLLM] 第四步)."""
    return walk(tokens, cu_seqlens, hist, token_map, pad_cid)[2]


# --------------------------------------------------------------------------
# 3. Multi-head multiply-XOR hashing ([vLLM] How it works, multi-head
#    hashing; [zLLM] 第一步: per-layer multipliers, prime buckets, offsets)
# --------------------------------------------------------------------------
def hash_window_scalar(w: Sequence[int], mult, prime, offset) -> List[int]:
    """Python-int twin for one window: the 24 row numbers."""
    rows = []
    for j in range(N_BUCKETS):
        x = 0
        for k in range(bucket_order(j)):
            x ^= (int(w[k]) * int(mult[j][k])) & MASK64
        rows.append(int(offset[j]) + x % int(prime[j]))
    return rows


def hash_windows(win: np.ndarray, dead: np.ndarray, mult: np.ndarray,
                 prime: np.ndarray, offset: np.ndarray) -> np.ndarray:
    """Vectorised over tokens: idx uint32[T][24]; DEAD tokens get DEAD_IDX."""
    T = win.shape[0]
    idx = np.zeros((T, N_BUCKETS), dtype=np.uint64)
    with np.errstate(over="ignore"):
        for j in range(N_BUCKETS):
            x = np.zeros(T, dtype=np.uint64)
            for k in range(bucket_order(j)):
                x ^= win[:, k] * np.uint64(mult[j][k])      # wraps mod 2^64
            idx[:, j] = np.uint64(offset[j]) + x % np.uint64(prime[j])
    idx[dead] = DEAD_IDX
    return idx.astype(np.uint32)


# --------------------------------------------------------------------------
# 4. MXFP8 decode ([zLLM] 第二步: E4M3 data with one E8M0 scale per 32
#    values; [Storage] FP8 E4M3 + UE8M0 group-32 scales decoded to BF16)
# --------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    """OCP E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
    infinities; S.1111.111 is NaN; exponent 0 is subnormal m/8 * 2^-6."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return math.copysign(m / 8.0 * 2.0 ** -6, sign)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(s: int) -> float:
    """E8M0: an unsigned power of two 2^(s-127); 255 encodes NaN."""
    return math.nan if s == 255 else 2.0 ** (s - 127)


_E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_E8M0 = np.array([e8m0_value(s) for s in range(256)], dtype=np.float64)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even), directly
    from float64 (no intermediate float32). Returns uint16 bit patterns.
    NaN becomes sign|0x7FC0; finite values beyond the BF16 range round to
    infinity; BF16 subnormals (quantum 2^-133) are kept."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x).astype(np.uint16) << np.uint16(15)
    a = np.abs(x)
    nan = np.isnan(x)
    fin = np.isfinite(x) & (a > 0)
    _, e2 = np.frexp(np.where(fin, a, 1.0))        # a = f * 2^e2, f in [0.5, 1)
    E = e2.astype(np.int64) - 1                     # a in [2^E, 2^(E+1))
    qexp = np.where(E >= -126, E - 7, -133)         # exponent of one unit in the last place
    n = np.rint(np.ldexp(np.where(fin, a, 0.0), -qexp))   # RNE to an integer count of quanta
    v = np.ldexp(n, qexp)                           # exactly representable in BF16 (or overflow)
    over = fin & (v >= 2.0 ** 128)
    v32 = np.where(fin & ~over, v, 0.0).astype(np.float32)
    bits = (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[fin] = bits[fin]
    out[over | np.isinf(x)] = 0x7F80
    out[nan] = 0x7FC0
    return out | sign


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of MXFP8 rows: code[c] * 2^(scale[c//32]-127).

    A NaN (NaN code, or scale 255) carries the sign bit of its code."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = _E4M3[codes] * np.repeat(_E8M0[np.asarray(scales, dtype=np.uint8)], 32, axis=-1)
    neg = (codes & 0x80) != 0
    return np.where(np.isnan(v), np.copysign(np.nan, np.where(neg, -1.0, 1.0)), v)


def gather_decode(idx: np.ndarray, row_source) -> np.ndarray:
    """The 6,144-wide memory vector of every token, as BF16 bits.

    `row_source(rows) -> (codes[R][256], scales[R][8])` supplies table rows
    (only the rows read are produced). Bucket j's row fills positions
    j*256 .. j*256+255 ([vLLM] How it works: rows are concatenated into one
    memory vector per position). DEAD tokens give all zeros.
    """
    T = idx.shape[0]
    mem = np.zeros((T, MEM), dtype=np.uint16)
    live = ~(idx[:, 0] == DEAD_IDX)
    if live.any():
        rows = idx[live].reshape(-1).astype(np.uint64)
        codes, scales = row_source(rows)
        vals = decode_rows(codes, scales)                     # [n*24][256]
        mem[live] = bf16_rne(vals).reshape(-1, MEM)
    return mem


# --------------------------------------------------------------------------
# 5. wkv projection ([zLLM] 第二步: wkv is 25,600 x 6,144 in BF16;
#    [Storage] 旋转合同: the last 5,120 rows are the value)
# --------------------------------------------------------------------------
def project(mem: np.ndarray, wkv: np.ndarray) -> np.ndarray:
    """kv[t] = wkv . mem[t] in float64, rounded once to BF16: uint16[T][(hc+1)H]."""
    m = bf16_to_f64(mem)
    w = bf16_to_f64(wkv)
    return bf16_rne(m @ w.T)


# --------------------------------------------------------------------------
# 6-7. Context gate and residual ([zLLM] 第三步; [vLLM] How it works, fusion)
# --------------------------------------------------------------------------
def gate_from_dot(dot: float) -> float:
    """gate = sigmoid(copysign(sqrt(max(|dot|, 1e-6)), dot))."""
    z = math.copysign(math.sqrt(max(abs(dot), 1e-6)), dot)
    return 1.0 / (1.0 + math.exp(-z))


def gate_dots(hidden: np.ndarray, kv: np.ndarray, wqk: np.ndarray, H: int, hc: int,
              eps: float, dot_scale: float) -> np.ndarray:
    """dot[t][b] = s * r_h * r_k * sum_i h_i k_i wqk_i for branch b, with
    r = 1/sqrt(mean(x^2) + eps) the RMS normalisation of h and of key b."""
    h = bf16_to_f64(hidden).reshape(-1, hc, H)
    k = bf16_to_f64(kv)[:, : hc * H].reshape(-1, hc, H)
    r_h = 1.0 / np.sqrt(np.mean(h * h, axis=2) + eps)
    r_k = 1.0 / np.sqrt(np.mean(k * k, axis=2) + eps)
    raw = np.sum(h * k * wqk.astype(np.float64)[None, :, :], axis=2)
    return dot_scale * r_h * r_k * raw


def gate_residual(hidden: np.ndarray, kv: np.ndarray, wqk: np.ndarray,
                  dead: np.ndarray, H: int, hc: int, eps: float, dot_scale: float
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per branch: g_b from the normalised dot, then h_b <- bf16(h_b + g_b v).

    DEAD positions skip the gate: hidden stays bit-identical, g is 0.
    Returns (new hidden uint16[T][hc][H], gate float64[T][hc], dot float64[T][hc]).
    """
    T = hidden.shape[0]
    dots = gate_dots(hidden, kv, wqk, H, hc, eps, dot_scale)
    g = np.array([[gate_from_dot(float(d)) for d in row] for row in dots]).reshape(T, hc)
    g[dead] = 0.0
    h = bf16_to_f64(hidden).reshape(T, hc, H)
    v = bf16_to_f64(kv)[:, hc * H:(hc + 1) * H]
    new = bf16_rne(h + g[:, :, None] * v[:, None, :])
    new[dead] = np.asarray(hidden).reshape(T, hc, H)[dead]
    return new, g, dots


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def forward(tokens, cu_seqlens, hist, token_map, params, row_source, wkv, wqk,
            hidden, H, hc, eps=1e-6, dot_scale=1.0):
    """One Engram layer: hash -> gather+decode -> project -> gate+residual.

    The history is read, not written: the caller appends once per step after
    all layers ([zLLM] 第四步). Returns a dict of every intermediate.
    """
    win, dead, _ = walk(tokens, cu_seqlens, hist, token_map, params.pad_cid)
    idx = hash_windows(win, dead, params.mult, params.prime, params.offset)
    mem = gather_decode(idx, row_source)
    kv = project(mem, wkv)
    new_hidden, g, dots = gate_residual(hidden, kv, wqk, dead, H, hc, eps, dot_scale)
    return {"idx": idx, "mem": mem, "kv": kv, "hidden": new_hidden, "gate": g,
            "dot": dots, "dead": dead, "windows": win}
