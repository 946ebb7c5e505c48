"""Seeded synthetic inputs for the Engram forward path.

This module is shared by the oracle, the tests and the benchmark. It holds
input generation only: token maps, token streams, DEAD spans, hash
parameters, the closed-form MXFP8 table and dense tensors. It contains none
of the method's arithmetic (no hashing, no decoding, no projection, no gate).

Sources (web pages on Engram) cited here:
  [zLLM]    zhuai.tech, "DeepSeek V4.1 Flash 的 Engram：让知识不必每次重新算"
  [Storage] lqnn.cn, "3.84 亿行 Embedding 的存法大揭秘"
  [FlagOS]  gitcode.csdn.net, FlagScale Engram article ("核心可配置参数")
  [vLLM]    data-sketchers.com wiki, "Engram: n-gram 조회를 통한 조건부 메모리"

The pages name no public text; seeded Zipf streams stand in for the
50,032-token prompt and the short decode prompt of [zLLM] (introduction).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

DEAD_TOKEN = 0xFFFFFFFF          # token value marking an image (DEAD) position
N_BUCKETS = 24                    # 3 orders x 8 heads
ROW_BYTES = 256                   # one E4M3 code per value
SCALES_PER_ROW = 8                # one E8M0 scale per 32 values
RAW_VOCAB = 129_280               # entries of the token map ([zLLM] 第一步)

MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15

# Stream numbers for np.random.default_rng([root, stream, ...]).
STREAM_MAP, STREAM_TOKENS, STREAM_HIST, STREAM_HIDDEN = 1, 2, 3, 4
STREAM_WKV, STREAM_NORMW, STREAM_MULT, STREAM_DEAD = 5, 6, 7, 10


# --------------------------------------------------------------------------
# SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014), used as a counter-based generator:
# splitmix64(x) is the first output of a SplitMix64 stream whose state is x.
# --------------------------------------------------------------------------
def splitmix64_int(x: int) -> int:
    z = (x + _GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64_np(x: np.ndarray) -> np.ndarray:
    """Vectorised SplitMix64 over uint64 arrays (wrap-around arithmetic)."""
    z = np.asarray(x, dtype=np.uint64) + np.uint64(_GOLDEN_GAMMA)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def table_keys(root: int, layer: int) -> Tuple[int, int]:
    """(key_data, key_scale) of one layer's synthetic table."""
    base = (root << 8) | ((layer & 0x7F) << 1)
    return splitmix64_int(base), splitmix64_int(base | 1)


# The 254 E4M3 codes that are not NaN, in ascending code order. The OCP
# E4M3 ("FN") encoding reserves S.1111.111 (0x7F, 0xFF) for NaN.
FINITE_E4M3_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F],
                             dtype=np.uint8)
SCALE_MIN, SCALE_SPAN = 119, 9    # E8M0 119..127, i.e. 2^-8 .. 2^0


def table_rows(rows: np.ndarray, key_data: int, key_scale: int
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Closed-form synthetic MXFP8 rows.

    code[r][c]  = FINITE[hi32(splitmix64(key_data + r*256 + c)) mod 254]
    scale[r][q] = 119 + hi32(splitmix64(key_scale + r*8 + q)) mod 9

    Returns (codes uint8[len(rows)][256], scales uint8[len(rows)][8]). Only
    the requested rows are produced, so a 384M-row table never exists on
    the host.
    """
    r = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    col = np.arange(ROW_BYTES, dtype=np.uint64).reshape(1, -1)
    z = splitmix64_np(np.uint64(key_data) + r * np.uint64(ROW_BYTES) + col)
    codes = FINITE_E4M3_CODES[(z >> np.uint64(32)) % np.uint64(254)]
    q = np.arange(SCALES_PER_ROW, dtype=np.uint64).reshape(1, -1)
    zs = splitmix64_np(np.uint64(key_scale) + r * np.uint64(SCALES_PER_ROW) + q)
    scales = (SCALE_MIN + (zs >> np.uint64(32)) % np.uint64(SCALE_SPAN)).astype(np.uint8)
    return codes.astype(np.uint8), scales


# --------------------------------------------------------------------------
# Hash parameters ([zLLM] 第一步: per-layer multipliers, prime buckets and
# bucket offsets expanded into static tables; [vLLM] "How it works": each
# (order, head) pair owns a distinct prime-sized bucket range).
# --------------------------------------------------------------------------
def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    i = 3
    while i * i <= n:
        if n % i == 0:
            return False
        i += 2
    return True


def primes_above(base: int, count: int) -> List[int]:
    """The `count` smallest primes strictly greater than `base`."""
    out, n = [], base + 1
    while len(out) < count:
        if _is_prime(n):
            out.append(n)
        n += 1
    return out


@dataclasses.dataclass
class HashParams:
    """One layer's hash parameters, in the layout the C-ABI takes."""
    mult: np.ndarray      # uint64[24][4]; mult[j][k] multiplies window slot k
    prime: np.ndarray     # uint32[24]
    offset: np.ndarray    # uint64[24]; offset[0] = 0, prefix sums of prime
    n_rows: int
    vocab_c: int
    pad_cid: int


def make_hash_params(root: int, layer: int, vocab_c: int, prime_base: int,
                     pad_cid: int) -> HashParams:
    """Seeded hash parameters for one layer.

    Buckets: the 24 smallest primes above `prime_base`, in increasing order
    (j = (n-2)*8 + head). Multipliers: four odd values per layer below
    floor((2^63-1)/vocab_c), so a compressed id times a multiplier never
    exceeds 63 bits; all 24 buckets use the same four and differ by their
    prime. Drawn from stream STREAM_MULT.
    """
    primes = primes_above(prime_base, N_BUCKETS)
    offs = np.zeros(N_BUCKETS, dtype=np.uint64)
    offs[1:] = np.cumsum(np.array(primes[:-1], dtype=np.uint64))
    bound = ((1 << 63) - 1) // vocab_c
    rng = np.random.default_rng([root, STREAM_MULT, layer])
    m4 = [2 * int(rng.integers(0, bound // 2)) + 1 for _ in range(4)]
    mult = np.tile(np.array(m4, dtype=np.uint64), (N_BUCKETS, 1))
    return HashParams(mult=mult, prime=np.array(primes, dtype=np.uint32),
                      offset=offs, n_rows=int(sum(primes)), vocab_c=vocab_c,
                      pad_cid=pad_cid)


def make_full_range_hash_params(root: int, layer: int, vocab_c: int, prime_base: int,
                                pad_cid: int) -> HashParams:
    """Like make_hash_params, but with 96 distinct odd multipliers drawn
    uniformly over [2^32, 2^64), one per (bucket, window slot): products of a
    compressed id and a multiplier wrap past 2^64 and XORs of them reach
    2^63 and above, so every bucket's own multipliers and the 64-bit wrap
    are exercised (the C ABI takes any uint64 table)."""
    base = make_hash_params(root, layer, vocab_c, prime_base, pad_cid)
    rng = np.random.default_rng([root, STREAM_MULT, layer, 1])
    seen = set()
    mult = np.zeros((N_BUCKETS, 4), dtype=np.uint64)
    for j in range(N_BUCKETS):
        for k in range(4):
            while True:
                m = int(rng.integers(1 << 31, 1 << 63, dtype=np.uint64)) * 2 + 1
                if m not in seen:
                    seen.add(m)
                    mult[j, k] = m
                    break
    return dataclasses.replace(base, mult=mult)


# --------------------------------------------------------------------------
# Token map: seeded many-to-one map raw id -> compressed id, onto 0..V_c-1
# (stand-in for the tokenizer normalisation of [vLLM] "How it works").
# --------------------------------------------------------------------------
def make_token_map(root: int, map_len: int, vocab_c: int) -> np.ndarray:
    rng = np.random.default_rng([root, STREAM_MAP])
    perm = rng.permutation(map_len)
    cmap = np.empty(map_len, dtype=np.uint32)
    cmap[perm[:vocab_c]] = np.arange(vocab_c, dtype=np.uint32)
    cmap[perm[vocab_c:]] = rng.integers(0, vocab_c, map_len - vocab_c, dtype=np.uint32)
    return cmap


def zipf_tokens(rng: np.random.Generator, n: int, n_ranks: int = RAW_VOCAB,
                a: float = 1.1) -> np.ndarray:
    """Truncated Zipf(a) over ranks 1..n_ranks by inverse CDF; id = rank-1."""
    w = np.arange(1, n_ranks + 1, dtype=np.float64) ** (-a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), n_ranks - 1).astype(np.uint32)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (torch's RNE cast); return bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Workload configurations
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    code: int             # c in the root seed 0xE46A0000 + c
    map_len: int
    vocab_c: int
    H: int
    hc: int
    layers: Tuple[int, ...]           # layer ids (the checkpoint's 1 and 14)
    prime_bases: Tuple[int, ...]      # per layer: primes strictly above this
    n_seqs: int
    tokens_per_seq: int
    history_prefix: int = 0           # tokens appended before the measured batch
    uniform_tokens: bool = False
    dead_spans_per_seq: int = 0
    dead_span_len: int = 0
    decode_steps: int = 0

    @property
    def root(self) -> int:
        return 0xE46A0000 + self.code

    @property
    def T(self) -> int:
        return self.n_seqs * self.tokens_per_seq


# Layer 14 of the two-layer configs takes the 24 primes after layer 1's.
_L14_BASE = 16_000_463

CONFIGS: Dict[str, Config] = {
    # Tiny: one layer, 1 sequence of 64 uniform tokens.
    "tiny": Config("tiny", 1, 4096, 1000, 256, 4, (1,), (1000,), 1, 64,
                   uniform_tokens=True),
    # Decode-shaped: 64 sequences, 1 new token each, 3-token history.
    "decode": Config("decode", 2, RAW_VOCAB, 100_000, 5120, 4, (1,), (666_666,),
                     64, 1, history_prefix=3),
    # Full-size one layer: prefill of 4,096 tokens.
    "full": Config("full", 3, RAW_VOCAB, 100_000, 5120, 4, (1,), (16_000_000,),
                   1, 4096),
    # Long prefill, two layers: 50,032 tokens.
    "long": Config("long", 4, RAW_VOCAB, 100_000, 5120, 4, (1, 14),
                   (16_000_000, _L14_BASE), 1, 50_032),
    # Multimodal batched decode: 256 prompts of 2,048 with 2 DEAD spans of
    # 576, then 128 decode steps of 1 token per sequence.
    "multimodal": Config("multimodal", 5, RAW_VOCAB, 100_000, 5120, 4, (1, 14),
                         (16_000_000, _L14_BASE), 256, 2048,
                         dead_spans_per_seq=2, dead_span_len=576, decode_steps=128),
}


def params_for(cfg: Config) -> List[HashParams]:
    tm0 = int(make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)[0])
    return [make_hash_params(cfg.root, layer, cfg.vocab_c, base, tm0)
            for layer, base in zip(cfg.layers, cfg.prime_bases)]


def dead_span_starts(rng: np.random.Generator, seq_len: int, n_spans: int,
                     span: int) -> List[int]:
    """Non-overlapping span starts; each span is followed by >= 1 text token
    and the sequence starts with >= 1 text token."""
    while True:
        starts = sorted(int(s) for s in rng.integers(1, seq_len - span, n_spans))
        ok = all(b - a >= span + 1 for a, b in zip(starts, starts[1:]))
        if ok and starts[-1] + span < seq_len:
            return starts


def token_batch(cfg: Config, batch: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Tokens u32[T] and cu_seqlens i32[S+1] of one measured batch.

    `batch` selects one of several distinct seeded streams of the same shape.
    DEAD spans ([zLLM] 第四步, image spans) are written as DEAD_TOKEN.
    """
    rng = np.random.default_rng([cfg.root, STREAM_TOKENS, batch])
    if cfg.uniform_tokens:
        tok = rng.integers(0, cfg.map_len, cfg.T, dtype=np.uint32)
    else:
        tok = zipf_tokens(rng, cfg.T, cfg.map_len)
    if cfg.dead_spans_per_seq:
        drng = np.random.default_rng([cfg.root, STREAM_DEAD, batch])
        L = cfg.tokens_per_seq
        for s in range(cfg.n_seqs):
            for st in dead_span_starts(drng, L, cfg.dead_spans_per_seq, cfg.dead_span_len):
                tok[s * L + st: s * L + st + cfg.dead_span_len] = DEAD_TOKEN
    cu = (np.arange(cfg.n_seqs + 1, dtype=np.int64) * cfg.tokens_per_seq).astype(np.int32)
    return tok, cu


def history_prefix_tokens(cfg: Config) -> Tuple[np.ndarray, np.ndarray]:
    """Tokens appended to a reset history before the measured batch (the
    decode config's 3-token Zipf history), with their cu_seqlens."""
    n = cfg.history_prefix
    rng = np.random.default_rng([cfg.root, STREAM_HIST])
    tok = zipf_tokens(rng, cfg.n_seqs * n, cfg.map_len)
    cu = (np.arange(cfg.n_seqs + 1, dtype=np.int64) * n).astype(np.int32)
    return tok, cu


def decode_tokens(cfg: Config, step: int) -> np.ndarray:
    """One decode step's tokens: one Zipf draw per sequence."""
    rng = np.random.default_rng([cfg.root, STREAM_TOKENS, 1000 + step])
    return zipf_tokens(rng, cfg.n_seqs, cfg.map_len)


HIDDEN_CHUNK = 4096


def hidden_bf16(cfg: Config, layer: int, T: int, batch: int = 0, first: int = 0) -> np.ndarray:
    """mHC hidden at layer entry, N(0,1) rounded to BF16: uint16[T][hc][H]
    for token rows [first, first+T). Rows are drawn in chunks of HIDDEN_CHUNK
    tokens, each from its own stream, so any row range can be regenerated
    alone and chunks can be generated in parallel."""
    out = np.empty((T, cfg.hc, cfg.H), dtype=np.uint16)
    if T == 0:
        return out
    for c in range(first // HIDDEN_CHUNK, (first + T - 1) // HIDDEN_CHUNK + 1):
        rng = np.random.default_rng([cfg.root, STREAM_HIDDEN, layer, batch, c])
        x = rng.standard_normal((HIDDEN_CHUNK, cfg.hc, cfg.H), dtype=np.float32)
        a = max(first, c * HIDDEN_CHUNK)
        b = min(first + T, (c + 1) * HIDDEN_CHUNK)
        out[a - first:b - first] = bf16_bits_from_f32(x[a - c * HIDDEN_CHUNK:b - c * HIDDEN_CHUNK])
    return out


def wkv_bf16(cfg: Config, layer: int) -> np.ndarray:
    """wkv N(0, 0.02^2) rounded to BF16: uint16[(hc+1)*H][6144]."""
    rng = np.random.default_rng([cfg.root, STREAM_WKV, layer])
    x = rng.standard_normal(((cfg.hc + 1) * cfg.H, N_BUCKETS * ROW_BYTES), dtype=np.float32)
    x *= np.float32(0.02)
    return bf16_bits_from_f32(x)


def norm_weights(cfg: Config, layer: int) -> np.ndarray:
    """Premultiplied elementwise norm weights w_q*w_k, float32[hc][H]
    ([zLLM] 第三步 stores the product of the q and k weights)."""
    rng = np.random.default_rng([cfg.root, STREAM_NORMW, layer])
    wq = (1.0 + 0.1 * rng.standard_normal((cfg.hc, cfg.H))).astype(np.float32)
    wk = (1.0 + 0.1 * rng.standard_normal((cfg.hc, cfg.H))).astype(np.float32)
    return (wq * wk).astype(np.float32)


def small_table(cfg: Config, layer_index: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Whole table of a small config on the host (Tiny, or tests)."""
    p = params_for(cfg)[layer_index]
    kd, ks = table_keys(cfg.root, cfg.layers[layer_index])
    return table_rows(np.arange(p.n_rows, dtype=np.uint64), kd, ks)
