"""Pins of the oracle to what the Engram pages and mathematics fix.

CPU only. Each group targets a plausible mistake in the oracle (a dropped
term, a wrong index or sign, a transposed operand, double rounding).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import engram_synth as synth
from oracle import engram_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAD = 0


def _facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def _mr_is_prime(n: int) -> bool:
    """Deterministic Miller-Rabin for n < 3.4e14 (bases 2..17); independent of
    the trial division used by the input generator."""
    if n < 2:
        return False
    small = (2, 3, 5, 7, 11, 13, 17)
    if n in small:
        return True
    if any(n % p == 0 for p in small):
        return False
    d, r = n - 1, 0
    while d % 2 == 0:
        d //= 2
        r += 1
    for a in small:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(r - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


# ---------------------------------------------------------------- page facts
def test_layout_facts_from_pages():
    f = _facts()
    assert len(f["ngram_orders"]) * f["heads_per_order"] == f["rows_per_token_per_layer"] == O.N_BUCKETS
    assert tuple(f["ngram_orders"]) == O.ORDERS
    assert f["rows_per_token_per_layer"] * f["row_width"] == f["memory_vector_width"] == O.MEM
    assert f["row_width"] == O.ROW and f["row_width"] % f["scale_group"] == 0
    n_out, k = f["wkv_shape"]
    assert k == O.MEM
    assert n_out == (f["mhc_branches"] + 1) * f["value_rows"]
    assert n_out * k * 2 == f["wkv_bf16_mib_approx"] * 2 ** 20      # exactly 300 MiB
    # 2 layers x 24 rows x 256 one-byte codes per token = 12 KiB
    assert 2 * f["rows_per_token_per_layer"] * f["row_width"] == f["code_kib_per_token_two_layers"] * 1024
    rows2 = f["rows_layer1"] + f["rows_layer14"]
    assert abs(rows2 * 256 / 2 ** 30 - f["code_gib_two_layers_approx"]) < 0.5
    assert abs(f["rows_layer1"] * 256 * 2 / 1e9 - f["bf16_table_gb_approx"]) / f["bf16_table_gb_approx"] < 1e-3
    assert abs(rows2 * (256 + 8) / 1e9 - f["fp8_plus_scales_two_layers_gb_approx"]) < 5


def test_prime_buckets_reproduce_the_pages_row_counts():
    """The 24 smallest primes above engram_vocab_size sum to layer 1's row
    count; the next 24 to layer 14's (the storage page's table)."""
    f = _facts()
    ps = synth.primes_above(f["engram_vocab_size"], 48)
    assert all(_mr_is_prime(p) for p in ps)
    # no prime skipped: every number strictly between consecutive picks is composite
    lo = f["engram_vocab_size"] + 1
    picked = set(ps)
    assert all(_mr_is_prime(n) == (n in picked) for n in range(lo, ps[-1] + 1))
    assert sum(ps[:24]) == f["rows_layer1"]
    assert sum(ps[24:]) == f["rows_layer14"]
    cfg = synth.CONFIGS["long"]
    p1, p14 = synth.params_for(cfg)
    assert p1.n_rows == f["rows_layer1"] and p14.n_rows == f["rows_layer14"]
    assert set(p1.prime.tolist()).isdisjoint(p14.prime.tolist())


@pytest.mark.parametrize("name", ["tiny", "decode", "full", "long"])
def test_bucket_ranges_disjoint_and_cover_table(name):
    for p in synth.params_for(synth.CONFIGS[name]):
        assert len(set(p.prime.tolist())) == 24
        ends = p.offset.astype(np.int64) + p.prime.astype(np.int64)
        assert p.offset[0] == 0 and np.all(p.offset[1:].astype(np.int64) == ends[:-1])
        assert int(ends[-1]) == p.n_rows < 0xFFFFFFFF
        bound = ((1 << 63) - 1) // p.vocab_c
        assert all(int(m) % 2 == 1 and int(m) < bound for m in p.mult.reshape(-1))


def test_token_map_is_a_surjection():
    for name in ("tiny", "decode"):
        cfg = synth.CONFIGS[name]
        m = synth.make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)
        assert len(m) == cfg.map_len and m.max() < cfg.vocab_c
        assert len(np.unique(m)) == cfg.vocab_c
    assert synth.CONFIGS["decode"].map_len == _facts()["token_map_entries"]


# ---------------------------------------------------------------- SplitMix64
def test_splitmix64_known_answers():
    """Published SplitMix64 sequence for state 1234567 (Steele/Lea/Flood;
    Vigna's reference splitmix64.c)."""
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    g = 0x9E3779B97F4A7C15
    got = [synth.splitmix64_int((1234567 + i * g) & synth.MASK64) for i in range(5)]
    assert got == want
    arr = np.array([(1234567 + i * g) & synth.MASK64 for i in range(5)], dtype=np.uint64)
    assert synth.splitmix64_np(arr).tolist() == want


def test_table_rows_closed_form():
    kd, ks = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    rows = np.array([0, 1, 7, 384006167], dtype=np.uint64)
    codes, scales = synth.table_rows(rows, kd, ks)
    for i, r in enumerate(rows.tolist()):
        for c in (0, 1, 128, 255):
            z = synth.splitmix64_int((kd + r * 256 + c) & synth.MASK64)
            assert codes[i, c] == synth.FINITE_E4M3_CODES[(z >> 32) % 254]
        for q in range(8):
            z = synth.splitmix64_int((ks + r * 8 + q) & synth.MASK64)
            assert scales[i, q] == 119 + (z >> 32) % 9
    assert len(synth.FINITE_E4M3_CODES) == 254
    assert 0x7F not in synth.FINITE_E4M3_CODES and 0xFF not in synth.FINITE_E4M3_CODES


# ---------------------------------------------------------------- windows / history
def _parse_slots(txt):
    return [PAD if t == "P" else (O.DEAD_TOKEN if t == "D" else int(t)) for t in txt.split()]


def _hand_cases():
    with open(os.path.join(GOLDEN, "windows_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, h, toks, wins, after = [p.strip() for p in line.split("|")]
            yield (name, _parse_slots(h), _parse_slots(toks),
                   [_parse_slots(w) for w in wins.split(";")], _parse_slots(after))


@pytest.mark.parametrize("case", list(_hand_cases()), ids=lambda c: c[0])
def test_windows_hand_built(case):
    _, h, toks, wins, after = case
    tmap = np.arange(64, dtype=np.uint32)
    tok = np.array(toks, dtype=np.uint32)
    cu = np.array([0, len(toks)], dtype=np.int32)
    win, dead, new_hist = O.walk(tok, cu, np.array([h], dtype=np.uint32), tmap, PAD)
    assert dead.tolist() == [t == O.DEAD_TOKEN for t in toks]
    assert win[~dead].tolist() == wins
    assert new_hist[0].tolist() == after
    # the same after-state through history_append
    assert O.history_append(np.array([h], dtype=np.uint32), tok, cu, tmap, PAD)[0].tolist() == after


def _tiny_world(seed=0, V=1000, T=200, S=1):
    rng = np.random.default_rng(seed)
    tmap = rng.integers(0, V, 4096).astype(np.uint32)
    params = synth.make_hash_params(0xABC + seed, 1, V, 1000, int(tmap[0]))
    tok = rng.integers(0, 4096, T).astype(np.uint32)
    return tmap, params, tok


def _idx(tok, cu, hist, tmap, p):
    win, dead, nh = O.walk(tok, cu, hist, tmap, p.pad_cid)
    return O.hash_windows(win, dead, p.mult, p.prime, p.offset), nh


def test_chunking_invariance_and_append_once():
    """Prefill split as 1 | 2 | 3 | rest (history carried by one append per
    chunk) gives the unsplit indices; appending a chunk twice does not."""
    tmap, p, tok = _tiny_world(1, T=120)
    h0 = O.history_reset(1, p.pad_cid)
    full, _ = _idx(tok, np.array([0, len(tok)], np.int32), h0, tmap, p)
    parts, h = [], h0
    for a, b in [(0, 1), (1, 3), (3, 6), (6, len(tok))]:
        cu = np.array([0, b - a], np.int32)
        i, _ = _idx(tok[a:b], cu, h, tmap, p)
        parts.append(i)
        h = O.history_append(h, tok[a:b], cu, tmap, p.pad_cid)
    assert np.array_equal(np.concatenate(parts), full)
    # token-by-token decode equals prefill
    h, dec = h0, []
    for t in range(len(tok)):
        cu = np.array([0, 1], np.int32)
        dec.append(_idx(tok[t:t + 1], cu, h, tmap, p)[0])
        h = O.history_append(h, tok[t:t + 1], cu, tmap, p.pad_cid)
    assert np.array_equal(np.concatenate(dec), full)
    # the bug the pages warn about: in decode, appending each token at both
    # layers puts it in the history twice and misaligns the n-grams
    one = np.array([0, 1], np.int32)
    h_once, h_twice = h0, h0
    for t in range(5):
        h_once = O.history_append(h_once, tok[t:t + 1], one, tmap, p.pad_cid)
        for _layer in range(2):
            h_twice = O.history_append(h_twice, tok[t:t + 1], one, tmap, p.pad_cid)
    i_once, _ = _idx(tok[5:9], np.array([0, 4], np.int32), h_once, tmap, p)
    i_twice, _ = _idx(tok[5:9], np.array([0, 4], np.int32), h_twice, tmap, p)
    assert np.array_equal(i_once, full[5:9])
    assert not np.array_equal(i_once, i_twice)


def test_fork_isolation():
    tmap, p, tok = _tiny_world(2, T=60)
    root = O.history_reset(1, p.pad_cid)
    parent = O.history_append(root, tok[:10], np.array([0, 10], np.int32), tmap, p.pad_cid)
    snapshot = parent.copy()
    child = O.history_fork(parent)
    child = O.history_append(child, tok[10:20], np.array([0, 10], np.int32), tmap, p.pad_cid)
    assert np.array_equal(parent, snapshot)
    got, _ = _idx(tok[20:30], np.array([0, 10], np.int32), child, tmap, p)
    fresh, _ = _idx(tok[:30], np.array([0, 30], np.int32), root, tmap, p)
    assert np.array_equal(got, fresh[20:30])
    # the parent still continues its own stream
    alt = tok[40:50]
    got_p, _ = _idx(alt, np.array([0, 10], np.int32), parent, tmap, p)
    ref_p, _ = _idx(np.concatenate([tok[:10], alt]), np.array([0, 20], np.int32), root, tmap, p)
    assert np.array_equal(got_p, ref_p[10:])


@pytest.mark.parametrize("span", [1, 2, 576])
def test_dead_breaks_ngrams(span):
    """The 3 text tokens after a DEAD span hash as at a fresh start."""
    tmap, p, tok = _tiny_world(3, T=40)
    stream = np.concatenate([tok[:20], np.full(span, O.DEAD_TOKEN, np.uint32), tok[20:23]])
    h0 = O.history_reset(1, p.pad_cid)
    idx, _ = _idx(stream, np.array([0, len(stream)], np.int32), h0, tmap, p)
    fresh, _ = _idx(tok[20:23], np.array([0, 3], np.int32), h0, tmap, p)
    assert np.array_equal(idx[-3:], fresh)
    assert np.all(idx[20:20 + span] == O.DEAD_IDX)
    valid = idx[idx[:, 0] != O.DEAD_IDX]
    assert valid.shape[0] == 23 and valid.shape[1] == 24


def test_multi_sequence_histories_are_independent():
    tmap, p, tok = _tiny_world(4, T=30)
    cu = np.array([0, 10, 10, 30], np.int32)        # includes an empty sequence
    rng = np.random.default_rng(9)
    hist = rng.integers(0, p.vocab_c, (3, 3)).astype(np.uint32)
    idx, nh = _idx(tok, cu, hist, tmap, p)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        one, h1 = _idx(tok[a:b], np.array([0, b - a], np.int32), hist[s:s + 1], tmap, p)
        assert np.array_equal(idx[a:b], one) and np.array_equal(nh[s], h1[0])


# ---------------------------------------------------------------- hashing
def test_hash_bruteforce_tiny_vocab():
    """V_c = 7: every window of every order; the vectorised hash equals the
    Python-int twin and stays in its bucket's range."""
    V = 7
    p = synth.make_hash_params(77, 1, V, 1000, 0)
    wins = np.array(list(itertools.product(range(V), repeat=4)), dtype=np.uint64)
    dead = np.zeros(len(wins), bool)
    got = O.hash_windows(wins, dead, p.mult, p.prime, p.offset)
    for w, row in zip(wins.tolist()[::7], got[::7].tolist()):
        assert row == O.hash_window_scalar(w, p.mult, p.prime, p.offset)
    lo = p.offset.astype(np.int64)
    hi = lo + p.prime.astype(np.int64)
    assert np.all((got >= lo) & (got < hi))
    # bucket j reads only the first n_j slots: all windows sharing those slots agree
    for j in range(24):
        n = O.bucket_order(j)
        key = wins[:, :n] @ (V ** np.arange(n, dtype=np.uint64))
        for kval in np.unique(key)[:50]:
            assert len(np.unique(got[key == kval, j])) == 1
    # 4-gram buckets see all 4 slots: windows differing only in slot 3 differ somewhere
    a = O.hash_window_scalar([1, 2, 3, 4], p.mult, p.prime, p.offset)
    b = O.hash_window_scalar([1, 2, 3, 5], p.mult, p.prime, p.offset)
    assert a[:16] == b[:16] and a[16:] != b[16:]


def test_hash_xor_of_disjoint_bit_fields():
    """With mult[j][k] = 2^(16k + j%4) and slots < 2^12, the products occupy
    disjoint bit fields, so their XOR is their sum: an independent closed
    form that fails if a slot's multiplier is swapped or a term dropped."""
    mult = np.array([[1 << (16 * k + j % 4) for k in range(4)] for j in range(24)], dtype=np.uint64)
    prime = np.array(synth.primes_above(1000, 24), dtype=np.uint32)
    offset = np.concatenate([[0], np.cumsum(prime[:-1].astype(np.uint64))]).astype(np.uint64)
    rng = np.random.default_rng(5)
    wins = rng.integers(0, 1 << 12, (200, 4)).astype(np.uint64)
    got = O.hash_windows(wins, np.zeros(200, bool), mult, prime, offset)
    for w, row in zip(wins.tolist(), got.tolist()):
        for j in range(24):
            n = 2 + j // 8
            x = sum(w[k] << (16 * k + j % 4) for k in range(n))
            assert row[j] == int(offset[j]) + x % int(prime[j])


def test_hash_special_cases():
    prime = np.array(synth.primes_above(5000, 24), dtype=np.uint32)
    offset = np.concatenate([[0], np.cumsum(prime[:-1].astype(np.uint64))]).astype(np.uint64)
    # multiplier [1,0,0,0]: every bucket reduces the current token alone
    mult = np.zeros((24, 4), np.uint64)
    mult[:, 0] = 1
    w = np.array([[123456, 7, 8, 9]], np.uint64)
    got = O.hash_windows(w, np.zeros(1, bool), mult, prime, offset)[0]
    assert got.tolist() == [int(offset[j]) + 123456 % int(prime[j]) for j in range(24)]
    # products wrap mod 2^64: (2^31+1)(2^40+3) = 2^71 + 2^40 + 3*2^31 + 3
    mult = np.zeros((24, 4), np.uint64)
    mult[:, 0] = (1 << 40) + 3
    w = np.array([[(1 << 31) + 1, 0, 0, 0]], np.uint64)
    got = O.hash_windows(w, np.zeros(1, bool), mult, prime, offset)[0]
    x = (1 << 40) + 3 * (1 << 31) + 3
    assert got.tolist() == [int(offset[j]) + x % int(prime[j]) for j in range(24)]
    assert O.hash_windows(w, np.ones(1, bool), mult, prime, offset)[0].tolist() == [O.DEAD_IDX] * 24


def test_hash_full_range_multipliers_match_big_integer_arithmetic():
    """With 96 distinct full-range multipliers (products wrap past 2^64, XORs
    reach 2^63 and above, each bucket has its own), the vectorised uint64
    hash equals exact arithmetic on Python integers reduced mod 2^64 by hand:
    per bucket j of order n, x = XOR over k < n of (w_k * m[j][k] mod 2^64),
    row = offset[j] + x mod prime[j]."""
    p = synth.make_full_range_hash_params(0xE46A0002, 1, 100_000, 666_666, 0)
    rng = np.random.default_rng(9)
    wins = rng.integers(0, 100_000, (300, 4)).astype(np.uint64)
    got = O.hash_windows(wins, np.zeros(len(wins), bool), p.mult, p.prime, p.offset)
    wrapped = high = 0
    for w, row in zip(wins.tolist(), got.tolist()):
        for j in range(24):
            x = 0
            for k in range(2 + j // 8):
                prod = int(w[k]) * int(p.mult[j][k])
                wrapped += prod >= 1 << 64
                x ^= prod % (1 << 64)
            high += x >= 1 << 63
            assert row[j] == int(p.offset[j]) + x % int(p.prime[j])
    assert wrapped > 1000 and high > 1000       # the inputs do exercise the wrap and the top bit


# ---------------------------------------------------------------- decode
def _fixture_bytes():
    with open(os.path.join(GOLDEN, "e4m3_bytes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, s, v, b = line.split()
            yield int(c, 16), int(s), v, int(b, 16)


@pytest.mark.parametrize("case", list(_fixture_bytes()), ids=lambda c: f"{c[0]:#04x}_{c[1]}")
def test_decode_hand_built_bytes(case):
    code, scale, v, bits = case
    codes = np.full((1, 256), code, np.uint8)
    scales = np.full((1, 8), scale, np.uint8)
    val = O.decode_rows(codes, scales)[0, 0]
    if v == "nan":
        assert math.isnan(val)
    else:
        assert val == float(v) and math.copysign(1, val) == math.copysign(1, float(v))
    assert int(O.bf16_rne(np.array([val]))[0]) == bits


def test_decode_matches_torch_float8_types_exhaustively():
    """E4M3 values vs torch.float8_e4m3fn, E8M0 vs torch.float8_e8m0fnu, and
    the full 256 x 256 (code, scale) grid of decoded BF16 against the torch
    values' product rounded by torch (the products are exact in float32)."""
    b = torch.arange(256, dtype=torch.uint8)
    e4 = b.view(torch.float8_e4m3fn).double().numpy()
    e8 = b.view(torch.float8_e8m0fnu).double().numpy()
    mine4 = np.array([O.e4m3_value(c) for c in range(256)])
    mine8 = np.array([O.e8m0_value(s) for s in range(256)])
    assert np.array_equal(np.isnan(mine4), np.isnan(e4))
    assert np.array_equal(mine4[~np.isnan(e4)], e4[~np.isnan(e4)])
    assert np.array_equal(np.signbit(mine4[~np.isnan(e4)]), np.signbit(e4[~np.isnan(e4)]))
    assert np.array_equal(np.isnan(mine8), np.isnan(e8))
    assert np.array_equal(mine8[~np.isnan(e8)], e8[~np.isnan(e8)])
    all_codes = np.arange(256, dtype=np.uint8).reshape(1, 256)     # one row holding every code
    for s in range(256):
        row = O.bf16_rne(O.decode_rows(all_codes, np.full((1, 8), s, np.uint8)))[0]
        prod = torch.from_numpy((e4 * e8[s]).astype(np.float64))
        finite = np.isfinite(prod.numpy())
        # exact product fits float32 unless it overflows or underflows float32's subnormals
        ok = finite & (np.abs(prod.numpy()) < 3.0e38) & ((prod.numpy() == 0) | (np.abs(prod.numpy()) >= 2.0 ** -149))
        ref = prod.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(row[ok], ref[ok]), s
        nan_ref = np.isnan(prod.numpy())
        assert np.all((row[nan_ref] & 0x7FFF) == 0x7FC0)
        assert np.array_equal(row[nan_ref] >> 15, (np.arange(256)[nan_ref] >> 7).astype(np.uint16))


def test_decode_scale_groups_of_32():
    codes = np.full((1, 256), 0x38, np.uint8)             # 1.0 everywhere
    scales = np.arange(120, 128, dtype=np.uint8).reshape(1, 8)
    vals = O.decode_rows(codes, scales)[0]
    for q in range(8):
        assert np.all(vals[32 * q: 32 * q + 32] == 2.0 ** (120 + q - 127))
    one = O.decode_rows(np.full((1, 256), 0x38, np.uint8), np.full((1, 8), 120, np.uint8))[0, :32]
    assert np.all(one == 2.0 ** -7)


def test_bf16_rne_against_torch_and_double_rounding():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    f32 = bits.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_rne(f32.astype(np.float64))
    assert np.array_equal(got, ref)
    # ties to even, and no double rounding through float32
    cases = {1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82, 1 + 2 ** -8 + 2 ** -40: 0x3F81,
             -(1 + 2 ** -8 + 2 ** -40): 0xBF81, 2.0 ** -133: 0x0001, 1.5 * 2.0 ** -133: 0x0002,
             0.5 * 2.0 ** -133: 0x0000, 0.5 * 2.0 ** -133 + 2.0 ** -180: 0x0001,
             3.3895313892515355e38: 0x7F7F, 2.0 ** 128: 0x7F80, -0.0: 0x8000}
    for x, want in cases.items():
        assert int(O.bf16_rne(np.array([x]))[0]) == want, x
    assert int(O.bf16_rne(np.array([np.inf]))[0]) == 0x7F80
    assert int(O.bf16_rne(np.array([-np.inf]))[0]) == 0xFF80


def test_gather_decode_places_bucket_j_at_j_times_256():
    rows_seen = []

    def src(rows):
        rows_seen.append(rows.copy())
        r = rows.astype(np.int64)
        codes = np.zeros((len(r), 256), np.uint8)
        codes[:, 0] = 0x38                                # 1.0 at column 0
        codes[:, 1] = (0x38 + (r % 8)).astype(np.uint8)     # 1 + (r%8)/8 at column 1
        scales = np.full((len(r), 8), 127, np.uint8)
        return codes, scales
    idx = np.array([np.arange(24) * 10 + 3, [O.DEAD_IDX] * 24], dtype=np.uint32)
    mem = O.gather_decode(idx, src)
    vals = O.bf16_to_f64(mem)
    for j in range(24):
        r = j * 10 + 3
        assert vals[0, j * 256] == 1.0 and vals[0, j * 256 + 1] == 1 + (r % 8) / 8
    assert np.all(mem[1] == 0)
    assert rows_seen[0].tolist() == (np.arange(24) * 10 + 3).tolist()


# ---------------------------------------------------------------- projection
def test_projection_one_hot_selects_a_column():
    rng = np.random.default_rng(3)
    wkv = synth.bf16_bits_from_f32(rng.standard_normal((40, 6144)).astype(np.float32))
    mem = np.zeros((3, 6144), np.uint16)
    cols = [0, 777, 6143]
    for t, c in enumerate(cols):
        mem[t, c] = 0x3F80                                   # 1.0
    kv = O.project(mem, wkv)
    for t, c in enumerate(cols):
        assert np.array_equal(kv[t], wkv[:, c])


def test_projection_integer_inputs_exact():
    """Small-integer operands make the float64 product exact; compare with an
    int64 matmul (non-square, so a transposed operand fails), then RNE."""
    rng = np.random.default_rng(4)
    mi = rng.integers(-3, 4, (5, 6144))
    wi = rng.integers(-3, 4, (37, 6144))
    mem = synth.bf16_bits_from_f32(mi.astype(np.float32))
    wkv = synth.bf16_bits_from_f32(wi.astype(np.float32))
    exact = mi.astype(np.int64) @ wi.astype(np.int64).T
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.all(np.abs(exact) < 2 ** 24)                  # exact in float32 too
    assert np.array_equal(O.project(mem, wkv), ref)


# ---------------------------------------------------------------- gate
def test_gate_closed_form_values():
    with open(os.path.join(GOLDEN, "gate_closed_form.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for d, g in rows:
        assert abs(O.gate_from_dot(float(d)) - float(g)) < 1e-10, d
    for x in (1e-3, 0.5, 3.0, 50.0):
        assert abs(O.gate_from_dot(-x) - (1 - O.gate_from_dot(x))) < 1e-15
        assert 0 < O.gate_from_dot(-x) < 0.5 < O.gate_from_dot(x) < 1


def _gate_inputs(T=3, H=256, hc=4, seed=0):
    rng = np.random.default_rng(seed)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    kv = synth.bf16_bits_from_f32(rng.standard_normal((T, (hc + 1) * H)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    return hidden, kv, wqk


def test_gate_dot_closed_form_when_key_equals_hidden():
    """h_b = k_b, wqk = 1, s = 1: dot = H * m / (m + eps), m = mean(h^2)."""
    H, hc, eps = 256, 4, 1e-6
    hidden, kv, _ = _gate_inputs(H=H)
    kv[:, : hc * H] = hidden.reshape(hidden.shape[0], -1)
    dots = O.gate_dots(hidden, kv, np.ones((hc, H), np.float32), H, hc, eps, 1.0)
    h = O.bf16_to_f64(hidden)
    m = np.mean(h * h, axis=2)
    assert np.allclose(dots, H * m / (m + eps), rtol=1e-12)
    dots_s = O.gate_dots(hidden, kv, np.ones((hc, H), np.float32), H, hc, eps, 1 / 16)
    assert np.allclose(dots_s, dots / 16, rtol=1e-12)


def test_gate_scale_invariance_and_sign():
    H, hc = 256, 4
    hidden, kv, wqk = _gate_inputs(H=H, seed=1)
    d0 = O.gate_dots(hidden, kv, wqk, H, hc, 1e-30, 1.0)
    h4 = O.bf16_rne(O.bf16_to_f64(hidden) * 4)             # power of two: exact
    k8 = kv.copy()
    k8[:, : hc * H] = O.bf16_rne(O.bf16_to_f64(kv[:, : hc * H]) / 8)
    assert np.allclose(O.gate_dots(h4, k8, wqk, H, hc, 1e-30, 1.0), d0, rtol=1e-12)
    kneg = kv.copy()
    kneg[:, : hc * H] ^= 0x8000                             # negate the keys only
    assert np.allclose(O.gate_dots(hidden, kneg, wqk, H, hc, 1e-30, 1.0), -d0, rtol=1e-12)
    # each branch uses its own key: swapping branch 0's and 1's keys swaps their dots
    ksw = kv.copy()
    ksw[:, :H], ksw[:, H:2 * H] = kv[:, H:2 * H], kv[:, :H]
    hsw = hidden.copy()
    hsw[:, 0], hsw[:, 1] = hidden[:, 1], hidden[:, 0]
    wsw = wqk[[1, 0, 2, 3]]
    d1 = O.gate_dots(hsw, ksw, wsw, H, hc, 1e-30, 1.0)
    assert np.allclose(d1[:, [1, 0, 2, 3]], d0, rtol=1e-12)


def test_gate_dot_per_branch_weight_constants():
    """wqk[b] = c_b everywhere, h_b = k_b, s = 1: dot_b = c_b * H * m_b / (m_b + eps)
    with m_b = mean(h_b^2). Distinct c_b per branch, so a dropped weight or a
    weight taken from another branch changes every dot ([zLLM] 第三步: each
    branch carries its own premultiplied q/k weights)."""
    H, hc, eps = 256, 4, 1e-6
    hidden, kv, _ = _gate_inputs(H=H, seed=5)
    kv[:, : hc * H] = hidden.reshape(hidden.shape[0], -1)
    c = np.array([0.5, 1.25, 2.0, 3.0], np.float32)
    wqk = np.repeat(c[:, None], H, axis=1).astype(np.float32)
    dots = O.gate_dots(hidden, kv, wqk, H, hc, eps, 1.0)
    h = O.bf16_to_f64(hidden)
    m = np.mean(h * h, axis=2)
    assert np.allclose(dots, c[None, :] * H * m / (m + eps), rtol=1e-12)


def test_gate_dot_one_hot_weight_selects_one_product():
    """Hidden entries +-a and key entries +-k (so RMS a and k exactly, eps -> 0)
    and a one-hot wqk[b] = w_b at column i_b: dot_b = s * sign(h_i k_i) * w_b,
    whatever a and k. Each branch has its own column and weight, so the
    weights of the wrong branch, or no weights, give other values."""
    H, hc, T = 128, 4, 3
    rng = np.random.default_rng(11)
    a, kmag = 0.5, 2.0                                        # exact in BF16
    hs = rng.choice([-1.0, 1.0], (T, hc, H))
    ks = rng.choice([-1.0, 1.0], (T, hc, H))
    hidden = O.bf16_rne(a * hs)
    kv = np.zeros((T, (hc + 1) * H), np.uint16)
    kv[:, : hc * H] = O.bf16_rne(kmag * ks).reshape(T, hc * H)
    cols = [3, 70, 101, 127]
    w = [0.75, -1.5, 2.5, 4.0]
    wqk = np.zeros((hc, H), np.float32)
    for b in range(hc):
        wqk[b, cols[b]] = w[b]
    for s in (1.0, 1 / 16):
        dots = O.gate_dots(hidden, kv, wqk, H, hc, 0.0, s)
        for t in range(T):
            for b in range(hc):
                want = s * hs[t, b, cols[b]] * ks[t, b, cols[b]] * w[b]
                assert dots[t, b] == pytest.approx(want, rel=1e-12), (t, b)


def test_residual_closed_form_and_pass_through():
    H, hc = 256, 4
    T = 2
    hidden = np.full((T, hc, H), 0x3F80, np.uint16)         # 1.0
    kv = np.zeros((T, (hc + 1) * H), np.uint16)
    kv[:, : hc * H] = 0x3F80                                 # keys 1.0 -> dot = H/(1+eps) ~ 256
    kv[:, hc * H:] = 0x3E00                                  # value 0.125
    wqk = np.ones((hc, H), np.float32)
    dead = np.array([False, True])
    new, g, _ = O.gate_residual(hidden, kv, wqk, dead, H, hc, 1e-6, 1.0)
    # gate = sigmoid(~16) = 0.99999989; 1 + 0.125 g rounds to 1.125 = 0x3F90
    assert np.all(new[0] == 0x3F90)
    assert np.all(new[1] == hidden[1]) and np.all(g[1] == 0)
    assert abs(g[0, 0] - 1 / (1 + math.exp(-16))) < 1e-9
    # zero value leaves hidden bit-identical
    h2, kv2, wqk2 = _gate_inputs(H=H, seed=2)
    kv2[:, hc * H:] = 0
    new2, _, _ = O.gate_residual(h2, kv2, wqk2, np.zeros(3, bool), H, hc, 1e-6, 1.0)
    assert np.array_equal(new2, h2)


# ---------------------------------------------------------------- whole layer
def test_forward_tiny_consistency():
    cfg = synth.CONFIGS["tiny"]
    tmap = synth.make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)
    (p,) = synth.params_for(cfg)
    kd, ks = synth.table_keys(cfg.root, cfg.layers[0])
    tok, cu = synth.token_batch(cfg)
    hist = O.history_reset(cfg.n_seqs, p.pad_cid)
    wkv = synth.wkv_bf16(cfg, cfg.layers[0])
    wqk = synth.norm_weights(cfg, cfg.layers[0])
    hidden = synth.hidden_bf16(cfg, cfg.layers[0], cfg.T)
    out = O.forward(tok, cu, hist, tmap, p, lambda r: synth.table_rows(r, kd, ks),
                    wkv, wqk, hidden, cfg.H, cfg.hc)
    assert out["idx"].shape == (64, 24) and out["mem"].shape == (64, 6144)
    assert out["kv"].shape == (64, 1280) and out["hidden"].shape == (64, 4, 256)
    assert np.all((out["gate"] > 0) & (out["gate"] < 1))
    # the memory vector is the decoded gathered rows
    codes, scales = synth.table_rows(out["idx"][5].astype(np.uint64), kd, ks)
    assert np.array_equal(out["mem"][5], O.bf16_rne(O.decode_rows(codes, scales)).reshape(-1))
