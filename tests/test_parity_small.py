"""GPU parity of every stage against the oracle at sizes the oracle finishes
in seconds (several tiles plus ragged tails), through the C ABI.

Bars: hash indices, decoded rows, history and tables bit-exact; k/v and
hidden within 2e-2 * max(|ref|, rms(ref row)); gate within 1e-3.
"""
import numpy as np
import pytest
import torch

import engram_synth as synth
from oracle import engram_oracle as O
from tests.conftest import gpu_available
from tests.gpu_helpers import (DEV, World, assert_bf16_close, check_gate_rows, device_table, down16,
                               down32, log,
                               forward_rows, up8, up16, up32, upf, workspace_views, live_positions)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_amd as E
    return E


def _gpu_hash(E, tok, cu, hist, tmap, p, err=None):
    T = len(tok)
    idx = torch.empty(T * 24, dtype=torch.int32, device=DEV)
    E.engram_hash(up32(tok), up32(cu), up32(hist), up32(tmap), p, idx, err_flags=err)
    return down32(idx).reshape(T, 24)


def _ref_hash(tok, cu, hist, tmap, p):
    win, dead, _ = O.walk(tok, cu, hist, tmap, p.pad_cid)
    return O.hash_windows(win, dead, p.mult, p.prime, p.offset)


# ---------------------------------------------------------------- tables
def test_gen_table_matches_the_closed_form(E):
    log("gen_table: tiny table, and rows at an offset")
    w = World.of("tiny")
    n = w.params[0].n_rows
    kd, ks = w.keys[0]
    codes, scales = device_table(E, n, kd, ks)
    rc, rs = synth.table_rows(np.arange(n, dtype=np.uint64), kd, ks)
    assert np.array_equal(codes.cpu().numpy().reshape(n, 256), rc)
    assert np.array_equal(scales.cpu().numpy().reshape(n, 8), rs)
    # a window of rows deep inside a 384M-row table, written through row_begin
    begin, cnt = 384_006_168 - 1000, 1000
    c2 = torch.empty(cnt * 256, dtype=torch.uint8, device=DEV)
    s2 = torch.empty(cnt * 8, dtype=torch.uint8, device=DEV)
    E.engram_gen_table(c2, s2, begin, cnt, kd, ks)
    rc, rs = synth.table_rows(np.arange(begin, begin + cnt, dtype=np.uint64), kd, ks)
    assert np.array_equal(c2.cpu().numpy().reshape(cnt, 256), rc)
    assert np.array_equal(s2.cpu().numpy().reshape(cnt, 8), rs)


# ---------------------------------------------------------------- decode
def test_decode_exhaustive_code_scale_grid(E):
    """Row r holds all 256 codes with every scale = r, so gathering rows
    0..255 decodes every (code, scale) pair, NaN and subnormals included."""
    log("gather_decode: exhaustive 256 x 256 (code, scale)")
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    T = 11
    idx = np.full(T * 24, O.DEAD_IDX, dtype=np.uint32)
    idx[:256] = np.arange(256)
    mem = torch.empty(T * 6144, dtype=torch.int16, device=DEV)
    E.engram_gather_decode(up32(idx), up8(codes), up8(scales), 256, mem)
    got = down16(mem).reshape(T * 24, 256)
    ref = O.bf16_rne(O.decode_rows(codes, scales))
    assert np.array_equal(got[:256], ref)
    assert np.all(got[256:] == 0)                    # DEAD rows give zeros


def test_gather_decode_tiny_and_error_flags(E):
    log("gather_decode: tiny config")
    w = World.of("tiny")
    p = w.params[0]
    tok, cu = synth.token_batch(w.cfg)
    hist = O.history_reset(1, p.pad_cid)
    idx = _ref_hash(tok, cu, hist, w.tmap, p)
    idx[7] = O.DEAD_IDX
    kd, ks = w.keys[0]
    codes, scales = device_table(E, p.n_rows, kd, ks)
    mem = torch.empty(len(tok) * 6144, dtype=torch.int16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    E.engram_gather_decode(up32(idx), codes, scales, p.n_rows, mem, err_flags=err)
    ref = O.gather_decode(idx, w.rows(0))
    assert np.array_equal(down16(mem).reshape(-1, 6144), ref)
    assert int(err.item()) == 0
    bad = idx.copy()
    bad[3, 5] = p.n_rows + 2                          # beyond the table: flagged, row zeroed
    E.engram_gather_decode(up32(bad), codes, scales, p.n_rows, mem, err_flags=err)
    assert int(err.item()) & 0x4
    got = down16(mem).reshape(-1, 24, 256)
    assert np.all(got[3, 5] == 0)
    assert np.array_equal(got[3, 4], ref.reshape(-1, 24, 256)[3, 4])


# ---------------------------------------------------------------- hashing and history
def test_hash_tiny(E):
    log("hash: tiny config")
    w = World.of("tiny")
    p = w.params[0]
    tok, cu = synth.token_batch(w.cfg)
    hist = O.history_reset(1, p.pad_cid)
    assert np.array_equal(_gpu_hash(E, tok, cu, hist, w.tmap, p), _ref_hash(tok, cu, hist, w.tmap, p))


def _ragged_batch(seed, lens, map_len, vocab_c, dead_spans=True):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tok = synth.zipf_tokens(rng, int(cu[-1]), map_len)
    if dead_spans:
        for s, L in enumerate(lens):
            if L >= 8:
                a = int(cu[s]) + int(rng.integers(1, L - 3))
                tok[a: a + int(rng.integers(1, 3))] = O.DEAD_TOKEN
        tok[int(cu[-1]) - 1] = O.DEAD_TOKEN            # a DEAD as the very last token
    hist = rng.integers(0, vocab_c, (len(lens), 3)).astype(np.uint32)
    return tok, cu, hist


def test_hash_ragged_sequences_dead_and_history(E):
    log("hash: ragged multi-sequence batch with DEAD spans and carried history")
    w = World.of("decode")
    p = w.params[0]
    tok, cu, hist = _ragged_batch(1, [0, 1, 2, 3, 5, 37, 300, 0, 4000], w.cfg.map_len, p.vocab_c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = _gpu_hash(E, tok, cu, hist, w.tmap, p, err)
    assert np.array_equal(got, _ref_hash(tok, cu, hist, w.tmap, p))
    assert int(err.item()) == 0


def test_hash_long_prefill_both_layers(E):
    log("hash: 50,032-token prefill, layers 1 and 14")
    w = World.of("long")
    tok, cu = synth.token_batch(w.cfg)
    for p in w.params:
        hist = O.history_reset(1, p.pad_cid)
        assert np.array_equal(_gpu_hash(E, tok, cu, hist, w.tmap, p), _ref_hash(tok, cu, hist, w.tmap, p))


def test_hash_flags_out_of_range_tokens(E):
    w = World.of("tiny")
    p = w.params[0]
    tok = np.array([1, 2, 4096, 3], dtype=np.uint32)        # 4096 >= map_len
    cu = np.array([0, 4], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _gpu_hash(E, tok, cu, O.history_reset(1, p.pad_cid), w.tmap, p, err)
    assert int(err.item()) & 0x1


def test_history_append_fork_reset(E):
    log("history: append / fork / reset over several steps")
    w = World.of("decode")
    p = w.params[0]
    lens = [0, 1, 2, 3, 4, 9, 50, 1]
    S = len(lens)
    hist_d = torch.empty(S * 3, dtype=torch.int32, device=DEV)
    E.engram_history_reset(hist_d, p.pad_cid)
    ref = O.history_reset(S, p.pad_cid)
    assert np.array_equal(down32(hist_d).reshape(S, 3), ref)
    tmap_d = up32(w.tmap)
    for step in range(4):
        tok, cu, _ = _ragged_batch(10 + step, lens, w.cfg.map_len, p.vocab_c)
        E.engram_history_append(hist_d, up32(tok), up32(cu), tmap_d, p.pad_cid)
        ref = O.history_append(ref, tok, cu, w.tmap, p.pad_cid)
        assert np.array_equal(down32(hist_d).reshape(S, 3), ref), step
    child = torch.empty_like(hist_d)
    E.engram_history_fork(child, hist_d)
    parent_before = down32(hist_d).copy()
    tok, cu, _ = _ragged_batch(99, lens, w.cfg.map_len, p.vocab_c)
    E.engram_history_append(child, up32(tok), up32(cu), tmap_d, p.pad_cid)
    assert np.array_equal(down32(hist_d), parent_before)
    assert np.array_equal(down32(child).reshape(S, 3),
                          O.history_append(parent_before.reshape(S, 3), tok, cu, w.tmap, p.pad_cid))


# ---------------------------------------------------------------- projection
def _mem_from_tiny(T, seed=0):
    w = World.of("tiny")
    p = w.params[0]
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, w.cfg.map_len, T).astype(np.uint32)
    cu = np.array([0, T], np.int32)
    idx = _ref_hash(tok, cu, O.history_reset(1, p.pad_cid), w.tmap, p)
    return O.gather_decode(idx, w.rows(0))


@pytest.mark.parametrize("T", [1, 16, 17, 33, 63, 64, 65, 128, 129, 192, 193, 256, 257, 300])
def test_project_tiny_widths(E, T):
    """Every skinny configuration (T <= 16, 32, 64, 128, 192, 256) and the
    switch to 256 x 256 tiles above T = 256, each at its edges."""
    log(f"project: tiny wkv (1,280 x 6,144), T={T}")
    cfg = synth.CONFIGS["tiny"]
    wkv = synth.wkv_bf16(cfg, 1)
    mem = _mem_from_tiny(T, seed=T)
    kv = torch.empty(T * 1280, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), cfg.H, cfg.hc, kv)
    assert_bf16_close(down16(kv).reshape(T, -1), O.project(mem, wkv), what="kv")


def test_project_one_hot_is_exact(E):
    cfg = synth.CONFIGS["tiny"]
    wkv = synth.wkv_bf16(cfg, 1)
    T = 70
    mem = np.zeros((T, 6144), np.uint16)
    cols = np.random.default_rng(0).integers(0, 6144, T)
    mem[np.arange(T), cols] = 0x3F80
    kv = torch.empty(T * 1280, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), cfg.H, cfg.hc, kv)
    assert np.array_equal(down16(kv).reshape(T, -1), wkv[:, cols].T)


def test_project_ragged_n(E):
    """N = (hc+1)*H = 192 is not a multiple of the 128-wide tile."""
    rng = np.random.default_rng(5)
    H, hc, T = 64, 2, 130
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32))
    mem = synth.bf16_bits_from_f32(rng.standard_normal((T, 6144)).astype(np.float32))
    kv = torch.empty(T * (hc + 1) * H, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), H, hc, kv)
    assert_bf16_close(down16(kv).reshape(T, -1), O.project(mem, wkv), what="kv")


@pytest.mark.parametrize("T", [1024, 1100, 2600])
def test_project_large_t_tiny_width(E, T):
    """Large T: several 256-row tiles of the wave-tile kernel plus a ragged tail."""
    log(f"project (256x256 tiles): tiny wkv, T={T}")
    cfg = synth.CONFIGS["tiny"]
    wkv = synth.wkv_bf16(cfg, 1)
    rng = np.random.default_rng(T)
    mem = synth.bf16_bits_from_f32(rng.standard_normal((T, 6144)).astype(np.float32) * 0.1)
    kv = torch.empty(T * 1280, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), cfg.H, cfg.hc, kv)
    assert_bf16_close(down16(kv).reshape(T, -1), O.project(mem, wkv), what="kv")


def test_project_large_t_ragged_n(E):
    rng = np.random.default_rng(6)
    H, hc, T = 64, 2, 1030
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32))
    mem = synth.bf16_bits_from_f32(rng.standard_normal((T, 6144)).astype(np.float32))
    kv = torch.empty(T * (hc + 1) * H, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), H, hc, kv)
    assert_bf16_close(down16(kv).reshape(T, -1), O.project(mem, wkv), what="kv")


def test_project_full_size_sampled_rows(E):
    """4,096 tokens x full wkv (the full-size prefill shape): rows sampled at
    tile edges and at random are compared with the oracle. The 1,600 tiles
    are six full groups of 256 in the XCD-interleaved order plus a partial
    group in plain order; kv starts as NaN, and no NaN may survive, so every
    tile was written."""
    log("project: 4,096 x 25,600 x 6,144, sampled rows")
    cfg = synth.CONFIGS["full"]
    T = 4096
    wkv = synth.wkv_bf16(cfg, 1)
    rng = np.random.default_rng(11)
    mem = synth.bf16_bits_from_f32(rng.standard_normal((T, 6144)).astype(np.float32) * 0.1)
    kv = torch.full((T * 25600,), 0x7FC1, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), cfg.H, cfg.hc, kv)
    assert not torch.isnan(kv.view(torch.bfloat16)).any().item(), "tile left unwritten"
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 257, 2047, 2048, 4094, 4095],
                                     rng.integers(0, T, 53)]))
    got = down16(kv).reshape(T, -1)[rows]
    assert_bf16_close(got, O.project(mem[rows], wkv), what="kv")


@pytest.mark.parametrize("T", [64, 128, 129, 192, 256, 257])
def test_project_full_width(E, T):
    log(f"project: full wkv 25,600 x 6,144, T={T}")
    cfg = synth.CONFIGS["decode"]
    wkv = synth.wkv_bf16(cfg, 1)
    mem = synth.bf16_bits_from_f32(
        np.random.default_rng(T).standard_normal((T, 6144)).astype(np.float32) * 0.1)
    kv = torch.empty(T * 25600, dtype=torch.int16, device=DEV)
    E.engram_project(up16(mem), up16(wkv), cfg.H, cfg.hc, kv)
    assert_bf16_close(down16(kv).reshape(T, -1), O.project(mem, wkv), what="kv")


# ---------------------------------------------------------------- packed decode layout
def _packed_index(N):
    """Index in the packed buffer of every value of wkv[N][6144], written out
    from the layout that include/engram.h states for engram_pack_wkv."""
    G = min(112, max(16, -(-N // 256)))
    n = torch.arange(N, device=DEV, dtype=torch.int64)
    grp = n // G
    lr = n - grp * G
    glim = torch.clamp(N - grp * G, max=G)
    t0 = (lr // 16) * 16
    i = lr - t0
    r = torch.clamp(glim - t0, max=16)
    n0 = grp * G + t0
    k = torch.arange(6144, device=DEV, dtype=torch.int64)
    s, g, j, e = k // 64, (k % 64) // 16, (k % 16) // 8, k % 8
    inner = ((2 * s + j) * 4 + g)[None, :] * r[:, None] + i[:, None]
    return n0[:, None] * 6144 + inner * 8 + e[None, :]


@pytest.mark.parametrize("H,hc", [(64, 1), (256, 4), (64, 2), (5120, 1), (5120, 4), (5120, 8),
                                  (2624, 1), (2752, 1)])
def test_pack_wkv_matches_the_stated_layout(E, H, hc):
    """engram_pack_wkv is the stated permutation: groups of 16-112 rows (the
    last one short for hc = 8: 46,080 rows = 411 x 112 + 48), 16-row tiles
    with a short last tile per group (5,248 rows: groups of 21 = 16 + 5, the
    last of 19 = 16 + 3; 5,504 rows: groups of 22, the last of 4), and every
    value moved exactly once."""
    N = (hc + 1) * H
    log(f"pack_wkv: N={N}")
    gen = torch.Generator(device=DEV).manual_seed(N)
    wkv = torch.randint(-32768, 32767, (N, 6144), dtype=torch.int16, device=DEV, generator=gen)
    packed = E.engram_pack_wkv(wkv, H, hc)
    idx = _packed_index(N).reshape(-1)
    assert int(idx.min().item()) >= 0 and int(idx.max().item()) < N * 6144
    seen = torch.zeros(N * 6144, dtype=torch.bool, device=DEV)
    seen[idx] = True     # N * 6144 indices reaching every slot: a permutation
    assert bool(seen.all().item()), "layout is not a permutation"
    want = torch.empty(N * 6144, dtype=torch.int16, device=DEV)
    want[idx] = wkv.reshape(-1)
    assert torch.equal(packed.reshape(-1), want)


@pytest.mark.parametrize("H,hc", [(5120, 4), (256, 4), (64, 2), (5120, 1), (5120, 8), (2624, 1),
                                  (2752, 1)])
def test_project_packed_matches_unpacked_bit_for_bit(E, H, hc):
    """Every decode configuration (T <= 16 .. 256) reads the packed layout with
    the same fragments in the same order as wkv itself, so kv is
    bit-identical; T = 257 uses the 256 x 256 tiles, which ignore it. Sampled
    rows of each T are also checked against the oracle. Small N leaves waves
    of a workgroup without rows (N = 192: one 16-row tile per group)."""
    N = (hc + 1) * H
    rng = np.random.default_rng(N)
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal((N, 6144)).astype(np.float32))
    wkv_d = up16(wkv)
    packed = E.engram_pack_wkv(wkv_d, H, hc)
    for T in (1, 16, 17, 33, 64, 65, 128, 129, 192, 193, 256, 257):
        log(f"project packed vs unpacked: N={N} T={T}")
        mem = synth.bf16_bits_from_f32(rng.standard_normal((T, 6144)).astype(np.float32) * 0.1)
        mem_d = up16(mem)
        a = torch.full((T * N,), 0x7FC1, dtype=torch.int16, device=DEV)
        b = torch.full((T * N,), 0x7FC1, dtype=torch.int16, device=DEV)
        E.engram_project(mem_d, wkv_d, H, hc, a)
        E.engram_project(mem_d, wkv_d, H, hc, b, wkv_packed=packed)
        torch.cuda.synchronize()
        assert not torch.isnan(b.view(torch.bfloat16)).any().item(), T
        assert torch.equal(a, b), T
        rows = np.unique(np.array([0, T // 2, T - 1]))
        assert_bf16_close(down16(b).reshape(T, N)[rows], O.project(mem[rows], wkv), what="kv")


# ---------------------------------------------------------------- gate
@pytest.mark.parametrize("dot_scale", [1.0, 1 / 16.0])
@pytest.mark.parametrize("H,hc", [(256, 4), (64, 1), (5120, 4), (128, 8)])
def test_gate_identical_inputs(E, H, hc, dot_scale):
    log(f"gate: H={H} hc={hc} dot_scale={dot_scale}")
    T = 67
    rng = np.random.default_rng(H + hc)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    kv = synth.bf16_bits_from_f32(rng.standard_normal((T, (hc + 1) * H)).astype(np.float32))
    # a few rows whose key equals hidden (large positive dot) or its negation
    kv[1, : hc * H] = hidden[1].reshape(-1)
    kv[2, : hc * H] = hidden[2].reshape(-1) ^ 0x8000
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    tok = rng.integers(0, 1000, T).astype(np.uint32)
    tok[[0, 5, 6, T - 1]] = O.DEAD_TOKEN
    dead = tok == O.DEAD_TOKEN
    h_d = up16(hidden)
    g_d = torch.empty(T * hc, dtype=torch.float32, device=DEV)
    E.engram_gate(h_d, up16(kv), upf(wqk), up32(tok), H, hc, 1e-6, dot_scale, gate_out=g_d)
    new, g, _ = O.gate_residual(hidden, kv, wqk, dead, H, hc, 1e-6, dot_scale)
    got_g = g_d.cpu().numpy().reshape(T, hc)
    assert np.max(np.abs(got_g - g)) <= 1e-3
    got_h = down16(h_d).reshape(T, hc, H)
    assert np.array_equal(got_h[dead], hidden[dead])          # DEAD rows bit-identical
    assert np.all(got_g[dead] == 0)
    assert_bf16_close(got_h.reshape(T * hc, H), new.reshape(T * hc, H), what="hidden")


def test_gate_without_dead_mask_and_zero_value(E):
    H, hc, T = 256, 4, 9
    rng = np.random.default_rng(3)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    kv = synth.bf16_bits_from_f32(rng.standard_normal((T, (hc + 1) * H)).astype(np.float32))
    kv[:, hc * H:] = 0
    h_d = up16(hidden)
    E.engram_gate(h_d, up16(kv), upf(np.ones((hc, H), np.float32)), None, H, hc)
    assert np.array_equal(down16(h_d).reshape(T, hc, H), hidden)


# ---------------------------------------------------------------- whole layer
def _run_forward(E, w, li, tok, cu, hist, hidden, dot_scale=1.0, packed=False):
    cfg, p = w.cfg, w.params[li]
    kd, ks = w.keys[li]
    codes, scales = device_table(E, p.n_rows, kd, ks)
    wkv = synth.wkv_bf16(cfg, cfg.layers[li])
    wqk = synth.norm_weights(cfg, cfg.layers[li])
    T = len(tok)
    h_d = up16(hidden)
    g_d = torch.empty(T * cfg.hc, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    wkv_d = up16(wkv)
    wkv_p = E.engram_pack_wkv(wkv_d, cfg.H, cfg.hc) if packed else None
    ws = E.engram_forward(up32(tok), up32(cu), up32(hist), up32(w.tmap), p, codes, scales,
                          wkv_d, upf(wqk), h_d, cfg.H, cfg.hc, 1e-6, dot_scale,
                          gate_out=g_d, err_flags=err, wkv_packed=wkv_p)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert T <= 1024 and len(cu) - 1 <= 1024   # rows kept in position order
    idx_d, _, mem_d, kv_d = workspace_views(ws, T, cfg.H, cfg.hc)
    idx = down32(idx_d).reshape(T, 24)
    mem = down16(mem_d).reshape(T, 6144)
    kv = down16(kv_d).reshape(T, -1)
    return dict(idx=idx, mem=mem, kv=kv, hidden=down16(h_d).reshape(T, cfg.hc, cfg.H),
                gate=g_d.cpu().numpy().reshape(T, cfg.hc)), (wkv, wqk)


def _check_forward(got, ref, hc, H, hidden, wqk, dot_scale=1.0):
    """idx and mem bit-exact, k/v within 2e-2; hidden end to end and, with the
    gate, on the kernel's own k/v (check_gate_rows)."""
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["mem"], ref["mem"])
    assert_bf16_close(got["kv"], ref["kv"], what="kv")
    T = got["hidden"].shape[0]
    assert_bf16_close(got["hidden"].reshape(T * hc, H), ref["hidden"].reshape(T * hc, H), what="hidden")
    check_gate_rows(got["hidden"], got["gate"], hidden, got["kv"], ref["kv"], wqk, ref["dead"], H, hc,
                    dot_scale, "forward")


@pytest.mark.parametrize("dot_scale", [1.0, 1 / 16.0])
def test_forward_tiny(E, dot_scale):
    log(f"forward: tiny config, dot_scale={dot_scale}")
    w = World.of("tiny")
    cfg, p = w.cfg, w.params[0]
    tok, cu = synth.token_batch(w.cfg)
    hist = O.history_reset(1, p.pad_cid)
    hidden = synth.hidden_bf16(cfg, 1, len(tok))
    got, (wkv, wqk) = _run_forward(E, w, 0, tok, cu, hist, hidden, dot_scale)
    ref = O.forward(tok, cu, hist, w.tmap, p, w.rows(0), wkv, wqk, hidden, cfg.H, cfg.hc,
                    1e-6, dot_scale)
    _check_forward(got, ref, cfg.hc, cfg.H, hidden, wqk, dot_scale)


def test_forward_is_deterministic(E):
    w = World.of("tiny")
    cfg, p = w.cfg, w.params[0]
    tok, cu = synth.token_batch(w.cfg)
    hist = O.history_reset(1, p.pad_cid)
    hidden = synth.hidden_bf16(cfg, 1, len(tok))
    a, _ = _run_forward(E, w, 0, tok, cu, hist, hidden)
    b, _ = _run_forward(E, w, 0, tok, cu, hist, hidden)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_forward_decode_config(E):
    """Decode-shaped: 64 sequences x 1 token, 16M-row table, 3-token history."""
    log("forward: decode-shaped config (16M-row table on device)")
    w = World.of("decode")
    cfg, p = w.cfg, w.params[0]
    ptok, pcu = synth.history_prefix_tokens(cfg)
    hist_d = torch.empty(cfg.n_seqs * 3, dtype=torch.int32, device=DEV)
    E.engram_history_reset(hist_d, p.pad_cid)
    E.engram_history_append(hist_d, up32(ptok), up32(pcu), up32(w.tmap), p.pad_cid)
    hist = O.history_append(O.history_reset(cfg.n_seqs, p.pad_cid), ptok, pcu, w.tmap, p.pad_cid)
    assert np.array_equal(down32(hist_d).reshape(-1, 3), hist)
    tok, cu = synth.token_batch(cfg)
    hidden = synth.hidden_bf16(cfg, 1, len(tok))
    got, (wkv, wqk) = _run_forward(E, w, 0, tok, cu, hist, hidden)
    ref = O.forward(tok, cu, hist, w.tmap, p, w.rows(0), wkv, wqk, hidden, cfg.H, cfg.hc)
    _check_forward(got, ref, cfg.hc, cfg.H, hidden, wqk)
    # the same step with wkv also passed in the packed decode layout
    got_p, _ = _run_forward(E, w, 0, tok, cu, hist, hidden, packed=True)
    _check_forward(got_p, ref, cfg.hc, cfg.H, hidden, wqk)
    for k in got:
        assert np.array_equal(got_p[k], got[k]), k


def _random_cut_batch(rng, S, T, map_len, vocab_c, n_bad=0):
    """S ragged sequences (some empty) holding T tokens, DEAD spans of 1-3
    positions, a random non-PAD history, and n_bad token ids >= map_len."""
    cuts = np.sort(rng.integers(0, T + 1, S - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    tok = rng.integers(0, map_len, T).astype(np.uint32)
    for a in rng.choice(T, size=T // 12, replace=False):
        tok[a:a + int(rng.integers(1, 4))] = O.DEAD_TOKEN
    if n_bad:
        tok[rng.choice(T, size=n_bad, replace=False)] = map_len + 7
    hist = rng.integers(0, vocab_c, (S, 3)).astype(np.uint32)
    return tok, cu, hist


@pytest.mark.parametrize("S,T,n_bad", [(1, 1, 0), (37, 300, 0), (64, 64, 0), (600, 1024, 0),
                                       (37, 300, 5), (40, 1025, 0), (1025, 1030, 0)])
def test_forward_small_batch_hash_gather_matches_stage_calls(E, S, T, n_bad):
    """engram_forward hashes, gathers and decodes batches of up to 1,024 tokens
    in up to 1,024 sequences with one kernel; its workspace idx and mem, and
    its error flags, equal engram_hash followed by engram_gather_decode bit
    for bit (ragged and empty sequences, DEAD spans, a random history, token
    ids past the map), on both sides of both limits; idx also equals the oracle."""
    log(f"forward: hash+gather vs stage calls, S={S} T={T} bad tokens={n_bad}")
    w = World.of("tiny")
    cfg, p = w.cfg, w.params[0]
    rng = np.random.default_rng(1000 * S + T + n_bad)
    tok, cu, hist = _random_cut_batch(rng, S, T, cfg.map_len, cfg.vocab_c, n_bad)
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    wkv = up16(synth.wkv_bf16(cfg, 1))
    wqk = upf(synth.norm_weights(cfg, 1))
    hidden = up16(synth.hidden_bf16(cfg, 1, T))
    tok_d, cu_d, hist_d, tmap_d = up32(tok), up32(cu), up32(hist), up32(w.tmap)
    err_f = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = E.engram_forward(tok_d, cu_d, hist_d, tmap_d, p, codes, scales, wkv, wqk, hidden,
                          cfg.H, cfg.hc, err_flags=err_f)
    idx_f = workspace_views(ws, T, cfg.H, cfg.hc)[0]
    mem_f, _, has = forward_rows(ws, T, S, cfg.H, cfg.hc, np.arange(T))
    err_s = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx_s = torch.empty(T * 24, dtype=torch.int32, device=DEV)
    mem_s = torch.empty(T * 6144, dtype=torch.int16, device=DEV)
    E.engram_hash(tok_d, cu_d, hist_d, tmap_d, p, idx_s, err_flags=err_s)
    E.engram_gather_decode(idx_s, codes, scales, p.n_rows, mem_s, err_flags=err_s)
    torch.cuda.synchronize()
    assert int(err_f.item()) == int(err_s.item()) == (1 if n_bad else 0)
    assert torch.equal(idx_f, idx_s)
    dead = tok == O.DEAD_TOKEN
    assert np.all(has | dead)       # packed batches (above the limits) have no rows for DEAD positions
    assert np.array_equal(mem_f[has], down16(mem_s).reshape(T, 6144)[has])
    if not n_bad:
        assert np.array_equal(down32(idx_f).reshape(T, 24), _ref_hash(tok, cu, hist, w.tmap, p))


@pytest.mark.parametrize("H,hc", [(256, 4), (5120, 4), (5120, 2)])
def test_forward_packs_live_rows_above_the_limits(E, H, hc):
    """Above 1,024 tokens engram_forward decodes and projects only the live
    (non-DEAD) positions, packed in order, and the gate reads each position's
    k/v through that packing. Against the oracle on sampled rows (every DEAD
    edge included) for each gate kernel (generic, streaming, per branch), plus
    every DEAD row's hidden unchanged and its gate 0."""
    log(f"forward: packed live rows, T=1,500 in 3 sequences with DEAD spans, H={H} hc={hc}")
    w = World.of("tiny")
    p = w.params[0]
    rng = np.random.default_rng(H + hc)
    lens = [700, 1, 799]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    tok = rng.integers(0, w.cfg.map_len, T).astype(np.uint32)
    for a, n in ((100, 576), (690, 10), (701 + 5, 1), (701 + 50, 2)):   # image spans of 576, 10, 1, 2
        tok[a:a + n] = O.DEAD_TOKEN
    hist = rng.integers(0, w.cfg.vocab_c, (3, 3)).astype(np.uint32)
    dead = tok == O.DEAD_TOKEN
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    h_d = up16(hidden)
    g_d = torch.full((T * hc,), float("nan"), dtype=torch.float32, device=DEV)
    ws = E.engram_forward(up32(tok), up32(cu), up32(hist), up32(w.tmap), p, codes, scales, up16(wkv),
                          upf(wqk), h_d, H, hc, gate_out=g_d)
    torch.cuda.synchronize()
    ref_idx = _ref_hash(tok, cu, hist, w.tmap, p)
    assert np.array_equal(down32(workspace_views(ws, T, H, hc)[0]).reshape(T, 24), ref_idx)
    # slot and the live positions are inverse maps over the live positions
    slot = down32(workspace_views(ws, T, H, hc)[1])
    n_live = int((~dead).sum())
    pos = down32(live_positions(ws, T, H, hc))[:n_live]
    assert np.array_equal(pos, np.nonzero(~dead)[0]) and np.array_equal(slot[pos], np.arange(n_live))
    got_h = down16(h_d).reshape(T, hc, H)
    got_g = g_d.cpu().numpy().reshape(T, hc)
    assert np.array_equal(got_h[dead], hidden[dead]) and np.all(got_g[dead] == 0)
    # every live position was gated (not only the sampled ones below)
    lg = got_g[~dead]
    assert np.all(np.isfinite(lg) & (lg >= 0) & (lg <= 1))      # written: the buffer held NaN
    assert np.all((got_h != hidden).any(axis=(1, 2))[~dead])
    change = np.nonzero(np.diff(dead.astype(np.int8)))[0]
    rows = np.unique(np.concatenate([change - 1, change, change + 1, change + 2, cu[:-1], cu[1:] - 1,
                                     rng.integers(0, T, 40)]))
    rows = rows[(rows >= 0) & (rows < T)]
    got_mem, got_kv, has = forward_rows(ws, T, len(lens), H, hc, rows)
    assert np.array_equal(has, ~dead[rows])
    ref_mem = O.gather_decode(ref_idx[rows], w.rows(0))
    assert np.array_equal(got_mem[has], ref_mem[has])
    ref_kv = O.project(ref_mem, wkv)
    assert_bf16_close(got_kv[has], ref_kv[has], what="kv")
    got_kv[~has] = 0
    check_gate_rows(got_h[rows], got_g[rows], hidden[rows], got_kv, ref_kv, wqk, dead[rows], H, hc, 1.0,
                    "packed rows")


def test_decode_steps_replayed_from_a_graph_match_eager(E):
    """Three decode steps (engram_forward, then the history append) captured in
    a HIP graph and replayed three times, each replay from the same starting
    history and hidden states restored by eager copies, give hidden states,
    gates and history bit-identical to running the steps eagerly."""
    log("forward: decode steps captured in a graph, three replays against eager")
    w = World.of("tiny")
    cfg, p = w.cfg, w.params[0]
    S, steps = 16, 3
    rng = np.random.default_rng(77)
    cu = up32(np.arange(S + 1, dtype=np.int32))
    toks = [up32(rng.integers(0, cfg.map_len, S).astype(np.uint32)) for _ in range(steps)]
    hist0 = up32(rng.integers(0, cfg.vocab_c, (S, 3)).astype(np.uint32))
    hidden0 = up16(synth.hidden_bf16(cfg, 1, S))
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    wkv = up16(synth.wkv_bf16(cfg, 1))
    wkv_p = E.engram_pack_wkv(wkv, cfg.H, cfg.hc)
    wqk = upf(synth.norm_weights(cfg, 1))
    tmap = up32(w.tmap)
    hist, hidden = hist0.clone(), hidden0.clone()
    gates = [torch.empty(S * cfg.hc, dtype=torch.float32, device=DEV) for _ in range(steps)]
    ws = torch.empty(E.engram_forward_workspace(S, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)

    def run():
        for i in range(steps):
            # the middle step reads wkv itself, the others its packed layout
            E.engram_forward(toks[i], cu, hist, tmap, p, codes, scales, wkv, wqk, hidden, cfg.H, cfg.hc,
                             ws=ws, gate_out=gates[i], wkv_packed=None if i == 1 else wkv_p)
            E.engram_history_append(hist, toks[i], cu, tmap, p.pad_cid)

    run()
    torch.cuda.synchronize()
    ref = (hidden.clone(), hist.clone(), [g.clone() for g in gates])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        hist.copy_(hist0)
        hidden.copy_(hidden0)
        for g in gates:
            g.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hidden, ref[0]), r
        assert torch.equal(hist, ref[1]), r
        for i in range(steps):
            assert torch.equal(gates[i], ref[2][i]), (r, i)


def test_gate_small_and_large_batch_kernels_agree_bitwise(E):
    """Up to 4 x (CU count) / hc tokens the gate runs one workgroup per
    (token, branch) (640 threads with one chunk each up to 3 x (CU count)
    workgroups, 320 threads with two chunks each above); above that, one
    persistent workgroup per CU. All form and reduce the sums in the same
    order: on 256 CUs, the first 192 tokens of a 257-token call (persistent
    kernel), a 256-token call (two chunks per thread) and a 192-token call
    (one chunk per thread) agree bit for bit, hidden and gates."""
    cfg = synth.CONFIGS["decode"]
    H, hc, T = cfg.H, cfg.hc, 257
    rng = np.random.default_rng(21)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    kv = synth.bf16_bits_from_f32(rng.standard_normal((T, (hc + 1) * H)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    tok = rng.integers(0, 1000, T).astype(np.uint32)
    tok[[3, 100]] = 0xFFFFFFFF
    outs = []
    for n in (T, 256, 192):
        h = up16(hidden[:n])
        g = torch.empty(n * hc, dtype=torch.float32, device=DEV)
        E.engram_gate(h, up16(kv[:n]), upf(wqk), up32(tok[:n]), H, hc, gate_out=g)
        torch.cuda.synchronize()
        outs.append((down16(h).reshape(n, hc, H)[:192], g.cpu().numpy().reshape(n, hc)[:192]))
    for o in outs[1:]:
        assert np.array_equal(outs[0][0], o[0])
        assert np.array_equal(outs[0][1].view(np.uint32), o[1].view(np.uint32))
    assert np.array_equal(outs[1][0][3], hidden[3]) and np.all(outs[1][1][[3, 100]] == 0)
