"""GPU parity against the oracle for the paths beyond the plain layer call:
full-range hash multipliers on every hashing path, every row of the gate's
position walk and live-row walk, the split layer (hidden-independent
precompute on a side stream, then the gate at layer entry), and tables in
pinned host memory, read in place or staged into device memory first.

Bars: hash indices and decoded rows bit-exact; k/v and hidden within
2e-2 * max(|ref|, rms(ref row)); gate within 1e-3 at every position, on the
kernel's own k/v (see check_gate_rows).
"""
import numpy as np
import pytest
import torch

import engram_synth as synth
from oracle import engram_oracle as O
from tests.conftest import gpu_available
from tests.gpu_helpers import (DEV, World, assert_bf16_close, check_gate_rows, device_table, down16,
                               down32, forward_rows, live_positions, log, up16, up32, upf,
                               workspace_views)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_amd as E
    return E


def _ref_idx(tok, cu, hist, tmap, p):
    win, dead, _ = O.walk(tok, cu, hist, tmap, p.pad_cid)
    return O.hash_windows(win, dead, p.mult, p.prime, p.offset), dead


def _ragged(rng, S, T, map_len, vocab_c, dead_every=16):
    cuts = np.sort(rng.integers(0, T + 1, S - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    tok = synth.zipf_tokens(rng, T, map_len)
    for a in rng.choice(T, size=max(1, T // dead_every), replace=False):
        tok[a:a + int(rng.integers(1, 4))] = O.DEAD_TOKEN
    hist = rng.integers(0, vocab_c, (S, 3)).astype(np.uint32)
    return tok, cu, hist


# ---------------------------------------------------------------- full-range multipliers
def test_full_range_multipliers_on_every_hashing_path(E):
    """96 distinct full-range multipliers (wrapping products, XORs above 2^63,
    one per bucket and slot) through engram_hash, the fused small-batch hash +
    gather, the packed large-batch path and the staged precompute: indices
    bit-exact against the oracle, decoded rows bit-exact on sampled rows."""
    w = World.of("decode")
    cfg = w.cfg
    p = synth.make_full_range_hash_params(cfg.root, 1, cfg.vocab_c, cfg.prime_bases[0],
                                          int(w.tmap[0]))
    assert len(set(p.mult.reshape(-1).tolist())) == 96
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    rng = np.random.default_rng(31)
    H, hc = 256, 4            # narrow k/v: this test is about the indices and rows
    wkv = up16(synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32)))
    for S, T in ((9, 4000), (37, 1000), (1, 1)):
        log(f"full-range multipliers: S={S} T={T}")
        tok, cu, hist = _ragged(rng, S, T, cfg.map_len, cfg.vocab_c)
        ref, dead = _ref_idx(tok, cu, hist, w.tmap, p)
        args = (up32(tok), up32(cu), up32(hist), up32(w.tmap), p)
        idx = torch.empty(T * 24, dtype=torch.int32, device=DEV)
        E.engram_hash(*args, idx)
        torch.cuda.synchronize()
        assert np.array_equal(down32(idx).reshape(T, 24), ref)
        rows = np.unique(np.concatenate([rng.integers(0, T, 24), np.flatnonzero(dead)[:3], [T - 1]]))
        ref_mem = O.gather_decode(ref[rows], w.rows(0))
        for flags in (0, E.PRECOMPUTE_STAGE_ROWS):
            err = torch.zeros(1, dtype=torch.int32, device=DEV)
            ws = E.engram_precompute(*args, codes, scales, wkv, H, hc, flags=flags, err_flags=err)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert np.array_equal(down32(workspace_views(ws, T, H, hc)[0]).reshape(T, 24), ref), flags
            got_mem, _, has = forward_rows(ws, T, S, H, hc, rows)
            assert np.array_equal(got_mem[has], ref_mem[has]), flags


# ---------------------------------------------------------------- gate walks
@pytest.mark.parametrize("T", [257, 1024])
def test_gate_position_walk_every_row(E, T):
    """engram_gate above 4 x (CU count) / hc tokens at H = 5,120, hc = 4 runs
    the persistent kernel's position walk: every row's hidden and gate
    against the oracle on the same BF16 inputs."""
    log(f"gate: position walk, T={T}, every row")
    H, hc = 5120, 4
    rng = np.random.default_rng(T)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    kv = synth.bf16_bits_from_f32(rng.standard_normal((T, (hc + 1) * H)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    tok = rng.integers(0, 1000, T).astype(np.uint32)
    tok[[0, 5, 6, T // 2, T - 1]] = O.DEAD_TOKEN
    dead = tok == O.DEAD_TOKEN
    h = up16(hidden)
    g = torch.full((T * hc,), float("nan"), dtype=torch.float32, device=DEV)
    E.engram_gate(h, up16(kv), upf(wqk), up32(tok), H, hc, dot_scale=1 / 16, gate_out=g)
    torch.cuda.synchronize()
    got_h = down16(h).reshape(T, hc, H)
    got_g = g.cpu().numpy().reshape(T, hc)
    new, ref_g, _ = O.gate_residual(hidden, kv, wqk, dead, H, hc, 1e-6, 1 / 16)
    assert_bf16_close(got_h.reshape(-1, H), new.reshape(-1, H), what="hidden")
    assert np.array_equal(got_h[dead], hidden[dead])
    assert np.max(np.abs(got_g - ref_g)) <= 1e-3           # identical inputs: every position


def _forward_every_row(E, w, H, hc, T, S, dead_spans, seed, dot_scale=1 / 16):
    """engram_forward at H, hc with a custom wkv; returns what the checks need."""
    p = w.params[0]
    rng = np.random.default_rng(seed)
    tok, cu, hist = _ragged(rng, S, T, w.cfg.map_len, w.cfg.vocab_c, dead_every=10 ** 9)
    for a, n in dead_spans:
        tok[a:a + n] = O.DEAD_TOKEN
    dead = tok == O.DEAD_TOKEN
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    hidden = np.empty((T, hc, H), np.uint16)
    for a in range(0, T, 2048):                     # bounded host temporaries
        b = min(T, a + 2048)
        hidden[a:b] = synth.bf16_bits_from_f32(rng.standard_normal((b - a, hc, H)).astype(np.float32))
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    h_d = up16(hidden)
    g_d = torch.full((T * hc,), float("nan"), dtype=torch.float32, device=DEV)
    ws = E.engram_forward(up32(tok), up32(cu), up32(hist), up32(w.tmap), p, codes, scales, up16(wkv),
                          upf(wqk), h_d, H, hc, 1e-6, dot_scale, gate_out=g_d)
    torch.cuda.synchronize()
    return dict(p=p, tok=tok, cu=cu, hist=hist, dead=dead, wkv=wkv, wqk=wqk, hidden=hidden, ws=ws,
                h=down16(h_d).reshape(T, hc, H), g=g_d.cpu().numpy().reshape(T, hc), rng=rng)


@pytest.mark.parametrize("T,S,spans", [(700, 3, ((10, 5), (300, 1), (699, 1))),
                                       (4096, 2, ((100, 576), (2000, 576), (4095, 1))),
                                       (20_000, 4, ((0, 3), (1000, 576), (9000, 576), (15000, 576),
                                                    (19990, 10)))])
def test_forward_gate_walks_every_row(E, T, S, spans):
    """engram_forward at H = 5,120, hc = 4: at 700 tokens the gate walks
    positions (one persistent workgroup per CU, three steps each); at 20,000
    tokens with image spans it walks the packed live rows, more than 64 steps
    per workgroup, so the kernel's per-64-step refill of the row map runs; at
    4,096 positions (rows packed, about 2,940 live) the projection's row tiles
    past the live count stop after their first loads. Every row's hidden and
    gate against the oracle's gate on the workspace's k/v (which is itself
    checked against the oracle on sampled rows)."""
    log(f"forward: gate walk, T={T} S={S}, every row")
    H, hc = 5120, 4
    w = World.of("tiny")
    r = _forward_every_row(E, w, H, hc, T, S, spans, seed=T)
    dead, ws = r["dead"], r["ws"]
    n_live = int((~dead).sum())
    if T > 10_000:
        assert n_live // 256 > 64        # live rows per workgroup of the walk
    ref_idx, ref_dead = _ref_idx(r["tok"], r["cu"], r["hist"], w.tmap, r["p"])
    assert np.array_equal(ref_dead, dead)
    assert np.array_equal(down32(workspace_views(ws, T, H, hc)[0]).reshape(T, 24), ref_idx)
    # k/v of sampled rows against the oracle's projection
    rng = r["rng"]
    rows = np.unique(np.concatenate([rng.integers(0, T, 24), [T - 1]]))
    got_mem, got_kv, has = forward_rows(ws, T, S, H, hc, rows)
    ref_mem = O.gather_decode(ref_idx[rows], w.rows(0))
    assert np.array_equal(got_mem[has], ref_mem[has])
    assert_bf16_close(got_kv[has], O.project(ref_mem, r["wkv"])[has], what="kv")
    # every row: gate and hidden against the oracle on the workspace's k/v
    _, slot_d, _, kv_d = workspace_views(ws, T, H, hc)
    kv_all = down16(kv_d).reshape(T, (hc + 1) * H)
    if T > 1024:
        slot = down32(slot_d)
        src = np.where(dead, 0, slot).astype(np.int64)
    else:
        src = np.arange(T)
    for a in range(0, T, 2048):
        sel = np.arange(a, min(T, a + 2048))
        check_gate_rows(r["h"][sel], r["g"][sel], r["hidden"][sel], kv_all[src[sel]], None, r["wqk"],
                    dead[sel], H, hc, 1 / 16, f"rows {a}..")
    assert np.all(np.isfinite(r["g"]))


# ---------------------------------------------------------------- split layer (f2)
def _two_layer_world(E, name="decode"):
    """Two layers of the decode-shaped size (16M-row tables, H = 5,120,
    hc = 4): layer 1 of the config and a second layer with the next 24
    primes, its own multipliers, table, wkv and norm weights."""
    w = World.of(name)
    cfg = w.cfg
    p1 = w.params[0]
    base2 = int(p1.prime[-1])
    p2 = synth.make_hash_params(cfg.root, 2, cfg.vocab_c, base2, int(w.tmap[0]))
    keys = [w.keys[0], synth.table_keys(cfg.root, 2)]
    layers = []
    for li, (p, (kd, ks)) in enumerate(zip((p1, p2), keys)):
        codes, scales = device_table(E, p.n_rows, kd, ks)
        wkv = synth.wkv_bf16(cfg, li + 1)
        layers.append(dict(p=p, codes=codes, scales=scales, wkv=wkv, wkv_d=up16(wkv),
                           wqk=synth.norm_weights(cfg, li + 1),
                           rows=(lambda kd=kd, ks=ks: (lambda r: synth.table_rows(r, kd, ks)))()))
    return w, layers


def test_split_layers_precompute_on_a_side_stream_against_oracle(E):
    """Three decode steps of two layers, as a serving loop would order them:
    both layers' hidden-independent precompute on a side stream (reading the
    history before the step), each layer's gate on the main stream after an
    event wait, the history append after both precomputes. Indices, hidden
    states, gates and the history against the oracle, step by step."""
    log("split layer: two layers' precompute on a side stream, gates on the main stream, 3 steps")
    w, layers = _two_layer_world(E)
    cfg = w.cfg
    S, H, hc = cfg.n_seqs, cfg.H, cfg.hc
    tmap = up32(w.tmap)
    cu_h = np.arange(S + 1, dtype=np.int32)
    cu = up32(cu_h)
    ptok, pcu = synth.history_prefix_tokens(cfg)
    pad = layers[0]["p"].pad_cid
    hist = torch.empty(S * 3, dtype=torch.int32, device=DEV)
    E.engram_history_reset(hist, pad)
    E.engram_history_append(hist, up32(ptok), up32(pcu), tmap, pad)
    ref_hist = O.history_append(O.history_reset(S, pad), ptok, pcu, w.tmap, pad)
    ws = [torch.empty(E.engram_forward_workspace(S, H, hc), dtype=torch.uint8, device=DEV)
          for _ in layers]
    wqk_d = [upf(L["wqk"]) for L in layers]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    for step in range(3):
        tok_h = synth.decode_tokens(cfg, step)
        tok_h[[step, 10 + step]] = O.DEAD_TOKEN            # image positions in the batch
        tok = up32(tok_h)
        hidden_in = [synth.hidden_bf16(cfg, li + 1, S, batch=step) for li in range(2)]
        hidden = [up16(h) for h in hidden_in]
        gates = [torch.empty(S * hc, dtype=torch.float32, device=DEV) for _ in layers]
        ready = [torch.cuda.Event() for _ in layers]
        side.wait_stream(main)                             # the previous step's append is done
        for li, L in enumerate(layers):
            E.engram_precompute(tok, cu, hist, tmap, L["p"], L["codes"], L["scales"], L["wkv_d"], H, hc,
                                ws=ws[li], stream=side)
            ready[li].record(side)
        for li in range(2):
            main.wait_event(ready[li])
            E.engram_gate_precomputed(hidden[li], ws[li], tok, S, wqk_d[li], H, hc, gate_out=gates[li],
                                      stream=main)
        main.wait_stream(side)
        E.engram_history_append(hist, tok, cu, tmap, pad, stream=main)
        torch.cuda.synchronize()
        for li, L in enumerate(layers):
            ref = O.forward(tok_h, cu_h, ref_hist, w.tmap, L["p"], L["rows"], L["wkv"], L["wqk"],
                            hidden_in[li], H, hc)
            assert np.array_equal(down32(workspace_views(ws[li], S, H, hc)[0]).reshape(S, 24), ref["idx"])
            _, got_kv, _ = forward_rows(ws[li], S, S, H, hc, np.arange(S))
            assert_bf16_close(got_kv[~ref["dead"]], ref["kv"][~ref["dead"]], what="kv")
            check_gate_rows(down16(hidden[li]).reshape(S, hc, H), gates[li].cpu().numpy().reshape(S, hc),
                        hidden_in[li], got_kv, ref["kv"], L["wqk"], ref["dead"], H, hc, 1.0,
                        f"step {step} layer {li}")
        ref_hist = O.history_append(ref_hist, tok_h, cu_h, w.tmap, pad)
        assert np.array_equal(down32(hist).reshape(S, 3), ref_hist), step


def test_split_layer_packed_batch_matches_forward_and_oracle(E):
    """A 3,000-token batch with image spans (rows packed) through the split
    calls, read in place and staged: bit-identical to engram_forward, and
    against the oracle on sampled rows (every DEAD edge) and on every gate."""
    log("split layer: packed 3,000-token batch, in place and staged")
    w = World.of("tiny")
    p = w.params[0]
    H, hc = 5120, 4
    rng = np.random.default_rng(5)
    lens = [1200, 0, 1800]
    S = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    tok = rng.integers(0, w.cfg.map_len, T).astype(np.uint32)
    for a, n in ((50, 576), (1199, 2), (2000, 576), (2999, 1)):
        tok[a:a + n] = O.DEAD_TOKEN
    dead = tok == O.DEAD_TOKEN
    hist = rng.integers(0, w.cfg.vocab_c, (S, 3)).astype(np.uint32)
    wkv = synth.bf16_bits_from_f32(0.02 * rng.standard_normal(((hc + 1) * H, 6144)).astype(np.float32))
    wqk = (1 + 0.1 * rng.standard_normal((hc, H))).astype(np.float32)
    hidden = synth.bf16_bits_from_f32(rng.standard_normal((T, hc, H)).astype(np.float32))
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    args = (up32(tok), up32(cu), up32(hist), up32(w.tmap), p)
    h_f = up16(hidden)
    g_f = torch.empty(T * hc, dtype=torch.float32, device=DEV)
    E.engram_forward(*args, codes, scales, up16(wkv), upf(wqk), h_f, H, hc, gate_out=g_f)
    outs = []
    for flags in (0, E.PRECOMPUTE_STAGE_ROWS):
        ws = E.engram_precompute(*args, codes, scales, up16(wkv), H, hc, flags=flags)
        h = up16(hidden)
        g = torch.empty(T * hc, dtype=torch.float32, device=DEV)
        E.engram_gate_precomputed(h, ws, up32(tok), S, upf(wqk), H, hc, gate_out=g)
        torch.cuda.synchronize()
        assert torch.equal(h, h_f) and torch.equal(g, g_f), flags
        outs.append(ws)
    ws = outs[1]
    ref_idx, _ = _ref_idx(tok, cu, hist, w.tmap, p)
    assert np.array_equal(down32(workspace_views(ws, T, H, hc)[0]).reshape(T, 24), ref_idx)
    n_live = int((~dead).sum())
    pos = down32(live_positions(ws, T, H, hc))[:n_live]
    assert np.array_equal(pos, np.flatnonzero(~dead))
    change = np.flatnonzero(np.diff(dead.astype(np.int8)))
    rows = np.unique(np.concatenate([change - 1, change, change + 1, change + 2, rng.integers(0, T, 30)]))
    rows = rows[(rows >= 0) & (rows < T)]
    got_mem, got_kv, has = forward_rows(ws, T, S, H, hc, rows)
    assert np.array_equal(has, ~dead[rows])
    ref_mem = O.gather_decode(ref_idx[rows], w.rows(0))
    assert np.array_equal(got_mem[has], ref_mem[has])
    ref_kv = O.project(ref_mem, wkv)
    assert_bf16_close(got_kv[has], ref_kv[has], what="kv")
    got_kv[~has] = 0
    check_gate_rows(down16(h_f).reshape(T, hc, H)[rows], g_f.cpu().numpy().reshape(T, hc)[rows], hidden[rows],
                got_kv, ref_kv, wqk, dead[rows], H, hc, 1.0, "sampled rows")


# ---------------------------------------------------------------- host-resident tables (f3)
def test_host_table_precompute_in_place_and_staged_against_oracle(E):
    """The decode config's 16M-row table in pinned host memory (mapped into
    the device's address space). The precompute runs on a side stream with
    the rows read in place across the host link, or staged into device memory
    first; the gate runs on the main stream. A decode step (64 sequences) and
    a 2,000-token packed batch: indices and decoded rows bit-exact, hidden and
    gates against the oracle."""
    log("host-resident table: precompute in place and staged, decode step and 2,000-token batch")
    w = World.of("decode")
    cfg, p = w.cfg, w.params[0]
    codes_h = torch.empty(p.n_rows * 256, dtype=torch.uint8, pin_memory=True)
    scales_h = torch.empty(p.n_rows * 8, dtype=torch.uint8, pin_memory=True)
    E.engram_gen_table(codes_h, scales_h, 0, p.n_rows, *w.keys[0])
    torch.cuda.synchronize()
    H, hc = cfg.H, cfg.hc
    wkv = synth.wkv_bf16(cfg, 1)
    wqk = synth.norm_weights(cfg, 1)
    wkv_d, wqk_d, tmap = up16(wkv), upf(wqk), up32(w.tmap)
    rng = np.random.default_rng(3)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    cases = [("decode step", synth.decode_tokens(cfg, 0), np.arange(cfg.n_seqs + 1, dtype=np.int32),
              rng.integers(0, cfg.vocab_c, (cfg.n_seqs, 3)).astype(np.uint32))]
    tok2, cu2, hist2 = _ragged(rng, 5, 2000, cfg.map_len, cfg.vocab_c)
    cases.append(("2,000-token batch", tok2, cu2, hist2))
    for name, tok, cu, hist in cases:
        T, S = len(tok), len(cu) - 1
        ref_idx, dead = _ref_idx(tok, cu, hist, w.tmap, p)
        rows = np.unique(np.concatenate([rng.integers(0, T, min(T, 40)), np.flatnonzero(dead)[:3]]))
        ref_mem = O.gather_decode(ref_idx[rows], w.rows(0))
        ref_kv = O.project(ref_mem, wkv)
        hidden = synth.hidden_bf16(cfg, 1, T)
        for flags in (0, E.PRECOMPUTE_STAGE_ROWS):
            log(f"  {name}, flags={flags}")
            err = torch.zeros(1, dtype=torch.int32, device=DEV)
            side.wait_stream(main)
            ws = E.engram_precompute(up32(tok), up32(cu), up32(hist), tmap, p, codes_h, scales_h, wkv_d,
                                     H, hc, flags=flags, err_flags=err, stream=side)
            done = torch.cuda.Event()
            done.record(side)
            main.wait_event(done)
            h = up16(hidden)
            g = torch.empty(T * hc, dtype=torch.float32, device=DEV)
            E.engram_gate_precomputed(h, ws, up32(tok), S, wqk_d, H, hc, gate_out=g, stream=main)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert np.array_equal(down32(workspace_views(ws, T, H, hc)[0]).reshape(T, 24), ref_idx)
            got_mem, got_kv, has = forward_rows(ws, T, S, H, hc, rows)
            assert np.array_equal(got_mem[has], ref_mem[has])
            assert_bf16_close(got_kv[has], ref_kv[has], what="kv")
            got_kv[~has] = 0
            check_gate_rows(down16(h).reshape(T, hc, H)[rows], g.cpu().numpy().reshape(T, hc)[rows],
                        hidden[rows], got_kv, ref_kv, wqk, dead[rows], H, hc, 1.0, name)


# ---------------------------------------------------------------- per-bucket tables (f3)
def _bucket_table(E, p, keys, pinned):
    """The layer's table as 24 allocations, bucket j holding rows offset[j] ..
    offset[j] + prime[j] - 1, written by the same closed-form generator."""
    codes, scales = [], []
    for j in range(24):
        n = int(p.prime[j])
        if pinned:
            c = torch.empty(n * 256, dtype=torch.uint8, pin_memory=True)
            s = torch.empty(n * 8, dtype=torch.uint8, pin_memory=True)
        else:
            c = torch.empty(n * 256, dtype=torch.uint8, device=DEV)
            s = torch.empty(n * 8, dtype=torch.uint8, device=DEV)
        E.engram_gen_table(c, s, int(p.offset[j]), n, *keys)
        codes.append(c)
        scales.append(s)
    torch.cuda.synchronize()
    return codes, scales


@pytest.mark.parametrize("where", ["device", "pinned host"])
def test_bucket_table_precompute_against_oracle(E, where):
    """The decode config's table held as 24 allocations (device memory, or
    pinned host memory mapped into the device's address space) through
    engram_precompute_buckets, read in place and staged: a decode step (the
    fused hash + gather kernel) and a 2,000-token packed batch. Indices and
    decoded rows bit-exact against the oracle and bit-identical (with k/v) to
    the one-allocation table; hidden states and gates against the oracle."""
    log(f"bucket table ({where}): decode step and 2,000-token batch, in place and staged")
    w = World.of("decode")
    cfg, p = w.cfg, w.params[0]
    bc, bs = _bucket_table(E, p, w.keys[0], pinned=where != "device")
    codes, scales = device_table(E, p.n_rows, *w.keys[0])
    H, hc = cfg.H, cfg.hc
    wkv = synth.wkv_bf16(cfg, 1)
    wqk = synth.norm_weights(cfg, 1)
    wkv_d, wqk_d, tmap = up16(wkv), upf(wqk), up32(w.tmap)
    rng = np.random.default_rng(17)
    cases = [(synth.decode_tokens(cfg, 1), np.arange(cfg.n_seqs + 1, dtype=np.int32),
              rng.integers(0, cfg.vocab_c, (cfg.n_seqs, 3)).astype(np.uint32))]
    cases.append(_ragged(rng, 4, 2000, cfg.map_len, cfg.vocab_c))
    for tok, cu, hist in cases:
        T, S = len(tok), len(cu) - 1
        args = (up32(tok), up32(cu), up32(hist), tmap, p)
        ref_idx, dead = _ref_idx(tok, cu, hist, w.tmap, p)
        rows = np.unique(np.concatenate([rng.integers(0, T, min(T, 40)), np.flatnonzero(dead)[:3]]))
        ref_mem = O.gather_decode(ref_idx[rows], w.rows(0))
        ref_kv = O.project(ref_mem, wkv)
        hidden = synth.hidden_bf16(cfg, 1, T, batch=3)
        ws_one = E.engram_precompute(*args, codes, scales, wkv_d, H, hc)
        for flags in (0, E.PRECOMPUTE_STAGE_ROWS):
            err = torch.zeros(1, dtype=torch.int32, device=DEV)
            ws = E.engram_precompute_buckets(*args, bc, bs, wkv_d, H, hc, flags=flags, err_flags=err)
            h = up16(hidden)
            g = torch.empty(T * hc, dtype=torch.float32, device=DEV)
            E.engram_gate_precomputed(h, ws, up32(tok), S, wqk_d, H, hc, gate_out=g)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            v_one, v_b = workspace_views(ws_one, T, H, hc), workspace_views(ws, T, H, hc)
            assert np.array_equal(down32(v_b[0]).reshape(T, 24), ref_idx)
            # rows in use: all T, or (packed) the live rows only, the rest unwritten
            n = T if T <= 1024 else int((~dead).sum())
            assert torch.equal(v_one[2][:n * 6144], v_b[2][:n * 6144])                  # mem
            assert torch.equal(v_one[3][:n * (hc + 1) * H], v_b[3][:n * (hc + 1) * H])  # k/v
            if T > 1024:
                assert torch.equal(v_one[1], v_b[1])                                    # slot
            got_mem, got_kv, has = forward_rows(ws, T, S, H, hc, rows)
            assert np.array_equal(got_mem[has], ref_mem[has])
            assert_bf16_close(got_kv[has], ref_kv[has], what="kv")
            got_kv[~has] = 0
            check_gate_rows(down16(h).reshape(T, hc, H)[rows], g.cpu().numpy().reshape(T, hc)[rows],
                            hidden[rows], got_kv, ref_kv, wqk, dead[rows], H, hc, 1.0, f"T={T} flags={flags}")
