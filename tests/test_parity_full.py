"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (engram_forward per layer, history appended once per step).

The oracle runs on what it can finish in seconds: the hash and the history
for every position (bit-exact), and decode, projection, gate and residual on
sampled positions (tile edges, history boundaries, every DEAD boundary of the
sampled sequences, and random positions).
"""
import gc

import numpy as np
import pytest
import torch

import engram_synth as synth
from oracle import engram_oracle as O
from tests.conftest import gpu_available
from tests.gpu_helpers import (DEV, World, assert_bf16_close, check_gate_rows, device_table, down16,
                               down32,
                               forward_rows, hidden_device, hidden_rows, log, up16, up32, upf, workspace_views)

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_amd as E
    return E


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _layer_inputs(E, w, li):
    cfg, p = w.cfg, w.params[li]
    kd, ks = w.keys[li]
    t0 = __import__("time").time()
    codes, scales = device_table(E, p.n_rows, kd, ks)
    torch.cuda.synchronize()
    log(f"  layer {cfg.layers[li]}: {p.n_rows:,}-row table on device in {__import__('time').time() - t0:.1f} s")
    wkv = synth.wkv_bf16(cfg, cfg.layers[li])
    wqk = synth.norm_weights(cfg, cfg.layers[li])
    wkv_d = up16(wkv)
    wkv_p = E.engram_pack_wkv(wkv_d, cfg.H, cfg.hc)     # decode layout, as the benchmark uses it
    return dict(codes=codes, scales=scales, wkv=wkv, wkv_d=wkv_d, wkv_p=wkv_p, wqk=wqk, wqk_d=upf(wqk))


def _check_sampled(w, li, L, rows, idx_all, ws, T, S, hid_in, hid_out, gate_d, dead):
    """Oracle on sampled rows: decode from the oracle's indices, project, gate.
    mem and kv are compared where the position has a row (packed batches
    skip DEAD positions, whose k/v the gate never reads)."""
    cfg, p = w.cfg, w.params[li]
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    ref_mem = O.gather_decode(idx_all[rows], w.rows(li))
    got_mem, got_kv, has = forward_rows(ws, T, S, cfg.H, cfg.hc, rows)
    assert np.all(has | dead[rows])
    assert np.array_equal(got_mem[has], ref_mem[has])
    ref_kv = O.project(ref_mem, L["wkv"])
    if has.any():
        assert_bf16_close(got_kv[has], ref_kv[has], what="kv")
    got_h = down16(hid_out).reshape(-1, cfg.hc, cfg.H)[rows]
    got_g = gate_d.cpu().numpy().reshape(-1, cfg.hc)[rows]
    got_kv[~has] = 0
    check_gate_rows(got_h, got_g, hid_in, got_kv, ref_kv, L["wqk"], dead[rows], cfg.H, cfg.hc, 1.0,
                    "sampled rows")


def _forward(E, w, li, L, tok_d, cu_d, hist_d, tmap_d, hidden_d, ws, T):
    """engram_forward as the benchmark calls it: wkv plus its packed decode
    layout (read by batches of at most 256 tokens, ignored above)."""
    cfg = w.cfg
    gate_d = torch.empty(T * cfg.hc, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    E.engram_forward(tok_d, cu_d, hist_d, tmap_d, w.params[li], L["codes"], L["scales"],
                     L["wkv_d"], L["wqk_d"], hidden_d, cfg.H, cfg.hc, 1e-6, 1.0, ws=ws,
                     gate_out=gate_d, err_flags=err, wkv_packed=L["wkv_p"])
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return gate_d


def _ranges_ok(idx, dead, p):
    live = idx[~dead]
    lo = p.offset.astype(np.int64)
    hi = lo + p.prime.astype(np.int64)
    assert np.all((live >= lo) & (live < hi))
    assert np.all(idx[dead] == O.DEAD_IDX)


def test_full_size_one_layer(E):
    """384,006,168-row table, 4,096-token prefill."""
    log("full-size one layer: 384M-row table, 4,096 tokens")
    w = World.of("full")
    cfg, p = w.cfg, w.params[0]
    tok, cu = synth.token_batch(cfg)
    T = len(tok)
    hist = O.history_reset(1, p.pad_cid)
    L = _layer_inputs(E, w, 0)
    hidden_d = hidden_device(cfg, 1, T)
    rng = np.random.default_rng(1)
    rows = np.concatenate([[0, 1, 2, 3, 255, 256, 4095], rng.integers(0, T, 41)])
    hid_in_rows = hidden_rows(cfg, 1, sorted(set(rows.tolist())))
    ws = torch.empty(E.engram_forward_workspace(T, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)
    gate_d = _forward(E, w, 0, L, up32(tok), up32(cu), up32(hist), up32(w.tmap), hidden_d, ws, T)
    idx_d = workspace_views(ws, T, cfg.H, cfg.hc)[0]
    win, dead, _ = O.walk(tok, cu, hist, w.tmap, p.pad_cid)
    ref_idx = O.hash_windows(win, dead, p.mult, p.prime, p.offset)
    got_idx = down32(idx_d).reshape(T, 24)
    assert np.array_equal(got_idx, ref_idx)
    _ranges_ok(got_idx, dead, p)
    _check_sampled(w, 0, L, rows, ref_idx, ws, T, len(cu) - 1, hid_in_rows, hidden_d, gate_d, dead)


def test_long_prefill_two_layers(E):
    """Both full tables resident; 50,032 tokens through layers 1 and 14 with one
    shared history, appended once after both layers."""
    log("long prefill: two 384M-row tables, 50,032 tokens, two layers")
    w = World.of("long")
    cfg = w.cfg
    tok, cu = synth.token_batch(cfg)
    T = len(tok)
    pad = w.params[0].pad_cid
    hist0 = O.history_reset(1, pad)
    hist_d = up32(hist0)
    tok_d, cu_d, tmap_d = up32(tok), up32(cu), up32(w.tmap)
    Ls = [_layer_inputs(E, w, li) for li in range(2)]
    ws = torch.empty(E.engram_forward_workspace(T, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(2)
    rows = sorted(set(np.concatenate([[0, 1, 2, 3, 4, 255, 256, 4095, 4096, 50031],
                                      rng.integers(0, 8192, 12)]).tolist()))
    win, dead, hist_after = O.walk(tok, cu, hist0, w.tmap, pad)
    for li in range(2):
        p = w.params[li]
        hidden_d = hidden_device(cfg, cfg.layers[li], T)
        hid_in_rows = hidden_rows(cfg, cfg.layers[li], rows)
        gate_d = _forward(E, w, li, Ls[li], tok_d, cu_d, hist_d, tmap_d, hidden_d, ws, T)
        idx_d = workspace_views(ws, T, cfg.H, cfg.hc)[0]
        ref_idx = O.hash_windows(win, dead, p.mult, p.prime, p.offset)
        got_idx = down32(idx_d).reshape(T, 24)
        assert np.array_equal(got_idx, ref_idx), f"layer {cfg.layers[li]}"
        _ranges_ok(got_idx, dead, p)
        _check_sampled(w, li, Ls[li], rows, ref_idx, ws, T, len(cu) - 1, hid_in_rows, hidden_d, gate_d,
                       dead)
        del hidden_d
    # both layers read the same history; it is appended once, after them
    assert np.array_equal(down32(hist_d).reshape(1, 3), hist0)
    E.engram_history_append(hist_d, tok_d, cu_d, tmap_d, pad)
    assert np.array_equal(down32(hist_d).reshape(1, 3), hist_after)


def test_multimodal_batched_decode(E):
    """256 sequences of 2,048 prompt tokens with two 576-position DEAD spans each,
    prefilled in chunks of 32 sequences (histories forked from a reset root), then
    decode steps of one token per sequence through both layers."""
    log("multimodal: 256 x 2,048 prompts with DEAD spans, chunked prefill, then decode")
    w = World.of("multimodal")
    cfg = w.cfg
    pad = w.params[0].pad_cid
    tok, cu = synth.token_batch(cfg)
    S, Lq = cfg.n_seqs, cfg.tokens_per_seq
    tmap_d = up32(w.tmap)
    Ls = [_layer_inputs(E, w, li) for li in range(2)]
    root = torch.empty(3, dtype=torch.int32, device=DEV)
    E.engram_history_reset(root, pad)
    hist_all = torch.empty(S * 3, dtype=torch.int32, device=DEV)
    for s in range(S):                                   # each sequence's own forked history
        E.engram_history_fork(hist_all[3 * s: 3 * s + 3], root)
    ref_hist = O.history_reset(S, pad)
    chunk = 32
    Tc = chunk * Lq
    ws = torch.empty(E.engram_forward_workspace(Tc, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(3)
    check_chunks = {0, S // chunk - 1}
    for c0 in range(0, S, chunk):
        sl = slice(c0 * Lq, (c0 + chunk) * Lq)
        ctok = tok[sl]
        ccu = (cu[c0: c0 + chunk + 1] - cu[c0]).astype(np.int32)
        h_in = ref_hist[c0: c0 + chunk]
        win, dead, h_out = O.walk(ctok, ccu, h_in, w.tmap, pad)
        hist_c = hist_all[3 * c0: 3 * (c0 + chunk)]
        tok_d, cu_d = up32(ctok), up32(ccu)
        for li in range(2):
            p = w.params[li]
            first = c0 * Lq
            checked = c0 // chunk in check_chunks
            # chunks checked on sampled rows get the seeded hidden; the others are
            # checked on indices and history only and get zeros
            hidden_d = (hidden_device(cfg, cfg.layers[li], Tc, first=first) if checked else
                        torch.zeros((Tc, cfg.hc, cfg.H), dtype=torch.int16, device=DEV))
            # samples: both DEAD spans' edges in the chunk's first sequence, plus random positions
            change = np.nonzero(np.diff(dead[:Lq].astype(np.int8)))[0]
            edges = np.unique(np.concatenate([change - 1, change, change + 1, change + 2,
                                              [0, 1, 2, Lq - 1, Lq, Tc - 1]]))
            rows = sorted(set(np.concatenate([edges[(edges >= 0) & (edges < Tc)],
                                              rng.integers(0, Tc, 6)]).tolist()))
            gate_d = _forward(E, w, li, Ls[li], tok_d, cu_d, hist_c, tmap_d, hidden_d, ws, Tc)
            idx_d = workspace_views(ws, Tc, cfg.H, cfg.hc)[0]
            ref_idx = O.hash_windows(win, dead, p.mult, p.prime, p.offset)
            got_idx = down32(idx_d).reshape(Tc, 24)
            assert np.array_equal(got_idx, ref_idx), (c0, li)
            _ranges_ok(got_idx, dead, p)
            if checked:
                assert dead[rows].any() and (~dead[rows]).any()
                hid_in_rows = hidden_rows(cfg, cfg.layers[li], np.array(rows) + first)
                _check_sampled(w, li, Ls[li], rows, ref_idx, ws, Tc, chunk, hid_in_rows, hidden_d,
                               gate_d, dead)
            del hidden_d
        E.engram_history_append(hist_c, tok_d, cu_d, tmap_d, pad)
        ref_hist[c0: c0 + chunk] = h_out
        assert np.array_equal(down32(hist_c).reshape(chunk, 3), h_out)
    log("  prefill done; decode steps")
    del ws
    ws = torch.empty(E.engram_forward_workspace(S, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)
    dcu = np.arange(S + 1, dtype=np.int32)
    dcu_d = up32(dcu)
    # all of the config's decode steps: indices and histories every step,
    # sampled rows (decoded rows, k/v, hidden, gates) every 16th step
    for step in range(cfg.decode_steps):
        dtok = synth.decode_tokens(cfg, step)
        dtok_d = up32(dtok)
        win, dead, h_out = O.walk(dtok, dcu, ref_hist, w.tmap, pad)
        checked = step % 16 == 0 or step == cfg.decode_steps - 1
        for li in range(2):
            p = w.params[li]
            hidden_d = (hidden_device(cfg, cfg.layers[li], S, batch=100 + step) if checked else
                        torch.zeros((S, cfg.hc, cfg.H), dtype=torch.int16, device=DEV))
            gate_d = _forward(E, w, li, Ls[li], dtok_d, dcu_d, hist_all, tmap_d, hidden_d, ws, S)
            idx_d = workspace_views(ws, S, cfg.H, cfg.hc)[0]
            ref_idx = O.hash_windows(win, dead, p.mult, p.prime, p.offset)
            assert np.array_equal(down32(idx_d).reshape(S, 24), ref_idx), (step, li)
            if checked:
                rows = sorted(set([0, 1, 2, 127, 128, 255] + rng.integers(0, S, 4).tolist()))
                hid_in_rows = hidden_rows(cfg, cfg.layers[li], rows, batch=100 + step)
                _check_sampled(w, li, Ls[li], rows, ref_idx, ws, S, S, hid_in_rows, hidden_d, gate_d,
                               dead)
        E.engram_history_append(hist_all, dtok_d, dcu_d, tmap_d, pad)
        ref_hist = h_out
        assert np.array_equal(down32(hist_all).reshape(S, 3), ref_hist)
        if step % 32 == 31:
            log(f"  decode step {step + 1} of {cfg.decode_steps}")
