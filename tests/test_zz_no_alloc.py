"""engram_forward_noalloc (the entry point that allocates nothing) against
engram_forward and the oracle, through the C ABI, on calls in a row that
each run on the device array the previous call left behind: a batch that
packs its live rows (above 1,024 tokens), a smaller one that does not, one
that packs because it has more than 1,024 sequences, and a decode-sized one."""
import numpy as np
import pytest
import torch

import engram_synth as synth
from oracle import engram_oracle as O
from tests.conftest import gpu_available
from tests.gpu_helpers import (DEV, World, assert_bf16_close, check_gate_rows, device_table, down16,
                               forward_rows, log, up16, up32, upf)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def _batch(rng, S, T, map_len, vocab_c):
    cuts = np.sort(rng.integers(0, T + 1, S - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    tok = synth.zipf_tokens(rng, T, map_len)
    for a in rng.choice(T, size=T // 16, replace=False):
        tok[a:a + int(rng.integers(1, 4))] = O.DEAD_TOKEN
    hist = rng.integers(0, vocab_c, (S, 3)).astype(np.uint32)
    return tok, cu, hist


def test_forward_noalloc_matches_forward_on_calls_in_a_row_then_rejects_oversize():
    import gram_hashed_embedding_amd as E
    w = World.of("decode")
    cfg, p = w.cfg, w.params[0]
    kd, ks = w.keys[0]
    codes, scales = device_table(E, p.n_rows, kd, ks)
    wkv = synth.wkv_bf16(cfg, 1)
    wqk = synth.norm_weights(cfg, 1)
    wkv_d, wqk_d, tmap_d = up16(wkv), upf(wqk), up32(w.tmap)
    rng = np.random.default_rng(77)
    for call, (S, T, dot_scale) in enumerate(((3, 1050, 1 / 16), (37, 1000, 1 / 16),
                                              (1030, 1040, 1 / 16), (64, 64, 1.0))):
        log(f"noalloc call {call}: S={S} T={T} dot_scale={dot_scale}")
        tok, cu, hist = _batch(rng, S, T, cfg.map_len, p.vocab_c)
        hidden = synth.hidden_bf16(cfg, 1, T, batch=call)
        args = (up32(tok), up32(cu), up32(hist), tmap_d, p, codes, scales, wkv_d, wqk_d)
        h_ref, h_na = up16(hidden), up16(hidden)
        g_ref = torch.empty(T * cfg.hc, dtype=torch.float32, device=DEV)
        g_na = torch.full((T * cfg.hc,), -1.0, dtype=torch.float32, device=DEV)
        e_ref = torch.zeros(1, dtype=torch.int32, device=DEV)
        e_na = torch.zeros(1, dtype=torch.int32, device=DEV)
        ws = torch.empty(E.engram_forward_workspace(T, cfg.H, cfg.hc), dtype=torch.uint8, device=DEV)
        E.engram_forward(*args, h_ref, cfg.H, cfg.hc, 1e-6, dot_scale, ws=ws, gate_out=g_ref,
                         err_flags=e_ref)
        E.engram_forward_noalloc(*args, h_na, cfg.H, cfg.hc, 1e-6, dot_scale, gate_out=g_na,
                                 err_flags=e_na)
        torch.cuda.synchronize()
        assert int(e_na.item()) == int(e_ref.item()) == 0
        # the same kernels on the same inputs: bit-identical to engram_forward
        assert torch.equal(h_na, h_ref)
        assert torch.equal(g_na, g_ref)
        # and within the oracle's bars on sampled rows (rows are independent):
        # k/v against the oracle's, hidden end to end, and the gate on the
        # k/v that engram_forward (bit-identical to this call) left in its
        # workspace
        win, dead, _ = O.walk(tok, cu, hist, w.tmap, p.pad_cid)
        rows = np.unique(np.concatenate([rng.choice(T, size=min(T, 40), replace=False),
                                         np.flatnonzero(dead)[:4], [T - 1]]))
        idx = O.hash_windows(win[rows], dead[rows], p.mult, p.prime, p.offset)
        kv = O.project(O.gather_decode(idx, w.rows(0)), wkv)
        _, got_kv, has = forward_rows(ws, T, S, cfg.H, cfg.hc, rows)
        live = has & ~dead[rows]
        assert_bf16_close(got_kv[live], kv[live], what=f"call {call} kv")
        got_h = down16(h_na).reshape(T, cfg.hc, cfg.H)[rows]
        got_g = g_na.cpu().numpy().reshape(T, cfg.hc)[rows]
        check_gate_rows(got_h, got_g, hidden[rows], got_kv, kv, wqk, dead[rows], cfg.H, cfg.hc,
                        dot_scale, what=f"call {call}")
    # a batch whose workspace exceeds the device array (64 MiB holds 1,055
    # tokens at H = 5,120, hc = 4) is rejected before any launch
    assert E.engram_forward_workspace(1055, cfg.H, cfg.hc) <= E.NOALLOC_WORKSPACE_BYTES
    assert E.engram_forward_workspace(1056, cfg.H, cfg.hc) > E.NOALLOC_WORKSPACE_BYTES
    T = 1056
    tok = np.zeros(T, np.uint32)
    cu = np.array([0, T], np.int32)
    h = torch.zeros(T * cfg.hc * cfg.H, dtype=torch.int16, device=DEV)
    with pytest.raises(E.EngramError) as ei:
        E.engram_forward_noalloc(up32(tok), up32(cu), up32(np.zeros(3, np.uint32)), tmap_d, p, codes,
                                 scales, wkv_d, wqk_d, h, cfg.H, cfg.hc)
    assert ei.value.status == -1 and "NOALLOC_WORKSPACE_BYTES" in str(ei.value)
    assert int(torch.count_nonzero(h).item()) == 0
