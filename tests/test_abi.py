"""The C ABI: the built library loads, exports every entry point the header
declares, and its host-side checks reject bad input (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import engram_synth as synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(engram_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_amd as E
    return E


def test_header_declares_the_stage_entry_points():
    names = _declared()
    for n in ("engram_hash", "engram_gather_decode", "engram_project", "engram_gate",
              "engram_forward", "engram_history_append", "engram_history_fork",
              "engram_history_reset", "engram_check_params", "engram_forward_workspace",
              "engram_pack_wkv", "engram_precompute", "engram_gate_precomputed",
              "engram_precompute_buckets"):
        assert n in names


def test_library_exports_every_declared_symbol(E):
    out = subprocess.run(["nm", "-D", "--defined-only", E.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (engram_\w+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        assert hasattr(E.lib, n)
    header_version = int(re.search(r"#define ENGRAM_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert E.lib.engram_abi_version() == header_version


def test_status_strings(E):
    for s in (0, -1, -2, -3, 7):
        assert E.lib.engram_status_string(s)


def _params(name="tiny"):
    cfg = synth.CONFIGS[name]
    return synth.params_for(cfg)[0], synth.make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)


def test_check_params_accepts_the_configs(E):
    for name in ("tiny", "decode", "full", "long"):
        cfg = synth.CONFIGS[name]
        tmap = synth.make_token_map(cfg.root, cfg.map_len, cfg.vocab_c)
        for p in synth.params_for(cfg):
            E.engram_check_params(p, tmap)


def _hp(E, p, **over):
    h = E.HashParams.from_any(p)
    for k, v in over.items():
        setattr(h, k, v)
    return h


@pytest.mark.parametrize("case", ["not_prime", "duplicate", "offset", "n_rows", "too_many_rows",
                                  "vocab0", "pad", "map_value"])
def test_check_params_rejects(E, case):
    p, tmap = _params()
    h = E.HashParams.from_any(p)
    m = tmap.copy()
    if case == "not_prime":
        h.prime[3] = 1001
    elif case == "duplicate":
        h.prime[4] = h.prime[3]
    elif case == "offset":
        h.offset[5] += 1
    elif case == "n_rows":
        h.n_rows += 1
    elif case == "too_many_rows":
        for j in range(24):
            h.prime[j] = 4294967291 if j == 23 else h.prime[j]
        h.n_rows = int(h.offset[23]) + 4294967291
    elif case == "vocab0":
        h.vocab_c = 0
    elif case == "pad":
        h.pad_cid = h.vocab_c
    elif case == "map_value":
        m[17] = p.vocab_c
    with pytest.raises(E.EngramError) as ei:
        E.engram_check_params(h, m)
    assert ei.value.status == -1
    assert E.lib.engram_last_error().decode()


def test_stage_entry_points_reject_bad_shapes_before_launch(E):
    """Host checks fire without touching a device (NULL stream, fake pointers
    are never dereferenced because validation fails first)."""
    L = E.lib
    p, _ = _params()
    hp = E.HashParams.from_any(p)
    fake = ctypes.c_void_p(0x10000)
    # H not a multiple of 64
    assert L.engram_project(fake, 4, fake, None, 100, 4, fake, None) == -1
    assert b"multiple of 64" in L.engram_last_error()
    # hc out of range
    assert L.engram_gate(fake, fake, fake, None, 4, 256, 9, 1e-6, 1.0, None, None) == -1
    # misaligned operand
    assert L.engram_project(ctypes.c_void_p(0x10002), 4, fake, None, 256, 4, fake, None) == -1
    assert L.engram_project(fake, 4, fake, ctypes.c_void_p(0x20008), 256, 4, fake, None) == -1
    assert b"wkv_packed" in L.engram_last_error()
    # tokens without sequences
    assert L.engram_hash(fake, fake, 0, 5, fake, fake, 10, ctypes.byref(hp), fake, None, None) == -1
    # workspace too small
    need = L.engram_forward_workspace(8, 256, 4)
    assert need > 0
    rc = L.engram_forward(fake, fake, 1, 8, fake, fake, 10, ctypes.byref(hp), fake, fake, fake,
                          None, fake, fake, 256, 4, 1e-6, 1.0, fake, need - 1, None, None, None,
                          None)
    assert rc == -1 and b"workspace" in L.engram_last_error()
    # bad params struct is caught by engram_hash too
    hp.prime[0] = 4
    assert L.engram_hash(fake, fake, 1, 5, fake, fake, 10, ctypes.byref(hp), fake, None, None) == -1
    # empty calls are no-ops that succeed without a device
    assert L.engram_gather_decode(None, 0, None, None, 0, None, None, None) == 0
    assert L.engram_project(None, 0, None, None, 256, 4, None, None) == 0


def test_forward_checks_its_stage_arguments_on_both_paths(E):
    """engram_forward runs hash + gather as one kernel for T <= 1,024 tokens in
    S <= 1,024 sequences and as two kernels otherwise; either way it applies
    engram_hash's and engram_gather_decode's host checks before any launch."""
    L = E.lib
    p, _ = _params()
    fake = ctypes.c_void_p(0x10000)
    H, hc = 256, 4
    for S, T in ((1, 8), (1, 2000), (1500, 1500)):
        need = L.engram_forward_workspace(T, H, hc)
        ws = ctypes.c_void_p(0x100000)   # 256-byte aligned, never dereferenced
        def fwd(hp, codes=fake, scales=fake, tmap_len=10):
            return L.engram_forward(fake, fake, S, T, fake, fake, tmap_len, ctypes.byref(hp), codes,
                                    scales, fake, None, fake, fake, H, hc, 1e-6, 1.0, ws, need, None,
                                    None, None, None)
        bad = E.HashParams.from_any(p)
        bad.prime[0] = 4
        assert fwd(bad) == -1, (S, T)
        hp = E.HashParams.from_any(p)
        assert fwd(hp, codes=ctypes.c_void_p(0x10008)) == -1, (S, T)     # codes not 16-byte aligned
        assert b"alignment" in L.engram_last_error()
        assert fwd(hp, tmap_len=0) == -1, (S, T)                         # empty token map
    # no tokens: nothing to launch, succeeds without a device
    hp = E.HashParams.from_any(p)
    assert L.engram_forward(None, fake, 1, 0, None, None, 0, ctypes.byref(hp), None, None, None,
                            None, None, None, H, hc, 1e-6, 1.0, None, 0, None, None, None,
                            None) == 0


def test_precompute_and_gate_precomputed_check_arguments_before_launch(E):
    """The split layer (hidden-independent precompute, then the gate at layer
    entry) applies the same host checks as engram_forward before any launch;
    none of these calls reaches a device."""
    L = E.lib
    p, _ = _params()
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x100000)
    H, hc = 256, 4
    for S, T in ((1, 8), (1, 2000)):
        need = L.engram_forward_workspace(T, H, hc)
        def pre(hp, flags=0, ws_bytes=need, w=ws, codes=fake):
            return L.engram_precompute(fake, fake, S, T, fake, fake, 10, ctypes.byref(hp), codes, fake,
                                       fake, None, H, hc, flags, w, ws_bytes, None, None)
        hp = E.HashParams.from_any(p)
        assert pre(hp, ws_bytes=need - 1) == -1 and b"workspace" in L.engram_last_error()
        assert pre(hp, w=ctypes.c_void_p(0x100010)) == -1 and b"256-byte" in L.engram_last_error()
        assert pre(hp, flags=0x2) == -1 and b"flags" in L.engram_last_error()
        assert pre(hp, codes=ctypes.c_void_p(0x10008)) == -1
        bad = E.HashParams.from_any(p)
        bad.prime[3] = 9
        assert pre(bad) == -1
        def gate(ws_bytes=need, tok=fake, S=S, wqk=fake, hidden=fake):
            return L.engram_gate_precomputed(hidden, ws, ws_bytes, tok, S, T, wqk, H, hc, 1e-6, 1.0,
                                             None, None)
        assert gate(ws_bytes=need - 1) == -1 and b"workspace" in L.engram_last_error()
        assert gate(tok=None) == -1
        assert gate(S=0) == -1
        assert gate(wqk=ctypes.c_void_p(0x10004)) == -1
        assert gate(hidden=None) == -1
        assert L.engram_gate_precomputed(fake, ws, need, fake, S, T, fake, 100, hc, 1e-6, 1.0, None,
                                         None) == -1                   # H % 64
    # no tokens: nothing to launch, succeeds without a device
    hp = E.HashParams.from_any(p)
    assert L.engram_precompute(None, fake, 1, 0, None, None, 0, ctypes.byref(hp), None, None, None,
                               None, H, hc, 0, None, 0, None, None) == 0
    assert L.engram_gate_precomputed(None, None, 0, None, 1, 0, None, H, hc, 1e-6, 1.0, None,
                                     None) == 0


def test_precompute_buckets_checks_the_bucket_table_before_launch(E):
    """engram_precompute_buckets rejects a missing table, a NULL or misaligned
    bucket pointer and the precompute's own bad arguments before any launch."""
    L = E.lib
    p, _ = _params()
    hp = E.HashParams.from_any(p)
    fake = ctypes.c_void_p(0x10000)
    H, hc, T = 256, 4, 8
    need = L.engram_forward_workspace(T, H, hc)
    ws = ctypes.c_void_p(0x100000)

    def call(tbl, hp=hp):
        return L.engram_precompute_buckets(fake, fake, 1, T, fake, fake, 10, ctypes.byref(hp),
                                           None if tbl is None else ctypes.byref(tbl), fake, None,
                                           H, hc, 0, ws, need, None, None)
    good = E.BucketTable()
    for j in range(24):
        good.codes[j] = 0x1000000 + j * 0x10000
        good.scales[j] = 0x2000000 + j * 0x1000
    assert call(None) == -1 and b"table" in L.engram_last_error()
    t = E.BucketTable.from_buffer_copy(good)
    t.codes[5] = None
    assert call(t) == -1 and b"bucket 5" in L.engram_last_error()
    t = E.BucketTable.from_buffer_copy(good)
    t.scales[23] = 0x2000004
    assert call(t) == -1 and b"bucket 23" in L.engram_last_error()
    bad = E.HashParams.from_any(p)
    bad.prime[0] = 4
    assert call(good, bad) == -1


def test_pack_wkv_rejects_bad_arguments_before_launch(E):
    """engram_pack_wkv checks shapes, pointers, alignment and overlap on the
    host; none of these calls reaches a device."""
    L = E.lib
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x40000000)
    assert L.engram_pack_wkv(a, 100, 4, b, None) == -1                   # H % 64
    assert L.engram_pack_wkv(a, 256, 0, b, None) == -1                   # hc
    assert L.engram_pack_wkv(None, 256, 4, b, None) == -1
    assert L.engram_pack_wkv(a, 256, 4, None, None) == -1
    assert L.engram_pack_wkv(a, 256, 4, ctypes.c_void_p(0x40000004), None) == -1
    # 5 x 256 rows x 12,288 B = 15.7 MB: a destination 1 MB past wkv overlaps it
    assert L.engram_pack_wkv(a, 256, 4, ctypes.c_void_p(0x100000 + (1 << 20)), None) == -1
    assert b"overlap" in L.engram_last_error()


def test_workspace_size_formula(E):
    T, H, hc = 1000, 5120, 4
    r = lambda x: (x + 255) // 256 * 256
    # idx | slot | live count and one count per 4,096 positions | mem | kv | live positions
    for T in (1, 1000, 4096, 4097, 50032):
        assert E.engram_forward_workspace(T, H, hc) == (r(T * 96) + r(T * 4) + r(4 * (1 + (T + 4095) // 4096))
                                                        + r(T * 12288) + r(T * 25600 * 2) + r(T * 4))
    assert E.engram_forward_workspace(0, H, hc) == 0
    # narrow layers: the kv section still holds the rows staged from a host table
    for T, H, hc in ((64, 256, 4), (3, 64, 1)):
        assert E.engram_forward_workspace(T, H, hc) == (r(T * 96) + r(T * 4) + r(4 * (1 + (T + 4095) // 4096))
                                                        + r(T * 12288) + r(max(T * (hc + 1) * H * 2, T * 24 * 264))
                                                        + r(T * 4))


def test_table_pointers_accept_pinned_host_memory_only(E):
    """Tables may be pinned host memory (mapped into the device's address
    space); plain host memory is refused by the binding before any call."""
    import torch
    plain = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="pinned host tensor"):
        E._ptr(plain, torch.uint8, "codes", host_ok=True)
    with pytest.raises(ValueError, match="device tensor"):
        E._ptr(plain, torch.uint8, "mem")


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "engram.h"

/* A C caller of the ABI, on the host only: version, workspace size and
 * argument checks that reject bad input before anything is launched. */
int main(void) {
  if (engram_abi_version() != ENGRAM_ABI_VERSION) return 10;
  if (engram_forward_workspace(0, 5120, 4) != 0) return 11;
  if (engram_forward_workspace(64, 5120, 4) == 0) return 12;
  if (engram_forward_workspace(1055, 5120, 4) > ENGRAM_NOALLOC_WORKSPACE_BYTES) return 13;
  engram_hash_params p;
  memset(&p, 0, sizeof p);
  if (engram_check_params(&p, NULL, 0) != ENGRAM_EINVAL) return 14;  /* prime[0] = 0 */
  if (strlen(engram_last_error()) == 0) return 15;
  /* H not a multiple of 64: rejected before any launch, whatever the pointers */
  if (engram_project(NULL, 1, NULL, NULL, 100, 4, NULL, 0) != ENGRAM_EINVAL) return 16;
  if (engram_gate(NULL, NULL, NULL, NULL, -1, 64, 1, 1e-6f, 1.0f, NULL, 0) != ENGRAM_EINVAL) return 17;
  printf("ok\n");
  return 0;
}
"""


def test_header_compiles_as_c_and_a_c_program_links_and_runs(E, tmp_path):
    """include/engram.h is plain C: a C99 program that includes it compiles
    with gcc, links against libengram.so and runs its host-only calls."""
    gcc = "gcc"
    if subprocess.run(["which", gcc], capture_output=True).returncode != 0:
        pytest.skip("gcc not found")
    src = tmp_path / "caller.c"
    exe = tmp_path / "caller"
    src.write_text(C_PROGRAM)
    lib_dir = os.path.dirname(E.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           str(src), f"-L{lib_dir}", "-lengram", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # warnings from engram.h itself would show the header is not clean C
    assert "engram.h" not in r.stderr, r.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout, run.stderr)
