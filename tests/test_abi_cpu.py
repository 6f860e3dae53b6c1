"""Host-side checks of libdsa.so that need no GPU: it loads, exports every
entry point include/dsa.h declares, and rejects bad arguments before any HIP
call (so no kernel is ever launched here)."""

import ctypes
import os
import re

import pytest

from dsa_sparse_attention_lightning_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

lib = _lib.load()
FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"dsa_index_scores", "dsa_topk", "dsa_sparse_attn", "spec_verify"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings_and_version():
    assert lib.dsa_abi_version() == 1
    for code in range(5):
        assert lib.dsa_status_str(code).decode().startswith("DSA_")
    assert b"unknown" in lib.dsa_status_str(99)


def _scores_call(**over):
    a = dict(q=FAKE, w=FAKE, k=FAKE, bt=FAKE, rl=FAKE, out=FAKE, B=1, R=1, H=64, D=128, page=64,
             max_pages=4, ld=256)
    a.update(over)
    return lib.dsa_index_scores(a["q"], a["w"], a["k"], a["bt"], a["rl"], a["out"], a["B"], a["R"],
                                a["H"], a["D"], a["page"], a["max_pages"], a["ld"], None)


def test_index_scores_validation():
    assert _scores_call(q=None) == _lib.DSA_ERR_INVALID_ARG
    assert b"null" in lib.dsa_last_error()
    assert _scores_call(B=0) == _lib.DSA_ERR_INVALID_ARG
    assert _scores_call(D=96) == _lib.DSA_ERR_UNSUPPORTED
    assert _scores_call(H=65) == _lib.DSA_ERR_UNSUPPORTED
    assert _scores_call(R=9) == _lib.DSA_ERR_UNSUPPORTED
    assert _scores_call(B=65536) == _lib.DSA_ERR_UNSUPPORTED          # grid limit
    assert _scores_call(q=MISALIGNED) == _lib.DSA_ERR_INVALID_ARG
    assert _scores_call(ld=(1 << 31) - 65536 + 1) == _lib.DSA_ERR_UNSUPPORTED   # past DSA_MAX_LD


def test_topk_validation():
    assert lib.dsa_topk_workspace_size(2, 1, 1000, 64) == 0          # one-workgroup path: none
    ws = lib.dsa_topk_workspace_size(2, 1, 200000, 64)
    assert ws > 0
    assert lib.dsa_topk_workspace_size(0, 1, 1000, 64) == 0
    assert lib.dsa_topk(None, FAKE, 1, 1, 100, 8, FAKE, FAKE, ws, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, FAKE, 1, 1, 100, 0, FAKE, FAKE, ws, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, FAKE, 1, 1, 100, 9000, FAKE, FAKE, ws, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(FAKE, FAKE, 2, 1, 200000, 64, FAKE, FAKE, ws - 1, None) == _lib.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(FAKE, FAKE, 2, 1, 200000, 64, FAKE, None, ws, None) == _lib.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(FAKE, FAKE, 8192, 8, 100, 8, FAKE, FAKE, ws, None) == _lib.DSA_ERR_UNSUPPORTED   # B*R > 65535
    max_ld = (1 << 31) - 65536                                          # DSA_MAX_LD
    assert lib.dsa_topk(FAKE, FAKE, 1, 1, max_ld + 1, 8, FAKE, FAKE, ws, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_workspace_size(1, 1, 35840, 64) == 0            # keys fit in LDS: one launch
    assert lib.dsa_topk_workspace_size(1, 1, 35841, 64) > 0


def _attn_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=64 * 64 * 128, rs=64 * 128, hs=128, bt=FAKE, idx=FAKE, idx_rows=1,
             B=1, S_q=1, H_q=64, H_kv=64, D_qk=128, D_v=128, page=64, max_pages=4, kk=2048, scale=0.1,
             out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return lib.dsa_sparse_attn(a["q"], a["k"], a["v"], a["ps"], a["rs"], a["hs"], a["bt"], a["idx"],
                               a["idx_rows"], a["B"], a["S_q"], a["H_q"], a["H_kv"], a["D_qk"], a["D_v"],
                               a["page"], a["max_pages"], a["kk"], a["scale"], a["out"], a["lse"],
                               a["ws"], a["ws_bytes"], None)


def test_sparse_attn_validation():
    assert _attn_call(q=None) == _lib.DSA_ERR_INVALID_ARG
    assert _attn_call(H_q=63) == _lib.DSA_ERR_INVALID_ARG            # H_q % H_kv
    assert _attn_call(H_kv=8, H_q=64) == _lib.DSA_ERR_UNSUPPORTED     # group 8
    assert _attn_call(D_qk=96, D_v=96) == _lib.DSA_ERR_UNSUPPORTED
    assert _attn_call(idx_rows=3, S_q=2) == _lib.DSA_ERR_INVALID_ARG
    assert _attn_call(rs=64 * 128 + 4) == _lib.DSA_ERR_INVALID_ARG    # row not 16-byte aligned
    assert _attn_call(out=ctypes.c_void_p(0x10004)) == _lib.DSA_ERR_INVALID_ARG   # out not 16-byte aligned
    assert _attn_call(scale=float("nan")) == _lib.DSA_ERR_INVALID_ARG
    assert _attn_call(B=65536) == _lib.DSA_ERR_UNSUPPORTED            # B*S_q grid limit
    need = lib.dsa_sparse_attn_workspace_size(1, 1, 64, 64, 128, 128, 2048)
    assert need > 0
    assert _attn_call(ws_bytes=need - 1) == _lib.DSA_ERR_WORKSPACE


def test_spec_verify_validation():
    ws = lib.spec_verify_workspace_size(4, 7, 1024)
    assert ws > 0
    call = lambda **o: lib.spec_verify(o.get("t", FAKE), FAKE, FAKE, o.get("B", 4), o.get("G", 7),
                                       o.get("V", 1024), None, 0, 0, FAKE, FAKE, None,
                                       o.get("ws", FAKE), o.get("wsb", ws), None)
    assert call(t=None) == _lib.DSA_ERR_INVALID_ARG
    assert call(G=0) == _lib.DSA_ERR_INVALID_ARG
    assert call(G=33) == _lib.DSA_ERR_UNSUPPORTED
    assert call(V=(1 << 20) + 1) == _lib.DSA_ERR_UNSUPPORTED
    assert call(B=5000) == _lib.DSA_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == _lib.DSA_ERR_WORKSPACE


def test_spec_verify_greedy_validation():
    ws = lib.spec_verify_greedy_workspace_size(4, 15, 1024)
    assert ws > 0
    assert lib.spec_verify_greedy_workspace_size(0, 15, 1024) == 0
    call = lambda **o: lib.spec_verify_greedy(o.get("t", FAKE), o.get("d", FAKE), o.get("B", 4), o.get("G", 15),
                                              o.get("V", 1024), FAKE, FAKE, o.get("ws", FAKE), o.get("wsb", ws), None)
    assert call(t=None) == _lib.DSA_ERR_INVALID_ARG
    assert call(d=None) == _lib.DSA_ERR_INVALID_ARG
    assert call(G=0) == _lib.DSA_ERR_INVALID_ARG
    assert call(G=33) == _lib.DSA_ERR_UNSUPPORTED
    assert call(V=(1 << 20) + 1) == _lib.DSA_ERR_UNSUPPORTED
    assert call(B=5000) == _lib.DSA_ERR_UNSUPPORTED
    assert call(wsb=ws - 1) == _lib.DSA_ERR_WORKSPACE
    assert call(ws=None) == _lib.DSA_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        _lib._lib_backup = _lib._lib
        try:
            _lib._lib = None
            _lib.load(str(tmp_path / "missing.so"))
        finally:
            _lib._lib = _lib._lib_backup


def _noalloc_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ps=64 * 64 * 128, rs=64 * 128, hs=128, bt=FAKE, idx=FAKE, idx_rows=1,
             B=1, S_q=1, H_q=64, H_kv=64, D_qk=128, D_v=128, page=64, max_pages=4, kk=2048, scale=0.1,
             out=FAKE, lse=None)
    a.update(over)
    return lib.dsa_sparse_attn_noalloc(a["q"], a["k"], a["v"], a["ps"], a["rs"], a["hs"], a["bt"], a["idx"],
                                       a["idx_rows"], a["B"], a["S_q"], a["H_q"], a["H_kv"], a["D_qk"], a["D_v"],
                                       a["page"], a["max_pages"], a["kk"], a["scale"], a["out"], a["lse"], None)


def test_sparse_attn_noalloc_validation():
    """The allocation-free entry point checks its arguments like
    dsa_sparse_attn, and refuses shapes whose split-k partials exceed its
    fixed scratch, all before any HIP call."""
    text = open(HEADER).read()
    m = re.search(r"#define DSA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc_call(q=None) == _lib.DSA_ERR_INVALID_ARG
    assert _noalloc_call(H_q=63) == _lib.DSA_ERR_INVALID_ARG
    assert _noalloc_call(D_qk=96, D_v=96) == _lib.DSA_ERR_UNSUPPORTED
    assert _noalloc_call(out=MISALIGNED) == _lib.DSA_ERR_INVALID_ARG
    need = lib.dsa_sparse_attn_workspace_size(1, 8, 64, 64, 128, 128, 131072)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc_call(S_q=8, kk=131072) == _lib.DSA_ERR_UNSUPPORTED
    assert b"scratch" in lib.dsa_last_error()


def _params(fn):
    """Parameter list of `fn` as declared in include/dsa.h (comments removed)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + fn + r"\s*\(([^)]*)\)", text)
    assert m, fn
    return [p.strip() for p in m.group(1).replace("\n", " ").split(",") if p.strip() and p.strip() != "void"]


def test_boundary_departures_are_the_recorded_ones():
    """Where the exported signatures differ from the boundary sketched for
    the four calls (status/version helpers, index_scores, topk, sparse_attn
    and spec_verify), each difference is deliberate and listed in the
    design notes; this pins every one of them."""
    assert _params("dsa_status_str") == ["int status"]                       # int, not the enum type
    idx = _params("dsa_index_scores")
    assert idx[-2:] == ["int64_t ld", "void* stream"]                         # 64-bit ld, stream as void*
    assert _params("dsa_topk_workspace_size") == ["int B", "int R", "int64_t ld", "int k"]
    ws = _params("dsa_sparse_attn_workspace_size")
    assert ws == ["int B", "int S_q", "int H_q", "int H_kv", "int D_qk", "int D_v", "int k"]   # + H_kv, D_qk
    attn = _params("dsa_sparse_attn")
    assert attn[7:9] == ["const int32_t* idx", "int idx_rows"]               # per-row index sets
    sv = _params("spec_verify")
    assert "const float* uniforms" in sv and sv.index("const float* uniforms") == 6   # caller-supplied uniforms
    assert "float* diag" in sv
    text = open(HEADER).read()
    assert "diag          fp32 [B, G+1, 4]" in text                          # p, q, u_acc, u_smp per position
    assert "D_I in {32, 64, 128}" in text
    # entry points beyond the four calls and their helpers
    for extra in ("dsa_last_error", "spec_verify_greedy", "spec_verify_greedy_workspace_size",
                  "dsa_sparse_attn_noalloc"):
        assert extra in declared_functions()


def test_verify_workspace_size_does_not_depend_on_the_schedule(monkeypatch):
    """The verify schedules (one pass, early exit) share one workspace size, so
    a workspace sized once serves either, whatever DSA_VERIFY_SCHEDULE says;
    the size covers the early-exit bookkeeping at every size."""
    shapes = [(1, 1, 10), (16, 7, 151552), (256, 7, 151552), (3, 32, 4099), (300, 1, 80000), (4, 7, 1 << 20)]
    sizes = {}
    for sched in (None, "onepass", "phased"):
        if sched is None:
            monkeypatch.delenv("DSA_VERIFY_SCHEDULE", raising=False)
        else:
            monkeypatch.setenv("DSA_VERIFY_SCHEDULE", sched)
        sizes[sched] = [(lib.spec_verify_workspace_size(B, G, V), lib.spec_verify_greedy_workspace_size(B, G, V))
                        for B, G, V in shapes]
    assert sizes[None] == sizes["onepass"] == sizes["phased"]
    for (B, G, V), (ws, gws) in zip(shapes, sizes[None]):
        # at least one (max, sum) partial per row, the reach flags and the
        # drafted tokens' logits; greedy: one argmax partial per row and the flags
        assert ws >= B * (2 * G + 1) * 8 + (G + 1) * B * 4 + B * G * 8
        assert gws >= B * (G + 1) * 8 + (G + 1) * B * 4
