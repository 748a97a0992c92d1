"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before any HIP
call. Every call here fails validation, so no kernel is ever launched (the
pointers are never dereferenced)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import block_scoring_top_amd as idx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH, NOMEM = 0, -1, -2, -3, -4, -5, -6
P = 1 << 20  # a 16-byte aligned fake device address; never dereferenced here


def declared():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(idx.lib_path()):
        pytest.skip("libidx.so not built")
    return idx.load()


def test_header_declares_the_entry_points():
    names = declared()
    for n in ["idx_score", "idx_topk", "idx_topk_bf16", "idx_select", "idx_select_noalloc",
              "idx_select_paged",
              "idx_select_prefill",
              "idx_prefill_workspace_bytes", "idx_pool_keys", "idx_assign",
              "idx_workspace_bytes",
              "idx_topk_workspace_bytes", "idx_assign_workspace_bytes", "idx_status_string",
              "idx_plan_create", "idx_plan_select", "idx_plan_workspace_bytes", "idx_plan_destroy"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", idx.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert idx.idx_status_string(OK) == "ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH, NOMEM):
        assert idx.idx_status_string(s) not in ("ok", "unknown status")
    assert idx.idx_status_string(12345) == "unknown status"


def test_workspace_sizes(lib):
    # 2 MiB of arrival counters (128 B each), then B rows of round_up(N_pad, 4) floats
    assert lib.idx_workspace_bytes(4, 8192, 4, 256, 0) == (2 << 20) + 4 * 8192 * 4
    assert lib.idx_workspace_bytes(1, 1001, 4, 8, 0) == (2 << 20) + 1004 * 4
    assert lib.idx_workspace_bytes(0, 10, 4, 8, 0) == 0
    assert lib.idx_assign_workspace_bytes(1024, 128) == 4096
    assert lib.idx_assign_workspace_bytes(1, 128) == 512
    assert lib.idx_assign_workspace_bytes(1031, 128) == 1152 * 4


def test_topk_workspace_sizes(lib):
    # few long rows: arrival lines for the most rows that are ever split (256 of
    # 128 bytes, whatever B is) + B * round_up(S*K, 4) candidate scores and ids;
    # here S = 4 segments (64 rows x 30000, K = 2048)
    assert lib.idx_topk_workspace_bytes(64, 30000, 2048, 0) == 256 * 128 + 64 * 8192 * 8
    assert lib.idx_topk_workspace_bytes(3, 40000, 100, 0) == 256 * 128 + 3 * 800 * 8
    assert lib.idx_topk_workspace_bytes(257, 40000, 100, 0) == 0   # no row is split
    assert lib.idx_topk_workspace_bytes(1000, 30000, 10, 0) == 0   # enough rows already
    assert lib.idx_topk_workspace_bytes(64, 2000, 10, 0) == 0       # short rows
    assert lib.idx_topk_workspace_bytes(0, 30000, 10, 0) == 0


def test_topk_long_rows_require_the_workspace(lib):
    assert topk_call(lib, B=64, N=30000, K=2048) == WORKSPACE
    assert topk_call(lib, B=64, N=30000, K=2048, ws=P, ws_bytes=100) == WORKSPACE
    assert topk_call(lib, B=64, N=30000, K=2048, ws=P + 16, ws_bytes=1 << 30) == WORKSPACE


def score_call(lib, **kw):
    a = dict(q=P, c=P, seq_len=P, scores=P, B=1, H=4, D=128, N_pad=64, page_size=16, dt=1)
    a.update(kw)
    return lib.idx_score(a["q"], a["c"], a["seq_len"], a["scores"], a["B"], a["H"], a["D"],
                         a["N_pad"], a["page_size"], a["dt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(c=None), INVALID), (dict(seq_len=None), INVALID),
    (dict(scores=None), INVALID), (dict(q=P + 8), INVALID), (dict(c=P + 4), INVALID),
    (dict(seq_len=P + 2), INVALID), (dict(B=0), INVALID), (dict(H=0), INVALID),
    (dict(N_pad=0), INVALID), (dict(page_size=0), INVALID), (dict(dt=7), INVALID),
    (dict(D=64), UNSUPPORTED), (dict(H=65), UNSUPPORTED), (dict(B=1 << 20, N_pad=1 << 12), INVALID),
])
def test_score_rejects(lib, kw, want):
    assert score_call(lib, **kw) == want


def topk_call(lib, **kw):
    a = dict(scores=P, n_valid=None, ids=P, counts=None, B=2, N=100, K=10, flags=0, ws=None,
             ws_bytes=0)
    a.update(kw)
    return lib.idx_topk(a["scores"], a["n_valid"], a["ids"], a["counts"], a["B"], a["N"], a["K"],
                        a["flags"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(scores=None), INVALID), (dict(ids=None), INVALID), (dict(scores=P + 4), INVALID),
    (dict(ids=P + 2), INVALID), (dict(n_valid=P + 1), INVALID), (dict(counts=P + 3), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(K=0), INVALID), (dict(flags=0x80), INVALID),
    (dict(K=4097, flags=1), UNSUPPORTED),
])
def test_topk_rejects(lib, kw, want):
    assert topk_call(lib, **kw) == want


def topk_bf16_call(lib, **kw):
    a = dict(scores=P, n_valid=None, ids=P, counts=None, B=2, N=100, K=10, flags=0, ws=None,
             ws_bytes=0)
    a.update(kw)
    return lib.idx_topk_bf16(a["scores"], a["n_valid"], a["ids"], a["counts"], a["B"], a["N"],
                             a["K"], a["flags"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(scores=None), INVALID), (dict(ids=None), INVALID), (dict(scores=P + 4), INVALID),
    (dict(scores=P + 2), INVALID), (dict(ids=P + 2), INVALID), (dict(n_valid=P + 1), INVALID),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(K=0), INVALID), (dict(flags=0x80), INVALID),
    (dict(K=4097, flags=1), UNSUPPORTED), (dict(B=64, N=30000, K=2048), WORKSPACE),
    (dict(flags=2), UNSUPPORTED),            # IDX_RADIX8: 32-bit keys only
])
def test_topk_bf16_rejects(lib, kw, want):
    assert topk_bf16_call(lib, **kw) == want


def select_call(lib, **kw):
    a = dict(q=P, c=P, seq_len=P, ids=P, counts=None, scores_out=None, B=2, H=4, D=128,
             N_pad=100, page_size=16, K=10, dt=1, flags=0, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    return lib.idx_select(a["q"], a["c"], a["seq_len"], a["ids"], a["counts"], a["scores_out"],
                          a["B"], a["H"], a["D"], a["N_pad"], a["page_size"], a["K"], a["dt"],
                          a["flags"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(ids=None), INVALID), (dict(ids=P + 1), INVALID),
    (dict(scores_out=P + 2), INVALID), (dict(K=0), INVALID), (dict(B=0), INVALID),
    (dict(flags=0x4), INVALID), (dict(flags=3 << 8), INVALID),
    (dict(flags=15 << 8), INVALID), (dict(D=256), UNSUPPORTED), (dict(K=5000, flags=1), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE), (dict(ws=P + 16), WORKSPACE),
    (dict(B=16385, N_pad=4), UNSUPPORTED),
])
def test_select_rejects(lib, kw, want):
    assert select_call(lib, **kw) == want


def noalloc_call(lib, **kw):
    a = dict(q=P, c=P, seq_len=P, ids=P, counts=None, scores_out=None, B=2, H=4, D=128,
             N_pad=100, page_size=16, K=10, dt=1, flags=0)
    a.update(kw)
    return lib.idx_select_noalloc(a["q"], a["c"], a["seq_len"], a["ids"], a["counts"],
                                  a["scores_out"], a["B"], a["H"], a["D"], a["N_pad"],
                                  a["page_size"], a["K"], a["dt"], a["flags"], None)


# the static scratch: 16 MiB = 4096 arrival lines of 128 B + 15.5 MiB of staging
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(ids=None), INVALID), (dict(ids=P + 1), INVALID),
    (dict(scores_out=P + 2), INVALID), (dict(K=0), INVALID), (dict(B=0), INVALID),
    (dict(flags=0x4), INVALID), (dict(D=256), UNSUPPORTED), (dict(K=5000, flags=1), UNSUPPORTED),
    (dict(B=16385, N_pad=4), UNSUPPORTED),
    (dict(B=4097, N_pad=4), SCRATCH),
    (dict(B=64, N_pad=63489), SCRATCH),      # 64 * 63492 * 4 B > 15.5 MiB of staging
    (dict(B=4096, N_pad=1000), SCRATCH),
])
def test_select_noalloc_rejects(lib, kw, want):
    assert noalloc_call(lib, **kw) == want


def test_noalloc_scratch_limits_in_the_header():
    src = open(os.path.join(ROOT, "include", "idx.h")).read()
    assert "#define IDX_NOALLOC_SCRATCH_BYTES (16u << 20)" in src
    assert "#define IDX_NOALLOC_MAX_REQUESTS 4096" in src


def paged_call(lib, **kw):
    a = dict(q=P, c=P, indptr=P, indices=P, ids=P, counts=None, scores_out=None, B=2, H=4, D=128,
             n_rows=1000, n_indices=500, max_pages=300, K=10, dt=1, flags=0, ws=None,
             ws_bytes=1 << 22)
    a.update(kw)
    return lib.idx_select_paged(a["q"], a["c"], a["indptr"], a["indices"], a["ids"], a["counts"],
                                a["scores_out"], a["B"], a["H"], a["D"], a["n_rows"],
                                a["n_indices"], a["max_pages"], a["K"], a["dt"], a["flags"],
                                a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(c=None), INVALID), (dict(indptr=None), INVALID),
    (dict(ids=None), INVALID), (dict(indices=None), INVALID), (dict(indptr=P + 2), INVALID),
    (dict(indices=P + 1), INVALID), (dict(c=P + 8), INVALID), (dict(B=0), INVALID),
    (dict(n_rows=0), INVALID), (dict(n_indices=-1), INVALID), (dict(max_pages=0), INVALID),
    (dict(K=0), INVALID), (dict(dt=5), INVALID), (dict(flags=0x4), INVALID),
    (dict(D=64), UNSUPPORTED), (dict(H=65), UNSUPPORTED), (dict(K=5000, flags=1), UNSUPPORTED),
    (dict(B=16385, max_pages=4), UNSUPPORTED), (dict(ws=None), WORKSPACE),
    (dict(ws=P, ws_bytes=100), WORKSPACE), (dict(ws=P + 16), WORKSPACE),
    (dict(flags=2), UNSUPPORTED),            # IDX_RADIX8: dense tables only
])
def test_select_paged_rejects(lib, kw, want):
    assert paged_call(lib, **kw) == want


def test_select_paged_accepts_an_empty_index_list_without_a_pointer(lib):
    # no list entries at all: a NULL list is legal; the call then fails only on
    # the (missing) workspace, before any launch
    assert paged_call(lib, indices=None, n_indices=0) == WORKSPACE


def prefill_call(lib, **kw):
    a = dict(q=P, c=P, pos0=P, ids=P, counts=None, scores_out=None, B=2, T=64, H=4, D=128,
             N_pad=500, page_size=16, K=10, dt=1, flags=0, ws=None, ws_bytes=1 << 22)
    a.update(kw)
    return lib.idx_select_prefill(a["q"], a["c"], a["pos0"], a["ids"], a["counts"],
                                  a["scores_out"], a["B"], a["T"], a["H"], a["D"], a["N_pad"],
                                  a["page_size"], a["K"], a["dt"], a["flags"], a["ws"],
                                  a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVALID), (dict(c=None), INVALID), (dict(pos0=None), INVALID),
    (dict(ids=None), INVALID), (dict(q=P + 8), INVALID), (dict(pos0=P + 2), INVALID),
    (dict(scores_out=P + 4), INVALID), (dict(B=0), INVALID), (dict(T=0), INVALID),
    (dict(N_pad=0), INVALID), (dict(page_size=0), INVALID), (dict(K=0), INVALID),
    (dict(dt=3), INVALID), (dict(flags=0x100), INVALID), (dict(dt=0), UNSUPPORTED),
    (dict(D=64), UNSUPPORTED), (dict(H=65), UNSUPPORTED), (dict(K=5000, flags=1), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws=P, ws_bytes=64), WORKSPACE), (dict(ws=P + 64), WORKSPACE),
    (dict(flags=2), UNSUPPORTED), (dict(flags=3), UNSUPPORTED),  # IDX_RADIX8
    # fp32 inputs only on the short-prompt route (T <= 8, B*T <= 256)
    (dict(dt=0, T=4), WORKSPACE), (dict(dt=0, B=32, T=8), WORKSPACE),
    (dict(dt=0, B=33, T=8), UNSUPPORTED), (dict(dt=0, B=1, T=9), UNSUPPORTED),
])
def test_select_prefill_rejects(lib, kw, want):
    assert prefill_call(lib, **kw) == want


def test_prefill_workspace_size(lib):
    # 256 arrival lines of 128 bytes, per-token block counts (256-byte aligned),
    # then B*T staged rows of round_up(N_pad, 4)
    assert lib.idx_prefill_workspace_bytes(2, 64, 500, 10, 0) == 256 * 128 + 512 + 128 * 500 * 4
    assert lib.idx_prefill_workspace_bytes(1, 3, 7, 10, 0) == 256 * 128 + 256 + 3 * 8 * 4
    assert lib.idx_prefill_workspace_bytes(0, 3, 7, 10, 0) == 0


def pool_call(lib, **kw):
    a = dict(k=P, seq_len=P, c=P, B=2, S_pad=1000, D=128, N_pad=63, page_size=16, dt=1)
    a.update(kw)
    return lib.idx_pool_keys(a["k"], a["seq_len"], a["c"], a["B"], a["S_pad"], a["D"], a["N_pad"],
                             a["page_size"], a["dt"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(k=None), INVALID), (dict(seq_len=None), INVALID), (dict(c=None), INVALID),
    (dict(k=P + 8), INVALID), (dict(c=P + 4), INVALID), (dict(seq_len=P + 1), INVALID),
    (dict(B=0), INVALID), (dict(S_pad=0), INVALID), (dict(N_pad=0), INVALID),
    (dict(page_size=0), INVALID), (dict(dt=9), INVALID), (dict(D=64), UNSUPPORTED),
    (dict(B=1 << 20, S_pad=1 << 12), INVALID),
])
def test_pool_keys_rejects(lib, kw, want):
    assert pool_call(lib, **kw) == want


def assign_call(lib, **kw):
    a = dict(x=P, c=P, assign=P, best=None, N=1000, C=64, D=128, dt=1, ws=P, ws_bytes=4096)
    a.update(kw)
    return lib.idx_assign(a["x"], a["c"], a["assign"], a["best"], a["N"], a["C"], a["D"], a["dt"],
                          a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), INVALID), (dict(c=None), INVALID), (dict(assign=None), INVALID),
    (dict(x=P + 8), INVALID), (dict(best=P + 1), INVALID), (dict(N=0), INVALID),
    (dict(C=0), INVALID), (dict(C=65537), INVALID), (dict(dt=0), UNSUPPORTED),
    (dict(D=64), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=4), WORKSPACE),
])
def test_assign_rejects(lib, kw, want):
    assert assign_call(lib, **kw) == want


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(idx, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(idx, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        idx.load()


def test_floor_launches_reject_bad_arguments(lib):
    assert "idx_floor_empty" in declared() and "idx_floor_read" in declared()
    assert lib.idx_floor_empty(0, None) == INVALID
    assert lib.idx_floor_empty(65537, None) == INVALID
    r = lib.idx_floor_read
    assert r(None, 1024, P, None, 4, 256, None) == INVALID      # no source
    assert r(P, 1024, None, None, 4, 256, None) == INVALID      # no sink
    assert r(P, 0, P, None, 4, 256, None) == INVALID            # nothing to read
    assert r(P, 1000, P, None, 4, 256, None) == INVALID         # not whole 16-byte words
    assert r(P + 8, 1024, P, None, 4, 256, None) == INVALID     # misaligned source
    assert r(P, 1024, P, None, 0, 256, None) == INVALID         # no workgroups
    assert r(P, 1024, P, None, 4, 512, None) == INVALID         # unsupported block size
    assert r(P, 1024, P, P + 2, 4, 256, None) == INVALID        # misaligned ticket
    assert "idx_floor_mfma" in declared()
    m = lib.idx_floor_mfma
    assert m(None, 4, 8, P, None) == INVALID                    # no fragments
    assert m(P, 4, 8, None, None) == INVALID                    # no sink
    assert m(P, 0, 8, P, None) == INVALID                       # no workgroups
    assert m(P, 65537, 8, P, None) == INVALID                   # too many
    assert m(P, 4, 0, P, None) == INVALID                       # no products
    assert m(P, 4, 12, P, None) == INVALID                      # not whole rounds of eight
    assert m(P, 4, 16392, P, None) == INVALID                   # beyond the exact-sum range
    assert m(P + 8, 4, 8, P, None) == INVALID                   # misaligned fragments
    assert m(P, 4, 8, P + 2, None) == INVALID                   # misaligned sink


def plan_create(lib, **kw):
    a = dict(B=4, H=4, D=128, N_pad=8192, page_size=16, K=256, dt=1, flags=0)
    a.update(kw)
    h = ctypes.c_void_p(12345)
    st = lib.idx_plan_create(ctypes.byref(h), a["B"], a["H"], a["D"], a["N_pad"], a["page_size"],
                             a["K"], a["dt"], a["flags"])
    return st, h


@pytest.mark.parametrize("kw,want", [
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(N_pad=0), INVALID),
    (dict(page_size=0), INVALID), (dict(K=0), INVALID), (dict(dt=7), INVALID),
    (dict(flags=0x4), INVALID), (dict(flags=3 << 8), INVALID), (dict(D=64), UNSUPPORTED),
    (dict(H=65), UNSUPPORTED), (dict(K=5000, flags=1), UNSUPPORTED),
    (dict(B=16385, N_pad=4), UNSUPPORTED), (dict(B=1 << 20, N_pad=1 << 12), INVALID),
])
def test_plan_create_rejects(lib, kw, want):
    st, h = plan_create(lib, **kw)
    assert st == want and h.value is None


def test_plan_create_resolves_on_the_host_and_checks_pointers(lib):
    st, h = plan_create(lib)
    assert st == OK and h.value is not None
    try:
        assert lib.idx_plan_workspace_bytes(h) == lib.idx_workspace_bytes(4, 8192, 4, 256, 0)
        ws = lib.idx_plan_workspace_bytes(h)
        call = lambda **kw: lib.idx_plan_select(
            kw.get("plan", h), kw.get("q", P), kw.get("c", P), kw.get("seq_len", P),
            kw.get("ids", P), kw.get("counts", None), kw.get("scores_out", None),
            kw.get("ws", P), kw.get("ws_bytes", ws), None)
        assert call(plan=None) == INVALID
        for k in ("q", "c", "seq_len", "ids"):
            assert call(**{k: None}) == INVALID, k
        assert call(q=P + 8) == INVALID and call(ids=P + 2) == INVALID
        assert call(counts=P + 1) == INVALID and call(scores_out=P + 2) == INVALID
        assert call(ws=None) == WORKSPACE and call(ws_bytes=ws - 1) == WORKSPACE
        assert call(ws=P + 16) == WORKSPACE
    finally:
        lib.idx_plan_destroy(h)
    lib.idx_plan_destroy(None)
    assert lib.idx_plan_workspace_bytes(None) == 0


def test_radix8_flag_in_the_header_and_accepted_by_a_plan(lib):
    src = open(os.path.join(ROOT, "include", "idx.h")).read()
    assert "#define IDX_RADIX8 0x2u" in src
    for flags in (2, 3):
        st, h = plan_create(lib, flags=flags)
        assert st == OK and h.value is not None
        lib.idx_plan_destroy(h)
