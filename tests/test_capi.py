"""CPU tests of the C ABI: the library loads, exports every symbol that
include/*.h declares, and rejects bad arguments with the documented status
before launching anything (no GPU needed: validation runs on the host)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

import attention_ragged_gqa_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ra.lib_path()):
        pytest.fail("libragattn.so is not built (run __graft_entry__.build())")
    return ra.library()


def test_header_declares_the_boundary():
    assert _declared() == set(ra.EXPORTED_SYMBOLS)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ra.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ra_[a-z_0-9]+)\b", out))
    assert _declared() <= exported
    for name in _declared():
        assert getattr(lib, name) is not None


def _tree(lib, **kw):
    a = dict(batch=1, total_q=4, total_kv=4, tree_size=4, h_q=8, h_kv=2, d=128, dtype=0, rot=0,
             scale=1.0, theta=1e4, sm=0.1)
    a.update(kw)
    P = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    nul = None
    ptrs = [P] * 10
    for i in kw.get("null", ()):
        ptrs[i] = nul
    return lib.ra_tree_attn(*ptrs, a["batch"], a["total_q"], a["total_kv"], a["tree_size"], a["h_q"],
                            a["h_kv"], a["d"], a["dtype"], a["rot"], a["scale"], a["theta"], a["sm"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=6, h_kv=4), ra.RA_EINVAL),
    (dict(h_kv=0), ra.RA_EINVAL),
    (dict(batch=-1), ra.RA_EINVAL),
    (dict(rot=2), ra.RA_EINVAL),
    (dict(sm=0.0), ra.RA_EINVAL),
    (dict(sm=float("nan")), ra.RA_EINVAL),
    (dict(rot=1, theta=-1.0), ra.RA_EINVAL),
    (dict(null=(0,)), ra.RA_EINVAL),            # q
    (dict(null=(7,)), ra.RA_EINVAL),            # tree_mask
    (dict(null=(4,)), ra.RA_EINVAL),            # kv_indptr
    (dict(rot=1, null=(5,)), ra.RA_EINVAL),     # q_rope_position
    (dict(d=96), ra.RA_EUNSUPPORTED),
    (dict(dtype=7), ra.RA_EUNSUPPORTED),
    # size limits: 32-bit (token, head) rows, 2^31-byte index arrays
    (dict(total_q=1 << 26, total_kv=4, h_q=64, h_kv=8), ra.RA_EUNSUPPORTED),   # total_q * h_q = 2^32
    (dict(total_q=(1 << 29) + 1, total_kv=4, h_q=2, h_kv=2), ra.RA_EUNSUPPORTED),
    (dict(tree_size=1 << 28), ra.RA_EUNSUPPORTED),
])
def test_tree_attn_rejects(lib, kw, status):
    assert _tree(lib, **kw) == status
    assert ra.ra_last_error() != ""


def test_empty_problem_is_ok_without_launch(lib):
    assert _tree(lib, batch=0, total_q=0) == ra.RA_OK
    assert ra.ra_last_error() == ""


def _paged(lib, **kw):
    a = dict(sliding=0, causal=1, batch=1, total_q=4, num_pages=4, nnz=4, tree_size=0, page=16,
             h_q=8, h_kv=2, d=128, dtype=1, rot=0, scale=1.0, theta=1e4, sm=0.1)
    a.update(kw)
    P = ctypes.c_void_p(0x1000)
    ptrs = {"q": P, "q_indptr": P, "pages": P, "page_indptr": P, "page_values": P, "length_info": P,
            "k_rope_pos_offset": None, "q_rope_position": None, "tree_order_indptr": None,
            "tree_order": None, "out": P, "lse": P}
    ptrs.update(kw.get("ptrs", {}))
    return lib.ra_paged_attn(ptrs["q"], ptrs["q_indptr"], ptrs["pages"], ptrs["page_indptr"],
                             ptrs["page_values"], ptrs["length_info"], a["sliding"],
                             ptrs["k_rope_pos_offset"], ptrs["q_rope_position"],
                             ptrs["tree_order_indptr"], ptrs["tree_order"], a["causal"], ptrs["out"],
                             ptrs["lse"], a["batch"], a["total_q"], a["num_pages"], a["nnz"],
                             a["tree_size"], a["page"], a["h_q"], a["h_kv"], a["d"], a["dtype"],
                             a["rot"], a["scale"], a["theta"], a["sm"], None)


P_ = ctypes.c_void_p(0x1000)


@pytest.mark.parametrize("kw,status", [
    (dict(page=32), ra.RA_EUNSUPPORTED),
    (dict(sliding=2), ra.RA_EINVAL),
    (dict(sliding=1, tree_size=4, ptrs={"tree_order_indptr": P_, "tree_order": P_}), ra.RA_EUNSUPPORTED),
    (dict(ptrs={"tree_order": P_}), ra.RA_EINVAL),                       # tree without indptr
    (dict(tree_size=4, ptrs={"tree_order_indptr": P_}), ra.RA_EINVAL),  # indptr without tree
    (dict(rot=1), ra.RA_EINVAL),                                          # no q_rope_position
    (dict(ptrs={"page_indptr": None}), ra.RA_EINVAL),
    (dict(ptrs={"length_info": None}), ra.RA_EINVAL),
    (dict(h_q=12, h_kv=8), ra.RA_EINVAL),
    (dict(d=256), ra.RA_EUNSUPPORTED),
    (dict(nnz=1 << 27), ra.RA_EUNSUPPORTED),
    (dict(total_q=(1 << 31) // 8, h_q=8, h_kv=2), ra.RA_EUNSUPPORTED),   # total_q * h_q = 2^31
])
def test_paged_attn_rejects(lib, kw, status):
    assert _paged(lib, **kw) == status
    assert ra.ra_last_error() != ""


def _split(lib, splits, ws_bytes, ws=ctypes.c_void_p(0x2000), **kw):
    a = dict(sliding=0, causal=1, batch=1, total_q=4, num_pages=4, nnz=4, tree_size=0, page=16,
             h_q=8, h_kv=2, d=128, dtype=1, rot=0, scale=1.0, theta=1e4, sm=0.1)
    a.update(kw)
    P = ctypes.c_void_p(0x1000)
    return lib.ra_paged_attn_split(P, P, P, P, P, P, a["sliding"], None, None, None, None,
                                   a["causal"], P, P, a["batch"], a["total_q"], a["num_pages"],
                                   a["nnz"], a["tree_size"], a["page"], a["h_q"], a["h_kv"], a["d"],
                                   a["dtype"], a["rot"], a["scale"], a["theta"], a["sm"], splits,
                                   ws, ws_bytes, None)


def test_split_workspace_size(lib):
    # splits * rows * (d + 1) floats, the output part rounded up to 256 bytes
    assert ra.ra_paged_attn_split_workspace(4, 8, 128, 1) == 0
    assert ra.ra_paged_attn_split_workspace(4, 8, 128, 3) == 3 * 32 * 128 * 4 + 3 * 32 * 4
    assert ra.ra_paged_attn_split_workspace(5, 3, 64, 2) == (2 * 15 * 64 * 4 + 255) // 256 * 256 + 2 * 15 * 4
    assert ra.ra_paged_attn_split_workspace(0, 8, 128, 4) == 0


def test_split_rejects(lib):
    need = ra.ra_paged_attn_split_workspace(4, 8, 128, 4)
    assert _split(lib, 65, 1 << 20) == ra.RA_EINVAL             # too many splits
    assert _split(lib, -1, 1 << 20) == ra.RA_EINVAL
    assert _split(lib, 4, need - 1) == ra.RA_EINVAL             # explicit count, workspace too small
    assert _split(lib, 4, need, ws=None) == ra.RA_EINVAL        # NULL workspace
    assert _split(lib, 4, need, d=96) == ra.RA_EUNSUPPORTED     # same checks as ra_paged_attn
    assert _split(lib, 4, need, batch=0, total_q=0) == ra.RA_OK  # nothing to do, no launch


def test_merge_rejects(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.ra_merge_states(P, P, 0, 4, 128, 1, P, P, None) == ra.RA_EINVAL
    assert lib.ra_merge_states(P, P, 65, 4, 128, 1, P, P, None) == ra.RA_EINVAL
    assert lib.ra_merge_states(P, P, 2, -1, 128, 1, P, P, None) == ra.RA_EINVAL
    assert lib.ra_merge_states(P, P, 2, 4, 96, 1, P, P, None) == ra.RA_EUNSUPPORTED
    assert lib.ra_merge_states(None, P, 2, 4, 128, 1, P, P, None) == ra.RA_EINVAL
    assert lib.ra_merge_states(P, P, 2, 0, 128, 1, P, P, None) == ra.RA_OK


def test_ragged_prefill_rejects(lib):
    P = ctypes.c_void_p(0x1000)
    def call(valid=P, pad=0, causal=1, batch=1, total_q=4, d=128, kv=P):
        return lib.ra_ragged_prefill(P, P, P, P, kv, valid, pad, causal, P, P, batch, total_q, 8, 8, 2,
                                     d, 1, 0.1, None)
    assert call(pad=3) == ra.RA_EINVAL
    assert call(pad=1, causal=1) == ra.RA_EINVAL       # right padding is not causal
    assert call(pad=2, causal=0) == ra.RA_EINVAL       # left padding is causal
    assert call(pad=1, causal=0, valid=None) == ra.RA_EINVAL
    assert call(kv=None) == ra.RA_EINVAL
    assert call(d=80) == ra.RA_EUNSUPPORTED
    assert call(batch=0, total_q=0) == ra.RA_OK


def test_append_rejects(lib):
    P = ctypes.c_void_p(0x1000)
    st = lib.ra_paged_kv_append(P, P, P, P, None, P, P, P, 0, 5, 4, 4, 16, 2, 128, 1, 1.0, 1e4, None)
    assert st == ra.RA_EINVAL                                   # tokens without sequences
    st = lib.ra_paged_kv_append(P, P, P, P, None, P, P, P, 1, 5, 4, 4, 8, 2, 128, 1, 1.0, 1e4, None)
    assert st == ra.RA_EUNSUPPORTED                             # page_size 8
    st = lib.ra_paged_kv_append(P, None, P, P, None, P, P, P, 1, 5, 4, 4, 16, 2, 128, 1, 1.0, 1e4, None)
    assert st == ra.RA_EINVAL                                   # v NULL
    st = lib.ra_paged_kv_append(P, P, P, P, None, P, P, P, 1, 0, 4, 4, 16, 2, 128, 1, 1.0, 1e4, None)
    assert st == ra.RA_OK                                       # nothing to append


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("RAGATTN_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ra, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        ra.library()


def test_set_workgroup_waves_validates(lib):
    for bad in (-1, 1, 2, 3, 5, 16):
        assert lib.ra_set_workgroup_waves(bad) == ra.RA_EINVAL
        assert "waves" in ra.ra_last_error()
    for good in (4, 8, 0):
        assert lib.ra_set_workgroup_waves(good) == ra.RA_OK


def test_workgroup_waves_policy(lib):
    """Eight waves when the 256-row items cover the 256 CUs at least twice,
    four otherwise and for split-KV launches; the override wins; invalid
    sizes give 0."""
    q = ra.ra_attn_workgroup_waves
    assert q(1024, 32, 8) == 4              # 16 trees x 64 nodes: 128 items of 256 rows
    assert q(11414, 32, 8) == 8             # ragged causal prefill: ~1427 items
    assert q(32768, 64, 8) == 8             # speculative tree: 8192 items
    assert q(16, 32, 8) == 4                # decode
    assert q(32768, 64, 8, 4) == 4          # split-KV
    assert q(16384, 4, 1) == 4 and q(32768, 4, 1) == 8   # boundary: 256 vs 512 items
    assert q(10, 6, 4) == 0 and q(-1, 8, 2) == 0 and q(10, 8, 0) == 0
    try:
        ra.ra_set_workgroup_waves(8)
        assert q(1024, 32, 8) == 8 and q(32768, 64, 8, 4) == 4
        ra.ra_set_workgroup_waves(4)
        assert q(32768, 64, 8) == 4
    finally:
        ra.ra_set_workgroup_waves(0)
    assert q(32768, 64, 8) == 8


def test_mla_rejects(lib):
    P = ctypes.c_void_p(0x1000)

    def call(batch=1, total_q=4, num_pages=4, nnz=4, page=16, h_q=16, d_qk=576, d_lat=512, dtype=1,
             sm=0.07, ptrs=None):
        p = dict(q=P, q_indptr=P, pages=P, page_indptr=P, page_values=P, last=P, out=P, lse=P)
        p.update(ptrs or {})
        return lib.ra_mla_paged_prefill(p["q"], p["q_indptr"], p["pages"], p["page_indptr"],
                                        p["page_values"], p["last"], 1, p["out"], p["lse"], batch,
                                        total_q, num_pages, nnz, page, h_q, d_qk, d_lat, dtype, sm, None)
    assert call(d_qk=192, d_lat=128) == ra.RA_EUNSUPPORTED     # only the 512 + 64 latent shape
    assert call(d_lat=256) == ra.RA_EUNSUPPORTED
    assert call(page=32) == ra.RA_EUNSUPPORTED
    assert call(dtype=5) == ra.RA_EUNSUPPORTED
    assert call(h_q=0) == ra.RA_EINVAL
    assert call(sm=0.0) == ra.RA_EINVAL
    assert call(batch=-1) == ra.RA_EINVAL
    assert call(ptrs={"last": None}) == ra.RA_EINVAL
    assert call(ptrs={"page_values": None}) == ra.RA_EINVAL
    assert call(ptrs={"out": None}) == ra.RA_EINVAL
    assert call(total_q=(1 << 31) // 16, h_q=16) == ra.RA_EUNSUPPORTED
    assert call(batch=0, total_q=0) == ra.RA_OK


@pytest.mark.parametrize("compiler,flags", [("gcc", ["-x", "c", "-std=c99"]), ("g++", ["-x", "c++", "-std=c++17"])])
def test_header_from_c_and_cpp(lib, tmp_path, compiler, flags):
    """include/ragattn.h compiles as C99 and as C++17, a program using it links
    against libragattn.so, and its calls answer as documented."""
    src = os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c")
    exe = str(tmp_path / "abi")
    libdir = os.path.dirname(ra.lib_path())
    cmd = [compiler, *flags, "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src, "-x", "none",
           "-L", libdir, "-lragattn", "-Wl,-rpath," + libdir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    lines = run.stdout.splitlines()
    assert lines[0] == "-1 num_splits must be in [1, 64]"
    assert lines[1].startswith("-2 dtype 7 not supported")   # RA_EUNSUPPORTED
    assert lines[2] == "0 "                                  # RA_OK clears the message
    rows = 16 * 32
    assert int(lines[3]) == (4 * rows * 128 * 4 + 255) // 256 * 256 + 4 * rows * 4

