"""The C ABI on the CPU: the library loads, exports every symbol aa.h declares,
and rejects bad arguments on the host before any launch.  No compute call is
made (this machine may have no GPU), so every call here must fail validation
or be a plan call, which touches no HIP API."""
import ctypes
import os
import re

import pytest

import associative_algebra_block_amd as aa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(aa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(aa.lib_path()):
        pytest.fail("libaa.so is not built (python -m associative_algebra_block_amd.build)")
    return aa.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(aa.EXPORTED) == declared


def test_only_aa_symbols_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", aa.lib_path()], capture_output=True, text=True).stdout
    funcs = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert funcs and all(f.startswith("aa_") for f in funcs), funcs


@pytest.mark.parametrize("law,q,n", [("Qq", 1, 1), ("Qq", 2, 6), ("Qq", 3, 15), ("Qq", 16, 496),
                                     ("Qq", 32, 2016), ("Qq", 256, 130816), ("Q2xQ2", 4, 36)])
def test_plan_counts(lib, law, q, n):
    p = aa.aa_plan_create(law, q, 16 * q, 32 * q)
    nb, nl, pe = aa.aa_plan_info(p)
    assert nb == n
    assert nl == q * q
    assert pe == 16 * q * 32 * q
    aa.aa_plan_destroy(p)


def test_packed_layout_version(lib):
    for law, q in [("Qq", 32), ("Q2xQ2", 4), ("Qq", 1)]:
        assert aa.aa_packed_layout_version(aa.aa_plan_create(law, q, 16 * q, 32 * q)) == 1
    assert aa.aa_packed_layout_version(aa.aa_plan_create_digraph(3, [(0, 1)], 48, 48)) == 1
    assert _raw(lib, "aa_packed_layout_version", None, None) == aa.AA_ERR_INVALID_ARG
    # the Qwen3-32B FFN widths at q = 256: 20 x 100 blocks, layout 2
    p = aa.aa_plan_create("Qq", 256, 5120, 25600)
    assert aa.aa_packed_layout_version(p) == 2
    assert aa.aa_plan_info(p) == (2 * 256 * 256 - 256, 256 * 256, 5120 * 25600)
    assert aa.aa_packed_layout_version(aa.aa_plan_create_digraph(3, [(0, 1)], 36, 60)) == 2


def test_layout2_limits_before_launch(lib):
    """Layout-2 plans: no gradients, no per-token decode types; both refused
    on the host."""
    p = aa.aa_plan_create("Qq", 4, 80, 48, "pos_mod", 0, "bf16", "f32")
    g = 0x1000000
    assert aa.aa_project_bwd_workspace(p, 100) == (0, 0)
    assert _raw(lib, "aa_project_bwd_data", p.handle, g, 2 * g, 3 * g, 100, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    assert _raw(lib, "aa_project_bwd_weight", p.handle, g, 2 * g, 3 * g, 100, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    assert _raw(lib, "aa_decode_gemv", p.handle, g, 2 * g, 3 * g, 2, 0, 4 * g, None) == aa.AA_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    (("Qq", 0, 64, 64), aa.AA_ERR_INVALID_ARG),
    (("Q2xQ2", 2, 64, 64), aa.AA_ERR_INVALID_ARG),
    (("Qq", 3, 64, 96), aa.AA_ERR_SHAPE),          # 3 does not divide 64
    (("Qq", 2, 36, 64), aa.AA_ERR_UNSUPPORTED),    # b_in = 18 is not a multiple of 4
    (("Q2xQ2", 4, 96, 64), aa.AA_ERR_UNSUPPORTED),  # 24 x 16 blocks: layout 2 takes Q_q and digraphs
    (("Qq", 2, 48, 64, "explicit"), aa.AA_ERR_UNSUPPORTED),   # layout 2 without explicit types
    (("Qq", 2, 48, 64, "pos_mod", 0, "f32", "f32"), aa.AA_ERR_UNSUPPORTED),   # layout 2 takes bf16
    (("Qq", 2, 264, 64), aa.AA_ERR_UNSUPPORTED),   # b_in = 132: layout 2 stops at 128
    (("Qq", 4, 64, 64, "pos_mod", 6), aa.AA_ERR_UNSUPPORTED),  # period not a multiple of q
    (("Qq", 4, 64, 64, "pos_mod", -4), aa.AA_ERR_INVALID_ARG),
    (("Qq", 2, -64, 64), aa.AA_ERR_INVALID_ARG),
])
def test_plan_rejects(lib, args, status):
    with pytest.raises(aa.AAError) as e:
        aa.aa_plan_create(*args)
    assert e.value.status == status
    assert aa.aa_last_error()


def test_digraph_plans(lib):
    """aa_plan_create_digraph: q + 2 |E| block products, the diagonal of the
    adjacency ignored, argument checks; no gradients."""
    p = aa.aa_plan_create_digraph(5, [(0, 1), (1, 2), (2, 0), (4, 3), (3, 3)], 80, 160)
    assert aa.aa_plan_info(p) == (5 + 2 * 4, 25, 80 * 160)
    full = aa.aa_plan_create_digraph(6, [(i, k) for i in range(6) for k in range(6)], 96, 96)
    assert aa.aa_plan_info(full)[0] == 2 * 36 - 6                 # the complete graph is Q_6
    assert aa.aa_plan_info(aa.aa_plan_create_digraph(4, [], 64, 64))[0] == 4
    adj = (ctypes.c_uint8 * 4)(0, 1, 0, 0)
    out = ctypes.c_void_p()
    assert lib.aa_plan_create_digraph(ctypes.byref(out), 2, None, 64, 64, 0, 0, 0, 0) == aa.AA_ERR_INVALID_ARG
    assert lib.aa_plan_create_digraph(None, 2, ctypes.cast(adj, ctypes.c_char_p), 64, 64, 0, 0, 0, 0) == \
        aa.AA_ERR_INVALID_ARG
    assert lib.aa_plan_create_digraph(ctypes.byref(out), 65, ctypes.cast(adj, ctypes.c_char_p), 65 * 16, 65 * 16,
                                      0, 0, 0, 0) == aa.AA_ERR_UNSUPPORTED
    assert lib.aa_plan_create_digraph(ctypes.byref(out), 2, ctypes.cast(adj, ctypes.c_char_p), 36, 64,
                                      0, 0, 0, 0) == aa.AA_ERR_UNSUPPORTED   # b_in = 18
    with pytest.raises(aa.AAError) as e:
        aa.aa_plan_create("digraph", 2, 64, 64)
    assert e.value.status == aa.AA_ERR_INVALID_ARG
    assert aa.aa_project_bwd_workspace(p, 100) == (0, 0)
    g = 0x1000000
    assert _raw(lib, "aa_project_bwd_data", p.handle, g, 2 * g, 3 * g, 100, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    assert _raw(lib, "aa_project_bwd_weight", p.handle, g, 2 * g, 3 * g, 100, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED


def test_plan_create_null_out(lib):
    assert lib.aa_plan_create(None, 0, 2, 64, 64, 0, 0, 0, 0) == aa.AA_ERR_INVALID_ARG


def test_status_strings(lib):
    assert aa.aa_status_string(aa.AA_OK) == "AA_OK"
    assert aa.aa_status_string(aa.AA_ERR_HIP) == "AA_ERR_HIP"
    assert aa.aa_status_string(99) == "AA_ERR_UNKNOWN"


def _raw(lib, name, *args):
    return getattr(lib, name)(*args)


def test_compute_calls_validate_before_launch(lib):
    p = aa.aa_plan_create("Qq", 2, 64, 64)
    h = p.handle
    good = 0x10000
    # NULL and misaligned pointers
    assert _raw(lib, "aa_project_fwd", h, None, good, good * 4, 8, 0, None, None) == aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_fwd", h, good + 2, good * 8, good * 16, 8, 0, None, None) == aa.AA_ERR_INVALID_ARG
    # negative M and offset
    assert _raw(lib, "aa_project_fwd", h, good, good * 8, good * 16, -1, 0, None, None) == aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_fwd", h, good, good * 8, good * 16, 8, -3, None, None) == aa.AA_ERR_INVALID_ARG
    # row types given to a position-typed plan
    assert _raw(lib, "aa_project_fwd", h, good, good * 8, good * 16, 8, 0, good * 32, None) == aa.AA_ERR_INVALID_ARG
    # Y overlapping X
    assert _raw(lib, "aa_project_fwd", h, good, good * 8, good + 64, 8, 0, None, None) == aa.AA_ERR_INVALID_ARG
    # M == 0 is a no-op that succeeds without touching the GPU
    assert _raw(lib, "aa_project_fwd", h, None, None, None, 0, 0, None, None) == aa.AA_OK
    # pack with overlapping buffers
    assert _raw(lib, "aa_pack_weights", h, good, good + 16, None) == aa.AA_ERR_INVALID_ARG
    # decode: NULL x
    assert _raw(lib, "aa_decode_gemv", h, None, good, good * 8, 1, 0, None, None) == aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_decode_gemv", h, good, good * 8, good * 16, -1, 0, None, None) == aa.AA_ERR_INVALID_ARG
    aa.aa_plan_destroy(p)


def test_block_rows_needs_divisible_M(lib):
    p = aa.aa_plan_create("Qq", 4, 64, 64, "block_rows")
    good = 0x10000
    assert _raw(lib, "aa_project_fwd", p.handle, good, good * 8, good * 16, 10, 0, None, None) == aa.AA_ERR_SHAPE
    # decode on a block-row plan needs explicit types
    assert _raw(lib, "aa_decode_gemv", p.handle, good, good * 8, good * 16, 1, 0, None, None) == aa.AA_ERR_INVALID_ARG


def test_explicit_needs_types(lib):
    p = aa.aa_plan_create("Qq", 4, 64, 64, "explicit")
    good = 0x10000
    assert _raw(lib, "aa_project_fwd", p.handle, good, good * 8, good * 16, 8, 0, None, None) == aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_fwd", p.handle, good, good * 8, good * 16, 8, 0, good * 32 + 2, None) == \
        aa.AA_ERR_INVALID_ARG


def test_swiglu_plan_mismatch(lib):
    up = aa.aa_plan_create("Qq", 4, 64, 128)
    down_q = aa.aa_plan_create("Qq", 2, 128, 64)
    down_law = aa.aa_plan_create("Q2xQ2", 4, 128, 64)
    down_shape = aa.aa_plan_create("Qq", 4, 128, 128)
    down_dtype = aa.aa_plan_create("Qq", 4, 128, 64, "pos_mod", 0, "f32", "f32")
    down_kind = aa.aa_plan_create("Qq", 4, 128, 64, "block_rows")
    g = 0x100000
    for d, st in [(down_q, aa.AA_ERR_SHAPE), (down_law, aa.AA_ERR_SHAPE), (down_shape, aa.AA_ERR_SHAPE),
                  (down_dtype, aa.AA_ERR_SHAPE), (down_kind, aa.AA_ERR_SHAPE)]:
        r = _raw(lib, "aa_swiglu_ffn_fwd", up.handle, d.handle, g, 2 * g, 3 * g, 4 * g, 5 * g, 6 * g, 8, 0, None, None)
        assert r == st, aa.aa_last_error()


def test_noalloc_swiglu_validates_before_launch(lib):
    """The allocation-free SwiGLU call checks like the other one and refuses a
    hidden activation larger than its static scratch, all before any HIP call."""
    up = aa.aa_plan_create("Qq", 4, 1024, 4096)
    down = aa.aa_plan_create("Qq", 4, 4096, 1024, "pos_mod", 0, "bf16", "f32")
    bad_down = aa.aa_plan_create("Qq", 2, 4096, 1024)
    g = 0x100000
    fn = "aa_swiglu_ffn_fwd_noalloc"
    assert _raw(lib, fn, up.handle, bad_down.handle, g, 2 * g, 3 * g, 4 * g, 6 * g, 8, 0, None, None) == \
        aa.AA_ERR_SHAPE
    assert _raw(lib, fn, up.handle, down.handle, None, 2 * g, 3 * g, 4 * g, 6 * g, 8, 0, None, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, fn, up.handle, down.handle, g, 2 * g, 3 * g, 4 * g, 6 * g, 0, 0, None, None) == aa.AA_OK
    too_many = aa.AA_NOALLOC_SCRATCH_BYTES // (2 * 4096) + 1
    assert _raw(lib, fn, up.handle, down.handle, g, 2 * g, 3 * g, 4 * g, 1 << 40, too_many, 0, None, None) == \
        aa.AA_ERR_UNSUPPORTED
    assert "scratch" in aa.aa_last_error()


def test_gradients_validate_before_launch(lib):
    import ctypes
    g = 0x1000000
    p = aa.aa_plan_create("Qq", 8, 1024, 1536)          # b_in 128, b_out 192
    h = p.handle
    nd, nw = ctypes.c_size_t(7), ctypes.c_size_t(7)
    assert lib.aa_project_bwd_workspace(h, 100, ctypes.byref(nd), ctypes.byref(nw)) == aa.AA_OK
    assert nd.value > 0 and nd.value % (100 * 128 * 4) == 0   # q = 8: the own-group leaf is split
    assert nw.value % (8 * 128 * 192 * 4) == 0           # whole partial diagonal blocks, if any
    assert lib.aa_project_bwd_workspace(h, 100, None, None) == aa.AA_OK
    assert aa.aa_project_bwd_workspace(aa.aa_plan_create("Qq", 2, 256, 256), 100)[0] == 0
    assert aa.aa_project_bwd_workspace(aa.aa_plan_create("Q2xQ2", 4, 256, 256), 100) == (0, 0)
    assert lib.aa_project_bwd_workspace(None, 100, None, None) == aa.AA_ERR_INVALID_ARG
    assert lib.aa_project_bwd_workspace(h, -1, None, None) == aa.AA_ERR_INVALID_ARG
    ws = nd.value
    # NULL operands, negative M or offset, a short or missing workspace, overlaps
    assert _raw(lib, "aa_project_bwd_data", h, None, 2 * g, 3 * g, 100, 0, None, 4 * g, ws, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, 3 * g, -1, 0, None, 4 * g, ws, None) == aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, 3 * g, 100, -2, None, 4 * g, ws, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, 3 * g, 100, 0, None, 4 * g, ws - 4, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, 3 * g, 100, 0, None, None, ws, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, g + 64, 100, 0, None, 4 * g, ws, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, g, 2 * g, 3 * g, 100, 0, None, 3 * g + 64, ws, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_data", h, None, None, None, 0, 0, None, None, 0, None) == aa.AA_OK
    wsw = max(nw.value, 16)
    assert _raw(lib, "aa_project_bwd_weight", h, None, 2 * g, 3 * g, 100, 0, None, 4 * g, wsw, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_weight", h, g, 2 * g, g + 64, 100, 0, None, 4 * g, wsw, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_weight", h, g, 2 * g, 3 * g, 100, 0, 4 * g, 5 * g, wsw, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_weight", h, None, None, None, 0, 0, None, None, 0, None) == aa.AA_OK
    # a plan whose weight gradient splits the types needs its workspace
    sp = aa.aa_plan_create("Qq", 16, 2048, 768)
    nws = aa.aa_project_bwd_workspace(sp, 2048)[1]
    assert nws > 0
    G = 0x100000000
    assert _raw(lib, "aa_project_bwd_weight", sp.handle, G, 2 * G, 3 * G, 2048, 0, None, 4 * G, nws - 16, None) == \
        aa.AA_ERR_INVALID_ARG
    assert _raw(lib, "aa_project_bwd_weight", sp.handle, G, 2 * G, 3 * G, 2048, 0, None, None, nws, None) == \
        aa.AA_ERR_INVALID_ARG
    # unsupported: fp32 operands, explicit type lists, blocks too wide
    f32 = aa.aa_plan_create("Qq", 4, 256, 256, "pos_mod", 0, "f32", "f32")
    assert _raw(lib, "aa_project_bwd_weight", f32.handle, g, 2 * g, 3 * g, 8, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    ex = aa.aa_plan_create("Qq", 4, 256, 256, "explicit")
    assert _raw(lib, "aa_project_bwd_weight", ex.handle, g, 2 * g, 3 * g, 8, 0, 4 * g, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    assert _raw(lib, "aa_project_bwd_data", ex.handle, g, 2 * g, 3 * g, 8, 0, 4 * g, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    wide = aa.aa_plan_create("Qq", 2, 1024, 64)          # b_in 512
    assert _raw(lib, "aa_project_bwd_weight", wide.handle, g, 2 * g, 3 * g, 8, 0, None, None, 0, None) == \
        aa.AA_ERR_UNSUPPORTED
    # block-row typing still needs q | M
    br = aa.aa_plan_create("Qq", 4, 256, 256, "block_rows")
    assert _raw(lib, "aa_project_bwd_weight", br.handle, g, 2 * g, 3 * g, 10, 0, None, None, 0, None) == \
        aa.AA_ERR_SHAPE


def test_last_error_is_thread_local(lib):
    import threading
    with pytest.raises(aa.AAError):
        aa.aa_plan_create("Qq", 0, 64, 64)
    mine = aa.aa_last_error()
    seen = []
    t = threading.Thread(target=lambda: seen.append(aa.aa_last_error()))
    t.start()
    t.join()
    assert mine and seen == [""]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libaa.so every entry point raises: there is no fallback path."""
    monkeypatch.setattr(aa, "_LIB", None)
    monkeypatch.setattr(aa, "lib_path", lambda: str(tmp_path / "libaa.so"))
    with pytest.raises(RuntimeError, match="is not built"):
        aa.load()
    with pytest.raises(RuntimeError, match="is not built"):
        aa.aa_plan_create("Qq", 4, 64, 64)
