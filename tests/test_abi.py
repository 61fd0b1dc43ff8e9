"""Host-side checks of the C ABI: exports, descriptor validation and workspace sizing.
None of these launches a kernel, so they run without a GPU."""

import ctypes
import os
import re

import pytest

import exact_attention_relative_amd as ear

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relpos_attn.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(relpos_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = ear.load_library()
    names = _declared()
    assert set(names) == set(ear.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_declared_symbol():
    """include/relpos_probe.h declares the measurement-only MFMA probe of librelpos_probe.so."""
    src = open(os.path.join(ROOT, "include", "relpos_probe.h")).read()
    names = set(re.findall(r"^\s*\w+\s+(relpos_\w+)\s*\(", src, re.M))
    assert names == {"relpos_probe_mfma_bf16"}
    path = os.path.join(ROOT, "exact_attention_relative_amd", "librelpos_probe.so")
    assert os.path.exists(path), "build the package first"
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert ear.relpos_status_string(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert ear.relpos_status_string(st) != "unknown status"
    assert ear.relpos_status_string(-99) == "unknown status"
    assert ear.relpos_version() >= 100


def _ws(desc, pass_=0):
    out = ctypes.c_size_t(0)
    st = ear.load_library().relpos_attn_workspace_size(ctypes.byref(desc), pass_, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,expected", [
    (dict(mech=7), ear.RELPOS_E_INVALID),
    (dict(dtype=5), ear.RELPOS_E_INVALID),
    (dict(batch=-1), ear.RELPOS_E_INVALID),
    (dict(heads=0), ear.RELPOS_E_INVALID),
    (dict(seqlen=-3), ear.RELPOS_E_INVALID),
    (dict(head_dim=0), ear.RELPOS_E_INVALID),
    (dict(head_dim=128), ear.RELPOS_E_UNSUPPORTED),
    (dict(window=(-2, 0)), ear.RELPOS_E_INVALID),
    (dict(rel_span=0), ear.RELPOS_E_INVALID),
    (dict(scale=-1.0), ear.RELPOS_E_INVALID),
    (dict(scale=float("nan")), ear.RELPOS_E_INVALID),
    (dict(max_partial_bytes=-1), ear.RELPOS_E_INVALID),
])
def test_invalid_descriptors(kw, expected):
    base = dict(mech="shaw", batch=2, heads=4, seqlen=100, head_dim=64, rel_span=8)
    base.update(kw)
    raw_dtype = base.pop("dtype", None)
    mech = base.pop("mech")
    desc = ear.make_desc(mech, base.pop("batch"), base.pop("heads"), base.pop("seqlen"),
                         base.pop("head_dim"), **base)
    if raw_dtype is not None:
        desc.dtype = raw_dtype
    assert _ws(desc)[0] == expected


@pytest.mark.parametrize("nb,md,bidir,ok", [(32, 128, True, True), (31, 128, True, False),
                                            (2, 128, True, False), (32, 8, True, False),
                                            (32, 9, True, True), (8, 5, False, True),
                                            (8, 4, False, False), (512, 4096, True, False)])
def test_t5_descriptor_rules(nb, md, bidir, ok):
    desc = ear.make_desc("t5", 1, 1, 64, num_buckets=nb, max_distance=md, bidirectional=bidir)
    st, _ = _ws(desc)
    assert (st == 0) == ok, st


def test_workspace_sizes_scale_with_shape():
    small = ear.make_desc("txl", 1, 2, 100)
    big = ear.make_desc("txl", 2, 2, 400)
    st1, n1 = _ws(small)
    st2, n2 = _ws(big)
    assert st1 == st2 == 0 and 0 < n1 < n2
    for mech in ("t5", "shaw", "txl", "deberta"):
        d = ear.make_desc(mech, 2, 3, 300, rel_span=5)
        s0, f = _ws(d, 0)
        s1, b = _ws(d, 1)
        assert s0 == s1 == 0 and b >= f > 0
    assert _ws(ear.make_desc("shaw", 1, 1, 10, rel_span=2), 2)[0] == ear.RELPOS_E_INVALID


def test_txl_partial_cap_groups_slices():
    """The T-XL key-side r partials take L^2 / 2 bytes per (batch, head) slice; a cap makes the
    backward process the slices in groups, and the workspace shrinks to one group's partials
    (never below one slice)."""
    def ws(cap):
        return _ws(ear.make_desc("txl", 2, 3, 1000, max_partial_bytes=cap), 1)
    st, full = ws(0)
    nb, rows = (1000 + 127) // 128, 1000 + 256
    per_slice = nb * rows * 64 * 4
    assert st == 0 and full >= 6 * per_slice
    for cap, group in ((per_slice, 1), (2 * per_slice + 5, 2), (4 * per_slice, 4), (1, 1)):
        st, n = ws(cap)
        assert st == 0 and n == full - (6 - group) * per_slice, (cap, group)


def test_t5_offset_partials_shrink_under_two_sided_window():
    """The query-side pass keeps one row of per-offset dS sums per wave (four per 128-row block):
    L + 256 offsets for a full sweep, or, under a two-sided window, only the wave's own sweep
    (wl + wr + 286 offsets, in whole 64-float steps) when that is fewer."""
    B, H, L = 2, 3, 1000
    owners = B * H * ((L + 127) // 128)
    st, full = _ws(ear.make_desc("t5", B, H, L), 1)
    assert st == 0
    for (wl, wr), rows in (((100, 37), 448), ((0, 0), 320), ((600, 600), L + 256),
                           ((2000, 2000), L + 256)):
        st, n = _ws(ear.make_desc("t5", B, H, L, window=(wl, wr)), 1)
        assert st == 0 and full - n == owners * 4 * (L + 256 - rows) * 4, (wl, wr)
    # one-sided windows sweep to the sequence end: no compaction
    for w in ((-1, 0), (50, -1)):
        st, n = _ws(ear.make_desc("t5", B, H, L, window=w, bidirectional=True), 1)
        assert st == 0 and n == full, w


def test_fwd_rejects_bad_pointers_without_launching():
    lib = ear.load_library()
    desc = ear.make_desc("shaw", 1, 1, 64, rel_span=4)
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) & ~255
    # missing q
    st = lib.relpos_attn_fwd(ctypes.byref(desc), None, base, base, base, None, None, None, base,
                             base, base, 1 << 12, None)
    assert st == ear.RELPOS_E_INVALID
    # misaligned k
    st = lib.relpos_attn_fwd(ctypes.byref(desc), base, base + 2, base, base, None, None, None,
                             base, base, base, 1 << 12, None)
    assert st == ear.RELPOS_E_INVALID
    # table slot that Shaw does not use
    st = lib.relpos_attn_fwd(ctypes.byref(desc), base, base, base, base, base, None, None, base,
                             base, base, 1 << 12, None)
    assert st == ear.RELPOS_E_INVALID
    # workspace too small / misaligned
    st = lib.relpos_attn_fwd(ctypes.byref(desc), base, base, base, base, None, None, None, base,
                             base, base, 16, None)
    assert st == ear.RELPOS_E_WORKSPACE
    st = lib.relpos_attn_fwd(ctypes.byref(desc), base, base, base, base, None, None, None, base,
                             base, base + 16, 1 << 12, None)
    assert st == ear.RELPOS_E_WORKSPACE


def test_missing_library_is_an_error(tmp_path):
    with pytest.raises(RuntimeError):
        ear.load_library(str(tmp_path / "nope.so"))


# ------------------------------------------------------------------------ projections
def _proj_ws(desc):
    out = ctypes.c_size_t(0)
    st = ear.load_library().relpos_project_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw", [dict(rows=-1), dict(rows=(1 << 24) + 1), dict(in_features=12),
                                dict(in_features=0), dict(heads=0), dict(head_dim=4),
                                dict(head_dim=12), dict(heads=2048, head_dim=64),
                                dict(dtype=3)])
def test_projection_invalid_descriptors(kw):
    base = dict(rows=100, in_features=64, heads=2, head_dim=64)
    base.update(kw)
    raw_dtype = base.pop("dtype", None)
    desc = ear.make_proj_desc(**base)
    if raw_dtype is not None:
        desc.dtype = raw_dtype
    assert _proj_ws(desc)[0] == ear.RELPOS_E_INVALID


def test_projection_workspace_sizes():
    # dW is split over the basis rows into at most 256 / (128 x 128 tiles) slices of at least 64
    # rows; one slice needs no workspace.  The T-XL basis of L = 8192 (16383 offsets, d_model
    # 512) uses 16 slices of [512, 512] fp32 partials.
    assert _proj_ws(ear.make_proj_desc(64, 64, 1, 64)) == (0, 0)
    assert _proj_ws(ear.make_proj_desc(0, 64, 1, 64)) == (0, 0)
    assert _proj_ws(ear.make_proj_desc(300, 64, 1, 64)) == (0, 5 * 64 * 64 * 4)
    assert _proj_ws(ear.make_proj_desc(16383, 512, 8, 64)) == (0, 16 * 512 * 512 * 4)
    assert _proj_ws(ear.make_proj_desc(1024, 64, 2, 64)) == (0, 16 * 64 * 128 * 4)
    assert _proj_ws(ear.make_proj_desc(100000, 4096, 1, 4096)) == (0, 0)   # 1024 tiles


def test_projection_rejects_bad_pointers_without_launching():
    lib = ear.load_library()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) & ~255
    desc = ear.make_proj_desc(100, 64, 1, 64)
    assert lib.relpos_project_fwd(ctypes.byref(desc), None, base, base, None) == ear.RELPOS_E_INVALID
    assert lib.relpos_project_fwd(ctypes.byref(desc), base, base + 8, base, None) == ear.RELPOS_E_INVALID
    assert lib.relpos_project_bwd(ctypes.byref(desc), base, base, None, base, base, None, 0,
                                  None) == ear.RELPOS_E_INVALID
    assert lib.relpos_project_bwd(ctypes.byref(desc), base, base, base, base + 4, None, None, 0,
                                  None) == ear.RELPOS_E_INVALID
    # nothing requested, or nothing to project: success without a launch
    assert lib.relpos_project_bwd(ctypes.byref(desc), base, base, base, None, None, None, 0,
                                  None) == ear.RELPOS_OK
    empty = ear.make_proj_desc(0, 64, 1, 64)
    assert lib.relpos_project_fwd(ctypes.byref(empty), None, None, None, None) == ear.RELPOS_OK
    # dW of a long basis needs the slice workspace
    big = ear.make_proj_desc(16383, 512, 8, 64)
    assert lib.relpos_project_bwd(ctypes.byref(big), base, base, base, None, base, base, 16,
                                  None) == ear.RELPOS_E_WORKSPACE
