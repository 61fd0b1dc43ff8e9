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


def test_probe_library_exports_its_declared_symbols():
    """include/relpos_probe.h declares the measurement-only MFMA and vector-ALU probes of
    librelpos_probe.so."""
    src = open(os.path.join(ROOT, "include", "relpos_probe.h")).read()
    names = set(re.findall(r"^\s*\w+\s+(relpos_\w+)\s*\(", src, re.M))
    assert names == {"relpos_probe_mfma_bf16", "relpos_probe_valu", "relpos_probe_overlap"}
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


def _al(n):
    return (n + 255) // 256 * 256


def test_t5_bias_gradient_partials_are_bucket_sums():
    """The T5 backward keeps, beyond the forward's tables, D (one float per row) and one row of
    num_buckets sums per 128-row query block: linear in L, the same under any window."""
    B, H, L = 2, 3, 1000
    owners = B * H * ((L + 127) // 128)
    for nbk in (8, 32, 256):
        st, f = _ws(ear.make_desc("t5", B, H, L, num_buckets=nbk), 0)
        assert st == 0
        for window in ((-1, -1), (100, 37), (0, 0), (-1, 0)):
            st, n = _ws(ear.make_desc("t5", B, H, L, num_buckets=nbk, window=window), 1)
            assert st == 0 and n - f == _al(B * H * L * 4) + _al(owners * nbk * 4), (nbk, window)


def test_txl_offset_partials_shrink_under_two_sided_window():
    """The T-XL query-side pass keeps one row of per-offset dS sums per wave (four per 128-row
    block): L + 256 offsets for a full sweep, or, under a two-sided window, only the wave's own
    sweep (wl + wr + 286 offsets, in whole 64-float steps) when that is fewer.  Checked through
    a window that leaves the key-side r partial at full height (wl + wr + 382 >= L + 256)."""
    B, H, L = 2, 3, 1000
    owners = B * H * ((L + 127) // 128)
    st, full = _ws(ear.make_desc("txl", B, H, L), 1)
    assert st == 0
    for (wl, wr), rows in (((450, 450), 1216), ((600, 600), L + 256), ((2000, 2000), L + 256)):
        st, n = _ws(ear.make_desc("txl", B, H, L, window=(wl, wr)), 1)
        assert st == 0 and full - n == _al(owners * 4 * (L + 256) * 4) - _al(owners * 4 * rows * 4), (wl, wr)


def test_general_pass_partials_fold_over_the_batch():
    """Shaw and DeBERTa: once one batch entry already gives a full wave of workgroups (H L / 128
    >= 512), the batch entries of a head share one set of table partials, so the backward
    workspace grows with B only by the per-row buffers (row constants, D, the light pass's fp32
    dX and dV, its end-row sums)."""
    H, L = 8, 8192
    rows = H * L
    for mech, k, per_row in (("shaw", 256, 8 + 4 + 256 + 8 + 256),
                             ("deberta", 512, 8 + 8 + 4 + 256 + 8 + 256)):
        sizes = {}
        for B in (1, 2, 4, 8):
            st, sizes[B] = _ws(ear.make_desc(mech, B, H, L, rel_span=k), 1)
            assert st == 0
        for B in (2, 4, 8):
            assert sizes[B] - sizes[1] == (B - 1) * rows * per_row, (mech, B)


def test_shared_tables_fold_whole_slices():
    """A Shaw / DeBERTa table shared by every head folds whole (batch, head) slices into the
    general passes' partial slots: one 32K batch entry of 8 heads (256 blocks each) keeps two
    groups of four slices (512 slots), where per-head tables keep one slot per (head, block)."""
    B, H, L, k = 1, 8, 32768, 512
    slot = 2 * k * 64 * 4                      # DeBERTa: 2k rows of 64 floats per side
    st, shared = _ws(ear.make_desc("deberta", B, H, L, rel_span=k), 1)
    st2, per_head = _ws(ear.make_desc("deberta", B, H, L, rel_span=k,
                                      rel_head_stride=2 * k * 64), 1)
    assert st == st2 == 0
    assert per_head - shared == 2 * (H * 256 - 512) * slot


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


@pytest.mark.parametrize("mech,stride,expected", [
    ("shaw", 0, ear.RELPOS_OK), ("shaw", 9 * 64, ear.RELPOS_OK), ("shaw", 9 * 64 + 8, ear.RELPOS_OK),
    ("shaw", 9 * 64 - 8, ear.RELPOS_E_INVALID), ("shaw", 9 * 64 + 4, ear.RELPOS_E_INVALID),
    ("shaw", -1, ear.RELPOS_E_INVALID), ("deberta", 8 * 64, ear.RELPOS_OK),
    ("deberta", 8 * 64 - 64, ear.RELPOS_E_INVALID), ("txl", 0, ear.RELPOS_OK),
    ("txl", 199 * 64, ear.RELPOS_OK), ("txl", 198 * 64, ear.RELPOS_E_INVALID),
    ("t5", 12345, ear.RELPOS_OK), ("alibi", 3, ear.RELPOS_OK), ("t5", -5, ear.RELPOS_E_INVALID),
])
def test_rel_head_stride_rules(mech, stride, expected):
    """0 = one table shared by every head; otherwise at least one table apart and a multiple of
    8 elements (16-byte aligned bf16 rows).  T5 and ALiBi ignore it (their tables are per head)."""
    desc = ear.make_desc(mech, 2, 3, 100, rel_span=4, rel_head_stride=stride)
    assert _ws(desc)[0] == expected


def test_default_rel_head_stride_follows_the_workloads():
    assert ear.make_desc("shaw", 1, 2, 50, rel_span=3).rel_head_stride == 0
    assert ear.make_desc("deberta", 1, 2, 50, rel_span=3).rel_head_stride == 0
    assert ear.make_desc("txl", 1, 2, 50).rel_head_stride == 99 * 64
    assert ear.make_desc("txl", 1, 2, 50, window=(-1, 0)).rel_head_stride == 50 * 64


@pytest.mark.parametrize("mech,dtype,kw,ok", [
    # bf16 slice rows: L * 64 * 2 bytes must stay below 2^32
    ("t5", "bf16", dict(seqlen=(1 << 25) - 1), True),
    ("t5", "bf16", dict(seqlen=1 << 25), False),
    ("t5", "fp32", dict(seqlen=(1 << 24) - 1), True),
    ("t5", "fp32", dict(seqlen=1 << 24), False),
    # Shaw table rows 2k + 1
    ("shaw", "bf16", dict(seqlen=64, rel_span=(1 << 24) - 1), True),
    ("shaw", "bf16", dict(seqlen=64, rel_span=1 << 24), False),
    # T-XL full-span table rows 2L - 1
    ("txl", "fp32", dict(seqlen=1 << 23), True),
    ("txl", "fp32", dict(seqlen=(1 << 23) + 1), False),
    ("txl", "bf16", dict(seqlen=(1 << 24) + 1), False),
    # DeBERTa table rows 2k
    ("deberta", "fp32", dict(seqlen=64, rel_span=1 << 23), False),
    ("deberta", "fp32", dict(seqlen=64, rel_span=(1 << 23) - 1), True),
])
def test_32bit_in_slice_offset_limit(mech, dtype, kw, ok):
    """Rows inside one (batch, head) slice or one head's table are addressed with 32-bit byte
    offsets: longer sequences or tables are refused with RELPOS_E_UNSUPPORTED."""
    desc = ear.make_desc(mech, 1, 1, kw.pop("seqlen"), dtype=dtype, **kw)
    st, _ = _ws(desc, 0)
    assert st == (ear.RELPOS_OK if ok else ear.RELPOS_E_UNSUPPORTED), st


def test_profile_hook_calls_from_another_thread():
    """The profiling hook is per host thread: setting or clearing it from another thread is a
    call of its own that succeeds there, and invalid ids fail on every thread."""
    import threading
    lib = ear.load_library()
    assert lib.relpos_profile_events(None, None, 7) == ear.RELPOS_E_INVALID
    res = []
    t = threading.Thread(target=lambda: res.append(lib.relpos_profile_events(None, None, 0)))
    t.start()
    t.join()
    assert res == [ear.RELPOS_OK]


def test_txl_default_partials_fold_the_batch():
    """With no byte cap and at most one wave of workgroups per batch entry (H L / 128 <= 512),
    the key-side pass folds the batch: the batch entries run as consecutive launches into one
    set of r partials, held for the H slices of each of the fewest groups of batch entries that
    still give 512 workgroups (two per compute unit on 256 compute units), or for every slice when
    even all of them give fewer.  Past one wave per batch entry it runs groups of as many slices
    as give 512 workgroups (at least one)."""
    def held(B, H, L):
        st, n = _ws(ear.make_desc("txl", B, H, L), 1)
        st1, n1 = _ws(ear.make_desc("txl", B, H, L, max_partial_bytes=1), 1)   # one slice
        nb = (L + 127) // 128
        per_slice = nb * (L + 256) * 64 * 4
        assert st == st1 == 0
        return (n - n1) // per_slice + 1
    assert held(4, 8, 8192) == 8           # 64 key blocks x 8 heads = 512: one group of 4 entries
    assert held(8, 8, 8192) == 8           # the same set for twice the batch
    assert held(4, 2, 8192) == 8           # 128 workgroups per entry: 4 groups of one entry
    assert held(2, 3, 1000) == 6           # 8 key blocks: every slice, no folding
    assert held(1, 4, 32768) == 2          # 256 key blocks x 4 heads: groups of 2 slices
    assert held(1, 2, 70000) == 1          # 547 key blocks, more than 512 -> one slice
