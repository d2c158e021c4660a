"""Host-side checks of libfrnn that need no GPU: the library loads, exports every entry point
include/frnn.h declares, validates arguments before touching a device, sizes workspaces, and plans
launches. No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import head_wise_lstm_amd as hw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "frnn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hw.lib_path()):
        from head_wise_lstm_amd import build as hb
        hb.build(verbose=False)
    return hw.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|size_t)\s+(frnn_\w+)\s*\(", text, re.M)))


def header_enum(name):
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", open(HEADER).read())
    return int(m.group(1))


def test_exports_every_declared_function(lib):
    funcs = header_functions()
    assert "frnn_fwd" in funcs and "frnn_lstm_stack_fwd" in funcs and len(funcs) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", hw.lib_path()], capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for f in funcs:
        assert f in exported, f"{f} declared in frnn.h but not exported"
        assert hasattr(lib, f)


def test_abi_version_and_status_strings(lib):
    m = re.search(r"#define FRNN_ABI_VERSION (\d+)", open(HEADER).read())
    assert hw.frnn_abi_version() == int(m.group(1))
    for code in ("FRNN_OK", "FRNN_EINVAL", "FRNN_EUNSUPPORTED", "FRNN_EWORKSPACE", "FRNN_ENORESIDENT", "FRNN_EHIP",
                 "FRNN_ETIMEOUT", "FRNN_EPLACEMENT", "FRNN_ENODEVICE", "FRNN_ENOINIT"):
        s = hw.frnn_status_str(header_enum(code))
        assert s and s != "unknown status"
    assert hw.frnn_status_str(12345) == "unknown status"


def D(B=2, T=3, N=1, Dm=64, cell=0, ind=1, outd=0, res=0, **strides):
    d = hw.Desc(B, T, N, Dm, cell, ind, outd, res)
    for k, v in strides.items():
        setattr(d, k, v)
    return d


def ws_bytes(desc, path):
    n = ctypes.c_size_t(0)
    rc = hw.load().frnn_workspace_bytes(ctypes.byref(desc), path, ctypes.byref(n))
    return rc, n.value


EINVAL, EUNSUP, EWS = -1, -2, -3
ENODEVICE, ENOINIT = -8, -9


@pytest.mark.parametrize("desc,code", [
    (D(B=0), EINVAL), (D(N=0), EINVAL), (D(Dm=0), EINVAL), (D(T=-1), EINVAL), (D(cell=3), EINVAL),
    (D(cell=-1), EINVAL),
    (D(ind=7), EINVAL), (D(outd=9), EINVAL), (D(res=1), EINVAL), (D(outd=1), EUNSUP), (D(Dm=48), EUNSUP),
    (D(Dm=2048), EUNSUP),
])
def test_workspace_bytes_validation(lib, desc, code):
    for path in (0, 1):
        assert ws_bytes(desc, path)[0] == code
    assert ws_bytes(D(), 3)[0] == EINVAL


def test_desc_layout_matches_header(lib):
    # 8 int32 fields, then 8 int64 strides: 96 bytes, the strides 8-byte aligned from byte 32
    assert ctypes.sizeof(hw.Desc) == 96 and hw.Desc.wx_sb.offset == 32 and hw.Desc.r_sd.offset == 88
    text = open(HEADER).read()
    body = text[text.index("typedef struct frnn_desc {"):text.index("} frnn_desc;")]
    names = re.findall(r"int(?:32|64)_t\s+(\w+);", body)
    assert names == [f[0] for f in hw.Desc._fields_]


@pytest.mark.parametrize("strides,code", [
    (dict(wx_sb=6), EINVAL), (dict(wx_st=-2), EINVAL), (dict(st_st=3), EINVAL), (dict(st_sb=-4 * 7), 0),
    (dict(wx_st=-4 * 64), 0), (dict(r_sd=-64), EINVAL), (dict(r_sg=-1), EINVAL), (dict(r_sd=65), 0),
    (dict(r_sg=64, r_sd=256, r_sn=0), 0), (dict(wx_sb=1 << 41), EINVAL), (dict(st_ss=4 * 999), 0),
])
def test_desc_stride_validation(lib, strides, code):
    """Wx and states strides may be negative but keep multiples of 4 elements; R strides are
    non-negative element offsets of any value."""
    for path in (0, 1):
        assert ws_bytes(D(**strides), path)[0] == code


def test_workspace_bytes_independent_of_T(lib):
    for path in (0, 1):
        rc1, n1 = ws_bytes(D(B=16, T=1, N=1, Dm=768), path)
        rc2, n2 = ws_bytes(D(B=16, T=100000, N=1, Dm=768), path)
        assert rc1 == rc2 == 0 and n1 == n2 > 256


def test_fwd_rejects_before_any_device_call(lib):
    """Every argument error is returned before the library looks for a device."""
    f = lib.frnn_fwd
    p = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x100002)
    d = D(B=2, T=3, N=1, Dm=64)
    need = ws_bytes(d, 1)[1]
    assert f(None, 1, p, p, None, None, p, p, p, need, None) == EINVAL
    assert f(ctypes.byref(D(B=0)), 1, p, p, None, None, p, p, p, need, None) == EINVAL
    assert f(ctypes.byref(d), 1, None, p, None, None, p, p, p, need, None) == EINVAL   # Wx NULL with T > 0
    assert f(ctypes.byref(d), 1, p, None, None, None, p, p, p, need, None) == EINVAL   # R NULL with T > 0
    assert f(ctypes.byref(d), 1, odd, p, None, None, p, p, p, need, None) == EINVAL    # misaligned
    assert f(ctypes.byref(d), 1, p, p, None, None, p, p, None, need, None) == EWS      # no workspace
    assert f(ctypes.byref(d), 1, p, p, None, None, p, p, p, need - 1, None) == EWS     # too small
    assert f(ctypes.byref(D(Dm=40)), 1, p, p, None, None, p, p, p, need, None) == EUNSUP


def test_stack_validation(lib):
    n = ctypes.c_size_t(0)
    g = lib.frnn_lstm_stack_workspace_bytes
    assert g(2, 1, 512, 32, 512, 512, 1, ctypes.byref(n)) == 0 and n.value > 512 * 32 * 2048 * 4
    one = n.value
    assert g(2, 2, 512, 32, 512, 512, 1, ctypes.byref(n)) == 0 and n.value > 2 * 512 * 32 * 2048 * 4 > one
    assert g(0, 1, 512, 32, 512, 512, 1, ctypes.byref(n)) == EINVAL
    assert g(2, 3, 512, 32, 512, 512, 1, ctypes.byref(n)) == EINVAL   # one or two directions
    assert g(2, 0, 512, 32, 512, 512, 1, ctypes.byref(n)) == EINVAL
    assert g(2, 1, 512, 32, 512, 500, 1, ctypes.byref(n)) == EUNSUP
    assert lib.frnn_lstm_stack_bwd_workspace_bytes(2, 1, 512, 32, 512, 512, 1, ctypes.byref(n)) == 0
    bwd_one = n.value
    assert lib.frnn_lstm_stack_bwd_workspace_bytes(2, 2, 512, 32, 512, 512, 1, ctypes.byref(n)) == 0
    assert n.value > bwd_one   # both directions' projections and states
    assert lib.frnn_lstm_stack_bwd_workspace_bytes(2, 3, 512, 32, 512, 512, 1, ctypes.byref(n)) == EINVAL
    arr = ctypes.c_void_p * 4
    p = ctypes.c_void_p(0x100000)
    ptrs = arr(0x100000, 0x100000, 0x100000, 0x100000)
    f = lib.frnn_lstm_stack_fwd
    assert f(2, 1, 4, 2, 64, 64, 1, p, None, ptrs, None, None, None, None, p, p, p, p, 1 << 30, None) == EINVAL
    assert f(2, 1, 4, 2, 64, 64, 1, p, ptrs, ptrs, None, None, None, None, p, p, p, p, 16, None) == EWS
    assert f(2, 2, 4, 2, 64, 64, 1, p, ptrs, ptrs, None, None, None, None, p, p, p, p, 16, None) == EWS
    odd = arr(0x100000, 0x100000, 0x100000, 0x100004)   # the fourth (layer 1, direction 1) misaligned
    assert f(2, 2, 4, 2, 64, 64, 1, p, ptrs, odd, None, None, None, None, p, p, p, p, 1 << 30, None) == EINVAL


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device answer")
def test_valid_call_without_device_reports_no_device(lib):
    d = D(B=2, T=3, N=1, Dm=64)
    p = ctypes.c_void_p(0x100000)
    need = ws_bytes(d, 1)[1]
    assert lib.frnn_fwd(ctypes.byref(d), 1, p, p, None, None, p, p, p, need, None) == header_enum("FRNN_ENODEVICE")
    assert lib.frnn_init() == header_enum("FRNN_ENODEVICE")


def _function_bodies(src):
    """Top-level function bodies of a C++ source: {name: body text} (brace matching)."""
    out = {}
    for m in re.finditer(r"^[A-Za-z_][\w:<>,\s\*&]*?\b(\w+)\s*\([^;{]*\)\s*(?:const\s*)?\{", src, re.M):
        i, depth = m.end(), 1
        while depth and i < len(src):
            depth += {"{": 1, "}": -1}.get(src[i], 0)
            i += 1
        out.setdefault(m.group(1), "")
        out[m.group(1)] += src[m.end():i]
    return out


def test_compute_entry_points_never_allocate_or_wait():
    """Only frnn_init (through init_device) and frnn_check may allocate, free or wait for the
    device; every other function of the library's sources only enqueues work."""
    csrc = os.path.join(ROOT, "head_wise_lstm_amd", "csrc")
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipDeviceSynchronize|hipStreamSynchronize|"
                        r"hipEventSynchronize|hipMemcpy|hipMemset|hipMallocAsync|hipFuncSetAttribute)\s*\(")
    allowed = {"init_device", "frnn_check", "raise_lds_limits"}
    seen = set()
    for fn in sorted(os.listdir(csrc)):
        if not fn.endswith((".hip", ".hpp")):
            continue
        src = open(os.path.join(csrc, fn)).read()
        src = re.sub(r"//[^\n]*", "", src)
        for name, body in _function_bodies(src).items():
            for m in banned.finditer(body):
                seen.add((name, m.group(1)))
                assert name in allowed, f"{fn}: {name} calls {m.group(1)}"
    assert ("init_device", "hipMalloc") in seen and ("frnn_check", "hipStreamSynchronize") in seen


def plan(desc, path):
    return hw.frnn_plan_str(desc, path)


@pytest.mark.skipif(torch.cuda.is_available(), reason="planner model of a 256-CU, 8-die device (no GPU here)")
def test_planner_choices_for_the_workloads(lib):
    # LSTM D=768 B=16: one head split over the 32 CUs of a die, two batch rows per die
    s = plan(D(B=16, T=1024, N=1, Dm=768), 1)
    assert "die-local" in s and "BR=2 " in s and "groups=8 " in s and "W=32 " in s
    # R^T of a 32-CU slice (147 KB) must stay in registers: a K split over 6 or 8 compute waves
    assert "NCW=8 KS=8 MTW=6 KTW=3" in s and "chunks=1 " in s
    # LSTM D=256 B=8 N=3: four rows per group, six groups of 32 workgroups (one tile each), four
    # compute waves (the step model charges every compute wave at the barrier)
    s = plan(D(B=8, T=1024, N=3, Dm=256), 1)
    assert "die-local" in s and "BR=4 " in s and "groups=6 " in s and "W=32 " in s and "NCW=4 KS=4" in s
    # Elman D=64: a whole head per workgroup, four batch rows each so that 192 workgroups fill the CUs
    s = plan(D(B=64, T=2048, N=12, Dm=64, cell=1), 1)
    assert "workgroup-local" in s and "BR=4 " in s and "groups=192 " in s
    # twelve LSTM heads of 64 units at B=16: a die-local design of four workgroups a head (measured
    # 0.81 us per step against 0.96 for a whole head per workgroup, whose I/O wave streams four
    # gates of Wx); the Elman and GRU heads of that shape keep the single-workgroup design
    s = plan(D(B=16, T=512, N=12, Dm=64), 1)
    assert "design=die-local " in s and "BR=4 " in s and "W=4 " in s
    assert "workgroup-local" in plan(D(B=16, T=512, N=12, Dm=64, cell=1), 1)
    assert "workgroup-local" in plan(D(B=16, T=512, N=12, Dm=64, cell=2), 1)
    # fp32 LSTM D=32
    s = plan(D(B=2, T=16, N=1, Dm=32, ind=0), 1)
    assert "workgroup-local" in s and "dtype=f32" in s
    # fp32 beyond the single-workgroup design is not offered on the fused path
    with pytest.raises(hw.FrnnError):
        plan(D(B=2, T=16, N=1, Dm=512, ind=0), 1)
    s = plan(D(B=2, T=16, N=1, Dm=512, ind=0), 0)
    assert s.startswith("alternating")


@pytest.mark.skipif(torch.cuda.is_available(), reason="planner model of a 256-CU, 8-die device (no GPU here)")
def test_planner_grid_fits_one_workgroup_per_cu(lib):
    for (B, N, Dm, cell) in [(16, 1, 768, 0), (8, 3, 256, 0), (32, 1, 512, 0), (5, 7, 256, 0), (64, 4, 512, 1),
                             (1, 1, 1024, 0), (16, 16, 256, 0)]:
        try:
            s = plan(D(B=B, T=8, N=N, Dm=Dm, cell=cell), 1)
        except hw.FrnnError:
            continue
        if "die-local" in s:
            grid = int(re.search(r"grid=(\d+)", s).group(1))
            slots = int(re.search(r"slots/die=(\d+)", s).group(1))
            assert grid <= 256 and slots <= 32


def test_gru_cell_accepted_and_sized(lib):
    """The GRU (cell 2) packs R^T with four rows per unit like the LSTM (its fourth is zero), so its
    workspace equals the LSTM's on both paths."""
    assert header_enum("FRNN_CELL_GRU") == 2
    for path in (0, 1):
        rc_g, n_g = ws_bytes(D(B=16, T=8, N=2, Dm=256, cell=2), path)
        rc_l, n_l = ws_bytes(D(B=16, T=8, N=2, Dm=256, cell=0), path)
        assert rc_g == rc_l == 0 and n_g == n_l
    s = plan(D(B=4, T=8, N=1, Dm=64, cell=2), 0)
    assert s.startswith("alternating cell=gru")


@pytest.mark.skipif(torch.cuda.is_available(), reason="planner model of a 256-CU, 8-die device (no GPU here)")
def test_planner_gru_matches_lstm_tiles(lib):
    """A GRU head has as many 16-row tiles as an LSTM head of the same width, so it gets the same
    design on these shapes (the predicted time differs: the single-workgroup step model has a base
    per cell)."""
    for (B, N, Dm) in [(16, 1, 768), (8, 3, 256), (2, 1, 32), (64, 12, 64)]:
        for ind in (0, 1):
            try:
                sl = plan(D(B=B, T=8, N=N, Dm=Dm, ind=ind), 1)
            except hw.FrnnError:
                with pytest.raises(hw.FrnnError):
                    plan(D(B=B, T=8, N=N, Dm=Dm, cell=2, ind=ind), 1)
                continue
            sg = plan(D(B=B, T=8, N=N, Dm=Dm, cell=2, ind=ind), 1)
            assert "cell=gru" in sg
            strip = lambda x: re.sub(r" predicted_us=\S+", "", x)
            assert strip(sg.replace("cell=gru", "cell=lstm")) == strip(sl)


def test_bwd_validation_and_workspace(lib):
    """frnn_bwd: validated before any device call; the workspace grows with T; the fused path
    takes fp32 inputs too (a valid call goes on to look for the device, which is absent here)."""
    f = lib.frnn_bwd
    p = ctypes.c_void_p(0x100000)
    d = D(B=2, T=3, N=1, Dm=64)
    n = ctypes.c_size_t(0)
    assert lib.frnn_bwd_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == 0
    need = n.value
    assert lib.frnn_bwd_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(n)) == 0 and n.value > need
    assert lib.frnn_bwd_workspace_bytes(ctypes.byref(D(B=2, T=3, N=1, Dm=64, ind=0)), 1, ctypes.byref(n)) == 0
    assert lib.frnn_bwd_workspace_bytes(ctypes.byref(D(B=2, T=300, N=1, Dm=64)), 0, ctypes.byref(n)) == 0
    assert n.value > need
    args = lambda ws, nb: (p, p, None, None, p, None, None, p, p, p, p, ws, nb, None)
    assert f(ctypes.byref(D(B=2, T=3, N=1, Dm=64, ind=0)), 1, *args(p, 1 << 30)) in (ENODEVICE, ENOINIT)  # fused fp32
    assert f(ctypes.byref(D(B=0)), 0, *args(p, need)) == EINVAL
    assert f(ctypes.byref(d), 0, p, p, None, None, None, None, None, p, p, p, p, p, need, None) == EINVAL  # states NULL
    assert f(ctypes.byref(d), 0, *args(None, need)) == EWS
    assert f(ctypes.byref(d), 0, *args(p, need - 1)) == EWS
    assert f(ctypes.byref(d), 0, ctypes.c_void_p(0x100004), *args(p, need)[1:]) == EINVAL  # misaligned Wx
    s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768), 0)
    assert s.startswith("backward path=alternating cell=lstm") and "hr_gemm=16384x3072x768" in s


@pytest.mark.skipif(torch.cuda.is_available(), reason="planner model of a 256-CU, 8-die device (no GPU here)")
def test_fused_bwd_planner(lib):
    """The fused backward splits a head's rows into 16-unit tiles over the workgroups of one die."""
    # the partial-sum design where it has a plan: 32 workgroups of 24 units each, K = 4 x 24
    s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768), 1)
    assert "design=die-local-partials" in s and "BR=2 " in s and "W=32 " in s and "NCW=8 KS=1 MTW=6 KTW=3" in s
    s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768, cell=2), 1)
    assert "design=die-local-partials" in s and "cell=gru" in s and "W=24 " in s and "KTW=3" in s
    s = hw.frnn_bwd_plan_str(D(B=8, T=1024, N=3, Dm=256), 1)
    assert "design=die-local-partials" in s
    # heads of 1024 units: 32 units a workgroup with part of their R in LDS (LSTM two of four
    # k-tiles, GRU one of three)
    s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=1024), 1)
    assert "design=die-local-partials" in s and "W=32 " in s and "NCW=8 KS=1 MTW=8 KTW=4 KTL=2 " in s, s
    s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=1024, cell=2), 1)
    assert "design=die-local-partials" in s and "W=32 " in s and "NCW=8 KS=1 MTW=8 KTW=3 KTL=1 " in s, s
    assert "KTL" not in hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768), 1)
    # twelve 64-unit Elman heads of 64 rows: the single-workgroup design, four rows a workgroup (a
    # step's records of four 64-unit rows fill one 8 KB ring slot), all 192 groups in one launch
    s = hw.frnn_bwd_plan_str(D(B=64, T=8, N=12, Dm=64, cell=1), 1)
    assert "design=workgroup-local " in s and "BR=4 " in s and "groups=192 " in s and "chunks=1 " in s, s
    # every bf16 head of at most 64 units takes it (on the bf16 MFMA: k-tiles of 32), wider ones
    # the partial sums
    for cell, G in ((0, 4), (2, 3)):
        s = hw.frnn_bwd_plan_str(D(B=16, T=8, N=1, Dm=64, cell=cell), 1)
        assert "design=workgroup-local " in s and f"KTW={G * 64 // 32} " in s, s
        s = hw.frnn_bwd_plan_str(D(B=16, T=8, N=1, Dm=64, cell=cell, ind=0), 1)
        assert "design=workgroup-local " in s and f"KTW={G * 64 // 4} " in s, s  # fp32: k-tiles of 4
        assert "die-local-partials" in hw.frnn_bwd_plan_str(D(B=16, T=8, N=1, Dm=128, cell=cell), 1)
    # the dR GEMM's K (T*B) is padded to whole k-tiles of every part: 64 parts for twelve narrow heads
    s = hw.frnn_bwd_plan_str(D(B=64, T=2048, N=12, Dm=64, cell=1), 0)
    assert "dR_gemm=65x64x131072 " in s, s
    s = hw.frnn_bwd_plan_str(D(B=3, T=5, N=12, Dm=64, cell=1), 0)
    assert "dR_gemm=65x64x256 " in s, s
    # the partial-sum design needs more launches than the da exchange there
    old = os.environ.get("FRNN_FUSED_BWD_PX")
    try:
        os.environ["FRNN_FUSED_BWD_PX"] = "0"
        s = hw.frnn_bwd_plan_str(D(B=64, T=8, N=12, Dm=64, cell=1), 1)
        assert "design=die-local " in s and "chunks=2 " in s
    finally:
        if old is None:
            os.environ.pop("FRNN_FUSED_BWD_PX", None)
        else:
            os.environ["FRNN_FUSED_BWD_PX"] = old
    # the da-exchange design, pinned: head split 24 ways, K = 4 x 768 split over 8 waves
    os.environ["FRNN_FUSED_BWD_PX"] = "0"
    try:
        s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768), 1)
        assert "design=die-local " in s and "BR=2 " in s and "W=24 " in s and "NCW=8 KS=8 MTW=2 KTW=12" in s
        s = hw.frnn_bwd_plan_str(D(B=16, T=1024, N=1, Dm=768, cell=2), 1)
        assert "cell=gru" in s and "W=24 " in s and "KTW=9" in s
    finally:
        del os.environ["FRNN_FUSED_BWD_PX"]
    for (B, N, Dm, cell) in [(16, 1, 768, 0), (8, 3, 256, 0), (5, 2, 64, 0), (9, 2, 256, 2), (7, 2, 128, 1),
                             (16, 1, 1024, 0), (40, 1, 1024, 2)]:
        s = hw.frnn_bwd_plan_str(D(B=B, T=8, N=N, Dm=Dm, cell=cell), 1)
        grid = int(re.search(r"grid=(\d+)", s).group(1))
        slots = int(re.search(r"slots/die=(\d+)", s).group(1))
        lds = int(re.search(r"lds=(\d+)", s).group(1))
        assert grid <= 256 and slots <= 32 and lds <= 160 * 1024, s


@pytest.mark.skipif(torch.cuda.is_available(), reason="planner model of a 256-CU, 8-die device (no GPU here)")
def test_planner_cost_model_and_chunks(lib):
    """The fused planner minimises predicted call time over its constraint set. It splits the head
    over more workgroups when that shortens the per-wave MFMA chain (B=16 D=512: W=32 rather than
    W=16 with one row per group, measured 0.98 vs 1.19 us per step), and runs a batch that cannot
    be co-resident as several launches over chunks of rows."""
    s = plan(D(B=16, T=512, N=1, Dm=512), 1)
    assert "BR=2 " in s and "W=32 " in s and "chunks=1 " in s
    s = plan(D(B=64, T=1024, N=1, Dm=768), 1)
    assert "die-local" in s and "chunks=4 " in s and "rows/chunk=16 " in s
    s = plan(D(B=40, T=8, N=1, Dm=768), 1)
    assert "chunks=3 " in s and "rows/chunk=14 " in s
    # predicted time grows with T and with the number of chunks
    def pred(desc):
        return float(re.search(r"predicted_us=([0-9.]+)", plan(desc, 1)).group(1))
    assert pred(D(B=16, T=2048, N=1, Dm=768)) > pred(D(B=16, T=1024, N=1, Dm=768))
    assert pred(D(B=64, T=1024, N=1, Dm=768)) > 3.5 * pred(D(B=16, T=1024, N=1, Dm=768))


def test_noalloc_entry_refuses_problems_beyond_its_array(lib):
    """frnn_fwd_noalloc's array holds FRNN_NOALLOC_SCRATCH_BYTES; a larger problem is refused with
    FRNN_EWORKSPACE before any device call, a fitting one reaches the device lookup."""
    m = re.search(r"#define FRNN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    cap = int(m.group(1)) << int(m.group(2))
    f = lib.frnn_fwd_noalloc
    p = ctypes.c_void_p(0x100000)
    big = D(B=64, T=8, N=4, Dm=1024)
    assert ws_bytes(big, 1)[1] > cap
    assert f(ctypes.byref(big), 1, p, p, None, None, p, p, None) == EWS
    small = D(B=16, T=8, N=1, Dm=768)  # the headline shape fits
    assert ws_bytes(small, 1)[1] <= cap and ws_bytes(small, 0)[1] <= cap
    assert f(ctypes.byref(D(B=0)), 1, p, p, None, None, p, p, None) == EINVAL
    if not torch.cuda.is_available():
        assert f(ctypes.byref(small), 1, p, p, None, None, p, p, None) == header_enum("FRNN_ENODEVICE")
