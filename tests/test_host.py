"""Host-side tests of the C ABI (no GPU needed, no kernel launched).

The library loads and exports every function include/norm_bwd.h declares; the
planner's rules hold; every invalid argument is rejected with the documented
status before anything touches the HIP runtime (fake device pointers are
never dereferenced on these paths).
"""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "norm_bwd.h")


@pytest.fixture(scope="module")
def nb():
    import rmsnorm_backward_amd as nbmod
    if not os.path.exists(nbmod.LIB_PATH):
        from rmsnorm_backward_amd import _build
        _build.build()
    nbmod.load_library()
    return nbmod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(norm_(?:bwd|fwd)_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for want in ("norm_bwd_layernorm", "norm_bwd_rmsnorm", "norm_bwd_workspace_bytes",
                 "norm_bwd_make_plan", "norm_bwd_execute", "norm_bwd_execute_partials",
                 "norm_bwd_reduce_partials", "norm_bwd_status_string", "norm_bwd_last_error",
                 "norm_bwd_probe_copy", "norm_fwd_layernorm", "norm_fwd_rmsnorm", "norm_bwd_ex",
                 "norm_bwd_wgrad", "norm_bwd_probe_triad", "norm_bwd_probe_triad_policy"):
        assert want in names


def test_library_exports_every_declared_symbol(nb):
    lib = ctypes.CDLL(nb.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_plan_struct_layout_matches_header(nb):
    # norm_bwd_plan_t: 4 int32, 4 int64, 7 int32, size_t -> 88 bytes
    assert ctypes.sizeof(nb.NormBwdPlan) == 88
    assert nb.NormBwdPlan.rows_per_wave.offset == 72
    assert nb.NormBwdPlan.workspace_bytes.offset == 80
    assert nb.NormBwdPlan.chunks.offset == 48


def _c_layout(struct, fields, tmp_path):
    """sizeof and field offsets of `struct` as the C compiler lays it out."""
    import subprocess
    src = tmp_path / "layout.c"
    body = "".join(f'  printf("{f} %zu\\n", offsetof({struct}, {f}));\n' for f in fields)
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"norm_bwd.h\"\n"
                   "int main(void) {\n"
                   f'  printf("sizeof %zu\\n", sizeof({struct}));\n{body}  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {k: int(v) for k, v in (line.split() for line in out.splitlines())}


@pytest.mark.parametrize("struct,pyname", [("norm_bwd_plan_t", "NormBwdPlan"),
                                           ("norm_bwd_args_t", "NormBwdArgs")])
def test_struct_layouts_match_the_c_compiler(nb, struct, pyname, tmp_path):
    cls = getattr(nb, pyname)
    names = [f for f, _ in cls._fields_]
    c = _c_layout(struct, names, tmp_path)
    assert c["sizeof"] == ctypes.sizeof(cls)
    for f in names:
        assert c[f] == getattr(cls, f).offset, f


def test_status_strings(nb):
    assert nb.norm_bwd_status_string(0) == "NORM_BWD_OK"
    assert nb.norm_bwd_status_string(1) == "NORM_BWD_ERR_INVALID_ARG"
    assert nb.norm_bwd_status_string(2) == "NORM_BWD_ERR_UNSUPPORTED"
    assert nb.norm_bwd_status_string(3) == "NORM_BWD_ERR_WORKSPACE"
    assert nb.norm_bwd_status_string(4) == "NORM_BWD_ERR_HIP"
    assert nb.norm_bwd_status_string(99) == "NORM_BWD_ERR_UNKNOWN"


def _row_stats_rows(p, db):
    """Rows in flight of the kernels that compute row statistics (forward,
    recompute mode) on plan p's lane layout: as many as fill 512 threads,
    within the launch bound; one when the combine buffer would not fit."""
    S, C, vec = p.waves_per_row, p.chunks, p.vec
    P = max(1, 512 // (64 * S))
    while P > 1 and S * P * 64 > (512 if vec * C > 16 else 1024):
        P //= 2
    if P > 1 and S * C * 64 * vec * 4 > 65536 - 1024:    # one combine plane
        P = 1
    return P


def _auto_groups(nb, kind, M, N, dt, recompute=False):
    """The documented rule: 256 groups, except in LayerNorm recompute mode:
    about 4096 waves in flight, the waves per workgroup coming from the
    (dbeta-less) lane layout with 512-thread workgroups (rows on the
    two-rows-per-wave layout, which has no barrier per row, keep 256);
    always >= 4 rows per group, above 256 a multiple of 256."""
    if M == 0:
        return 0
    p = nb.norm_bwd_make_plan(kind, 1, N, dt, False) if N else None
    if recompute and kind == "layernorm" and not (p and p.rows_per_wave == 2):
        waves = 8
        if N:
            waves = p.waves_per_row * _row_stats_rows(p, False)
        g = 4096 // waves
    else:
        g = 256
    g = min(g, -(-M // 4))
    if g > 256:
        g -= g % 256
    return max(1, g)


@pytest.mark.parametrize("kind,M,N,dt,db", [
    ("layernorm", 128, 512, torch.float32, True),
    ("rmsnorm", 128, 512, torch.float32, False),
    ("layernorm", 1151, 8192, torch.float16, True),
    ("layernorm", 2000, 2048, torch.bfloat16, True),
    ("rmsnorm", 3000, 1024, torch.bfloat16, False),
    ("rmsnorm", 16384, 4096, torch.bfloat16, False),
    ("layernorm", 65536, 8192, torch.bfloat16, True),
    ("rmsnorm", 262144, 768, torch.bfloat16, False),
    ("layernorm", 262144, 768, torch.bfloat16, True),     # two rows per wave
    ("layernorm", 5000, 384, torch.float32, True),
    ("rmsnorm", 0, 768, torch.bfloat16, True),
    ("layernorm", 5, 0, torch.float16, True),
])
def test_workspace_bytes_rule(nb, kind, M, N, dt, db):
    got = nb.norm_bwd_workspace_bytes(kind, M, N, dt, db)
    groups = max(_auto_groups(nb, kind, M, N, dt), _auto_groups(nb, kind, M, N, dt, True))
    # the wide-row path's recompute statistics (4 or 8 bytes per row) also fit
    wide = M * 4 * (2 if kind == "layernorm" else 1)
    assert got == max((2 if db else 1) * groups * N * 4, wide)
    plan = nb.norm_bwd_make_plan(kind, M, N, dt, db)   # the saved-statistics plan
    assert plan.workspace_bytes <= got
    assert plan.workspace_bytes == (2 if db else 1) * _auto_groups(nb, kind, M, N, dt) * N * 4


def test_workspace_bytes_rejects_bad_arguments(nb):
    lib = nb.load_library()
    bad = ctypes.c_size_t(-1).value
    assert lib.norm_bwd_workspace_bytes(7, 10, 10, 0, 0) == bad
    assert lib.norm_bwd_workspace_bytes(0, 10, 10, 9, 0) == bad
    assert lib.norm_bwd_workspace_bytes(0, -1, 10, 0, 0) == bad
    assert lib.norm_bwd_workspace_bytes(0, 10, 1 << 31, 2, 0) == bad
    # M * N beyond what the entry points accept (and M * 8 would wrap)
    assert lib.norm_bwd_workspace_bytes(0, 1 << 62, 1, 0, 0) == bad
    assert lib.norm_bwd_workspace_bytes(1, 1 << 40, 1 << 21, 2, 0) == bad
    # rows wider than the fused path: the wide-row path's statistics only
    assert lib.norm_bwd_workspace_bytes(0, 10, 40000, 2, 1) == 10 * 8
    assert lib.norm_bwd_workspace_bytes(1, 10, 40000, 2, 0) == 10 * 4


GEOMS = [(kind, dt, M, N, db, g)
         for kind in ("layernorm", "rmsnorm")
         for dt in (torch.float32, torch.float16, torch.bfloat16)
         for (M, N) in ((1, 1), (3, 7), (17, 63), (64, 64), (65, 65), (1151, 8192),
                        (2, 768), (100, 4096), (7, 16384), (9, 1000), (300, 256),
                        (1000, 384), (33, 128), (5000, 768), (65536, 8192), (131072, 4096))
         for db in (False, True)
         for g in (0, 1, 5)]


@pytest.mark.parametrize("kind,dt,M,N,db,groups", GEOMS)
def test_plan_invariants(nb, kind, dt, M, N, db, groups):
    eb = torch.tensor([], dtype=dt).element_size()
    if N > (16384 if eb == 4 or db else 32768):
        return
    p = nb.norm_bwd_make_plan(kind, M, N, dt, db, groups)
    S, P, C, vec = p.waves_per_row, p.rows_in_flight, p.chunks, p.vec
    assert vec in (1, 16 // eb) and (vec == 1 or N % vec == 0)
    nacc = 2 if db else 1
    vw = 16 // eb
    # rows that 64-lane waves would cover with idle lanes and 32 lanes cover
    # exactly (N = 32 * vw * 1 or 3) take two rows per wave, with 8 KiB
    # (RMSNorm) or 16 KiB (LayerNorm) of x and dy in flight
    c2 = next((c for c in (1, 3) if N == c * 32 * vw), 0) if N % (64 * vw) else 0
    if c2:
        assert p.rows_per_wave == 2 and vec == vw and S == 1 and C == c2
        want = 2
        while want * 32 < 512 and want * 2 * N * eb < (16384 if kind == "layernorm" else 8192):
            want *= 2
        assert P == want and p.threads == 32 * P
        assert p.lds_bytes == (nacc * C * 32 * vec * 4 if P > 2 else 0)
        # groups of adjacent row pairs: never an empty one
        pairs = -(-M // 2)
        assert 1 <= p.groups <= pairs and p.rows_per_group == 2 * -(-pairs // p.groups)
        if groups:
            assert p.groups == min(groups, pairs)
        assert p.workspace_bytes == nacc * p.groups * N * 4
        return
    assert p.rows_per_wave == 1
    # rows in flight: the fewest (a power of two) whose x and dy reach 16 KiB,
    # within 16 waves and the kernel's launch bound; one when the combine
    # buffer (one plane of per-lane partials) would not fit; two when a group
    # sweeps more than 2 MiB of each operand (kernel A's general loop) and
    # the same limits allow it
    max_thr = 512 if vec * C > 16 else 1024
    plane = S * C * 64 * vec * 4
    # RMSNorm rows laid out on 16-byte lanes with an odd wave count (no
    # exact 32-byte layout exists) aim at 12 KiB of x and dy in flight
    exact16 = (kind == "rmsnorm" and C == 1 and vec == vw and S * 64 * vec == N
               and S % 2 == 1 and S > 1)
    want = 1
    while want < 16 and want * 2 * N * eb < (12288 if exact16 else 16384):
        want *= 2
    while want > 1 and (S * want > 16 or S * want * 64 > max_thr):
        want //= 2
    if want > 1 and plane > 65536 - 1024:
        want = 1
    if (want == 1 and -(-M // p.groups) * N * eb > 2 << 20 and 2 * S <= 16
            and 2 * S * 64 <= max_thr and plane <= 65536 - 1024):
        want = 2
    assert P == want
    assert S * 64 * vec * C >= N                       # the lanes cover the row
    assert p.threads == 64 * S * P and 1 <= S * P <= 16
    assert C in (1, 2, 4, 8)
    assert 1 <= p.groups <= M                          # no empty group
    assert p.rows_per_group == -(-M // p.groups)       # largest group
    if groups:
        assert p.groups == min(groups, M)
    else:
        assert p.groups == _auto_groups(nb, kind, M, N, dt)
    assert 1 <= p.grid <= p.groups
    nacc = 2 if db else 1
    assert p.workspace_bytes == nacc * p.groups * N * 4
    assert p.lds_bytes == (S * C * 64 * vec * 4 if P > 1 else 0)
    assert p.lds_bytes <= 65536


def test_two_row_plans_group_row_pairs(nb):
    """Two-row plans group adjacent row pairs: groups are clamped to the pair
    count, rows_per_group counts whole pairs, any group count keeps the layout
    (a pair spans one row stride), and an edited plan that breaks these rules
    is refused."""
    p = nb.norm_bwd_make_plan("rmsnorm", 1 << 23, 768, torch.bfloat16, False, 3 << 20)
    assert p.rows_per_wave == 2 and p.groups == 3 << 20
    p = nb.norm_bwd_make_plan("rmsnorm", 7, 768, torch.bfloat16, False, 100)
    assert p.rows_per_wave == 2 and p.groups == 4 and p.rows_per_group == 2
    p = nb.norm_bwd_make_plan("rmsnorm", 1001, 768, torch.bfloat16, False, 10)
    assert p.rows_per_group == 2 * 51
    lib = nb.load_library()
    for field, value in (("groups", 5), ("rows_per_group", 1)):
        q = nb.norm_bwd_make_plan("rmsnorm", 7, 768, torch.bfloat16, False, 100)
        setattr(q, field, value)
        if field == "groups":
            q.workspace_bytes = 5 * 768 * 4
        st = lib.norm_bwd_execute(ctypes.byref(q), _addr(0), _addr(1), _addr(2), None,
                                  _addr(3), 0, _addr(4), _addr(5), None, _addr(6),
                                  q.workspace_bytes, None)
        assert st == 1, field


def test_general_loop_groups_take_two_rows(nb):
    """Groups sweeping more than 2 MiB of each operand (kernel A's general
    loop) get two rows in flight; groups within it keep one. The planner and
    the kernel hold the 2 MiB bound separately and must agree."""
    csrc = os.path.join(ROOT, "rmsnorm_backward_amd", "csrc")
    pat = re.compile(r"constexpr int64_t kSteadyGroupBytes = \(int64_t\)(\d+) << (\d+);")
    vals = [pat.findall(open(os.path.join(csrc, f)).read()) for f in ("plan.cpp", "nb_device.hpp")]
    assert len(vals[0]) == 1 and vals[0] == vals[1], vals
    bf = torch.bfloat16
    p = nb.norm_bwd_make_plan("rmsnorm", 16384, 4096, bf, False)      # 512 KiB per group
    assert (p.rows_in_flight, p.threads, p.lds_bytes) == (1, 256, 0)
    p = nb.norm_bwd_make_plan("layernorm", 65536, 8192, bf, True)     # 4 MiB per group
    assert (p.waves_per_row, p.rows_in_flight, p.threads, p.lds_bytes) == (8, 2, 1024, 32768)
    p = nb.norm_bwd_make_plan("rmsnorm", 131072, 4096, bf, False)
    assert (p.waves_per_row, p.rows_in_flight, p.threads, p.lds_bytes) == (4, 2, 512, 16384)
    p = nb.norm_bwd_make_plan("rmsnorm", 32768, 8192, bf, False)      # exactly 2 MiB
    assert p.rows_in_flight == 1
    # explicit groups count too: 8 groups of 2048 rows hold 16 MiB each
    p = nb.norm_bwd_make_plan("rmsnorm", 16384, 4096, bf, False, 8)
    assert p.rows_in_flight == 2
    # fp32 rows of 8192 need 16 waves: a second row would exceed 16 waves
    p = nb.norm_bwd_make_plan("rmsnorm", 65536, 8192, torch.float32, False)
    assert (p.waves_per_row, p.rows_in_flight) == (16, 1)


@pytest.mark.parametrize("dt,N,S", [
    (torch.bfloat16, 3072, 3), (torch.bfloat16, 5120, 5), (torch.float16, 6144, 6),
    (torch.bfloat16, 7168, 7), (torch.bfloat16, 10240, 10), (torch.bfloat16, 12288, 12),
    (torch.bfloat16, 14336, 14), (torch.float32, 1536, 3), (torch.float32, 5120, 10),
    (torch.float32, 7168, 14)])
@pytest.mark.parametrize("kind,db", [("rmsnorm", False), ("layernorm", True)])
def test_exact_wave_counts(nb, kind, db, dt, N, S):
    """Widths that waves of 32-byte lanes cover exactly take that many waves,
    a power of two or not: no idle lanes."""
    p = nb.norm_bwd_make_plan(kind, 4096, N, dt, db)
    eb = torch.tensor([], dtype=dt).element_size()
    assert p.rows_per_wave == 1 and p.vec * p.chunks * eb == 32
    assert p.waves_per_row == S and S * 64 * p.vec * p.chunks == N


@pytest.mark.parametrize("kind,db,dt,N,S,P", [
    ("rmsnorm", False, torch.bfloat16, 1536, 3, 2), ("rmsnorm", False, torch.bfloat16, 2560, 5, 2),
    ("rmsnorm", False, torch.bfloat16, 3584, 7, 1), ("rmsnorm", False, torch.float16, 4608, 9, 1),
    ("layernorm", True, torch.bfloat16, 2560, 5, 2), ("layernorm", True, torch.bfloat16, 3584, 7, 2),
    ("rmsnorm", False, torch.float32, 1280, 5, 2), ("layernorm", True, torch.float32, 1280, 5, 2)])
def test_exact_sixteen_byte_lanes(nb, kind, db, dt, N, S, P):
    """Widths that 32-byte lanes cannot cover exactly but 16-byte lanes can,
    with an odd wave count, take one chunk per lane; RMSNorm aims at 12 KiB
    of rows in flight, LayerNorm keeps 16 KiB and takes the layout only at
    two rows or fewer."""
    p = nb.norm_bwd_make_plan(kind, 32768, N, dt, db)
    assert p.rows_per_wave == 1 and p.chunks == 1 and p.waves_per_row == S
    assert S * 64 * p.vec == N and p.rows_in_flight == P


@pytest.mark.parametrize("kind,dt,N", [("rmsnorm", torch.bfloat16, 1280),
                                       ("layernorm", torch.bfloat16, 1280),
                                       ("layernorm", torch.bfloat16, 1536),
                                       ("layernorm", torch.float32, 768)])
def test_inexact_widths_keep_power_of_two_waves(nb, kind, dt, N):
    """Widths no exact layout covers (or, for LayerNorm, only one with more
    than two rows in flight) keep the fewest power-of-two waves."""
    p = nb.norm_bwd_make_plan(kind, 4096, N, dt, kind == "layernorm")
    S = p.waves_per_row
    assert S & (S - 1) == 0 and S * 64 * p.vec * p.chunks > N
    assert (S // 2) * 64 * p.vec * p.chunks < N


def test_groups_do_not_depend_on_device(nb):
    # the plan is a pure function of its arguments (no device query)
    a = nb.norm_bwd_make_plan("rmsnorm", 16384, 4096, torch.bfloat16, False).as_dict()
    b = nb.norm_bwd_make_plan("rmsnorm", 16384, 4096, torch.bfloat16, False).as_dict()
    assert a == b


def test_make_plan_rejects(nb):
    lib = nb.load_library()
    p = nb.NormBwdPlan()
    assert lib.norm_bwd_make_plan(5, 1, 1, 0, 0, 0, ctypes.byref(p)) == nb.ERR_INVALID_ARG
    assert lib.norm_bwd_make_plan(0, 1, 1, 3, 0, 0, ctypes.byref(p)) == nb.ERR_UNSUPPORTED
    assert lib.norm_bwd_make_plan(0, -1, 1, 0, 0, 0, ctypes.byref(p)) == nb.ERR_INVALID_ARG
    assert lib.norm_bwd_make_plan(0, 1, -1, 0, 0, 0, ctypes.byref(p)) == nb.ERR_INVALID_ARG
    assert lib.norm_bwd_make_plan(0, 1, 1, 0, 0, -2, ctypes.byref(p)) == nb.ERR_INVALID_ARG
    assert lib.norm_bwd_make_plan(0, 1, 16385, 0, 0, 0, ctypes.byref(p)) == nb.ERR_UNSUPPORTED
    assert lib.norm_bwd_make_plan(0, 1, 32769, 2, 0, 0, ctypes.byref(p)) == nb.ERR_UNSUPPORTED
    assert lib.norm_bwd_make_plan(1, 1, 32768, 2, 0, 0, ctypes.byref(p)) == nb.OK
    assert lib.norm_bwd_make_plan(1, 1, 32768, 2, 1, 0, ctypes.byref(p)) == nb.ERR_UNSUPPORTED
    assert lib.norm_bwd_make_plan(1, 1, 16384, 2, 1, 0, ctypes.byref(p)) == nb.OK
    assert lib.norm_bwd_make_plan(0, 1, 1, 0, 2, 0, ctypes.byref(p)) == nb.ERR_INVALID_ARG
    assert "N exceeds" in nb.norm_bwd_last_error() or nb.norm_bwd_last_error()


# ---- argument rejection in the entry points (host checks only) -------------
# These calls pass fake device addresses and must be rejected before any
# launch. As a second guard they only run where no GPU is visible, so a test
# mistake can never hand a fake address to a kernel.
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-pointer rejection tests run only without a GPU")
B = 1 << 40   # fake, 256-byte aligned device addresses; never dereferenced
M_, N_ = 64, 256


def _addr(i):
    return ctypes.c_void_p(B + i * (1 << 30))


def _rms(nb, **over):
    a = dict(x=_addr(0), dy=_addr(1), gamma=_addr(2), rstd=_addr(3), M=M_, N=N_, io=2, wg=0,
             eps=1e-6, dx=_addr(4), dgamma=_addr(5), dbeta=None, ws=_addr(6),
             wsb=nb.norm_bwd_workspace_bytes("rmsnorm", M_, N_, 2, False), stream=None)
    a.update(over)
    lib = nb.load_library()
    return lib.norm_bwd_rmsnorm(a["x"], a["dy"], a["gamma"], a["rstd"], a["M"], a["N"], a["io"],
                                a["wg"], a["eps"], a["dx"], a["dgamma"], a["dbeta"], a["ws"],
                                a["wsb"], a["stream"])


def _ln(nb, **over):
    a = dict(x=_addr(0), dy=_addr(1), gamma=_addr(2), mean=_addr(7), rstd=_addr(3), M=M_, N=N_,
             io=1, wg=1, eps=1e-5, dx=_addr(4), dgamma=_addr(5), dbeta=_addr(8), ws=_addr(6),
             wsb=nb.norm_bwd_workspace_bytes("layernorm", M_, N_, 1, True), stream=None)
    a.update(over)
    lib = nb.load_library()
    return lib.norm_bwd_layernorm(a["x"], a["dy"], a["gamma"], a["mean"], a["rstd"], a["M"],
                                  a["N"], a["io"], a["wg"], a["eps"], a["dx"], a["dgamma"],
                                  a["dbeta"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(x=None), 1), (dict(dy=None), 1), (dict(gamma=None), 1),
    (dict(dx=None), 1), (dict(dgamma=None), 1),
    (dict(rstd=None, x=None), 1), (dict(rstd=None, eps=-1.0), 1),   # recompute mode checks too
    (dict(M=-1), 1), (dict(N=-3), 1), (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1),
    (dict(eps=float("inf")), 1),
    (dict(io=5), 2), (dict(wg=1), 2), (dict(wg=7), 2), (dict(N=1 << 31), 2),
    (dict(ws=None), 3), (dict(wsb=16), 3),
    (dict(ws=ctypes.c_void_p(B + 6 * (1 << 30) + 8)), 1),
    (dict(dx=_addr(0)), 1),                                  # dx aliases x
    (dict(dgamma=ctypes.c_void_p(B + 4 * (1 << 30) + 64)), 1),  # dgamma inside dx
    (dict(ws=_addr(5)), 1),                                  # workspace aliases dgamma
    (dict(dbeta=_addr(5), wsb=1 << 20), 1),                  # dbeta aliases dgamma
])
@no_gpu
def test_rmsnorm_rejects(nb, over, status):
    assert _rms(nb, **over) == status
    assert nb.norm_bwd_last_error().startswith(nb.norm_bwd_status_string(status))


@pytest.mark.parametrize("over,status", [
    (dict(mean=None), 1), (dict(rstd=None), 1),               # exactly one statistic NULL
    (dict(mean=None, rstd=None, dx=_addr(0)), 1),             # recompute: dx aliases x
    (dict(mean=None, rstd=None, wsb=100), 3),
    (dict(wg=2), 2), (dict(dbeta=_addr(6)), 1),
    (dict(wsb=100), 3),
    (dict(mean=_addr(4)), 1),                                 # dx overlaps mean
])
@no_gpu
def test_layernorm_rejects(nb, over, status):
    assert _ln(nb, **over) == status


@no_gpu
def test_execute_rejects_edited_plans(nb):
    lib = nb.load_library()
    base = nb.norm_bwd_make_plan("rmsnorm", M_, N_, torch.bfloat16, False)

    def run(p):
        return lib.norm_bwd_execute(ctypes.byref(p), _addr(0), _addr(1), _addr(2), None,
                                    _addr(3), 0, _addr(4), _addr(5), None, _addr(6),
                                    p.workspace_bytes, None)

    edits = [
        ("threads", 100), ("chunks", 3), ("vec", 2), ("waves_per_row", 0),
        ("rows_in_flight", 17), ("groups", base.groups + 5), ("rows_per_group", base.rows_per_group + 1),
        ("grid", 0), ("grid", base.groups + 1), ("lds_bytes", 4), ("workspace_bytes", 8),
        ("kind", 3), ("io_dtype", 9), ("with_dbeta", 1),
    ]
    for field, value in edits:
        p = base.copy()
        setattr(p, field, value)
        assert run(p) in (1, 2), (field, value)
    # geometry that does not cover N
    p = nb.norm_bwd_make_plan("rmsnorm", M_, 4096, torch.bfloat16, False)
    assert p.waves_per_row * 64 * p.vec * p.chunks >= 4096
    p.chunks = 1
    p.waves_per_row = 1
    p.rows_in_flight = 1
    p.threads = 64
    p.lds_bytes = 0
    assert run(p) == 1
    # the plan entry points have no eps, so they always need the statistics
    p = base.copy()
    assert lib.norm_bwd_execute(ctypes.byref(p), _addr(0), _addr(1), _addr(2), None, None, 0,
                                _addr(4), _addr(5), None, _addr(6), p.workspace_bytes, None) == 1
    assert lib.norm_bwd_execute_partials(ctypes.byref(p), _addr(0), _addr(1), _addr(2), None,
                                         None, _addr(4), _addr(6), p.workspace_bytes, None) == 1
    # misaligned x for a vectorised plan
    p = base.copy()
    assert lib.norm_bwd_execute(ctypes.byref(p), ctypes.c_void_p(B + 2), _addr(1), _addr(2),
                                None, _addr(3), 0, _addr(4), _addr(5), None, _addr(6),
                                p.workspace_bytes, None) == 1


@no_gpu
def test_reduce_and_probe_reject(nb):
    lib = nb.load_library()
    assert lib.norm_bwd_reduce_partials(-1, 8, 0, _addr(0), 1 << 20, _addr(1), None, None) == 1
    assert lib.norm_bwd_reduce_partials(4, 8, 0, _addr(0), 16, _addr(1), None, None) == 3
    assert lib.norm_bwd_reduce_partials(4, 8, 0, _addr(0), 1 << 20, None, None, None) == 1
    assert lib.norm_bwd_reduce_partials(4, 8, 5, _addr(0), 1 << 20, _addr(1), None, None) == 2
    assert lib.norm_bwd_reduce_partials(4, 8, 1, _addr(0), 16, _addr(1), None, None) == 3
    # groups * N whose byte count would wrap around to a small size
    assert lib.norm_bwd_reduce_partials(1 << 61, 8, 0, _addr(0), 1 << 20, _addr(1), None, None) == 1
    assert lib.norm_bwd_reduce_partials(1 << 59, 1 << 4, 0, _addr(0), 0, _addr(1), _addr(2),
                                        None) == 1
    assert lib.norm_bwd_probe_copy(_addr(0), _addr(1), 17, None) == 1
    assert lib.norm_bwd_probe_copy(_addr(0), ctypes.c_void_p(B + 8), 1024, None) == 1
    # the triad probe: sizes, alignment, unroll, grid and overlap, nothing launched
    T = lib.norm_bwd_probe_triad
    assert T(_addr(0), _addr(1), _addr(2), 0, 0, 4, None) == 0          # nothing to do
    assert T(_addr(0), _addr(1), _addr(2), 24, 0, 4, None) == 1         # not a 16-byte multiple
    assert T(ctypes.c_void_p(B + 8), _addr(1), _addr(2), 1024, 0, 4, None) == 1
    assert T(None, _addr(1), _addr(2), 1024, 0, 4, None) == 1
    assert T(_addr(0), _addr(1), _addr(2), 1024, 0, 3, None) == 1       # unroll
    assert T(_addr(0), _addr(1), _addr(2), 1024, -1, 4, None) == 1      # grid
    assert T(_addr(0), _addr(1), _addr(2), 1024, (1 << 20) + 1, 4, None) == 1
    assert T(_addr(0), _addr(1), ctypes.c_void_p(B + 512), 1024, 0, 4, None) == 1  # c overlaps a
    # the cache-policy triad: sizes (4096 * unroll multiples, 32-bit range),
    # unroll, policy bits, alignment and overlap, nothing launched
    TP = lib.norm_bwd_probe_triad_policy
    assert TP(_addr(0), _addr(1), _addr(2), 0, 1, 2, 2, None) == 0
    assert TP(_addr(0), _addr(1), _addr(2), 2048, 1, 2, 2, None) == 1
    assert TP(_addr(0), _addr(1), _addr(2), 4096, 2, 2, 2, None) == 1
    assert TP(_addr(0), _addr(1), _addr(2), 8192, 8, 2, 2, None) == 1
    assert TP(_addr(0), _addr(1), _addr(2), 1 << 32, 1, 2, 2, None) == 1
    assert TP(_addr(0), _addr(1), _addr(2), 4096, 1, 4, 2, None) == 1  # not a policy bit
    assert TP(_addr(0), _addr(1), _addr(2), 4096, 1, 2, 32, None) == 1
    assert TP(_addr(0), _addr(1), _addr(2), 4096, 1, -1, 2, None) == 1
    assert TP(ctypes.c_void_p(B + 8), _addr(1), _addr(2), 4096, 1, 2, 2, None) == 1
    assert TP(_addr(0), _addr(1), ctypes.c_void_p(B + 512), 4096, 1, 2, 2, None) == 1


def _fwd(nb, kind, **over):
    a = dict(x=_addr(0), gamma=_addr(1), beta=_addr(2), M=M_, N=N_, io=2, eps=1e-5, y=_addr(3),
             mean=_addr(4), rstd=_addr(5), stream=None)
    a.update(over)
    lib = nb.load_library()
    if kind == "layernorm":
        return lib.norm_fwd_layernorm(a["x"], a["gamma"], a["beta"], a["M"], a["N"], a["io"],
                                      a["eps"], a["y"], a["mean"], a["rstd"], a["stream"])
    return lib.norm_fwd_rmsnorm(a["x"], a["gamma"], a["M"], a["N"], a["io"], a["eps"], a["y"],
                                a["rstd"], a["stream"])


@pytest.mark.parametrize("kind", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("over,status", [
    (dict(x=None), 1), (dict(gamma=None), 1), (dict(y=None), 1),
    (dict(M=-1), 1), (dict(N=-1), 1), (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1),
    (dict(io=3), 2), (dict(N=1 << 31), 2),
    (dict(y=_addr(0)), 1),                                    # y aliases x
    (dict(rstd=ctypes.c_void_p(B + 3 * (1 << 30) + 256)), 1),  # rstd inside y
    (dict(rstd=_addr(1)), 1),                                 # rstd aliases gamma
])
@no_gpu
def test_forward_rejects(nb, kind, over, status):
    assert _fwd(nb, kind, **over) == status
    assert nb.norm_bwd_last_error().startswith(nb.norm_bwd_status_string(status))


@no_gpu
def test_forward_layernorm_rejects_overlapping_statistics(nb):
    assert _fwd(nb, "layernorm", mean=_addr(5)) == 1          # mean aliases rstd
    assert _fwd(nb, "layernorm", mean=_addr(2)) == 1          # mean aliases beta
    # empty problems return OK without touching any pointer
    assert _fwd(nb, "layernorm", M=0, x=None, y=None) == 0
    assert _fwd(nb, "rmsnorm", N=0, x=None, y=None) == 0


def _ex(nb, **over):
    a = nb.NormBwdArgs()
    vals = dict(kind=1, io_dtype=2, wgrad_dtype=0, flags=0, M=M_, N=N_, groups=0,
                x=B, ldx=0, dy=B + (1 << 30), lddy=0, gamma=B + 2 * (1 << 30), mean=None,
                rstd=B + 3 * (1 << 30), dx=B + 4 * (1 << 30), lddx=0,
                dgamma=B + 5 * (1 << 30), dbeta=None, workspace=B + 6 * (1 << 30),
                workspace_bytes=1 << 20, stream=None, eps=1e-6, reserved=0)
    vals.update(over)
    for k, v in vals.items():
        setattr(a, k, v)
    return nb.load_library().norm_bwd_ex(ctypes.byref(a))


@pytest.mark.parametrize("over,status", [
    (dict(flags=2), 1), (dict(reserved=1), 1), (dict(kind=4), 1), (dict(groups=-1), 1),
    (dict(ldx=N_ - 1), 1), (dict(lddy=-8), 1), (dict(lddx=1), 1),
    (dict(M=-1), 1), (dict(eps=-1.0), 1), (dict(io_dtype=7), 2),
    (dict(kind=0, mean=B + 7 * (1 << 30), rstd=None), 1),          # exactly one statistic
    (dict(ldx=1 << 60), 1),                                          # M * stride overflows
    (dict(lddx=2 * N_, dx=B + 1024), 1),                             # dx's span overlaps x
    (dict(workspace_bytes=64), 3), (dict(groups=M_, workspace_bytes=4 * N_ * 8), 3),
])
@no_gpu
def test_ex_rejects(nb, over, status):
    assert _ex(nb, **over) == status
    assert nb.norm_bwd_last_error().startswith(nb.norm_bwd_status_string(status))


@no_gpu
def test_ex_empty_accumulate_is_a_no_op(nb):
    # M = 0 with NORM_BWD_ACCUMULATE adds nothing: no launch, status OK
    assert _ex(nb, M=0, flags=1) == 0
    assert _ex(nb, N=0) == 0


def _wg(nb, **over):
    a = dict(kind=0, x=_addr(0), dy=_addr(1), mean=_addr(2), rstd=_addr(3), M=M_, N=N_, io=2,
             wg=0, dgamma=_addr(4), dbeta=_addr(5), flags=0, stream=None)
    a.update(over)
    return nb.load_library().norm_bwd_wgrad(a["kind"], a["x"], a["dy"], a["mean"], a["rstd"],
                                            a["M"], a["N"], a["io"], a["wg"], a["dgamma"],
                                            a["dbeta"], a["flags"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(kind=2), 1), (dict(flags=4), 1), (dict(io=9), 2), (dict(wg=1), 2), (dict(wg=5), 2),
    (dict(M=-1), 1), (dict(N=-1), 1), (dict(N=1 << 31), 2),
    (dict(x=None), 1), (dict(dy=None), 1), (dict(rstd=None), 1), (dict(mean=None), 1),
    (dict(dgamma=None), 1), (dict(dgamma=_addr(0)), 1), (dict(dbeta=_addr(3)), 1),
    (dict(dbeta=ctypes.c_void_p(B + 4 * (1 << 30) + 64)), 1),
])
@no_gpu
def test_wgrad_rejects(nb, over, status):
    assert _wg(nb, **over) == status
    assert nb.norm_bwd_last_error().startswith(nb.norm_bwd_status_string(status))


@no_gpu
def test_wgrad_trivial_cases_launch_nothing(nb):
    assert _wg(nb, N=0) == 0
    assert _wg(nb, M=0, flags=1, x=None, dy=None, mean=None, rstd=None) == 0
    assert _wg(nb, kind=1, mean=None, M=0, flags=1) == 0


def test_binding_refuses_cpu_tensors(nb):
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    g = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        nb.norm_bwd_rmsnorm(x, x, g, torch.ones(4))
    for kind in ("layernorm", "rmsnorm", 0, 1):
        with pytest.raises(ValueError, match="GPU"):
            nb.norm_bwd_ex(kind, x, x, g, None, None)
    with pytest.raises(ValueError, match="GPU"):
        nb.norm_fwd_layernorm(x, g, None)
    with pytest.raises(ValueError, match="GPU"):
        nb.norm_fwd_rmsnorm(x, g)
    with pytest.raises(ValueError, match="GPU"):
        nb.norm_bwd_wgrad("rmsnorm", x, x, None, torch.ones(4))


def _log_probe(env_value):
    """A fresh process that makes one failing call; returns its stderr."""
    import os
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("NORM_BWD_LOG", None)
    if env_value is not None:
        env["NORM_BWD_LOG"] = env_value
    code = ("import ctypes, rmsnorm_backward_amd as nb\n"
            "lib = nb.load_library()\n"
            "p = nb.NormBwdPlan()\n"
            "assert lib.norm_bwd_make_plan(7, 4, 8, 0, 0, 0, ctypes.byref(p)) == 1\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stderr


def test_errors_print_only_with_norm_bwd_log():
    """The library is silent by default; NORM_BWD_LOG=1 writes each failure's
    message to stderr (the same text norm_bwd_last_error returns)."""
    assert "norm_bwd:" not in _log_probe(None)
    assert "norm_bwd:" not in _log_probe("0")
    err = _log_probe("1")
    assert "norm_bwd: NORM_BWD_ERR_INVALID_ARG" in err
