"""Host-side checks of libdpg that need no GPU: exported symbols, the planner,
workspace sizing, the plan cache and argument validation (every case here is
rejected before any HIP call)."""
import ctypes

import pytest

dpg = pytest.importorskip("deterministic_bf16_projection_amd")

L = dpg.lib()
_i, _p, _c, _z = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
BF16, F32 = dpg.BF16, dpg.F32


def test_exports_every_header_symbol():
    names = dpg.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_version():
    assert "gfx950" in dpg.version()


def plan(pass_, T, N, K, out=BF16, det=1, split=0):
    buf = ctypes.create_string_buffer(1024)
    assert L.dpg_plan_describe(pass_, T, N, K, out, det, split, buf, 1024) == 0
    return dpg.parse_plan(buf.value.decode())


@pytest.mark.parametrize("pass_", [0, 1, 2])
@pytest.mark.parametrize("T", [16384, 16231])
def test_big_projection_whole_k_per_tile(pass_, T):
    """4096 -> 12288 at T 16384 / 16231: the deterministic plan reduces the
    whole K inside each output tile (one K split), as the row-half-release
    page's plans do."""
    p = plan(pass_, T, 12288, 4096)
    assert p["kind"] == "gemm"
    assert p["splits"] == "1"
    assert p["workspace"] == "0"
    assert p["tile"] == "256x256x64"


@pytest.mark.parametrize("pass_", [0, 1, 2])
def test_t_plus_minus_one_same_plan(pass_):
    """Neighbouring token counts keep program, raster group and K partition
    (planner test design on the row-half-release page)."""
    base = plan(pass_, 16384, 12288, 4096)
    for T in (16383, 16385):
        p = plan(pass_, T, 12288, 4096)
        for key in ("tile", "group_m", "splits", "layout"):
            assert p[key] == base[key], (T, key)


@pytest.mark.parametrize("T,blocks", [(1025, 17), (4031, 63), (16173, 253), (16384, 256), (65537, 1025)])
def test_wgrad_two_way_partition(T, blocks):
    """Two K splits over ceil(T/64) 64-token blocks: split 0 takes the first
    ceil(B/2) blocks (odd block counts included)."""
    p = plan(2, T, 64, 4096, out=F32, det=0, split=2)
    assert int(p["kt_total"]) == blocks
    assert int(p["splits"]) == 2
    assert int(p["kt_per_split"]) == (blocks + 1) // 2
    assert int(p["workspace"]) == 2 * 64 * 4096 * 4


def test_forced_split_one():
    p = plan(2, 16384, 128, 4096, out=BF16, det=0, split=1)
    assert p["splits"] == "1" and p["workspace"] == "0"


def test_skinny_unit_shapes():
    """Skinny weight gradients: 128-column units when they give at least half
    as many workgroups as CUs, 64-column units otherwise (forced small split
    counts); one or two 64-row blocks of dW.  One row block: operands straight
    from registers (128 columns) or the LDS-staged kernel (64 columns); two row
    blocks: operands fetched straight into LDS (both widths).  The
    exact-integer GPU shapes together reach all four variants."""
    def tile(T, N, K, det, split):
        p = plan(2, T, N, K, out=F32, det=det, split=split)
        assert p["kernel"] == "skinny", p
        return p["tile"]
    assert tile(16384, 64, 4096, 1, 0) == "64x128x64"
    assert tile(16384, 128, 4096, 1, 0) == "128x128x64"
    assert tile(16384, 64, 4096, 0, 2) == "64x64x64"
    assert tile(16384, 128, 4096, 0, 1) == "128x64x64"
    assert tile(16384, 48, 5120, 1, 0) == "64x128x64"
    # long token ranges keep 128-column units (with the LDS-fetching kernel they
    # are faster than 256-column ones)
    assert tile(65537, 128, 4096, 1, 0) == "128x128x64"
    assert tile(65537, 64, 4096, 1, 0) == "64x128x64"
    assert tile(65537, 128, 4096, 0, 2) == "128x64x64"
    assert tile(32768, 104, 4096, 1, 0) == "128x128x64"
    p = plan(2, 16400, 40, 1000, out=F32, det=1, split=0)
    assert p["tile"] == "64x128x64" and p["splits"] == "16" and p["kt_per_split"] == "17", p
    p = plan(2, 16400, 104, 1000, out=F32, det=1, split=0)
    assert p["tile"] == "128x128x64" and p["splits"] == "16" and p["kt_per_split"] == "17", p
    seen = set()
    for T, N, K in [(4031, 128, 4096), (16384, 48, 5120), (1025, 104, 1024), (16384, 128, 4096), (65537, 104, 3968),
                    (16400, 40, 1000), (16400, 104, 1000)]:
        for det, split in [(1, 0), (0, 1), (0, 2), (1, 3)]:
            seen.add(tile(T, N, K, det, split))
    assert seen == {"64x64x64", "64x128x64", "128x64x64", "128x128x64"}


def test_medium_projection_plans():
    """Plans the cost model picks for the checkpointed-step shapes (measured on
    MI355X to be the fastest or within 3% of it among forced split counts):
    4096->1024 passes whole-K on 256x256 tiles except the weight gradient
    (4 splits); 4096->512 forward on two 128x128 workgroups per CU, unsplit."""
    def pick(pass_, N):
        p = plan(pass_, 16384, N, 4096, out=F32)
        return p["tile"], p["splits"]
    assert pick(0, 1024) == ("256x256x64", "1")
    assert pick(1, 1024) == ("256x256x64", "1")
    assert pick(2, 1024) == ("256x256x64", "4")
    assert pick(0, 512) == ("128x128x64", "1")
    assert pick(1, 512) == ("256x256x64", "1")
    assert pick(2, 512) == ("256x256x64", "8")


def test_router_uses_bf16x3():
    p = plan(3, 64, 256, 4096, out=F32)
    assert p["x3"] == "1"
    assert plan(4, 1024, 256, 4096, out=F32)["layout"] == "Akmajor_Bmnmajor"
    assert plan(5, 256, 256, 4096, out=F32)["layout"] == "Amnmajor_Bmnmajor"


def test_deterministic_plan_ignores_device():
    """The deterministic plan is a function of the shape only."""
    a = plan(0, 64, 1024, 4096)
    b = plan(0, 64, 1024, 4096)
    assert a == b


def test_empty_shapes():
    assert plan(0, 0, 64, 64)["kind"] == "noop"
    assert plan(2, 0, 64, 64)["kind"] == "zero_fill"   # empty reduction writes zeros
    assert plan(0, 16, 64, 0)["kind"] == "zero_fill"
    assert plan(1, 16, 0, 64)["kind"] == "zero_fill"
    assert plan(2, 16, 0, 64)["kind"] == "noop"


def test_workspace_size_matches_plan():
    for args in [(2, 16384, 64, 4096, F32, 0, 2), (0, 64, 1024, 4096, BF16, 1, 0), (3, 64, 256, 4096, F32, 1, 0)]:
        p = plan(args[0], args[1], args[2], args[3], out=args[4], det=args[5], split=args[6])
        assert L.dpg_workspace_size(*args) == int(p["workspace"])
    assert L.dpg_workspace_size(3, 64, 256, 4096, BF16, 1, 0) == ctypes.c_size_t(-1).value


def test_plan_describe_rejects():
    buf = ctypes.create_string_buffer(16)
    assert L.dpg_plan_describe(0, -1, 8, 8, BF16, 1, 0, buf, 16) == 1
    assert L.dpg_plan_describe(9, 1, 8, 8, BF16, 1, 0, buf, 16) == 1
    assert L.dpg_plan_describe(0, 1, 8, 8, BF16, 1, 0, None, 0) == 1
    # truncation keeps a NUL-terminated prefix
    assert L.dpg_plan_describe(0, 64, 64, 64, BF16, 1, 0, buf, 16) == 0
    assert len(buf.value) == 15


def test_cache_generation():
    e0, g0 = dpg.plan_cache_stats()
    dpg.clear_plan_cache()
    e1, g1 = dpg.plan_cache_stats()
    assert e1 == 0 and g1 == g0 + 1


# ------------------------------------------------------ validation (no launch) --
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case fails validation first


def fwd(x=FAKE, ldx=64, w=FAKE, ldw=64, y=FAKE, ldy=64, out=BF16, T=16, N=64, K=64, det=1, split=0, ws=None, wsb=0):
    return L.dpg_forward(x, ldx, w, ldw, y, ldy, out, T, N, K, det, split, ws, wsb, None)


def test_validation_errors():
    assert fwd(T=-1) == 1
    assert fwd(x=None) == 1                       # NULL for non-empty data
    assert fwd(ldx=32) == 1                       # ld < cols
    assert fwd(x=FAKE + 2) == 3                   # misaligned base
    assert fwd(ldy=68) == 3                       # ld * 2 bytes not a multiple of 16
    assert fwd(K=60, ldx=64, ldw=64) == 3         # contiguous extent not a multiple of 8
    assert fwd(out=7) == 1                        # bad dtype
    assert fwd(split=65) == 2
    assert fwd(split=-1) == 2
    # a forced split needs a workspace
    assert L.dpg_wgrad(FAKE, 64, FAKE, 64, FAKE, 64, F32, 4096, 64, 64, 0, 2, None, 0, None) == 4
    assert L.dpg_router_forward(FAKE, 64, FAKE + 4, 64, FAKE, 64, 16, 64, 64, 1, 0, None, 0, None) == 3


def test_status_strings():
    for s in range(6):
        assert L.dpg_status_string(s)


def test_deterministic_switch_resolution():
    """torch.use_deterministic_algorithms(True) turns a fast-plan request into a
    deterministic one, with a single warning."""
    import warnings
    import torch
    from deterministic_bf16_projection_amd import autograd as dag
    assert dag.resolve_deterministic(True) is True
    prev = torch.are_deterministic_algorithms_enabled()
    try:
        torch.use_deterministic_algorithms(False)
        assert dag.resolve_deterministic(False) is False
        torch.use_deterministic_algorithms(True)
        dag._warned[0] = False
        with warnings.catch_warnings(record=True) as rec:
            warnings.simplefilter("always")
            assert dag.resolve_deterministic(False) is True
            assert dag.resolve_deterministic(False) is True
        assert len([r for r in rec if "deterministic" in str(r.message)]) == 1
    finally:
        torch.use_deterministic_algorithms(prev)


def _plan_b(pass_, batch, T, N, K, out=BF16, det=1, split=0, wl=0):
    buf = ctypes.create_string_buffer(1024)
    assert L.dpg_plan_describe_batched(pass_, wl, batch, T, N, K, out, det, split, buf, 1024) == 0
    return dpg.parse_plan(buf.value.decode())


def test_batched_plans():
    """Batched plans: the unit stream covers every problem, the workspace holds
    batch x splits planes, the skinny kernel is single-problem only, and a
    [K,N] weight flips the operand majorness as the GEMM view says."""
    p = _plan_b(0, 16, 2048, 128, 512)
    assert p["batch"] == "16" and p["layout"] == "Akmajor_Bkmajor"
    assert int(p["grid"]) == int(p["tiles"].split("x")[0]) * int(p["tiles"].split("x")[1]) * int(p["splits"]) * 16
    assert _plan_b(0, 16, 2048, 128, 512, wl=1)["layout"] == "Akmajor_Bmnmajor"
    assert _plan_b(1, 16, 2048, 128, 512, wl=1)["layout"] == "Akmajor_Bkmajor"
    q = _plan_b(2, 4, 1025, 64, 512, out=F32, det=0, split=2)
    assert q["kernel"] != "skinny" and q["splits"] == "2"
    assert int(q["workspace"]) == 4 * 2 * 64 * 512 * 4
    assert L.dpg_workspace_size_batched(2, 0, 4, 1025, 64, 512, F32, 0, 2) == 4 * 2 * 64 * 512 * 4
    r = _plan_b(2, 3, 1025, 64, 512, wl=1)   # dW as [K, N]: M = K, N = N
    assert r["M"] == "512" and r["N"] == "64"
    assert _plan_b(2, 1, 16384, 64, 4096)["kernel"] == "skinny"
    assert _plan_b(0, 0, 64, 64, 64)["kind"] == "noop"
    buf = ctypes.create_string_buffer(64)
    assert L.dpg_plan_describe_batched(3, 0, 1, 64, 256, 4096, F32, 1, 0, buf, 64) == 1   # no batched router
    assert L.dpg_plan_describe_batched(0, 2, 1, 64, 64, 64, BF16, 1, 0, buf, 64) == 1     # bad layout


def test_batched_validation_errors():
    """Rejected before any launch: overlapping batched outputs, misaligned or
    negative batch strides, bad layouts."""
    FAKE = 0x10000
    fwd = L.dpg_forward_batched
    # x [B,T,K] = [2, 64, 64], w [64, 64], y [2, 64, 64]
    args = lambda sx, sw, sy, wl=0: (FAKE, 64, sx, FAKE, 64, sw, wl, FAKE, 64, sy, BF16, 2, 64, 64, 64, 1, 0,
                                     None, 0, None)
    assert fwd(*args(4096, 0, 64 * 64 - 8)) == 1      # outputs overlap
    assert fwd(*args(4096, 0, -4096)) == 1            # negative output stride
    assert fwd(*args(4100, 0, 4096)) == 3             # batch stride not 16-byte aligned
    assert fwd(*args(4096, 0, 4096, wl=5)) == 1       # bad layout
    assert fwd(FAKE, 64, 4096, FAKE, 64, 0, 0, FAKE, 64, 4096, BF16, -1, 64, 64, 64, 1, 0, None, 0, None) == 1
