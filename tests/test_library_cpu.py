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
    assert p["tile"] == "64x128x64" and p["splits"] == "32" and p["kt_per_split"] == "9", p
    p = plan(2, 16400, 104, 1000, out=F32, det=1, split=0)
    assert p["tile"] == "128x128x64" and p["splits"] == "32" and p["kt_per_split"] == "9", p
    # at least 8 token blocks a split from 24 blocks on, 16 below
    assert plan(2, 1472, 64, 4096, out=F32)["splits"] == "1"
    assert plan(2, 1473, 64, 4096, out=F32)["splits"] == "3"
    assert plan(2, 4031, 64, 4096, out=F32)["splits"] == "7"
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


# shapes of every workload (T, N, K as the entry points take them) plus K tails
FORCED_SPLIT_SHAPES = [
    (64, 1024, 4096), (16384, 12288, 4096), (16231, 12288, 4096), (16384, 64, 4096), (65537, 128, 4096),
    (1025, 48, 5120), (4031, 64, 5120), (16384, 512, 4096), (333, 200, 264), (1, 8, 8), (4096, 4104, 1032),
]
ROUTER_SHAPES = [(64, 256, 4096), (256, 256, 4096), (1024, 256, 4096), (4096, 256, 4104), (96, 256, 1024)]


def _reduction_blocks(pass_, T, N, K):
    return -(-{0: K, 1: N, 2: T}[pass_ % 3] // 64)


def _check_plan(pass_, T, N, K, out, det, split):
    p = plan(pass_, T, N, K, out=out, det=det, split=split)
    assert p["kind"] == "gemm", p
    blocks = _reduction_blocks(pass_, T, N, K)
    assert int(p["kt_total"]) == blocks
    s = int(p["splits"])
    assert s == (min(split, blocks) if split else s) and 1 <= s <= blocks, (split, p)
    assert int(p["kt_per_split"]) == -(-blocks // s)
    assert int(p["grid"]) >= 1
    # every plan names a compiled kernel: pipelined 256x256 / 128x128 (BF16x3 on
    # 128x128 only), the skinny kernels, or the generic kernel on 64x64 tiles
    kernel, tile = p["kernel"], p["tile"]
    assert kernel in ("pipelined", "generic", "skinny"), p
    if kernel == "generic":
        assert tile == "64x64x64", p
    if kernel == "pipelined":
        assert tile in ("256x256x64", "128x128x64"), p
        assert p["x3"] == "0" or tile == "128x128x64", p
    M, Nn = int(p["M"]), int(p["N"])
    if p["streamk"] == "1":
        # split-K mode, no forced split: stream-K keeps two FP32 tile slots per workgroup
        assert split == 0 and det == 0 and s == 1, p
        bm, bn = (int(v) for v in p["tile"].split("x")[:2])
        assert int(p["workspace"]) == 2 * int(p["grid"]) * bm * bn * 4, p
    else:
        assert int(p["workspace"]) == (s * M * Nn * 4 if s > 1 else 0), p
    assert L.dpg_workspace_size(pass_, T, N, K, out, det, split) == int(p["workspace"])
    return p


@pytest.mark.parametrize("split", range(0, 65))
def test_forced_split_counts_all_passes(split):
    """Any split_k in 1..64 gives min(split_k, B) splits of the balanced
    partition (B = 64-element blocks of the reduction) on a compiled kernel,
    with the workspace sized for exactly those splits, for every pass."""
    for T, N, K in FORCED_SPLIT_SHAPES:
        for pass_ in (0, 1, 2):
            for out in (BF16, F32):
                for det in (1, 0):
                    _check_plan(pass_, T, N, K, out, det, split)
    for T, E, H in ROUTER_SHAPES:
        for pass_ in (3, 4, 5):
            for det in (1, 0):
                p = _check_plan(pass_, T, E, H, F32, det, split)
                assert p["x3"] == "1"


def test_k_tails_take_the_generic_64_tile():
    """A K-major reduction that is not a multiple of 64 has no pipelined
    kernel: the plan is the generic kernel on 64x64 tiles (the 256x256 and
    128x128 generic variants are not compiled), whatever the split."""
    for pass_, T, N, K in [(0, 16384, 12288, 4104), (0, 4096, 4096, 1032), (1, 4096, 1032, 4096),
                           (1, 16384, 4104, 12288), (3, 4096, 256, 4104)]:
        for split in (0, 1, 2, 5):
            p = plan(pass_, T, N, K, out=F32, det=1, split=split)
            assert p["kernel"] == "generic" and p["tile"] == "64x64x64", p
    # the weight gradient's operands are MN-major: ragged T stays pipelined
    p = plan(2, 16231, 12288, 4096)
    assert p["kernel"] == "pipelined", p


def test_balanced_partition_sizes():
    """Forced split counts that do not divide the block count: sizes differ by
    at most one block and none is empty (63 splits of 64 blocks: 62 of one
    block and one of two, not 32 splits of two)."""
    p = plan(0, 1024, 1024, 4096, det=0, split=63)
    assert p["splits"] == "63" and p["kt_per_split"] == "2", p
    p = plan(0, 1024, 1024, 4096, det=0, split=5)
    assert p["splits"] == "5" and p["kt_per_split"] == "13", p
    p = plan(2, 16384, 64, 4096, out=F32, det=0, split=7)
    assert p["kernel"] == "skinny" and p["splits"] == "7" and p["kt_per_split"] == "37", p


def test_plan_cache_bounded():
    """10k distinct token counts keep the cache at its capacity (least
    recently used plans dropped); a cleared cache starts a new generation."""
    dpg.clear_plan_cache()
    cap = dpg.plan_cache_capacity()
    assert 0 < cap <= 100000
    for T in range(1, 10001):
        assert L.dpg_workspace_size(2, T, 64, 4096, F32, 1, 0) != ctypes.c_size_t(-1).value
    e, g = dpg.plan_cache_stats()
    assert e == min(cap, 10000)
    # a recently used key stays cached while older ones are dropped
    L.dpg_workspace_size(2, 10000, 64, 4096, F32, 1, 0)
    e2, g2 = dpg.plan_cache_stats()
    assert e2 == e and g2 == g
    dpg.clear_plan_cache()
    e3, g3 = dpg.plan_cache_stats()
    assert e3 == 0 and g3 == g + 1


def test_streamk_plans():
    """Split-K mode takes stream-K on the 256x256 pipelined tile where the last round
    of tiles would leave most CUs idle (workspace: two FP32 slots of a tile
    per workgroup; grid: exactly the workgroups the partition is cut for);
    the deterministic mode, forced split counts, batched calls and the
    4096->12288 workloads (whole rounds) never take it."""
    for pass_, T, N, K, tile, G, outs in [(0, 4352, 4096, 4096, 256, 256, (BF16, F32)),
                                          (0, 8448, 4096, 4096, 256, 256, (BF16, F32)),
                                          (1, 4352, 4352, 4096, 256, 256, (BF16, F32)),
                                          (2, 4352, 4352, 4096, 256, 256, (BF16, F32)),
                                          (0, 4608, 4352, 8192, 256, 256, (BF16, F32))]:
        for out in outs:
            p = plan(pass_, T, N, K, out=out, det=0)
            assert p["streamk"] == "1" and p["kernel"] == "pipelined", p
            assert p["tile"] == "%dx%dx64" % (tile, tile) and int(p["grid"]) == G, p
            assert int(p["workspace"]) == 2 * G * tile * tile * 4, p
            assert L.dpg_workspace_size(pass_, T, N, K, out, 0, 0) == int(p["workspace"])
            assert plan(pass_, T, N, K, out=out, det=1)["streamk"] == "0"
            assert plan(pass_, T, N, K, out=out, det=0, split=2)["streamk"] == "0"
    for pass_ in (0, 1, 2):
        for T in (16384, 16231):
            assert plan(pass_, T, 12288, 4096, det=0)["streamk"] == "0"
    assert _plan_b(0, 2, 4352, 4096, 4096, det=0)["streamk"] == "0"
    # fewer tiles than workgroups (no whole round) stay with split-K plans
    assert plan(1, 8448, 4096, 1024, out=F32, det=0)["streamk"] == "0"


def test_router_arithmetic_setting():
    """The router arithmetic setting is part of the plan: 'fp32' plans the FP32
    FMA kernel (no BF16x3), 'bf16x3' never does, for every router pass, shape
    and forced split; projection passes ignore the setting; bad values are
    refused."""
    prev = dpg.set_router_arithmetic("fp32")
    try:
        for T in (64, 256, 1024, 4096):
            for pass_ in (3, 4, 5):
                for split in (0, 1, 2, 5):
                    p = plan(pass_, T, 256, 4096, out=F32, det=1, split=split)
                    assert p["kernel"] == "ffma" and p["arith"] == "fp32fma" and p["x3"] == "0", p
                    assert p["tile"] == "64x64x64", p
                    if split:
                        assert int(p["splits"]) == min(split, -(-{3: 4096, 4: 256, 5: T}[pass_] // 64)), p
        assert plan(0, 64, 1024, 4096)["arith"] == "bf16"
        dpg.set_router_arithmetic("bf16x3")
        for T in (64, 256, 1024, 4096):
            for pass_ in (3, 4, 5):
                p = plan(pass_, T, 256, 4096, out=F32)
                assert p["kernel"] != "ffma" and p["arith"] == "bf16x3", p
        assert dpg.get_router_arithmetic() == "bf16x3"
        assert L.dpg_set_router_arithmetic(7) == 1
        assert dpg.get_router_arithmetic() == "bf16x3"
    finally:
        dpg.set_router_arithmetic(prev)


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
    # forced split counts outside the old list are planned, not rejected:
    # without a workspace the call stops at the workspace check (no launch)
    for split in (5, 7, 63):
        assert L.dpg_wgrad(FAKE, 64, FAKE, 64, FAKE, 64, F32, 4096, 64, 64, 0, split, None, 0, None) == 4
        assert L.dpg_router_forward(FAKE, 4096, FAKE, 4096, FAKE, 256, 64, 256, 4096, 1, split, None, 0,
                                    None) == 4
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


def _edges(pass_, N, K, out, t_max):
    from tests.plan_windows import plan_key
    prev, edges = None, []
    for T in range(1, t_max + 1):
        k = plan_key(dpg.plan_describe(pass_, T, N, K, out, True, 0))
        if prev is not None and k != prev:
            edges.append(T)
        prev = k
    return edges


def test_plan_windows_are_the_listed_ones():
    """The deterministic plans change exactly at the T values the window-edge
    GPU tests check (both sides of each)."""
    import torch
    from tests import plan_windows as pw
    for (K, N), edges in pw.SKINNY_EDGES.items():
        for out in (torch.bfloat16, torch.float32):
            assert _edges(dpg.PASS_WGRAD, N, K, out, pw.SKINNY_T_MAX) == edges, (K, N, out)
    for op, edges in pw.ROUTER_EDGES.items():
        p = {"fwd": dpg.PASS_ROUTER_FORWARD, "dgrad": dpg.PASS_ROUTER_DGRAD, "wgrad": dpg.PASS_ROUTER_WGRAD}[op]
        assert _edges(p, 256, 4096, torch.float32, pw.ROUTER_T_MAX) == edges, op
    for op, edges in pw.SMALL_EDGES.items():
        p = {"fwd": dpg.PASS_FORWARD, "dgrad": dpg.PASS_DGRAD, "wgrad": dpg.PASS_WGRAD}[op]
        assert _edges(p, 1024, 4096, torch.bfloat16, pw.SMALL_T_MAX) == edges, op


def test_describe_buffer_edges_and_stats_pointers():
    """dpg_plan_describe truncates to buflen - 1 characters (NUL-terminated),
    rejects a NULL or empty buffer; dpg_plan_cache_stats accepts NULL
    pointers; every status has a text."""
    full = ctypes.create_string_buffer(1024)
    assert L.dpg_plan_describe(0, 64, 1024, 4096, BF16, 1, 0, full, 1024) == 0
    text = full.value
    assert text.startswith(b"pass=forward") and len(text) < 1023
    for n in (1, 2, 17):
        buf = ctypes.create_string_buffer(b"\xff" * 32, 32)
        assert L.dpg_plan_describe(0, 64, 1024, 4096, BF16, 1, 0, buf, n) == 0
        assert buf.raw[:n] == text[:n - 1] + b"\x00"
        assert buf.raw[n:32] == b"\xff" * (32 - n)  # nothing past buflen
    assert L.dpg_plan_describe(0, 64, 1024, 4096, BF16, 1, 0, None, 64) == 1
    assert L.dpg_plan_describe(0, 64, 1024, 4096, BF16, 1, 0, full, 0) == 1
    L.dpg_plan_cache_stats(None, None)
    e = ctypes.c_int64(-1)
    L.dpg_plan_cache_stats(ctypes.byref(e), None)
    assert e.value >= 0
    for st in range(0, 6):
        assert L.dpg_status_string(st) and L.dpg_status_string(st) != b"unknown status"
    assert L.dpg_status_string(99) == b"unknown status"
