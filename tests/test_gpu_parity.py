"""Parity of the HIP path with the FP64 oracle, through the C ABI (GPU).

Budgets are those of the K1 weight-gradient page (description): BF16 output
atol = rtol = 1e-2 with no element outside; FP32 output relative Frobenius
error <= 5e-5 and max error <= 1e-3 * max |ref|.  Exact-integer inputs make
any FP32 accumulation order exact, so there the outputs must match the oracle
bit for bit (FP32) or its nearest-even BF16 rounding (BF16).
"""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import budgets
from tests.gpu_util import dev_bf16, dev_f32, host_bits, host_f64, report, sample_positions

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

OUT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _run(pass_name, a, b, out_dtype, det=True, split=0, out=None):
    fn = {"fwd": dpg.dpg_forward, "dgrad": dpg.dpg_dgrad, "wgrad": dpg.dpg_wgrad}[pass_name]
    r = fn(a, b, out=out, out_dtype=out_dtype, deterministic=det, split_k=split)
    torch.cuda.synchronize()
    return r


def _oracle(pass_name, a_bits, b_bits, rows=None, cols=None):
    fn = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[pass_name]
    return fn(a_bits, b_bits, rows=rows, cols=cols)


def _operands(pass_name, x, w, dy):
    return {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[pass_name]


def _assert_exact(out_t, ref, out_name):
    if out_name == "f32":
        np.testing.assert_array_equal(host_f64(out_t), ref)
    else:
        np.testing.assert_array_equal(host_bits(out_t), oracle.f64_to_bf16(ref))


# ---------------------------------------------------- exact-integer, bitwise --
# Shapes span several tiles of every tile size with ragged row tails; the planner
# picks 64-, 128- and 256-wide tiles across them.
INT_SHAPES = [
    (64, 1024, 4096),     # projection 4096->1024 at T = 64
    (333, 200, 264),      # ragged everywhere (T odd, N and K multiples of 8 only)
    (1, 8, 8),            # smallest
    (1025, 64, 512),      # 17 blocks of 64 tokens, last holds 1
    (700, 520, 136),
    (2100, 1280, 256),    # large enough for 256x256 tiles
]


@pytest.mark.parametrize("T,N,K", INT_SHAPES)
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("out_name", ["bf16", "f32"])
def test_exact_integer_bitwise(T, N, K, pass_name, out_name):
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=7, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    ref = _oracle(pass_name, a, b)
    da, db = dev_bf16(a), dev_bf16(b)
    for det, split in [(True, 0), (False, 0), (False, 1), (False, 2), (True, 3)]:
        out = _run(pass_name, da, db, OUT[out_name], det=det, split=split)
        _assert_exact(out, ref, out_name)


@pytest.mark.parametrize("T,N,K", [(4096, 4096, 1024), (16231, 12288, 4096)])
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_exact_integer_sampled_large(T, N, K, pass_name):
    """256x256 tiles at full size: exact-integer inputs, sampled positions."""
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=8, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    out = _run(pass_name, dev_bf16(a), dev_bf16(b), torch.float32)
    rows, cols = out.shape
    ii, jj = sample_positions(rows, cols, 3000, seed=1)
    ref = _oracle(pass_name, a, b, rows=ii, cols=jj)
    np.testing.assert_array_equal(host_f64(out)[ii, jj], ref)


# ------------------------------------------- projection 4096 -> 1024, T = 64 --
@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_small_projection_budget(seed, pass_name):
    x, w, dy = dpg_inputs.dense(64, 1024, 4096, seed_group=seed)
    a, b = _operands(pass_name, x, w, dy)
    ref = _oracle(pass_name, a, b)
    da, db = dev_bf16(a), dev_bf16(b)
    out = _run(pass_name, da, db, torch.bfloat16)
    rep = budgets.check_bf16(host_f64(out), ref)
    report("cfg1", pass_=pass_name, seed=seed, worst_ratio=rep["worst_ratio"], violations=rep["violations"])
    assert rep["ok"], rep
    for _ in range(3):
        again = _run(pass_name, da, db, torch.bfloat16)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))


# ----------------------------------------------------- FP32 router, BF16x3 --
@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("T", [64, 256, 1024])
@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_router_budget(T, op, seed):
    """Every element of every router output, seeds 0..9, in the deterministic
    mode, the split-K mode's own plan and a forced two-way split: the FP32
    budget against the exact product, and |GPU - c3| within Higham's bound for
    FP32 summation of the three products against the exact BF16x3 value."""
    E, H = 256, 4096
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=seed)
    fn = {"fwd": dpg.dpg_router_forward, "dgrad": dpg.dpg_router_dgrad, "wgrad": dpg.dpg_router_wgrad}[op]
    orc = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[op]
    a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]
    ref = orc(a, b)
    c3 = orc(a, b, mode="bf16x3")
    s = orc(a, b, mode="abs")
    R = {"fwd": H, "dgrad": E, "wgrad": T}[op]
    gamma = 3 * R * 2.0 ** -24
    da, db = dev_f32(a), dev_f32(b)
    for det, split in [(True, 0), (False, 0), (False, 2)]:
        out = fn(da, db, deterministic=det, split_k=split)
        torch.cuda.synchronize()
        got = host_f64(out)
        rep = budgets.check_f32(got, ref)
        bound_ratio = float(np.max(np.abs(got - c3) / (gamma * s + 1e-30)))
        report("cfg2", op=op, T=T, seed=seed, det=det, split=split, rel_fro=rep["rel_fro"],
               max_abs_ratio=rep["max_abs"] / (budgets.F32_MAX_ABS_REL * rep["max_ref"]),
               c3_bound_ratio=bound_ratio)
        assert rep["ok"], (det, split, rep)
        # against the exact BF16x3 value: only FP32 accumulation error remains
        assert bound_ratio <= 1.02, (det, split, bound_ratio)


def _top8(scores):
    """Indices of the 8 largest entries per row, larger first, ties to the
    lower index."""
    order = np.lexsort((np.arange(scores.shape[1])[None, :].repeat(scores.shape[0], 0), -scores), axis=1)
    return order[:, :8], order


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("T", [64, 256, 1024])
@pytest.mark.parametrize("det,split", [(True, 0), (False, 0)])
def test_router_top8_and_strict_filter(T, det, split, seed, record_property):
    """The router pages' stricter filter (relative Frobenius error <= 2e-6 and
    the same top-8 experts per token) is reported, not enforced, except that a
    token's top-8 set may differ from the FP64 one only where the FP64 gap
    between its 8th and 9th expert is within twice that row's largest error."""
    E, H = 256, 4096
    x, w, _ = dpg_inputs.router(T, E, H, seed_group=seed)
    got = host_f64(dpg.dpg_router_forward(dev_f32(x), dev_f32(w), deterministic=det, split_k=split))
    ref = oracle.forward(x, w)
    rel_fro = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    record_property("rel_fro", rel_fro)
    record_property("strict_filter_rel_fro_ok", rel_fro <= 2e-6)
    top_ref, order_ref = _top8(ref)
    top_got, _ = _top8(got)
    row_err = np.abs(got - ref).max(axis=1)
    mismatched = 0
    for t in range(T):
        if set(top_ref[t]) != set(top_got[t]):
            mismatched += 1
            gap = ref[t, order_ref[t, 7]] - ref[t, order_ref[t, 8]]
            assert gap <= 2 * row_err[t], (t, gap, row_err[t])
    record_property("top8_mismatched_tokens", mismatched)
    report("cfg2_strict", T=T, seed=seed, det=det, split=split, rel_fro=rel_fro, strict_ok=rel_fro <= 2e-6,
           top8_mismatched_tokens=mismatched)
    assert rel_fro <= 5e-5


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("det,split", [(True, 0), (False, 3)])
def test_router_exact_bf16x3(op, det, split):
    """a = hi + lo inputs: the GPU equals the exact three-product value (lo*lo
    dropped, hi*lo and lo*hi kept), bit for bit."""
    T, E, H = 96, 256, 1024
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=3, kind="exact")
    fn = {"fwd": dpg.dpg_router_forward, "dgrad": dpg.dpg_router_dgrad, "wgrad": dpg.dpg_router_wgrad}[op]
    orc = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[op]
    a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]
    out = fn(dev_f32(a), dev_f32(b), deterministic=det, split_k=split)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_f64(out), orc(a, b, mode="bf16x3"))


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("det,split", [(True, 0), (False, 3)])
def test_router_exact_bf16x3_pipelined(op, det, split):
    """T = H = 4096: every router pass runs the pipelined BF16x3 kernel
    (128x128 tiles, hi/lo planes split while staging); a = hi + lo inputs make
    the three-product sum exact, so sampled outputs equal the oracle's BF16x3
    value bit for bit."""
    T, E, H = 4096, 256, 4096
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=12, kind="exact")
    pass_id = {"fwd": 3, "dgrad": 4, "wgrad": 5}[op]
    plan = dpg.parse_plan(dpg.plan_describe(pass_id, T, E, H, torch.float32, det, split))
    assert plan["kernel"] == "pipelined" and plan["x3"] == "1", plan
    fn = {"fwd": dpg.dpg_router_forward, "dgrad": dpg.dpg_router_dgrad, "wgrad": dpg.dpg_router_wgrad}[op]
    orc = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[op]
    a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]
    out = fn(dev_f32(a), dev_f32(b), deterministic=det, split_k=split)
    torch.cuda.synchronize()
    rows, cols = out.shape
    ii, jj = sample_positions(rows, cols, 3000, seed=7)
    ref = orc(a, b, mode="bf16x3", rows=ii, cols=jj)
    np.testing.assert_array_equal(host_f64(out)[ii, jj], ref)


# ----------------------------------------- projection 4096 -> 12288, full size --
@pytest.fixture(scope="module")
def big_inputs():
    cache = {}

    def get(T, seed):
        if (T, seed) not in cache:
            cache.clear()
            x, w, dy = dpg_inputs.dense(T, 12288, 4096, seed_group=seed)
            cache[(T, seed)] = (x, w, dy, dev_bf16(x), dev_bf16(w), dev_bf16(dy))
        return cache[(T, seed)]
    return get


# seed 0 at both token counts, seeds 1..9 at 16384 (sampled outputs: a full
# FP64 reference is 1.6e12 multiply-adds per pass)
BIG_CASES = [(16384, 0), (16231, 0)] + [(16384, s) for s in range(1, 10)]


@pytest.mark.parametrize("T,seed", BIG_CASES)
def test_big_projection_sampled(big_inputs, T, seed):
    x, w, dy, dx_, dw_, ddy = big_inputs(T, seed)
    for pass_name, out_name in [("fwd", "bf16"), ("dgrad", "bf16"), ("dgrad", "f32"), ("wgrad", "bf16")]:
        a, b = _operands(pass_name, x, w, dy)
        da, db = _operands(pass_name, dx_, dw_, ddy)
        out = _run(pass_name, da, db, OUT[out_name])
        rows, cols = out.shape
        ii, jj = sample_positions(rows, cols, 4000, seed=T + seed)
        ref = _oracle(pass_name, a, b, rows=ii, cols=jj)
        got = host_f64(out[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
        rep = budgets.check(got, ref, out_name)
        report("cfg3", pass_=pass_name, out=out_name, T=T, seed=seed, samples=len(ii),
               **({"worst_ratio": rep["worst_ratio"]} if out_name == "bf16" else {"rel_fro": rep["rel_fro"]}))
        assert rep["ok"], (pass_name, out_name, rep)
        assert torch.isfinite(out.float()).all()
        if seed == 0:
            again = _run(pass_name, da, db, OUT[out_name])
            view = torch.int16 if out_name == "bf16" else torch.int32
            assert torch.equal(again.view(view), out.view(view))
        del out


# Whole outputs at full size, 4096 -> 12288 at T = 16384 and the ragged
# T = 16231 (last 64-token block of the weight gradient holds 39 tokens), in
# the launch configuration of the timed step (deterministic, planner's plan)
# and in the split-K / stream-K mode.  One operand of each pass is an integer matrix of
# rank 16 (the product of two integer factors with entries in -2..2), the
# other a full-rank integer matrix with entries in -3..3.  Every partial sum is
# an integer below 2**24, so any accumulation order is exact in FP32 and the
# whole output has a closed form at O(16) operations per element: the same
# product regrouped around the rank-16 factor (associativity of exact integer
# arithmetic), e.g. X W^T = (X V^T) U^T for W = U V.  The factor rows are
# pairwise distinct (checked), so a misplaced row, column or K tile changes
# some output element; BF16 outputs are compared with the nearest-even
# rounding of the exact value.
FULL_N, FULL_K, FULL_RANK = 12288, 4096, 16


def _low_rank_case(pass_name, T):
    N, K, R = FULL_N, FULL_K, FULL_RANK
    f = np.float64
    if pass_name == "fwd":                  # Y = X W^T, W = U V
        x = dpg_inputs.int_values((T, K), -3, 3, 21, 0)
        u, v = dpg_inputs.int_factors(N, K, R, 21, 1)
        a, b, fac = x, u.astype(f) @ v.astype(f), u
        ref = (x.astype(f) @ v.T.astype(f)) @ u.T.astype(f)
    elif pass_name == "dgrad":              # dX = dY W, W = U V
        dy = dpg_inputs.int_values((T, N), -3, 3, 21, 2)
        u, v = dpg_inputs.int_factors(N, K, R, 21, 1)
        a, b, fac = dy, u.astype(f) @ v.astype(f), v.T
        ref = (dy.astype(f) @ u.astype(f)) @ v.astype(f)
    else:                                   # dW = dY^T X, X = P Q
        dy = dpg_inputs.int_values((T, N), -3, 3, 21, 2)
        p, q = dpg_inputs.int_factors(T, K, R, 21, 3)
        a, b, fac = dy, p.astype(f) @ q.astype(f), q.T
        ref = (dy.T.astype(f) @ p.astype(f)) @ q.astype(f)
    # distinct factor rows: output columns (fwd) / K columns (dgrad, wgrad) differ
    assert np.unique(fac, axis=0).shape[0] == fac.shape[0]
    assert np.abs(ref).max() < 2.0 ** 24
    return dpg_inputs.ints_to_bf16_bits(a), dpg_inputs.ints_to_bf16_bits(b), ref


@pytest.mark.parametrize("T", [16384, 16231])
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_big_projection_whole_output_exact(pass_name, T):
    a, b, ref = _low_rank_case(pass_name, T)
    da, db = dev_bf16(a), dev_bf16(b)
    del a, b
    ref32 = ref.astype(np.float32)
    ref_bits = oracle.f64_to_bf16(ref)
    del ref
    for det, split in [(True, 0), (False, 0)]:
        out = _run(pass_name, da, db, torch.float32, det=det, split=split)
        got = out.cpu().numpy()
        bad = int(np.count_nonzero(got != ref32))
        report("cfg3_whole", pass_=pass_name, T=T, out="f32", det=det, mismatches=bad, elements=got.size)
        assert bad == 0, (pass_name, det, bad)
        del out, got
        out = _run(pass_name, da, db, torch.bfloat16, det=det, split=split)
        got = host_bits(out)
        bad = int(np.count_nonzero(got != ref_bits))
        report("cfg3_whole", pass_=pass_name, T=T, out="bf16", det=det, mismatches=bad, elements=got.size)
        assert bad == 0, (pass_name, det, bad)
        del out, got


# ---------------------------------------------------- skinny-N weight gradient --
SKINNY = [(4096, 64), (4096, 128), (5120, 48), (5120, 64)]
SKINNY_T = [1025, 4031, 16173, 16384, 65537]


@pytest.fixture(scope="module")
def skinny_x():
    cache = {}

    def get(T, K, seed):
        if (T, K, seed) not in cache:
            cache.clear()
            x = dpg_inputs.normal_bf16((T, K), 1.0, seed, 0)
            cache[(T, K, seed)] = (x, dev_bf16(x))
        return cache[(T, K, seed)]
    return get


def _skinny_check(skinny_x, T, K, N, seed, outs, modes):
    """Every element of dW against the full FP64 oracle, for each output dtype
    and mode; reruns bitwise equal.  Reports each case's margin."""
    x, dx_ = skinny_x(T, K, seed)
    dy = dpg_inputs.normal_bf16((T, N), 1.0, seed, 2)
    ddy = dev_bf16(dy)
    ref = oracle.wgrad(dy, x)
    for out_name in outs:
        for det, split in modes:
            out = _run("wgrad", ddy, dx_, OUT[out_name], det=det, split=split)
            rep = budgets.check(host_f64(out), ref, out_name)
            report("cfg4", shape="%d->%d" % (K, N), T=T, seed=seed, out=out_name, det=det, split=split,
                   **({"worst_ratio": rep["worst_ratio"], "violations": rep["violations"]} if out_name == "bf16"
                      else {"rel_fro": rep["rel_fro"],
                            "max_abs_ratio": rep["max_abs"] / (budgets.F32_MAX_ABS_REL * rep["max_ref"])}))
            assert rep["ok"], (out_name, det, split, rep)
            again = _run("wgrad", ddy, dx_, OUT[out_name], det=det, split=split)
            assert torch.equal(again.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("T", SKINNY_T)
@pytest.mark.parametrize("K,N", SKINNY)
def test_skinny_wgrad(skinny_x, T, K, N):
    """All 20 (K -> N, T) points, seed 0: BF16 and FP32 output in the
    deterministic mode and with one and two forced splits, full output."""
    _skinny_check(skinny_x, T, K, N, 0, ("bf16", "f32"), [(True, 0), (False, 1), (False, 2)])


@pytest.mark.parametrize("seed", range(1, 10))
@pytest.mark.parametrize("T", [16173, 65537])
@pytest.mark.parametrize("K,N", SKINNY)
def test_skinny_wgrad_seeds(skinny_x, T, K, N, seed):
    """Seeds 1..9 at the long odd token counts, BF16 output (the budget the
    weight-gradient page reports misses for at large T), deterministic mode,
    every element."""
    _skinny_check(skinny_x, T, K, N, seed, ("bf16",), [(True, 0)])


# Exact-integer inputs through the skinny kernels: one and two 64-row blocks of
# dW with 128-column units (auto plans with enough units: operands straight from
# registers for one row block, fetched straight into LDS for two) and 64-column
# units (forced small split counts: the LDS-staged kernel for one row block, the
# LDS-fetching kernel for two), ragged token tails.
# (The planner's choices for these shapes are checked on the CPU.)
SKINNY_EXACT = [
    (4031, 128, 4096),   # two row blocks; 63 token blocks, last holds 63
    (16384, 48, 5120),   # one row block, ragged N inside the block
    (1025, 104, 1024),   # two row blocks, N ragged; 17 token blocks, last holds 1
    (16384, 128, 4096),  # two row blocks, 128-column units
    (65537, 104, 3968),  # two row blocks, N ragged, 31 units of 128 columns, 8 splits
    (16400, 40, 1000),   # one row block, N ragged, last 128-column unit partial, 32 splits of
                         # 9 or 8 token blocks, last block 16 tokens (29 16-token steps over 8 waves)
    (16400, 104, 1000),  # the same with two row blocks, N ragged, 9 or 8 blocks a split
]


@pytest.mark.parametrize("T,N,K", SKINNY_EXACT)
def test_skinny_exact_integer(T, N, K):
    x, _, dy = dpg_inputs.dense(T, N, K, seed_group=9, kind="int")
    ddy, dx_ = dev_bf16(dy), dev_bf16(x)
    ii, jj = sample_positions(N, K, 3000, seed=T)
    ref = oracle.wgrad(dy, x, rows=ii, cols=jj)
    for det, split in [(True, 0), (False, 1), (False, 2), (True, 3)]:
        for out_name in ("f32", "bf16"):
            plan = dpg.parse_plan(dpg.plan_describe(dpg.PASS_WGRAD, T, N, K, OUT[out_name], det, split))
            assert plan["kernel"] == "skinny", plan
            out = _run("wgrad", ddy, dx_, OUT[out_name], det=det, split=split)
            got = out[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()]
            if out_name == "f32":
                np.testing.assert_array_equal(host_f64(got), ref)
            else:
                np.testing.assert_array_equal(host_bits(got), oracle.f64_to_bf16(ref))


# Skinny weight gradients through row strides wider than the rows: dY and X
# are column slices of wider buffers, dW is written into a column slice of a
# NaN-filled buffer.  The planner's plans take the register-direct kernel
# (16400x40x1000), the LDS-fetching kernel (16384x128x4096) and the LDS-staged
# kernel (4031x64x4096, and the N <= 64 shapes with the forced split count of
# 2; 16384x128x4096 then takes the LDS-fetching kernel's 64-column form).
@pytest.mark.parametrize("T,N,K", [(16400, 40, 1000), (16384, 128, 4096), (4031, 64, 4096)])
def test_skinny_padded_strides(T, N, K):
    x, _, dy = dpg_inputs.dense(T, N, K, seed_group=12, kind="int")

    def padded(bits, extra):
        t = torch.zeros((bits.shape[0], bits.shape[1] + extra), dtype=torch.bfloat16, device="cuda")
        t[:, :bits.shape[1]] = dev_bf16(bits)
        return t[:, :bits.shape[1]]
    X, DY = padded(x, 72), padded(dy, 24)
    assert X.stride(0) == K + 72 and DY.stride(0) == N + 24
    ii, jj = sample_positions(N, K, 3000, seed=T + 1)
    ref = oracle.wgrad(dy, x, rows=ii, cols=jj)
    ti, tj = torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()
    for det, split in [(True, 0), (False, 2)]:
        plan = dpg.parse_plan(dpg.plan_describe(dpg.PASS_WGRAD, T, N, K, torch.float32, det, split))
        assert plan["kernel"] == "skinny", plan
        big = torch.full((N + 2, K + 40), float("nan"), dtype=torch.float32, device="cuda")
        view = big[1:N + 1, 8:8 + K]
        _run("wgrad", DY, X, torch.float32, det=det, split=split, out=view)
        np.testing.assert_array_equal(host_f64(view[ti, tj]), ref)
        mask = torch.ones_like(big, dtype=torch.bool)
        mask[1:N + 1, 8:8 + K] = False
        assert torch.isnan(big[mask]).all()


# ------------------------------------------- checkpointed step 2fwd + bwd --
@pytest.mark.parametrize("N", [1024, 512])
def test_checkpointed_step(N):
    T, K = 16384, 4096
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=0)
    dx_, dw_, ddy = dev_bf16(x), dev_bf16(w), dev_bf16(dy)

    def step():
        y1 = dpg.dpg_forward(dx_, dw_, out_dtype=torch.float32)
        y2 = dpg.dpg_forward(dx_, dw_, out_dtype=torch.float32)
        gx = dpg.dpg_dgrad(ddy, dw_, out_dtype=torch.float32)
        gw = dpg.dpg_wgrad(ddy, dx_, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return y1, y2, gx, gw

    y1, y2, gx, gw = step()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    for name, out, a, b in [("fwd", y1, x, w), ("dgrad", gx, dy, w), ("wgrad", gw, dy, x)]:
        ref = _oracle(name, a, b)
        rep = budgets.check_f32(host_f64(out), ref)
        report("cfg5", N=N, pass_=name, rel_fro=rep["rel_fro"],
               max_abs_ratio=rep["max_abs"] / (budgets.F32_MAX_ABS_REL * rep["max_ref"]))
        assert rep["ok"], (name, rep)
        del ref
    z = step()
    for u, v in zip((y1, y2, gx, gw), z):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))


# ---------------------------------------------------------- determinism --
def test_twenty_reruns_bitwise():
    T, N, K = 4031, 128, 4096
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=1)
    dx_, ddy = dev_bf16(x), dev_bf16(dy)
    for det, split in [(True, 0), (False, 2)]:
        first = _run("wgrad", ddy, dx_, torch.float32, det=det, split=split)
        for _ in range(20):
            again = _run("wgrad", ddy, dx_, torch.float32, det=det, split=split)
            assert torch.equal(again.view(torch.int32), first.view(torch.int32))
    xr, wr, dyr = dpg_inputs.router(256, 256, 4096, seed_group=1)
    a, b = dev_f32(xr), dev_f32(wr)
    first = dpg.dpg_router_forward(a, b, deterministic=False, split_k=4)
    for _ in range(20):
        again = dpg.dpg_router_forward(a, b, deterministic=False, split_k=4)
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))


# One point of every workload, 20 reruns each, in each mode the workload
# names (the pages qualify a point with repeated runs): every rerun must be
# bitwise equal to the first.  Between reruns a 256 MB fill runs, so the
# caches hold other data each time.
RERUN_CASES = [
    ("cfg1", "fwd", (64, 1024, 4096), "bf16", [(True, 0)]),
    ("cfg1", "dgrad", (64, 1024, 4096), "bf16", [(True, 0)]),
    ("cfg1", "wgrad", (64, 1024, 4096), "bf16", [(True, 0)]),
    ("cfg2", "fwd", (256, 256, 4096), "router", [(True, 0), (False, 0)]),
    ("cfg2", "dgrad", (1024, 256, 4096), "router", [(True, 0), (False, 0)]),
    ("cfg2", "wgrad", (64, 256, 4096), "router", [(True, 0), (False, 0)]),
    ("cfg3", "fwd", (16384, 12288, 4096), "bf16", [(True, 0)]),
    ("cfg3", "dgrad", (16231, 12288, 4096), "f32", [(True, 0)]),
    ("cfg3", "wgrad", (16384, 12288, 4096), "bf16", [(True, 0)]),
    ("cfg4", "wgrad", (16173, 64, 4096), "bf16", [(True, 0), (False, 1), (False, 2)]),
    ("cfg4", "wgrad", (65537, 48, 5120), "f32", [(True, 0), (False, 1), (False, 2)]),
    ("cfg5", "fwd", (16384, 1024, 4096), "f32", [(True, 0)]),
    ("cfg5", "dgrad", (16384, 512, 4096), "f32", [(True, 0)]),
    ("cfg5", "wgrad", (16384, 1024, 4096), "f32", [(True, 0)]),
]


@pytest.mark.parametrize("cfg,pass_name,shape,out_name,modes", RERUN_CASES,
                         ids=["%s-%s-%d" % (c[0], c[1], c[2][0]) for c in RERUN_CASES])
def test_twenty_reruns_every_workload(cfg, pass_name, shape, out_name, modes):
    T, N, K = shape
    fill = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
    if out_name == "router":
        x, w, dy = dpg_inputs.router(T, N, K, seed_group=3)
        a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[pass_name]
        da, db = dev_f32(a), dev_f32(b)
        fn = {"fwd": dpg.dpg_router_forward, "dgrad": dpg.dpg_router_dgrad, "wgrad": dpg.dpg_router_wgrad}[pass_name]
        call = lambda det, split: fn(da, db, deterministic=det, split_k=split)
    else:
        x, w, dy = dpg_inputs.dense(T, N, K, seed_group=3)
        a, b = _operands(pass_name, x, w, dy)
        da, db = dev_bf16(a), dev_bf16(b)
        del x, w, dy, a, b
        call = lambda det, split: _run(pass_name, da, db, OUT[out_name], det=det, split=split)
    for det, split in modes:
        first = call(det, split)
        view = torch.int16 if first.dtype == torch.bfloat16 else torch.int32
        for r in range(20):
            fill.fill_(float(r))
            again = call(det, split)
            torch.cuda.synchronize()
            assert torch.equal(again.view(view), first.view(view)), (cfg, pass_name, shape, det, split, r)
            del again
        del first


def test_other_stream_and_graph_replay():
    T, N, K = 1025, 64, 4096
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=2)
    dx_, ddy = dev_bf16(x), dev_bf16(dy)
    ref = _run("wgrad", ddy, dx_, torch.float32, det=False, split=2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = dpg.dpg_wgrad(ddy, dx_, out_dtype=torch.float32, deterministic=False, split_k=2)
    s.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # HIP graph: capture the two launches (GEMM + fixed-order reduce) once
    out = torch.empty_like(ref)
    ws = torch.empty(dpg.workspace_size(dpg.PASS_WGRAD, T, N, K, torch.float32, False, 2),
                     dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dpg.dpg_wgrad(ddy, dx_, out=out, deterministic=False, split_k=2, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), i
        _run("fwd", dx_, dev_bf16(w), torch.bfloat16)  # eager work between replays


# --------------------------------------------------------- output layout --
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("out_name", ["bf16", "f32"])
def test_padded_output_untouched(pass_name, out_name):
    """Write into a column slice of a wider NaN-filled buffer: the slice holds
    the result, everything outside it stays NaN."""
    T, N, K = 197, 136, 264
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=4, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    ref = _oracle(pass_name, a, b)
    rows, cols = ref.shape
    big = torch.full((rows + 3, cols + 40), float("nan"), dtype=OUT[out_name], device="cuda")
    view = big[1:rows + 1, 16:16 + cols]
    _run(pass_name, dev_bf16(a), dev_bf16(b), OUT[out_name], out=view, det=False, split=2)
    _assert_exact(view, ref, out_name)
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[1:rows + 1, 16:16 + cols] = False
    assert torch.isnan(big.float()[mask]).all()


def test_empty_reductions_write_zeros():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((32, 64), float("nan"), device="cuda")
    dpg.dpg_wgrad(dy, x, out=dw)
    torch.cuda.synchronize()
    assert torch.equal(dw, torch.zeros_like(dw))
    y = dpg.dpg_forward(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda"))
    assert y.shape == (0, 16)


# --------------------------------------- leading dimensions of 2^22 and more --
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("log2_ld", [22, 23])
def test_huge_leading_dimension(pass_name, log2_ld):
    """Row strides of 2^22 elements and more leave the pipelined kernel, and
    of 2^23 and more the skinny kernel (32-bit tile offsets), for the generic
    kernel (64-bit addressing); exact-integer inputs, bit for bit."""
    T, N, K = 5, 64, 256
    big = (1 << log2_ld) + 64
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=11, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    ref = _oracle(pass_name, a, b)

    def padded(bits):
        t = torch.zeros((bits.shape[0], big), dtype=torch.bfloat16, device="cuda")
        t[:, :bits.shape[1]] = dev_bf16(bits)
        return t[:, :bits.shape[1]]
    A, B = padded(a), padded(b)
    assert A.stride(0) == big and B.stride(0) == big
    for det, split in [(True, 0), (False, 2)]:
        out = _run(pass_name, A, B, torch.float32, det=det, split=split)
        np.testing.assert_array_equal(host_f64(out), ref)
