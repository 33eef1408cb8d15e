"""The router's FP32 fused-multiply-add kernel (dpg_set_router_arithmetic
'fp32') through the C ABI, against the FP64 oracle (GPU).

Small-integer FP32 inputs ({-3..3}/4) make every product and partial sum exact,
so the kernel must equal the oracle bit for bit, split reductions included.
Config-2 inputs (router page: 256 experts, hidden 4096, T = 64 / 256 / 1024)
must meet the FP32 budget, stay within the bound of plain FP32 summation
against the exact result (each FMA and each split addition rounds once), and
repeat bitwise.  The router pages' stricter filter is reported (PARITY)."""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import budgets
from tests.gpu_util import dev_f32, host_f64, report

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

OPS = {"fwd": (dpg.PASS_ROUTER_FORWARD, dpg.dpg_router_forward, oracle.forward),
       "dgrad": (dpg.PASS_ROUTER_DGRAD, dpg.dpg_router_dgrad, oracle.dgrad),
       "wgrad": (dpg.PASS_ROUTER_WGRAD, dpg.dpg_router_wgrad, oracle.wgrad)}


@pytest.fixture(autouse=True)
def fp32_router():
    prev = dpg.set_router_arithmetic("fp32")
    yield
    dpg.set_router_arithmetic(prev)


def _operands(op, x, w, dy):
    return {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("T,H", [(64, 4096), (333, 1032), (1024, 4096)])
def test_fp32_router_exact(op, T, H):
    E = 256
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=41, kind="int")
    pass_id, fn, orc = OPS[op]
    a, b = _operands(op, x, w, dy)
    ref = orc(a, b)
    da, db = dev_f32(a), dev_f32(b)
    for det, split in [(True, 0), (False, 0), (True, 1), (False, 3), (True, 7)]:
        p = dpg.parse_plan(dpg.plan_describe(pass_id, T, E, H, torch.float32, det, split))
        assert p["kernel"] == "ffma" and p["arith"] == "fp32fma", p
        out = fn(da, db, deterministic=det, split_k=split)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_f64(out), ref)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("T", [64, 256, 1024])
@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_fp32_router_budget(op, T, seed):
    E, H = 256, 4096
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=seed)
    pass_id, fn, orc = OPS[op]
    a, b = _operands(op, x, w, dy)
    ref = orc(a, b)
    s = orc(a, b, mode="abs")
    R = {"fwd": H, "dgrad": E, "wgrad": T}[op]
    da, db = dev_f32(a), dev_f32(b)
    for det, split in [(True, 0), (False, 0), (False, 4)]:
        p = dpg.parse_plan(dpg.plan_describe(pass_id, T, E, H, torch.float32, det, split))
        S = int(p["splits"])
        out = fn(da, db, deterministic=det, split_k=split)
        torch.cuda.synchronize()
        got = host_f64(out)
        rep = budgets.check_f32(got, ref)
        # one rounding per FMA along a split's range, one per split addition
        gamma = (R + S) * 2.0 ** -24
        bound_ratio = float(np.max(np.abs(got - ref) / (gamma * s + 1e-30)))
        report("cfg2_fp32fma", op=op, T=T, seed=seed, det=det, split=split, splits=S, rel_fro=rep["rel_fro"],
               strict_rel_fro_ok=rep["rel_fro"] <= 2e-6, bound_ratio=bound_ratio)
        assert rep["ok"], rep
        assert bound_ratio <= 1.0, bound_ratio
        for _ in range(3):
            again = fn(da, db, deterministic=det, split_k=split)
            torch.cuda.synchronize()
            assert torch.equal(again.view(torch.int32), out.view(torch.int32))
