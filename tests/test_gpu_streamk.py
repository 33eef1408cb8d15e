"""Stream-K plans (split-K mode, deterministic=False) through the C ABI (GPU).

For shapes whose tile count leaves a partial last round the planner takes
stream-K: whole rounds run data-parallel, the K iterations of the remaining
tiles are cut into one even range per workgroup, and tiles that ranges share
are summed by a fix-up kernel in range order.  Exact-integer inputs make
every plan's result exact, so the stream-K output must equal the oracle at
sampled positions and the deterministic plan's output at every position, bit
for bit; random inputs must meet the budgets and repeat bitwise."""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import budgets
from tests.gpu_util import dev_bf16, host_bits, host_f64, report, sample_positions

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

PASS = {"fwd": dpg.PASS_FORWARD, "dgrad": dpg.PASS_DGRAD, "wgrad": dpg.PASS_WGRAD}
RUN = {"fwd": dpg.dpg_forward, "dgrad": dpg.dpg_dgrad, "wgrad": dpg.dpg_wgrad}
ORC = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}
OUT = {"bf16": torch.bfloat16, "f32": torch.float32}

# (pass, T, N, K, tile): 272 tiles of 256x256 (one data-parallel round and 16
# tail tiles, each shared by 16 workgroups), 528 tiles (two rounds + 16), 306
# tiles at K = 8192 (50 tail tiles), and the MN-major layouts
SK_CASES = [("fwd", 4352, 4096, 4096, "256x256x64", ("f32", "bf16")),
            ("fwd", 8448, 4096, 4096, "256x256x64", ("f32", "bf16")),
            ("dgrad", 4352, 4352, 4096, "256x256x64", ("f32", "bf16")),
            ("wgrad", 4352, 4352, 4096, "256x256x64", ("f32", "bf16")),
            ("fwd", 4608, 4352, 8192, "256x256x64", ("f32", "bf16"))]


def _operands(pass_name, x, w, dy):
    return {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[pass_name]


@pytest.mark.parametrize("pass_name,T,N,K,tile,outs", SK_CASES)
def test_streamk_exact(pass_name, T, N, K, tile, outs):
    for out_name in outs:
        p = dpg.parse_plan(dpg.plan_describe(PASS[pass_name], T, N, K, OUT[out_name], False, 0))
        assert p["streamk"] == "1" and p["tile"] == tile, p
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=51, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    da, db = dev_bf16(a), dev_bf16(b)
    for out_name in outs:
        sk = RUN[pass_name](da, db, out_dtype=OUT[out_name], deterministic=False)
        det = RUN[pass_name](da, db, out_dtype=OUT[out_name], deterministic=True)
        torch.cuda.synchronize()
        view = torch.int32 if out_name == "f32" else torch.int16
        assert torch.equal(sk.view(view), det.view(view))
        rows, cols = sk.shape
        ii, jj = sample_positions(rows, cols, 3000, seed=T + N)
        ref = ORC[pass_name](a, b, rows=ii, cols=jj)
        if out_name == "f32":
            np.testing.assert_array_equal(host_f64(sk)[ii, jj], ref)
        else:
            np.testing.assert_array_equal(host_bits(sk)[ii, jj], oracle.f64_to_bf16(ref))


@pytest.mark.parametrize("pass_name,T,N,K,tile,outs", SK_CASES[:2] + SK_CASES[4:])
def test_streamk_budget_and_reruns(pass_name, T, N, K, tile, outs):
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=52)
    a, b = _operands(pass_name, x, w, dy)
    da, db = dev_bf16(a), dev_bf16(b)
    od = OUT[outs[-1]]
    assert dpg.parse_plan(dpg.plan_describe(PASS[pass_name], T, N, K, od, False, 0))["streamk"] == "1"
    out = RUN[pass_name](da, db, out_dtype=od, deterministic=False)
    torch.cuda.synchronize()
    rows, cols = out.shape
    ii, jj = sample_positions(rows, cols, 4000, seed=7)
    ref = ORC[pass_name](a, b, rows=ii, cols=jj)
    rep = budgets.check(host_f64(out)[ii, jj], ref, outs[-1])
    report("streamk", pass_=pass_name, T=T, N=N, K=K, out=outs[-1],
           **({"worst_ratio": rep["worst_ratio"]} if outs[-1] == "bf16" else {"rel_fro": rep["rel_fro"]}))
    assert rep["ok"], rep
    view = torch.int16 if outs[-1] == "bf16" else torch.int32
    for _ in range(5):
        again = RUN[pass_name](da, db, out_dtype=od, deterministic=False)
        torch.cuda.synchronize()
        assert torch.equal(again.view(view), out.view(view))
