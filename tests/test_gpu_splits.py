"""Forced split counts, K tails and wide row strides through the C ABI (GPU).

Exact-integer inputs ({-3..3}/4, exact in BF16) make every FP32 partial sum
exact, so any K partition must give the oracle's value bit for bit (FP32 out)
or its nearest-even rounding (BF16 out); BF16x3-exact router inputs (a = hi +
lo) make the three-product sum exact likewise.  Each case first checks, on the
host, which plan the library runs.
"""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from tests.gpu_util import dev_bf16, dev_f32, host_bits, host_f64, sample_positions

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

PASS = {"fwd": dpg.PASS_FORWARD, "dgrad": dpg.PASS_DGRAD, "wgrad": dpg.PASS_WGRAD}
RUN = {"fwd": dpg.dpg_forward, "dgrad": dpg.dpg_dgrad, "wgrad": dpg.dpg_wgrad}
ORC = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}


def _operands(pass_name, x, w, dy):
    return {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[pass_name]


def _blocks(pass_name, T, N, K):
    return -(-{"fwd": K, "dgrad": N, "wgrad": T}[pass_name] // 64)


# (pass, T, N, K): 64+ reduction blocks so that 63 splits stay 63; the weight
# gradient both as a GEMM (N > 128) and as a skinny stream (N <= 128)
SPLIT_SHAPES = [("fwd", 333, 200, 4096), ("dgrad", 333, 4096, 264), ("wgrad", 4100, 200, 264),
                ("wgrad", 4100, 64, 1032), ("wgrad", 4100, 104, 520)]


@pytest.mark.parametrize("pass_name,T,N,K", SPLIT_SHAPES)
@pytest.mark.parametrize("split", [5, 7, 63])
def test_forced_split_exact(pass_name, T, N, K, split):
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=21, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    ref = ORC[pass_name](a, b)
    da, db = dev_bf16(a), dev_bf16(b)
    for det in (True, False):
        for out_dtype in (torch.float32, torch.bfloat16):
            p = dpg.parse_plan(dpg.plan_describe(PASS[pass_name], T, N, K, out_dtype, det, split))
            assert int(p["splits"]) == min(split, _blocks(pass_name, T, N, K)), p
            out = RUN[pass_name](da, db, out_dtype=out_dtype, deterministic=det, split_k=split)
            torch.cuda.synchronize()
            if out_dtype == torch.float32:
                np.testing.assert_array_equal(host_f64(out), ref)
            else:
                np.testing.assert_array_equal(host_bits(out), oracle.f64_to_bf16(ref))
            again = RUN[pass_name](da, db, out_dtype=out_dtype, deterministic=det, split_k=split)
            torch.cuda.synchronize()
            assert torch.equal(again.view(torch.int16), out.view(torch.int16))


ROUTER = {"fwd": (dpg.PASS_ROUTER_FORWARD, dpg.dpg_router_forward),
          "dgrad": (dpg.PASS_ROUTER_DGRAD, dpg.dpg_router_dgrad),
          "wgrad": (dpg.PASS_ROUTER_WGRAD, dpg.dpg_router_wgrad)}


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("split", [5, 7, 63])
@pytest.mark.parametrize("T", [96, 4096])
def test_router_forced_split_exact(op, split, T):
    """BF16x3-exact inputs, forced split counts: the GPU equals the exact
    three-product value bit for bit (generic 64x64 kernel at T = 96, the
    pipelined BF16x3 kernel at T = 4096; sampled outputs there)."""
    E, H = 256, 4096
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=22, kind="exact")
    pass_id, fn = ROUTER[op]
    a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]
    R = {"fwd": H, "dgrad": E, "wgrad": T}[op]
    for det in (True, False):
        p = dpg.parse_plan(dpg.plan_describe(pass_id, T, E, H, torch.float32, det, split))
        assert p["x3"] == "1" and int(p["splits"]) == min(split, -(-R // 64)), p
        out = fn(dev_f32(a), dev_f32(b), deterministic=det, split_k=split)
        torch.cuda.synchronize()
        got = host_f64(out)
        if T <= 256:
            np.testing.assert_array_equal(got, ORC[op](a, b, mode="bf16x3"))
        else:
            ii, jj = sample_positions(got.shape[0], got.shape[1], 2000, seed=split)
            np.testing.assert_array_equal(got[ii, jj], ORC[op](a, b, mode="bf16x3", rows=ii, cols=jj))


@pytest.mark.parametrize("pass_name,T,N,K", [("fwd", 4096, 4096, 1032), ("dgrad", 4096, 1032, 4096),
                                             ("fwd", 16384, 12288, 4104)])
def test_k_tail_generic_kernel_large(pass_name, T, N, K):
    """K-major reductions that are not a multiple of 64 run the generic 64x64
    kernel (the only generic tile compiled) at large shapes; exact-integer
    inputs, sampled outputs bit for bit, ragged edges included."""
    p = dpg.parse_plan(dpg.plan_describe(PASS[pass_name], T, N, K, torch.float32, True, 0))
    assert p["kernel"] == "generic" and p["tile"] == "64x64x64", p
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=23, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    da, db = dev_bf16(a), dev_bf16(b)
    for det, split in [(True, 0), (False, 3)]:
        out = RUN[pass_name](da, db, out_dtype=torch.float32, deterministic=det, split_k=split)
        torch.cuda.synchronize()
        rows, cols = out.shape
        ii, jj = sample_positions(rows, cols, 3000, seed=K)
        ref = ORC[pass_name](a, b, rows=ii, cols=jj)
        np.testing.assert_array_equal(host_f64(out)[ii, jj], ref)


@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_wide_stride_large_shape(pass_name):
    """Row strides just above 2^22 elements at a shape whose plan uses the
    pipelined kernel (128x128 tiles): the launch runs the same K partition on
    the generic 64x64 kernel.  Exact-integer inputs, sampled outputs (edges
    included) bit for bit, deterministic and two-split plans."""
    T, N, K = 1024, 2048, 2048
    big = (1 << 22) + 64
    p = dpg.parse_plan(dpg.plan_describe(PASS[pass_name], T, N, K, torch.float32, True, 0))
    assert p["kernel"] == "pipelined", p
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=24, kind="int")
    a, b = _operands(pass_name, x, w, dy)
    rows, cols = {"fwd": (T, N), "dgrad": (T, K), "wgrad": (N, K)}[pass_name]
    ii, jj = sample_positions(rows, cols, 3000, seed=5)
    ref = ORC[pass_name](a, b, rows=ii, cols=jj)

    def padded(bits):
        t = torch.zeros((bits.shape[0], big), dtype=torch.bfloat16, device="cuda")
        t[:, :bits.shape[1]] = dev_bf16(bits)
        return t[:, :bits.shape[1]]
    A, B = padded(a), padded(b)
    assert A.stride(0) == big
    for det, split in [(True, 0), (False, 2)]:
        out = RUN[pass_name](A, B, out_dtype=torch.float32, deterministic=det, split_k=split)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_f64(out)[ii, jj], ref)
    del A, B
    torch.cuda.empty_cache()
