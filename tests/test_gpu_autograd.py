"""The training wrappers over the C ABI (GPU): autograd projection and router
gradients equal the direct entry-point calls bit for bit and meet the oracle's
budgets; the captured checkpointed step replays bitwise equal to eager calls."""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import budgets
from tests.gpu_util import dev_bf16, dev_f32, host_bits, host_f64

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
from deterministic_bf16_projection_amd import autograd as dag  # noqa: E402


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("lead", [(200,), (2, 100)])
def test_projection_autograd_matches_entry_points(lead):
    T, N, K = int(np.prod(lead)), 264, 512
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=4)
    X = dev_bf16(x).reshape(*lead, K).requires_grad_(True)
    W = dev_bf16(w).requires_grad_(True)
    DY = dev_bf16(dy)
    y = dag.projection(X, W)
    assert y.shape == (*lead, N) and y.dtype == torch.bfloat16
    y.backward(DY.reshape(*lead, N))
    torch.cuda.synchronize()
    X2, W2 = X.detach().reshape(T, K), W.detach()
    assert torch.equal(_bits(y.detach().reshape(T, N)), _bits(dpg.dpg_forward(X2, W2)))
    assert torch.equal(_bits(X.grad.reshape(T, K)), _bits(dpg.dpg_dgrad(DY, W2)))
    assert torch.equal(_bits(W.grad), _bits(dpg.dpg_wgrad(DY, X2)))
    for got, ref in [(X.grad.reshape(T, K), oracle.dgrad(dy, w)), (W.grad, oracle.wgrad(dy, x))]:
        rep = budgets.check_bf16(host_f64(got), ref)
        assert rep["ok"], rep


def test_router_autograd_matches_entry_points():
    T, E, H = 96, 256, 1024
    x, w, dy = dpg_inputs.router(T, E, H, seed_group=5)
    X = dev_f32(x).requires_grad_(True)
    W = dev_f32(w).requires_grad_(True)
    DY = dev_f32(dy)
    y = dag.router_gating(X, W)
    y.backward(DY)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y.detach()), _bits(dpg.dpg_router_forward(X.detach(), W.detach())))
    assert torch.equal(_bits(X.grad), _bits(dpg.dpg_router_dgrad(DY, W.detach())))
    assert torch.equal(_bits(W.grad), _bits(dpg.dpg_router_wgrad(DY, X.detach())))
    rep = budgets.check_f32(host_f64(W.grad), oracle.wgrad(dy, x))
    assert rep["ok"], rep


def test_deterministic_switch_forces_deterministic_plans():
    T, N, K = 64, 1024, 4096
    x, w, _ = dpg_inputs.dense(T, N, K, seed_group=6)
    X, W = dev_bf16(x), dev_bf16(w)
    ref = dpg.dpg_forward(X, W, deterministic=True)
    prev = torch.are_deterministic_algorithms_enabled()
    try:
        torch.use_deterministic_algorithms(True, warn_only=True)
        y = dag.projection(X, W, deterministic=False)
    finally:
        torch.use_deterministic_algorithms(prev)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(ref))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_checkpointed_step_graph_replays(out_dtype):
    T, N, K = 2048, 512, 1024
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=7)
    step = dag.CheckpointedStep(dev_bf16(x), dev_bf16(w), dev_bf16(dy), out_dtype=out_dtype)
    eager = [t.clone() for t in step.eager()]
    torch.cuda.synchronize()
    assert torch.equal(_bits(eager[0]), _bits(eager[1]))  # the recomputed forward equals the first
    for _ in range(3):
        got = step.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, eager):
            assert torch.equal(_bits(a), _bits(b))
        # eager work on the same buffers between replays
        step.eager()
        torch.cuda.synchronize()
    # new inputs copied in place are picked up by the graph
    x2 = dpg_inputs.normal_bf16((T, K), 1.0, 8, 0)
    step.x.copy_(dev_bf16(x2))
    y = step.replay()[0]
    torch.cuda.synchronize()
    ref = oracle.forward(x2, w)
    rep = budgets.check(host_f64(y), ref, "f32" if out_dtype == torch.float32 else "bf16")
    assert rep["ok"], rep


def test_projection_fp32_gradient_rounding_is_explicit():
    """With an FP32 forward output the incoming gradient is FP32: backward
    refuses it unless round_grad_to_bf16=True, which equals rounding it to BF16
    by hand before the gradient entry points."""
    T, N, K = 128, 256, 512
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=9)
    X = dev_bf16(x).requires_grad_(True)
    W = dev_bf16(w).requires_grad_(True)
    g = torch.randn(T, N, device="cuda")
    y = dag.projection(X, W, out_dtype=torch.float32)
    assert y.dtype == torch.float32
    with pytest.raises(TypeError):
        y.backward(g)
    y = dag.projection(X, W, out_dtype=torch.float32, round_grad_to_bf16=True)
    y.backward(g)
    torch.cuda.synchronize()
    gb = g.to(torch.bfloat16)
    assert torch.equal(_bits(X.grad), _bits(dpg.dpg_dgrad(gb, W.detach())))
    assert torch.equal(_bits(W.grad), _bits(dpg.dpg_wgrad(gb, X.detach())))
