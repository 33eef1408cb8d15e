"""Batched projection GEMMs (GPU), through the C ABI: every problem of a
batched call against the FP64 oracle, bit for bit on exact-integer inputs, for
both weight layouts, all passes, BF16 and FP32 outputs, deterministic and
split plans, shared weights and interleaved per-head views; budgets on a
per-head shape with random inputs."""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import budgets
from tests.gpu_util import dev_bf16, host_bits, host_f64, sample_positions

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

OUT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _problems(B, T, N, K, seed, kind="int"):
    xs, ws, dys = [], [], []
    for b in range(B):
        x, w, dy = dpg_inputs.dense(T, N, K, seed_group=100 * seed + b, kind=kind)
        xs.append(x)
        ws.append(w)
        dys.append(dy)
    return np.stack(xs), np.stack(ws), np.stack(dys)


def _ref(pass_name, wl, x, w, dy, rows=None, cols=None):
    """The oracle's result for one problem; a [K,N] weight is handed to the
    oracle in its [N,K] form, a [K,N] weight gradient is the transpose of the
    [N,K] one."""
    if pass_name == "fwd":
        return oracle.forward(x, w, rows=rows, cols=cols)
    if pass_name == "dgrad":
        return oracle.dgrad(dy, w, rows=rows, cols=cols)
    if wl == "kn":
        if rows is None:
            return oracle.wgrad(dy, x).T
        return oracle.wgrad(dy, x, rows=cols, cols=rows)  # position (k, n) of dW[K,N] is (n, k) of dW[N,K]
    return oracle.wgrad(dy, x, rows=rows, cols=cols)


def _run(pass_name, wl, X, W, DY, out_dtype, det, split):
    if pass_name == "fwd":
        return dpg.dpg_forward_batched(X, W, out_dtype=out_dtype, weight_layout=wl, deterministic=det, split_k=split)
    if pass_name == "dgrad":
        return dpg.dpg_dgrad_batched(DY, W, out_dtype=out_dtype, weight_layout=wl, deterministic=det, split_k=split)
    return dpg.dpg_wgrad_batched(DY, X, out_dtype=out_dtype, weight_layout=wl, deterministic=det, split_k=split)


def _check_exact(out, ref, out_name):
    if out_name == "f32":
        np.testing.assert_array_equal(host_f64(out), ref)
    else:
        np.testing.assert_array_equal(host_bits(out), oracle.f64_to_bf16(ref))


@pytest.mark.parametrize("B,T,N,K", [(3, 333, 200, 264), (4, 1025, 64, 512), (2, 520, 1280, 256)])
@pytest.mark.parametrize("wl", ["nk", "kn"])
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_batched_exact_integer(B, T, N, K, wl, pass_name):
    x, w, dy = _problems(B, T, N, K, seed=1)
    # the weight as the caller stores it: [B, N, K] or [B, K, N]
    w_st = w if wl == "nk" else np.ascontiguousarray(np.swapaxes(w, 1, 2))
    X, W, DY = dev_bf16(x), dev_bf16(w_st), dev_bf16(dy)
    refs = [_ref(pass_name, wl, x[b], w[b], dy[b]) for b in range(B)]
    for out_name in ("f32", "bf16"):
        for det, split in [(True, 0), (False, 2), (True, 3)]:
            out = _run(pass_name, wl, X, W, DY, OUT[out_name], det, split)
            torch.cuda.synchronize()
            for b in range(B):
                _check_exact(out[b], refs[b], out_name)


def test_batched_shared_weight_and_head_views():
    """A 2-D weight shared by every problem (batch stride 0), and per-head
    inputs taken as views of a token-major [T, heads, K] buffer (row stride
    heads x K, batch stride K)."""
    H, T, N, K = 4, 700, 136, 128
    x, w, dy = _problems(H, T, N, K, seed=2)
    xt = np.ascontiguousarray(np.swapaxes(x, 0, 1))            # [T, H, K]
    Xt = dev_bf16(xt)
    Xv = Xt.transpose(0, 1)                                    # [H, T, K] view
    W0 = dev_bf16(w[0])
    y = dpg.dpg_forward_batched(Xv, W0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_array_equal(host_f64(y[h]), oracle.forward(x[h], w[0]))
    # outputs into a [T, H, N] buffer through a view as well
    yt = torch.full((T, H, N), float("nan"), dtype=torch.float32, device="cuda")
    dpg.dpg_forward_batched(Xv, W0, out=yt.transpose(0, 1))
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_array_equal(host_f64(yt[:, h, :]), oracle.forward(x[h], w[0]))
    # weight gradient of every head against the shared weight's layout
    DYv = dev_bf16(np.ascontiguousarray(np.swapaxes(dy, 0, 1))).transpose(0, 1)
    dw = dpg.dpg_wgrad_batched(DYv, Xv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_array_equal(host_f64(dw[h]), oracle.wgrad(dy[h], x[h]))


def test_batch_of_one_equals_single_entry_point():
    T, N, K = 1025, 64, 4096
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=3)
    X, W, DY = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    for single, batched, a, b in [(dpg.dpg_forward, dpg.dpg_forward_batched, X, W),
                                  (dpg.dpg_dgrad, dpg.dpg_dgrad_batched, DY, W),
                                  (dpg.dpg_wgrad, dpg.dpg_wgrad_batched, DY, X)]:
        s = single(a, b, out_dtype=torch.float32)
        bt = batched(a.unsqueeze(0), b.unsqueeze(0), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(s.view(torch.int32), bt[0].view(torch.int32))


@pytest.mark.parametrize("wl", ["nk", "kn"])
@pytest.mark.parametrize("pass_name", ["fwd", "dgrad", "wgrad"])
def test_batched_per_head_budget(wl, pass_name):
    """A per-head shape with random inputs (16 heads, 2048 tokens, 512 -> 128),
    BF16 budget on sampled positions of every head; reruns bitwise equal."""
    B, T, N, K = 16, 2048, 128, 512
    x, w, dy = _problems(B, T, N, K, seed=4, kind="normal")
    w_st = w if wl == "nk" else np.ascontiguousarray(np.swapaxes(w, 1, 2))
    X, W, DY = dev_bf16(x), dev_bf16(w_st), dev_bf16(dy)
    out = _run(pass_name, wl, X, W, DY, torch.bfloat16, True, 0)
    again = _run(pass_name, wl, X, W, DY, torch.bfloat16, True, 0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    rows, cols = out.shape[1], out.shape[2]
    for b in range(B):
        ii, jj = sample_positions(rows, cols, 400, seed=b)
        ref = _ref(pass_name, wl, x[b], w[b], dy[b], rows=ii, cols=jj)
        got = host_f64(out[b])[ii, jj]
        rep = budgets.check_bf16(got, ref)
        assert rep["ok"], (b, rep)
