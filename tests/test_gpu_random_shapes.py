"""Seeded random shapes, modes, split requests, weight layouts and strides
through every entry point, bit for bit against the FP64 oracle (GPU).

Inputs are exact: projections take small integers times 2^-2 (every partial sum
exact in FP32), the router takes hi + lo values whose three BF16 products and
their sums are exact (BF16x3 arithmetic forced) or small integers (FP32
arithmetic forced).  So any accumulation order gives the oracle's value, and
the check is equality: FP32 outputs equal the exact result, BF16 outputs its
nearest-even rounding.  Operands are views with padded row strides; outputs
are views into NaN-filled buffers whose padding must stay NaN.  The cases are
drawn once from a fixed generator, so every run checks the same ones."""
import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from tests.gpu_util import dev_bf16, dev_f32, host_bits, host_f64

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

MODES = [(True, 0), (False, 0), (True, 1), (False, 2), (True, 3), (False, 5), (True, 13), (False, 64)]
KINDS = ["fwd", "dgrad", "wgrad", "rfwd", "rdgrad", "rwgrad", "bfwd", "bdgrad", "bwgrad"]


def _draw_cases(n=216, seed=20261203):
    g = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        kind = KINDS[len(cases) % len(KINDS)]
        T = int(g.choice([int(g.integers(1, 200)), int(g.integers(200, 4097))]))
        N = 8 * int(g.integers(1, 400))
        K = 8 * int(g.integers(1, 400))
        if kind.startswith("r"):
            N = 8 * int(g.integers(1, 64))  # experts
            red = {"rfwd": K, "rdgrad": N, "rwgrad": T}[kind]
            if red > 4096:
                continue
        batch = int(g.integers(2, 4)) if kind.startswith("b") else 1
        if batch * T * N * K > 1.5e9:
            continue
        det, split = MODES[int(g.integers(0, len(MODES)))]
        cases.append({"kind": kind, "T": T, "N": N, "K": K, "batch": batch, "det": det, "split": split,
                      "out": "f32" if kind.startswith("r") else ("bf16" if g.integers(0, 2) else "f32"),
                      "pad_a": 8 * int(g.integers(0, 4)), "pad_b": 8 * int(g.integers(0, 4)),
                      "layout": "kn" if (kind.startswith("b") and g.integers(0, 2)) else "nk",
                      "shared_w": bool(kind in ("bfwd", "bdgrad") and g.integers(0, 2)),
                      "arith": ("bf16x3" if g.integers(0, 3) else "fp32") if kind.startswith("r") else None})
    return cases


CASES = _draw_cases()


def _case_id(c):
    return "%s-T%d-N%d-K%d-b%d-%s-%s-s%d-%s" % (c["kind"], c["T"], c["N"], c["K"], c["batch"], c["out"],
                                                "det" if c["det"] else "fast", c["split"], c["layout"])


def _padded(t, pad):
    """The same values in a buffer with `pad` more elements per row (a view)."""
    if pad == 0:
        return t
    shape = list(t.shape)
    shape[-1] += pad
    buf = torch.zeros(shape, dtype=t.dtype, device=t.device)
    buf[..., :t.shape[-1]] = t
    return buf[..., :t.shape[-1]]


def _out_view(shape, dtype):
    """A view of `shape` inside a NaN-filled buffer with one more row and 16 more
    columns, and the mask of the buffer's elements outside the view."""
    big_shape = list(shape)
    big_shape[-2] += 1
    big_shape[-1] += 16
    big = torch.full(big_shape, float("nan"), dtype=dtype, device="cuda")
    view = big[..., 1:shape[-2] + 1, 8:8 + shape[-1]]
    mask = torch.ones(big_shape, dtype=torch.bool, device="cuda")
    mask[..., 1:shape[-2] + 1, 8:8 + shape[-1]] = False
    return big, view, mask


def _expect(out_t, ref, out_name):
    if out_name == "f32":
        np.testing.assert_array_equal(host_f64(out_t), ref)
    else:
        np.testing.assert_array_equal(host_bits(out_t), oracle.f64_to_bf16(ref))


@pytest.mark.parametrize("c", CASES, ids=[_case_id(c) for c in CASES])
def test_random_shape_exact(c):
    kind, T, N, K, B = c["kind"], c["T"], c["N"], c["K"], c["batch"]
    det, split, out_name = c["det"], c["split"], c["out"]
    odt = torch.bfloat16 if out_name == "bf16" else torch.float32
    if kind.startswith("r"):
        prev = dpg.get_router_arithmetic()
        dpg.set_router_arithmetic(c["arith"])
        try:
            x, w, dy = dpg_inputs.router(T, N, K, seed_group=5, kind="exact" if c["arith"] == "bf16x3" else "int")
            mode = "bf16x3" if c["arith"] == "bf16x3" else "exact"
            op = kind[1:]
            a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[op]
            ref = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[op](a, b, mode=mode)
            fn = {"fwd": dpg.dpg_router_forward, "dgrad": dpg.dpg_router_dgrad, "wgrad": dpg.dpg_router_wgrad}[op]
            big, view, mask = _out_view(ref.shape, torch.float32)
            fn(_padded(dev_f32(a), c["pad_a"]), _padded(dev_f32(b), c["pad_b"]), out=view, deterministic=det,
               split_k=split)
            torch.cuda.synchronize()
        finally:
            dpg.set_router_arithmetic(prev)
        np.testing.assert_array_equal(host_f64(view), ref)
        assert torch.isnan(big[mask]).all()
        return

    if not kind.startswith("b"):
        x, w, dy = dpg_inputs.dense(T, N, K, seed_group=6, kind="int")
        a, b = {"fwd": (x, w), "dgrad": (dy, w), "wgrad": (dy, x)}[kind]
        ref = {"fwd": oracle.forward, "dgrad": oracle.dgrad, "wgrad": oracle.wgrad}[kind](a, b)
        fn = {"fwd": dpg.dpg_forward, "dgrad": dpg.dpg_dgrad, "wgrad": dpg.dpg_wgrad}[kind]
        big, view, mask = _out_view(ref.shape, odt)
        fn(_padded(dev_bf16(a), c["pad_a"]), _padded(dev_bf16(b), c["pad_b"]), out=view, deterministic=det,
           split_k=split)
        torch.cuda.synchronize()
        _expect(view, ref, out_name)
        assert torch.isnan(big.float()[mask]).all()
        return

    # batched: B problems, weight [B, N, K] / [B, K, N] or one shared 2-D weight
    op, kn = kind[1:], c["layout"] == "kn"
    probs = [dpg_inputs.dense(T, N, K, seed_group=7 + p, kind="int") for p in range(B)]
    shared = c["shared_w"]
    if shared:
        probs = [(x, probs[0][1], dy) for (x, _, dy) in probs]
    xs = np.stack([p[0] for p in probs])
    dys = np.stack([p[2] for p in probs])
    ws_nk = [p[1] for p in probs]
    w_store = [np.ascontiguousarray(wk.T) if kn else wk for wk in ws_nk]
    if op == "fwd":
        refs = [oracle.forward(probs[p][0], ws_nk[p]) for p in range(B)]
        wdev = dev_bf16(w_store[0]) if shared else dev_bf16(np.stack(w_store))
        big, view, mask = _out_view((B, T, N), odt)
        dpg.dpg_forward_batched(_padded(dev_bf16(xs), c["pad_a"]), _padded(wdev, c["pad_b"]), out=view,
                                weight_layout=c["layout"], deterministic=det, split_k=split)
    elif op == "dgrad":
        refs = [oracle.dgrad(probs[p][2], ws_nk[p]) for p in range(B)]
        wdev = dev_bf16(w_store[0]) if shared else dev_bf16(np.stack(w_store))
        big, view, mask = _out_view((B, T, K), odt)
        dpg.dpg_dgrad_batched(_padded(dev_bf16(dys), c["pad_a"]), _padded(wdev, c["pad_b"]), out=view,
                              weight_layout=c["layout"], deterministic=det, split_k=split)
    else:
        refs = [oracle.wgrad(probs[p][2], probs[p][0]) for p in range(B)]
        if kn:
            refs = [np.ascontiguousarray(r.T) for r in refs]
        big, view, mask = _out_view((B,) + refs[0].shape, odt)
        dpg.dpg_wgrad_batched(_padded(dev_bf16(dys), c["pad_a"]), _padded(dev_bf16(xs), c["pad_b"]), out=view,
                              weight_layout=c["layout"], deterministic=det, split_k=split)
    torch.cuda.synchronize()
    for p in range(B):
        _expect(view[p], refs[p], out_name)
    assert torch.isnan(big.float()[mask]).all()
