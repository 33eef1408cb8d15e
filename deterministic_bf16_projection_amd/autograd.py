"""Training wrappers over the C ABI.

``projection(x, w)`` and ``router_gating(x, w)`` are torch autograd functions:
the forward calls ``dpg_forward`` / ``dpg_router_forward`` and saves only its
inputs; the backward calls the input-gradient and weight-gradient entry points
on the incoming gradient.  ``CheckpointedStep`` prepares the launches of one
checkpointed training step of a projection (forward, recomputed forward, input
gradient, weight gradient) with static buffers and captures them in one HIP
graph, so a replay costs no host work per kernel.

Argument marshalling only, as in the rest of the package: every product runs
in the library's kernels.  ``deterministic=False`` asks for the fast plans; when
``torch.use_deterministic_algorithms(True)`` is in force the deterministic
plans are used instead and a warning is given once.
"""
import warnings

import torch

from . import (dpg_dgrad, dpg_forward, dpg_router_dgrad, dpg_router_forward, dpg_router_wgrad, dpg_wgrad,
               workspace_size, PASS_FORWARD, PASS_DGRAD, PASS_WGRAD)

_warned = [False]


def resolve_deterministic(deterministic):
    """The plan family a call runs: deterministic if asked for, or if torch's
    deterministic-algorithms switch is on (then warns once)."""
    if deterministic:
        return True
    if torch.are_deterministic_algorithms_enabled():
        if not _warned[0]:
            warnings.warn("torch.use_deterministic_algorithms(True) is set: the projection GEMMs run their "
                          "deterministic plans", stacklevel=3)
            _warned[0] = True
        return True
    return False


def _rows(t):
    """[..., C] as a contiguous [R, C] view (the library takes unit column stride)."""
    t2 = t.reshape(-1, t.shape[-1])
    return t2 if t2.is_contiguous() else t2.contiguous()


class _Projection(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, deterministic, out_dtype, round_grad):
        x2 = _rows(x)
        y = dpg_forward(x2, w, out_dtype=out_dtype, deterministic=deterministic)
        ctx.save_for_backward(x2, w)
        ctx.deterministic = deterministic
        ctx.round_grad = round_grad
        ctx.x_shape = x.shape
        return y.reshape(*x.shape[:-1], w.shape[0])

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        # the library's gradient passes take a BF16 dY; any other incoming
        # gradient is rounded (nearest even) only when the caller asked for it
        if dy.dtype != torch.bfloat16:
            if not ctx.round_grad:
                raise TypeError("projection: the incoming gradient is %s, but the gradient GEMMs take BF16; "
                                "pass round_grad_to_bf16=True to round it to BF16 explicitly" % dy.dtype)
            dy = dy.to(torch.bfloat16)
        dy2 = _rows(dy)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = dpg_dgrad(dy2, w, out_dtype=torch.bfloat16, deterministic=ctx.deterministic).reshape(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            dw = dpg_wgrad(dy2, x2, out_dtype=torch.bfloat16, deterministic=ctx.deterministic)
        return dx, dw, None, None, None


class _Router(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, deterministic):
        x2 = _rows(x)
        y = dpg_router_forward(x2, w, deterministic=deterministic)
        ctx.save_for_backward(x2, w)
        ctx.deterministic = deterministic
        ctx.x_shape = x.shape
        return y.reshape(*x.shape[:-1], w.shape[0])

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        dy2 = _rows(dy if dy.dtype == torch.float32 else dy.to(torch.float32))
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = dpg_router_dgrad(dy2, w, deterministic=ctx.deterministic).reshape(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            dw = dpg_router_wgrad(dy2, x2, deterministic=ctx.deterministic)
        return dx, dw, None


def projection(x, w, deterministic=True, out_dtype=torch.bfloat16, round_grad_to_bf16=False):
    """y[..., N] = x[..., K] w[N, K]^T with BF16 operands and FP32 accumulation;
    differentiable in x and w (gradients in BF16).

    The gradient GEMMs take a BF16 incoming gradient.  With ``out_dtype=float32``
    the incoming gradient is FP32: backward then raises unless
    ``round_grad_to_bf16=True``, which rounds it to BF16 (nearest even) first."""
    return _Projection.apply(x, w, resolve_deterministic(deterministic), out_dtype, bool(round_grad_to_bf16))


def router_gating(x, w, deterministic=True):
    """FP32 router logits y[..., E] = x[..., H] w[E, H]^T by BF16x3;
    differentiable in x and w (FP32 gradients)."""
    return _Router.apply(x, w, resolve_deterministic(deterministic))


class CheckpointedStep:
    """One checkpointed training step of a projection with prepared launches:
    forward, recomputed forward, input gradient and weight gradient of
    x[T, K], w[N, K] and the incoming gradient dy[T, N], into static outputs
    (y, y_recomputed, dx, dw) of dtype ``out_dtype``, captured in one HIP
    graph on first use.  The caller refreshes the inputs in place (copy_) and
    calls ``replay()``; ``eager()`` issues the same launches without the graph.
    """

    def __init__(self, x, w, dy, out_dtype=torch.float32, deterministic=True):
        self.x, self.w, self.dy = x, w, dy
        T, K = x.shape
        N = w.shape[0]
        dev = x.device
        self.deterministic = resolve_deterministic(deterministic)
        self.y = torch.empty((T, N), dtype=out_dtype, device=dev)
        self.y2 = torch.empty((T, N), dtype=out_dtype, device=dev)
        self.dx = torch.empty((T, K), dtype=out_dtype, device=dev)
        self.dw = torch.empty((N, K), dtype=out_dtype, device=dev)

        def ws(pass_):
            n = workspace_size(pass_, T, N, K, out_dtype, self.deterministic, 0)
            return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        # the two forwards run back to back on one stream and may share a workspace
        self.ws = {PASS_FORWARD: ws(PASS_FORWARD), PASS_DGRAD: ws(PASS_DGRAD), PASS_WGRAD: ws(PASS_WGRAD)}
        self.graph = None

    def eager(self):
        d = self.deterministic
        dpg_forward(self.x, self.w, out=self.y, deterministic=d, workspace=self.ws[PASS_FORWARD])
        dpg_forward(self.x, self.w, out=self.y2, deterministic=d, workspace=self.ws[PASS_FORWARD])
        dpg_dgrad(self.dy, self.w, out=self.dx, deterministic=d, workspace=self.ws[PASS_DGRAD])
        dpg_wgrad(self.dy, self.x, out=self.dw, deterministic=d, workspace=self.ws[PASS_WGRAD])
        return self.y, self.y2, self.dx, self.dw

    def replay(self):
        if self.graph is None:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.eager()  # plans resolved and cached before capture
            torch.cuda.current_stream().wait_stream(side)
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                self.eager()
        self.graph.replay()
        return self.y, self.y2, self.dx, self.dw
