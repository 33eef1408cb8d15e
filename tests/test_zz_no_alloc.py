"""The weight gradient that allocates nothing (dpg_wgrad_noalloc) against
dpg_wgrad, through the C ABI: same plan, so the same bits, on two calls in a
row (the second with a smaller input, so the scratch holds the first call's
partials when it starts), with split plans that use the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import dpg_inputs
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

L = dpg.lib()


def _noalloc(dy, x, out, det, split):
    T, N = dy.shape
    K = x.shape[1]
    code = dpg.F32 if out.dtype == torch.float32 else dpg.BF16
    return L.dpg_wgrad_noalloc(dy.data_ptr(), dy.stride(0), x.data_ptr(), x.stride(0), out.data_ptr(),
                               out.stride(0), code, T, N, K, int(det), split,
                               torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("det,split", [(True, 0), (False, 2), (False, 7), (True, 1)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_wgrad(det, split, out_dtype):
    assert L.dpg_noalloc_scratch_bytes() == 64 << 20
    # first a skinny stream with split planes, then a smaller GEMM-path shape
    for T, N, K in [(16384, 128, 4096), (1025, 200, 512)]:
        x, _, dy = dpg_inputs.dense(T, N, K, seed_group=31)
        X, DY = dev_bf16(x), dev_bf16(dy)
        ws = dpg.workspace_size(dpg.PASS_WGRAD, T, N, K, out_dtype, det, split)
        assert ws <= L.dpg_noalloc_scratch_bytes()
        ref = dpg.dpg_wgrad(DY, X, out_dtype=out_dtype, deterministic=det, split_k=split)
        out = torch.full((N, K), float("nan"), dtype=out_dtype, device="cuda")
        assert _noalloc(DY, X, out, det, split) == 0
        torch.cuda.synchronize()
        bits = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(bits), ref.view(bits)), (T, N, K)


def test_noalloc_rejects_oversized_plans():
    """A plan whose partials exceed the scratch is refused before any launch."""
    T, N, K = 16384, 4096, 4096
    need = dpg.workspace_size(dpg.PASS_WGRAD, T, N, K, torch.float32, False, 64)
    assert need > L.dpg_noalloc_scratch_bytes()
    dy = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    assert _noalloc(dy, x, out, False, 64) == 4
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
