"""Argument checks of the Python binding (GPU tensors, but every case is
rejected before any launch): outputs of the wrong shape or device, operands
that do not match, a workspace that is not on the device."""
import pytest
import torch

pytestmark = pytest.mark.gpu

dpg = pytest.importorskip("deterministic_bf16_projection_amd")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def test_output_shape_and_device_checked():
    x, w, dy = _bf16(64, 128), _bf16(256, 128), _bf16(64, 256)
    with pytest.raises(ValueError):
        dpg.dpg_forward(x, w, out=_bf16(32, 256))          # too few rows
    with pytest.raises(ValueError):
        dpg.dpg_forward(x, w, out=_bf16(64, 255 + 1)[:, :248])  # too few columns
    with pytest.raises(ValueError):
        dpg.dpg_dgrad(dy, w, out=torch.zeros(64, 128, dtype=torch.bfloat16))  # host tensor
    with pytest.raises(ValueError):
        dpg.dpg_wgrad(dy, x, out=_f32(128, 256))            # transposed shape
    with pytest.raises(TypeError):
        dpg.dpg_forward(x, w, out=torch.zeros(64, 256, dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()


def test_router_operand_shapes_checked():
    x, w, dy = _f32(64, 512), _f32(256, 512), _f32(64, 256)
    with pytest.raises(ValueError):
        dpg.dpg_router_forward(x, _f32(256, 520))           # H mismatch
    with pytest.raises(ValueError):
        dpg.dpg_router_dgrad(dy, _f32(128, 512))            # E mismatch
    with pytest.raises(ValueError):
        dpg.dpg_router_wgrad(dy, _f32(32, 512))             # T mismatch
    with pytest.raises(ValueError):
        dpg.dpg_router_forward(x, w, out=_f32(64, 128))
    with pytest.raises(TypeError):
        dpg.dpg_router_forward(x, w, out=_bf16(64, 256))


def test_batched_output_shape_checked():
    x, w = _bf16(2, 64, 128), _bf16(2, 256, 128)
    with pytest.raises(ValueError):
        dpg.dpg_forward_batched(x, w, out=_bf16(2, 64, 128))
    with pytest.raises(ValueError):
        dpg.dpg_wgrad_batched(_bf16(2, 64, 256), x, out=_bf16(2, 256, 128), weight_layout="kn")


def test_workspace_device_checked():
    dy, x = _bf16(4096, 64), _bf16(4096, 512)
    host_ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError):
        dpg.dpg_wgrad(dy, x, out_dtype=torch.float32, deterministic=False, split_k=2, workspace=host_ws)


def test_workspace_lives_on_the_call_stream():
    """A call on a stream other than the current one: the binding allocates the
    output and the split workspace on that stream, so memory the current
    stream allocates and fills right after the call cannot be the workspace
    the delayed kernels still use.  The result equals a current-stream run bit
    for bit."""
    import dpg_inputs
    from tests.gpu_util import dev_bf16
    T, N, K = 4031, 64, 4096
    x, _, dy = dpg_inputs.dense(T, N, K, seed_group=13)
    X, DY = dev_bf16(x), dev_bf16(dy)
    ref = dpg.dpg_wgrad(DY, X, out_dtype=torch.float32, deterministic=False, split_k=2)
    torch.cuda.synchronize()
    need = dpg.workspace_size(dpg.PASS_WGRAD, T, N, K, torch.float32, False, 2)
    assert need > 0
    s = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s):
            for _ in range(8):  # keep stream s busy so the call's kernels start late
                big = big @ big
                big = big / big.abs().max()
        out = dpg.dpg_wgrad(DY, X, out_dtype=torch.float32, deterministic=False, split_k=2, stream=s)
        junk = torch.empty(need // 4, dtype=torch.float32, device="cuda").fill_(float("nan"))
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
        del junk, out
