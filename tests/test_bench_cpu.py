"""Host logic of bench.py that needs no GPU: how the cold-cache timer turns
profiler records into per-call kernel spans (first start to last end of the
library's kernels between two flushes)."""
import os
import sys
import types

import pytest

torch = pytest.importorskip("torch")
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _ev(start, end, name, device=True):
    dt = torch.autograd.DeviceType.CUDA if device else torch.autograd.DeviceType.CPU
    return types.SimpleNamespace(time_range=types.SimpleNamespace(start=start, end=end), name=name, device_type=dt)


def _spans(events):
    timer = bench.ColdTimer.__new__(bench.ColdTimer)
    timer.torch = torch
    return timer._kernel_spans(types.SimpleNamespace(events=lambda: events))


def test_spans_group_kernels_between_flushes():
    ev = [
        _ev(0.0, 100.0, "void at::native::vectorized_elementwise_kernel<FillFunctor>"),
        _ev(101.0, 110.0, "void dpg::skinny_lds_kernel<1, 2>(dpg::SkinnyParams)"),
        _ev(111.5, 113.0, "void dpg::splitk_reduce_kernel<1>(float const*)"),
        _ev(115.0, 200.0, "void at::native::vectorized_elementwise_kernel<FillFunctor>"),
        _ev(201.0, 205.0, "void dpg::skinny_direct_kernel<2>(dpg::SkinnyParams)"),
        _ev(0.0, 300.0, "hipLaunchKernel", device=False),  # host records are ignored
    ]
    assert _spans(ev) == [12.0, 4.0]


def test_spans_sorted_by_start_and_none_without_library_kernels():
    ev = [
        _ev(50.0, 60.0, "void dpg::gemm_fast_kernel<256, 256>"),
        _ev(0.0, 40.0, "Memset (Device)"),
        _ev(70.0, 80.0, "reduce_kernel"),
    ]
    assert _spans(ev) == [10.0]
    assert _spans([_ev(0.0, 1.0, "reduce_kernel"), _ev(2.0, 3.0, "FillFunctor")]) == []
