"""Helpers shared by the GPU tests: moving seeded inputs to the device, reading
outputs back, and sampling output positions for full-size checks."""
import numpy as np
import torch


def dev_bf16(bits):
    """numpy uint16 BF16 bit patterns -> device torch.bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_f64(t):
    """Device tensor (bf16 or f32) -> float64 numpy, exact."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_bits(t):
    """Device bf16 tensor -> uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sample_positions(rows, cols, n, seed=0, edges=True):
    """n random (row, col) positions plus the corners and the last row/column
    (the ragged tile edges)."""
    g = np.random.default_rng(seed)
    ii = [g.integers(0, rows, n)]
    jj = [g.integers(0, cols, n)]
    if edges:
        k = min(cols, 64)
        for r in (0, rows - 1):
            ii.append(np.full(k, r))
            jj.append(np.linspace(0, cols - 1, k).astype(np.int64))
        k = min(rows, 64)
        for c in (0, cols - 1):
            ii.append(np.linspace(0, rows - 1, k).astype(np.int64))
            jj.append(np.full(k, c))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)


def report(tag, **fields):
    """One line of measured accuracy (error-to-budget margins and the like) on
    stdout, prefixed PARITY, for runs that collect them (pytest -s)."""
    import json
    print("PARITY %s %s" % (tag, json.dumps(fields, sort_keys=True)), flush=True)
