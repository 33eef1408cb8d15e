"""Pins of the FP64 oracle against things other than itself (CPU only).

Each pin is a function of an ``Oracle`` instance so that the mutation tests at
the end can run it against a copy of the oracle with a planted mistake and
show that the pin fails there.
"""
import os
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import dpg_inputs
import oracle
from oracle import bf16_to_f64

U53 = 2.0 ** -53


def _frac_matmul(A, B):
    """Exact rational C = A @ B from float64 entries."""
    M, R = A.shape
    R2, N = B.shape
    assert R == R2
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    return [[sum((Af[i][r] * Bf[r][j] for r in range(R)), Fraction(0)) for j in range(N)] for i in range(M)]


def _vals(a):
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


# ---------------------------------------------------------------- pins ----

def pin_bruteforce(orc, T, N, K, dtype, seed):
    """All three passes vs exact rational sums, within R * 2**-53 * sum|ab|."""
    if dtype == "bf16":
        x, w, dy = dpg_inputs.dense(T, N, K, seed)
    else:
        x, w, dy = dpg_inputs.router(T, N, K, seed)
    X, W, DY = _vals(x), _vals(w), _vals(dy)
    cases = [
        ("fwd", orc.forward(x, w), X, W.T),
        ("dgrad", orc.dgrad(dy, w), DY, W),
        ("wgrad", orc.wgrad(dy, x), DY.T, X),
    ]
    for name, got, A, B in cases:
        exact = _frac_matmul(A, B)
        R = A.shape[1]
        scale = np.abs(A) @ np.abs(B)
        for i in range(A.shape[0]):
            for j in range(B.shape[1]):
                err = abs(Fraction(float(got[i, j])) - exact[i][j])
                assert float(err) <= max(R, 1) * U53 * scale[i, j] + 1e-300, (name, i, j)


def pin_integer(orc, T, N, K, seed):
    """Exact-integer inputs: every pass equals an int64 matmul (exact), scaled."""
    x, w, dy = dpg_inputs.dense(T, N, K, seed, kind="int")
    Xi = np.rint(_vals(x) * 4).astype(np.int64)
    Wi = np.rint(_vals(w) * 4).astype(np.int64)
    Di = np.rint(_vals(dy) * 4).astype(np.int64)
    np.testing.assert_array_equal(orc.forward(x, w) * 16, (Xi @ Wi.T).astype(np.float64))
    np.testing.assert_array_equal(orc.dgrad(dy, w) * 16, (Di @ Wi).astype(np.float64))
    np.testing.assert_array_equal(orc.wgrad(dy, x) * 16, (Di.T @ Xi).astype(np.float64))


def pin_adjoint(orc, T, N, K, seed):
    """<dY, X W^T> = <dY W, X> = <dY^T X, W>, all in FP64 to 1e-12 relative."""
    x, w, dy = dpg_inputs.dense(T, N, K, seed)
    X, W, DY = _vals(x), _vals(w), _vals(dy)
    s1 = float(np.sum(DY * orc.forward(x, w)))
    s2 = float(np.sum(orc.dgrad(dy, w) * X))
    s3 = float(np.sum(orc.wgrad(dy, x) * W))
    scale = float(np.sum(np.abs(DY) * (np.abs(X) @ np.abs(W).T)))
    assert abs(s1 - s2) <= 1e-12 * scale
    assert abs(s1 - s3) <= 1e-12 * scale


def pin_transpose(orc, T, N, K, seed):
    """(dY^T X)^T = X^T dY, the second computed with the operands swapped."""
    x, w, dy = dpg_inputs.dense(T, N, K, seed)
    a = orc.wgrad(dy, x)
    b = orc.wgrad(x, dy)
    np.testing.assert_array_equal(a, b.T)


def pin_special(orc):
    """W = I gives Y = X; a one-hot row of X selects a column of W^T; T = 1 gives
    an outer product; an all-zero operand gives zeros."""
    x, _, dy = dpg_inputs.dense(5, 16, 16, 3)
    eye = oracle.f32_to_bf16(np.eye(16, dtype=np.float32))
    np.testing.assert_array_equal(orc.forward(x, eye), _vals(x))
    _, w, _ = dpg_inputs.dense(5, 16, 16, 3)
    onehot = np.zeros((16, 16), dtype=np.float32)
    onehot[np.arange(16), (np.arange(16) * 7) % 16] = 1.0
    y = orc.forward(oracle.f32_to_bf16(onehot), w)
    np.testing.assert_array_equal(y, _vals(w)[:, (np.arange(16) * 7) % 16].T)
    x1, _, dy1 = dpg_inputs.dense(1, 9, 11, 4)
    np.testing.assert_array_equal(orc.wgrad(dy1, x1), np.outer(_vals(dy1)[0], _vals(x1)[0]))
    z = np.zeros((4, 16), dtype=np.uint16)
    assert not np.any(orc.forward(z, w[:, :16] if w.shape[1] >= 16 else w))


def pin_sampled(orc):
    """Sampled outputs equal the full outputs bit for bit."""
    x, w, dy = dpg_inputs.dense(33, 24, 40, 5)
    g = np.random.default_rng(0)
    for fn, a, b, shape in [(orc.forward, x, w, (33, 24)), (orc.dgrad, dy, w, (33, 40)),
                            (orc.wgrad, dy, x, (24, 40))]:
        full = fn(a, b)
        ii = g.integers(0, shape[0], 50)
        jj = g.integers(0, shape[1], 50)
        np.testing.assert_array_equal(fn(a, b, rows=ii, cols=jj), full[ii, jj])


def _rne_cases():
    """(fp32 bits, expected bf16 bits, note) from tests/golden/bf16_rne.txt."""
    path = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne.txt")
    out = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()[:2]
            out.append((int(a, 16), int(b, 16)))
    return out


def pin_rne(orc):
    """Crafted FP32 -> BF16 cases (ties, signed zeros, subnormals, carries into
    the exponent, overflow) and agreement with torch's BF16 conversion."""
    cases = _rne_cases()
    f = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = orc.f32_to_bf16(f)
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    g = np.random.default_rng(7)
    u = g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_bf16(v), ref)


def pin_split(orc):
    """hi = bf16(a) and lo = bf16(a - hi) agree with torch; |a - hi - lo| <= 2**-16 |a|."""
    g = np.random.default_rng(11)
    a = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    hi, lo = orc.split_bf16x3(a)
    t = torch.from_numpy(a)
    th = t.to(torch.bfloat16)
    tl = (t - th.float()).to(torch.bfloat16)
    np.testing.assert_array_equal(hi, th.float().numpy())
    np.testing.assert_array_equal(lo, tl.float().numpy())
    res = np.abs(a.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64))
    assert np.all(res <= 2.0 ** -16 * np.abs(a.astype(np.float64)) + 1e-45)


def pin_bf16x3_exact(orc, T=7, E=5, H=64):
    """Inputs a = hi + lo (hi = +-1, lo in {+-1,+-3}*2**-11): the three-product
    value is known in closed form from integers, and differs from the exact
    product sum by the dropped lo*lo terms."""
    x, w, dy = dpg_inputs.router(T, E, H, 2, kind="exact")

    def parts(a):
        a64 = a.astype(np.float64)
        h = np.sign(a64)
        lo_i = np.rint((a64 - h) * 2 ** 11).astype(np.int64)  # in {+-1, +-3}
        return h.astype(np.int64), lo_i

    xh, xl = parts(x)
    wh, wl = parts(w)
    dh, dl = parts(dy)

    def c3(Ah, Al, Bh, Bl):
        # hi*hi + hi*lo + lo*hi, scaled by 2**11
        return ((Ah @ Bh) * 2 ** 11 + Ah @ Bl + Al @ Bh).astype(np.float64) / 2 ** 11

    def exact(Ah, Al, Bh, Bl):
        return ((Ah @ Bh) * 2 ** 22 + (Ah @ Bl + Al @ Bh) * 2 ** 11 + Al @ Bl).astype(np.float64) / 2 ** 22

    np.testing.assert_array_equal(orc.forward(x, w, mode="bf16x3"), c3(xh, xl, wh.T, wl.T))
    np.testing.assert_array_equal(orc.dgrad(dy, w, mode="bf16x3"), c3(dh, dl, wh, wl))
    np.testing.assert_array_equal(orc.wgrad(dy, x, mode="bf16x3"), c3(dh.T, dl.T, xh, xl))
    np.testing.assert_array_equal(orc.forward(x, w), exact(xh, xl, wh.T, wl.T))
    assert np.any(orc.forward(x, w, mode="bf16x3") != orc.forward(x, w))


def pin_bf16x3_bound(orc, T=16, E=256, H=512, seed=0):
    """|c3 - c| <= (u^2 (1+u)^2 + 2 u^2 (1+u^2) + u^4 + 3R 2**-53) sum|a b|, u = 2**-8."""
    x, w, dy = dpg_inputs.router(T, E, H, seed)
    u = 2.0 ** -8
    for fn, a, b, R in [(orc.forward, x, w, H), (orc.dgrad, dy, w, E), (orc.wgrad, dy, x, T)]:
        c = fn(a, b)
        c3 = fn(a, b, mode="bf16x3")
        s = fn(a, b, mode="abs")
        bound = (u * u * (1 + u) ** 2 + 2 * u * u * (1 + u * u) + u ** 4 + 3 * R * U53) * s
        assert np.all(np.abs(c3 - c) <= bound)
        # and the emulation is far better than plain BF16 rounding on average
        assert np.linalg.norm(c3 - c) / np.linalg.norm(c) < 1e-4


# ------------------------------------------------------------- the tests ----

@pytest.mark.parametrize("T,N,K", [(1, 3, 4), (3, 5, 7), (9, 8, 9), (4, 1, 1), (65, 3, 2), (129, 2, 3)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bruteforce(T, N, K, dtype):
    pin_bruteforce(oracle.default(), T, N, K, dtype, seed=T + N + K)


@pytest.mark.parametrize("T,N,K", [(130, 72, 200), (65, 48, 128), (1, 16, 8)])
def test_integer(T, N, K):
    pin_integer(oracle.default(), T, N, K, seed=1)


def test_adjoint():
    pin_adjoint(oracle.default(), 37, 29, 53, seed=2)


def test_transpose():
    pin_transpose(oracle.default(), 31, 12, 20, seed=3)


def test_special():
    pin_special(oracle.default())


def test_sampled():
    pin_sampled(oracle.default())


def test_rne():
    pin_rne(oracle.default())


def test_split():
    pin_split(oracle.default())


def test_bf16x3_exact():
    pin_bf16x3_exact(oracle.default())


def test_bf16x3_bound():
    pin_bf16x3_bound(oracle.default())


def test_inputs_recipe():
    """The generator draws FP32 normals and rounds to BF16 with nearest-even."""
    a = dpg_inputs.normal_f32((64, 32), 0.02, 3, 1)
    b = dpg_inputs.normal_bf16((64, 32), 0.02, 3, 1)
    np.testing.assert_array_equal(b, oracle.f32_to_bf16(a))
    assert abs(float(np.std(a)) - 0.02) < 0.003


# ----------------------------------------------- planted mistakes (CPU) ----

_MUTANTS = {
    # name: (original text, replacement, pin that must fail)
    "drop_first_term": ("for (int64_t r = 0; r < R; ++r)\n          s +=", "for (int64_t r = 1; r < R; ++r)\n          s +=",
                        lambda o: pin_bruteforce(o, 3, 5, 7, "bf16", 1)),
    "wrong_sign": ("row[j] += pair_term", "row[j] -= pair_term", lambda o: pin_integer(o, 17, 9, 13, 1)),
    "transposed_b": ("r * b_sr + j * b_sj, mode);\n        c[i", "r * b_sj + j * b_sr, mode);\n        c[i",
                     lambda o: pin_bruteforce(o, 6, 6, 6, "bf16", 2)),
    "no_hi_lo": ("return xh * yh + xh * yl + xl * yh;", "return xh * yh + xl * yh;", lambda o: pin_bf16x3_exact(o)),
    "with_lo_lo": ("return xh * yh + xh * yl + xl * yh;", "return xh * yh + xh * yl + xl * yh + xl * yl;",
                   lambda o: pin_bf16x3_exact(o)),
    "truncate": ("(u + 0x7fffu + lsb) >> 16", "(u + 0u * lsb) >> 16", lambda o: pin_rne(o)),
    "ties_away": ("(u + 0x7fffu + lsb) >> 16", "(u + 0x8000u + 0u * lsb) >> 16", lambda o: pin_rne(o)),
    "lo_unrounded": ("float l = bf16_bits_to_float(orc_f32_to_bf16(r));", "float l = r;", lambda o: pin_split(o)),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="orc_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_dir):
    old, new, pin = _MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dpg_oracle.c")).read()
    assert src.count(old) == 1, name
    path = os.path.join(mutant_dir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, src=path, out=os.path.join(mutant_dir, name + ".so"))
    with pytest.raises(AssertionError):
        pin(oracle.Oracle(lib))


def test_thread_count_does_not_change_results():
    """Each output is one ascending FP64 sum computed by one thread, so the
    thread count (the bench times the oracle on one thread and on all) cannot
    change a bit of the result."""
    x, w, dy = dpg_inputs.dense(37, 72, 200, seed_group=3)
    rx, rw, rdy = dpg_inputs.router(19, 24, 256, seed_group=3)
    n_all = oracle.num_threads()
    try:
        outs = []
        for n in (n_all, 1):
            oracle.set_num_threads(n)
            assert oracle.num_threads() == n
            outs.append([oracle.forward(x, w), oracle.dgrad(dy, w), oracle.wgrad(dy, x),
                         oracle.forward(rx, rw, mode="bf16x3"), oracle.wgrad(rdy, rx)])
    finally:
        oracle.set_num_threads(n_all)
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.int64), b.view(np.int64))
