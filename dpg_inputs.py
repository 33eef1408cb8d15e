"""Seeded synthetic inputs for the projection GEMMs (shared by tests and the bench).

This module holds no arithmetic of the GEMMs themselves: it only draws numbers
and stores them as BF16 bit patterns (numpy ``uint16``) or FP32 arrays.  Both
the FP64 oracle and the HIP library consume exactly these bits.

Recipe (the pages fix no generator):
* NumPy ``default_rng(seed)`` (PCG64); tensor number ``i`` of seed group ``s``
  uses seed ``1000*s + i``;
* dense values are FP32 ``standard_normal`` times sigma, then rounded to BF16
  (nearest, ties to even) where the operand is BF16;
* X and dY have sigma 1, W has sigma 0.02, as in the workloads of the
  projection pages (4096->1024, 4096->12288, skinny N = 48..128, router with
  256 experts).
"""
import numpy as np

SIGMA_W = 0.02


def _to_bf16_bits(f32):
    """FP32 -> BF16 bit patterns, nearest-even (inputs are finite normals)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _rng(seed_group, index):
    return np.random.default_rng(1000 * seed_group + index)


def normal_f32(shape, sigma, seed_group, index):
    g = _rng(seed_group, index)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def normal_bf16(shape, sigma, seed_group, index):
    return _to_bf16_bits(normal_f32(shape, sigma, seed_group, index))


def small_int_bf16(shape, seed_group, index):
    """Values in {-3..3} * 2**-2, exact in BF16.  Every partial sum of products of
    such values is a multiple of 2**-4; up to reductions of ~10**6 terms they are
    exact in FP32, so any accumulation order gives the same bits."""
    g = _rng(seed_group, index)
    v = g.integers(-3, 4, size=shape).astype(np.float32) * np.float32(0.25)
    return _to_bf16_bits(v)


def small_int_f32(shape, seed_group, index):
    """FP32 values in {-3..3} * 2**-2: products and their partial sums (up to
    ~10**6 terms) are exact in FP32, so any summation order gives the same bits."""
    g = _rng(seed_group, index)
    return g.integers(-3, 4, size=shape).astype(np.float32) * np.float32(0.25)


def router_exact_f32(shape, seed_group, index):
    """FP32 values a = hi + lo with hi in {+-1} and lo in {+-1, +-3} * 2**-11.

    |lo| is below half a BF16 ulp of hi, so bf16(a) = hi and a - hi = lo exactly;
    all products and their sums (up to 4096 terms) are exact in FP32."""
    g = _rng(seed_group, index)
    hi = np.where(g.integers(0, 2, size=shape) == 0, -1.0, 1.0)
    lo = g.choice(np.array([-3.0, -1.0, 1.0, 3.0]), size=shape) * 2.0 ** -11
    return (hi + lo).astype(np.float32)


def dense(T, N, K, seed_group=0, kind="normal"):
    """X[T,K], W[N,K], dY[T,N] as BF16 bits."""
    if kind == "normal":
        x = normal_bf16((T, K), 1.0, seed_group, 0)
        w = normal_bf16((N, K), SIGMA_W, seed_group, 1)
        dy = normal_bf16((T, N), 1.0, seed_group, 2)
    elif kind == "int":
        x = small_int_bf16((T, K), seed_group, 0)
        w = small_int_bf16((N, K), seed_group, 1)
        dy = small_int_bf16((T, N), seed_group, 2)
    else:
        raise ValueError(kind)
    return x, w, dy


def router(T, E, H, seed_group=0, kind="normal"):
    """X[T,H], W[E,H], dY[T,E] as FP32."""
    if kind == "normal":
        x = normal_f32((T, H), 1.0, seed_group, 0)
        w = normal_f32((E, H), SIGMA_W, seed_group, 1)
        dy = normal_f32((T, E), 1.0, seed_group, 2)
    elif kind == "exact":
        x = router_exact_f32((T, H), seed_group, 0)
        w = router_exact_f32((E, H), seed_group, 1)
        dy = router_exact_f32((T, E), seed_group, 2)
    elif kind == "int":
        x = small_int_f32((T, H), seed_group, 0)
        w = small_int_f32((E, H), seed_group, 1)
        dy = small_int_f32((T, E), seed_group, 2)
    else:
        raise ValueError(kind)
    return x, w, dy


def skinny(T, N, K, seed_group=0):
    """dY[T,N], X[T,K] ~ N(0,1) as BF16 bits (skinny-N weight gradient)."""
    return normal_bf16((T, N), 1.0, seed_group, 2), normal_bf16((T, K), 1.0, seed_group, 0)


def int_values(shape, lo, hi, seed_group, index):
    """Integers drawn uniformly from lo..hi (inclusive), as int32."""
    return _rng(seed_group, index).integers(lo, hi + 1, size=shape).astype(np.int32)


def int_factors(rows, cols, rank, seed_group, index, lo=-2, hi=2):
    """Integer factors U[rows, rank] and V[rank, cols] drawn from lo..hi; a
    caller that multiplies them gets an integer matrix of rank <= `rank`."""
    g = _rng(seed_group, index)
    u = g.integers(lo, hi + 1, size=(rows, rank)).astype(np.int32)
    v = g.integers(lo, hi + 1, size=(rank, cols)).astype(np.int32)
    return u, v


def ints_to_bf16_bits(a):
    """Integers of magnitude <= 256 as BF16 bit patterns (exact: BF16 holds
    every such integer)."""
    a = np.asarray(a)
    if a.size and int(np.abs(a).max()) > 256:
        raise ValueError("integer beyond the exact BF16 range")
    return _to_bf16_bits(a.astype(np.float32))
