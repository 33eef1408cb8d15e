"""Windows of the token count T that share one deterministic plan.

The planner keys plans by exact T (row-half-release page, description: programs
keyed to exact token counts); as T grows, the tile, the kernel, the number of
K splits or (router) the arithmetic change at the first T of each window listed
here.  The configs' own token counts sit on such edges (64 and 65 for the
4096 -> 1024 projection, 256 / 257 and 1024 / 1025 for the router), and the
weight-gradient page reports budget misses of its own plans at window edges, so
the GPU tests check both sides of every edge.  test_library_cpu checks that the
planner's windows are exactly these."""

# skinny weight gradient dW[N, K] (K -> N), BF16 and FP32 output alike; the
# plan stays the same from the last edge on (checked up to T = 70000)
SKINNY_EDGES = {
    (4096, 64): [1473, 1985, 2497, 3009, 3521, 4033],
    (4096, 128): [1473, 1985, 2497, 3009, 3521, 4033],
    (5120, 48): [1473, 1985, 2497, 3009],
    (5120, 64): [1473, 1985, 2497, 3009],
}
SKINNY_T_MAX = 70000

# FP32 router (E = 256 experts, H = 4096), automatic arithmetic; checked up to T = 2048
ROUTER_EDGES = {
    "fwd": [129, 257, 321, 513, 641, 1025, 1281, 1345],
    "dgrad": [513],
    "wgrad": [1729, 1793, 1857],
}
ROUTER_T_MAX = 2048

# projection 4096 -> 1024, BF16 output; checked up to T = 512
SMALL_EDGES = {"fwd": [65, 129, 257, 321], "dgrad": [], "wgrad": []}
SMALL_T_MAX = 512


def plan_key(text):
    """The fields of a plan description that define the computation's order:
    tile, kernel, K splits, arithmetic, threads, stream-K."""
    d = dict(kv.split("=", 1) for kv in text.split())
    return tuple(d[f] for f in ("tile", "kernel", "splits", "arith", "threads", "streamk"))
