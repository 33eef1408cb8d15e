// Host planner of the projection GEMM library: maps a call's key to a launch
// plan (kernel variant, tile, raster group, K split and its partition,
// workspace).  Pure C++, no HIP calls, so it can be exercised without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dpg {

enum PlanKind { PLAN_NOOP = 0, PLAN_ZERO = 1, PLAN_GEMM = 2 };
enum Layout { LAYOUT_FWD = 0, LAYOUT_DGRAD = 1, LAYOUT_WGRAD = 2 };

// Tile shapes compiled into the library (all 256 threads, 32x32x16 MFMA).
struct TileShape {
  int bm, bn, bk;
  int threads;
  int occupancy;   // workgroups that fit one CU at once
  double eff;      // sustained fraction of the CU's MFMA rate, BF16 operands (model)
  double eff_one;  // the same when only one of its workgroups runs on a CU (0: as eff)
  double x3_eff;   // the same for BF16x3 (FP32 operands), counted in executed FLOP
  double x3_eff_two;  // BF16x3 with two workgroups on each CU (0: as x3_eff)
  int x3_occupancy;  // workgroups per CU with BF16x3 (hi and lo planes)
  bool x3_ok;      // BF16x3 plans use this tile
  bool fast_ok;    // a software-pipelined variant exists for this tile
  bool ffma;       // FP32 fused multiply-adds on the vector ALUs (router only)
};
constexpr int kNumTiles = 4;
constexpr int kGenericTile = 2;  // the only tile with a generic (non-pipelined) MFMA kernel
constexpr int kFfmaTile = 3;     // the FP32 FMA router kernel
extern const TileShape kTiles[kNumTiles];

// Arithmetic of the router passes: the planner's choice (BF16x3 on the
// matrix cores, or FP32 FMA where that measured faster), or one of them forced.
enum RouterArith { ROUTER_AUTO = 0, ROUTER_BF16X3 = 1, ROUTER_FP32 = 2 };

enum WeightLayout { WEIGHT_NK = 0, WEIGHT_KN = 1 };

struct PlanKey {
  int pass;        // dpg_pass
  int64_t T, N, K;
  int out;         // dpg_dtype
  int det;         // 0/1
  int split_req;   // 0 = auto
  int cus;         // CU count the plan was made for (fixed 256 in deterministic mode)
  int64_t batch = 1;         // independent problems of the same shape in one launch
  int wlayout = WEIGHT_NK;   // weight (or weight-gradient) stored [N,K] or [K,N]
  int router_arith = ROUTER_AUTO;  // router passes only
  int64_t generation = 0;    // plan-cache generation (the planner ignores it)
  bool operator==(const PlanKey& o) const {
    return pass == o.pass && T == o.T && N == o.N && K == o.K && out == o.out && det == o.det &&
           split_req == o.split_req && cus == o.cus && batch == o.batch && wlayout == o.wlayout &&
           router_arith == o.router_arith && generation == o.generation;
  }
};

struct Plan {
  int kind;
  int layout;          // operand majorness (LAYOUT_*)
  int x3;              // BF16x3 router arithmetic (0 for the FP32 FMA router kernel)
  int out;             // dpg_dtype of the output
  int64_t M, N, K;     // GEMM view: C[M,N] = sum_k A(m,k) B(n,k)
  int64_t batch;       // problems per launch (the unit stream runs over all of them)
  int swap_ab;         // weight gradient into a [K,N] output: A is X, B is dY
  int tile;            // index into kTiles
  int fast;            // software-pipelined kernel (gemm_fast.h) instead of the generic one
  int ffma;            // FP32 FMA router kernel (gemm_ffma.h)
  int streamk;         // stream-K work split over exactly `grid` workgroups (gemm_fast.h StreamKWork)
  int skinny;          // streaming weight-gradient kernel for N <= 128 (skinny_wgrad.h)
  int skinny_cols;     // columns of K per skinny work unit (64 or 128)
  int tiles_m, tiles_n;
  int splits, kt_total, kt_per_split;
  int group_m;
  int64_t grid;        // workgroups of the GEMM launch (skinny: of the skinny kernel)
  size_t ws_bytes;     // FP32 partials: splits * M * N * 4 when splits > 1
  double est_us;       // model estimate
};

// Deterministic CU count used by the deterministic planner (MI355X).
constexpr int kDetCus = 256;

// Builds the plan for a key; returns false for arguments no plan covers.
// A GEMM plan of S > 1 splits partitions the kt_total K tiles (64 elements, or
// 64 tokens for a weight gradient) evenly: with q = kt_total / S and r =
// kt_total % S, the first r splits take q + 1 tiles and the rest q (split s
// starts at tile s q + min(s, r)); kt_per_split is the largest split.  A forced split
// count is min(split_req, kt_total).  Every plan names a kernel that exists:
// the pipelined kernels (256x256, 128x128, and BF16x3 on 128x128) need whole
// K tiles on K-major operands, otherwise the generic 64x64 kernel runs.
bool make_plan(const PlanKey& key, Plan* plan);

// Moves a GEMM plan onto the generic 64x64 kernel (64-bit addressing), for
// calls whose row strides are beyond the pipelined and skinny kernels' 32-bit
// tile offsets.  The K partition, hence the workspace size and (for one MFMA
// instruction and k order) the output bits, stays the same; a stream-K plan
// (split-K mode only) becomes a one-split plan, which needs no more workspace.
// Returns false if the launch would exceed the grid limit.
bool generic_fallback(Plan* plan);

// One-line description of a plan.
int describe_plan(const PlanKey& key, const Plan& plan, char* buf, size_t buflen);

}  // namespace dpg
