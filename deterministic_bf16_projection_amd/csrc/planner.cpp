// Host planner: see planner.h.
#include "planner.h"

#include <stdio.h>

#include <algorithm>
#include <cmath>

namespace dpg {

// Rates are per CU, shared by the workgroups resident on it (measured on
// MI355X: one 64x64 workgroup already sustains most of what a CU gives that
// kernel, while the 128x128 tile gains from its second workgroup: FP32-output
// projections at 16384 tokens ran at 0.40-0.45 of the CU rate with two per CU,
// against 0.26-0.41 with one depending on layout).  BF16x3 plans use the
// pipelined 128x128 tile or the generic 64x64 one.  Two generic BF16x3
// workgroups on a CU run faster than the one-workgroup rate says in the
// weight-gradient layout and, in the K-major layouts, with short units (up to
// 10 K tiles): router forward (hidden 4096) at 768 and 1024 tokens, 8 splits
// on 64x64 tiles, 19.9 and 21.9 us measured against 25 us modelled; router
// weight gradient at 1760-2048 tokens, 2 splits on 64x64 tiles 31.6-34.2 us
// against 37.3-40.2 us for the 128x128 tile the one-workgroup rate chose.
// With longer forward units that rate fits (1200-2048 tokens, where the
// pipelined 128x128 tile with 8-12 splits is faster).
const TileShape kTiles[kNumTiles] = {
    // bm, bn, bk, threads, occupancy, eff, eff_one, x3_eff, x3_eff_two, x3_occupancy, x3_ok, fast_ok, ffma
    {256, 256, 64, 256, 1, 0.55, 0.0, 0.0, 0.0, 0, false, true, false},
    {128, 128, 64, 256, 2, 0.43, 0.36, 0.28, 0.0, 1, true, true, false},
    {64, 64, 64, 256, 4, 0.20, 0.0, 0.19, 0.26, 2, true, false, false},
    // FP32 FMA (router): eff is the fraction of the CU's FP32 vector rate
    // with two or more workgroups on a CU, eff_one with one (a workgroup has
    // one wave per SIMD, too few to cover its LDS and FMA latencies): router
    // at 1024 tokens, forward 42.5 us with 8 splits (two per CU) against 62.8
    // us with 4 (one per CU), weight gradient 40.9 us with 2 splits against
    // 58.2 us with 1
    {64, 64, 64, 256, 4, 0.42, 0.25, 0.0, 0.0, 0, false, false, true},
};

namespace {

constexpr double kCuFlops = 2.2e15 / 256;  // sustained BF16 MFMA FLOP/s of one CU (measured loop)
constexpr double kCuFp32 = 256.0 * 2.4e9;  // FP32 vector FLOP/s of one CU (64 lanes x 4 SIMDs x FMA)
constexpr double kHbm = 5.0e12;            // sustained HBM bytes/s
constexpr double kLaunchUs = 3.0;          // per kernel launch
constexpr double kUnitUs = 1.0;            // fixed latency of a unit (first loads, last MFMAs)
constexpr double kCuStore = 25e9;          // bytes/s of epilogue stores per CU
constexpr double kReduceLatUs = 0.5;       // split reduction: per group of 8 dependent plane loads
constexpr double kWgFetch = 40e9;          // operand bytes/s one generic-kernel workgroup fetches

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// GEMM view of a pass: C[M,N] = sum_k A(m,k) B(n,k).  A weight stored [K,N]
// turns the forward's B and the input gradient's B around (MN-major <->
// K-major); a weight gradient written [K,N] swaps the operands.
void gemm_view(int pass, int wlayout, int64_t T, int64_t N, int64_t K, int64_t* m, int64_t* n, int64_t* k,
               int* layout, int* swap_ab) {
  *swap_ab = 0;
  switch (pass % 3) {
    case 0:  // forward: Y[T,N] = X[T,K] W^T
      *m = T; *n = N; *k = K; *layout = wlayout == WEIGHT_KN ? LAYOUT_DGRAD : LAYOUT_FWD;
      break;
    case 1:  // input gradient: dX[T,K] = dY[T,N] W
      *m = T; *n = K; *k = N; *layout = wlayout == WEIGHT_KN ? LAYOUT_FWD : LAYOUT_DGRAD;
      break;
    default:  // weight gradient: dW = dY^T X (as [N,K]) or X^T dY (as [K,N])
      if (wlayout == WEIGHT_KN) {
        *m = K; *n = N; *swap_ab = 1;
      } else {
        *m = N; *n = K;
      }
      *k = T; *layout = LAYOUT_WGRAD;
      break;
  }
}

// Time model of one plan (microseconds).  The units (tile x split) run on
// cus * occupancy workgroup slots in rounds; the workgroups resident on a CU
// share its rate.  A round costs the unit latency, the MFMA work and the
// epilogue stores of its units; the persistent pipelined kernel pays latency
// and one epilogue only once (later epilogues overlap the next unit's loads).
// Memory: operands once and the output; split partials are written, then read
// back by the reduce kernel, whose dependent loads cost latency when the
// output is small.
double estimate_us(const TileShape& ts, bool fast, int64_t batch, int64_t M, int64_t N, int64_t K, int x3,
                   int layout, int out_bytes, int in_bytes, int splits_req, int cus, int* splits_out,
                   int* kt_per_out) {
  const int64_t tiles = cdiv(M, ts.bm) * cdiv(N, ts.bn) * batch;
  const int64_t kt_total = cdiv(K, ts.bk);
  // balanced partition: min(request, K tiles) splits, the largest kt_per tiles
  const int64_t s = std::max<int64_t>(1, std::min<int64_t>(splits_req, kt_total));
  const int64_t kt_per = cdiv(kt_total, s);
  const int64_t units = tiles * s;
  const double flop_unit = 2.0 * ts.bm * ts.bn * (double)(kt_per * ts.bk) * (x3 ? 3 : 1);
  const int64_t occ_used = std::min<int64_t>(x3 ? ts.x3_occupancy : ts.occupancy, cdiv(units, cus));
  const int64_t rounds = cdiv(units, (int64_t)cus * occ_used);
  // a lone four-wave workgroup leaves the CU's MFMA pipes idler than two do
  const double eff = (occ_used == 1 && ts.eff_one > 0) ? ts.eff_one : ts.eff;
  // two BF16x3 workgroups on a CU: weight-gradient layout, or short units (up
  // to 10 K tiles) of the K-major layouts
  const bool two = occ_used == 2 && ts.x3_eff_two > 0 && (layout == LAYOUT_WGRAD || kt_per <= 10);
  const double x3_eff = two ? ts.x3_eff_two : ts.x3_eff;
  const double cu_rate = ts.ffma ? kCuFp32 * eff : kCuFlops * (x3 ? x3_eff : eff);
  const double epi_us = (double)occ_used * ts.bm * ts.bn * (s > 1 ? 4 : out_bytes) / kCuStore * 1e6;
  double mfma_round_us = (double)occ_used * flop_unit / cu_rate * 1e6;
  // the generic kernel stages through registers without a deep pipeline: a
  // workgroup's operand fetch, (bm + bn) x bk elements a K tile, bounds a long
  // unit (32 K tiles or more; 4096 -> 1024 forward at 1024 tokens, one split
  // on 64x64 tiles: 40.4 us measured against 23.9 us from the MFMA rate
  // alone; the 128x128 tile with 4 splits ran 22.8 us).  Shorter units ran
  // at the MFMA rate.
  if (!fast && !ts.ffma && kt_per >= 32)
    mfma_round_us = std::max(mfma_round_us, (double)(ts.bm + ts.bn) * kt_per * ts.bk * in_bytes / kWgFetch * 1e6);
  double t_gemm = fast ? rounds * mfma_round_us + kUnitUs + epi_us : rounds * (mfma_round_us + kUnitUs + epi_us);
  const double bytes = ((double)(M * K + N * K) * in_bytes + (double)M * N * out_bytes) * batch;
  double t = std::max(t_gemm, bytes / kHbm * 1e6) + kLaunchUs;
  if (s > 1) {
    const double red_bytes = (double)M * N * 4.0 * (s + 1) * batch;
    t += std::max(red_bytes / kHbm * 1e6, (double)cdiv(s, 8) * kReduceLatUs) + kLaunchUs;
  }
  *splits_out = (int)s;
  *kt_per_out = (int)kt_per;
  return t;
}

// Time model of a stream-K plan on a pipelined tile: G = cus x occupancy
// workgroups; whole rounds of tiles run data-parallel, the K iterations of
// the remaining tiles are split evenly over the G workgroups; partial tiles
// are written as FP32 slots (one or two per workgroup) and summed by a
// fix-up kernel.  A round of whole 256x256 tiles at K = 4096 measured ~111 us
// on MI355X, i.e. about the rate kCuFlops * eff gives.
double estimate_streamk_us(const TileShape& ts, int64_t M, int64_t N, int64_t K, int out_bytes, int in_bytes,
                           int cus, int64_t* grid_out) {
  const int64_t tiles = cdiv(M, ts.bm) * cdiv(N, ts.bn);
  const int64_t kt = cdiv(K, ts.bk);
  const int64_t G = (int64_t)cus * ts.occupancy;
  const int64_t D = (tiles / G) * G;
  const int64_t tail_iters = (tiles - D) * kt;
  // offered from one whole round of tiles on (where it was measured); fewer
  // tiles than workgroups are split-K territory
  if (tiles * kt >= INT32_MAX / 2 || tail_iters == 0 || D == 0) return 1e300;
  const int64_t per = cdiv(tail_iters, G);
  const double flop_iter = 2.0 * ts.bm * ts.bn * ts.bk;
  const double iter_us = (double)ts.occupancy * flop_iter / (kCuFlops * ts.eff) * 1e6;
  const double tile_bytes = (double)ts.bm * ts.bn * 4.0;
  // partial slots: one per workgroup, a second where a range crosses a tile end
  const double slots = (double)std::min<int64_t>(2 * G, G + (tiles - D));
  const double epi_us = (double)ts.occupancy * tile_bytes / kCuStore * 1e6;  // a partial slot per workgroup
  const double t_gemm = (double)(D / G * kt + per) * iter_us + kUnitUs + epi_us;
  const double bytes = ((double)(M * K + N * K) * in_bytes + (double)M * N * out_bytes);
  *grid_out = G;
  return std::max(t_gemm, bytes / kHbm * 1e6) + kLaunchUs + (slots * tile_bytes + (double)(tiles - D) * ts.bm * ts.bn *
                                                              out_bytes) / kHbm * 1e6 + kLaunchUs;
}

}  // namespace

bool make_plan(const PlanKey& key, Plan* p) {
  if (key.pass < 0 || key.pass > 5 || key.T < 0 || key.N < 0 || key.K < 0) return false;
  if (key.out != 0 && key.out != 1) return false;
  if (key.split_req < 0 || key.split_req > 64) return false;
  if (key.batch < 0 || key.batch > INT32_MAX / 2) return false;
  if (key.wlayout != WEIGHT_NK && key.wlayout != WEIGHT_KN) return false;
  if (key.pass >= 3 && (key.wlayout != WEIGHT_NK || key.batch != 1)) return false;  // router: single, [E,H]
  *p = Plan();
  p->x3 = key.pass >= 3;
  p->out = key.out;
  p->batch = key.batch;
  gemm_view(key.pass, key.wlayout, key.T, key.N, key.K, &p->M, &p->N, &p->K, &p->layout, &p->swap_ab);
  if (p->M > INT32_MAX / 2 || p->N > INT32_MAX / 2 || p->K > INT32_MAX / 2) return false;
  if (p->M == 0 || p->N == 0 || p->batch == 0) {
    p->kind = PLAN_NOOP;
    return true;
  }
  if (p->K == 0) {
    p->kind = PLAN_ZERO;
    return true;
  }
  p->kind = PLAN_GEMM;
  if (!p->x3 && p->layout == LAYOUT_WGRAD && p->M <= 128 && p->batch == 1 && !p->swap_ab) {
    // skinny weight gradient: units of (all N rows, 128 or 64 columns of K,
    // token split); tiles_m / tiles_n keep the 64x64 tile counts of the
    // generic kernel, which runs the plan when a leading dimension is too large
    p->skinny = 1;
    p->tile = 2;
    p->tiles_m = (int)cdiv(p->M, 64);
    p->tiles_n = (int)cdiv(p->N, 64);
    p->kt_total = (int)cdiv(p->K, 64);  // 64-token blocks
    // (256-column units for two row blocks over long token ranges were faster
    // with the register-staged kernel; with operands fetched straight into LDS
    // 128-column units win there too: 4096->128 at 65537 tokens 118-120 ->
    // 112-115 us, at 32768 66 -> 58 us.)
    const int64_t units = cdiv(p->N, 128);
    int64_t s;
    if (key.split_req > 0) {
      s = key.split_req;
    } else {
      s = (key.cus + units / 2) / units;
      // at least 8 token blocks a split (16 below 24 blocks, where one split
      // was as fast): from a cold cache the 2-4 more splits this allows than
      // 16 blocks a split measured 0-12% faster at 1600-7105 tokens (kernel
      // spans after a read flush; within -11..+6% after a zero fill)
      s = std::min<int64_t>(s, std::max<int64_t>(1, p->kt_total >= 24 ? p->kt_total / 8 : p->kt_total / 16));
    }
    // balanced partition of the 64-token blocks (split_begin in the kernels)
    s = std::max<int64_t>(1, std::min<int64_t>(s, p->kt_total));
    p->splits = (int)s;
    p->kt_per_split = (int)cdiv(p->kt_total, s);
    // 64-column units when 128-column ones would leave more than half the CUs idle
    p->skinny_cols = units * p->splits * 2 >= key.cus ? 128 : 64;
    p->group_m = 1;
    p->grid = cdiv(p->N, p->skinny_cols) * p->splits;
    p->ws_bytes = p->splits > 1 ? (size_t)p->splits * (size_t)p->M * (size_t)p->N * 4u : 0;
    const double bytes = 2.0 * (p->K * p->N + p->K * p->M) + (double)p->M * p->N * (p->splits > 1 ? 8.0 * p->splits : 4.0);
    p->est_us = bytes / kHbm * 1e6 + kLaunchUs * (p->splits > 1 ? 2 : 1);
    return p->grid <= INT32_MAX;
  }
  const int in_bytes = p->x3 ? 4 : 2;
  const int out_bytes = key.out == 1 ? 4 : 2;
  // the split counts the planner tries on its own; a forced request is
  // evaluated as it is (any 1..64), on every tile that has a kernel
  static const int kSplitChoices[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
  const int forced[1] = {key.split_req};
  const int* choices = key.split_req > 0 ? forced : kSplitChoices;
  const int n_choices = key.split_req > 0 ? 1 : (int)(sizeof(kSplitChoices) / sizeof(kSplitChoices[0]));
  // the pipelined kernels need whole 64-wide K tiles on K-major operands;
  // without them only the generic 64x64 kernel is compiled
  const bool kmajor_ok = p->layout == LAYOUT_WGRAD || (p->K % 64) == 0;
  double best = 1e300;
  int best_tile = -1;
  const bool router = key.pass >= 3;
  for (int ti = 0; ti < kNumTiles; ++ti) {
    const TileShape& ts = kTiles[ti];
    const bool fast = ts.fast_ok && kmajor_ok;
    if (ts.ffma) {
      // FP32 FMA: router passes whose arithmetic allows it
      if (!router || key.router_arith == ROUTER_BF16X3) continue;
    } else {
      if (!fast && ti != kGenericTile) continue;
      if (router && (!ts.x3_ok || key.router_arith == ROUTER_FP32)) continue;
    }
    for (int c = 0; c < n_choices; ++c) {
      int s, ktp;
      const double t = estimate_us(ts, fast, p->batch, p->M, p->N, p->K, ts.ffma ? 0 : p->x3, p->layout, out_bytes,
                                   in_bytes, choices[c], key.cus, &s, &ktp);
      if (best_tile < 0 || t < best * 0.97) {  // prefer the earlier (larger tile, fewer splits) unless 3% faster
        best = t;
        best_tile = ti;
        p->splits = s;
        p->kt_per_split = ktp;
      }
    }
  }
  if (best_tile < 0) return false;
  p->tile = best_tile;
  // split-K mode (deterministic = 0, no forced split count): stream-K on the
  // 256x256 pipelined tile where the model says it is 3% faster (measured on
  // MI355X: 7-19% faster than the best split-K or whole-tile plan on shapes
  // with a partial last round, e.g. 4352 x 4096 x 4096 forward 188.5 -> 152.6
  // us; on 128x128 tiles it lost to the 256x256 whole-tile plan, 96.5 vs 83.7
  // us for an 8448 x 4096 x 1024 input gradient, so those are not offered)
  int64_t sk_grid = 0;
  if (!key.det && key.split_req == 0 && !router && p->batch == 1 && kmajor_ok) {
    for (int ti = 0; ti < 1; ++ti) {
      const TileShape& ts = kTiles[ti];
      int64_t g;
      const double t = estimate_streamk_us(ts, p->M, p->N, p->K, out_bytes, in_bytes, key.cus, &g);
      if (t < best * 0.97) {
        best = t;
        p->tile = ti;
        p->streamk = 1;
        sk_grid = g;
      }
    }
  }
  const TileShape& ts = kTiles[p->tile];
  if (ts.ffma) p->x3 = 0;
  if (p->streamk) {
    p->splits = 1;
    p->kt_per_split = (int)cdiv(p->K, ts.bk);
  }
  p->tiles_m = (int)cdiv(p->M, ts.bm);
  p->tiles_n = (int)cdiv(p->N, ts.bn);
  p->kt_total = (int)cdiv(p->K, ts.bk);
  p->group_m = std::min(p->tiles_m, 8);
  p->fast = (ts.fast_ok && kmajor_ok) ? 1 : 0;
  p->ffma = ts.ffma ? 1 : 0;
  p->grid = (int64_t)p->tiles_m * p->tiles_n * p->splits * p->batch;
  p->ws_bytes = p->splits > 1 ? (size_t)p->batch * p->splits * (size_t)p->M * (size_t)p->N * 4u : 0;
  if (p->streamk) {
    p->grid = sk_grid;
    p->ws_bytes = (size_t)2 * sk_grid * ts.bm * ts.bn * 4u;
  }
  p->est_us = best;
  return p->grid <= INT32_MAX;
}

bool generic_fallback(Plan* p) {
  if (p->kind != PLAN_GEMM || p->ffma) return true;  // the FP32 FMA kernel addresses with 64 bits
  // stream-K runs on the pipelined kernels only: one split on the generic
  // kernel instead (split-K mode, whose bits may differ between plans)
  if (p->streamk) {
    p->streamk = 0;
    p->splits = 1;
    p->kt_per_split = p->kt_total;
  }
  const TileShape& ts = kTiles[kGenericTile];
  p->tile = kGenericTile;
  p->fast = 0;
  p->skinny = 0;
  p->skinny_cols = 0;
  p->tiles_m = (int)cdiv(p->M, ts.bm);
  p->tiles_n = (int)cdiv(p->N, ts.bn);
  p->group_m = std::min(p->tiles_m, 8);
  p->grid = (int64_t)p->tiles_m * p->tiles_n * p->splits * p->batch;
  return p->grid <= INT32_MAX;
}

int describe_plan(const PlanKey& key, const Plan& p, char* buf, size_t buflen) {
  static const char* kPass[] = {"forward", "dgrad", "wgrad", "router_forward", "router_dgrad", "router_wgrad"};
  static const char* kLayout[] = {"Akmajor_Bkmajor", "Akmajor_Bmnmajor", "Amnmajor_Bmnmajor"};
  if (p.kind == PLAN_NOOP)
    return snprintf(buf, buflen, "pass=%s kind=noop", kPass[key.pass]);
  if (p.kind == PLAN_ZERO)
    return snprintf(buf, buflen, "pass=%s kind=zero_fill M=%lld N=%lld", kPass[key.pass], (long long)p.M,
                    (long long)p.N);
  const TileShape& ts = kTiles[p.tile];
  return snprintf(buf, buflen,
                  "pass=%s kind=gemm det=%d M=%lld N=%lld K=%lld layout=%s x3=%d arith=%s out=%s tile=%dx%dx%d threads=%d "
                  "kernel=%s tiles=%dx%d group_m=%d splits=%d kt_total=%d kt_per_split=%d grid=%lld workspace=%zu est_us=%.1f "
                  "batch=%lld weight=%s streamk=%d",
                  kPass[key.pass], key.det, (long long)p.M, (long long)p.N, (long long)p.K, kLayout[p.layout], p.x3,
                  p.ffma ? "fp32fma" : (p.x3 ? "bf16x3" : "bf16"), p.out ? "f32" : "bf16", p.skinny ? (int)cdiv(p.M, 64) * 64 : ts.bm, p.skinny ? p.skinny_cols : ts.bn,
                  ts.bk,
                  (p.skinny || (p.fast && p.tile == 0)) ? 512 : ts.threads,
                  p.skinny ? "skinny" : (p.ffma ? "ffma" : (p.fast ? "pipelined" : "generic")), p.tiles_m, p.tiles_n,
                  p.group_m, p.splits,
                  p.kt_total, p.kt_per_split, (long long)p.grid, p.ws_bytes, p.est_us, (long long)p.batch,
                  key.wlayout == WEIGHT_KN ? "kn" : "nk", p.streamk);
}

}  // namespace dpg
