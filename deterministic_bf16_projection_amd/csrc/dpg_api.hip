// C ABI of the projection GEMM library: argument validation, the plan cache,
// and the launches.  Declarations and conventions are in include/dpg.h.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <list>
#include <mutex>
#include <unordered_map>

#include "dpg.h"
#include "gemm_fast.h"
#include "gemm_kernel.h"
#include "gemm_ffma.h"
#include "skinny_wgrad.h"
#include "skinny_direct.h"
#include "skinny_lds.h"
#include "planner.h"

namespace dpg {
namespace {

// ------------------------------------------------------- kernel registry --
// The generic kernel is compiled for the 64x64 tile only (the planner's
// kGenericTile): K tails on K-major operands and row strides beyond 32-bit
// tile offsets run it; everything else runs the pipelined or skinny kernels.
typedef TileCfg<64, 64, 64, 2, 2> TileS;

typedef void (*KernelFn)(GemmParams);

template <int LAYOUT, bool X3, int OUT>
constexpr KernelFn generic_for() {
  return &gemm_kernel<TileS, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, X3, OUT>;
}

template <int LAYOUT, bool X3>
struct GenericRow {
  static constexpr KernelFn fns[3] = {X3 ? nullptr : generic_for<LAYOUT, X3, OUT_BF16>(),
                                      generic_for<LAYOUT, X3, OUT_F32>(), generic_for<LAYOUT, X3, OUT_PARTIAL>()};
};

// generic 64x64 kernel for (layout, x3, out kind); null where not compiled
KernelFn lookup_generic_kernel(int layout, int x3, int out_kind) {
#define DPG_GROW(L, X) {GenericRow<L, X>::fns[0], GenericRow<L, X>::fns[1], GenericRow<L, X>::fns[2]}
  static const KernelFn table[3][2][3] = {
      {DPG_GROW(0, false), DPG_GROW(0, true)},
      {DPG_GROW(1, false), DPG_GROW(1, true)},
      {DPG_GROW(2, false), DPG_GROW(2, true)},
  };
#undef DPG_GROW
  if (layout < 0 || layout > 2 || x3 < 0 || x3 > 1 || out_kind < 0 || out_kind > 2) return nullptr;
  return table[layout][x3][out_kind];
}

// software-pipelined kernels for the 256x256 and 128x128 tiles (BF16x3: the
// 128x128 tile, FP32 or partial output)
template <int BM, int BN, int WM_, int WN_, int LAYOUT>
struct FastRow {
  static constexpr KernelFn fns[3] = {
      &gemm_fast_kernel<BM, BN, WM_, WN_, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_BF16>,
      &gemm_fast_kernel<BM, BN, WM_, WN_, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_F32>,
      &gemm_fast_kernel<BM, BN, WM_, WN_, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_PARTIAL>};
};

template <int LAYOUT>
struct FastRowX3 {
  static constexpr KernelFn fns[3] = {
      nullptr,
      &gemm_fast_kernel<128, 128, 2, 2, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_F32, true>,
      &gemm_fast_kernel<128, 128, 2, 2, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_PARTIAL, true>};
};

KernelFn lookup_fast_kernel(int tile, int layout, int x3, int out_kind) {
#define DPG_FROW(BM, BN, WM_, WN_, L) \
  {FastRow<BM, BN, WM_, WN_, L>::fns[0], FastRow<BM, BN, WM_, WN_, L>::fns[1], FastRow<BM, BN, WM_, WN_, L>::fns[2]}
  static const KernelFn table[2][3][3] = {
      {DPG_FROW(256, 256, 2, 4, 0), DPG_FROW(256, 256, 2, 4, 1), DPG_FROW(256, 256, 2, 4, 2)},
      {DPG_FROW(128, 128, 2, 2, 0), DPG_FROW(128, 128, 2, 2, 1), DPG_FROW(128, 128, 2, 2, 2)},
  };
#undef DPG_FROW
  static const KernelFn table_x3[3][3] = {
      {FastRowX3<0>::fns[0], FastRowX3<0>::fns[1], FastRowX3<0>::fns[2]},
      {FastRowX3<1>::fns[0], FastRowX3<1>::fns[1], FastRowX3<1>::fns[2]},
      {FastRowX3<2>::fns[0], FastRowX3<2>::fns[1], FastRowX3<2>::fns[2]},
  };
  if (layout < 0 || layout > 2 || out_kind < 0 || out_kind > 2) return nullptr;
  if (x3) return tile == 1 ? table_x3[layout][out_kind] : nullptr;
  if (tile < 0 || tile > 1) return nullptr;
  return table[tile][layout][out_kind];
}

// stream-K variants of the pipelined 256x256 BF16 kernel (BF16 or FP32 output)
template <int LAYOUT>
struct StreamKRow {
  static constexpr KernelFn fns[2] = {
      &gemm_fast_kernel<256, 256, 2, 4, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_BF16, false, true>,
      &gemm_fast_kernel<256, 256, 2, 4, LAYOUT != LAYOUT_WGRAD, LAYOUT == LAYOUT_FWD, OUT_F32, false, true>};
};

KernelFn lookup_streamk_kernel(int tile, int layout, int out_kind) {
  static const KernelFn table[3][2] = {{StreamKRow<0>::fns[0], StreamKRow<0>::fns[1]},
                                       {StreamKRow<1>::fns[0], StreamKRow<1>::fns[1]},
                                       {StreamKRow<2>::fns[0], StreamKRow<2>::fns[1]}};
  if (tile != 0 || layout < 0 || layout > 2 || (out_kind != OUT_BF16 && out_kind != OUT_F32)) return nullptr;
  return table[layout][out_kind];
}

// FP32 FMA router kernel for (layout, out kind); FP32 or partial output only
KernelFn lookup_ffma_kernel(int layout, int out_kind) {
  static const KernelFn table[3][2] = {
      {&ffma_kernel<true, true, OUT_F32>, &ffma_kernel<true, true, OUT_PARTIAL>},
      {&ffma_kernel<true, false, OUT_F32>, &ffma_kernel<true, false, OUT_PARTIAL>},
      {&ffma_kernel<false, false, OUT_F32>, &ffma_kernel<false, false, OUT_PARTIAL>},
  };
  if (layout < 0 || layout > 2 || (out_kind != OUT_F32 && out_kind != OUT_PARTIAL)) return nullptr;
  return table[layout][out_kind == OUT_F32 ? 0 : 1];
}

// skinny weight-gradient kernels: (64-row blocks NB, 64-column blocks CB, out kind)
typedef void (*SkinnyFn)(SkinnyParams);
template <int NB, int CB>
struct SkinnyRow {
  static constexpr SkinnyFn fns[3] = {&skinny_wgrad_kernel<NB, CB, OUT_BF16>, &skinny_wgrad_kernel<NB, CB, OUT_F32>,
                                      &skinny_wgrad_kernel<NB, CB, OUT_PARTIAL>};
};

SkinnyFn lookup_skinny_kernel(int nb, int cb, int out_kind) {
  // one row block and 128-column units: the kernel without LDS staging
  if (nb == 1 && cb == 2) {
    static const SkinnyFn direct[3] = {&skinny_direct_kernel<OUT_BF16>, &skinny_direct_kernel<OUT_F32>,
                                       &skinny_direct_kernel<OUT_PARTIAL>};
    return out_kind >= 0 && out_kind <= 2 ? direct[out_kind] : nullptr;
  }
  // two row blocks, 128- or 64-column units: operands fetched straight into LDS
  if (nb == 2 && (cb == 1 || cb == 2)) {
    static const SkinnyFn lds[2][3] = {
        {&skinny_lds_kernel<1, OUT_BF16>, &skinny_lds_kernel<1, OUT_F32>, &skinny_lds_kernel<1, OUT_PARTIAL>},
        {&skinny_lds_kernel<2, OUT_BF16>, &skinny_lds_kernel<2, OUT_F32>, &skinny_lds_kernel<2, OUT_PARTIAL>}};
    return out_kind >= 0 && out_kind <= 2 ? lds[cb - 1][out_kind] : nullptr;
  }
  // one row block and 64-column units (forced small split counts): the
  // LDS-staged kernel with register transposes (the LDS-fetching kernel, whose
  // second row block would read zeros, measured 11% slower there)
  if (nb == 1 && cb == 1 && out_kind >= 0 && out_kind <= 2) return SkinnyRow<1, 1>::fns[out_kind];
  return nullptr;
}

// ----------------------------------------------------------- plan cache --
struct KeyHash {
  size_t operator()(const PlanKey& k) const {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&h](uint64_t v) { h = (h ^ v) * 1099511628211ull; };
    mix((uint64_t)k.pass);
    mix((uint64_t)k.T);
    mix((uint64_t)k.N);
    mix((uint64_t)k.K);
    mix((uint64_t)k.out);
    mix((uint64_t)k.det);
    mix((uint64_t)k.split_req);
    mix((uint64_t)k.cus);
    mix((uint64_t)k.batch);
    mix((uint64_t)k.wlayout);
    mix((uint64_t)k.router_arith);
    mix((uint64_t)k.generation);
    return (size_t)h;
  }
};

// Plans cached per key (never a data pointer).  The cache holds at most
// kCacheCap plans and drops the least recently used one beyond that, so a
// stream of distinct token counts keeps it bounded.  Keys carry the cache
// generation that dpg_clear_plan_cache bumps.
constexpr size_t kCacheCap = 4096;
struct CacheEntry {
  PlanKey key;
  Plan plan;
};
std::atomic<int> g_router_arith{ROUTER_AUTO};
std::mutex g_mu;
std::list<CacheEntry>* g_lru = nullptr;  // most recently used first
std::unordered_map<PlanKey, std::list<CacheEntry>::iterator, KeyHash>* g_index = nullptr;
int64_t g_generation = 0;

// CU count of the current device (fast mode only), cached per device id.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDetCus;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = kDetCus;
    cached[dev] = cus;
  }
  return cached[dev];
}

bool get_plan(const PlanKey& key_in, Plan* plan) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_lru) {
    g_lru = new std::list<CacheEntry>();
    g_index = new std::unordered_map<PlanKey, std::list<CacheEntry>::iterator, KeyHash>();
  }
  PlanKey key = key_in;
  key.generation = g_generation;
  auto it = g_index->find(key);
  if (it != g_index->end()) {
    g_lru->splice(g_lru->begin(), *g_lru, it->second);
    *plan = it->second->plan;
    return true;
  }
  if (!make_plan(key, plan)) return false;
  g_lru->push_front(CacheEntry{key, *plan});
  (*g_index)[key] = g_lru->begin();
  while (g_lru->size() > kCacheCap) {
    g_index->erase(g_lru->back().key);
    g_lru->pop_back();
  }
  return true;
}

PlanKey make_key(int pass, int64_t T, int64_t N, int64_t K, int out, int det, int split_k, bool query_device) {
  PlanKey k;
  k.pass = pass;
  k.T = T;
  k.N = N;
  k.K = K;
  k.out = out;
  k.det = det ? 1 : 0;
  k.split_req = split_k;
  k.cus = det ? kDetCus : (query_device ? device_cus() : kDetCus);
  k.router_arith = pass >= 3 ? g_router_arith.load() : ROUTER_AUTO;
  return k;
}

// ----------------------------------------------------------- validation --
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Mat {
  const void* ptr;
  int64_t ld, rows, cols;
  int elt;  // bytes per element
};

dpg_status check_mat(const Mat& m) {
  if (m.rows < 0 || m.cols < 0) return DPG_ERR_INVALID_ARG;
  if (m.rows == 0 || m.cols == 0) return DPG_OK;  // empty: pointer and ld unused
  if (!m.ptr) return DPG_ERR_INVALID_ARG;
  if (m.ld < m.cols) return DPG_ERR_INVALID_ARG;
  if (!aligned16(m.ptr) || (m.ld * m.elt) % 16 != 0 || m.cols % 8 != 0) return DPG_ERR_ALIGNMENT;
  return DPG_OK;
}

// fixed-order sum of the split partials in the workspace, converted to the output type
dpg_status launch_reduce(const Plan& plan, void* ws, void* c, int64_t ldc, int64_t c_batch, int out,
                         hipStream_t stream) {
  // x: 256 quads of a row per workgroup; y: rows of all problems, up to about
  // 2048 workgroups in all
  const int gx = (int)((plan.N / 4 + 255) / 256);
  const int gy = (int)std::max<int64_t>(1, std::min<int64_t>(plan.M * plan.batch, std::max(1, 2048 / gx)));
  const float* wsf = (const float*)ws;
  int S = plan.splits, M = (int)plan.M, Nn = (int)plan.N;
  int64_t stride = plan.M * plan.N;
  int64_t batch = plan.batch;
  void* rargs[] = {&wsf, &S, &stride, &M, &Nn, &c, &ldc, &batch, &c_batch};
  hipError_t e = hipLaunchKernel(out == DPG_BF16 ? (const void*)&splitk_reduce_kernel<OUT_BF16>
                                                 : (const void*)&splitk_reduce_kernel<OUT_F32>,
                                 dim3(gx, gy), dim3(256), rargs, 0, stream);
  return e == hipSuccess ? DPG_OK : DPG_ERR_HIP;
}

// One operand or output of a call: pointer, row stride, shape, element size
// and the stride between consecutive problems of a batched call.
struct Operand {
  const void* ptr;
  int64_t ld, rows, cols;
  int elt;
  int64_t bstride;
};

dpg_status check_operand(const Operand& o, int64_t batch, bool output) {
  dpg_status st = check_mat(Mat{o.ptr, o.ld, o.rows, o.cols, o.elt});
  if (st != DPG_OK) return st;
  if (o.cols % 8) return DPG_ERR_ALIGNMENT;
  if (batch > 1 && o.rows > 0 && o.cols > 0) {
    if (o.bstride < 0) return DPG_ERR_INVALID_ARG;
    if ((o.bstride * o.elt) % 16 != 0) return DPG_ERR_ALIGNMENT;
    // outputs of different problems must not overlap: either stacked (each
    // problem past the previous one's last element) or interleaved within
    // rows (disjoint column ranges of one row stride)
    if (output) {
      const bool stacked = o.bstride >= (o.rows - 1) * o.ld + o.cols;
      const bool interleaved = o.bstride >= o.cols && (batch - 1) * o.bstride + o.cols <= o.ld;
      if (!stacked && !interleaved) return DPG_ERR_INVALID_ARG;
    }
  }
  return DPG_OK;
}

// ---------------------------------------------------------------- launch --
// Runs `batch` problems of one pass.  For the projection passes (a, b) are
// (x, w), (dy, w) and (dy, x) as in the entry points; `wlayout` says whether the
// weight (for the weight gradient: the output) is stored [N,K] or [K,N].
dpg_status run(int pass, int wlayout, int64_t batch, const void* a, int64_t lda, int64_t sa, const void* b,
               int64_t ldb, int64_t sb, void* c, int64_t ldc, int64_t sc, int out, int64_t T, int64_t N, int64_t K,
               int det, int split_k, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (out != DPG_BF16 && out != DPG_F32) return DPG_ERR_INVALID_ARG;
  if (T < 0 || N < 0 || K < 0 || batch < 0) return DPG_ERR_INVALID_ARG;
  if (wlayout != WEIGHT_NK && wlayout != WEIGHT_KN) return DPG_ERR_INVALID_ARG;
  if (split_k < 0 || split_k > 64) return DPG_ERR_UNSUPPORTED;
  const int in_elt = pass >= 3 ? 4 : 2;
  const int out_elt = out == DPG_F32 ? 4 : 2;
  const bool kn = wlayout == WEIGHT_KN;
  // operand and output shapes as the caller holds them
  Operand ma, mb, mc;
  switch (pass % 3) {
    case 0:  // Y[T,N] = X[T,K] W^T, W [N,K] or [K,N]
      ma = {a, lda, T, K, in_elt, sa};
      mb = kn ? Operand{b, ldb, K, N, in_elt, sb} : Operand{b, ldb, N, K, in_elt, sb};
      mc = {c, ldc, T, N, out_elt, sc};
      break;
    case 1:  // dX[T,K] = dY[T,N] W
      ma = {a, lda, T, N, in_elt, sa};
      mb = kn ? Operand{b, ldb, K, N, in_elt, sb} : Operand{b, ldb, N, K, in_elt, sb};
      mc = {c, ldc, T, K, out_elt, sc};
      break;
    default:  // dW = dY^T X into [N,K], or X^T dY into [K,N]
      ma = {a, lda, T, N, in_elt, sa};
      mb = {b, ldb, T, K, in_elt, sb};
      mc = kn ? Operand{c, ldc, K, N, out_elt, sc} : Operand{c, ldc, N, K, out_elt, sc};
      break;
  }
  dpg_status st;
  if ((st = check_operand(ma, batch, false)) != DPG_OK) return st;
  if ((st = check_operand(mb, batch, false)) != DPG_OK) return st;
  if ((st = check_operand(mc, batch, true)) != DPG_OK) return st;

  PlanKey key = make_key(pass, T, N, K, out, det, split_k, true);
  key.batch = batch;
  key.wlayout = wlayout;
  Plan plan;
  if (!get_plan(key, &plan)) return DPG_ERR_INVALID_ARG;
  if (plan.kind == PLAN_NOOP) return DPG_OK;
  if (plan.ws_bytes > 0) {
    if (ws_bytes < plan.ws_bytes) return DPG_ERR_WORKSPACE;
    if (!ws || !aligned16(ws)) return DPG_ERR_WORKSPACE;
  }
  // GEMM operands: a weight gradient into [K,N] takes X as A and dY as B
  if (plan.swap_ab) {
    std::swap(a, b);
    std::swap(lda, ldb);
    std::swap(sa, sb);
  }

  if (plan.kind == PLAN_ZERO) {
    const int64_t quads = batch * plan.M * (plan.N / 4);
    const int grid = (int)std::min<int64_t>((quads + 255) / 256, 4096);
    int M = (int)plan.M, Nn = (int)plan.N;
    int64_t bt = batch;
    void* args[] = {&M, &Nn, &c, &ldc, &bt, &sc};
    hipError_t e = hipLaunchKernel(out == DPG_BF16 ? (const void*)&zero_fill_kernel<OUT_BF16>
                                                   : (const void*)&zero_fill_kernel<OUT_F32>,
                                   dim3(grid), dim3(256), args, 0, stream);
    return e == hipSuccess ? DPG_OK : DPG_ERR_HIP;
  }

  // The skinny kernels' 64-token tiles span at most 64 * ld * 2 bytes of
  // 32-bit buffer offsets (below 2^31 for ld < 2^23), the pipelined kernels'
  // 256-row K-major tiles 256 * ld * 2 bytes (ld < 2^22); wider strides run the
  // same plan (same K partition and workspace) on the generic kernel.
  const int64_t ld_max = std::max(lda, ldb);
  if ((plan.skinny && ld_max >= (1 << 23)) || (!plan.skinny && plan.fast && ld_max >= (1 << 22))) {
    if (!generic_fallback(&plan)) return DPG_ERR_UNSUPPORTED;
  }
  if (plan.skinny) {
    SkinnyParams q;
    q.dy = a;
    q.x = b;
    q.lddy = lda;
    q.ldx = ldb;
    q.T = (int)plan.K;
    q.N = (int)plan.M;
    q.K = (int)plan.N;
    q.splits = plan.splits;
    q.tb_total = plan.kt_total;
    q.tb_per_split = plan.kt_per_split;
    q.k_blocks = (int)((plan.N + plan.skinny_cols - 1) / plan.skinny_cols);
    const int nb = plan.M > 64 ? 2 : 1;  // 64-row blocks of dW per unit
    const int cb = plan.skinny_cols / 64;
    const int okind = plan.splits > 1 ? OUT_PARTIAL : (out == DPG_BF16 ? OUT_BF16 : OUT_F32);
    const void* kfn = (const void*)lookup_skinny_kernel(nb, cb, okind);
    if (!kfn) return DPG_ERR_INVALID_ARG;
    if (plan.splits > 1) {
      q.out = ws;
      q.ldo = plan.N;
      q.split_stride = plan.M * plan.N;
    } else {
      q.out = c;
      q.ldo = ldc;
      q.split_stride = 0;
    }
    void* sargs[] = {&q};
    hipError_t e = hipLaunchKernel(kfn, dim3((unsigned)plan.grid), dim3(512), sargs, 0, stream);
    if (e != hipSuccess) return DPG_ERR_HIP;
    if (plan.splits > 1) return launch_reduce(plan, ws, c, ldc, sc, out, stream);
    return DPG_OK;
  }

  GemmParams p{};
  p.a = a;
  p.b = b;
  p.lda = lda;
  p.ldb = ldb;
  p.M = (int)plan.M;
  p.N = (int)plan.N;
  p.K = (int)plan.K;
  p.tiles_m = plan.tiles_m;
  p.tiles_n = plan.tiles_n;
  p.splits = plan.splits;
  p.kt_total = plan.kt_total;
  p.kt_per_split = plan.kt_per_split;
  p.group_m = plan.group_m;
  p.batch = (int)batch;
  p.batch_a = sa;
  p.batch_b = sb;
  int out_kind;
  if (plan.splits > 1) {
    p.c = ws;
    p.ldc = plan.N;
    p.split_stride = plan.M * plan.N;
    p.batch_c = (int64_t)plan.splits * p.split_stride;
    out_kind = OUT_PARTIAL;
  } else {
    p.c = c;
    p.ldc = ldc;
    p.split_stride = 0;
    p.batch_c = sc;
    out_kind = out == DPG_BF16 ? OUT_BF16 : OUT_F32;
  }
  if (plan.streamk) {
    // stream-K: exactly plan.grid workgroups (the partition depends on it),
    // then the fix-up of the tail tiles that ranges share
    p.sk_ws = ws;
    KernelFn sfn = lookup_streamk_kernel(plan.tile, plan.layout, out_kind);
    if (!sfn) return DPG_ERR_INVALID_ARG;
    void* sargs[] = {&p};
    hipError_t e = hipLaunchKernel((const void*)sfn, dim3((unsigned)plan.grid), dim3(512), sargs, 0, stream);
    if (e != hipSuccess) return DPG_ERR_HIP;
    const int tiles = plan.tiles_m * plan.tiles_n;
    const int G = (int)plan.grid;
    const int D = (tiles / G) * G;
    int bm = kTiles[plan.tile].bm, bn = kTiles[plan.tile].bn;
    void* fargs[] = {&p, &bm, &bn, (void*)&G};
    e = hipLaunchKernel(out == DPG_BF16 ? (const void*)&streamk_fixup_kernel<OUT_BF16>
                                        : (const void*)&streamk_fixup_kernel<OUT_F32>,
                        dim3((unsigned)(std::max(tiles - D, 1) * kStreamKFixupChunks)), dim3(256), fargs, 0, stream);
    return e == hipSuccess ? DPG_OK : DPG_ERR_HIP;
  }
  const bool fast = plan.fast != 0;
  KernelFn fn = plan.ffma ? lookup_ffma_kernel(plan.layout, out_kind)
                : fast    ? lookup_fast_kernel(plan.tile, plan.layout, plan.x3, out_kind)
                          : (plan.tile == kGenericTile ? lookup_generic_kernel(plan.layout, plan.x3, out_kind) : nullptr);
  if (!fn) return DPG_ERR_INVALID_ARG;
  void* args[] = {&p};
  const int threads = (fast && plan.tile == 0) ? 512 : 256;
  // the pipelined kernel is persistent: one workgroup per CU slot walks its units
  // (one per CU for the 256x256 tile and for BF16x3, whose two hi/lo planes
  // fill the LDS; two for the BF16 128x128 tile)
  int64_t grid = plan.grid;
  if (fast) grid = std::min<int64_t>(grid, (int64_t)device_cus() * ((plan.tile == 0 || plan.x3) ? 1 : 2));
  hipError_t e = hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3(threads), args, 0, stream);
  if (e != hipSuccess) return DPG_ERR_HIP;
  if (plan.splits > 1) return launch_reduce(plan, ws, c, ldc, sc, out, stream);
  return DPG_OK;
}

// the single-problem form used by the unbatched entry points
dpg_status run(int pass, const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc, int out,
               int64_t T, int64_t N, int64_t K, int det, int split_k, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  return run(pass, WEIGHT_NK, 1, a, lda, 0, b, ldb, 0, c, ldc, 0, out, T, N, K, det, split_k, ws, ws_bytes,
             stream);
}

}  // namespace
}  // namespace dpg

// ------------------------------------------------ no-allocation scratch --
// Split partials of dpg_wgrad_noalloc live in this array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy (from the first
// use of the library's code on that device until the process ends).  Host
// code never passes the array's name to a kernel: it uses the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[DPG_NOALLOC_SCRATCH_BYTES];

namespace dpg {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of the current device's scratch array, looked up once per
// device (with that device current); null on failure.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace dpg

using namespace dpg;

extern "C" {

dpg_status dpg_forward(const void* x, int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                       dpg_dtype y_dtype, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_FORWARD, x, ldx, w, ldw, y, ldy, y_dtype, T, N, K, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_dgrad(const void* dy, int64_t lddy, const void* w, int64_t ldw, void* dx, int64_t lddx,
                     dpg_dtype dx_dtype, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_DGRAD, dy, lddy, w, ldw, dx, lddx, dx_dtype, T, N, K, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_wgrad(const void* dy, int64_t lddy, const void* x, int64_t ldx, void* dw, int64_t lddw,
                     dpg_dtype dw_dtype, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_WGRAD, dy, lddy, x, ldx, dw, lddw, dw_dtype, T, N, K, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_wgrad_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx, void* dw, int64_t lddw,
                             dpg_dtype dw_dtype, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                             hipStream_t stream) {
  // the plan (and so the bits) of dpg_wgrad; its partials go to the scratch
  // array, and a plan that needs more than the array holds is refused before
  // any launch (run() checks the size against the bytes passed here)
  void* ws = device_scratch();
  if (!ws) return DPG_ERR_HIP;
  return run(DPG_PASS_WGRAD, dy, lddy, x, ldx, dw, lddw, dw_dtype, T, N, K, deterministic, split_k, ws,
             (size_t)DPG_NOALLOC_SCRATCH_BYTES, stream);
}

size_t dpg_noalloc_scratch_bytes(void) { return (size_t)DPG_NOALLOC_SCRATCH_BYTES; }

dpg_status dpg_router_forward(const float* x, int64_t ldx, const float* w, int64_t ldw, float* y, int64_t ldy,
                              int64_t T, int64_t E, int64_t H, int deterministic, int split_k, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_ROUTER_FORWARD, x, ldx, w, ldw, y, ldy, DPG_F32, T, E, H, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_router_dgrad(const float* dy, int64_t lddy, const float* w, int64_t ldw, float* dx, int64_t lddx,
                            int64_t T, int64_t E, int64_t H, int deterministic, int split_k, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_ROUTER_DGRAD, dy, lddy, w, ldw, dx, lddx, DPG_F32, T, E, H, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_router_wgrad(const float* dy, int64_t lddy, const float* x, int64_t ldx, float* dw, int64_t lddw,
                            int64_t T, int64_t E, int64_t H, int deterministic, int split_k, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_ROUTER_WGRAD, dy, lddy, x, ldx, dw, lddw, DPG_F32, T, E, H, deterministic, split_k, workspace,
             workspace_bytes, stream);
}

dpg_status dpg_forward_batched(const void* x, int64_t ldx, int64_t stride_x, const void* w, int64_t ldw,
                               int64_t stride_w, dpg_weight_layout w_layout, void* y, int64_t ldy, int64_t stride_y,
                               dpg_dtype y_dtype, int64_t batch, int64_t T, int64_t N, int64_t K, int deterministic,
                               int split_k, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_FORWARD, (int)w_layout, batch, x, ldx, stride_x, w, ldw, stride_w, y, ldy, stride_y, y_dtype,
             T, N, K, deterministic, split_k, workspace, workspace_bytes, stream);
}

dpg_status dpg_dgrad_batched(const void* dy, int64_t lddy, int64_t stride_dy, const void* w, int64_t ldw,
                             int64_t stride_w, dpg_weight_layout w_layout, void* dx, int64_t lddx, int64_t stride_dx,
                             dpg_dtype dx_dtype, int64_t batch, int64_t T, int64_t N, int64_t K, int deterministic,
                             int split_k, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_DGRAD, (int)w_layout, batch, dy, lddy, stride_dy, w, ldw, stride_w, dx, lddx, stride_dx,
             dx_dtype, T, N, K, deterministic, split_k, workspace, workspace_bytes, stream);
}

dpg_status dpg_wgrad_batched(const void* dy, int64_t lddy, int64_t stride_dy, const void* x, int64_t ldx,
                             int64_t stride_x, void* dw, int64_t lddw, int64_t stride_dw, dpg_weight_layout w_layout,
                             dpg_dtype dw_dtype, int64_t batch, int64_t T, int64_t N, int64_t K, int deterministic,
                             int split_k, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run(DPG_PASS_WGRAD, (int)w_layout, batch, dy, lddy, stride_dy, x, ldx, stride_x, dw, lddw, stride_dw,
             dw_dtype, T, N, K, deterministic, split_k, workspace, workspace_bytes, stream);
}

size_t dpg_workspace_size_batched(dpg_pass pass, dpg_weight_layout w_layout, int64_t batch, int64_t T, int64_t N,
                                  int64_t K, dpg_dtype out_dtype, int deterministic, int split_k) {
  if ((int)pass < 0 || (int)pass >= 3) return (size_t)-1;
  PlanKey key = make_key((int)pass, T, N, K, (int)out_dtype, deterministic, split_k, true);
  key.batch = batch;
  key.wlayout = (int)w_layout;
  Plan plan;
  if (!get_plan(key, &plan)) return (size_t)-1;
  return plan.kind == PLAN_GEMM ? plan.ws_bytes : 0;
}

dpg_status dpg_plan_describe_batched(dpg_pass pass, dpg_weight_layout w_layout, int64_t batch, int64_t T, int64_t N,
                                     int64_t K, dpg_dtype out_dtype, int deterministic, int split_k, char* buf,
                                     size_t buflen) {
  if (!buf || buflen == 0) return DPG_ERR_INVALID_ARG;
  if ((int)pass < 0 || (int)pass >= 3) return DPG_ERR_INVALID_ARG;
  PlanKey key = make_key((int)pass, T, N, K, (int)out_dtype, deterministic, split_k, false);
  key.batch = batch;
  key.wlayout = (int)w_layout;
  Plan plan;
  if (!make_plan(key, &plan)) return DPG_ERR_INVALID_ARG;
  describe_plan(key, plan, buf, buflen);
  return DPG_OK;
}

size_t dpg_workspace_size(dpg_pass pass, int64_t T, int64_t N, int64_t K, dpg_dtype out_dtype, int deterministic,
                          int split_k) {
  if ((int)pass >= 3 && out_dtype != DPG_F32) return (size_t)-1;
  Plan plan;
  if (!get_plan(make_key((int)pass, T, N, K, (int)out_dtype, deterministic, split_k, true), &plan))
    return (size_t)-1;
  return plan.kind == PLAN_GEMM ? plan.ws_bytes : 0;
}

dpg_status dpg_plan_describe(dpg_pass pass, int64_t T, int64_t N, int64_t K, dpg_dtype out_dtype, int deterministic,
                             int split_k, char* buf, size_t buflen) {
  if (!buf || buflen == 0) return DPG_ERR_INVALID_ARG;
  if ((int)pass >= 3 && out_dtype != DPG_F32) return DPG_ERR_INVALID_ARG;
  // host-only: the split-K mode is described for the nominal CU count
  PlanKey key = make_key((int)pass, T, N, K, (int)out_dtype, deterministic, split_k, false);
  Plan plan;
  if (!make_plan(key, &plan)) return DPG_ERR_INVALID_ARG;
  describe_plan(key, plan, buf, buflen);
  return DPG_OK;
}

dpg_status dpg_set_router_arithmetic(dpg_router_arith arith) {
  if ((int)arith < DPG_ROUTER_AUTO || (int)arith > DPG_ROUTER_FP32) return DPG_ERR_INVALID_ARG;
  g_router_arith.store((int)arith);
  return DPG_OK;
}

dpg_router_arith dpg_get_router_arithmetic(void) { return (dpg_router_arith)g_router_arith.load(); }

void dpg_clear_plan_cache(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_lru) {
    g_index->clear();
    g_lru->clear();
  }
  ++g_generation;
}

void dpg_plan_cache_stats(int64_t* entries, int64_t* generation) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (entries) *entries = g_lru ? (int64_t)g_lru->size() : 0;
  if (generation) *generation = g_generation;
}

int64_t dpg_plan_cache_capacity(void) { return (int64_t)kCacheCap; }

const char* dpg_status_string(dpg_status status) {
  switch (status) {
    case DPG_OK: return "ok";
    case DPG_ERR_INVALID_ARG: return "invalid argument";
    case DPG_ERR_UNSUPPORTED: return "unsupported: split_k outside 0..64, or a launch beyond the grid limit";
    case DPG_ERR_ALIGNMENT: return "pointer, leading dimension or column count not 16-byte compatible";
    case DPG_ERR_WORKSPACE: return "workspace missing or too small";
    case DPG_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* dpg_version(void) { return "dpg 0.1.0 gfx950"; }

}  // extern "C"
