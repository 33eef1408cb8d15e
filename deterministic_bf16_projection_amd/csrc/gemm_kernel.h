// Tiled BF16 MFMA GEMM for gfx950: C[M,N] = sum_k A(m,k) * B(n,k).
//
// One kernel template serves the three projection passes and the router:
//   forward  : A = X  (K-major), B = W (K-major)
//   dgrad    : A = dY (K-major), B = W (MN-major: contiguous along the output)
//   wgrad    : A = dY (MN-major), B = X (MN-major), reducing over tokens
// X3 = true reads FP32 operands and applies the BF16x3 split while staging
// them into LDS; each k-step then issues lo*hi, hi*lo, hi*hi MFMAs into one
// FP32 accumulator.
//
// Data path per workgroup (one BM x BN output tile, one K split):
//   global --16 B vector loads--> registers --> LDS (two stages)
//   LDS --ds_read_b128 (K-major) / ds_read_b64_tr_b16 (MN-major)--> MFMA
//   32x32x16 BF16 MFMA, FP32 accumulators, fixed k order
//   epilogue: BF16 (nearest even) or FP32 to the output, or FP32 partial
//   tiles to the workspace (reduced later in ascending split order).
#pragma once
#include <type_traits>

#include "device_common.h"

namespace dpg {

enum OutKind { OUT_BF16 = 0, OUT_F32 = 1, OUT_PARTIAL = 2 };

struct GemmParams {
  const void* a;
  const void* b;
  void* c;          // output, or the workspace when OUT_PARTIAL
  int64_t lda, ldb, ldc;
  int64_t split_stride;  // elements between split planes of the workspace
  int M, N, K;
  int tiles_m, tiles_n;
  int splits;
  int kt_total;      // ceil(K / BK)
  int kt_per_split;  // K tiles of the largest split (splits differ by at most one; see split_begin)
  int group_m;       // raster: tiles of one group run down this many tile rows
  int batch;         // independent problems in the launch (units run over all of them)
  int64_t batch_a, batch_b;  // elements between consecutive problems' A and B
  int64_t batch_c;           // elements between outputs (workspace: splits * split_stride)
  void* sk_ws;               // stream-K partial slots (stream-K plans only)
};

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
};

// ---------------------------------------------------------------- operands --
// An operand tile holds R rows (M or N side) by BK reduction elements.
//  K-major source: element (row, k) at ptr[row * ld + k].  LDS layout [R][BK],
//    16-byte chunks XOR-swizzled within each row against bank conflicts.
//  MN-major source: element (row, k) at ptr[k * ld + row].  LDS layout
//    [BK][R + PAD] (rows of the source copied as they are), read back with the
//    transposing ds_read_b64_tr_b16.
template <int R, int BK, bool KMAJ, bool X3, int NT>
struct Operand {
  static constexpr int PAD = 16;                     // MN-major row padding (elements)
  static constexpr int CHUNKS_PER_ROW = BK / 8;      // K-major: 16 B chunks per row
  static constexpr int PLANE = KMAJ ? R * BK : BK * (R + PAD);  // elements per plane
  static constexpr int PLANES = X3 ? 2 : 1;          // hi (and lo) planes
  static constexpr int STAGE_ELEMS = PLANE * PLANES;
  static constexpr int NCHUNK = R * BK / 8;          // 8-element chunks per tile
  static constexpr int PER_THREAD = (NCHUNK + NT - 1) / NT;
  static constexpr bool EXACT = (NCHUNK % NT) == 0;
  typedef typename std::conditional<X3, float, __bf16>::type InT;

  // registers holding one prefetched tile
  u32x4 r0[PER_THREAD];
  u32x4 r1[X3 ? PER_THREAD : 1];

  // which (row, k) a chunk index names, in tile coordinates
  static __device__ __forceinline__ void chunk_coords(int idx, int& row, int& k) {
    if (KMAJ) {
      row = idx / CHUNKS_PER_ROW;
      k = (idx % CHUNKS_PER_ROW) * 8;
    } else {
      k = idx / (R / 8);
      row = (idx % (R / 8)) * 8;
    }
  }

  // Load the tile whose first row is row0 and first reduction index k0.
  // rows_valid / k_valid bound the source; chunks outside read as zero.
  __device__ __forceinline__ void load(const InT* __restrict__ src, int64_t ld, int row0, int k0, int rows_valid,
                                       int k_valid, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int idx = tid + i * NT;
      int row, k;
      chunk_coords(idx, row, k);
      const int grow = row0 + row, gk = k0 + k;
      bool ok = (EXACT || idx < NCHUNK) && grow < rows_valid && gk < k_valid;
      const InT* p = KMAJ ? src + (int64_t)grow * ld + gk : src + (int64_t)gk * ld + grow;
      if (X3) {
        f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
          v0 = *(const f32x4*)(p);
          v1 = *(const f32x4*)(p + 4);
        }
        r0[i] = __builtin_bit_cast(u32x4, v0);
        r1[i] = __builtin_bit_cast(u32x4, v1);
      } else {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = *(const u32x4*)(p);
        r0[i] = v;
      }
    }
  }

  // LDS element offset of chunk (row, k) in a plane
  static __device__ __forceinline__ int lds_offset(int row, int k) {
    if (KMAJ) {
      const int c = k / 8;
      return row * BK + ((c ^ swz(row)) * 8);
    }
    return k * (R + PAD) + row;
  }

  // XOR swizzle of 16-byte chunks within a K-major row: rows that one
  // ds_read_b128 phase touches land on distinct banks.
  static __device__ __forceinline__ int swz(int row) {
    constexpr int ROWS_PER_128B = (BK * 2 >= 128) ? 1 : 128 / (BK * 2);
    constexpr int MASK = (CHUNKS_PER_ROW < 8 ? CHUNKS_PER_ROW : 8) - 1;
    return ((row / ROWS_PER_128B) ^ (row / (8 * ROWS_PER_128B))) & MASK;
  }

  __device__ __forceinline__ void store(__bf16* stage, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int idx = tid + i * NT;
      if (!EXACT && idx >= NCHUNK) continue;
      int row, k;
      chunk_coords(idx, row, k);
      const int off = lds_offset(row, k);
      if (X3) {
        u32x4 hi, lo;
        split3_x8(__builtin_bit_cast(f32x4, r0[i]), __builtin_bit_cast(f32x4, r1[i]), hi, lo);
        if (KMAJ) {
          *(u32x4*)(stage + off) = hi;
          *(u32x4*)(stage + PLANE + off) = lo;
        } else {
          // 8 consecutive rows at one k: contiguous in the MN-major plane
          *(u32x4*)(stage + off) = hi;
          *(u32x4*)(stage + PLANE + off) = lo;
        }
      } else {
        *(u32x4*)(stage + off) = r0[i];
      }
    }
  }

  // MFMA 32x32x16 operand fragment: lane l holds row (row0 + l % 32) and the
  // 8 reduction elements k16 * 16 + (l / 32) * 8 + [0, 8).
  static __device__ __forceinline__ bf16x8 frag(const __bf16* plane, int row0, int k16, int lane) {
    if (KMAJ) {
      const int row = row0 + (lane & 31);
      const int c = k16 * 2 + (lane >> 5);
      return as_bf16x8(*(const u32x4*)(plane + row * BK + ((c ^ swz(row)) * 8)));
    } else {
      // Two transposing reads, each giving 4 consecutive k of one row.
      const int g = lane >> 4, s = lane & 15;
      const int kb = k16 * 16 + (g >> 1) * 8 + (s >> 2);
      const int rb = row0 + 16 * (g & 1) + 4 * (s & 3);
      const u32x2 lo = lds_read_tr16(plane + kb * (R + PAD) + rb);
      const u32x2 hi = lds_read_tr16(plane + (kb + 4) * (R + PAD) + rb);
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  }
};

// --------------------------------------------------------------- the kernel --
template <class Cfg, bool A_KMAJ, bool B_KMAJ, bool X3, int OUT>
__global__ void __launch_bounds__(Cfg::NT) gemm_kernel(GemmParams p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  typedef Operand<BM, BK, A_KMAJ, X3, NT> OpA;
  typedef Operand<BN, BK, B_KMAJ, X3, NT> OpB;
  typedef typename OpA::InT InT;
  constexpr int STAGE = OpA::STAGE_ELEMS + OpB::STAGE_ELEMS;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  // problem, tile and split of this workgroup
  const int tiles = p.tiles_m * p.tiles_n;
  const int per_batch = tiles * p.splits;
  const int pid_all = xcd_remap(blockIdx.x, per_batch * p.batch);
  const int bidx = pid_all / per_batch;
  const int pid = pid_all - bidx * per_batch;
  const int split = pid / tiles;
  const int t = pid % tiles;
  const int per_group = p.group_m * p.tiles_n;
  const int group = t / per_group;
  const int first_m = group * p.group_m;
  const int gsize = min(p.tiles_m - first_m, p.group_m);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int row0 = tm * BM, col0 = tn * BN;

  const SplitParts sp = split_parts(p.splits, p.kt_total);
  const int kt0 = split_begin(split, sp);
  const int kt1 = split_begin(split + 1, sp);
  const int nkt = kt1 - kt0;

  const InT* A = (const InT*)p.a + bidx * p.batch_a;
  const InT* B = (const InT*)p.b + bidx * p.batch_b;
  const int64_t c_off = bidx * p.batch_c;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  OpA opa;
  OpB opb;
  if (nkt > 0) {
    opa.load(A, p.lda, row0, kt0 * BK, p.M, p.K, tid);
    opb.load(B, p.ldb, col0, kt0 * BK, p.N, p.K, tid);
    opa.store(smem, tid);
    opb.store(smem + OpA::STAGE_ELEMS, tid);
  }
  __syncthreads();

  for (int it = 0; it < nkt; ++it) {
    const bool more = it + 1 < nkt;
    if (more) {
      const int k0 = (kt0 + it + 1) * BK;
      opa.load(A, p.lda, row0, k0, p.M, p.K, tid);
      opb.load(B, p.ldb, col0, k0, p.N, p.K, tid);
    }
    const __bf16* sa = smem + (it & 1) * STAGE;
    const __bf16* sb = sa + OpA::STAGE_ELEMS;
#pragma unroll
    for (int k16 = 0; k16 < BK / 16; ++k16) {
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = OpA::frag(sa, wm * Cfg::WM + i * 32, k16, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = OpB::frag(sb, wn * Cfg::WN + j * 32, k16, lane);
      if (X3) {
        bf16x8 la[FM], lb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) la[i] = OpA::frag(sa + OpA::PLANE, wm * Cfg::WM + i * 32, k16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) lb[j] = OpB::frag(sb + OpB::PLANE, wn * Cfg::WN + j * 32, k16, lane);
        // fixed order per k-step: lo*hi, hi*lo, hi*hi
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = mfma32(la[i], fb[j], acc[i][j]);
            acc[i][j] = mfma32(fa[i], lb[j], acc[i][j]);
            acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
      }
    }
    if (more) {
      __bf16* dst = smem + ((it + 1) & 1) * STAGE;
      opa.store(dst, tid);
      opb.store(dst + OpA::STAGE_ELEMS, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane l owns column (l % 32) and rows (r/4)*8 + (l/32)*4 + r%4
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + wn * Cfg::WN + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * Cfg::WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= p.M) continue;
        const float v = acc[i][j][r];
        if (OUT == OUT_BF16) {
          ((unsigned short*)p.c)[c_off + (int64_t)row * p.ldc + col] = (unsigned short)bf16_bits(v);
        } else if (OUT == OUT_F32) {
          ((float*)p.c)[c_off + (int64_t)row * p.ldc + col] = v;
        } else {
          ((float*)p.c)[c_off + (int64_t)split * p.split_stride + (int64_t)row * p.ldc + col] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------ split-K reduction --
// out[b][m, n] = sum over s = 0, 1, ..., S-1 of ws[b][s][m][n], in that order,
// then converted to the output type.  Four columns per thread (N % 8 == 0);
// grid x covers the quads of a row, grid y strides over the rows of all
// problems.  The loads of up to eight planes are issued together and then
// added one after another, so the sum order stays ascending in s.
// v += planes s0, s0 + 1, ..., s0 + R - 1 (in that order) at src; all R loads
// are issued before the first add
template <int R>
__device__ __forceinline__ void add_planes(f32x4& v, const float* src, int s0, int64_t stride) {
  f32x4 w[R];
#pragma unroll
  for (int u = 0; u < R; ++u) w[u] = *(const f32x4*)(src + (int64_t)(s0 + u) * stride);
#pragma unroll
  for (int u = 0; u < R; ++u) {
    v[0] += w[u][0];
    v[1] += w[u][1];
    v[2] += w[u][2];
    v[3] += w[u][3];
  }
}

// v = plane 0 + plane 1 + ... + plane R-1 (in that order) at src
template <int R>
__device__ __forceinline__ void first_planes(f32x4& v, const float* src, int64_t stride) {
  f32x4 w[R];
#pragma unroll
  for (int u = 0; u < R; ++u) w[u] = *(const f32x4*)(src + (int64_t)u * stride);
  v = w[0];
#pragma unroll
  for (int u = 1; u < R; ++u) {
    v[0] += w[u][0];
    v[1] += w[u][1];
    v[2] += w[u][2];
    v[3] += w[u][3];
  }
}

template <int OUT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws, int S, int64_t split_stride,
                                                            int M, int N, void* out, int64_t ldo, int64_t batch,
                                                            int64_t out_batch) {
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= N) return;
  for (int64_t mm = blockIdx.y; mm < batch * M; mm += gridDim.y) {
    const int64_t b = mm / M;
    const int m = (int)(mm - b * M);
    const float* src = ws + b * S * split_stride + (int64_t)m * N + n;
    // planes in batches (the first min(S, 8), then full batches of eight,
    // then the remainder); every load of a batch is issued before its first
    // add (a plane-at-a-time loop waits out one memory round trip per plane),
    // and the adds run in ascending plane order from plane 0
    f32x4 v;
    switch (min(S, 8)) {
      case 8: first_planes<8>(v, src, split_stride); break;
      case 7: first_planes<7>(v, src, split_stride); break;
      case 6: first_planes<6>(v, src, split_stride); break;
      case 5: first_planes<5>(v, src, split_stride); break;
      case 4: first_planes<4>(v, src, split_stride); break;
      case 3: first_planes<3>(v, src, split_stride); break;
      case 2: first_planes<2>(v, src, split_stride); break;
      default: first_planes<1>(v, src, split_stride); break;
    }
    int s = min(S, 8);
    for (; s + 8 <= S; s += 8) add_planes<8>(v, src, s, split_stride);
    switch (S - s) {
      case 7: add_planes<7>(v, src, s, split_stride); break;
      case 6: add_planes<6>(v, src, s, split_stride); break;
      case 5: add_planes<5>(v, src, s, split_stride); break;
      case 4: add_planes<4>(v, src, s, split_stride); break;
      case 3: add_planes<3>(v, src, s, split_stride); break;
      case 2: add_planes<2>(v, src, s, split_stride); break;
      case 1: add_planes<1>(v, src, s, split_stride); break;
      default: break;
    }
    if (OUT == OUT_BF16) {
      u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *(u32x2*)((unsigned short*)out + b * out_batch + (int64_t)m * ldo + n) = o;
    } else {
      *(f32x4*)((float*)out + b * out_batch + (int64_t)m * ldo + n) = v;
    }
  }
}

// Zeros for an empty reduction: out[b][m, n] = 0 for b < batch, m < M, n < N
// (N % 8 == 0); problem b's output starts out_batch elements after b - 1's.
template <int OUT>
__global__ void __launch_bounds__(256) zero_fill_kernel(int M, int N, void* out, int64_t ldo, int64_t batch,
                                                        int64_t out_batch) {
  const int64_t quads = batch * M * (N / 4);
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t mm = q / (N / 4);
    const int64_t b = mm / M;
    const int64_t m = mm - b * M;
    const int n = (int)(q % (N / 4)) * 4;
    const int64_t off = b * out_batch + m * ldo + n;
    if (OUT == OUT_BF16) {
      *(u32x2*)((unsigned short*)out + off) = u32x2{0u, 0u};
    } else {
      *(f32x4*)((float*)out + off) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

}  // namespace dpg
