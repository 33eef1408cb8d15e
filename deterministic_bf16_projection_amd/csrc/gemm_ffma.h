// FP32 router GEMM on the vector ALUs (no matrix cores): C[M,N] = sum_k
// A(m,k) * B(n,k) with FP32 operands, one FP32 fused multiply-add per product,
// in ascending k.  The small-T window of the router page, where library FP32
// calls beat the BF16x3 emulation (router page, ratio table; the wgrad page's
// timeline keeps a router FFMA window).
//
// Workgroup = one 64x64 output tile of one K split, 256 threads, each thread
// a 4x4 block of outputs (rows 4 (t / 16) .., columns 4 (t % 16) ..).  The
// split's K range is walked in chunks of 16: a chunk of each operand (64 rows
// x 16 k) is fetched with one 16-byte load per thread into registers (the
// next chunk's loads are issued before the current chunk's products), then
// written to LDS k-major ([k][row], row padded to 68 floats), from where each
// thread reads 4 consecutive A rows and 4 consecutive B columns per k.  Rows
// past M / N and k past K read as zero.  The output (FP32, or the split's
// partial plane) is written as 16-byte row segments.
#pragma once
#include "device_common.h"
#include "gemm_kernel.h"

namespace dpg {

template <bool KMAJ>
struct FfmaOperand {
  static constexpr int LD = 68;  // floats per k-row of the LDS chunk [16][64 + 4]
  f32x4 v;
  // chunk of 64 rows x 16 k at (row0, k0): K-major thread t takes row t / 4,
  // k 4 (t % 4) ..; MN-major (element (row, k) at ptr[k ld + row]) k t / 16,
  // rows 4 (t % 16) ..
  __device__ __forceinline__ void load(const float* __restrict__ ptr, int64_t ld, int row0, int rows, int k0, int K,
                                       int tid) {
    int r, k;
    if (KMAJ) {
      r = tid >> 2;
      k = (tid & 3) * 4;
    } else {
      k = tid >> 4;
      r = (tid & 15) * 4;
    }
    const int gr = row0 + r, gk = k0 + k;
    v = f32x4{0.f, 0.f, 0.f, 0.f};
    // K % 4 == 0 and rows % 4 == 0 (contiguous extents are multiples of 8), so
    // a 4-wide group is either all inside or all outside
    if (gr < rows && gk < K) v = KMAJ ? *(const f32x4*)(ptr + (int64_t)gr * ld + gk) : *(const f32x4*)(ptr + (int64_t)gk * ld + gr);
  }
  __device__ __forceinline__ void store(float* lds, int tid) const {
    if (KMAJ) {
      const int r = tid >> 2, k = (tid & 3) * 4;
      lds[(k + 0) * LD + r] = v[0];
      lds[(k + 1) * LD + r] = v[1];
      lds[(k + 2) * LD + r] = v[2];
      lds[(k + 3) * LD + r] = v[3];
    } else {
      const int k = tid >> 4, r = (tid & 15) * 4;
      *(f32x4*)(lds + k * LD + r) = v;
    }
  }
};

template <bool A_KMAJ, bool B_KMAJ, int OUT>
__global__ void __launch_bounds__(256) ffma_kernel(GemmParams p) {
  static_assert(OUT == OUT_F32 || OUT == OUT_PARTIAL, "FP32 output");
  constexpr int LD = FfmaOperand<true>::LD;
  constexpr int CHUNK = 16 * LD;
  __shared__ __attribute__((aligned(16))) float sa[2][CHUNK];
  __shared__ __attribute__((aligned(16))) float sb[2][CHUNK];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  // tile and split of this workgroup (the generic kernel's mapping)
  const int tiles = p.tiles_m * p.tiles_n;
  const int pid = xcd_remap(blockIdx.x, tiles * p.splits);
  const int split = pid / tiles;
  const int t = pid - split * tiles;
  const int per_group = p.group_m * p.tiles_n;
  const int group = t / per_group;
  const int first_m = group * p.group_m;
  const int gsize = min(p.tiles_m - first_m, p.group_m);
  const int row0 = (first_m + (t % per_group) % gsize) * 64;
  const int col0 = ((t % per_group) / gsize) * 64;
  const SplitParts sp = split_parts(p.splits, p.kt_total);
  const int k_begin = split_begin(split, sp) * 64;
  const int k_end = min(split_begin(split + 1, sp) * 64, p.K);

  const float* A = (const float*)p.a;
  const float* B = (const float*)p.b;
  FfmaOperand<A_KMAJ> oa;
  FfmaOperand<B_KMAJ> ob;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  int buf = 0;
  if (k_begin < k_end) {
    oa.load(A, p.lda, row0, p.M, k_begin, p.K, tid);
    ob.load(B, p.ldb, col0, p.N, k_begin, p.K, tid);
    oa.store(sa[0], tid);
    ob.store(sb[0], tid);
  }
  __syncthreads();
  for (int k0 = k_begin; k0 < k_end; k0 += 16) {
    const bool more = k0 + 16 < k_end;
    if (more) {
      oa.load(A, p.lda, row0, p.M, k0 + 16, p.K, tid);
      ob.load(B, p.ldb, col0, p.N, k0 + 16, p.K, tid);
    }
    const float* ca = sa[buf];
    const float* cb = sb[buf];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const f32x4 a = *(const f32x4*)(ca + kk * LD + ty * 4);
      const f32x4 b = *(const f32x4*)(cb + kk * LD + tx * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (more) {
      oa.store(sa[buf ^ 1], tid);
      ob.store(sb[buf ^ 1], tid);
    }
    __syncthreads();
    buf ^= 1;
  }

  const int n = col0 + tx * 4;
  if (n >= p.N) return;
  float* out = (float*)p.c + (OUT == OUT_PARTIAL ? (int64_t)split * p.split_stride : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = row0 + ty * 4 + i;
    if (m < p.M) *(f32x4*)(out + (int64_t)m * p.ldc + n) = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
  }
}

}  // namespace dpg
