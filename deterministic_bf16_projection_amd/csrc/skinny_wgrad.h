// Streaming weight gradient for skinny outputs (N <= 128 rows of dW):
//   dW[n, k] = sum_t dY[t, n] * X[t, k]
// The pass reads X[T, K] once from HBM and is bandwidth-bound.
//
// Work unit = (64-row block of N, 64-column block of K, token split).  A
// workgroup has 8 waves; wave w of a unit takes the unit's 64-token blocks
// w, w + 8, w + 16, ... (a fixed assignment), each wave with its own
// accumulators and its own 16 KB LDS region, so the streaming loop has no
// workgroup barrier.  Per block a lane loads one 8x8 BF16 sub-block of X and
// one of dY (16-byte buffer loads; rows past T read as zero), transposes both
// in registers and writes them K-contiguous into the wave's LDS region; the
// MFMA fragments are then single ds_read_b128.  The next block's loads are in
// flight while the current block's MFMAs issue (X two blocks ahead).  At the end the 8 per-wave
// partial tiles are summed in LDS in wave order 0..7 and written once: to the
// output (one token split) or to the FP32 workspace plane of the split.
#pragma once
#include "device_common.h"
#include "gemm_fast.h"

namespace dpg {

struct SkinnyParams {
  const void* dy;  // [T, N] BF16
  const void* x;   // [T, K] BF16
  void* out;       // output [N, K] or FP32 workspace [splits][N][K]
  int64_t lddy, ldx, ldo;
  int64_t split_stride;  // elements between workspace planes
  int T, N, K;
  int n_blocks, k_blocks, splits;
  int tb_total, tb_per_split;  // 64-token blocks and blocks per split
};

template <int OUT>
__global__ void __launch_bounds__(512, 1) skinny_wgrad_kernel(SkinnyParams p) {
  constexpr int W = 8;            // waves
  constexpr int WAVE_ELEMS = 8192;  // BF16 per wave region: dY^T [64][64] + X^T [64][64]
  constexpr int RED_LD = 68;      // FP32 row stride of the reduction buffer
  __shared__ __attribute__((aligned(16))) float smem_f[W * 64 * RED_LD];
  __bf16* smem = (__bf16*)smem_f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // units consecutive in (K block, N block) order share X columns; the XCD
  // remap keeps consecutive units on one XCD so the N blocks of a K block
  // read X through the same L2
  const int per_split = p.n_blocks * p.k_blocks;
  const int unit = xcd_remap(blockIdx.x, per_split * p.splits);
  const int split = unit / per_split;
  const int r = unit - split * per_split;
  const int kb = r / p.n_blocks, nb = r - kb * p.n_blocks;
  const int n0 = nb * 64, c0 = kb * 64;
  const int tb0 = split * p.tb_per_split;
  const int tb1 = min(tb0 + p.tb_per_split, p.tb_total);

  const __bf16* dy = (const __bf16*)p.dy;
  const __bf16* x = (const __bf16*)p.x;
  const int lddy = (int)p.lddy, ldx = (int)p.ldx;

  // lane's 8x8 sub-block: token rows kc*8 + [0,8), columns cb*8 + [0,8)
  const int kc = lane & 7, cb = lane >> 3;
  uint32_t voff_y[8], voff_x[8];
  int lds_off[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    voff_y[l] = (uint32_t)(((kc * 8 + l) * lddy + cb * 8) * 2);
    voff_x[l] = (uint32_t)(((kc * 8 + l) * ldx + cb * 8) * 2);
    lds_off[l] = lds_chunk_off(cb * 8 + l, kc);
  }
  __bf16* wy = smem + wave * WAVE_ELEMS;  // dY^T rows n, 64 tokens each
  __bf16* wx = wy + 4096;                 // X^T rows k, 64 tokens each

  auto rsrc_rows = [&](const __bf16* base, int ld, int col0, int cols, int t0) {
    const int rows = min(p.T - t0, 64);
    int bytes = ((rows - 1) * ld + (cols - col0)) * 2;
    bytes = rows > 0 ? max(bytes, 0) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base + (int64_t)t0 * ld + col0), (short)0, bytes,
                                             0x00020000);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  const int sw = fswz(lr);
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = ((2 * s + lh) ^ sw) << 3;

  // X (streamed from HBM) is fetched two of this wave's blocks ahead; dY (the
  // same rows for every K block, mostly L2 hits) one step before its use.
  u32x4 gx0[8], gx1[8], gy[8];
  auto load_x = [&](u32x4 (&g)[8], int blk) {
    const rsrc_t rx = rsrc_rows(x, ldx, c0, p.K, blk * 64);
#pragma unroll
    for (int l = 0; l < 8; ++l) g[l] = buf_load16(rx, voff_x[l]);
  };
  auto load_y = [&](int blk) {
    const rsrc_t ry = rsrc_rows(dy, lddy, n0, p.N, blk * 64);
#pragma unroll
    for (int l = 0; l < 8; ++l) gy[l] = buf_load16(ry, voff_y[l]);
  };
  auto stage = [&](const u32x4 (&g)[8], __bf16* dst) {
    u32x4 t[8];
    transpose8x8(g, t);
#pragma unroll
    for (int m = 0; m < 8; ++m) *(u32x4*)(dst + lds_off[m]) = t[m];
  };
  auto compute = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = as_bf16x8(*(const u32x4*)(wy + (i * 32 + lr) * 64 + koff[s]));
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = as_bf16x8(*(const u32x4*)(wx + (j * 32 + lr) * 64 + koff[s]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
  };
  // blocks of this wave: b0, b0 + W, b0 + 2W, ...; the loop handles two per trip
  const int b0 = tb0 + wave;
  if (b0 < tb1) load_x(gx0, b0);
  if (b0 + W < tb1) load_x(gx1, b0 + W);
  for (int b = b0; b < tb1; b += 2 * W) {
    load_y(b);
    stage(gx0, wx);
    if (b + 2 * W < tb1) load_x(gx0, b + 2 * W);
    stage(gy, wy);
    compute();
    if (b + W >= tb1) break;
    load_y(b + W);
    stage(gx1, wx);
    if (b + 3 * W < tb1) load_x(gx1, b + 3 * W);
    stage(gy, wy);
    compute();
  }

  // ---- fixed-order reduction of the 8 waves' tiles: acc[i][j] holds D[k][n];
  // lane l owns n = i*32 + l%32 and k = j*32 + (q/4)*8 + (l/32)*4 + [0,4).
  __syncthreads();
  float* red = smem_f + wave * 64 * RED_LD;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = i * 32 + lr;
        const int k = j * 32 + q * 8 + lh * 4;
        *(f32x4*)(red + n * RED_LD + k) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
  __syncthreads();
  const int n = tid >> 3, k = (tid & 7) * 8;
  f32x4 s0 = *(const f32x4*)(smem_f + n * RED_LD + k);
  f32x4 s1 = *(const f32x4*)(smem_f + n * RED_LD + k + 4);
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const float* src = smem_f + (w * 64 + n) * RED_LD + k;
    const f32x4 a = *(const f32x4*)src;
    const f32x4 c = *(const f32x4*)(src + 4);
    s0[0] += a[0]; s0[1] += a[1]; s0[2] += a[2]; s0[3] += a[3];
    s1[0] += c[0]; s1[1] += c[1]; s1[2] += c[2]; s1[3] += c[3];
  }
  const int gn = n0 + n, gk = c0 + k;
  if (gn >= p.N || gk >= p.K) return;
  if (OUT == OUT_BF16) {
    *(u32x4*)((unsigned short*)p.out + (int64_t)gn * p.ldo + gk) =
        u32x4{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]), pack_bf16x2(s1[0], s1[1]),
              pack_bf16x2(s1[2], s1[3])};
  } else {
    float* dst = (float*)p.out + (OUT == OUT_PARTIAL ? (int64_t)split * p.split_stride : 0) + (int64_t)gn * p.ldo + gk;
    *(f32x4*)dst = s0;
    *(f32x4*)(dst + 4) = s1;
  }
}

}  // namespace dpg
