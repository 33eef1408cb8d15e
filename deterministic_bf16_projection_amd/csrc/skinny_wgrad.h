// Streaming weight gradient for skinny outputs (N <= 128 rows of dW):
//   dW[n, k] = sum_t dY[t, n] * X[t, k]
// The pass reads X[T, K] once from HBM and is bandwidth-bound.
//
// Work unit = (all N rows, a block of CB * 64 columns of K, token split).  A
// workgroup has 8 waves arranged as NB row blocks x CB column blocks x TG token
// groups (NB * CB * TG = 8; NB = 1 for N <= 64, 2 for N <= 128; CB = 2, or 1
// when a small forced split count leaves too few units), each wave owning a
// 64 x 64 block of dW.  Per iteration, token group g takes the unit's 64-token
// block (iteration * TG + g): its X tiles (64 tokens x 64 columns) and dY tiles
// (64 tokens x 64 rows) are fetched once with 16-byte buffer loads (rows past T
// read as zero), transposed in registers (8x8 BF16 blocks) and written
// K-contiguous into LDS, where the waves that share a tile read it.  The loads
// of the next iteration are issued before this iteration's MFMAs.  At the end
// the TG partial tiles of each output block are summed in LDS in token-group
// order 0..TG-1 and written once: to the output (one token split) or to the
// FP32 workspace plane of the split.
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
  int k_blocks, splits;        // column blocks of K (CB * 64 columns); token splits
  int tb_total, tb_per_split;  // 64-token blocks and blocks per split
};

template <int NB, int CB, int OUT>
__global__ void __launch_bounds__(512, 1) skinny_wgrad_kernel(SkinnyParams p) {
  constexpr int W = 8;
  constexpr int TG = W / (NB * CB);     // token groups
  static_assert((NB == 1 || NB == 2) && (CB == 1 || CB == 2), "row and column blocks");
  constexpr int TILE = 4096;            // BF16 elements of one transposed 64x64 tile
  constexpr int X_TILES = CB * TG, Y_TILES = NB * TG;
  constexpr int RED_LD = 68;            // FP32 row stride of the reduction buffer
  constexpr int STAGE_ELEMS = (X_TILES + Y_TILES) * TILE;
  constexpr int RED_FLOATS = W * 64 * RED_LD;
  constexpr int SMEM_FLOATS = (STAGE_ELEMS / 2 > RED_FLOATS) ? STAGE_ELEMS / 2 : RED_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem_f[SMEM_FLOATS];
  __bf16* smem = (__bf16*)smem_f;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // wave -> (row block nb, column block cb, token group g)
  const int nb = wave % NB, cb = (wave / NB) % CB, g = wave / (NB * CB);

  // units consecutive in K-block order share dY rows; the XCD remap keeps
  // consecutive units on one XCD
  const int unit = xcd_remap(blockIdx.x, p.k_blocks * p.splits);
  const int split = unit / p.k_blocks;
  const int kb = unit - split * p.k_blocks;
  const int c0 = kb * (CB * 64);
  const int tb0 = split * p.tb_per_split;
  const int tb1 = min(tb0 + p.tb_per_split, p.tb_total);
  const int n_iter = (tb1 - tb0 + TG - 1) / TG;

  const __bf16* dy = (const __bf16*)p.dy;
  const __bf16* x = (const __bf16*)p.x;
  const int lddy = (int)p.lddy, ldx = (int)p.ldx;

  // Staging: X tile (cb, g) is shared by the NB waves (*, cb, g) and dY tile
  // (nb, g) by the CB waves (nb, *, g).  A tile is 8 x 8 sub-blocks of 8x8; lane
  // (kc, sb) = (lane / 8, lane % 8) owns token rows kc*8.. and columns sb*8.., so
  // the 8 lanes of one token row read 128 contiguous bytes; each of a tile's
  // sharers fetches an equal range of token rows.
  const int kc = lane >> 3, sb = lane & 7;
  const bool x_lane = kc / (8 / NB) == nb;
  const bool y_lane = kc / (8 / CB) == cb;
  // Lanes with odd kc hold transposed column m ^ 1 in slot m (a per-lane choice
  // of byte selectors), so that the 16 lanes of one LDS write phase cover rows of
  // both parities; with the row swizzle the writes are then conflict-free.
  const int odd = kc & 1;
  const uint32_t sel_even = odd ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = odd ? 0x05040100u : 0x07060302u;
  uint32_t voff_x[8], voff_y[8];
  int lds_off[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    voff_x[l] = (uint32_t)(((kc * 8 + l) * ldx + cb * 64 + sb * 8) * 2);
    voff_y[l] = (uint32_t)(((kc * 8 + l) * lddy + nb * 64 + sb * 8) * 2);
    const int row = sb * 8 + (l ^ odd);
    lds_off[l] = lds_chunk_off(row, kc);
  }
  __bf16* x_tile = smem + (g * CB + cb) * TILE;            // shared with the NB waves (*, cb, g)
  __bf16* y_tile = smem + (X_TILES + g * NB + nb) * TILE;  // shared with the CB waves (nb, *, g)

  auto rsrc_rows = [&](const __bf16* base, int ld, int col0, int cols, int t0) {
    const int rows = min(p.T - t0, 64);
    int bytes = ((rows - 1) * ld + (cols - col0)) * 2;
    bytes = rows > 0 ? max(bytes, 0) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base + (int64_t)max(t0, 0) * ld + col0), (short)0,
                                             bytes, 0x00020000);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // fragment rows i*32 + lr: fswz(i*32 + lr) = fswz(lr) ^ 4i, i.e. chunk
  // (2s + lh) of fragment 1 sits where chunk (2(s^2) + lh) of fragment 0 does
  const int lr = lane & 31, lh = lane >> 5;
  const int sw = fswz(lr);
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = ((2 * s + lh) ^ sw) << 3;

  u32x4 gx[8], gy[8];
  auto load = [&](int it) {
    const int blk = tb0 + it * TG + g;
    const int t0 = blk < tb1 ? blk * 64 : p.T;  // past this split: empty descriptors
    if (x_lane) {
      const rsrc_t rx = rsrc_rows(x, ldx, c0, p.K, t0);
#pragma unroll
      for (int l = 0; l < 8; ++l) gx[l] = buf_load16(rx, voff_x[l]);
    }
    if (y_lane) {
      const rsrc_t ry = rsrc_rows(dy, lddy, 0, p.N, t0);
#pragma unroll
      for (int l = 0; l < 8; ++l) gy[l] = buf_load16(ry, voff_y[l]);
    }
  };
  auto stage = [&]() {
    u32x4 t[8];
    if (x_lane) {
      transpose8x8_sel(gx, t, sel_even, sel_odd);
#pragma unroll
      for (int m = 0; m < 8; ++m) *(u32x4*)(x_tile + lds_off[m]) = t[m];
    }
    if (y_lane) {
      transpose8x8_sel(gy, t, sel_even, sel_odd);
#pragma unroll
      for (int m = 0; m < 8; ++m) *(u32x4*)(y_tile + lds_off[m]) = t[m];
    }
  };

  if (n_iter > 0) load(0);
  for (int it = 0; it < n_iter; ++it) {
    stage();
    if (it + 1 < n_iter) load(it + 1);
    __syncthreads();  // shared tiles complete
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = as_bf16x8(*(const u32x4*)(y_tile + (i * 32 + lr) * 64 + koff[s ^ (2 * i)]));
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = as_bf16x8(*(const u32x4*)(x_tile + (j * 32 + lr) * 64 + koff[s ^ (2 * j)]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
    __syncthreads();  // tiles consumed before the next iteration overwrites them
  }

  // ---- fixed-order reduction over the token groups: acc[i][j] holds D[k][n];
  // lane l owns n = i*32 + l%32 and k = j*32 + (q/4)*8 + (l/32)*4 + [0,4).
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
  // output block (nb, cb) = waves nb + NB * cb + NB * CB * g for g = 0..TG-1
  constexpr int OUT_PER_THREAD = NB * CB * 64 * 64 / 512;  // elements per thread (8, 16 or 32)
#pragma unroll
  for (int h = 0; h < OUT_PER_THREAD / 8; ++h) {
    const int e = (tid + h * 512) * 8;           // element index in [NB*CB] x 64 x 64
    const int blk = e / 4096, rem = e % 4096;    // blk = nb + NB * cb
    const int n = rem / 64, k = rem % 64;
    const int bnb = blk % NB, bcb = blk / NB;
    f32x4 s0 = *(const f32x4*)(smem_f + (blk * 64 + n) * RED_LD + k);
    f32x4 s1 = *(const f32x4*)(smem_f + (blk * 64 + n) * RED_LD + k + 4);
#pragma unroll
    for (int gg = 1; gg < TG; ++gg) {
      const float* src = smem_f + ((blk + gg * NB * CB) * 64 + n) * RED_LD + k;
      const f32x4 a = *(const f32x4*)src;
      const f32x4 c = *(const f32x4*)(src + 4);
      s0[0] += a[0]; s0[1] += a[1]; s0[2] += a[2]; s0[3] += a[3];
      s1[0] += c[0]; s1[1] += c[1]; s1[2] += c[2]; s1[3] += c[3];
    }
    const int gn = bnb * 64 + n, gk = c0 + bcb * 64 + k;
    if (gn >= p.N || gk >= p.K) continue;
    if (OUT == OUT_BF16) {
      *(u32x4*)((unsigned short*)p.out + (int64_t)gn * p.ldo + gk) =
          u32x4{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]), pack_bf16x2(s1[0], s1[1]),
                pack_bf16x2(s1[2], s1[3])};
    } else {
      float* dst =
          (float*)p.out + (OUT == OUT_PARTIAL ? (int64_t)split * p.split_stride : 0) + (int64_t)gn * p.ldo + gk;
      *(f32x4*)dst = s0;
      *(f32x4*)(dst + 4) = s1;
    }
  }
}

}  // namespace dpg
