// Streaming weight gradient for outputs of at most 64 rows, with no operand
// staging through LDS:
//   dW[n, k] = sum_t dY[t, n] * X[t, k]
// X[T, K] is read once from HBM; the pass is bandwidth-bound.
//
// Work unit = (128 columns of K, token split of whole 64-token blocks).  The 8
// waves of a workgroup are token groups: wave g takes the unit's 16-token steps
// g, g + 8, g + 16, ... and keeps a 64 x 128 FP32 partial of dW in registers.
//
// MFMA operands straight from registers.  For one step, lane l = 32 h + c
// (c < 32, h < 2) loads tokens 8 h .. 8 h + 7 of
//   X:  columns 4 c .. 4 c + 3 of the unit (an 8-byte load per token; the 32
//       lanes of one half read 256 contiguous bytes of a token row),
//   dY: rows 2 c, 2 c + 1 (a 4-byte load per token; 128 contiguous bytes).
// A BF16 transpose in registers (v_perm_b32) turns that into, per column 4 c + f
// (f < 4) and per row 2 c + a (a < 2), the 8 consecutive tokens the lane
// contributes to a 32x32x16 MFMA operand: B fragment f covers columns
// {4 c + f : c < 32}, A fragment a covers rows {2 c + a : c < 32}.  So a wave
// issues 8 MFMAs per 16 tokens with no LDS traffic and no barrier; the output
// columns of a fragment are strided by 4, which the final reduction undoes.
//
// Reduction (fixed order): waves 4..7 write their partials to LDS slots 0..3,
// wave g < 4 adds slot g to its own (P_g = acc_g + acc_{g+4}) and writes it
// back, and the output element is ((P_0 + P_1) + P_2) + P_3, written once: to
// the output (one token split) or to the FP32 workspace plane of the split.
//
// Rows >= N, columns >= K and tokens >= T read as zero (per-lane offsets past
// the buffer range, and buffer descriptors ending at the last valid token).
// Requirements (launcher): N <= 64 and K multiples of 8, row strides below 2^23
// elements.
#pragma once
#include "device_common.h"
#include "gemm_kernel.h"
#include "skinny_wgrad.h"

namespace dpg {

template <int OUT>
__global__ void __launch_bounds__(512, 1) skinny_direct_kernel(SkinnyParams p) {
  constexpr int W = 8;                   // waves = token groups
  constexpr int COLS = 128;              // columns of K per unit
  constexpr int RED_LD = COLS + 4;       // FP32 row stride of a reduction slot
  constexpr int SLOT = 64 * RED_LD;      // floats per slot (64 rows)
  __shared__ __attribute__((aligned(16))) float red[4 * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;

  const int unit = xcd_remap(blockIdx.x, p.k_blocks * p.splits);
  const int split = unit / p.k_blocks;
  const int kb = unit - split * p.k_blocks;
  const int c0 = kb * COLS;
  const SplitParts sp = split_parts(p.splits, p.tb_total);
  const int tb0 = split_begin(split, sp);
  const int tb1 = split_begin(split + 1, sp);
  const int steps = max(tb1 - tb0, 0) * 4;          // 16-token steps of the unit
  const int n_my = steps > wave ? (steps - wave + W - 1) / W : 0;

  const __bf16* dy = (const __bf16*)p.dy;
  const __bf16* x = (const __bf16*)p.x + c0;
  const int lddy = (int)p.lddy, ldx = (int)p.ldx;
  // per-lane byte offsets within a step; lanes whose columns / rows lie outside
  // the matrix point past every buffer range (reads return zero)
  constexpr uint32_t kOut = 0x80000000u;
  const uint32_t vx = (c0 + 4 * c < p.K) ? (uint32_t)((8 * h * ldx + 4 * c) * 2) : kOut;
  const uint32_t vy = (2 * c < p.N) ? (uint32_t)((8 * h * lddy + 2 * c) * 2) : kOut;
  const uint32_t sx = (uint32_t)(ldx * 2), sy = (uint32_t)(lddy * 2);
  const int xcols = p.K - c0;

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][f][r] = 0.f;

  struct Regs {
    u32x2 xv[8];      // X: token i, columns 4c..4c+3
    uint32_t yv[8];   // dY: token i, rows 2c, 2c+1
  };
  // step j of this wave (j >= n_my: empty descriptors, no memory access)
  auto load = [&](Regs& R, int j) {
    const int t0 = (tb0 * 64) + 16 * (wave + W * j);
    const bool ok = j < n_my && t0 < p.T;
    const int rows = ok ? min(p.T - t0, 16) : 0;
    const int tc = ok ? t0 : 0;
    const int xb = rows > 0 ? ((rows - 1) * ldx + xcols) * 2 : 0;
    const int yb = rows > 0 ? ((rows - 1) * lddy + p.N) * 2 : 0;
    const rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(x + (int64_t)tc * ldx), (short)0, xb,
                                                        0x00020000);
    const rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dy + (int64_t)tc * lddy), (short)0, yb,
                                                        0x00020000);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      R.xv[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, (int)(vx + (uint32_t)i * sx), 0, 0));
      R.yv[i] = __builtin_amdgcn_raw_buffer_load_b32(ry, (int)(vy + (uint32_t)i * sy), 0, 0);
    }
  };
  auto compute = [&](const Regs& R) {
    // fragment words: word e holds tokens 2e (low half) and 2e + 1
    bf16x8 fx[4], fy[2];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(R.xv[2 * e + 1][f >> 1], R.xv[2 * e][f >> 1], sel);
      fx[f] = as_bf16x8(v);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t sel = a ? 0x07060302u : 0x05040100u;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(R.yv[2 * e + 1], R.yv[2 * e], sel);
      fy[a] = as_bf16x8(v);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[a][f] = mfma32(fx[f], fy[a], acc[a][f]);
  };

  // two register buffers: step j + 2 is fetched while step j's MFMAs run.  The
  // loop runs whole pairs of steps (one exit keeps the accumulators in place);
  // a step past the wave's last reads nothing and adds zero products.
  Regs b0, b1;
  load(b0, 0);
  load(b1, 1);
  const int pairs = (n_my + 1) >> 1;
  for (int jj = 0; jj < pairs; ++jj) {
    compute(b0);
    load(b0, 2 * jj + 2);
    compute(b1);
    load(b1, 2 * jj + 3);
  }

  // ---- fixed-order reduction.  acc[a][f] lane l, register 4q + e holds
  // row n = 2 (l % 32) + a and unit column 4 b + f, b = 8q + 4 (l / 32) + e.
  auto put = [&](float* slot) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 2 * c + a, b = 8 * q + 4 * h + e;
          *(f32x4*)(slot + n * RED_LD + 4 * b) =
              f32x4{acc[a][0][4 * q + e], acc[a][1][4 * q + e], acc[a][2][4 * q + e], acc[a][3][4 * q + e]};
        }
  };
  if (wave >= 4) put(red + (wave - 4) * SLOT);
  __syncthreads();
  if (wave < 4) {
    float* slot = red + wave * SLOT;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 2 * c + a, b = 8 * q + 4 * h + e;
          const f32x4 o = *(const f32x4*)(slot + n * RED_LD + 4 * b);
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[a][f][4 * q + e] += o[f];
        }
    put(slot);
  }
  __syncthreads();
  // 64 x 128 outputs, 8 consecutive columns per thread and chunk
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int e = (tid + hh * 512) * 8;
    const int n = e / COLS, k = e % COLS;
    const float* s0 = red + n * RED_LD + k;
    f32x4 v0 = *(const f32x4*)s0, v1 = *(const f32x4*)(s0 + 4);
#pragma unroll
    for (int g = 1; g < 4; ++g) {
      const f32x4 a0 = *(const f32x4*)(s0 + g * SLOT), a1 = *(const f32x4*)(s0 + g * SLOT + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[r] += a0[r];
        v1[r] += a1[r];
      }
    }
    const int gk = c0 + k;
    if (n >= p.N || gk >= p.K) continue;
    if (OUT == OUT_BF16) {
      *(u32x4*)((unsigned short*)p.out + (int64_t)n * p.ldo + gk) =
          u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                pack_bf16x2(v1[2], v1[3])};
    } else {
      float* dst = (float*)p.out + (OUT == OUT_PARTIAL ? (int64_t)split * p.split_stride : 0) + (int64_t)n * p.ldo + gk;
      *(f32x4*)dst = v0;
      *(f32x4*)(dst + 4) = v1;
    }
  }
}

}  // namespace dpg
