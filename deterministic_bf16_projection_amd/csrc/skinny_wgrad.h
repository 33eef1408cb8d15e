// Streaming weight gradient for skinny outputs (N <= 128 rows of dW):
//   dW[n, k] = sum_t dY[t, n] * X[t, k]
// The pass reads X[T, K] once from HBM and is bandwidth-bound.
//
// Work unit = (all N rows, a block of CB * 64 columns of K, token split).  A
// workgroup has 8 waves arranged as NB row blocks x CB column blocks x TG token
// groups (NB * CB * TG = 8; NB = 1 for N <= 64, 2 for N <= 128).  The library
// runs it for N <= 64 with 64-column units (NB = CB = 1), which the planner
// picks when a small forced split count would leave too few 128-column units;
// 128-column units run skinny_direct.h (N <= 64), and every unit with two row
// blocks runs skinny_lds.h,
// each wave owning a 64 x 64 block of dW.  Per iteration, token group g takes the unit's 64-token
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
  int tb_total, tb_per_split;  // 64-token blocks; blocks of the largest split (see split_begin)
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

  // the wave index is uniform: keep it (and all that derives from it) in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave -> (row block nb, column block cb, token group g)
  const int nb = wave % NB, cb = (wave / NB) % CB, g = wave / (NB * CB);

  // units consecutive in K-block order share dY rows; the XCD remap keeps
  // consecutive units on one XCD
  const int unit = xcd_remap(blockIdx.x, p.k_blocks * p.splits);
  const int split = unit / p.k_blocks;
  const int kb = unit - split * p.k_blocks;
  const int c0 = kb * (CB * 64);
  const SplitParts sp = split_parts(p.splits, p.tb_total);
  const int tb0 = split_begin(split, sp);
  const int tb1 = split_begin(split + 1, sp);
  const int n_iter = (tb1 - tb0 + TG - 1) / TG;

  const __bf16* dy = (const __bf16*)p.dy;
  const __bf16* x = (const __bf16*)p.x;
  const int lddy = (int)p.lddy, ldx = (int)p.ldx;

  // Staging.  An iteration needs X_TILES + Y_TILES tiles of 64 tokens x 64
  // columns; wave w fetches tile w + 8 r in round r (X tiles first, then dY
  // tiles).  A tile is 8 x 8 sub-blocks of 8x8: lane (kc, sb) = (lane / 8,
  // lane % 8) owns token rows kc*8.. and columns sb*8.., so the 8 lanes of one
  // token row read 128 contiguous bytes.  With one round (N > 64 and 128-column
  // units) the loads run two iterations ahead in two register buffers; with two
  // rounds, one iteration ahead.
  constexpr int TILES = X_TILES + Y_TILES;
  constexpr int ROUNDS = (TILES + W - 1) / W;
  constexpr int AHEAD = ROUNDS == 1 ? 2 : 1;
  const int kc = lane >> 3, sb = lane & 7;
  // Lanes with odd kc hold transposed column m ^ 1 in slot m (a per-lane choice
  // of byte selectors), so that the 16 lanes of one LDS write phase cover rows
  // of both parities; with the row swizzle the writes are then conflict-free.
  // Slot m goes to row sb*8 + (m ^ odd) of the tile, element offset lds0 ^ 72 m
  // (the closed form of lds_chunk_off for these rows).
  const int odd = kc & 1;
  const uint32_t sel_even = odd ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = odd ? 0x05040100u : 0x07060302u;
  const int lds0 = (sb * 512) | (((9 * odd) ^ ((kc ^ sb) & 7)) << 3);

  // the tile this wave fetches in round r (wave-uniform)
  struct Fetch {
    const __bf16* base;  // first column of the tile's source rows
    int ld, cols;        // row stride; readable columns from base
    int g;               // token group
    int valid;
    __bf16* dst;         // LDS tile
  };
  Fetch f[ROUNDS];
  uint32_t voff[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int t = wave + W * r;
    f[r].valid = t < TILES;
    if (t < X_TILES) {  // X tile (g, cb'): columns c0 + cb' * 64 ..
      const int cbt = t % CB;
      f[r].g = t / CB;
      f[r].base = x + c0 + cbt * 64;
      f[r].ld = ldx;
      f[r].cols = p.K - c0 - cbt * 64;
    } else {  // dY tile (g, nb'): rows nb' * 64 .. of dW
      const int yt = min(t, TILES - 1) - X_TILES;
      const int nbt = yt % NB;
      f[r].g = yt / NB;
      f[r].base = dy + nbt * 64;
      f[r].ld = lddy;
      f[r].cols = p.N - nbt * 64;
    }
    f[r].dst = smem + min(t, TILES - 1) * TILE;
    voff[r] = (uint32_t)((kc * 8 * f[r].ld + sb * 8) * 2);
  }
  __bf16* x_tile = smem + (g * CB + cb) * TILE;            // read by the NB waves (*, cb, g)
  __bf16* y_tile = smem + (X_TILES + g * NB + nb) * TILE;  // read by the CB waves (nb, *, g)

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

  // Buffer descriptor of round r's tile at iteration it: token rows
  // [t0, min(T, t0 + 64)), columns [0, cols) from base; rows past T, columns
  // past the matrix and iterations past the split read zeros (empty range).
  auto rsrc = [&](int r, int it) {
    const int blk = tb0 + it * TG + f[r].g;
    const int t0 = blk < tb1 ? blk * 64 : p.T;
    const int rows = min(p.T - t0, 64);
    int bytes = ((rows - 1) * f[r].ld + f[r].cols) * 2;
    bytes = (rows > 0 && f[r].cols > 0) ? max(bytes, 0) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(f[r].base + (int64_t)min(t0, p.T - 1) * f[r].ld),
                                             (short)0, bytes, 0x00020000);
  };
  u32x4 gbuf[AHEAD][ROUNDS][8];
  auto load = [&](u32x4(&gb)[ROUNDS][8], int it) {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (f[r].valid) {
        const rsrc_t rs = rsrc(r, it);
#pragma unroll
        for (int l = 0; l < 8; ++l) gb[r][l] = buf_load16(rs, voff[r] + (uint32_t)(l * f[r].ld * 2));
      }
    }
  };
  auto stage = [&](const u32x4(&gb)[ROUNDS][8]) {
    int o = lds0;
    asm volatile("" : "+v"(o));  // form the slot offsets here, not in the loop preheader
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (f[r].valid) {
        u32x4 t[8];
        transpose8x8_sel(gb[r], t, sel_even, sel_odd);
#pragma unroll
        for (int m = 0; m < 8; ++m) *(u32x4*)(f[r].dst + (o ^ (72 * m))) = t[m];
      }
    }
  };
  auto compute = [&]() {
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
  };

  // iteration it is staged from buffer it % AHEAD; the buffer is refilled with
  // iteration it + AHEAD right after staging (past the end: no memory access)
#pragma unroll
  for (int b = 0; b < AHEAD; ++b) load(gbuf[b], b);
  for (int it = 0; it < n_iter; it += 2) {
    stage(gbuf[0]);
    load(gbuf[0], it + AHEAD);
    compute();
    if (it + 1 >= n_iter) break;
    stage(gbuf[AHEAD - 1]);
    load(gbuf[AHEAD - 1], it + 1 + AHEAD);
    compute();
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
