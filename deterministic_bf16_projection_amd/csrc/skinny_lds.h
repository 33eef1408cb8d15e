// Streaming weight gradient for 64 < N <= 128 rows of dW with the operands
// fetched straight into LDS:
//   dW[n, k] = sum_t dY[t, n] * X[t, k]
// X[T, K] is read once from HBM; the pass is bandwidth-bound, and what limits
// it is how many bytes of X each CU keeps in flight.
//
// Work unit = (CB * 64 columns of K, token split of whole 64-token blocks);
// one 64-token block per iteration.  CB = 2 (128-column units, the planner's
// plans) or 1 (64-column units, forced small split counts).  The 8 waves are
// 2 row blocks x CB column blocks x 4 / CB k-step groups: wave (nb, cb, ks)
// owns the 64 x 64 block (rows 64 nb.., columns 64 cb..) of dW over CB of the
// block's four 16-token k-steps (k-steps CB ks ..).
//
// Staging without registers: a stage holds the block's CB X tiles and two dY
// tiles (64 tokens x 64 columns / rows each, row-major as in memory, 128 B a
// token row, 24 or 32 KB in all) and is filled by buffer_load ... lds, 1 KB (8
// token rows) per instruction, CB + 2 instructions per wave.  The 16-byte chunk c of token
// row r sits at chunk position c ^ 2 (r % 4); the swizzle is applied on the
// source side (each lane fetches the chunk that belongs at its destination).
// Four stages: while a block is computed, the next three are in flight (five
// measured no faster).  One barrier per iteration: each wave waits for its own
// fetches of the block (vmcnt), the barrier then publishes the whole stage and
// frees the stage computed last, which the fetch of block it + 3 refills.
//
// Fragments: the transposing LDS read (ds_read_b64_tr_b16) gathers, for a lane,
// 4 consecutive tokens of one column; two of them form the 8 tokens a lane
// contributes to a 32x32x16 MFMA operand (the index math of the generic
// kernel's MN-major operand).  With the chunk swizzle above every read phase
// touches distinct banks (checked by enumeration for 32 and 64 banks).
//
// The k-step groups' partials of each output block are summed in LDS in the
// fixed order ks = 0, 1, ... and written once: to the output (one token split) or to the
// FP32 workspace plane of the split.  Rows >= N, columns >= K and tokens >= T
// read as zero (per-lane offsets past the buffer range, and buffer descriptors
// ending at the last valid token).  Requirements (launcher): 64 < N <= 128,
// N and K multiples of 8, row strides below 2^23 elements.
#pragma once
#include "device_common.h"
#include "gemm_kernel.h"
#include "skinny_wgrad.h"

namespace dpg {

template <int CB, int OUT>
__global__ void __launch_bounds__(512, 1) skinny_lds_kernel(SkinnyParams p) {
  static_assert(CB == 1 || CB == 2, "64-column blocks per unit");
  constexpr int NSTAGE = 4;
  constexpr int TILE = 64 * 64;         // BF16 elements of one 64-token tile
  constexpr int STAGE = (CB + 2) * TILE;  // X tiles 0 .. CB-1 (column blocks), then 2 dY tiles (row blocks)
  constexpr int NCH = CB + 2;           // 1 KB fetches per wave per stage (8 waves, 8 per tile)
  constexpr int KG = 4 / CB;            // k-step groups; a group takes 4 / KG of a block's 4 k-steps
  constexpr int RED_LD = 68;            // FP32 row stride of the reduction buffer
  constexpr int RED_FLOATS = 8 * 64 * RED_LD;
  constexpr int SMEM_FLOATS = (NSTAGE * STAGE / 2 > RED_FLOATS) ? NSTAGE * STAGE / 2 : RED_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem_f[SMEM_FLOATS];
  __bf16* smem = (__bf16*)smem_f;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = wave & 1, cb = (wave >> 1) % CB, ks = wave / (2 * CB);

  const int unit = xcd_remap(blockIdx.x, p.k_blocks * p.splits);
  const int split = unit / p.k_blocks;
  const int kb = unit - split * p.k_blocks;
  const int c0 = kb * (64 * CB);
  const SplitParts sp = split_parts(p.splits, p.tb_total);
  const int tb0 = split_begin(split, sp);
  const int tb1 = split_begin(split + 1, sp);
  const int n_iter = max(tb1 - tb0, 0);

  const int lddy = (int)p.lddy, ldx = (int)p.ldx;
  // Fetch assignment: the 8 NCH chunks of 1 KB of a stage, chunk q = NCH w + j
  // of wave w: tile q / 8 (X tiles first, then dY; uniform per wave and j),
  // token rows 8 (q % 8) .. + 7.  Lane l lands at row 8 (q % 8) + l / 8, chunk
  // position l % 8, and fetches source chunk (l % 8) ^ 2 (row % 4).
  constexpr uint32_t kOut = 0x80000000u;  // past every buffer range: reads zero
  uint32_t voff[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int q = NCH * wave + j;
    const int tile = q >> 3;
    const int r = 8 * (q & 7) + (lane >> 3);
    const int src = (lane & 7) ^ (2 * (r & 3));
    if (tile < CB) {
      const int col = c0 + 64 * tile + 8 * src;
      voff[j] = col < p.K ? (uint32_t)((r * ldx + col) * 2) : kOut;
    } else {
      const int row = 64 * (tile - CB) + 8 * src;
      voff[j] = row < p.N ? (uint32_t)((r * lddy + row) * 2) : kOut;
    }
  }
  auto fetch = [&](int it, int buf) {
    const int blk = tb0 + it;
    const bool ok = blk < tb1;
    const int t0 = ok ? blk * 64 : 0;
    const int rows = ok ? min(p.T - t0, 64) : 0;
    const int xb = rows > 0 ? ((rows - 1) * ldx + p.K) * 2 : 0;
    const int yb = rows > 0 ? ((rows - 1) * lddy + p.N) * 2 : 0;
    const rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>((const __bf16*)p.x + (int64_t)t0 * ldx),
                                                        (short)0, xb, 0x00020000);
    const rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>((const __bf16*)p.dy + (int64_t)t0 * lddy),
                                                        (short)0, yb, 0x00020000);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = NCH * wave + j;
      __bf16* dst = smem + buf * STAGE + (q >> 3) * TILE + (q & 7) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds((q >> 3) < CB ? rx : ry, (lds_void_t*)dst, 16, (int)voff[j], 0, 0, 0);
    }
  };

  // element (token k, column c) of a tile
  auto off = [](int k, int c) { return k * 64 + (((c >> 3) ^ (2 * (k & 3))) << 3) + (c & 7); };
  // LDS byte address of the first of the two transposing reads that give a
  // lane's 32x32x16 operand fragment (column c0f + l % 32, tokens 16 k16 +
  // 8 (l / 32) .. + 8); the second read is 4 token rows (512 bytes) further
  const int g = lane >> 4, sl = lane & 15;
  auto frag_addr = [&](const __bf16* plane, int c0f, int k16) {
    const int kk = k16 * 16 + (g >> 1) * 8 + (sl >> 2);
    const int cc = c0f + 16 * (g & 1) + 4 * (sl & 3);
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) __bf16*)(plane + off(kk, cc));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) fetch(s, s);
  for (int it = 0; it < n_iter; ++it) {
    // This wave's fetches of block it have landed (those of blocks it + 1 and
    // it + 2, 2 (CB + 2) instructions, may still be in flight; vmcnt counts
    // them in issue order).  After the barrier every wave's fetches of block it are in
    // LDS, and every wave has finished reading the stage of block it - 1 (its
    // reads completed inside their asm blocks), which the fetch below refills.
    // Written out because the compiler would otherwise wait for all fetches
    // here (the release fence of __syncthreads() covers LDS fetches).
    if constexpr (NCH == 4)
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    fetch(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
    const __bf16* st = smem + (it % NSTAGE) * STAGE;
    const __bf16* xt = st + cb * TILE;
    const __bf16* yt = st + (CB + nb) * TILE;
#pragma unroll
    for (int s = 0; s < 4 / KG; ++s) {
      const int k16 = (4 / KG) * ks + s;
      // the eight transposing reads of this k-step, complete when the block
      // ends (the compiler would otherwise wait for all in-flight fetches
      // before each read, as it cannot tell the addresses apart)
      u32x2 a0l, a0h, a1l, a1h, b0l, b0h, b1l, b1h;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
          "ds_read_b64_tr_b16 %2, %9\n\t"
          "ds_read_b64_tr_b16 %3, %9 offset:512\n\t"
          "ds_read_b64_tr_b16 %4, %10\n\t"
          "ds_read_b64_tr_b16 %5, %10 offset:512\n\t"
          "ds_read_b64_tr_b16 %6, %11\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:512\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0l), "=&v"(a0h), "=&v"(a1l), "=&v"(a1h), "=&v"(b0l), "=&v"(b0h), "=&v"(b1l), "=&v"(b1h)
          : "v"(frag_addr(yt, 0, k16)), "v"(frag_addr(yt, 32, k16)), "v"(frag_addr(xt, 0, k16)),
            "v"(frag_addr(xt, 32, k16))
          : "memory");
      const bf16x8 fa[2] = {as_bf16x8(u32x4{a0l[0], a0l[1], a0h[0], a0h[1]}),
                            as_bf16x8(u32x4{a1l[0], a1l[1], a1h[0], a1h[1]})};
      const bf16x8 fb[2] = {as_bf16x8(u32x4{b0l[0], b0l[1], b0h[0], b0h[1]}),
                            as_bf16x8(u32x4{b1l[0], b1l[1], b1h[0], b1h[1]})};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
  }
  // fetches past the last block still write (zeros) into the stages, which the
  // reduction buffer overlaps: wait for all of them, and for every wave's reads
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // ---- fixed-order reduction over the k-step halves: acc[i][j] holds D[k][n];
  // lane l owns n = i*32 + l%32 and k = j*32 + (q/4)*8 + (l/32)*4 + [0,4).
  const int lr = lane & 31, lh = lane >> 5;
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
  // output block (nb, cb) = the sum of waves nb + 2 cb + 2 CB ks, ks = 0 .. KG-1 in order
#pragma unroll
  for (int hh = 0; hh < 2 * CB; ++hh) {
    const int e = (tid + hh * 512) * 8;         // element index in [2 CB blocks] x 64 x 64
    const int blk = e / 4096, rem = e % 4096;   // blk = nb + 2 cb
    const int n = rem / 64, k = rem % 64;
    const float* s0p = smem_f + (blk * 64 + n) * RED_LD + k;
    f32x4 s0 = *(const f32x4*)s0p, s1 = *(const f32x4*)(s0p + 4);
#pragma unroll
    for (int gg = 1; gg < KG; ++gg) {
      const float* sp = smem_f + ((blk + 2 * CB * gg) * 64 + n) * RED_LD + k;
      const f32x4 a = *(const f32x4*)sp, b = *(const f32x4*)(sp + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] += a[r];
        s1[r] += b[r];
      }
    }
    const int gn = (blk & 1) * 64 + n, gk = c0 + (blk >> 1) * 64 + k;
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
