// Software-pipelined BF16 MFMA GEMM for gfx950 (the path of the large
// projection passes).  C[M,N] = sum_k A(m,k) * B(n,k), FP32 accumulation.
//
// Compared with the generic kernel in gemm_kernel.h:
// * Operands are fetched with raw buffer loads.  The buffer descriptor of each
//   operand covers exactly the valid part of the current K tile, so rows past
//   the matrix end and reduction rows past K read as zero in hardware: the main
//   loop has no branches.
// * MN-major operands (input gradient B, both weight-gradient operands) are
//   transposed in registers (8x8 blocks of BF16 through v_perm_b32) on their
//   way to LDS, so LDS always holds K-contiguous rows and every MFMA fragment
//   is one ds_read_b128.
// * LDS rows are 64 BF16 (128 B) with 16-byte chunks XOR-swizzled per row.
// * Per K tile (64) each wave runs 4 k-steps of 16; the fragments of step s+1
//   are read while the MFMAs of step s issue, the global loads of the tile
//   after next are issued right after the staged registers are written to the
//   other LDS stage, and the single barrier per tile sits in the middle of the
//   last step's MFMAs.
// Requirements (checked by the planner): K-major operands have K % 64 == 0;
// all contiguous extents are multiples of 8 elements; operand spans fit the
// 32-bit buffer range.
#pragma once
#include "device_common.h"
#include "gemm_kernel.h"

namespace dpg {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t clamped = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)clamped, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// 8x8 transpose of BF16: in[k] holds 8 values along m for row k (dword d =
// m 2d | 2d+1); out[m] holds the 8 values along k for column m.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[m][e] = __builtin_amdgcn_perm(in[2 * e + 1][m >> 1], in[2 * e][m >> 1], sel);
  }
}

// LDS K-major layout: row r (64 BF16 = 8 chunks of 16 B); chunk c stored at
// position c ^ swz(r).  Rows r and r + 8 use different patterns so that the
// 16 rows one ds_read_b128 phase may touch fall on distinct banks.
__device__ __forceinline__ int fswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_chunk_off(int r, int c) { return r * 64 + ((c ^ fswz(r)) << 3); }

// One operand: R rows (M or N side) by 64 reduction elements per K tile.
template <int R, bool KMAJ, int NT>
struct FastOperand {
  // K-major: 16-byte chunks (row, k-chunk) per thread, rows tid/8 + (NT/8) i.
  // MN-major: one 8x8 block per thread for the first R threads (R <= NT), or
  // R/NT blocks per thread.
  static constexpr int LOADS = KMAJ ? R * 8 / NT : (R >= NT ? R * 8 / NT : 8);
  static constexpr int BLOCK_THREADS = KMAJ ? NT : (R >= NT ? NT : R);  // threads that own data
  u32x4 g[LOADS];
  uint32_t voff[LOADS];
  int lds_off[LOADS];  // element offsets within one operand plane
  bool owner;

  // set up per-thread offsets; ld in elements
  __device__ __forceinline__ void init(int tid, int64_t ld) {
    owner = tid < BLOCK_THREADS;
    if (KMAJ) {
      const int c = tid & 7;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = (tid >> 3) + (NT / 8) * i;
        voff[i] = (uint32_t)(r * ld * 2 + c * 16);
        lds_off[i] = lds_chunk_off(r, c);
      }
    } else {
      // block: kc = tid & 7 (which 8 reduction rows), mb = tid >> 3 (+32 per block)
      const int kc = tid & 7;
#pragma unroll
      for (int b = 0; b < LOADS / 8; ++b) {
        const int mb = (tid >> 3) + (NT / 8) * b;
#pragma unroll
        for (int l = 0; l < 8; ++l) {
          voff[b * 8 + l] = (uint32_t)((kc * 8 + l) * ld * 2 + mb * 16);
          lds_off[b * 8 + l] = lds_chunk_off(mb * 8 + l, kc);
        }
      }
    }
  }

  __device__ __forceinline__ void load(rsrc_t r) {
    if (BLOCK_THREADS < NT && !owner) return;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) g[i] = buf_load16(r, voff[i]);
  }

  __device__ __forceinline__ void store(__bf16* plane) const {
    if (BLOCK_THREADS < NT && !owner) return;
    if (KMAJ) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) *(u32x4*)(plane + lds_off[i]) = g[i];
    } else {
#pragma unroll
      for (int b = 0; b < LOADS / 8; ++b) {
        u32x4 in[8], out[8];
#pragma unroll
        for (int l = 0; l < 8; ++l) in[l] = g[b * 8 + l];
        transpose8x8(in, out);
#pragma unroll
        for (int m = 0; m < 8; ++m) *(u32x4*)(plane + lds_off[b * 8 + m]) = out[m];
      }
    }
  }
};

// Buffer descriptor of the K tile starting at k0 (32-bit arithmetic only: the
// launcher guarantees ld < 2^23, so one tile spans less than 2^31 bytes).
//  K-major (element (row, k) at ptr[row * ld + k]): rows [row0, rows), k < K.
//  MN-major (element (row, k) at ptr[k * ld + row]): reduction rows
//  [k0, min(K, k0 + 64)), columns [row0, rows) of each.
template <bool KMAJ>
__device__ __forceinline__ rsrc_t tile_rsrc(const __bf16* ptr, int ld, int row0, int rows, int k0, int K) {
  int bytes;
  const __bf16* base;
  if (KMAJ) {
    const int valid = min(rows - row0, 256);
    bytes = ((valid - 1) * ld + (K - k0)) * 2;
    base = ptr + (int64_t)row0 * ld + k0;
  } else {
    const int kr = min(K - k0, 64);
    bytes = ((kr - 1) * ld + (rows - row0)) * 2;
    bytes = kr > 0 ? bytes : 0;
    base = ptr + (int64_t)k0 * ld + row0;
  }
  bytes = max(bytes, 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base), (short)0, bytes, 0x00020000);
}

// Scheduling groups: MFMA, DS read, DS write, VMEM read.
#define DPG_SG_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, n, 0)
#define DPG_SG_DSR(n) __builtin_amdgcn_sched_group_barrier(0x100, n, 0)
#define DPG_SG_DSW(n) __builtin_amdgcn_sched_group_barrier(0x200, n, 0)
#define DPG_SG_VMR(n) __builtin_amdgcn_sched_group_barrier(0x020, n, 0)

// Interleave NM MFMAs with NR DS reads, then NW DS writes and NV VMEM reads.
// Reads come first (program order and LDS dependences require it): with
// writes or loads present they share the first half of the MFMAs and the
// writes / loads the second half; otherwise reads spread over all MFMAs.
template <int NM, int NR, int NW, int NV, int I = 0>
__device__ __forceinline__ void sched_step() {
  if constexpr (I < NM) {
    constexpr int HR = (NW + NV > 0) ? (NM + 1) / 2 : NM;  // MFMAs that carry reads
    constexpr int HW = NM - HR > 0 ? NM - HR : NM;        // MFMAs that carry writes / loads
    constexpr int IR = I < HR ? I : HR;
    constexpr int IW = (NW + NV > 0 && I >= NM - HW) ? I - (NM - HW) : -1;
    constexpr int r = I < HR ? (NR * (IR + 1)) / HR - (NR * IR) / HR : 0;
    constexpr int w = IW >= 0 ? (NW * (IW + 1)) / HW - (NW * IW) / HW : 0;
    constexpr int v = IW >= 0 ? (NV * (IW + 1)) / HW - (NV * IW) / HW : 0;
    if constexpr (r > 0) DPG_SG_DSR(r);
    DPG_SG_MFMA(1);
    if constexpr (w > 0) DPG_SG_DSW(w);
    if constexpr (v > 0) DPG_SG_VMR(v);
    sched_step<NM, NR, NW, NV, I + 1>();
  }
}

// Which operands a wave stages: both (four-wave tiles), or only A / only B
// (eight-wave tiles: waves 0-3 stage A, waves 4-7 stage B).
enum StageRole { ROLE_BOTH = 0, ROLE_A = 1, ROLE_B = 2 };

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, int ROLE>
struct FastMainLoop {
  static constexpr int BK = 64;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int NTL = ROLE == ROLE_BOTH ? NT : NT / 2;  // threads staging one operand
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int PLANE_A = BM * BK, PLANE_B = BN * BK, STAGE = PLANE_A + PLANE_B;
  typedef FastOperand<BM, A_KMAJ, NTL> OpA;
  typedef FastOperand<BN, B_KMAJ, NTL> OpB;
  static constexpr bool DO_A = ROLE != ROLE_B, DO_B = ROLE != ROLE_A;

  static __device__ __forceinline__ void run(__bf16* smem, const GemmParams& p, int ltid, int lane, int wm, int wn,
                                             int row0, int col0, int kt0, int nkt, f32x16 (&acc)[FM][FN]) {
    const __bf16* A = (const __bf16*)p.a;
    const __bf16* B = (const __bf16*)p.b;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    OpA opa;
    OpB opb;
    if (DO_A) opa.init(ltid, lda);
    if (DO_B) opb.init(ltid, ldb);

    // fragment read offsets (elements) for this lane: row part and chunk part
    const int lr = lane & 31, lh = lane >> 5;
    const int sw = fswz(lr);  // rows of a fragment start at multiples of 32
    int a_row[FM], b_row[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a_row[i] = (wm * WM + i * 32 + lr) * 64;
#pragma unroll
    for (int j = 0; j < FN; ++j) b_row[j] = PLANE_A + (wn * WN + j * 32 + lr) * 64;
    int koff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) koff[s] = ((2 * s + lh) ^ sw) << 3;

    bf16x8 fa[2][FM], fb[2][FN];
    auto read_frags = [&](const __bf16* stage, int s, int buf) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[buf][i] = as_bf16x8(*(const u32x4*)(stage + a_row[i] + koff[s]));
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[buf][j] = as_bf16x8(*(const u32x4*)(stage + b_row[j] + koff[s]));
    };
    auto mfmas = [&](int buf, int i_begin, int i_end) {
#pragma unroll
      for (int i = i_begin; i < i_end; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fa[buf][i], fb[buf][j], acc[i][j]);
    };
    auto load = [&](int k) {
      if (DO_A) opa.load(tile_rsrc<A_KMAJ>(A, lda, row0, p.M, k, p.K));
      if (DO_B) opb.load(tile_rsrc<B_KMAJ>(B, ldb, col0, p.N, k, p.K));
    };
    auto store = [&](__bf16* stage) {
      if (DO_A) opa.store(stage);
      if (DO_B) opb.store(stage + PLANE_A);
    };

    if (nkt > 0) {
      load(kt0 * BK);
      store(smem);
      load((kt0 + 1) * BK);
      __syncthreads();
      read_frags(smem, 0, 0);
    }

    constexpr int NM = FM * FN;  // MFMAs per k-step
    constexpr int NR = FM + FN;  // fragment reads per k-step
    constexpr int NW = (DO_A ? OpA::LOADS : 0) + (DO_B ? OpB::LOADS : 0);  // LDS writes per tile
    constexpr int NV = NW;                                                 // buffer loads per tile
    for (int it = 0; it < nkt; ++it) {
      const __bf16* cur = smem + (it & 1) * STAGE;
      __bf16* nxt = smem + ((it + 1) & 1) * STAGE;
      // k-step 0: fragments of step 1 while the MFMAs of step 0 issue
      read_frags(cur, 1, 1);
      mfmas(0, 0, FM);
      sched_step<NM, NR, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // k-step 1: fragments of step 2; stage the next tile into the other buffer
      read_frags(cur, 2, 0);
      mfmas(1, 0, FM);
      store(nxt);
      sched_step<NM, NR, NW, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // k-step 2: fragments of step 3; fetch the tile after next
      read_frags(cur, 3, 1);
      mfmas(0, 0, FM);
      load((kt0 + it + 2) * BK);
      sched_step<NM, NR, 0, NV>();
      __builtin_amdgcn_sched_barrier(0);
      // k-step 3: half the MFMAs, barrier, first fragments of the next tile, rest
      mfmas(1, 0, FM / 2);
      __syncthreads();
      read_frags(nxt, 0, 0);  // unused after the last tile (in-bounds LDS)
      mfmas(1, FM / 2, FM);
      sched_step<NM / 2, NR, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, int OUT>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1) gemm_fast_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(NT == 256 || NT == 512, "four or eight waves");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (BM + BN) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int tiles = p.tiles_m * p.tiles_n;
  const int pid = xcd_remap(blockIdx.x, tiles * p.splits);
  const int split = pid / tiles;
  const int t = pid % tiles;
  const int per_group = p.group_m * p.tiles_n;
  const int group = t / per_group;
  const int first_m = group * p.group_m;
  const int gsize = min(p.tiles_m - first_m, p.group_m);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int row0 = tm * BM, col0 = tn * BN;

  const int kt0 = split * p.kt_per_split;
  const int kt1 = min(kt0 + p.kt_per_split, p.kt_total);
  const int nkt = kt1 - kt0;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if constexpr (NT == 512) {
    if (wave < 4)
      FastMainLoop<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, ROLE_A>::run(smem, p, tid, lane, wm, wn, row0, col0, kt0,
                                                                           nkt, acc);
    else
      FastMainLoop<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, ROLE_B>::run(smem, p, tid - 256, lane, wm, wn, row0, col0,
                                                                           kt0, nkt, acc);
  } else {
    FastMainLoop<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, ROLE_BOTH>::run(smem, p, tid, lane, wm, wn, row0, col0, kt0,
                                                                          nkt, acc);
  }

  // ---- epilogue: lane l owns column (l % 32) and rows (r/4)*8 + (l/32)*4 + r%4
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + wn * WN + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= p.M) continue;
        const float v = acc[i][j][r];
        if (OUT == OUT_BF16) {
          ((unsigned short*)p.c)[(int64_t)row * p.ldc + col] = (unsigned short)bf16_bits(v);
        } else if (OUT == OUT_F32) {
          ((float*)p.c)[(int64_t)row * p.ldc + col] = v;
        } else {
          ((float*)p.c)[(int64_t)split * p.split_stride + (int64_t)row * p.ldc + col] = v;
        }
      }
    }
  }
}

}  // namespace dpg
