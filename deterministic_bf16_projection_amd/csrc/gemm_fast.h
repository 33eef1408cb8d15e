// Software-pipelined MFMA GEMM for gfx950 (the path of the large projection
// passes and of the BF16x3 router from about a thousand tokens up).
// C[M,N] = sum_k A(m,k) * B(n,k), FP32 accumulation.
//
// Compared with the generic kernel in gemm_kernel.h:
// * Operands are fetched with raw buffer loads.  The buffer descriptor of each
//   operand covers exactly the valid part of the current K tile, so rows past
//   the matrix end and reduction rows past K read as zero in hardware: the main
//   loop has no branches.
// * MN-major operands (input gradient B, both weight-gradient operands) are
//   transposed in registers (8x8 blocks of BF16 through v_perm_b32, or of FP32
//   by renaming) on their way to LDS, so LDS always holds K-contiguous rows and
//   every MFMA fragment is one ds_read_b128.  Consecutive lanes read
//   consecutive 16-byte chunks of one global row.
// * LDS rows are 64 BF16 (128 B) with 16-byte chunks XOR-swizzled per row.
// * Per K tile (64) each wave runs 4 k-steps of 16; the fragments of step s+1
//   are read while the MFMAs of step s issue, the global loads of the tile
//   after next are issued right after the staged registers are written to the
//   other LDS stage, and the single barrier per tile sits in the middle of the
//   last step's MFMAs.
// * A K-major A is fetched straight into LDS (buffer_load ... lds), and so is
//   a K-major B where A is (the forward's W).  In the eight-wave kernel the
//   staging goes to the waves that win the issue arbitration (waves 0-3)
//   wherever their registers allow it (forward and input gradient), and the
//   other four waves only read fragments and issue MFMAs.
// * The grid is persistent: each workgroup walks a stream of (problem, tile,
//   K split) units with the K pipeline running across unit boundaries.
// * A finished unit is written through a 4 KB per-wave LDS buffer that turns
//   the MFMA output layout into rows, so each store instruction writes whole
//   128-byte row segments.
// * BF16x3 (FP32 operands): hi and lo BF16 planes per operand, split while
//   staging; each k-step adds lo*hi, hi*lo, hi*hi into one accumulator.
// Requirements: K-major operands have K % 64 == 0 (planner); all contiguous
// extents are multiples of 8 elements; row strides below 2^22 elements so a
// tile spans less than 2^31 bytes of buffer offsets (launcher).
#pragma once
#include "device_common.h"
#include "gemm_kernel.h"


namespace dpg {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

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

// The same transpose with the byte selectors of even and odd output slots
// passed in: swapping them (a per-lane choice) puts column m ^ 1 in slot m.
__device__ __forceinline__ void transpose8x8_sel(const u32x4 (&in)[8], u32x4 (&out)[8], uint32_t sel_even,
                                                 uint32_t sel_odd) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      out[m][e] = __builtin_amdgcn_perm(in[2 * e + 1][m >> 1], in[2 * e][m >> 1], (m & 1) ? sel_odd : sel_even);
  }
}

// LDS K-major layout: row r (64 BF16 = 8 chunks of 16 B); chunk c stored at
// position c ^ fswz(r), a 3-bit pattern of r and r / 8.  The 16 rows one
// ds_read_b128 phase touches (16 consecutive rows) fall on distinct banks, and
// so do the rows 8 mb + m of a transposed-block write phase (see FastOperand).
// For a row 32 q + l (l < 32), fswz = fswz(l) ^ 4 (q & 1).
__device__ __forceinline__ int fswz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_chunk_off(int r, int c) { return r * 64 + ((c ^ fswz(r)) << 3); }

// One operand: R rows (M or N side) by 64 reduction elements per K tile.
template <int R, bool KMAJ, int NT>
struct FastOperand {
  // K-major: 16-byte chunks (row, k-chunk) per thread, rows tid/8 + 32 i.
  // MN-major: one 8x8 block per thread for the first R threads.
  static_assert(NT == 256 && (KMAJ || R <= NT), "one block per thread, 32 rows per K-major load");
  static constexpr int LOADS = KMAJ ? R * 8 / NT : 8;
  static constexpr int BLOCK_THREADS = KMAJ ? NT : R;  // threads that own data
  static constexpr int NLOADS = LOADS, NWRITES = LOADS;  // per K tile (scheduling)
  u32x4 g[LOADS];
  // Load i reads at voff0 + i * vstep bytes, and LDS slot i goes to lds0 with
  // a per-slot constant (added for K-major, XORed for MN-major).
  uint32_t voff0, vstep;
  int lds0;
  uint32_t sel_even, sel_odd;  // transpose byte selectors (MN-major)
  bool owner;

  // set up per-thread offsets; ld in elements
  __device__ __forceinline__ void init(int tid, int64_t ld) {
    owner = tid < BLOCK_THREADS;
    if (KMAJ) {
      // rows r + 32 i: offset lds_chunk_off(r, c) + 2048 i, with chunk bit 2
      // flipped for odd i (fswz(r + 32) = fswz(r) ^ 4)
      const int c = tid & 7, r = tid >> 3;
      voff0 = (uint32_t)(r * ld * 2 + c * 16);
      vstep = (uint32_t)(32 * ld * 2);
      lds0 = lds_chunk_off(r, c);
    } else {
      // mb = tid % (R/8) (8 columns), kc = tid / (R/8) (8 reduction rows), so
      // consecutive lanes read consecutive 16-byte chunks of one row.  Lanes
      // with (mb / 8) odd keep column m ^ 1 in slot m: the 16 lanes of a write
      // phase then cover rows of both parities and, with the row swizzle, 16
      // distinct bank groups.  Slot m goes to row 8 mb + (m ^ flip), i.e. to
      // element offset lds0 ^ 72 m with lds0 = 512 mb | 8 (9 flip ^ (kc ^ mb) % 8).
      const int mb = tid % (R / 8), kc = (tid / (R / 8)) & 7;
      const int flip = (mb >> 3) & 1;
      sel_even = flip ? 0x07060302u : 0x05040100u;
      sel_odd = flip ? 0x05040100u : 0x07060302u;
      voff0 = (uint32_t)(kc * 8 * ld * 2 + mb * 16);
      vstep = (uint32_t)(ld * 2);
      lds0 = (mb * 512) | ((((9 * flip) ^ ((kc ^ mb) & 7))) << 3);
    }
  }

  __device__ __forceinline__ void load(rsrc_t r) {
    if (BLOCK_THREADS < NT && !owner) return;
    const uint32_t v = voff0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) g[i] = buf_load16(r, v + (uint32_t)i * vstep);
  }

  __device__ __forceinline__ void store(__bf16* plane, __bf16* /*lo plane: BF16x3 only*/ = nullptr) const {
    if (BLOCK_THREADS < NT && !owner) return;
    int o = lds0;
    // MN-major: form the eight slot offsets here rather than in the loop
    // preheader (the eight-wave kernels would otherwise run out of registers)
    if constexpr (!KMAJ) asm volatile("" : "+v"(o));
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) *(u32x4*)(plane + ((i & 1) ? (o ^ 32) : o) + 2048 * i) = g[i];
    } else {
      u32x4 out[8];
      transpose8x8_sel(g, out, sel_even, sel_odd);
#pragma unroll
      for (int m = 0; m < 8; ++m) *(u32x4*)(plane + (o ^ (72 * m))) = out[m];
    }
  }
};

// BF16x3 operand: an FP32 source split while staging into hi = bf16(a) and
// lo = bf16(a - hi) (round to nearest even), written to two BF16 planes with
// FastOperand's LDS layout.  K-major: each thread stages whole 8-element
// chunks (two 16-byte loads each) of rows tid / 8 + 32 i.  MN-major: one 8x8
// block (8 reduction rows x 8 output rows, sixteen 16-byte loads) per thread
// for the first R threads, with FastOperand's lane numbering; the transpose of
// FP32 values is a renaming of registers, and lanes with (mb / 8) odd take
// column m ^ 1 into slot m by a per-lane select.
template <int R, bool KMAJ, int NT>
struct FastOperandX3 {
  static_assert(NT == 256 && R <= NT && (KMAJ || R % 8 == 0), "one block per thread, 32 rows per K-major chunk");
  static constexpr int CHUNKS = KMAJ ? R * 8 / NT : 1;  // K-major chunks per thread
  static constexpr int LOADS = KMAJ ? 2 * CHUNKS : 16;
  static constexpr int BLOCK_THREADS = KMAJ ? NT : R;
  static constexpr int NLOADS = LOADS, NWRITES = KMAJ ? 2 * CHUNKS : 16;
  u32x4 g[LOADS];
  uint32_t voff0, vstep;
  int lds0;
  int flip;
  bool owner;

  __device__ __forceinline__ void init(int tid, int64_t ld) {
    owner = tid < BLOCK_THREADS;
    if (KMAJ) {
      const int c = tid & 7, r = tid >> 3;
      voff0 = (uint32_t)((r * ld + c * 8) * 4);
      vstep = (uint32_t)(32 * ld * 4);
      lds0 = lds_chunk_off(r, c);
      flip = 0;
    } else {
      const int mb = tid % (R / 8), kc = (tid / (R / 8)) & 7;
      flip = (mb >> 3) & 1;
      voff0 = (uint32_t)((kc * 8 * ld + mb * 8) * 4);
      vstep = (uint32_t)(ld * 4);
      lds0 = (mb * 512) | ((((9 * flip) ^ ((kc ^ mb) & 7))) << 3);
    }
  }

  __device__ __forceinline__ void load(rsrc_t r) {
    if (BLOCK_THREADS < NT && !owner) return;
    const uint32_t v = voff0;
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        g[2 * i] = buf_load16(r, v + (uint32_t)i * vstep);
        g[2 * i + 1] = buf_load16(r, v + (uint32_t)i * vstep + 16u);
      }
    } else {
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        g[2 * l] = buf_load16(r, v + (uint32_t)l * vstep);
        g[2 * l + 1] = buf_load16(r, v + (uint32_t)l * vstep + 16u);
      }
    }
  }

  __device__ __forceinline__ void store(__bf16* hi_plane, __bf16* lo_plane) const {
    if (BLOCK_THREADS < NT && !owner) return;
    int o = lds0;
    asm volatile("" : "+v"(o));
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        u32x4 hi, lo;
        split3_x8(__builtin_bit_cast(f32x4, g[2 * i]), __builtin_bit_cast(f32x4, g[2 * i + 1]), hi, lo);
        const int off = ((i & 1) ? (o ^ 32) : o) + 2048 * i;
        *(u32x4*)(hi_plane + off) = hi;
        *(u32x4*)(lo_plane + off) = lo;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        // column m ^ flip of the block: element j = m ^ flip of each row's 8 values
        float f[8];
#pragma unroll
        for (int l = 0; l < 8; ++l) {
          const u32x4 q = g[2 * l + (m >> 2)];
          const uint32_t a = q[m & 3], b = q[(m & 3) ^ 1];
          f[l] = __builtin_bit_cast(float, flip ? b : a);
        }
        u32x4 hi, lo;
        split3_x8(f32x4{f[0], f[1], f[2], f[3]}, f32x4{f[4], f[5], f[6], f[7]}, hi, lo);
        *(u32x4*)(hi_plane + (o ^ (72 * m))) = hi;
        *(u32x4*)(lo_plane + (o ^ (72 * m))) = lo;
      }
    }
  }
};

// K-major operand fetched straight into LDS (buffer_load ... lds): each
// instruction moves 64 lanes x 16 B into 1 KB of consecutive LDS, i.e. 8 rows
// of the 64-wide K tile.  Lane l lands at row l / 8, chunk position l % 8 of
// its group and fetches the logical chunk the row swizzle puts there, so the
// LDS layout is the one lds_chunk_off describes.  Completion is tracked by
// vmcnt: the wave waits for its own fetch before the workgroup barrier.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int R, int NTL>
struct DmaOperand {
  static constexpr int NW = NTL / 64;
  static constexpr int GROUPS = R / 8;
  static constexpr int LOADS = GROUPS / NW;
  uint32_t voff[LOADS];
  int group0;
  __device__ __forceinline__ void init(int ltid, int64_t ld) {
    const int lane = ltid & 63, w = ltid >> 6;
    group0 = w;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int g = j * NW + w;
      const int r = g * 8 + (lane >> 3);
      const int c = (lane & 7) ^ fswz(r);
      voff[j] = (uint32_t)((r * ld + c * 8) * 2);
    }
  }
  __device__ __forceinline__ void load(rsrc_t rs, __bf16* plane) const {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int g = j * NW + group0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(plane + g * 512), 16, (int)voff[j], 0, 0, 0);
    }
  }
};

// Buffer descriptor of the K tile starting at k0 (32-bit arithmetic only: the
// launcher guarantees ld < 2^22, so one tile of at most 256 rows of BF16, or
// 128 rows of FP32, spans less than 2^31 bytes).
//  K-major (element (row, k) at ptr[row * ld + k]): rows [row0, rows), k < K.
//  MN-major (element (row, k) at ptr[k * ld + row]): reduction rows
//  [k0, min(K, k0 + 64)), columns [row0, rows) of each.
template <bool KMAJ, int TILE_ROWS = 256, class T>
__device__ __forceinline__ rsrc_t tile_rsrc(const T* ptr, int ld, int row0, int rows, int k0, int K) {
  int bytes;
  const T* base;
  if (KMAJ) {
    const int valid = min(rows - row0, TILE_ROWS);
    bytes = ((valid - 1) * ld + (K - k0)) * (int)sizeof(T);
    base = ptr + (int64_t)row0 * ld + k0;
  } else {
    const int kr = min(K - k0, 64);
    bytes = ((kr - 1) * ld + (rows - row0)) * (int)sizeof(T);
    bytes = kr > 0 ? bytes : 0;
    base = ptr + (int64_t)k0 * ld + row0;
  }
  bytes = max(bytes, 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, bytes, 0x00020000);
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

// Scheduling of one k-step: the pinned interleave above, or (IGLP) the
// compiler's own MFMA / DS interleave strategy (iglp_opt(0)).  The forward
// layout (both operands K-major) measured faster with the latter: the
// eight-wave 256x256 tile by 1.7% (five interleaved repeats of the 4096 ->
// 12288 step, every pair faster), the four-wave 128x128 tile by ~7% (4096 ->
// 512 at 16384 tokens, FP32 out); the gradient layouts were 3-4% slower, so
// only the forward layout uses it (BF16x3 tiles keep the pinned order).
template <bool IGLP, int NM, int NR, int NW, int NV>
__device__ __forceinline__ void sched_kstep() {
  if constexpr (IGLP)
    __builtin_amdgcn_iglp_opt(0);
  else
    sched_step<NM, NR, NW, NV>();
}

// Work units of a launch: one (output tile, K split) pair each.  The grid is
// persistent: workgroup b takes units b, b + grid, b + 2 grid, ...  Unit ids
// are mapped through the XCD remap and a grouped raster so that the units the
// workgroups of one XCD run at the same time form a compact block of tiles
// (shared A rows and B columns stay in that XCD's L2).
struct UnitMap {
  int tiles_m, tiles_n, group_m, splits, kt_per, kt_total, total;
  int per_batch;  // units of one problem (tiles x splits); total = per_batch x problems
  SplitParts sp;  // K partition of the splits
};

// Position of a stream of (unit, K tile) steps.
struct StepCursor {
  int u;            // unit id (>= total when past the end)
  int kt;           // K tile index within the unit's split
  int nkt, kt0;     // the unit's K tiles and first K tile
  int row0, col0;   // the unit's tile origin
  int split;
  int b;            // the unit's problem
};

template <int BM, int BN>
__device__ __forceinline__ StepCursor cursor_at(const UnitMap& m, int unit) {
  StepCursor c;
  c.u = unit;
  c.kt = 0;
  const int tiles = m.tiles_m * m.tiles_n;
  const int pid_all = xcd_remap(min(unit, m.total - 1), m.total);
  c.b = pid_all / m.per_batch;
  const int pid = pid_all - c.b * m.per_batch;
  const int split = pid / tiles;
  const int t = pid - split * tiles;
  const int per_group = m.group_m * m.tiles_n;
  const int group = t / per_group;
  const int first_m = group * m.group_m;
  const int gsize = min(m.tiles_m - first_m, m.group_m);
  const int r = t - group * per_group;
  c.row0 = (first_m + r % gsize) * BM;
  c.col0 = (r / gsize) * BN;
  c.split = split;
  c.kt0 = split_begin(split, m.sp);
  c.nkt = split_begin(split + 1, m.sp) - c.kt0;
  return c;
}

template <int BM, int BN>
__device__ __forceinline__ StepCursor cursor_next(const UnitMap& m, const StepCursor& c, int stride) {
  if (c.kt + 1 < c.nkt) {
    StepCursor n = c;
    n.kt = c.kt + 1;
    return n;
  }
  return cursor_at<BM, BN>(m, c.u + stride);
}

__device__ __forceinline__ bool cursor_valid(const UnitMap& m, const StepCursor& c) { return c.u < m.total; }

// Stream-K work of one workgroup (deterministic=0 plans; no split of K into
// planes).  Of the `tiles` output tiles the first D (whole rounds of the grid:
// D = (tiles / G) G) are data-parallel: workgroup g computes whole tiles g,
// g + G, ... (XCD-remapped like the unit stream).  The remaining tiles' K
// iterations (64-wide K tiles) form one sequence that is cut into G even
// ranges (split_begin over G), range g' = xcd_remap(g) for workgroup g, so
// every workgroup ends at the same time.
// A range covers parts of one or two tiles (or whole tiles): a tile covered
// whole is written out directly, a part goes to partial slot 2 g' (the range's
// first segment) or 2 g' + 1 (its last), which a fix-up kernel adds in range
// order, i.e. in ascending K.  A cursor position u counts K iterations along
// the workgroup's work list: data-parallel tiles first (KT each), then its
// range.
struct StreamKWork {
  int G, D, KT;        // grid, data-parallel tiles, K iterations per tile
  int dp_count;        // data-parallel tiles of this workgroup
  int g, i0, i1;       // this workgroup, its range's index and its iterations in the tail sequence
};

template <int BM, int BN>
__device__ __forceinline__ void tile_origin(const UnitMap& m, int t, int& row0, int& col0) {
  const int per_group = m.group_m * m.tiles_n;
  const int group = t / per_group;
  const int first_m = group * m.group_m;
  const int gsize = min(m.tiles_m - first_m, m.group_m);
  const int r = t - group * per_group;
  row0 = (first_m + r % gsize) * BM;
  col0 = (r / gsize) * BN;
}

template <int BM, int BN>
__device__ __forceinline__ StepCursor sk_cursor(const UnitMap& m, const StreamKWork& w, int u) {
  StepCursor c;
  c.u = u;
  c.kt = 0;
  c.b = 0;
  const int dp_iters = w.dp_count * w.KT;
  int t;
  if (u < dp_iters) {
    t = xcd_remap(w.g + (u / w.KT) * w.G, w.D);
    c.kt0 = 0;
    c.nkt = w.KT;
    c.split = 0;
  } else {
    const int i = w.i0 + (u - dp_iters);
    const int tt = i / w.KT;
    t = w.D + tt;
    c.kt0 = i - tt * w.KT;
    c.nkt = min(w.i1, (tt + 1) * w.KT) - i;
    c.split = i == w.i0 ? 0 : 1;
  }
  tile_origin<BM, BN>(m, min(t, m.tiles_m * m.tiles_n - 1), c.row0, c.col0);
  return c;
}

template <int BM, int BN>
__device__ __forceinline__ StepCursor sk_next(const UnitMap& m, const StreamKWork& w, const StepCursor& c) {
  if (c.kt + 1 < c.nkt) {
    StepCursor n = c;
    n.kt = c.kt + 1;
    return n;
  }
  return sk_cursor<BM, BN>(m, w, c.u + c.nkt);
}

// Which operands a wave stages: both (four-wave tiles), or only A / only B
// (eight-wave tiles: waves 0-3 stage A, waves 4-7 stage B).
enum StageRole { ROLE_BOTH = 0, ROLE_A = 1, ROLE_B = 2 };

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, int OUT, int ROLE, bool X3 = false,
          bool SK = false>
struct FastGemm {
  static constexpr int BK = 64;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int NTL = ROLE == ROLE_BOTH ? NT : NT / 2;  // threads staging one operand
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static_assert(WM % 64 == 0 && WN % 64 == 0, "fragment swizzle parity follows the fragment index");
  static_assert(!X3 || ROLE == ROLE_BOTH, "BF16x3 runs on the four-wave tile");
  static constexpr int FM0 = WM / 32, FN = WN / 32;
  // Rows of the tile per role.  Where waves 0-3 fetch A straight into LDS
  // (forward, input gradient) they are the late ones even with the issue
  // priority (timed inside the kernel, input gradient: waves 4-7 waited 18%
  // of the loop at the barrier, waves 0-3 7%; forward 9% and 5%), so there
  // waves 0-3 compute 96 of the 256 rows and waves 4-7 160: input gradient
  // 1.5-2.4%, forward 1.2-1.8% faster over four interleaved repeats, bitwise
  // equal (64 / 192 rows was level for the input gradient).  Elsewhere each
  // role computes WM rows.
  static constexpr bool SPLIT_ROWS = ROLE != ROLE_BOTH && !X3 && A_KMAJ;
  static constexpr int FM = SPLIT_ROWS ? (ROLE == ROLE_A ? FM0 - 1 : FM0 + 1) : FM0;
  // first row of this wave's part of the tile, and the swizzle parity of its
  // first fragment (fragment rows 32 q + l carry fswz(l) ^ 4 (q & 1))
  static __device__ __forceinline__ int row_start(int wm) {
    return SPLIT_ROWS ? (ROLE == ROLE_A ? 0 : (FM0 - 1) * 32) : wm * WM;
  }
  static constexpr int PAR = (SPLIT_ROWS && ROLE == ROLE_B) ? ((FM0 - 1) & 1) : 0;
  // BF16x3: every operand has a hi and a lo plane (A hi, A lo, B hi, B lo)
  static constexpr int PLANES = X3 ? 2 : 1;
  static constexpr int PLANE_A = BM * BK, PLANE_B = BN * BK, STAGE = (PLANE_A + PLANE_B) * PLANES;
  static constexpr int B_BASE = PLANE_A * PLANES;  // first B plane in a stage
  typedef typename std::conditional<X3, float, __bf16>::type InT;
  typedef typename std::conditional<X3, FastOperandX3<BM, A_KMAJ, NTL>, FastOperand<BM, A_KMAJ, NTL>>::type OpA;
  typedef typename std::conditional<X3, FastOperandX3<BN, B_KMAJ, NTL>, FastOperand<BN, B_KMAJ, NTL>>::type OpB;
  // Who stages what.  A K-major A (X in the forward pass, dY in the input
  // gradient) is fetched straight into LDS (buffer_load ... lds: no staging
  // registers, no LDS write instructions), which relieves the LDS issue
  // queue: 2.7% faster for the input gradient, 1.8% for the forward (six
  // interleaved repeats of the 4096 -> 12288 step at 16384 tokens).
  // Waves 0-3 (the A waves) win the issue arbitration against waves 4-7 on
  // each SIMD: timed inside the kernel, with equal work the A waves spent
  // about a third of every K tile waiting at the barrier for the B waves.
  // Where A is K-major the A waves therefore do all the staging and the B
  // waves only read fragments and issue MFMAs (forward: A waves' barrier wait
  // 32% -> 9-12%, 4-8.5% faster on two boxes; input gradient 5.5% faster).
  // In the forward the A waves fetch W straight into LDS as well (the LDS
  // fetch moves ~44 GB/s per CU from L2 against ~39 through registers): 4%
  // faster, no W staging registers (204 VGPRs); with the B waves fetching W
  // instead it was 11% slower.  The four-wave 128x128 forward tile fetches
  // both operands into LDS from all four waves (4096 -> 512 at 16384 tokens,
  // FP32 out: 82-98 -> 72-74 us).  The input gradient's W is MN-major and
  // stays on the register path (transposed there).  With both operands MN-major
  // (the weight gradient) each role stages its own operand: the A waves have
  // no registers for both transposed operands (23 VGPRs spilled, 60% slower).
  static constexpr bool A_INTO_LDS = !X3 && A_KMAJ && (ROLE != ROLE_BOTH || B_KMAJ);
  static constexpr bool DMA = A_INTO_LDS && ROLE != ROLE_B;               // this wave fetches A (and W, B_INTO_LDS)
  static constexpr bool DO_A = !A_INTO_LDS && ROLE != ROLE_B;             // A through registers
  static constexpr bool B_INTO_LDS = A_INTO_LDS && B_KMAJ;                // forward: W fetched by the A waves too
  static constexpr bool DO_B = B_INTO_LDS ? false : (A_INTO_LDS ? ROLE == ROLE_A : ROLE != ROLE_A);  // B through registers
  // Single-buffered A fragments (each row's fragment of the next k-step is
  // read right after that row's MFMAs issue; B fragments stay double
  // buffered): 16 fewer VGPRs, which the input gradient's A waves need to
  // hold the dY fetch and the transposed W staging together.
  static constexpr bool SB = A_INTO_LDS && !B_KMAJ;
  // Wait (s_waitcnt encoding) for this wave's own LDS fetch of the next
  // stage before the barrier; when the wave also stages B, the NLOADS B
  // loads issued after that fetch (for the K tile after next) stay in
  // flight: vmcnt retires loads in issue order.
  static_assert(!(DMA && DO_B) || OpB::NLOADS < 16, "vmcnt field");
  static constexpr int DMA_DONE = 0x0F70 | (DMA && DO_B ? OpB::NLOADS : 0);
  // k-step scheduling by the compiler's interleave strategy (see sched_kstep)
  static constexpr bool IGLP = !X3 && A_KMAJ && B_KMAJ;

  // Accumulators hold the transposed product: acc[i][j] is the 32x32 block
  // D[n][m] = sum_k B(n,k) A(m,k), so that lane l owns output row m = l % 32
  // and the four consecutive columns n = (r/4)*8 + (l/32)*4 + [0,4).
  //
  // The output leaves through a 4 KB per-wave LDS buffer of 32 rows x 128 B
  // (16-byte chunks swizzled with fswz): a block row of the wave's tile (32
  // rows x 64 BF16 columns, or x 32 FP32 columns per block) is written there
  // in the MFMA layout and read back so that 8 consecutive lanes hold one
  // row's 128 contiguous bytes.  Every store instruction then writes 8 whole
  // 128-byte row segments instead of 32 pieces of 32 B: for the FP32
  // input gradient of 4096 -> 1024 at 16384 tokens, 189 -> 139 us.
  static __device__ __forceinline__ void epilogue(const GemmParams& p, const StepCursor& c, int lane, int wm, int wn,
                                                  f32x16 (&acc)[FM][FN], char* scr) {
    char* out;
    if (OUT == OUT_PARTIAL)
      out = (char*)p.c + ((int64_t)c.b * p.batch_c + (int64_t)c.split * p.split_stride) * 4;
    else
      out = (char*)p.c + (int64_t)c.b * p.batch_c * (OUT == OUT_BF16 ? 2 : 4);
    store_tile<OUT>(out, p.ldc, 0, 0, p.M, p.N, c.row0, c.col0, lane, wm, wn, acc, scr);
  }

  // The unit's tile (rows row0.., columns col0..) as EOUT: element (m, n), m <
  // M and n < N, goes to out + ((m - mo) ldc + (n - no)) elements.
  template <int EOUT>
  static __device__ __forceinline__ void store_tile(char* out, int64_t ldc, int mo, int no, int M, int N, int row0,
                                                    int col0, int lane, int wm, int wn, f32x16 (&acc)[FM][FN],
                                                    char* scr) {
    static_assert(FN == 2, "a wave's row segment is 64 columns");
    // lane-derived offsets are formed here rather than kept live across the
    // main loop (which would run the MN-major kernels out of registers)
    asm volatile("" : "+v"(lane));
    const int lr = lane & 31, lh = lane >> 5;
    const int sw = fswz(lr);
    // read-back: lane l takes row 8 k + l / 8, chunk l % 8; fswz(8 k + rr) = rr ^ k
    const int rr = lane >> 3, cc = lane & 7;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m0 = row0 + row_start(wm) + i * 32;
      if constexpr (EOUT == OUT_BF16) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          // Columns 16 h + [0, 16) of block j: lane l (< 32) holds 16 h + [0, 4)
          // (group 2h) and 16 h + [8, 12) (group 2h + 1), lane l + 32 the next
          // four of each.  Swapping group 2h of the upper lanes with group 2h + 1
          // of the lower lanes leaves lane l with 16 h + [0, 8) and lane l + 32
          // with 16 h + [8, 16): chunk 4 j + 2 h + l / 32 of the row.
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int q0 = 2 * h, q1 = 2 * h + 1;
            const uint32_t x0 = pack_bf16x2(acc[i][j][4 * q0], acc[i][j][4 * q0 + 1]);
            const uint32_t x1 = pack_bf16x2(acc[i][j][4 * q0 + 2], acc[i][j][4 * q0 + 3]);
            const uint32_t y0 = pack_bf16x2(acc[i][j][4 * q1], acc[i][j][4 * q1 + 1]);
            const uint32_t y1 = pack_bf16x2(acc[i][j][4 * q1 + 2], acc[i][j][4 * q1 + 3]);
            const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
            const int chunk = 4 * j + 2 * h + lh;
            *(u32x4*)(scr + lr * 128 + ((chunk ^ sw) << 4)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = 8 * k + rr;
          const u32x4 v = *(const u32x4*)(scr + r * 128 + ((cc ^ rr ^ k) << 4));
          const int m = m0 + r, n = col0 + wn * WN + cc * 8;
          if (m < M && n < N) *(u32x4*)(out + ((int64_t)(m - mo) * ldc + (n - no)) * 2) = v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          // group q of lane l is chunk 2 q + l / 32 of the block's 32-column row
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(f32x4*)(scr + lr * 128 + (((2 * q + lh) ^ sw) << 4)) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + rr;
            const f32x4 v = *(const f32x4*)(scr + r * 128 + ((cc ^ rr ^ k) << 4));
            const int m = m0 + r, n = col0 + wn * WN + j * 32 + cc * 4;
            if (m < M && n < N) *(f32x4*)(out + ((int64_t)(m - mo) * ldc + (n - no)) * 4) = v;
          }
        }
      }
    }
  }

  static __device__ __forceinline__ void run(__bf16* smem, const GemmParams& p, int ltid, int lane, int wm, int wn) {
    // this wave's epilogue buffer, after the two pipeline stages
    char* scr = (char*)(smem + 2 * STAGE) + (wm * WAVES_N + wn) * 4096;
    const InT* A = (const InT*)p.a;
    const InT* B = (const InT*)p.b;
    const int lda = (int)p.lda, ldb = (int)p.ldb;
    StreamKWork skw = {};
    if constexpr (SK) {
      const int tiles = p.tiles_m * p.tiles_n;
      skw.G = gridDim.x;
      skw.KT = p.kt_total;
      skw.D = (tiles / skw.G) * skw.G;
      skw.dp_count = skw.D / skw.G;
      skw.g = blockIdx.x;
      const SplitParts sp = split_parts(skw.G, (tiles - skw.D) * skw.KT);
      const int gr = xcd_remap(blockIdx.x, skw.G);
      skw.i0 = split_begin(gr, sp);
      skw.i1 = split_begin(gr + 1, sp);
    }
    const UnitMap um = {p.tiles_m, p.tiles_n, p.group_m, p.splits, p.kt_per_split, p.kt_total,
                        SK ? skw.dp_count * skw.KT + (skw.i1 - skw.i0) : p.tiles_m * p.tiles_n * p.splits * p.batch,
                        p.tiles_m * p.tiles_n * p.splits, split_parts(p.splits, p.kt_total)};
    const int stride = gridDim.x;
    // the workgroup's unit stream: (tile, K split) units, or its stream-K work
    auto first_step = [&]() -> StepCursor {
      if constexpr (SK)
        return sk_cursor<BM, BN>(um, skw, 0);
      else
        return cursor_at<BM, BN>(um, blockIdx.x);
    };
    auto next_step = [&](const StepCursor& c) -> StepCursor {
      if constexpr (SK)
        return sk_next<BM, BN>(um, skw, c);
      else
        return cursor_next<BM, BN>(um, c, stride);
    };
    OpA opa;
    OpB opb;
    DmaOperand<BM, NTL> opd;
    DmaOperand<BN, NTL> opdb;
    if constexpr (DMA) opd.init(ltid, lda);
    if constexpr (DMA && B_INTO_LDS) opdb.init(ltid, ldb);
    if (DO_A) opa.init(ltid, lda);
    if (DO_B) opb.init(ltid, ldb);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragment read offsets (elements) for this lane: row part and chunk part
    const int lr = lane & 31, lh = lane >> 5;
    // fragment rows start at multiples of 32: fragment i sits at pattern
    // fswz(lr) ^ 4 ((i + PAR) & 1), so it reads chunk (2 S + lh) at
    // koff[S ^ 2 ((i + PAR) & 1)]
    const int sw = fswz(lr);
    int a_row[FM], b_row[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a_row[i] = (row_start(wm) + i * 32 + lr) * 64;
#pragma unroll
    for (int j = 0; j < FN; ++j) b_row[j] = B_BASE + (wn * WN + j * 32 + lr) * 64;
    int koff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) koff[s] = ((2 * s + lh) ^ sw) << 3;

    bf16x8 fa[2][FM], fb[2][FN];
    bf16x8 fal[2][FM], fbl[2][FN];  // BF16x3 lo fragments
#define DPG_READ_A(stage, S, BUF, i)                                                                         \
  do {                                                                                                     \
    fa[BUF][i] = as_bf16x8(*(const u32x4*)((stage) + a_row[i] + koff[(S) ^ (2 * (((i) + PAR) & 1))]));             \
    if constexpr (X3)                                                                                      \
      fal[BUF][i] = as_bf16x8(*(const u32x4*)((stage) + PLANE_A + a_row[i] + koff[(S) ^ (2 * (((i) + PAR) & 1))])); \
  } while (0)
#define DPG_READ_B(stage, S, BUF, j)                                                                         \
  do {                                                                                                     \
    fb[BUF][j] = as_bf16x8(*(const u32x4*)((stage) + b_row[j] + koff[(S) ^ (2 * ((j) & 1))]));             \
    if constexpr (X3)                                                                                      \
      fbl[BUF][j] = as_bf16x8(*(const u32x4*)((stage) + PLANE_B + b_row[j] + koff[(S) ^ (2 * ((j) & 1))])); \
  } while (0)
    // fragments of k-step S (0..3) of a stage into buffer BUF (hi and, for
    // BF16x3, lo planes).  Weight gradient: in the order the MFMAs use them
    // (A row 0, all of B, the other A rows), measured 2.5% faster there; the
    // other layouts keep A before B, which measured 1.4% faster for the forward.
#define DPG_READ_FRAGS(stage, S, BUF)                                                                      \
  do {                                                                                                     \
    if constexpr (!A_KMAJ) {                                                                               \
      DPG_READ_A(stage, S, BUF, 0);                                                                        \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) DPG_READ_B(stage, S, BUF, j);                         \
      _Pragma("unroll") for (int i = 1; i < FM; ++i) DPG_READ_A(stage, S, BUF, i);                         \
    } else {                                                                                               \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) DPG_READ_A(stage, S, BUF, i);                         \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) DPG_READ_B(stage, S, BUF, j);                         \
    }                                                                                                      \
  } while (0)
    // MFMAs of rows [I0, I1) of the wave tile from fragment buffer BUF; BF16x3
    // adds lo*hi, hi*lo, hi*hi in that order into each accumulator
#define DPG_MFMAS(BUF, I0, I1)                                                                             \
  do {                                                                                                     \
    _Pragma("unroll") for (int i = (I0); i < (I1); ++i) _Pragma("unroll") for (int j = 0; j < FN; ++j) {   \
      if constexpr (X3) {                                                                                  \
        acc[i][j] = mfma32(fb[BUF][j], fal[BUF][i], acc[i][j]);                                            \
        acc[i][j] = mfma32(fbl[BUF][j], fa[BUF][i], acc[i][j]);                                            \
      }                                                                                                    \
      acc[i][j] = mfma32(fb[BUF][j], fa[BUF][i], acc[i][j]);                                               \
    }                                                                                                      \
  } while (0)
    // loads of the step at cursor L (out-of-range steps read nothing)
    auto load = [&](const StepCursor& L) {
      // a step past the last unit gets empty descriptors (one row, no K left)
      const bool ok = cursor_valid(um, L);
      const int kk = ok ? (L.kt0 + L.kt) * BK : p.K;
      if (DO_A)
        opa.load(tile_rsrc<A_KMAJ, BM>(A + L.b * p.batch_a, lda, L.row0, ok ? p.M : L.row0 + 1, kk, p.K));
      if (DO_B)
        opb.load(tile_rsrc<B_KMAJ, BN>(B + L.b * p.batch_b, ldb, L.col0, ok ? p.N : L.col0 + 1, kk, p.K));
    };
    auto store = [&](__bf16* stage) {
      if (DO_A) opa.store(stage, stage + PLANE_A);
      if (DO_B) opb.store(stage + B_BASE, stage + B_BASE + PLANE_B);
    };
    auto dma = [&](const StepCursor& L, __bf16* stage) {
      const bool ok = cursor_valid(um, L);
      const int kk = ok ? (L.kt0 + L.kt) * BK : p.K;
      opd.load(tile_rsrc<true, BM>(A + L.b * p.batch_a, lda, L.row0, ok ? p.M : L.row0 + 1, kk, p.K), stage);
      if constexpr (B_INTO_LDS)
        opdb.load(tile_rsrc<true, BN>(B + L.b * p.batch_b, ldb, L.col0, ok ? p.N : L.col0 + 1, kk, p.K),
                  stage + B_BASE);
    };

    StepCursor C = first_step();
    if (!cursor_valid(um, C)) return;
    StepCursor L = C;
    // prologue: K tile 0 into stage 0, the loads of K tile 1 in flight
    if constexpr (DMA) dma(L, smem);
    if constexpr (DO_A || DO_B) load(L);
    L = next_step(L);
    if constexpr (DO_A || DO_B) {
      store(smem);
      load(L);
    }
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(DMA_DONE);
    __syncthreads();
    if constexpr (DMA) dma(L, smem + STAGE);
    L = next_step(L);
    bf16x8 fa1[FM];  // single-buffered A fragments (SB)
#define DPG_SB_READ_B(stage, S, BUF)                                                                       \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) fb[BUF][j] =                                              \
      as_bf16x8(*(const u32x4*)((stage) + b_row[j] + koff[(S) ^ (2 * (j & 1))]))
#define DPG_SB_READ_A(stage, S, i) \
  fa1[i] = as_bf16x8(*(const u32x4*)((stage) + a_row[i] + koff[(S) ^ (2 * (((i) + PAR) & 1))]))
#define DPG_SB_ROW(BUF, i) \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fb[BUF][j], fa1[i], acc[i][j])
    if constexpr (SB) {
      DPG_SB_READ_B(smem, 0, 0);
#pragma unroll
      for (int i = 0; i < FM; ++i) DPG_SB_READ_A(smem, 0, i);
    } else {
      DPG_READ_FRAGS(smem, 0, 0);
    }

    constexpr int NM = FM * FN * (X3 ? 3 : 1);  // MFMAs per k-step
    constexpr int NR = (FM + FN) * PLANES;        // fragment reads per k-step
    constexpr int NW = (DO_A ? OpA::NWRITES : 0) + (DO_B ? OpB::NWRITES : 0);  // LDS writes per tile
    constexpr int NV = (DO_A ? OpA::NLOADS : 0) + (DO_B ? OpB::NLOADS : 0);    // buffer loads per tile
    for (int it = 0; cursor_valid(um, C); ++it) {
      const __bf16* cur = smem + (it & 1) * STAGE;
      __bf16* nxt = smem + ((it + 1) & 1) * STAGE;
      if constexpr (SB) {
        // k-steps 0-2: the next step's B fragments, then row by row the MFMAs
        // and the next step's A fragment of that row; the A waves stage in
        // k-step 1
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          DPG_SB_READ_B(cur, s + 1, (s + 1) & 1);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            DPG_SB_ROW(s & 1, i);
            DPG_SB_READ_A(cur, s + 1, i);
          }
          if (s == 1 && (DO_A || DO_B)) {
            store(nxt);
            load(L);
          }
          sched_kstep<IGLP, NM, NR, 0, 0>();
          __builtin_amdgcn_sched_barrier(0);
        }
        // k-step 3: half the rows, barrier, the next K tile's first fragments
        // as the other rows' MFMAs issue
#pragma unroll
        for (int i = 0; i < FM / 2; ++i) DPG_SB_ROW(1, i);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DMA) __builtin_amdgcn_s_waitcnt(DMA_DONE);
        __syncthreads();
        if constexpr (DMA) dma(L, (__bf16*)cur);
        DPG_SB_READ_B(nxt, 0, 0);
#pragma unroll
        for (int i = 0; i < FM / 2; ++i) DPG_SB_READ_A(nxt, 0, i);
#pragma unroll
        for (int i = FM / 2; i < FM; ++i) {
          DPG_SB_ROW(1, i);
          DPG_SB_READ_A(nxt, 0, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // k-step 0: fragments of step 1 while the MFMAs of step 0 issue
        DPG_READ_FRAGS(cur, 1, 1);
        DPG_MFMAS(0, 0, FM);
        sched_kstep<IGLP, NM, NR, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1: fragments of step 2.  The A waves (and the four-wave
        // tile's waves) write their staged registers of the next K tile into
        // the other buffer and fetch the one after next here; B waves that
        // stage through registers (weight gradient) do it in k-step 2, so the
        // two waves sharing a SIMD wait for memory at different times.
        DPG_READ_FRAGS(cur, 2, 0);
        DPG_MFMAS(1, 0, FM);
        if constexpr (ROLE != ROLE_B && (DO_A || DO_B)) {
          store(nxt);
          load(L);
          sched_kstep<IGLP, NM, NR, NW, NV>();
        } else {
          sched_kstep<IGLP, NM, NR, 0, 0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-step 2: fragments of step 3
        DPG_READ_FRAGS(cur, 3, 1);
        DPG_MFMAS(0, 0, FM);
        if constexpr (ROLE == ROLE_B && (DO_A || DO_B)) {
          store(nxt);
          load(L);
          sched_kstep<IGLP, NM, NR, NW, NV>();
        } else {
          sched_kstep<IGLP, NM, NR, 0, 0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-step 3: half the MFMAs, barrier, first fragments of the next K tile, rest
        DPG_MFMAS(1, 0, FM / 2);
        // keep these MFMAs ahead of the barrier: MFMAs have no side effects, so
        // the scheduler would otherwise sink them past it
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DMA) __builtin_amdgcn_s_waitcnt(DMA_DONE);
        __syncthreads();
        if constexpr (DMA) dma(L, (__bf16*)cur);
        DPG_READ_FRAGS(nxt, 0, 0);  // garbage after the last step (in-bounds LDS)
        DPG_MFMAS(1, FM / 2, FM);
        if constexpr (DMA)
          sched_kstep<IGLP, NM / 2, NR, 0, decltype(opd)::LOADS * (B_INTO_LDS ? 2 : 1)>();
        else
          sched_kstep<IGLP, NM / 2, NR, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
      }
      L = next_step(L);
      if (C.kt + 1 >= C.nkt) {
        // the unit is complete: write it while the next unit's loads are in flight
        if constexpr (SK) {
          if (C.kt0 == 0 && C.nkt == p.kt_total) {
            epilogue(p, C, lane, wm, wn, acc, scr);
          } else {
            const int gr = xcd_remap(skw.g, skw.G);
            char* slot = (char*)p.sk_ws + (int64_t)(2 * gr + C.split) * (BM * BN * 4);
            store_tile<OUT_PARTIAL>(slot, BN, C.row0, C.col0, p.M, p.N, C.row0, C.col0, lane, wm, wn, acc, scr);
          }
        } else {
          epilogue(p, C, lane, wm, wn, acc, scr);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
      }
      C = next_step(C);
    }
#undef DPG_SB_READ_B
#undef DPG_SB_READ_A
#undef DPG_SB_ROW
#undef DPG_READ_FRAGS
#undef DPG_READ_A
#undef DPG_READ_B
#undef DPG_MFMAS
  }
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, int OUT, bool X3 = false,
          bool SK = false>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1) gemm_fast_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  static_assert(NT == 256 || NT == 512, "four or eight waves");
  static_assert(!X3 || NT == 256, "BF16x3 runs on the four-wave tile");
  // two pipeline stages, then 4 KB of epilogue buffer per wave (160 KB in all for
  // the eight-wave tile)
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (BM + BN) * BK * (X3 ? 2 : 1) + NT / 64 * 2048];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: SGPR
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  if constexpr (NT == 512) {
    if (wave < 4)
      FastGemm<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, OUT, ROLE_A, false, SK>::run(smem, p, tid, lane, wm, wn);
    else
      FastGemm<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, OUT, ROLE_B, false, SK>::run(smem, p, tid - 256, lane, wm, wn);
  } else {
    FastGemm<BM, BN, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, OUT, ROLE_BOTH, X3, SK>::run(smem, p, tid, lane, wm, wn);
  }
}

// Stream-K fix-up: each tail tile that two or more ranges share (see
// StreamKWork) is the sum of their partial slots in range order (ascending
// K), converted to the output type; other tiles were written by the GEMM
// kernel.  kStreamKFixupChunks workgroups per tail tile, each a 1/16 of its
// BM x BN elements (a tail tile can hold the partials of many ranges).
constexpr int kStreamKFixupChunks = 16;

template <int OUT>
__global__ void __launch_bounds__(256) streamk_fixup_kernel(GemmParams p, int BM, int BN, int G) {
  const int tiles = p.tiles_m * p.tiles_n;
  const int KT = p.kt_total;
  const int D = (tiles / G) * G;
  const int t = D + (int)blockIdx.x / kStreamKFixupChunks;
  const int chunk = (int)blockIdx.x % kStreamKFixupChunks;
  if (t >= tiles) return;
  const SplitParts sp = split_parts(G, (tiles - D) * KT);
  const int a = (t - D) * KT, b = a + KT - 1;
  // the range holding iteration i: the first r ranges have q + 1 iterations
  auto owner = [&](int i) {
    const int big = sp.r * (sp.q + 1);
    return i < big ? i / (sp.q + 1) : sp.r + (i - big) / sp.q;
  };
  const int g0 = owner(a), g1 = owner(b);
  if (g0 == g1) return;
  const UnitMap um = {p.tiles_m, p.tiles_n, p.group_m, 1, KT, KT, tiles, tiles, SplitParts{KT, 0}};
  int row0, col0;
  tile_origin<1, 1>(um, t, row0, col0);
  row0 *= BM;
  col0 *= BN;
  const float* ws = (const float*)p.sk_ws;
  const int per_chunk = BM * BN / 4 / kStreamKFixupChunks;
  for (int e = chunk * per_chunk + threadIdx.x; e < (chunk + 1) * per_chunk; e += 256) {
    const int r = e / (BN / 4), c4 = (e - r * (BN / 4)) * 4;
    const int m = row0 + r, n = col0 + c4;
    if (m >= p.M || n >= p.N) continue;
    const int64_t off = (int64_t)r * BN + c4;
    // ranges g0 .. g1 in order; range g's part of this tile is its first
    // segment (slot 2 g) when the range starts inside the tile, else its last
    f32x4 v = *(const f32x4*)(ws + (int64_t)(2 * g0 + (split_begin(g0, sp) >= a ? 0 : 1)) * BM * BN + off);
    for (int g = g0 + 1; g <= g1; ++g) {
      const f32x4 w = *(const f32x4*)(ws + (int64_t)(2 * g) * BM * BN + off);
      v[0] += w[0];
      v[1] += w[1];
      v[2] += w[2];
      v[3] += w[3];
    }
    if (OUT == OUT_BF16)
      *(u32x2*)((unsigned short*)p.c + (int64_t)m * p.ldc + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
      *(f32x4*)((float*)p.c + (int64_t)m * p.ldc + n) = v;
  }
}

}  // namespace dpg
