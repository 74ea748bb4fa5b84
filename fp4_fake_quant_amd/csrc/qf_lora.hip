// LoRA merge-then-quantize for MoE experts and the STE gradients of the adapters.
//
// What is computed: QATFactory project page, "Method" section, "Quantization-
// aware distillation": LoRA keeps one frozen base, trains only the adapters and
// quantizes the merged weight; for MoE models it merges and quantizes one expert
// at a time to bound peak memory.  With the identity STE ("Framework
// overview") the gradient G of the QDQ'd merged weight reaches the adapters as
// dB = G . A^T and dA = B^T . G.
//
// Merge (bit-exact, include/qf.h): acc = 0; for k = 0 .. r-1, acc = fma(B[i,k],
// A[k,j], acc) (each bf16 x bf16 product is exact in fp32, so this is the sum
// with one rounding per step, in k order); M[i,j] = bf16(fl(W[i,j] + acc)).
//
// The two merge passes compute this sum in two ways that give the same bits: pass 1 on
// the fp32 matrix cores (a chain of K = 1 steps is the same sequence of fused steps),
// pass 2 with vector FMAs.
//
// Kernels
//   k_lora_merge_amax  pass 1: M = W + B.A per 32 x 64 tile, S on the matrix cores with W
//                      and B streamed through a per-wave LDS ring; stores M (or not, M
//                      null) and folds max|M| into its tied group's partial.
//   k_lora_merge_qdq   pass 2 without M in memory: merges again (vector FMAs, a 512-column
//                      slab per wave, one row at a time) and NVFP4-QDQs and packs the
//                      merged rows in registers.
//   k_lora_grads       dB = G . A^T and dA = B^T . G in one pass over G, both on the
//                      16x16x32 BF16 MFMA (G staged through LDS); per-slab dB partials and
//                      per-row-block dA partials, added in a fixed order by
//                      k_lora_grad_reduce (same inputs, same bits).
#include <algorithm>

#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Keeps the scheduler from moving instructions across this point: rows (or column
// steps) stay in program order, so each waits only for its own prefetched load.
#define LORA_FENCE() __builtin_amdgcn_sched_barrier(0)


__device__ __forceinline__ void unpack8(uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Expert e of a descriptor: its tensors, each stacked contiguously after expert e - 1's,
// and its tied group.
struct LoraMat {
  const uint16_t* W;
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* G;
  uint16_t* M;
  uint16_t* y;
  uint8_t* codes;
  uint8_t* scales;
  float* dA;
  float* dB;
  float* dA_partial;
  float* dB_partial;
  int group;
};

template <typename P>
__device__ __forceinline__ P* lora_at(P* p, int64_t off) {
  return p ? p + off : p;
}

__device__ __forceinline__ LoraMat lora_mat(const LoraTensor& T, int e, int da_rows) {
  const int64_t rc = T.rows * T.cols, r = T.r;
  LoraMat m;
  m.W = lora_at(T.W, e * T.rows * T.ldw);
  m.A = lora_at(T.A, e * r * T.cols);
  m.B = lora_at(T.B, e * T.rows * r);
  m.G = lora_at(T.G, e * rc);
  m.M = lora_at(T.M, e * rc);
  m.y = lora_at(T.y, e * rc);
  m.codes = lora_at(T.codes, e * rc / 2);
  m.scales = lora_at(T.scales, e * rc / 16);
  m.dA = lora_at(T.dA, e * r * T.cols);
  m.dB = lora_at(T.dB, e * T.rows * r);
  m.dA_partial = lora_at(T.dA_partial, e * ((T.rows + da_rows - 1) / da_rows) * LORA_MAX_R * T.cols);
  m.dB_partial = lora_at(T.dB_partial, e * (int64_t)T.slabs * T.rows * LORA_MAX_R);
  m.group = T.group + e * T.group_stride;
  return m;
}

// Descriptor of a launch-wide index x: the number of descriptors after the first whose
// first index (field F, increasing with the descriptor) is at most x.  All of them are
// compared at once, so the kernel-argument reads are independent (no chain of dependent
// scalar loads, as a search loop would make).
template <int32_t LoraTensor::*F>
__device__ __forceinline__ int lora_desc_of(const LoraArgs& a, int64_t x) {
  int di = 0;
#pragma unroll
  for (int i = 1; i < QF_MAX_GROUPED; ++i) di += (i < a.n && x >= (int64_t)(a.d[i].*F)) ? 1 : 0;
  return di;
}

// --------------------------------------------------- merge, passes 1 and 2 ------
// The low-rank product S = B.A runs on the fp32 matrix cores: v_mfma_f32_32x32x1_2b_f32
// multiplies one fp32 value per lane of its A operand by one of its B operand (K = 1) and
// adds the product to the accumulator with one fp32 rounding, ties to even, subnormals
// kept -- the same operation as fma(b, a, acc), since every bf16 x bf16 product is exact
// in fp32.  A chain of r such steps, k = 0 .. r-1, is therefore bit for bit the merge's
// sequential sum.  (The BF16 K = 16 instruction is not: its 16-product sums round
// differently.)
//
// Tile = 32 rows x 64 columns of one matrix.  The instruction works on two 32 x 32 blocks.
// MFMA columns are the tile's 32 rows (B operand: lane l supplies B[row l % 32][k] for
// block l / 32); MFMA rows are 32 of the 64 columns per block (A operand: lane l supplies
// A[k][col(l)]).  Lane l then holds, in its 32 accumulators, block q's result for tile row
// l % 32 at MFMA rows 8 (w / 4) + 4 h + w % 4 (w = 0..15, h = l / 32).  col() maps MFMA
// row 8 (w / 4) + 4 h + w % 4 of block q to tile column 32 q + 16 h + w, so each lane ends
// with two whole NVFP4 16-blocks of one row: columns 16 h .. 16 h + 15 and
// 32 + 16 h .. 32 + 16 h + 15.  The block maximum, scale and codes stay in the lane.
//
// Work split: the launch's tiles in one flat order are cut into equal contiguous runs, one
// per wave of a grid that stays resident on the chip, so every wave streams the same
// number of tiles (give or take one).  The order is descriptor, band of merge_band row
// tiles (the run length), 64-column tile, 32-row tile: a run goes down one column of a
// band, with A's values for that column in registers (reloaded where the run enters the
// next column or matrix), and the waves running side by side read the same rows of
// neighbouring columns, so each row of W is read whole at about the same time.
//
// Loads: each wave streams its tiles through its own ring of MM_DEPTH LDS stages with
// buffer loads that write LDS directly (no registers held while in flight), MM_DEPTH - 1
// tiles ahead, across column and matrix boundaries.  A stage holds the W tile (32 rows x
// 128 bytes, loaded as four fully coalesced 1 KiB windows; the 16-byte chunks of row r
// are stored XOR-rotated by (r >> 1) & 7 so that the lanes' row reads hit distinct banks)
// and the tile's 32 rows of B (contiguous in memory).  Columns past the matrix's last
// 32-column group and rows past the matrix read zeros; their stores are dropped, and
// rows past the matrix are left out of the maximum.
constexpr int MM_COLS = LORA_MERGE_COLS;
constexpr int MM_ROWS = LORA_MERGE_ROWS;
constexpr int MM_DEPTH = 2;                      // ring stages per wave
constexpr int MM_WBYTES = MM_ROWS * MM_COLS * 2; // 4 KiB of W per tile
constexpr int MM_STAGE = MM_WBYTES + 1024;       // + B rows (32 x up to 16 bf16)
constexpr int MM_LOADS = 4 + 4;                  // buffer-to-LDS loads per tile per lane

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(n) with the LDS and export counters left at their maximum
#define MM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

typedef float f32x32_t __attribute__((ext_vector_type(32)));

__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (int)off, 0, 0);
}

// A tile's place in the flat order (wave-uniform): descriptor, row tile, column tile, the
// row band [b0, b1) of the row tile, and the descriptor's row and column tile counts.
struct MmTile {
  int di, e, ct, rt, b0, b1, rtiles, ctiles;
};

__device__ __forceinline__ void mm_next(const LoraArgs& a, MmTile& p) {
  if (++p.rt < p.b1) return;
  if (++p.ct == p.ctiles) {
    p.ct = 0;
    if (p.b1 == p.rtiles) {                                      // next expert or descriptor, first band
      if (++p.e >= a.d[p.di].count) {
        p.e = 0;
        if (++p.di >= a.n) return;
        p.rtiles = a.d[p.di].merge_rtiles;
        p.ctiles = a.d[p.di].merge_ctiles;
      }
      p.b0 = 0;
      p.b1 = min(a.merge_band, p.rtiles);
    } else {
      p.b0 = p.b1;
      p.b1 = min(p.b1 + a.merge_band, p.rtiles);
    }
  }
  p.rt = p.b0;
}

// Place of tile tb of the launch.
__device__ __forceinline__ MmTile mm_locate(const LoraArgs& a, int64_t tb) {
  MmTile p;
  const int di = lora_desc_of<&LoraTensor::merge_tile_begin>(a, tb);
  const LoraTensor& T = a.d[di];
  p.rtiles = T.merge_rtiles;
  p.ctiles = T.merge_ctiles;
  int loc = (int)(tb - T.merge_tile_begin);
  p.e = loc / (p.rtiles * p.ctiles);
  loc -= p.e * p.rtiles * p.ctiles;
  const int bands = (p.rtiles + a.merge_band - 1) / a.merge_band;
  const int band = min(loc / (a.merge_band * p.ctiles), bands - 1);
  p.di = di;
  p.b0 = band * a.merge_band;
  p.b1 = min(p.b0 + a.merge_band, p.rtiles);
  const int q = loc - p.b0 * p.ctiles, hb = p.b1 - p.b0;
  p.ct = q / hb;
  p.rt = p.b0 + (q - p.ct * hb);
  return p;
}

// Folds a lane maximum into the workgroup's maximum of group g (LDS).
__device__ __forceinline__ void mm_flush(uint32_t m, uint32_t* gmax, int g) {
  m = umax(m, dpp_xor1(m));
  m = umax(m, dpp_xor2(m));
  m = umax(m, dpp_hmirror(m));
  m = umax(m, dpp_mirror(m));
  m = umax(m, swz_xor16(m));
  m = umax((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 32));
  if ((threadIdx.x & 63) == 0) atomicMax(gmax + g, m);
}

template <int RK, bool STORE_M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_lora_merge_amax(LoraArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t mm_lds[4 * MM_DEPTH * MM_STAGE];
  __shared__ uint32_t gmax[QF_MAX_GROUPS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if ((int)threadIdx.x < QF_MAX_GROUPS) gmax[threadIdx.x] = 0;
  __syncthreads();
  // this wave's run of tiles [tb, tb + nt)
  const int64_t nw = (int64_t)gridDim.x * 4, w = (int64_t)blockIdx.x * 4 + wave;
  const int64_t tb = w * a.merge_tiles / nw;
  const int nt = (int)((w + 1) * a.merge_tiles / nw - tb);
  uint32_t m = 0;                                                  // max |M| bits of group mg
  int mg = -1;
  if (nt > 0) {
    const int h = lane >> 5, lr = lane & 31;
    uint8_t* const ring = mm_lds + wave * (MM_DEPTH * MM_STAGE);
    MmTile pe = mm_locate(a, tb);      // the tile computed next
    MmTile pl = pe;                    // the tile loaded next
    // W window j of a tile: lane i fills row 8j + i/8 at chunk position i%8 with the row's
    // global chunk (i%8) ^ ((row >> 1) & 7)
    uint32_t wrow[4], wchunk[4];
#pragma unroll
    for (int jw = 0; jw < 4; ++jw) {
      wrow[jw] = 8u * jw + (uint32_t)(lane >> 3);
      wchunk[jw] = (uint32_t)(lane & 7) ^ ((wrow[jw] >> 1) & 7u);
    }
    // Loads of the wave's j-th tile into stage st: always MM_LOADS instructions (past the
    // run they read nothing and write zeros), so that the waits below count right.
    auto issue = [&](int j, uint8_t* st) {
      __amdgpu_buffer_rsrc_t rw = make_buf(nullptr, 0), rb = make_buf(nullptr, 0);
      uint32_t wo[4] = {BUF_OOR, BUF_OOR, BUF_OOR, BUF_OOR}, bo[4] = {BUF_OOR, BUF_OOR, BUF_OOR, BUF_OOR};
      if (j < nt) {
        const LoraTensor& T = a.d[pl.di];
        const LoraMat X = lora_mat(T, pl.e, a.da_rows);
        const int r = RK ? RK : T.r;
        const int64_t c0 = (int64_t)pl.ct * MM_COLS, r0 = (int64_t)pl.rt * MM_ROWS;
        const int nrows = (int)min((int64_t)MM_ROWS, T.rows - r0);
        const int cw = (int)min((int64_t)MM_COLS, T.cols - c0);
        rw = make_buf(X.W + r0 * T.ldw + c0, ((int64_t)(nrows - 1) * T.ldw + cw) * 2);
        // B rows of the tile (4-byte aligned; with an odd rank the last row may end in the
        // middle of a word, so the 2 bytes after it are in range)
        rb = make_buf(X.B + r0 * r, (int64_t)nrows * r * 2 + 2);
#pragma unroll
        for (int jw = 0; jw < 4; ++jw)
          wo[jw] = cw > 32 * (int)(wchunk[jw] >> 2) ? (uint32_t)((wrow[jw] * T.ldw + 8 * wchunk[jw]) * 2) : BUF_OOR;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const int d = 64 * jb + lane;                              // dword of the tile's B bytes
          bo[jb] = d < 16 * r ? (uint32_t)(4 * d) : BUF_OOR;
        }
        mm_next(a, pl);
      }
#pragma unroll
      for (int jw = 0; jw < 4; ++jw)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(st + 1024 * jw), 16, wo[jw], 0, 0, 0);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(st + MM_WBYTES + 256 * jb), 4, bo[jb], 0, 0, 0);
    };
    // stores per tile (counted by vmcnt like the loads): 4 (M; dropped for a null M), or none
    // when no descriptor of the launch keeps M
    constexpr int STORES = STORE_M ? 4 : 0;
    const uint32_t rot = ((uint32_t)lr >> 1) & 7u;
    // The chain always takes LORA_MAX_R steps: a rank r < 16 runs 16 - r leading steps on
    // +0 x +0, which leave the accumulator at +0 exactly, so the sum is still the r-step one.
    // A operand of step j: A[j - (16 - r)][c0 + colA], colA = this lane's MFMA row's column.
    const int colA = 32 * h + 16 * ((lr >> 2) & 1) + 4 * (lr >> 3) + (lr & 3);
    float av[LORA_MAX_R];
    int a_di = -1, a_e = -1, a_ct = -1;
    // A's values for the column of tile p; then no load is left pending, so no later wait
    // has to cover them
    auto load_a = [&](const MmTile& p) {
      const LoraTensor& T = a.d[p.di];
      const int r = RK ? RK : T.r, lead = LORA_MAX_R - r;
      const __amdgpu_buffer_rsrc_t ra = make_buf(lora_mat(T, p.e, a.da_rows).A, (int64_t)r * T.cols * 2);
      const int cA = p.ct * MM_COLS + colA, ncol = (int)T.cols;     // below 2^16 + 64
#pragma unroll
      for (int j = 0; j < LORA_MAX_R; ++j) {
        const uint32_t off = (j >= lead && cA < ncol) ? (uint32_t)(((j - lead) * ncol + cA) * 2) : BUF_OOR;
        av[j] = __uint_as_float((uint32_t)buf_load2(ra, off) << 16);
      }
      MM_WAIT_VM(0);
      a_di = p.di;
      a_e = p.e;
      a_ct = p.ct;
    };
    // The tile's LDS reads (stage st, rank r) in one block that waits for its own results:
    // written as plain loads, the compiler cannot tell the ring stages' buffer-to-LDS writes
    // apart and would wait for the next tiles' loads too (the caller's wait covers this
    // tile's).  wc: the lane's W chunks, global chunks 2h, 2h+1 (group 0), 4+2h, 5+2h
    // (group 1); bk[j]: B[lr][j - (16 - r)], 0 for the leading steps.
    auto read_tile = [&](const uint8_t* st, int r, uint4 (&wc)[4], float (&bk)[LORA_MAX_R]) {
      uint32_t wa[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t g = (uint32_t)(2 * h + (c & 1) + 4 * (c >> 1));
        wa[c] = lds_addr(st + lr * 128 + ((g ^ rot) << 4));
      }
      u32x4_t w0, w1, w2, w3;
      if constexpr (RK == LORA_MAX_R) {
        const uint32_t ba = lds_addr(st + MM_WBYTES + lr * 32);
        u32x4_t b0v, b1v;
        asm volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %7\n\t"
            "ds_read_b128 %2, %8\n\t"
            "ds_read_b128 %3, %9\n\t"
            "ds_read_b128 %4, %10\n\t"
            "ds_read_b128 %5, %10 offset:16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(b0v), "=&v"(b1v)
            : "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "v"(ba)
            : "memory");
        const uint32_t bwv[8] = {b0v[0], b0v[1], b0v[2], b0v[3], b1v[0], b1v[1], b1v[2], b1v[3]};
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          bk[2 * q2] = bf16_lo(bwv[q2]);
          bk[2 * q2 + 1] = bf16_hi(bwv[q2]);
        }
      } else {
        // halfword j at B-row start + 2 (j - lead): from the W area's end (lead <= 15
        // halfwords before row 0) to the B area's (31 r + r halfwords); k < 0 dropped
        const int lead = LORA_MAX_R - r;
        const uint32_t ba = lds_addr(st + MM_WBYTES + (lr * r - lead) * 2);
        uint32_t bh[LORA_MAX_R];
        asm volatile(
            "ds_read_b128 %0, %20\n\t"
            "ds_read_b128 %1, %21\n\t"
            "ds_read_b128 %2, %22\n\t"
            "ds_read_b128 %3, %23\n\t"
            "ds_read_u16 %4, %24\n\t"
            "ds_read_u16 %5, %24 offset:2\n\t"
            "ds_read_u16 %6, %24 offset:4\n\t"
            "ds_read_u16 %7, %24 offset:6\n\t"
            "ds_read_u16 %8, %24 offset:8\n\t"
            "ds_read_u16 %9, %24 offset:10\n\t"
            "ds_read_u16 %10, %24 offset:12\n\t"
            "ds_read_u16 %11, %24 offset:14\n\t"
            "ds_read_u16 %12, %24 offset:16\n\t"
            "ds_read_u16 %13, %24 offset:18\n\t"
            "ds_read_u16 %14, %24 offset:20\n\t"
            "ds_read_u16 %15, %24 offset:22\n\t"
            "ds_read_u16 %16, %24 offset:24\n\t"
            "ds_read_u16 %17, %24 offset:26\n\t"
            "ds_read_u16 %18, %24 offset:28\n\t"
            "ds_read_u16 %19, %24 offset:30\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(bh[0]), "=&v"(bh[1]), "=&v"(bh[2]),
              "=&v"(bh[3]), "=&v"(bh[4]), "=&v"(bh[5]), "=&v"(bh[6]), "=&v"(bh[7]), "=&v"(bh[8]), "=&v"(bh[9]),
              "=&v"(bh[10]), "=&v"(bh[11]), "=&v"(bh[12]), "=&v"(bh[13]), "=&v"(bh[14]), "=&v"(bh[15])
            : "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "v"(ba)
            : "memory");
#pragma unroll
        for (int j = 0; j < LORA_MAX_R; ++j) bk[j] = j >= lead ? __uint_as_float((bh[j] & 0xFFFFu) << 16) : 0.0f;
      }
      wc[0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
      wc[1] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      wc[2] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
      wc[3] = make_uint4(w3[0], w3[1], w3[2], w3[3]);
    };
    auto chain = [&](const float (&bk)[LORA_MAX_R]) {
      f32x32_t acc;
#pragma unroll
      for (int v = 0; v < 32; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int j = 0; j < LORA_MAX_R; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(av[j], bk[j], acc, 0, 0, 0);
      return acc;
    };
    // Step t: tile t + 1 is loaded into the stage of tile t - 1 (read one step earlier),
    // tile t is read from its stage, multiplied on the matrix cores and finished.
    static_assert(MM_DEPTH == 2, "one tile loaded ahead");
    auto step = [&](int t, int si) {
      LORA_FENCE();
      issue(t + 1, ring + (si ^ 1) * MM_STAGE);
      LORA_FENCE();
      // wait for tile t's loads: younger than them are the next tile's loads and tile
      // t - 1's stores (none before tile 0; A reloads drain everything)
      if (t >= 1) MM_WAIT_VM(MM_LOADS + STORES);
      else MM_WAIT_VM(MM_LOADS);
      asm volatile("" ::: "memory");
      if (pe.di != a_di || pe.e != a_e || pe.ct != a_ct) load_a(pe);
      const LoraTensor& T = a.d[pe.di];
      const LoraMat X = lora_mat(T, pe.e, a.da_rows);
      const int r = RK ? RK : T.r;
      const int64_t cols = T.cols, c0 = (int64_t)pe.ct * MM_COLS, r0 = (int64_t)pe.rt * MM_ROWS;
      const int nrows = (int)min((int64_t)MM_ROWS, T.rows - r0);
      uint8_t* const st = ring + si * MM_STAGE;
      uint4 wc[4];
      float bk[LORA_MAX_R];
      read_tile(st, r, wc, bk);
      const f32x32_t acc = chain(bk);
      // M = bf16(fl(W + S)) for the lane's 32 elements: chunk c holds columns 8c .. 8c+7 of
      // the lane's groups (c = 0, 1: group 0; c = 2, 3: group 1)
      uint4 mo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float wf[8];
        unpack8(wc[c], wf);
        const int v0 = 16 * (c >> 1) + 8 * (c & 1);
        mo[c].x = pack_bf16x2(wf[0] + acc[v0 + 0], wf[1] + acc[v0 + 1]);
        mo[c].y = pack_bf16x2(wf[2] + acc[v0 + 2], wf[3] + acc[v0 + 3]);
        mo[c].z = pack_bf16x2(wf[4] + acc[v0 + 4], wf[5] + acc[v0 + 5]);
        mo[c].w = pack_bf16x2(wf[6] + acc[v0 + 6], wf[7] + acc[v0 + 7]);
      }
      const uint32_t mt = umax(umax(amax_bits8(mo[0]), amax_bits8(mo[1])), umax(amax_bits8(mo[2]), amax_bits8(mo[3])));
      if constexpr (STORE_M) {
        // M leaves through the stage just read (free until the next step loads into it):
        // the lanes write their pieces of rows where the W chunks were and read whole rows
        // back (window k: row 8k + lane / 8, global chunk wchunk[k] at position lane % 8),
        // so that a store instruction writes 8 rows of 128 bytes instead of 16-byte pieces
        // of 32 rows
        const bool ok1 = c0 + 32 < cols;                           // the second 32-column group
        uint32_t xa[4], yoff[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t g = (uint32_t)(2 * h + (c & 1) + 4 * (c >> 1));
          xa[c] = lds_addr(st + lr * 128 + ((g ^ rot) << 4));
          yoff[c] = ok1 || wchunk[c] < 4 ? (uint32_t)((wrow[c] * cols + 8 * wchunk[c]) * 2) : BUF_OOR;
        }
        const uint32_t xr = lds_addr(st + 16 * lane);
        u32x4_t mo0, mo1, mo2, mo3;
        const u32x4_t m0 = {mo[0].x, mo[0].y, mo[0].z, mo[0].w}, m1 = {mo[1].x, mo[1].y, mo[1].z, mo[1].w};
        const u32x4_t m2 = {mo[2].x, mo[2].y, mo[2].z, mo[2].w}, m3 = {mo[3].x, mo[3].y, mo[3].z, mo[3].w};
        asm volatile(
            "ds_write_b128 %[a0], %[m0]\n\t"
            "ds_write_b128 %[a1], %[m1]\n\t"
            "ds_write_b128 %[a2], %[m2]\n\t"
            "ds_write_b128 %[a3], %[m3]\n\t"
            "ds_read_b128 %[o0], %[xr]\n\t"
            "ds_read_b128 %[o1], %[xr] offset:1024\n\t"
            "ds_read_b128 %[o2], %[xr] offset:2048\n\t"
            "ds_read_b128 %[o3], %[xr] offset:3072\n\t"
            "s_waitcnt lgkmcnt(0)"
            : [o0] "=&v"(mo0), [o1] "=&v"(mo1), [o2] "=&v"(mo2), [o3] "=&v"(mo3)
            : [a0] "v"(xa[0]), [a1] "v"(xa[1]), [a2] "v"(xa[2]), [a3] "v"(xa[3]), [m0] "v"(m0), [m1] "v"(m1),
              [m2] "v"(m2), [m3] "v"(m3), [xr] "v"(xr)
            : "memory");
        // rows past the matrix fall outside the range
        const int64_t e0 = r0 * cols + c0, ne = (int64_t)nrows * cols - c0;
        const __amdgpu_buffer_rsrc_t rm = make_buf((const uint16_t*)((uintptr_t)X.M + (uintptr_t)(e0 * 2)),
                                                   X.M ? ne * 2 : 0);
        buf_store16(rm, yoff[0], make_uint4(mo0[0], mo0[1], mo0[2], mo0[3]));
        buf_store16(rm, yoff[1], make_uint4(mo1[0], mo1[1], mo1[2], mo1[3]));
        buf_store16(rm, yoff[2], make_uint4(mo2[0], mo2[1], mo2[2], mo2[3]));
        buf_store16(rm, yoff[3], make_uint4(mo3[0], mo3[1], mo3[2], mo3[3]));
      }
      if (X.group != mg) {                                         // the run enters another group
        if (mg >= 0) mm_flush(m, gmax, mg);
        m = 0;
        mg = X.group;
      }
      m = umax(m, lr < nrows ? mt : 0u);                           // rows past the matrix: left out
      if (t + 1 < nt) mm_next(a, pe);
      LORA_FENCE();
    };
    // prologue: A for tile 0's column, tile 0 in flight
    load_a(pe);
    issue(0, ring);
#pragma unroll 1
    for (int t = 0; t < nt; t += 2) {
      step(t, 0);
      if (t + 1 < nt) step(t + 1, 1);
    }
    MM_WAIT_VM(0);                                                 // no load may still write LDS at exit
    mm_flush(m, gmax, mg);
  }
  // workgroup maxima -> partial[g * grid + b] for every group (0 where none was seen)
  __syncthreads();
  if ((int)threadIdx.x < a.n_groups) a.partial[threadIdx.x * gridDim.x + blockIdx.x] = gmax[threadIdx.x];
}

// ------------------------------------------------ pass 2 without M in memory ---
// Merge again and NVFP4-QDQ + pack in registers.  A unit is one wave's share: LORA_SLAB
// = 512 columns of a run of merge_rows rows (lane l owns columns 8l .. 8l+7 of the slab,
// lanes 2i and 2i+1 one 16-block), walked one row at a time with LORA_PREFETCH rows of W
// in flight.  Lanes keep their 16 x 8 slice of A in registers, so a row costs one 16-byte
// load, 128 FMAs, the QDQ of 8 values and row-contiguous stores; the row's B values are
// the same for every lane and come through the scalar cache.  The sum is the same
// sequential fp32 one as on the matrix cores in pass 1, so M has the same bits.  (This
// layout keeps every load and store a whole contiguous row piece, which the QDQ outputs
// need; pass 1 stores nothing when M is not kept.)
constexpr int LORA_PREFETCH = 4;
constexpr int BW = LORA_MAX_R / 2 + 1;   // 32-bit words that can hold one row of B
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

__device__ __forceinline__ int find_desc_wg(const LoraArgs& a, int b) {
  return lora_desc_of<&LoraTensor::merge_wg_begin>(a, b);
}

// Workgroup b of the merge-and-QDQ layout: its descriptor, expert, and the unit of wave
// `wave` (u >= merge_units: padding past the expert's last unit).
struct LoraUnit {
  int di, e, u;
};
__device__ __forceinline__ LoraUnit lora_unit(const LoraArgs& a, int b, int wave) {
  LoraUnit q;
  q.di = find_desc_wg(a, b);
  const LoraTensor& T = a.d[q.di];
  const int wpe = (T.merge_units + 3) / 4;                           // workgroups per expert
  const int lb = b - T.merge_wg_begin;
  q.e = lb / wpe;
  q.u = (lb - q.e * wpe) * 4 + wave;
  return q;
}

// Scalar words of B's row `row` (B contiguous [rows, r], 4-byte aligned; the row starts
// at element row * r, which may be odd; with r odd the last row's last word may hold the
// 2 bytes after B).  RK is the rank when known at compile time (16: 8 aligned words).
template <int RK>
__device__ __forceinline__ void fetch_b_words(const uint16_t* B, int64_t row, int r, uint32_t (&w)[BW]) {
  if constexpr (RK == LORA_MAX_R) {
    const const_u32_ptr bw = (const_u32_ptr)(reinterpret_cast<const uint32_t*>(B) + row * (RK / 2));
#pragma unroll
    for (int q = 0; q < RK / 2; ++q) w[q] = bw[q];
    w[BW - 1] = 0u;
  } else {
    const int64_t e0 = row * r;
    const const_u32_ptr bw = (const_u32_ptr)(reinterpret_cast<const uint32_t*>(B) + (e0 >> 1));
    const int nw = ((int)(e0 & 1) + r + 1) >> 1;
#pragma unroll
    for (int q = 0; q < BW; ++q) w[q] = q < nw ? bw[q] : 0u;
  }
}

// B values of the row as fp32, zero past r: the padded steps fma(+0, +0, acc) come after
// the r real ones and leave acc unchanged bit for bit.  (Adding +0 changes only acc = -0,
// and a sum that starts at +0 reaches -0 only through a product below fp32's range.)
template <int RK>
__device__ __forceinline__ void b_row_values(const uint32_t (&w)[BW], int64_t row, int r, float (&bk)[LORA_MAX_R]) {
  if constexpr (RK == LORA_MAX_R) {
#pragma unroll
    for (int q = 0; q < RK / 2; ++q) {
      bk[2 * q] = bf16_lo(w[q]);
      bk[2 * q + 1] = bf16_hi(w[q]);
    }
  } else {
    const uint32_t odd = (uint32_t)((row * r) & 1);
#pragma unroll
    for (int q = 0; q < LORA_MAX_R / 2; ++q) {
      const uint32_t v = odd ? ((w[q] >> 16) | (w[q + 1] << 16)) : w[q];
      bk[2 * q] = 2 * q < r ? bf16_lo(v) : 0.0f;
      bk[2 * q + 1] = 2 * q + 1 < r ? bf16_hi(v) : 0.0f;
    }
  }
}

// Loop bodies are branch-free: W and A are read through buffer resources that span
// exactly the valid rows (and A's r rows), lanes past the last column use an
// out-of-range offset, and the rows of the last group past the end are computed on zeros
// and dropped by the range check, so the compiler keeps every prefetched load in flight.
template <int RK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_lora_merge_qdq(LoraArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const LoraUnit uq = lora_unit(a, blockIdx.x, wave);
  const LoraTensor& T = a.d[uq.di];
  const int u = uq.u;
  if (u >= T.merge_units) return;
  const LoraMat X = lora_mat(T, uq.e, a.da_rows);
  const int64_t cols = T.cols, ldw = T.ldw;
  const int r = RK ? RK : T.r;
  const int rb = u / T.slabs;
  const int64_t cs = (int64_t)(u - rb * T.slabs) * LORA_SLAB;        // first column of the slab
  const int64_t r0 = (int64_t)rb * a.merge_rows;
  const int rows = (int)min((int64_t)a.merge_rows, T.rows - r0);
  const bool active = cs + 8 * lane < cols;
  const uint32_t lo = active ? 16u * lane : BUF_OOR;                  // lane's byte offset in a row
  const int64_t e0 = r0 * cols + cs;                                  // first element of the unit
  const __amdgpu_buffer_rsrc_t rw = make_buf(X.W + r0 * ldw + cs, (int64_t)rows * ldw * 2);
  const __amdgpu_buffer_rsrc_t ra = make_buf(X.A + cs, (int64_t)r * cols * 2 - cs * 2);
  const uint32_t wstride = (uint32_t)(ldw * 2), mstride = (uint32_t)(cols * 2);
  // outputs (an empty resource drops the stores)
  const bool wy = X.y, wp = X.codes;
  const __amdgpu_buffer_rsrc_t ry = make_buf(wy ? X.y + e0 : nullptr, wy ? (int64_t)rows * cols * 2 : 0);
  const __amdgpu_buffer_rsrc_t rc = make_buf(wp ? X.codes + e0 / 2 : nullptr, wp ? (int64_t)rows * cols / 2 : 0);
  const __amdgpu_buffer_rsrc_t rs = make_buf(wp ? X.scales + e0 / 16 : nullptr, wp ? (int64_t)rows * cols / 16 : 0);
  const uint32_t clo = active ? 4u * lane : BUF_OOR;
  const uint32_t slo = active && (lane & 1) == 0 ? (uint32_t)lane / 2u : BUF_OOR;
  const uint32_t cstride = (uint32_t)(cols / 2), sstride = (uint32_t)(cols / 16);
  const float s_t = a.tscale[X.group], k6 = 6.0f * s_t;
  uint4 wv[LORA_PREFETCH];
#pragma unroll
  for (int q = 0; q < LORA_PREFETCH; ++q) {
    wv[q] = buf_load16_nt(rw, lo + q * wstride);
    LORA_FENCE();
  }
  uint32_t bw[BW];
  // B's rows are addressed from expert 0's (4-byte aligned) base: expert e's rows follow
  // as rows e * rows + i, which keeps the word alignment right when rows * r is odd
  const int64_t br0 = (int64_t)uq.e * T.rows + r0;
  fetch_b_words<RK>(T.B, br0, r, bw);
  float av[LORA_MAX_R][8];                                           // rows k >= r read as 0
#pragma unroll
  for (int k = 0; k < LORA_MAX_R; ++k) unpack8(buf_load16(ra, lo + k * mstride), av[k]);
  const bool odd = lane & 1;
#pragma unroll 1
  for (int i = 0; i < rows; i += LORA_PREFETCH) {
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; q += 2) {
      uint4 o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        LORA_FENCE();
        const int ii = i + q + h;                                    // may pass the last row
        float bk[LORA_MAX_R];
        b_row_values<RK>(bw, br0 + min(ii, rows - 1), r, bk);
        fetch_b_words<RK>(T.B, br0 + min(ii + 1, rows - 1), r, bw);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(bk[k], av[k][e], acc[e]);
        float w[8];
        unpack8(wv[q + h], w);
        o[h].x = pack_bf16x2(w[0] + acc[0], w[1] + acc[1]);
        o[h].y = pack_bf16x2(w[2] + acc[2], w[3] + acc[3]);
        o[h].z = pack_bf16x2(w[4] + acc[4], w[5] + acc[5]);
        o[h].w = pack_bf16x2(w[6] + acc[6], w[7] + acc[7]);
      }
      // Block scales of the two rows: lanes 2j and 2j + 1 hold the two halves of one
      // 16-block in each row, so the even lane works out row q's scale, the odd lane row
      // q + 1's, and each takes the other row's from its neighbour (one scale computation
      // per lane for two rows instead of one per row, the same arithmetic).
      uint32_t m0 = amax_bits8(o[0]);
      m0 = umax(m0, dpp_xor1(m0));
      uint32_t m1 = amax_bits8(o[1]);
      m1 = umax(m1, dpp_xor1(m1));
      const Nvfp4Scale mine = nvfp4_block_scale(odd ? m1 : m0, s_t, k6);
      const uint32_t oS = dpp_xor1(mine.S);
      const float os = __uint_as_float(dpp_xor1(__float_as_uint(mine.s)));
      const float orr = __uint_as_float(dpp_xor1(__float_as_uint(mine.r)));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ii = i + q + h;
        const bool own = odd == (h == 1);                            // this lane computed row h's scale
        const uint32_t S = own ? mine.S : oS;
        const Nvfp4Enc e = nvfp4_encode_chunk(o[h], own ? mine.s : os, s_t, own ? mine.r : orr);
        buf_store16(ry, lo + ii * mstride, e.y);                     // rows past the end: dropped
        buf_store4(rc, clo + ii * cstride, e.codes);
        buf_store1(rs, slo + ii * sstride, (uint8_t)S);
        wv[q + h] = buf_load16_nt(rw, lo + (ii + LORA_PREFETCH) * wstride);   // past the end: zeros
      }
    }
  }
}

// dA[k][j] (+)= sum over row blocks, in block order; dB[i][k] (+)= sum over slabs, in slab
// order.  The partial loads are issued LORA_RED_BATCH at a time before any add, so an
// entry costs a few memory latencies instead of one per partial; the order of the adds
// is unchanged.
constexpr int LORA_RED_BATCH = 8;

// Matrix m of the launch (blockIdx.y of the reduces): its descriptor.
__device__ __forceinline__ int find_desc_mat(const LoraArgs& a, int m) {
  return lora_desc_of<&LoraTensor::mat_begin>(a, m);
}

// Adapter gradients from the partials of k_lora_grads, one thread per gradient entry:
// dB[i][k] (+)= the slab partials and dA[k][j] (+)= the row-block partials, each added in
// index order.  One launch for both: blocks [0, gB) of x walk dB, the others dA (each part
// grid-strides over its own blocks); y is the matrix.
// Sums of four adjacent entries: count partials p[0], p[stride], ... of each, loaded 16
// bytes at a time (the partial buffers are 16-byte aligned: the workspace is, and every
// offset into it is a multiple of 16 floats) and added per entry in index order from +0.
__device__ __forceinline__ float4 sum_partials4(const float* p, int64_t stride, int count) {
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 1
  for (int q0 = 0; q0 < count; q0 += LORA_RED_BATCH) {
    float4 v[LORA_RED_BATCH];
#pragma unroll
    for (int i = 0; i < LORA_RED_BATCH; ++i)
      v[i] = q0 + i < count ? *reinterpret_cast<const float4*>(p + (int64_t)(q0 + i) * stride)
                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < LORA_RED_BATCH; ++i)
      if (q0 + i < count) {
        s.x += v[i].x;
        s.y += v[i].y;
        s.z += v[i].z;
        s.w += v[i].w;
      }
  }
  return s;
}

__global__ __launch_bounds__(256) void k_lora_grad_reduce(LoraArgs a, int accumulate, int gB) {
  const LoraTensor& T = a.d[find_desc_mat(a, blockIdx.y)];
  const LoraMat X = lora_mat(T, (int)blockIdx.y - T.mat_begin, a.da_rows);
  if ((int)blockIdx.x < gB) {
    const int64_t n = T.rows * LORA_MAX_R;
    for (int64_t idx = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x); idx < n;
         idx += (int64_t)4 * gB * blockDim.x) {
      // partial q holds LORA_MAX_R adapters of every row; entry (i, k) of dB is at idx
      const int64_t row = idx / LORA_MAX_R;
      const int k = (int)(idx - row * LORA_MAX_R);                   // a multiple of 4
      if (k >= T.r) continue;
      float* dst = X.dB + row * T.r + k;
      const float4 s4 = sum_partials4(X.dB_partial + idx, T.rows * LORA_MAX_R, T.slabs);
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};                 // entries k + e >= r: unused
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k + e < T.r) dst[e] = accumulate ? dst[e] + sv[e] : sv[e];
    }
    return;
  }
  const int gA = (int)gridDim.x - gB;
  const int64_t n = (int64_t)T.r * T.cols;
  const int nblk = (int)((T.rows + a.da_rows - 1) / a.da_rows);
  for (int64_t idx = 4 * ((int64_t)(blockIdx.x - gB) * blockDim.x + threadIdx.x); idx < n;
       idx += (int64_t)4 * gA * blockDim.x) {
    // partial q holds rows k = 0 .. 15 of cols columns; entry (k, j) of dA is at idx
    // (cols is a multiple of 32, so four adjacent entries share k)
    const float4 s4 = sum_partials4(X.dA_partial + idx, (int64_t)LORA_MAX_R * T.cols, nblk);
    const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) X.dA[idx + e] = accumulate ? X.dA[idx + e] + sv[e] : sv[e];
  }
}

// ------------------------------------------- pass 1 without M: bounded merge ---
// max|M| of a tied group needs M exactly only where an element could reach the running
// maximum L, and a cheap bound says where.  For element (i, j) the computed sum obeys
// |S_ij| <= U_i,l = fl(bsum_i * a_l) + 2^-100, with bsum_i = sum_k |B[i][k]| (row i) and a_l
// = 1.001 max |A| over the 16 x 8 slice of the lane: the relative slack (1e-3) covers the
// sum's 16 roundings and those of bsum and the product many times over, the absolute one
// products and sums below fp32's normal range.  Rounding is monotone, so
// |M_ij| = |bf16(fl(W_ij + S_ij))| <= bf16(fl(|W_ij| + U)), and with t = fl(max|W| + U)
// over the lane's 8 elements, t <= prev(L) (the bf16 value below L) proves that none of them
// exceeds L.  The lane's row is merged exactly (the same sequential fp32 sum as everywhere
// else) only when some lane of the wave fails that test; a NaN or an infinity anywhere in
// W, A or B makes t fail it, and a NaN L makes every test fail.  L only ever holds exactly
// merged values of the group, so the group's maximum (bit pattern included) is the one a
// full merge finds.
//
// Work split: the units of the merge-and-QDQ pass (a 512-column slab of merge_rows rows,
// lane l on columns 8l .. 8l+7), four per workgroup of that pass, taken here slab by slab
// within each expert (so that consecutive units share A's slice), cut into equal contiguous
// runs, one per wave of a grid that stays resident; the running maximum is kept per wave
// across the units of one group, and shared through the workgroup's LDS maximum.
constexpr int LORA_P1_PREFETCH = 8;                    // rows of W in flight per wave

template <int RK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_lora_merge_amax_bounded(LoraArgs a) {
  __shared__ uint32_t gmax[QF_MAX_GROUPS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if ((int)threadIdx.x < QF_MAX_GROUPS) gmax[threadIdx.x] = 0;
  __syncthreads();
  const int64_t units = 4 * (int64_t)a.qdq_wg;
  const int64_t nw = (int64_t)gridDim.x * 4, w = (int64_t)blockIdx.x * 4 + wave;
  const int64_t u0 = w * units / nw, u1 = (w + 1) * units / nw;
  uint32_t L = 0;                                                    // wave-uniform, group mg
  int mg = -1;
  uint4 ap[LORA_MAX_R];                                              // A's slice, bf16 (rows k >= r: 0)
  float a_l = 0.0f;
  int a_di = -1, a_e = -1, a_slab = -1;
#pragma unroll 1
  for (int64_t uf = u0; uf < u1; ++uf) {
    const LoraUnit uq = lora_unit(a, (int)(uf >> 2), (int)(uf & 3));
    const LoraTensor& T = a.d[uq.di];
    const int ul = uq.u;
    if (ul >= T.merge_units) continue;                               // padding of the expert's last workgroup
    const LoraMat X = lora_mat(T, uq.e, a.da_rows);
    if (X.group != mg) {
      if (mg >= 0 && lane == 0) atomicMax(gmax + mg, L);
      L = 0;
      mg = X.group;
    }
    const int64_t cols = T.cols, ldw = T.ldw;
    const int r = RK ? RK : T.r;
    // units slab by slab (all row blocks of a slab in turn), so that a run of units keeps
    // the slab's A in registers
    const int rblocks = (int)((T.rows + a.merge_rows - 1) / a.merge_rows);
    const int slab = ul / rblocks, rb = ul - slab * rblocks;
    const int64_t cs = (int64_t)slab * LORA_SLAB;
    const int64_t r0 = (int64_t)rb * a.merge_rows;
    const int rows = (int)min((int64_t)a.merge_rows, T.rows - r0);   // at most 32
    const bool active = cs + 8 * lane < cols;
    const uint32_t lo = active ? 16u * lane : BUF_OOR;
    const __amdgpu_buffer_rsrc_t rw = make_buf(X.W + r0 * ldw + cs, (int64_t)rows * ldw * 2);
    const uint32_t wstride = (uint32_t)(ldw * 2), mstride = (uint32_t)(cols * 2);
    if (uq.di != a_di || uq.e != a_e || slab != a_slab) {
      const __amdgpu_buffer_rsrc_t ra = make_buf(X.A + cs, (int64_t)r * cols * 2 - cs * 2);
#pragma unroll
      for (int k = 0; k < LORA_MAX_R; ++k) ap[k] = buf_load16(ra, lo + k * mstride);
      uint32_t amx = 0;
#pragma unroll
      for (int k = 0; k < LORA_MAX_R; ++k) amx = umax(amx, amax_bits8(ap[k]));
      a_l = __uint_as_float(amx << 16) * 1.001f;
      a_di = uq.di;
      a_e = uq.e;
      a_slab = slab;
    }
    // bsum of row r0 + lane (lanes below rows)
    float bsum = 0.0f;
    {
      const __amdgpu_buffer_rsrc_t rbb = make_buf(X.B + r0 * r, (int64_t)rows * r * 2);
      const uint32_t bo = lane < rows ? (uint32_t)(lane * r * 2) : BUF_OOR;
      if constexpr (RK == LORA_MAX_R) {
        const uint4 b0 = buf_load16(rbb, bo), b1 = buf_load16(rbb, bo + 16);
        const uint32_t bwv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) bsum = (bsum + fabsf(bf16_lo(bwv[q]))) + fabsf(bf16_hi(bwv[q]));
      } else {
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k)
          bsum += fabsf(__uint_as_float((uint32_t)buf_load2(rbb, k < r ? bo + 2u * k : BUF_OOR) << 16));
      }
    }
    uint4 wv[LORA_P1_PREFETCH];
#pragma unroll
    for (int q = 0; q < LORA_P1_PREFETCH; ++q) {
      LORA_FENCE();
      wv[q] = buf_load16(rw, lo + q * wstride);
    }
    LORA_FENCE();
    // t of the lane's 8 elements of row ii (w: the row's chunk); true where the lane's
    // elements could exceed L
    auto test = [&](const uint4& wq, int ii) {
      const float sb = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(bsum), ii & 31));
      const float ub = __builtin_fmaf(sb, a_l, 0x1p-100f);
      const float t = __uint_as_float(amax_bits8(wq) << 16) + ub;
      const float prevL = L ? __uint_as_float((L - 1u) << 16) : -1.0f;
      return ii < rows && !(t <= prevL);
    };
#pragma unroll 1
    for (int i = 0; i < rows; i += LORA_P1_PREFETCH) {
      {
        const uint32_t gl = __hip_atomic_load(gmax + mg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        L = umax(L, (uint32_t)__builtin_amdgcn_readfirstlane((int)gl));
      }
      // the batch's rows are tested first; rows that may hold a new maximum are merged
      // after, one at a time (their chunk loaded again, from the cache)
      uint32_t cmask = 0;
#pragma unroll
      for (int q = 0; q < LORA_P1_PREFETCH; ++q) {
        LORA_FENCE();
        if (__builtin_amdgcn_ballot_w64(test(wv[q], i + q))) cmask |= 1u << q;
        wv[q] = buf_load16(rw, lo + (i + q + LORA_P1_PREFETCH) * wstride);   // past the end: zeros
      }
      LORA_FENCE();
#pragma unroll 1
      while (cmask) {
        const int ii = i + __builtin_ctz(cmask);
        cmask &= cmask - 1;
        const uint4 wq = buf_load16(rw, lo + ii * wstride);
        if (!__builtin_amdgcn_ballot_w64(test(wq, ii))) continue;      // L has grown since
        uint32_t bw[BW];
        // B's rows from expert 0's aligned base (expert e's row i is row e * rows + i)
        fetch_b_words<RK>(T.B, (int64_t)uq.e * T.rows + r0 + ii, r, bw);
        float bk[LORA_MAX_R];
        b_row_values<RK>(bw, (int64_t)uq.e * T.rows + r0 + ii, r, bk);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        // A is unpacked here, not once per unit (128 more registers would not fit): the
        // packed words pass through an opaque zero made inside the loop, so the compiler
        // cannot hoist the unpacking
        uint32_t z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k) {
          const uint4 apk = make_uint4(ap[k].x ^ z, ap[k].y ^ z, ap[k].z ^ z, ap[k].w ^ z);
          float av[8];
          unpack8(apk, av);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(bk[k], av[e], acc[e]);
        }
        float wf[8];
        unpack8(wq, wf);
        uint4 o;
        o.x = pack_bf16x2(wf[0] + acc[0], wf[1] + acc[1]);
        o.y = pack_bf16x2(wf[2] + acc[2], wf[3] + acc[3]);
        o.z = pack_bf16x2(wf[4] + acc[4], wf[5] + acc[5]);
        o.w = pack_bf16x2(wf[6] + acc[6], wf[7] + acc[7]);
        uint32_t mt = active ? amax_bits8(o) : 0u;
        mt = umax(mt, dpp_xor1(mt));
        mt = umax(mt, dpp_xor2(mt));
        mt = umax(mt, dpp_hmirror(mt));
        mt = umax(mt, dpp_mirror(mt));
        mt = umax(mt, swz_xor16(mt));
        mt = umax((uint32_t)__builtin_amdgcn_readlane((int)mt, 0), (uint32_t)__builtin_amdgcn_readlane((int)mt, 32));
        L = umax(L, mt);
      }
    }
  }
  if (mg >= 0 && lane == 0) atomicMax(gmax + mg, L);
  __syncthreads();
  if ((int)threadIdx.x < a.n_groups) a.partial[threadIdx.x * gridDim.x + blockIdx.x] = gmax[threadIdx.x];
}

// --------------------------------------------- fused adapter gradients ---
// One pass over G for both gradients.  A workgroup owns a unit of up to a.da_rows (256
// or 512) rows of one LORA_SLAB-column slab and walks it 32 rows at a time: the
// 32 x 512 chunk of G is loaded with 16-byte coalesced loads (a wave instruction covers
// one row of the slab), the next chunk's loads are issued, and the chunk is written to
// LDS, where both gradients read it on the 16x16x32 BF16 MFMA:
//   dB (rows x 16): G rows as the MFMA's A operand in their natural layout, A's rows as
//     its B operand (kept in registers for the unit); wave w sums columns 128w ..
//     128w+127 of the chunk's 32 rows and the 4 waves' sums are added in LDS in a fixed
//     order, giving one partial per slab (k_lora_grad_reduce adds the slabs in order);
//   dA (16 x cols): B's rows transposed as the A operand (K = the chunk's 32 rows), G as
//     the B operand read transposed from LDS (each lane gathers 8 rows of one column);
//     wave w owns columns 128w .. 128w+127 of the slab and sums over all rows of the
//     unit, giving one partial per unit (k_lora_grad_reduce adds the units in order).
// One pass instead of one per gradient: 149 us for 8 experts with a pass per gradient,
// 73 us now (with both reduces, from cold caches).
// Staged rows are 1040 bytes apart (16 B of padding) and rows 16..31 swap their 16-byte
// chunks in pairs, so the natural reads (16 rows, one chunk) and the transposed reads
// (4 groups of 8 rows, two chunks) both hit distinct banks.
constexpr int GR_ROWS = 32;
constexpr int GR_PITCH = 2 * LORA_SLAB + 16;
constexpr int GR_BUF = GR_ROWS * GR_PITCH;

__device__ __forceinline__ uint32_t gr_off(uint32_t r, uint32_t c) {
  return r * GR_PITCH + ((c ^ (((r >> 4) & 1u) << 1)) << 4);
}

__global__ __launch_bounds__(256) void k_lora_grads(LoraArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t gl[2 * GR_BUF];
  __shared__ float red[4][2][256];                         // dB sums of the 4 waves
  const int b = blockIdx.x;
  const int di = lora_desc_of<&LoraTensor::grad_wg_begin>(a, b);
  const LoraTensor& T = a.d[di];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63u;
  const uint32_t l16 = lane & 15u, lq = lane >> 4;
  const int wpe = (int)((T.rows + a.da_rows - 1) / a.da_rows) * T.slabs;   // workgroups per expert
  const int e = (b - T.grad_wg_begin) / wpe;
  const int u = b - T.grad_wg_begin - e * wpe;
  const LoraMat X = lora_mat(T, e, a.da_rows);
  const int rb = u / T.slabs;
  const int slab = u - rb * T.slabs;
  const int64_t cols = T.cols, cs = (int64_t)slab * LORA_SLAB;
  const int r = T.r;
  const int64_t r0 = (int64_t)rb * a.da_rows;
  const int rows = (int)min((int64_t)a.da_rows, T.rows - r0);
  const int nchunk = (rows + GR_ROWS - 1) / GR_ROWS;

  // G loads: lane t takes 8 columns (t & 63) of rows (t >> 6) + 4 i of the chunk
  const __amdgpu_buffer_rsrc_t rg = make_buf(X.G + r0 * cols + cs, (int64_t)rows * cols * 2);
  const bool col_ok = cs + 8 * (int64_t)lane < cols;
  const uint32_t goff = col_ok ? ((tid >> 6) * (uint32_t)cols + 8u * lane) * 2u : BUF_OOR;
  const uint32_t gstep = (uint32_t)(4 * cols) * 2u, gchunk = (uint32_t)(GR_ROWS * cols) * 2u;
  auto load_chunk = [&](int ci, uint4 (&gv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = buf_load16_nt(rg, goff + i * gstep + (uint32_t)ci * gchunk);
  };
  auto stage_chunk = [&](uint8_t* buf, const uint4 (&gv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(buf + gr_off((tid >> 6) + 4u * i, lane)) = gv[i];
  };

  // dB: adapter A fragments of this wave's columns (K steps 4w .. 4w+3 of the slab):
  // lane l supplies adapter row l%16, columns 32 ks + 8 (l/16) .. +7
  const __amdgpu_buffer_rsrc_t ra = make_buf(X.A + cs, (int64_t)r * cols * 2 - cs * 2);
  bf16x8_t af[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t c = 32u * (4u * wave + s) + 8u * lq;
    const uint32_t off = (cs + c < cols) ? (l16 * (uint32_t)cols + c) * 2u : BUF_OOR;   // rows >= r read 0
    af[s] = __builtin_bit_cast(bf16x8_t, buf_load16(ra, off));
  }
  // dA: B rows of the chunk transposed: lane l supplies adapter l%16, rows 8 (l/16) .. +7
  const __amdgpu_buffer_rsrc_t rbb = make_buf(X.B + r0 * r, (int64_t)rows * r * 2);
  // dB partials of this unit's rows in this slab
  const __amdgpu_buffer_rsrc_t rdbp =
      make_buf(X.dB_partial + ((int64_t)slab * T.rows + r0) * LORA_MAX_R, (int64_t)rows * LORA_MAX_R * 4);

  // a chunk's B values for dA (rows past the end and adapters past r read 0), loaded
  // as 8 half words and packed into the MFMA operand only where it is used, so that
  // nothing waits for these loads when they are issued
  // (one 32-bit register per half word: packed 16-bit lanes would be merged, and
  // waited for, right at the load)
  auto load_bt = [&](int ci, uint32_t (&raw)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t row = 32u * ci + 8u * lq + t;
      const uint32_t off = ((int)l16 < r) ? (row * (uint32_t)r + l16) * 2u : BUF_OOR;
      raw[t] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rbb, (int)off, 0, 0);
    }
  };
  auto pack_bt = [&](const uint32_t (&raw)[8]) {
    const uint4 w = make_uint4(raw[0] | (raw[1] << 16), raw[2] | (raw[3] << 16), raw[4] | (raw[5] << 16),
                               raw[6] | (raw[7] << 16));
    return __builtin_bit_cast(bf16x8_t, w);
  };

  f32x4_t accA[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) accA[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Loads complete in issue order.  Each step computes chunk ci from LDS and stores its
  // dB partials, then waits for chunk ci + 1, stages it into the other buffer and
  // requests chunk ci + 2 into the registers it came from (B values before G rows), so
  // the wait at the staging point covers exactly the oldest 16 loads, the same on every
  // step.  (Two chunks in flight instead of one, in a second register set, measured
  // the same.)  Chunks past the unit's last row lie outside the resources and read
  // zeros, with no memory traffic.
  auto compute_chunk = [&](int ci, const bf16x8_t& bt) {
    uint8_t* buf = gl + (ci & 1) * GR_BUF;
    __syncthreads();                                       // chunk ci is in LDS
    // dB over this wave's 128 columns, both 16-row groups of the chunk
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4_t accB = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t gx = *reinterpret_cast<const bf16x8_t*>(buf + gr_off(16u * g + l16, 4u * (4u * wave + s) + lq));
        accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gx, af[s], accB, 0, 0, 0);
      }
      // lane holds rows 16 g + 4 (l/16) + e of the chunk, adapter l%16
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][g][(4u * lq + e) * 16u + l16] = accB[e];
    }
    // dA over this wave's 8 column tiles (16 columns each) and the chunk's 32 rows.  The
    // operand lane l needs is column l%16 of the tile at rows 8 (l/16) .. +7; two LDS
    // transpose reads give it: lane L of a 16-lane group points at 4 columns 4 (L%4) ..
    // +3 of row 8 (l/16) + L/4 (+ 4 for the second read), and lane i of the group then
    // receives element i%4 from lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4, i.e. column i of
    // those 4 rows.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c8 = 16u * wave + 2u * j + ((l16 & 3u) >> 1);   // 16-byte chunk of the 4 columns
      const uint32_t half = 8u * (l16 & 1u);
      const uint32_t row = 8u * lq + (l16 >> 2);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(buf + gr_off(row, c8) + half));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(buf + gr_off(row + 4u, c8) + half));
      const bf16x8_t gt = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt, gt, accA[j], 0, 0, 0);
    }
    __syncthreads();                                       // red is complete
    // dB partial of this slab: lane t adds the 4 waves' sums for 2 of the 512 outputs.
    // The stores are unconditional (outputs past r or past the last row get an
    // out-of-range offset), so every step issues the same number of memory operations.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t o = tid + 256u * h;                  // (group, row-in-group, adapter)
      const uint32_t g = o >> 8, rr = (o >> 4) & 15u, k = o & 15u;
      const float v = ((red[0][g][o & 255u] + red[1][g][o & 255u]) + red[2][g][o & 255u]) + red[3][g][o & 255u];
      const uint32_t row = 32u * ci + 16u * g + rr;        // within the unit
      const uint32_t off = ((int)k < r && (int)row < rows) ? (row * LORA_MAX_R + k) * 4u : BUF_OOR;
      buf_store4(rdbp, off, __float_as_uint(v));
    }
    LORA_FENCE();
  };
  // stage chunk ci + 1 (its buffer was last read by chunk ci - 1) and refill its registers
  auto stage_and_refill = [&](int ci, uint4 (&gv)[8], uint32_t (&braw)[8], bf16x8_t& bt) {
    stage_chunk(gl + ((ci + 1) & 1) * GR_BUF, gv);
    bt = pack_bt(braw);
    LORA_FENCE();
    load_bt(ci + 2, braw);
    LORA_FENCE();
    load_chunk(ci + 2, gv);
    LORA_FENCE();
  };
  bf16x8_t bt;
  uint4 gv[8];
  uint32_t braw[8];
  load_bt(0, braw);
  LORA_FENCE();
  load_chunk(0, gv);
  LORA_FENCE();
  stage_chunk(gl, gv);
  bt = pack_bt(braw);
  LORA_FENCE();
  load_bt(1, braw);
  LORA_FENCE();
  load_chunk(1, gv);
  LORA_FENCE();
#pragma unroll 1
  for (int ci = 0; ci < nchunk; ++ci) {
    compute_chunk(ci, bt);
    stage_and_refill(ci, gv, braw, bt);
  }
  // dA partial of this unit: lane holds adapters 4 (l/16) + e of columns 128 w + 16 j + l%16
  float* part = X.dA_partial + (int64_t)rb * LORA_MAX_R * cols + cs;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t col = 128 * wave + 16 * j + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * (int)lq + e;
      if (k < r && cs + col < cols) part[(int64_t)k * cols + col] = accA[j][e];
    }
  }
}

// ------------------------------------------------------------ launchers ----
static bool all_rank16(const LoraArgs& a) {
  for (int i = 0; i < a.n; ++i)
    if (a.d[i].r != LORA_MAX_R) return false;
  return true;
}

hipError_t launch_lora_merge(const LoraArgs& a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  bool any_m = false;
  for (int i = 0; i < a.n; ++i) any_m = any_m || a.d[i].M;
  // Without M, launches large enough for 32-row slab units take the bounded pass; smaller
  // ones (8- or 16-row units, e.g. one expert per launch) keep the matrix-core pass, where
  // the bounded pass's per-unit loads of A and B would outweigh the merges it skips
  // (one expert per launch: 2.28 against 3.01 ms per 128 experts).
  const bool bounded = !any_m && a.merge_rows == LORA_QDQ_ROWS;
  if (all_rank16(a)) {
    if (any_m)
      hipLaunchKernelGGL((k_lora_merge_amax<LORA_MAX_R, true>), dim3(grid), dim3(256), 0, s, a);
    else if (bounded)
      hipLaunchKernelGGL(k_lora_merge_amax_bounded<LORA_MAX_R>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_lora_merge_amax<LORA_MAX_R, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (any_m)
      hipLaunchKernelGGL((k_lora_merge_amax<0, true>), dim3(grid), dim3(256), 0, s, a);
    else if (bounded)
      hipLaunchKernelGGL(k_lora_merge_amax_bounded<0>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_lora_merge_amax<0, false>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_lora_merge_qdq(const LoraArgs& a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (all_rank16(a))
    hipLaunchKernelGGL(k_lora_merge_qdq<LORA_MAX_R>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_lora_merge_qdq<0>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lora_grads(const LoraArgs& a, int grid, int accumulate, hipStream_t s) {
  if (a.n == 0 || grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lora_grads, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one thread per four adjacent gradient entries (grid-stride past 8192 workgroups); the
  // partial buffers' 16-byte alignment comes from the entry point's check on the workspace
  int64_t nB = 0, nA = 0;
  for (int i = 0; i < a.n; ++i) {
    nB = std::max<int64_t>(nB, a.d[i].rows * LORA_MAX_R);
    nA = std::max<int64_t>(nA, (int64_t)a.d[i].r * a.d[i].cols);
    if ((uintptr_t)a.d[i].dA_partial % 16 != 0 || (uintptr_t)a.d[i].dB_partial % 16 != 0) return hipErrorInvalidValue;
  }
  const int gB = (int)std::min<int64_t>((nB / 4 + 255) / 256, 8192), gA = (int)std::min<int64_t>((nA / 4 + 255) / 256, 8192);
  hipLaunchKernelGGL(k_lora_grad_reduce, dim3(gB + gA, a.n_mats), dim3(256), 0, s, a, accumulate, gB);
  return hipGetLastError();
}

}  // namespace qf
