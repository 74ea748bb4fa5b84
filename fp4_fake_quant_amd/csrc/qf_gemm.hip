// W4A4 MXFP4 simulated-quantization GEMM on gfx950: Y = QDQ(X) . QDQ(W)^T.
//
// What is computed: QATFactory project page, "Overview" (weights, and
// optionally activations, rounded onto the format's grid while every matrix
// multiplication runs in BF16) and "Key findings" 02 (MXFP4 benefits from
// quantizing activations too, i.e. W4A4 training).  X is [M, K] (tokens x
// hidden), W is [N, K] (out x in), both bf16 row-major; the MXFP4 blocks run
// along K.  Products are accumulated in fp32 by the BF16 MFMA units; Y is
// rounded to bf16 (RNE) once.
//
// Structure:
//   - a workgroup of 512 lanes (8 waves, 2 per SIMD, laid out 2 x 4) owns a 256 x 256
//     tile of Y; each wave a 128 (X rows) x 64 (W rows) sub-tile = 4 x 2
//     v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators per lane).  Two waves per
//     SIMD let the hardware issue one wave's QDQ arithmetic, LDS traffic and waits
//     while the other's MFMAs run (7% faster than 4 waves of 128 x 128);
//   - K advances 64 at a time through two LDS stages of X and W slices
//     (2 x 64 KiB).  16-byte chunks are XOR-swizzled by row so that the MFMA
//     fragment reads (32 rows x 16 bytes per half-wave) hit distinct banks;
//   - QDQ on load: the slice for step k+1 is loaded from global memory into
//     registers while step k's MFMAs run; each MXFP4 block of 32 elements sits
//     in 4 adjacent lanes (one 16-byte chunk each), its maximum is reduced with
//     two DPP steps and the block is rounded onto the MXFP4 grid with the gfx950
//     scaled FP4 conversions (bf16 -> E2M1 codes -> bf16, E8M0 scale in the
//     operand's exponent field) before it is written to LDS.  The MFMAs then
//     consume bf16 values that are exactly QDQ(X) and QDQ(W);
//   - W is passed as the MFMA "A" operand and X as "B", so each lane ends
//     with runs of 4 consecutive output columns of one output row (8-byte
//     stores);
//   - workgroups are mapped XCD-aware: consecutive workgroup ids go to the
//     eight XCDs in turn, so XCD x is handed the x-th eighth of a grouped
//     tile order (8 tile rows at a time) and its concurrently running
//     workgroups share X and W panels in its L2;
//   - the grid is persistent (at most one workgroup per CU, each running
//     several tiles in turn): a tile's last K step already loads the next
//     tile's first slice, and its epilogue stores drain while that tile starts.
#include "qf_device.h"
#include "qf_gemm_epilogue.h"
#include "qf_kernels.h"

namespace qf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int G_THREADS = 512;
constexpr int G_CHUNKS = GBK / 8;                      // 16-byte chunks per row of a K slice
constexpr int G_SLICE_BYTES = GBM * GBK * 2;           // one operand slice in LDS
constexpr int G_LOADS = GBM * G_CHUNKS / G_THREADS;    // chunks per lane per operand per K step (4)
constexpr int G_GROUP_M = 8;                           // tile rows per group of the tile order

// LDS byte offset of chunk c of row r in a slice (rows of 128 bytes).  Chunks are
// XOR-swizzled with f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2), which takes 8 distinct values
// on any 8 consecutive rows and, on 16 consecutive rows, 8 distinct values on each row
// parity: a 16-byte-per-lane fragment read (one chunk of 32 consecutive rows) then hits
// distinct banks whether the LDS serves 8 or 16 lanes of it per cycle.
__device__ __forceinline__ uint32_t lds_off(uint32_t r, uint32_t c) {
  const uint32_t f = ((r >> 1) & 7u) ^ ((r & 1u) << 2);
  return (r * G_CHUNKS + (c ^ f)) * 16u;
}

// MXFP4 QDQ of one 16-byte chunk; lanes 4i..4i+3 hold one 32-element block.
// The scale operand carries E in its exponent field: E = max(floor(log2 amax) - 2 + 127, 0)
// is the block maximum's bf16 exponent field minus 2, clamped at 0 (a saturating
// subtract on the field moved to bits 23..30).
// NOCLIP: the noclip rule, E = min(max(that field - 2 + [significand > 1.5], 0), 252).
template <bool NOCLIP = false>
__device__ __forceinline__ uint4 mxfp4_qdq_chunk(uint4 w) {
  uint32_t ebits;
  if constexpr (NOCLIP) {
    uint32_t m = amax_bits8(w);
    m = umax(m, dpp_xor1(m));
    m = umax(m, dpp_xor2(m));
    ebits = __builtin_elementwise_sub_sat((m & 0x7F80u) << 16, (m & 0x7Fu) > 0x40u ? 0x00800000u : 0x01000000u);
    ebits = ebits < ((uint32_t)MX_NOCLIP_E_MAX << 23) ? ebits : ((uint32_t)MX_NOCLIP_E_MAX << 23);
  } else {
    // only the exponent of the block maximum matters: E = its bf16 exponent field - 2
    uint32_t m = maxexp_bits8(w);
    m = umax(m, dpp_xor1(m));
    m = umax(m, dpp_xor2(m));
    ebits = __builtin_elementwise_sub_sat(m << 16, 0x01000000u);
  }
  const float sc = __uint_as_float(ebits);
  uint32_t codes = w.x;                        // every byte is overwritten below
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.x), sc, 0);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.y), sc, 1);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.z), sc, 2);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.w), sc, 3);
  uint4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
  return o;
}

// Buffer resource over the `rows_left` (<= 256) rows of a tile starting at p: loads past
// the last row come back as zero, which is how partial tiles are handled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* p, int64_t ld, int rows_left) {
  const int rows = rows_left < GBM ? rows_left : GBM;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)((int64_t)rows * ld * 2), 0x00020000);
}

__device__ __forceinline__ uint4 load_chunk_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// Grids of the in-kernel quantizer: MXFP4 (block 32 along K, E8M0 scale; lanes 4i..4i+3
// hold one block) or NVFP4 (block 16 along K, E4M3 scale under the operand's FP32 tensor
// scale s_t; lanes 2i and 2i+1 hold one block, the pairing nvfp4_qdq_chunk needs).
enum { GRID_MX = 0, GRID_NV = 1, GRID_MX_NOCLIP = 2 };

template <int GRID, bool QDQ>
__device__ __forceinline__ void store_chunk(uint8_t* lds, uint32_t r, uint32_t c, uint4 v, float s_t, float k6) {
  uint4 q = v;
  if constexpr (QDQ) {
    if constexpr (GRID == GRID_NV) q = nvfp4_qdq_chunk(v, s_t, k6).y;
    else q = mxfp4_qdq_chunk<GRID == GRID_MX_NOCLIP>(v);
  }
  *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = q;
}

#define QF_FENCE() __builtin_amdgcn_sched_barrier(0)

// Origin (m0, n0) of tile t of the launch order, XCD-aware: when the tile count is a
// multiple of 8, t & 7 picks one eighth of a grouped order (G_GROUP_M tile rows at a time)
// and t >> 3 the tile within it, so the workgroups of one XCD (ids congruent mod 8) work
// on neighbouring tiles and share X and W panels in that XCD's L2.
__device__ __forceinline__ void tile_origin(int t, int tiles_m, int tiles_n, int& m0, int& n0) {
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int group = t / (G_GROUP_M * tiles_n);
  const int first_m = group * G_GROUP_M;
  const int gsize = min(tiles_m - first_m, G_GROUP_M);
  const int in_group = t - group * G_GROUP_M * tiles_n;
  m0 = (first_m + in_group % gsize) * GBM;
  n0 = (in_group / gsize) * GBN;
}

// The workgroup's tiles of Y: blockIdx.x, blockIdx.x + gridDim.x, ...  The grid holds at
// most one workgroup per CU (the LDS admits no second one) and is a multiple of 8 when the
// tiles outnumber it, so every tile of a workgroup comes from its XCD's part of the order.
// Consecutive tiles overlap: the last K step of a tile loads the first K slice of the
// workgroup's next tile, which is in flight during the epilogue, and the epilogue's
// stores drain while the next tile starts.
//
// smem is the kernel's 128 KiB of LDS, sx / sw the NVFP4 tensor scales of X and W (unused
// for MXFP4).  YLDS: Y leaves through LDS (store_tile_lds); otherwise from the
// accumulators, 8 bytes (y_vec = 1) or one element (y_vec = 0) at a time.
template <int GRID, bool QA, bool QW, bool YLDS>
__device__ __forceinline__ void gemm_tiles(const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W,
                                           int64_t ldw, uint16_t* __restrict__ Y, int64_t ldy, int M, int N, int K,
                                           int y_vec, float sx, float sw, uint8_t* smem) {
  const float kx = 6.0f * sx, kw = 6.0f * sw;
  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = (N + GBN - 1) / GBN;
  const int total = tiles_m * tiles_n;

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wave >> 2, wn = wave & 3u;           // 2 x 4 waves: X rows wm*128, W rows wn*64
  const uint32_t frow = lane & 31u, fhalf = lane >> 5;     // MFMA fragment row, k half

  // global -> register loads: lane t takes chunk (t & 7) of rows (t >> 3) + 64 i
  const uint32_t lrow = threadIdx.x >> 3, lchunk = threadIdx.x & 7u;
  const uint32_t xoff = (uint32_t)(lrow * ldx + lchunk * 8) * 2u, xstep = (uint32_t)(64 * ldx) * 2u;
  const uint32_t woff = (uint32_t)(lrow * ldw + lchunk * 8) * 2u, wstep = (uint32_t)(64 * ldw) * 2u;

  uint4 raw[2 * G_LOADS];                                 // 4 X chunks, then 4 W chunks
  auto issue_load = [&](__amdgpu_buffer_rsrc_t lx, __amdgpu_buffer_rsrc_t lw, int idx, uint32_t kbyte) {
    if (idx < G_LOADS) raw[idx] = load_chunk_buf(lx, xoff + idx * xstep + kbyte);
    else raw[idx] = load_chunk_buf(lw, woff + (idx - G_LOADS) * wstep + kbyte);
  };
  auto stage_chunk = [&](int idx, uint8_t* stage) {
    if (idx < G_LOADS) store_chunk<GRID, QA>(stage, lrow + 64 * idx, lchunk, raw[idx], sx, kx);
    else store_chunk<GRID, QW>(stage + G_SLICE_BYTES, lrow + 64 * (idx - G_LOADS), lchunk, raw[idx], sw, kw);
  };

  const int nk = K / GBK;
  const uint32_t kb1 = (uint32_t)min(1, nk - 1) * GBK * 2u;
  int t = blockIdx.x, m0, n0;
  tile_origin(t, tiles_m, tiles_n, m0, n0);
  __amdgpu_buffer_rsrc_t rx = tile_rsrc(X + (int64_t)m0 * ldx, ldx, M - m0);
  __amdgpu_buffer_rsrc_t rw = tile_rsrc(W + (int64_t)n0 * ldw, ldw, N - n0);
  // step 0 of the first tile
#pragma unroll
  for (int idx = 0; idx < 2 * G_LOADS; ++idx) issue_load(rx, rw, idx, 0);
  // Later tiles reach the loop head with their step-0 loads followed by the epilogue's
  // stores in flight; stores to no memory put the first tile in the same state, so the
  // wait for those loads is the same on both paths and never waits for the stores.
  if constexpr (YLDS) epilogue_store_balance(Y);
  QF_FENCE();

  for (;;) {
    // the workgroup's next tile (a resource of no bytes when there is none: its loads return 0)
    const bool more = t < total - (int)gridDim.x;          // (t + gridDim.x could overflow)
    int m1 = 0, n1 = 0;
    if (more) tile_origin(t + (int)gridDim.x, tiles_m, tiles_n, m1, n1);
    const __amdgpu_buffer_rsrc_t rx1 = tile_rsrc(X + (int64_t)m1 * ldx, ldx, more ? M - m1 : 0);
    const __amdgpu_buffer_rsrc_t rw1 = tile_rsrc(W + (int64_t)n1 * ldw, ldw, more ? N - n1 : 0);

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: step 0's chunks (in registers) into stage 0, then step 1's chunks into
    // registers, in the loop's slot order (slot j stages and reloads chunk j)
#pragma unroll
    for (int slot = 0; slot < 2 * G_LOADS; ++slot) {
      stage_chunk(slot, smem);
      issue_load(rx, rw, slot, kb1);
      QF_FENCE();
    }
    __syncthreads();

    // fragments of substep s: fx[i] = X rows wm*128 + 32i + frow, fw[j] = W rows wn*64 + 32j + frow,
    // k chunk 2s + fhalf; two register sets, so substep s+1's fragments load during substep s
    bf16x8_t fx[2][4], fw[2][2];
    auto read_x = [&](int set, const uint8_t* base, int s, int i) {
      fx[set][i] = *reinterpret_cast<const bf16x8_t*>(base + lds_off(wm * 128 + i * 32 + frow, 2u * s + fhalf));
    };
    auto read_w = [&](int set, const uint8_t* base, int s, int j) {
      fw[set][j] = *reinterpret_cast<const bf16x8_t*>(base + G_SLICE_BYTES + lds_off(wn * 64 + j * 32 + frow, 2u * s + fhalf));
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) read_x(0, smem, 0, i);
#pragma unroll
    for (int j = 0; j < 2; ++j) read_w(0, smem, 0, j);

    // Substep s (16 of K) is 8 MFMAs in 4 pairs; pair q of substeps 0-2 also reads
    // fragments for substep s+1 and stages/reloads chunk slots (3, 3, 2 per substep).
    // Substep 3 follows the barrier and reads the next step's first fragments.  Measured
    // alternatives, all slower: a finer MFMA/VALU interleave asked of the scheduler with
    // sched_group_barrier (-3%), one QDQ piece after every MFMA (-1%), staging spread
    // over all four substeps with the barrier at the end of the step (-2%), and a
    // ping-pong in which waves 0-3 run their MFMAs while waves 4-7 stage and then the
    // reverse, with a barrier per phase (-26%).
    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      const uint8_t* base = smem + 2 * cur * G_SLICE_BYTES;
      uint8_t* next = smem + 2 * (cur ^ 1) * G_SLICE_BYTES;
      // loads of step ks+2 (the last step's repeated near the end); the last step loads
      // step 0 of the next tile
      const bool last = ks == nk - 1;
      const __amdgpu_buffer_rsrc_t lx = last ? rx1 : rx, lw = last ? rw1 : rw;
      const uint32_t kb2 = last ? 0u : (uint32_t)min(ks + 2, nk - 1) * GBK * 2u;
#pragma unroll
      for (int s = 0; s < GBK / 16; ++s) {
        const int fs = s & 1;
        if (s == 3) __syncthreads();                          // step ks+1's slice is in `next`
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // plain product: the wave issuing an MFMA pair goes first (1% faster; with QDQ
          // work between the pairs it measured 3% slower)
          if constexpr (!QA && !QW) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[q][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[fs][j], fx[fs][q], acc[q][j], 0, 0, 0);
          if constexpr (!QA && !QW) __builtin_amdgcn_s_setprio(0);
          const uint8_t* rb = (s < 3) ? base : next;
          const int rs = (s < 3) ? s + 1 : 0;
          const int rset = (s < 3) ? (fs ^ 1) : 0;
          if (q < 2) { read_x(rset, rb, rs, 2 * q); read_x(rset, rb, rs, 2 * q + 1); }
          else if (q == 2) { read_w(rset, rb, rs, 0); read_w(rset, rb, rs, 1); }
          if (s < 3) {
            // slots: s=0 -> 0,1,2; s=1 -> 3,4,5; s=2 -> 6,7
            const int slot = 3 * s + q;
            if (q < 3 && slot < 2 * G_LOADS) {
              stage_chunk(slot, next);                        // step ks+1's chunk (loaded during ks-1)
              issue_load(lx, lw, slot, kb2);                  // step ks+2's chunk
            }
          }
          QF_FENCE();
        }
      }
    }

    // ---- epilogue: lane holds Y row (i*32 + frow), columns j*32 + 8g + 4*fhalf + 0..3 ----
    if constexpr (YLDS) {
      store_tile_lds(acc, smem, Y, ldy, m0, n0, M, N);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + (int)(wm * 128 + i * 32 + frow);
        if (row >= M) continue;
        uint16_t* yr = Y + (int64_t)row * ldy;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + (int)(wn * 64 + j * 32 + 8 * g + 4 * fhalf);
            const uint32_t lo = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            const uint32_t hi = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            if (y_vec && col + 3 < N) {
              *reinterpret_cast<uint2*>(yr + col) = make_uint2(lo, hi);
            } else {
              const uint16_t v[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
              for (int e = 0; e < 4; ++e)
                if (col + e < N) yr[col + e] = v[e];
            }
          }
        }
      }
    }
    if (!more) break;
    t += (int)gridDim.x;
    m0 = m1;
    n0 = n1;
    rx = rx1;
    rw = rw1;
    __syncthreads();                                        // no wave reads the LDS any more
  }
}

#define QF_GEMM_KERNEL(NAME, GRID)                                                                               \
  template <bool QA, bool QW, bool YLDS>                                                                         \
  __global__ __launch_bounds__(G_THREADS) void NAME(const uint16_t* __restrict__ X, int64_t ldx,                 \
                                                    const uint16_t* __restrict__ W, int64_t ldw,                 \
                                                    uint16_t* __restrict__ Y, int64_t ldy, int M, int N, int K, \
                                                    int y_vec) {                                                 \
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * G_SLICE_BYTES]; /* 128 KiB of the 160 KiB */       \
    gemm_tiles<GRID, QA, QW, YLDS>(X, ldx, W, ldw, Y, ldy, M, N, K, y_vec, 1.0f, 1.0f, smem);                    \
  }

QF_GEMM_KERNEL(k_gemm_mxfp4, GRID_MX)
// MXFP4 under the noclip shared-exponent rule.
QF_GEMM_KERNEL(k_gemm_mxfp4_noclip, GRID_MX_NOCLIP)
#undef QF_GEMM_KERNEL

// NVFP4 W4A4: the tensor scales come from device memory (computed by the tensor-scale
// pass, or any fp32 the caller keeps there, e.g. a tracked activation maximum).
template <bool QA, bool QW, bool YLDS>
__global__ __launch_bounds__(G_THREADS) void k_gemm_nvfp4(const uint16_t* __restrict__ X, int64_t ldx,
                                                            const uint16_t* __restrict__ W, int64_t ldw,
                                                            uint16_t* __restrict__ Y, int64_t ldy,
                                                            int M, int N, int K, int y_vec,
                                                            const float* __restrict__ d_sx,
                                                            const float* __restrict__ d_sw) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * G_SLICE_BYTES];
  gemm_tiles<GRID_NV, QA, QW, YLDS>(X, ldx, W, ldw, Y, ldy, M, N, K, y_vec, QA ? *d_sx : 1.0f, QW ? *d_sw : 1.0f,
                                    smem);
}

// Workgroups of a launch: one per tile up to one per CU, a multiple of 8 beyond that.
static dim3 gemm_grid(int tiles) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  if (cus < 8) cus = 256;
  return dim3(tiles <= cus ? tiles : cus & ~7);
}

// One of the eight instantiations (QA, QW, YLDS) of kernel K, launched with its arguments.
#define QF_GEMM_LAUNCH(K, QA_, QW_, ...)                                                  \
  do {                                                                                   \
    if (y_vec == 2) hipLaunchKernelGGL((K<QA_, QW_, true>), g, b, 0, s, __VA_ARGS__);    \
    else hipLaunchKernelGGL((K<QA_, QW_, false>), g, b, 0, s, __VA_ARGS__);              \
  } while (0)

hipError_t launch_gemm_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, unsigned flags, const float* d_sx, const float* d_sw,
                             hipStream_t s) {
  const int tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  const bool qa = flags & QF_QDQ_A, qw = flags & QF_QDQ_W;
  const int y_vec = y_store_mode(Y, ldy, N);
  const dim3 g = gemm_grid(tiles), b(G_THREADS);
  if (qa && qw) QF_GEMM_LAUNCH(k_gemm_nvfp4, true, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec, d_sx, d_sw);
  else if (qa) QF_GEMM_LAUNCH(k_gemm_nvfp4, true, false, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec, d_sx, d_sw);
  else QF_GEMM_LAUNCH(k_gemm_nvfp4, false, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec, d_sx, d_sw);
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, unsigned flags, hipStream_t s) {
  const int tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  const bool qa = flags & QF_QDQ_A, qw = flags & QF_QDQ_W;
  // 2: Y through LDS in 16-byte stores; 1: 8-byte stores from the accumulators; 0: element stores
  const int y_vec = y_store_mode(Y, ldy, N);
  const dim3 g = gemm_grid(tiles), b(G_THREADS);
  if (flags & QF_MX_NOCLIP) {
    if (qa && qw) QF_GEMM_LAUNCH(k_gemm_mxfp4_noclip, true, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
    else if (qa) QF_GEMM_LAUNCH(k_gemm_mxfp4_noclip, true, false, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
    else QF_GEMM_LAUNCH(k_gemm_mxfp4_noclip, false, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
    return hipGetLastError();
  }
  if (qa && qw) QF_GEMM_LAUNCH(k_gemm_mxfp4, true, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
  else if (qa) QF_GEMM_LAUNCH(k_gemm_mxfp4, true, false, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
  else if (qw) QF_GEMM_LAUNCH(k_gemm_mxfp4, false, true, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
  else QF_GEMM_LAUNCH(k_gemm_mxfp4, false, false, X, ldx, W, ldw, Y, ldy, M, N, K, y_vec);
  return hipGetLastError();
}
#undef QF_GEMM_LAUNCH

}  // namespace qf
