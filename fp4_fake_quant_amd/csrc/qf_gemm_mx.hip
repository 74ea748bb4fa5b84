// W4A4 MXFP4 GEMM on gfx950's scaled FP4 matrix cores: Y = QDQ(X) . QDQ(W)^T.
//
// What is computed is the same as in qf_gemm.hip (QATFactory project page,
// "Overview" and "Key findings" 02): every QDQ'd MXFP4 value is exactly
// E2M1(code) * 2^(E - 127), so QDQ(x) * QDQ(w) is exact in any format wide enough,
// and the BF16 matmul of the QDQ'd operands is the fp32 sum of these exact
// products.  v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands forms the same
// exact products from the E2M1 codes and the E8M0 block scales and accumulates
// them in fp32, so the result obeys the same error bound as the BF16 path while
// the matrix cores do 4x the work per cycle and no dequantization is needed.
//
// Operand layout of the instruction (checked on the device): lane l supplies row
// l%32 of its operand and one 32-element K block (l/32) as 16 bytes of E2M1 codes
// (two per byte, the same packing as qf_pack_mxfp4 produces), and byte 0 (with
// op_sel 0) of its scale register is that block's E8M0 exponent.  The output
// layout is that of the other 32x32 MFMAs.
//
// Structure (512 lanes, 8 waves laid out 2 x 4, a 256 x 256 tile of Y; each wave
// 128 rows of X by 64 rows of W = 4 x 2 MFMA tiles of 32 x 32, K = 64 per step):
//   - X (and, unless it comes packed, W) is loaded as bf16 16-byte chunks; lanes
//     4i..4i+3 hold one 32-element block: block maximum by two DPP steps, E8M0
//     exponent from its bf16 exponent field, E2M1 codes by four scaled
//     conversions; 4 code bytes per lane and the block's exponent byte go to LDS;
//   - packed W (codes [N][K/2], exponents [N][K/32]) is copied to LDS as is;
//   - LDS holds three stages (18 KiB each): while step k computes from stage k,
//     step k+1's fragments are read from stage k+1 and step k+2's operands are
//     written to stage k+2, so one barrier per step suffices and fragment reads
//     never wait on the barrier;
//   - code rows are 32 bytes (two 16-byte K blocks); the two blocks swap places on
//     rows with bit 3 set, so 16 lanes reading 16 consecutive rows hit distinct banks;
//   - global loads run one step ahead of staging (one register set, refilled
//     right after its chunk is staged) with exact waits (branch-free body);
//   - XCD-aware grouped tile order as in qf_gemm.hip, 2 tile rows per group
//     (measured: 2.35 ms at 2, 2.46 at 4 and 8, 2.99 at 16 for the packed-W path);
//   - K = 64 per step: the 128 variant is written but needs more registers than
//     two waves per SIMD allow (it spills), so it is not the default.
#include "qf_device.h"
#include "qf_gemm_epilogue.h"
#include "qf_kernels.h"

namespace qf {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// The instruction reads 4 registers per FP4 operand; the builtin's operand type has 8
// elements, the upper four left undefined so that they take no registers.
__device__ __forceinline__ i32x8_t fp4_operand(i32x4_t v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1); }
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int MX_BM = 256, MX_BN = 256;
constexpr int MX_THREADS = 512;
constexpr int MX_GROUP_M = 2;                               // tile rows per group of the tile order

// One operand slice of a K step of BK elements in LDS: codes [256 rows][BK/2 bytes]
// (BK/32 16-byte K blocks per row), then the E8M0 exponents, 4 bytes per row (K
// blocks 0..3 of the step; BK = 64 uses the first two).
template <int BK> struct MxLayout {
  static constexpr int KB = BK / 32;                       // K blocks per row per step
  static constexpr int ROW = BK / 2;                       // code bytes per row
  static constexpr int CODES = MX_BM * ROW;
  static constexpr int OPER = CODES + MX_BM * 4;
  static constexpr int STAGE = 2 * OPER;                   // X then W
  // byte offset of K block kb of row r: blocks are rotated by row so that 16 lanes
  // reading block kb of 16 consecutive rows hit distinct banks
  static __device__ __forceinline__ uint32_t off(uint32_t r, uint32_t kb) {
    const uint32_t sw = KB == 2 ? ((r >> 3) & 1u) : ((r >> 2) & 3u);
    return r * ROW + ((kb ^ sw) << 4);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* p, int64_t row_bytes, int rows_left) {
  const int rows = rows_left < MX_BM ? rows_left : MX_BM;
  return make_buf(p, (int64_t)rows * row_bytes);
}

// E2M1 codes of one 16-byte bf16 chunk (lanes 4i..4i+3 hold one 32-element block) and
// the block's E8M0 exponent E = max(floor(log2 amax) - 2 + 127, 0).
__device__ __forceinline__ uint32_t mx_quant_chunk(uint4 w, uint32_t& e) {
  uint32_t m = maxexp_bits8(w);               // only the exponent of the block maximum matters
  m = umax(m, dpp_xor1(m));
  m = umax(m, dpp_xor2(m));
  const uint32_t ebits = __builtin_elementwise_sub_sat(m << 16, 0x01000000u);
  e = ebits >> 23;
  const float sc = __uint_as_float(ebits);
  uint32_t codes = w.x;                        // every byte is overwritten below
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.x), sc, 0);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.y), sc, 1);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.z), sc, 2);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w.w), sc, 3);
  return codes;
}

#define MX_FENCE() __builtin_amdgcn_sched_barrier(0)

// WPACKED: W arrives as packed codes Wc [N][K/2] and exponents Ws [N][K/32] (row-major,
// contiguous); otherwise W is bf16 [N][ldw] and is quantized here like X.  BK: K per
// step (64 or 128); each step is BK/64 substeps of one MFMA per output tile.
template <bool WPACKED, int BK>
__global__ __launch_bounds__(MX_THREADS) void k_gemm_mx4(const uint16_t* __restrict__ X, int64_t ldx,
                                                         const uint16_t* __restrict__ W, int64_t ldw,
                                                         const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
                                                         uint16_t* __restrict__ Y, int64_t ldy, int M, int N, int K,
                                                         int y_vec) {
  using L = MxLayout<BK>;
  constexpr int SUB = BK / 64;                              // MFMA substeps per step
  constexpr int CPR = BK / 8;                               // bf16 chunks per row per step
  constexpr int RPP = MX_THREADS / CPR;                     // rows per load pass
  constexpr int NX = MX_BM / RPP;                           // X chunks per lane per step
  constexpr int NWQ = WPACKED ? 0 : NX;                     // W chunks to quantize per lane
  constexpr int NWC = WPACKED ? MX_BM * L::KB / MX_THREADS : 0;   // packed W code pieces per lane
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * L::STAGE];

  // ---- tile of this workgroup (XCD-aware grouped order) ----
  const int tiles_m = (M + MX_BM - 1) / MX_BM, tiles_n = (N + MX_BN - 1) / MX_BN;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int group = t / (MX_GROUP_M * tiles_n);
  const int first_m = group * MX_GROUP_M;
  const int gsize = min(tiles_m - first_m, MX_GROUP_M);
  const int in_group = t - group * MX_GROUP_M * tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * MX_BM, n0 = tn * MX_BN;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wm = wave >> 2, wn = wave & 3u;            // X rows wm*128, W rows wn*64
  const uint32_t frow = lane & 31u, fblk = lane >> 5;       // fragment row, K block of a substep

  // bf16 chunk loads: lane t takes chunk (t % CPR) of rows t / CPR + RPP i
  const uint32_t lrow = tid / CPR, lchunk = tid % CPR;
  const uint32_t lkb = lchunk >> 2, lpos = lchunk & 3u;
  const __amdgpu_buffer_rsrc_t rx = mx_rsrc(X + (int64_t)m0 * ldx, ldx * 2, M - m0);
  const uint32_t xoff = (lrow * (uint32_t)ldx + lchunk * 8u) * 2u, xstep = (uint32_t)(RPP * ldx) * 2u;
  __amdgpu_buffer_rsrc_t rw, rwc, rws;
  uint32_t woff = 0, wstep = 0, wsoff = 0;
  const int64_t kc = K / 2, ks32 = K / 32;                   // packed row lengths in bytes
  if constexpr (WPACKED) {
    // codes: piece p = tid + 512 j is K block p % KB of row p / KB; exponents: lanes
    // 0..255 copy the step's KB bytes of row tid (out-of-range offset for the others)
    rwc = mx_rsrc(Wc + (int64_t)n0 * kc, kc, N - n0);
    rws = mx_rsrc(Ws + (int64_t)n0 * ks32, ks32, N - n0);
    wsoff = tid < 256 ? tid * (uint32_t)ks32 : BUF_OOR;
  } else {
    rw = mx_rsrc(W + (int64_t)n0 * ldw, ldw * 2, N - n0);
    woff = (lrow * (uint32_t)ldw + lchunk * 8u) * 2u;
    wstep = (uint32_t)(RPP * ldw) * 2u;
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  uint4 xr[NX], wr[NWQ > 0 ? NWQ : 1], wcr[NWC > 0 ? NWC : 1];
  uint32_t wsr = 0;                                         // packed: the row's exponent bytes

  // the loads and stagings of a step come in two halves
  auto issue_loads = [&](int step, int part) {
    const uint32_t kb = (uint32_t)step * BK;
#pragma unroll
    for (int i = part * NX / 2; i < (part + 1) * NX / 2; ++i) xr[i] = buf_load16(rx, xoff + i * xstep + kb * 2u);
    if constexpr (WPACKED) {
      if (part == 0) {
#pragma unroll
        for (int j = 0; j < NWC; ++j) {
          const uint32_t p = tid + MX_THREADS * j;
          wcr[j] = buf_load16(rwc, (p / L::KB) * (uint32_t)kc + (p % L::KB) * 16u + kb / 2u);
        }
        if constexpr (L::KB == 4) wsr = __builtin_amdgcn_raw_buffer_load_b32(rws, (int)(wsoff + kb / 32u), 0, 0);
        else wsr = __builtin_amdgcn_raw_buffer_load_b16(rws, (int)(wsoff + kb / 32u), 0, 0);
      }
    } else {
#pragma unroll
      for (int i = part * NWQ / 2; i < (part + 1) * NWQ / 2; ++i) wr[i] = buf_load16(rw, woff + i * wstep + kb * 2u);
    }
  };
  auto stage_part = [&](uint8_t* st, int part) {
    uint8_t* xc = st;
    uint8_t* xs = st + L::CODES;
#pragma unroll
    for (int i = part * NX / 2; i < (part + 1) * NX / 2; ++i) {
      uint32_t e;
      const uint32_t c = mx_quant_chunk(xr[i], e);
      const uint32_t r = lrow + RPP * i;
      *reinterpret_cast<uint32_t*>(xc + L::off(r, lkb) + 4u * lpos) = c;
      xs[r * 4u + lkb] = (uint8_t)e;
    }
    uint8_t* wc = st + L::OPER;
    uint8_t* ws = wc + L::CODES;
    if constexpr (WPACKED) {
      if (part == 0) {
#pragma unroll
        for (int j = 0; j < NWC; ++j) {
          const uint32_t p = tid + MX_THREADS * j;
          *reinterpret_cast<uint4*>(wc + L::off(p / L::KB, p % L::KB)) = wcr[j];
        }
        if (tid < 256) {
          if constexpr (L::KB == 4) *reinterpret_cast<uint32_t*>(ws + tid * 4u) = wsr;
          else *reinterpret_cast<uint16_t*>(ws + tid * 4u) = (uint16_t)wsr;
        }
      }
    } else {
#pragma unroll
      for (int i = part * NWQ / 2; i < (part + 1) * NWQ / 2; ++i) {
        uint32_t e;
        const uint32_t c = mx_quant_chunk(wr[i], e);
        const uint32_t r = lrow + RPP * i;
        *reinterpret_cast<uint32_t*>(wc + L::off(r, lkb) + 4u * lpos) = c;
        ws[r * 4u + lkb] = (uint8_t)e;
      }
    }
  };

  // fragments of a substep: fx[i] = X row wm*128 + 32i + frow, fw[j] = W row wn*64 + 32j +
  // frow, K block 2 sub + fblk; exponent registers hold the row's exponent bytes shifted so
  // that byte 0 is the lane's block
  i32x4_t fx[2][4], fw[2][2];
  uint32_t sx[2][4], sw[2][2];
  auto read_frags = [&](int set, const uint8_t* st, int sub) {
    const uint32_t kb = 2u * sub + fblk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = wm * 128u + 32u * i + frow;
      fx[set][i] = *reinterpret_cast<const i32x4_t*>(st + L::off(r, kb));
      sx[set][i] = *reinterpret_cast<const uint32_t*>(st + L::CODES + r * 4u) >> (8u * kb);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t r = wn * 64u + 32u * j + frow;
      fw[set][j] = *reinterpret_cast<const i32x4_t*>(st + L::OPER + L::off(r, kb));
      sw[set][j] = *reinterpret_cast<const uint32_t*>(st + L::OPER + L::CODES + r * 4u) >> (8u * kb);
    }
  };

  const int nk = K / BK;
  // prologue: steps 0 and 1 staged, step 2 in registers, step 0's first fragments read
  issue_loads(0, 0);
  issue_loads(0, 1);
  MX_FENCE();
  stage_part(smem, 0);
  issue_loads(min(1, nk - 1), 0);
  MX_FENCE();
  stage_part(smem, 1);
  issue_loads(min(1, nk - 1), 1);
  MX_FENCE();
  stage_part(smem + L::STAGE, 0);
  issue_loads(min(2, nk - 1), 0);
  MX_FENCE();
  stage_part(smem + L::STAGE, 1);
  issue_loads(min(2, nk - 1), 1);
  MX_FENCE();
  __syncthreads();
  read_frags(0, smem, 0);

  // step k: SUB substeps of MFMAs, each on the fragment set read during the previous
  // substep; the last substep reads step k+1's first fragments from stage k+1.  Step
  // k+2 (loaded during step k-1) is staged into stage k+2 and step k+3 is loaded.
  // Steps past the end reload the last slice and stage into a stage nobody reads.
  // The loop body covers two steps so that the fragment set of every substep is a
  // compile-time index (sets alternate with every substep).
  int s_cur = 0;
#pragma unroll 1
  for (int k0 = 0; k0 < nk; k0 += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + h;
      if (k >= nk) break;
      const int s_nxt = s_cur == 2 ? 0 : s_cur + 1;
      const int s_stg = s_nxt == 2 ? 0 : s_nxt + 1;
      const int st3 = min(k + 3, nk - 1);
#pragma unroll
      for (int sub = 0; sub < SUB; ++sub) {
        const int fs = (SUB * h + sub) & 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[q][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(fw[fs][j]), fp4_operand(fx[fs][q]),
                                                                          acc[q][j], 4, 4, 0, (int)sw[fs][j], 0,
                                                                          (int)sx[fs][q]);
          if (q == 0) {
            if (sub + 1 < SUB) read_frags(fs ^ 1, smem + s_cur * L::STAGE, sub + 1);
            else read_frags(fs ^ 1, smem + s_nxt * L::STAGE, 0);
          }
          if (q == 1 && sub == 0) { stage_part(smem + s_stg * L::STAGE, 0); issue_loads(st3, 0); }
          if (q == 2 && sub == SUB - 1) { stage_part(smem + s_stg * L::STAGE, 1); issue_loads(st3, 1); }
          MX_FENCE();
        }
      }
      __syncthreads();
      s_cur = s_nxt;
    }
  }

  // ---- epilogue: lane holds Y row (i*32 + frow), columns j*32 + 8g + 4*fblk + 0..3 ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + (int)(wm * 128 + i * 32 + frow);
    if (row >= M) continue;
    uint16_t* yr = Y + (int64_t)row * ldy;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + (int)(wn * 64 + j * 32 + 8 * g + 4 * fblk);
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

// ---------------------------------------------------------------------------
// Both operands packed (codes [rows][K/2], exponents [rows][K/32], as qf_pack_mxfp4
// writes them): no arithmetic before the MFMAs at all.  Operands go from memory
// straight into LDS with buffer loads that write LDS (16 bytes per lane into a
// 1 KiB window per wave instruction, 4 bytes per lane for the exponents), three
// steps ahead through a four-stage ring (K = 128 per step, 34 KiB per stage).  Each
// lane loads the global block that belongs at its place in the window, so the
// bank-spreading rotation of the code rows costs nothing.  The barrier sits after
// the first of the step's two MFMA substeps, so the next step's fragments are read
// while the second substep's MFMAs run.
constexpr int PP_BK = 128;
constexpr int PP_STAGES = 4;
constexpr int PP_AHEAD = PP_STAGES - 1;                   // steps of loads in flight
using PPL = MxLayout<PP_BK>;

// s_waitcnt that waits until at most n vector-memory operations are outstanding (the
// LDS and export counters left at their maximum)
#define PP_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// Workgroup barrier for the buffer-to-LDS ring: wait until at most n vector-memory
// operations (this lane's later steps) are outstanding and all LDS reads are back, then
// s_barrier.  A __syncthreads() here would wait for every load in flight (the compiler
// cannot tell that only the oldest step's loads must have landed); the empty asm with a
// memory clobber keeps the compiler from moving LDS accesses across the barrier.
#define PP_BARRIER(n)                                                                       \
  do {                                                                                      \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (0 << 8));      \
    __builtin_amdgcn_s_barrier();                                                           \
    asm volatile("" ::: "memory");                                                          \
  } while (0)

// 8 waves: 2 per SIMD laid out 2 x 4, each 128 rows of X by 64 of W (4 x 2 MFMA tiles).
// (4 waves, one per SIMD with 128 x 128 wave tiles, would read a third fewer fragment
// bytes from LDS per MFMA, but the compiler keeps its 256 accumulators in VGPRs and
// spills; the code keeps the wave count as a parameter for that layout.)  What bounds this kernel: per
// substep the 8 waves read 48 KiB of fragments and the loads write 17 KiB into LDS,
// close to the LDS bandwidth the 16 MFMAs per SIMD take to run; timing without the
// loads (stale data) still gives 1.07 ms against 1.45 ms with them.
constexpr int WAVES = 8;
__global__ __launch_bounds__(64 * WAVES) void k_gemm_mx4pp(const uint8_t* __restrict__ Xc, const uint8_t* __restrict__ Xs,
                                                           const uint8_t* __restrict__ Wc, const uint8_t* __restrict__ Ws,
                                                           uint16_t* __restrict__ Y, int64_t ldy, int M, int N, int K,
                                                           int y_vec) {
  constexpr int NJ = WAVES == 8 ? 2 : 4;                   // 32-row W tiles per wave
  constexpr int WN = 32 * NJ;                              // W rows per wave
  constexpr int CW = 16 / WAVES;                           // code windows per wave per operand
  constexpr int SW = 8 / WAVES;                            // exponent windows per wave
  constexpr int LOADS = 2 * CW + SW;                       // buffer-to-LDS loads per lane per step
  __shared__ __attribute__((aligned(16))) uint8_t smem[PP_STAGES * PPL::STAGE];   // 136 KiB

  // ---- tile of this workgroup (XCD-aware grouped order) ----
  const int tiles_m = (M + MX_BM - 1) / MX_BM, tiles_n = (N + MX_BN - 1) / MX_BN;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int group = t / (MX_GROUP_M * tiles_n);
  const int first_m = group * MX_GROUP_M;
  const int gsize = min(tiles_m - first_m, MX_GROUP_M);
  const int in_group = t - group * MX_GROUP_M * tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * MX_BM, n0 = tn * MX_BN;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wm = wave / (256 / WN), wn = wave % (256 / WN);
  const uint32_t frow = lane & 31u, fblk = lane >> 5;

  const int64_t kc = K / 2, ks32 = K / 32;
  const __amdgpu_buffer_rsrc_t rxc = mx_rsrc(Xc + (int64_t)m0 * kc, kc, M - m0);
  const __amdgpu_buffer_rsrc_t rwc = mx_rsrc(Wc + (int64_t)n0 * kc, kc, N - n0);
  const __amdgpu_buffer_rsrc_t rxs = mx_rsrc(Xs + (int64_t)m0 * ks32, ks32, M - m0);
  const __amdgpu_buffer_rsrc_t rws = mx_rsrc(Ws + (int64_t)n0 * ks32, ks32, N - n0);
  // code windows: wave w fills windows CW w .. CW w + CW-1 (16 rows each) of both operands;
  // lane l of window v holds row 16v + l/4 at slot l%4, which is K block (l%4) ^ rotation(row)
  uint32_t coff[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const uint32_t row = 16u * (CW * wave + i) + (lane >> 2);
    const uint32_t kb = (lane & 3u) ^ ((row >> 2) & 3u);
    coff[i] = row * (uint32_t)kc + kb * 16u;
  }
  // exponent windows (64 rows x 4 bytes): 8 of them, X rows 64v + l for v < 4, W rows
  // 64(v-4) + l for v >= 4; wave w fills windows SW w .. SW w + SW-1
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto issue_step = [&](int step) {
    const int k = min(step, K / PP_BK - 1);               // past the end: reload the last step
    uint8_t* st = smem + (step % PP_STAGES) * PPL::STAGE;
    const uint32_t kb = (uint32_t)k * (PP_BK / 2);          // code bytes into the row
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const uint32_t win = CW * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rxc, (lds_ptr_t)(st + win * 1024u), 16, coff[i] + kb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rwc, (lds_ptr_t)(st + PPL::OPER + win * 1024u), 16, coff[i] + kb, 0, 0, 0);
    }
    const uint32_t eb = (uint32_t)k * (PP_BK / 32);
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      const uint32_t v = SW * wave + i;                     // uniform
      const uint32_t off = (64u * (v & 3u) + lane) * (uint32_t)ks32 + eb;
      if (v < 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, (lds_ptr_t)(st + PPL::CODES + 256u * v), 4, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, (lds_ptr_t)(st + PPL::OPER + PPL::CODES + 256u * (v - 4)), 4, off,
                                                    0, 0, 0);
    }
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  i32x4_t fx[2][4], fw[2][NJ];
  uint32_t ex[2][4], ew[2][NJ];                             // exponent words of the step's rows
  auto read_codes = [&](int set, const uint8_t* st, int sub) {
    const uint32_t kb = 2u * sub + fblk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fx[set][i] = *reinterpret_cast<const i32x4_t*>(st + PPL::off(wm * 128u + 32u * i + frow, kb));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fw[set][j] = *reinterpret_cast<const i32x4_t*>(st + PPL::OPER + PPL::off(wn * WN + 32u * j + frow, kb));
  };
  auto read_exps = [&](int set, const uint8_t* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ex[set][i] = *reinterpret_cast<const uint32_t*>(st + PPL::CODES + (wm * 128u + 32u * i + frow) * 4u);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      ew[set][j] = *reinterpret_cast<const uint32_t*>(st + PPL::OPER + PPL::CODES + (wn * WN + 32u * j + frow) * 4u);
  };

  const int nk = K / PP_BK;
  // prologue: steps 0 .. PP_AHEAD-1 in flight, step 0 landed and its first fragments read
#pragma unroll
  for (int s = 0; s < PP_AHEAD; ++s) issue_step(s);
  PP_BARRIER((PP_AHEAD - 1) * LOADS);
  read_codes(0, smem, 0);
  read_exps(0, smem);

  // Step k: load step k+3; substep 0 on fragment set 0 while set 1 (substep 1) is read;
  // wait for step k+1's loads and barrier; substep 1 on set 1 while step k+1's set 0 and
  // exponents are read.  Exponent sets alternate with steps (unrolled by two).
#pragma unroll 1
  for (int k0 = 0; k0 < nk; k0 += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + h;
      if (k >= nk) break;
      const uint8_t* cur = smem + (k % PP_STAGES) * PPL::STAGE;
      const uint8_t* nxt = smem + ((k + 1) % PP_STAGES) * PPL::STAGE;
      issue_step(k + PP_AHEAD);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (sub == 1) PP_BARRIER((PP_AHEAD - 1) * LOADS);   // step k+1 has landed (k+2, k+3 may fly)
        const int sh = 8 * (2 * sub) + 8 * (int)fblk;
        uint32_t sxs[4], sws[NJ];                           // the substep's exponent bytes in byte 0
#pragma unroll
        for (int i = 0; i < 4; ++i) sxs[i] = ex[h][i] >> sh;
#pragma unroll
        for (int j = 0; j < NJ; ++j) sws[j] = ew[h][j] >> sh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[q][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fp4_operand(fw[sub][j]), fp4_operand(fx[sub][q]), acc[q][j], 4, 4, 0, (int)sws[j], 0, (int)sxs[q]);
          if (q == 0) {
            if (sub == 0) read_codes(1, cur, 1);
            else { read_codes(0, nxt, 0); read_exps(h ^ 1, nxt); }
          }
          MX_FENCE();
        }
      }
    }
  }
  PP_WAIT_VM(0);                                           // no load may still write LDS at exit
  if (y_vec == 2) {                                          // 16-byte aligned rows: through LDS
    store_tile_lds(acc, smem, Y, ldy, m0, n0, M, N);
    return;
  }

  // ---- epilogue: lane holds Y row (i*32 + frow), columns j*32 + 8g + 4*fblk + 0..3 ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + (int)(wm * 128 + i * 32 + frow);
    if (row >= M) continue;
    uint16_t* yr = Y + (int64_t)row * ldy;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + (int)(wn * WN + j * 32 + 8 * g + 4 * fblk);
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

hipError_t launch_gemm_mx4pp(const uint8_t* Xc, const uint8_t* Xs, const uint8_t* Wc, const uint8_t* Ws, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, hipStream_t s) {
  const int tiles = ((M + MX_BM - 1) / MX_BM) * ((N + MX_BN - 1) / MX_BN);
  const int y_vec = y_store_mode(Y, ldy, N);
  hipLaunchKernelGGL(k_gemm_mx4pp, dim3(tiles), dim3(64 * WAVES), 0, s, Xc, Xs, Wc, Ws, Y, ldy, M, N, K, y_vec);
  return hipGetLastError();
}

hipError_t launch_gemm_mx4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, const uint8_t* Wc,
                           const uint8_t* Ws, uint16_t* Y, int64_t ldy, int M, int N, int K, hipStream_t s) {
  const int tiles = ((M + MX_BM - 1) / MX_BM) * ((N + MX_BN - 1) / MX_BN);
  const int y_vec = (ldy % 4 == 0) && ((uintptr_t)Y % 8 == 0);
  const dim3 g(tiles), b(MX_THREADS);
  // K = 64 per step for both forms: 128 measured slower for each
  if (Wc)
    hipLaunchKernelGGL((k_gemm_mx4<true, 64>), g, b, 0, s, X, ldx, W, ldw, Wc, Ws, Y, ldy, M, N, K, y_vec);
  else
    hipLaunchKernelGGL((k_gemm_mx4<false, 64>), g, b, 0, s, X, ldx, W, ldw, Wc, Ws, Y, ldy, M, N, K, y_vec);
  return hipGetLastError();
}

}  // namespace qf
