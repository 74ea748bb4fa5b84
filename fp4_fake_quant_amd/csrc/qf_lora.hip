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
// Merge work split: a unit is one wave's share, LORA_SLAB = 512 columns (lane l owns
// columns 8l .. 8l+7 of the slab) of a run of rows.  Lanes keep their 16 x 8 slice
// of A in registers, so the per-row work is one 16-byte load, 128 FMAs and one
// 16-byte store per lane.  The row's B values are the same for every lane: they are
// loaded once per row through the scalar cache, where the FMAs read them.
//
// Kernels
//   k_lora_merge     M = W + B.A for up to LORA_ROWS rows per unit; either stores M
//                    (or not) and folds max|M| of the workgroup into its tied group's
//                    partial (NVFP4 pass 1), or merges again and NVFP4-QDQs and packs
//                    the merged rows in registers (pass 2 without M in memory).
//   k_lora_grads     dB = G . A^T and dA = B^T . G in one pass over G, both on the
//                    16x16x32 BF16 MFMA (G staged through LDS); per-slab dB partials and
//                    per-row-block dA partials, added in a fixed order by
//                    k_lora_dB_reduce and k_lora_dA_reduce (same inputs, same bits).
#include <algorithm>

#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Keeps the scheduler from moving instructions across this point: rows (or column
// steps) stay in program order, so each waits only for its own prefetched load.
#define LORA_FENCE() __builtin_amdgcn_sched_barrier(0)

// B[row, 0 .. r-1] as fp32 in scalar registers (entries past r are 0).  B is
// contiguous [rows, r] and 4-byte aligned; the row starts at element row * r,
// which may be odd: the 32-bit words holding it are read through the scalar
// cache (B is never written while these kernels run) and realigned by one half
// word if so.  With r odd, the last row's last word may hold the 2 bytes after B.
// (fetch_b_words / b_row_values below.)
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

__device__ __forceinline__ void unpack8(uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

__device__ __forceinline__ int find_desc_wg(const LoraArgs& a, int b) {
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && b >= a.d[di + 1].merge_wg_begin) ++di;
  return di;
}

// ------------------------------------------------------------- pass 1 ------
// Rows are software-pipelined: LORA_PREFETCH rows of W are always in flight, and the
// next row's B words are requested (scalar loads) while the current row is computed.
constexpr int LORA_PREFETCH = 4;
constexpr int BW = LORA_MAX_R / 2 + 1;   // 32-bit words that can hold one row of B

// Scalar words of B's row `row`, realigned into fp32 values by b_row_values.  RK is
// the rank when it is known at compile time (16: the row is 8 aligned words), else 0.
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

// B values of the row as fp32, zero past r: the padded steps fma(0, a, acc) leave acc
// unchanged bit for bit (a zero product added to acc gives acc, also for acc = -0).
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

// Loop bodies are branch-free: W, M, G and A are accessed through buffer resources
// that span exactly the valid rows (and A's r rows), lanes past the last column use
// an out-of-range offset, and the rows of the last group past the end are computed on
// zeros and dropped by the range check, so the compiler can keep every prefetched
// load in flight across rows.
//
// QDQ = false: M is stored (unless T.M is null: the resource is then empty and every
// store is dropped) and the workgroup's max|M| goes to its tied group's partial.
// QDQ = true: the merged row stays in registers and is NVFP4-QDQ'd and packed with the
// group's tensor scale (lanes 2i and 2i+1 hold one 16-block), so no M round trip
// through memory is needed; the merge arithmetic is the same, so the values are the
// same bits as QDQ of the stored M.
template <int RK, bool QDQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_lora_merge(LoraArgs a) {
  const int b = blockIdx.x;
  const LoraTensor& T = a.d[find_desc_wg(a, b)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;   // wave index: uniform
  const int u = (b - T.merge_wg_begin) * 4 + wave;
  uint32_t m = 0;
  if (u < T.merge_units) {
    const int64_t cols = T.cols, ldw = T.ldw;
    const int r = RK ? RK : T.r;
    const int rb = u / T.slabs;
    const int64_t cs = (int64_t)(u - rb * T.slabs) * LORA_SLAB;        // first column of the slab
    const int64_t r0 = (int64_t)rb * a.merge_rows;
    const int rows = (int)min((int64_t)a.merge_rows, T.rows - r0);
    const bool active = cs + 8 * lane < cols;
    const uint32_t lo = active ? 16u * lane : BUF_OOR;                  // lane's byte offset in a row
    const int64_t e0 = r0 * cols + cs;                                  // first element of the unit
    const __amdgpu_buffer_rsrc_t rw = make_buf(T.W + r0 * ldw + cs, (int64_t)rows * ldw * 2);
    const __amdgpu_buffer_rsrc_t ra = make_buf(T.A + cs, (int64_t)r * cols * 2 - cs * 2);
    const uint32_t wstride = (uint32_t)(ldw * 2), mstride = (uint32_t)(cols * 2);
    // outputs: M, or y / codes / scales (an empty resource drops the stores)
    const bool wm = !QDQ && T.M, wy = QDQ && T.y, wp = QDQ && T.codes;
    const __amdgpu_buffer_rsrc_t rm = make_buf(wm ? T.M + e0 : nullptr, wm ? (int64_t)rows * cols * 2 : 0);
    const __amdgpu_buffer_rsrc_t ry = make_buf(wy ? T.y + e0 : nullptr, wy ? (int64_t)rows * cols * 2 : 0);
    const __amdgpu_buffer_rsrc_t rc = make_buf(wp ? T.codes + e0 / 2 : nullptr, wp ? (int64_t)rows * cols / 2 : 0);
    const __amdgpu_buffer_rsrc_t rs = make_buf(wp ? T.scales + e0 / 16 : nullptr, wp ? (int64_t)rows * cols / 16 : 0);
    const uint32_t clo = active ? 4u * lane : BUF_OOR;
    const uint32_t slo = active && (lane & 1) == 0 ? (uint32_t)lane / 2u : BUF_OOR;
    const uint32_t cstride = (uint32_t)(cols / 2), sstride = (uint32_t)(cols / 16);
    const float s_t = QDQ ? a.tscale[T.group] : 0.0f, k6 = 6.0f * s_t;
    uint4 wv[LORA_PREFETCH];
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; ++q) {
      wv[q] = buf_load16_nt(rw, lo + q * wstride);
      LORA_FENCE();
    }
    uint32_t bw[BW];
    fetch_b_words<RK>(T.B, r0, r, bw);
    float av[LORA_MAX_R][8];                                           // rows k >= r read as 0
#pragma unroll
    for (int k = 0; k < LORA_MAX_R; ++k) unpack8(buf_load16(ra, lo + k * mstride), av[k]);
#pragma unroll 1
    for (int i = 0; i < rows; i += LORA_PREFETCH) {
#pragma unroll
      for (int q = 0; q < LORA_PREFETCH; ++q) {
        LORA_FENCE();
        const int ii = i + q;                                          // may pass the last row
        float bk[LORA_MAX_R];
        b_row_values<RK>(bw, r0 + min(ii, rows - 1), r, bk);
        fetch_b_words<RK>(T.B, r0 + min(ii + 1, rows - 1), r, bw);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(bk[k], av[k][e], acc[e]);
        float w[8];
        unpack8(wv[q], w);
        uint4 o;
        o.x = pack_bf16x2(w[0] + acc[0], w[1] + acc[1]);
        o.y = pack_bf16x2(w[2] + acc[2], w[3] + acc[3]);
        o.z = pack_bf16x2(w[4] + acc[4], w[5] + acc[5]);
        o.w = pack_bf16x2(w[6] + acc[6], w[7] + acc[7]);
        if constexpr (QDQ) {                                           // rows past the end: dropped
          const Nvfp4Chunk qc = nvfp4_qdq_chunk(o, s_t, k6);
          buf_store16(ry, lo + ii * mstride, qc.y);
          buf_store4(rc, clo + ii * cstride, qc.codes);
          buf_store1(rs, slo + ii * sstride, (uint8_t)qc.S);
        } else {
          buf_store16(rm, lo + ii * mstride, o);                       // past the end: dropped
          const uint32_t mo = amax_bits8(o);
          m = umax(m, (active && ii < rows) ? mo : 0u);
        }
        wv[q] = buf_load16_nt(rw, lo + (ii + LORA_PREFETCH) * wstride);   // past the end: zeros
      }
    }
  }
  if constexpr (!QDQ) {
    // workgroup maximum -> partial[g * grid + b]: this descriptor's group, 0 for the others
    m = umax(m, dpp_xor1(m));
    m = umax(m, dpp_xor2(m));
    m = umax(m, dpp_hmirror(m));
    m = umax(m, dpp_mirror(m));
    m = umax(m, swz_xor16(m));
    m = umax((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 32));
    __shared__ uint32_t wm[4];
    if (lane == 0) wm[wave] = m;
    __syncthreads();
    if ((int)threadIdx.x < a.n_groups) {
      const uint32_t v = (int)threadIdx.x == T.group ? umax(umax(wm[0], wm[1]), umax(wm[2], wm[3])) : 0u;
      a.partial[threadIdx.x * gridDim.x + b] = v;
    }
  }
}

// dA[k][j] (+)= sum over row blocks, in block order.
// Sum of count partials p[0], p[stride], ... added in index order from +0.  The loads
// are issued LORA_RED_BATCH at a time before any add, so one element costs a few memory
// latencies instead of one per partial; the order of the adds is unchanged.
constexpr int LORA_RED_BATCH = 8;

__device__ __forceinline__ float sum_partials(const float* p, int64_t stride, int count) {
  float s = 0.0f;
#pragma unroll 1
  for (int q0 = 0; q0 < count; q0 += LORA_RED_BATCH) {
    float v[LORA_RED_BATCH];
#pragma unroll
    for (int i = 0; i < LORA_RED_BATCH; ++i) v[i] = q0 + i < count ? p[(int64_t)(q0 + i) * stride] : 0.0f;
#pragma unroll
    for (int i = 0; i < LORA_RED_BATCH; ++i)
      if (q0 + i < count) s += v[i];
  }
  return s;
}

__global__ __launch_bounds__(256) void k_lora_dA_reduce(LoraArgs a, int accumulate) {
  const LoraTensor& T = a.d[blockIdx.y];
  const int64_t n = (int64_t)T.r * T.cols;
  const int nblk = (int)((T.rows + a.da_rows - 1) / a.da_rows);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    // partial q holds rows k = 0 .. 15 of cols columns; entry (k, j) of dA is at idx
    const float s = sum_partials(T.dA_partial + idx, (int64_t)LORA_MAX_R * T.cols, nblk);
    T.dA[idx] = accumulate ? T.dA[idx] + s : s;
  }
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
//     order, giving one partial per slab (k_lora_dB_reduce adds the slabs in order);
//   dA (16 x cols): B's rows transposed as the A operand (K = the chunk's 32 rows), G as
//     the B operand read transposed from LDS (each lane gathers 8 rows of one column);
//     wave w owns columns 128w .. 128w+127 of the slab and sums over all rows of the
//     unit, giving one partial per unit (k_lora_dA_reduce adds the units in order).
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
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && b >= a.d[di + 1].grad_wg_begin) ++di;
  const LoraTensor& T = a.d[di];
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63u;
  const uint32_t l16 = lane & 15u, lq = lane >> 4;
  const int u = b - T.grad_wg_begin;
  const int rb = u / T.slabs;
  const int slab = u - rb * T.slabs;
  const int64_t cols = T.cols, cs = (int64_t)slab * LORA_SLAB;
  const int r = T.r;
  const int64_t r0 = (int64_t)rb * a.da_rows;
  const int rows = (int)min((int64_t)a.da_rows, T.rows - r0);
  const int nchunk = (rows + GR_ROWS - 1) / GR_ROWS;

  // G loads: lane t takes 8 columns (t & 63) of rows (t >> 6) + 4 i of the chunk
  const __amdgpu_buffer_rsrc_t rg = make_buf(T.G + r0 * cols + cs, (int64_t)rows * cols * 2);
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
  const __amdgpu_buffer_rsrc_t ra = make_buf(T.A + cs, (int64_t)r * cols * 2 - cs * 2);
  bf16x8_t af[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t c = 32u * (4u * wave + s) + 8u * lq;
    const uint32_t off = (cs + c < cols) ? (l16 * (uint32_t)cols + c) * 2u : BUF_OOR;   // rows >= r read 0
    af[s] = __builtin_bit_cast(bf16x8_t, buf_load16(ra, off));
  }
  // dA: B rows of the chunk transposed: lane l supplies adapter l%16, rows 8 (l/16) .. +7
  const __amdgpu_buffer_rsrc_t rbb = make_buf(T.B + r0 * r, (int64_t)rows * r * 2);
  // dB partials of this unit's rows in this slab
  const __amdgpu_buffer_rsrc_t rdbp =
      make_buf(T.dB_partial + ((int64_t)slab * T.rows + r0) * LORA_MAX_R, (int64_t)rows * LORA_MAX_R * 4);

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
    // dA over this wave's 8 column tiles (16 columns each) and the chunk's 32 rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t col = 128u * wave + 16u * j + l16;   // column within the slab
      bf16x8_t gt;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        gt[t] = *reinterpret_cast<const __bf16*>(buf + gr_off(8u * lq + t, col >> 3) + 2u * (col & 7u));
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
  float* part = T.dA_partial + (int64_t)rb * LORA_MAX_R * cols + cs;
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

// dB[row][k] (+)= sum over slabs, in slab order.
__global__ __launch_bounds__(256) void k_lora_dB_reduce(LoraArgs a, int accumulate) {
  const LoraTensor& T = a.d[blockIdx.y];
  const int64_t n = T.rows * LORA_MAX_R;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / LORA_MAX_R;
    const int k = (int)(idx - row * LORA_MAX_R);
    if (k >= T.r) continue;
    const float s = sum_partials(T.dB_partial + idx, T.rows * LORA_MAX_R, T.slabs);
    float* dst = T.dB + row * T.r + k;
    *dst = accumulate ? *dst + s : s;
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
  if (all_rank16(a))
    hipLaunchKernelGGL((k_lora_merge<LORA_MAX_R, false>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_lora_merge<0, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lora_merge_qdq(const LoraArgs& a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (all_rank16(a))
    hipLaunchKernelGGL((k_lora_merge<LORA_MAX_R, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_lora_merge<0, true>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lora_grads(const LoraArgs& a, int grid, int accumulate, hipStream_t s) {
  if (a.n == 0 || grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lora_grads, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one thread per gradient entry (grid-stride past 8192 workgroups)
  int64_t nB = 0, nA = 0;
  for (int i = 0; i < a.n; ++i) {
    nB = std::max<int64_t>(nB, a.d[i].rows * LORA_MAX_R);
    nA = std::max<int64_t>(nA, (int64_t)a.d[i].r * a.d[i].cols);
  }
  const int gB = (int)std::min<int64_t>((nB + 255) / 256, 8192), gA = (int)std::min<int64_t>((nA + 255) / 256, 8192);
  if (gB > 0) hipLaunchKernelGGL(k_lora_dB_reduce, dim3(gB, a.n), dim3(256), 0, s, a, accumulate);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gA > 0) hipLaunchKernelGGL(k_lora_dA_reduce, dim3(gA, a.n), dim3(256), 0, s, a, accumulate);
  return hipGetLastError();
}

}  // namespace qf
