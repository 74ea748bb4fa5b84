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
// Work split: a unit is one wave's share, LORA_SLAB = 512 columns (lane l owns
// columns 8l .. 8l+7 of the slab) of a run of rows.  Lanes keep their 16 x 8
// slice of A (or of the dA sums) in registers, so the per-row work is one
// 16-byte load, 128 FMAs and (merge) one 16-byte store per lane.  The row's B
// values are the same for every lane: they are loaded once per row and moved to
// scalar registers, where the FMAs read them.
//
// Kernels
//   k_lora_merge     M = W + B.A for up to LORA_ROWS rows per unit; folds max|M| of the
//                    workgroup into its tied group's partial (NVFP4 pass 1).
//   k_lora_dB        dB = G . A^T on the 16x16x32 BF16 MFMA: a wave owns 16 rows
//                    and walks all columns 32 at a time (G rows are the MFMA's A
//                    operand as stored; A's rows are its B operand), so every dB
//                    element is finished in one wave and no reduction is needed.
//   k_lora_dA        dA = B^T . G with fp32 FMAs over LORA_DA_ROWS rows per unit;
//                    each unit writes a partial that k_lora_dA_reduce sums in row
//                    block order (same inputs, same bits).
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
template <int RK>
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
    const __amdgpu_buffer_rsrc_t rw = make_buf(T.W + r0 * ldw + cs, (int64_t)rows * ldw * 2);
    const __amdgpu_buffer_rsrc_t rm = make_buf(T.M + r0 * cols + cs, (int64_t)rows * cols * 2);
    const __amdgpu_buffer_rsrc_t ra = make_buf(T.A + cs, (int64_t)r * cols * 2 - cs * 2);
    const uint32_t wstride = (uint32_t)(ldw * 2), mstride = (uint32_t)(cols * 2);
    uint4 wv[LORA_PREFETCH];
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; ++q) {
      wv[q] = buf_load16(rw, lo + q * wstride);
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
        buf_store16(rm, lo + ii * mstride, o);                         // past the end: dropped
        const uint32_t mo = amax_bits8(o);
        m = umax(m, (active && ii < rows) ? mo : 0u);
        wv[q] = buf_load16(rw, lo + (ii + LORA_PREFETCH) * wstride);   // past the end: zeros
      }
    }
  }
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

// ------------------------------------------------------- dB = G . A^T ------
// v_mfma_f32_16x16x32_bf16: lane l supplies row l%16 and k-chunk l/16 (8 elements) of
// the A operand, column l%16 and the same k-chunk of the B operand, and receives C rows
// 4(l/16) .. 4(l/16)+3 of column l%16.  A wave owns LORA_DB_ROWS rows (row groups of
// 16 that share each fragment of the adapter A) and walks all columns with
// DB_PREFETCH column steps in flight; steps past the last column load zeros.
#ifndef QF_DB_PREFETCH
#define QF_DB_PREFETCH 4
#endif
constexpr int DB_PREFETCH = QF_DB_PREFETCH;
constexpr int DB_GROUPS = LORA_DB_ROWS / 16;

__global__ __launch_bounds__(256) void k_lora_dB(LoraArgs a, int accumulate) {
  const int gw = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);   // global wave (uniform)
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && gw >= a.d[di + 1].dB_wave_begin) ++di;
  const LoraTensor& T = a.d[di];
  const int64_t row0 = (int64_t)(gw - T.dB_wave_begin) * LORA_DB_ROWS;
  if (row0 >= T.rows) return;
  const int64_t cols = T.cols;
  const int r = T.r;
  const int vrows = (int)min((int64_t)LORA_DB_ROWS, T.rows - row0);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t lr = lane & 15u, lk = lane >> 4;
  const uint32_t rowb = (uint32_t)(cols * 2);
  // rows past vrows and adapter rows past r are out of range: they read 0
  const __amdgpu_buffer_rsrc_t rg = make_buf(T.G + row0 * cols, (int64_t)vrows * cols * 2);
  const __amdgpu_buffer_rsrc_t ra = make_buf(T.A, (int64_t)r * cols * 2);
  uint32_t go[DB_GROUPS];
#pragma unroll
  for (int h = 0; h < DB_GROUPS; ++h) go[h] = (16u * h + lr) * rowb + 16u * lk;
  const uint32_t ao = lr * rowb + 16u * lk;
  const int nsteps = (int)(cols / 32);
  bf16x8_t x[DB_GROUPS][DB_PREFETCH], y[DB_PREFETCH];
#pragma unroll
  for (int q = 0; q < DB_PREFETCH; ++q) {
    const uint32_t so = q < nsteps ? 64u * q : BUF_OOR;
#pragma unroll
    for (int h = 0; h < DB_GROUPS; ++h) x[h][q] = __builtin_bit_cast(bf16x8_t, buf_load16(rg, go[h] + so));
    y[q] = __builtin_bit_cast(bf16x8_t, buf_load16(ra, ao + so));
    LORA_FENCE();
  }
  f32x4_t acc[DB_GROUPS];
#pragma unroll
  for (int h = 0; h < DB_GROUPS; ++h) acc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
  for (int s = 0; s < nsteps; s += DB_PREFETCH) {
#pragma unroll
    for (int q = 0; q < DB_PREFETCH; ++q) {
      LORA_FENCE();
#pragma unroll
      for (int h = 0; h < DB_GROUPS; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[h][q], y[q], acc[h], 0, 0, 0);
      const int sn = s + q + DB_PREFETCH;
      const uint32_t so = sn < nsteps ? 64u * (uint32_t)sn : BUF_OOR;
#pragma unroll
      for (int h = 0; h < DB_GROUPS; ++h) x[h][q] = __builtin_bit_cast(bf16x8_t, buf_load16(rg, go[h] + so));
      y[q] = __builtin_bit_cast(bf16x8_t, buf_load16(ra, ao + so));
    }
  }
  // lane holds dB rows row0 + 16 h + 4 lk + e (e = 0..3), adapter column lr
  if ((int)lr < r) {
#pragma unroll
    for (int h = 0; h < DB_GROUPS; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + 16 * h + 4 * lk + e;
        if (row < T.rows) {
          float* dst = T.dB + row * r + lr;
          *dst = accumulate ? *dst + acc[h][e] : acc[h][e];
        }
      }
    }
  }
}

// ------------------------------------------------------- dA = B^T . G ------
// A workgroup owns one slab of LORA_SLAB columns of LORA_DA_ROWS rows; its 4 waves
// take a quarter of the rows each (lane l: columns 8l .. 8l+7, 16 x 8 sums in
// registers) and their sums are added in LDS in a fixed order (w0 + w2, w1 + w3,
// then the two) before the workgroup writes its partial.

template <int RK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_lora_dA(LoraArgs a) {
  const int b = blockIdx.x;
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && b >= a.d[di + 1].dA_wg_begin) ++di;
  const LoraTensor& T = a.d[di];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;   // wave index: uniform
  const int u = b - T.dA_wg_begin;                  // one unit per workgroup
  const int rb = u / T.slabs;
  const int64_t cols = T.cols;
  const int64_t cs = (int64_t)(u - rb * T.slabs) * LORA_SLAB;
  const bool active = cs + 8 * lane < cols;
  const int r = RK ? RK : T.r;
  float acc[LORA_MAX_R][8];
#pragma unroll
  for (int k = 0; k < LORA_MAX_R; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.0f;
  const int wave_rows = a.da_rows / 4;
  const int64_t r0 = (int64_t)rb * a.da_rows + (int64_t)wave * wave_rows;
  const int rows = (int)max((int64_t)0, min((int64_t)wave_rows, T.rows - r0));
  if (rows > 0) {
    const uint32_t lo = active ? 16u * lane : BUF_OOR;
    const uint32_t stride = (uint32_t)(cols * 2);
    const __amdgpu_buffer_rsrc_t rg = make_buf(T.G + r0 * cols + cs, (int64_t)rows * cols * 2);
    uint4 gv[LORA_PREFETCH];
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; ++q) {
      gv[q] = buf_load16(rg, lo + q * stride);
      LORA_FENCE();
    }
    uint32_t bw[BW];
    fetch_b_words<RK>(T.B, r0, r, bw);
    // rows of the last group past the end read G = 0 and take the last row's (finite)
    // B values, so they add exact zeros; with non-finite B the result is unspecified
#pragma unroll 1
    for (int i = 0; i < rows; i += LORA_PREFETCH) {
#pragma unroll
      for (int q = 0; q < LORA_PREFETCH; ++q) {
        LORA_FENCE();
        const int ii = i + q;
        float bk[LORA_MAX_R];
        b_row_values<RK>(bw, r0 + min(ii, rows - 1), r, bk);
        fetch_b_words<RK>(T.B, r0 + min(ii + 1, rows - 1), r, bw);
        float g[8];
        unpack8(gv[q], g);
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[k][e] = __builtin_fmaf(bk[k], g[e], acc[k][e]);
        gv[q] = buf_load16(rg, lo + (ii + LORA_PREFETCH) * stride);   // past the end: zeros
      }
    }
  }
  // fixed-order reduction of the 4 waves through LDS, half of the 16 x 8 sums at a
  // time: w0 + w2 and w1 + w3, then (w0 + w2) + (w1 + w3); wave 0 writes the partial
  constexpr int H = LORA_MAX_R / 2;
  __shared__ float red[2][H * 8][64];
  float* part = T.dA_partial + (int64_t)rb * LORA_MAX_R * cols + cs + 8 * lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wave >= 2) {
#pragma unroll
      for (int k = 0; k < H; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave - 2][k * 8 + e][lane] = acc[h * H + k][e];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int k = 0; k < H; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h * H + k][e] += red[wave][k * 8 + e][lane];
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int k = 0; k < H; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[0][k * 8 + e][lane] = acc[h * H + k][e];
    }
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
      for (int k = 0; k < H; ++k) {
        if (h * H + k < r) {
          float sm[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) sm[e] = acc[h * H + k][e] + red[0][k * 8 + e][lane];
          float4* p = reinterpret_cast<float4*>(part + (int64_t)(h * H + k) * cols);
          p[0] = make_float4(sm[0], sm[1], sm[2], sm[3]);
          p[1] = make_float4(sm[4], sm[5], sm[6], sm[7]);
        }
      }
    }
    __syncthreads();                                 // red is reused by the next half
  }
}

// dA[k][j] (+)= sum over row blocks, in block order.
__global__ __launch_bounds__(256) void k_lora_dA_reduce(LoraArgs a, int accumulate) {
  const LoraTensor& T = a.d[blockIdx.y];
  const int64_t n = (int64_t)T.r * T.cols;
  const int nblk = (int)((T.rows + a.da_rows - 1) / a.da_rows);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = idx / T.cols, j = idx - k * T.cols;
    float s = 0.0f;
    for (int q = 0; q < nblk; ++q) s += T.dA_partial[((int64_t)q * LORA_MAX_R + k) * T.cols + j];
    T.dA[idx] = accumulate ? T.dA[idx] + s : s;
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
    hipLaunchKernelGGL(k_lora_merge<LORA_MAX_R>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_lora_merge<0>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lora_grads(const LoraArgs& a, int dB_waves, int dA_grid, int accumulate, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (dB_waves > 0) {
    hipLaunchKernelGGL(k_lora_dB, dim3((dB_waves + 3) / 4), dim3(256), 0, s, a, accumulate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dA_grid > 0) {
    if (all_rank16(a))
      hipLaunchKernelGGL(k_lora_dA<LORA_MAX_R>, dim3(dA_grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_lora_dA<0>, dim3(dA_grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lora_dA_reduce, dim3(64, a.n), dim3(256), 0, s, a, accumulate);
  }
  return hipGetLastError();
}

}  // namespace qf
