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
//   k_lora_merge     M = W + B.A for LORA_ROWS rows per unit; folds max|M| of the
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

// B[row, 0 .. r-1] as fp32 in scalar registers (entries past r are 0).  B is
// contiguous [rows, r] and 4-byte aligned; the row starts at element row * r,
// which may be odd: the 32-bit words holding it are read through the scalar
// cache (B is never written while these kernels run) and realigned by one half
// word if so.  With r odd, the last row's last word may hold the 2 bytes after B.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

__device__ __forceinline__ void load_b_row(const uint16_t* B, int64_t row, int r, float (&bk)[LORA_MAX_R]) {
  const int64_t e0 = row * r;
  const const_u32_ptr bw = (const_u32_ptr)(reinterpret_cast<const uint32_t*>(B) + (e0 >> 1));
  const uint32_t odd = (uint32_t)(e0 & 1);
  const int nw = ((int)odd + r + 1) >> 1;          // words that hold the row
  uint32_t w[LORA_MAX_R / 2 + 1];
#pragma unroll
  for (int q = 0; q < LORA_MAX_R / 2 + 1; ++q) w[q] = q < nw ? bw[q] : 0u;
#pragma unroll
  for (int q = 0; q < LORA_MAX_R / 2; ++q) {
    const uint32_t v = odd ? ((w[q] >> 16) | (w[q + 1] << 16)) : w[q];
    bk[2 * q] = 2 * q < r ? bf16_lo(v) : 0.0f;
    bk[2 * q + 1] = 2 * q + 1 < r ? bf16_hi(v) : 0.0f;
  }
}

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
constexpr int LORA_PREFETCH = 4;   // rows whose loads are issued before the first is used

__global__ __launch_bounds__(256) void k_lora_merge(LoraArgs a) {
  const int b = blockIdx.x;
  const LoraTensor& T = a.d[find_desc_wg(a, b)];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = (b - T.merge_wg_begin) * 4 + wave;
  uint32_t m = 0;
  if (u < T.merge_units) {
    const int rb = u / T.slabs;
    const int64_t c0 = (int64_t)(u - rb * T.slabs) * LORA_SLAB + 8 * lane;
    const bool active = c0 < T.cols;
    const int r = T.r;
    float av[LORA_MAX_R][8];
#pragma unroll
    for (int k = 0; k < LORA_MAX_R; ++k) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (active && k < r) w = *reinterpret_cast<const uint4*>(T.A + (int64_t)k * T.cols + c0);
      unpack8(w, av[k]);
    }
    const int64_t r0 = (int64_t)rb * LORA_ROWS;
    const int rows = (int)min((int64_t)LORA_ROWS, T.rows - r0);
#pragma unroll 1
    for (int i = 0; i < rows; i += LORA_PREFETCH) {
      uint4 wv[LORA_PREFETCH];
#pragma unroll
      for (int q = 0; q < LORA_PREFETCH; ++q) {
        // rows past the end re-read the last row (never stored)
        const int64_t row = r0 + min(i + q, rows - 1);
        wv[q] = active ? *reinterpret_cast<const uint4*>(T.W + row * T.ldw + c0) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < LORA_PREFETCH; ++q) {
        if (i + q >= rows) break;
        const int64_t row = r0 + i + q;
        float bk[LORA_MAX_R];
        load_b_row(T.B, row, r, bk);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < LORA_MAX_R; ++k) {
          if (k < r) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(bk[k], av[k][e], acc[e]);
          }
        }
        float w[8];
        unpack8(wv[q], w);
        uint4 o;
        o.x = pack_bf16x2(w[0] + acc[0], w[1] + acc[1]);
        o.y = pack_bf16x2(w[2] + acc[2], w[3] + acc[3]);
        o.z = pack_bf16x2(w[4] + acc[4], w[5] + acc[5]);
        o.w = pack_bf16x2(w[6] + acc[6], w[7] + acc[7]);
        if (active) {
          *reinterpret_cast<uint4*>(T.M + row * T.cols + c0) = o;
          m = umax(m, amax_bits8(o));
        }
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
// 4(l/16) .. 4(l/16)+3 of column l%16.
__global__ __launch_bounds__(256) void k_lora_dB(LoraArgs a, int accumulate) {
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;   // global wave
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && gw >= a.d[di + 1].dB_wave_begin) ++di;
  const LoraTensor& T = a.d[di];
  const int64_t row0 = (int64_t)(gw - T.dB_wave_begin) * 16;
  if (row0 >= T.rows) return;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t lr = lane & 15u, lk = lane >> 4;
  const int r = T.r;
  const int64_t grow = min(row0 + lr, T.rows - 1);               // rows past the end: clamp, not stored
  const uint16_t* gp = T.G + grow * T.cols + 8 * lk;
  const uint16_t* ap = T.A + (int64_t)min((int)lr, r - 1) * T.cols + 8 * lk;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int64_t j = 0; j < T.cols; j += 32) {
    const bf16x8_t g = *reinterpret_cast<const bf16x8_t*>(gp + j);
    const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(ap + j);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g, av, acc, 0, 0, 0);
  }
  // lane holds dB rows row0 + 4 lk + e (e = 0..3), adapter column lr
  if ((int)lr < r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = row0 + 4 * lk + e;
      if (row < T.rows) {
        float* dst = T.dB + row * r + lr;
        *dst = accumulate ? *dst + acc[e] : acc[e];
      }
    }
  }
}

// ------------------------------------------------------- dA = B^T . G ------
__global__ __launch_bounds__(256) void k_lora_dA(LoraArgs a) {
  const int b = blockIdx.x;
  int di = 0;
#pragma unroll 1
  while (di + 1 < a.n && b >= a.d[di + 1].dA_wg_begin) ++di;
  const LoraTensor& T = a.d[di];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = (b - T.dA_wg_begin) * 4 + wave;
  if (u >= T.dA_units) return;
  const int rb = u / T.slabs;
  const int64_t c0 = (int64_t)(u - rb * T.slabs) * LORA_SLAB + 8 * lane;
  const bool active = c0 < T.cols;
  const int r = T.r;
  float acc[LORA_MAX_R][8];
#pragma unroll
  for (int k = 0; k < LORA_MAX_R; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.0f;
  const int64_t r0 = (int64_t)rb * LORA_DA_ROWS;
  const int rows = (int)min((int64_t)LORA_DA_ROWS, T.rows - r0);
#pragma unroll 1
  for (int i = 0; i < rows; i += LORA_PREFETCH) {
    uint4 gv[LORA_PREFETCH];
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; ++q) {
      const int64_t row = r0 + min(i + q, rows - 1);
      gv[q] = active ? *reinterpret_cast<const uint4*>(T.G + row * T.cols + c0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < LORA_PREFETCH; ++q) {
      if (i + q >= rows) break;
      float bk[LORA_MAX_R];
      load_b_row(T.B, r0 + i + q, r, bk);
      float g[8];
      unpack8(gv[q], g);
#pragma unroll
      for (int k = 0; k < LORA_MAX_R; ++k) {
        if (k < r) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[k][e] = __builtin_fmaf(bk[k], g[e], acc[k][e]);
        }
      }
    }
  }
  if (active) {
    float* part = T.dA_partial + (int64_t)rb * LORA_MAX_R * T.cols;
#pragma unroll
    for (int k = 0; k < LORA_MAX_R; ++k) {
      if (k < r) {
        float4* p = reinterpret_cast<float4*>(part + (int64_t)k * T.cols + c0);
        p[0] = make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
        p[1] = make_float4(acc[k][4], acc[k][5], acc[k][6], acc[k][7]);
      }
    }
  }
}

// dA[k][j] (+)= sum over row blocks, in block order.
__global__ __launch_bounds__(256) void k_lora_dA_reduce(LoraArgs a, int accumulate) {
  const LoraTensor& T = a.d[blockIdx.y];
  const int64_t n = (int64_t)T.r * T.cols;
  const int nblk = (int)((T.rows + LORA_DA_ROWS - 1) / LORA_DA_ROWS);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = idx / T.cols, j = idx - k * T.cols;
    float s = 0.0f;
    for (int q = 0; q < nblk; ++q) s += T.dA_partial[((int64_t)q * LORA_MAX_R + k) * T.cols + j];
    T.dA[idx] = accumulate ? T.dA[idx] + s : s;
  }
}

// ------------------------------------------------------------ launchers ----
hipError_t launch_lora_merge(const LoraArgs& a, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lora_merge, dim3(grid), dim3(256), 0, s, a);
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
    hipLaunchKernelGGL(k_lora_dA, dim3(dA_grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lora_dA_reduce, dim3(64, a.n), dim3(256), 0, s, a, accumulate);
  }
  return hipGetLastError();
}

}  // namespace qf
