// Transpose of a bf16 matrix, optionally MXFP4-QDQ'd on the way, for the backward
// products of a quantized linear layer (QATFactory project page, "Method",
// "Framework overview": the STE backward needs dX = dY . Wq and dWq = dY^T . Xq; the
// MXFP4 grid is the "Supported formats" table's).  The GEMM kernel multiplies A . B^T
// with both operands contiguous along the reduction axis, so dX takes Wq^T [K, N] and
// dWq takes dY^T [N, M] and Xq^T [K, M]; these come from one pass here.
//
// A workgroup of 256 lanes moves a 64 x 64 tile through LDS.  Reads: lane t takes the
// 16-byte chunks (t & 7) of rows (t >> 3) + 32 i, so an MXFP4 block of 32 source
// elements sits in 4 adjacent lanes and is quantized in registers exactly as k_mxfp4
// does it.  Writes: lane t builds the 8 elements of output row (t & 63), columns
// 8 (t >> 6) + 32 i .. +7, from 8 LDS half-word reads (a wave's reads cover 64
// consecutive columns of one LDS row: no bank conflicts), and stores them as 16 bytes.
#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

constexpr int TR_TILE = 64;
constexpr int TR_PITCH = TR_TILE + 8;                      // elements; rows stay 16-byte aligned

// MXFP4 QDQ of one 16-byte chunk; lanes 4i..4i+3 hold one 32-element block (the rule of
// qf_qdq_mxfp4: E = max(bf16 exponent field of the block maximum - 2, 0)).
__device__ __forceinline__ uint4 tr_mxfp4_qdq(uint4 w) {
  uint32_t m = amax_bits8(w);
  m = umax(m, dpp_xor1(m));
  m = umax(m, dpp_xor2(m));
  const int ef = (int)(m >> 7);
  const uint32_t E = (uint32_t)(ef > 2 ? ef - 2 : 0);
  const float sc = __uint_as_float(E << 23);
  uint32_t codes = 0;
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

// dst [C, R] (row stride ldd) = src [R, C] (row stride lds) transposed, QDQ'd along C
// first when QDQ.  Grid: x over column tiles of src, y over row tiles.
template <bool QDQ>
__global__ __launch_bounds__(256) void k_transpose(const uint16_t* __restrict__ src, int64_t lds, int R, int C,
                                                   uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ __attribute__((aligned(16))) uint16_t t[TR_TILE * TR_PITCH];
  const int r0 = blockIdx.y * TR_TILE, c0 = blockIdx.x * TR_TILE;
  const uint32_t tid = threadIdx.x;
  uint4 v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (int)(tid >> 3) + 32 * i, c = 8 * (int)(tid & 7u);
    v[i] = make_uint4(0, 0, 0, 0);
    if (r0 + r < R && c0 + c < C) v[i] = *reinterpret_cast<const uint4*>(src + (int64_t)(r0 + r) * lds + c0 + c);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (int)(tid >> 3) + 32 * i, c = 8 * (int)(tid & 7u);
    *reinterpret_cast<uint4*>(t + r * TR_PITCH + c) = QDQ ? tr_mxfp4_qdq(v[i]) : v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = (int)(tid & 63u);                        // output row = source column c0 + j
    const int q = 8 * ((int)(tid >> 6) + 4 * i);           // output columns = source rows r0 + q ..
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(q + 2 * e) * TR_PITCH + j] | ((uint32_t)t[(q + 2 * e + 1) * TR_PITCH + j] << 16);
    if (c0 + j < C && r0 + q < R)
      *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + j) * ldd + r0 + q) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose(const uint16_t* src, int64_t lds, int R, int C, uint16_t* dst, int64_t ldd, bool qdq,
                            hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 g((unsigned)((C + TR_TILE - 1) / TR_TILE), (unsigned)((R + TR_TILE - 1) / TR_TILE)), b(256);
  if (qdq) hipLaunchKernelGGL(k_transpose<true>, g, b, 0, s, src, lds, R, C, dst, ldd);
  else hipLaunchKernelGGL(k_transpose<false>, g, b, 0, s, src, lds, R, C, dst, ldd);
  return hipGetLastError();
}

}  // namespace qf
