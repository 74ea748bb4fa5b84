// Transpose of a bf16 matrix, optionally MXFP4-QDQ'd on the way, for the backward
// products of a quantized linear layer (QATFactory project page, "Method",
// "Framework overview": the STE backward needs dX = dY . Wq and dWq = dY^T . Xq; the
// MXFP4 grid is the "Supported formats" table's).  The GEMM kernel multiplies A . B^T
// with both operands contiguous along the reduction axis, so dX takes Wq^T [K, N] and
// dWq takes dY^T [N, M] and Xq^T [K, M]; these come from one pass here.
//
// A workgroup of 256 lanes moves a 64-row x 128-column tile through LDS.  Reads: lane t
// takes the 16-byte chunks (t & 15) of rows (t >> 4) + 16 i (4 loads in flight), so an
// MXFP4 block of 32 source elements sits in 4 adjacent lanes and is quantized in
// registers exactly as k_mxfp4 does it; the chunk goes to LDS as four 32-bit words.
// Writes: lane t builds the 8 elements of output row (t >> 3) + 32 i, columns
// 8 (t & 7) .. +7, from 8 LDS half-word reads, and stores them as 16 bytes, so 8
// consecutive lanes write one whole 128-byte output row segment.  The LDS row pitch of
// 130 elements (65 words) puts the 8 source rows 8 apart that one read instruction
// touches on 8 different bank groups.
#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

constexpr int TR_ROWS = 64, TR_COLS = 128;               // source tile
constexpr int TR_PITCH = TR_COLS + 2;                      // elements (65 words): rows 4-byte aligned

// MXFP4 QDQ of one 16-byte chunk; lanes 4i..4i+3 hold one 32-element block (the rules of
// qf_qdq_mxfp4: E = max(bf16 exponent field of the block maximum - 2, 0); under NOCLIP one
// more when the maximum's significand exceeds 1.5, at most MX_NOCLIP_E_MAX).
template <bool NOCLIP>
__device__ __forceinline__ uint4 tr_mxfp4_qdq(uint4 w) {
  uint32_t m = amax_bits8(w);
  m = umax(m, dpp_xor1(m));
  m = umax(m, dpp_xor2(m));
  const int ef = (int)(m >> 7);
  int e2 = ef - 2 + (NOCLIP && (m & 0x7Fu) > 0x40u ? 1 : 0);
  if (NOCLIP) e2 = e2 < MX_NOCLIP_E_MAX ? e2 : MX_NOCLIP_E_MAX;
  const uint32_t E = (uint32_t)(e2 > 0 ? e2 : 0);
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
// first unless MODE is TR_COPY.  Grid: x over column tiles of src, y over row tiles.
template <int MODE>
__global__ __launch_bounds__(256) void k_transpose(const uint16_t* __restrict__ src, int64_t lds, int R, int C,
                                                   uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ __attribute__((aligned(16))) uint16_t t[TR_ROWS * TR_PITCH];
  uint32_t* tw = reinterpret_cast<uint32_t*>(t);
  const int r0 = blockIdx.y * TR_ROWS, c0 = blockIdx.x * TR_COLS;
  const uint32_t tid = threadIdx.x;
  constexpr int NL = TR_ROWS * TR_COLS / 8 / 256;          // 16-byte chunks per lane (4)
  uint4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = (int)(tid >> 4) + 16 * i, c = 8 * (int)(tid & 15u);
    v[i] = make_uint4(0, 0, 0, 0);
    if (r0 + r < R && c0 + c < C) {                        // read once: non-temporal
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t n = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + (int64_t)(r0 + r) * lds + c0 + c));
      v[i] = make_uint4(n.x, n.y, n.z, n.w);
    }
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = (int)(tid >> 4) + 16 * i, c = 8 * (int)(tid & 15u);
    const uint4 q = MODE == TR_COPY ? v[i] : tr_mxfp4_qdq<MODE == TR_QDQ_NOCLIP>(v[i]);
    uint32_t* row = tw + (r * TR_PITCH + c) / 2;
    row[0] = q.x;
    row[1] = q.y;
    row[2] = q.z;
    row[3] = q.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TR_COLS / 32; ++i) {
    const int j = (int)(tid >> 3) + 32 * i;                // output row = source column c0 + j
    const int q = 8 * (int)(tid & 7u);                     // output columns = source rows r0 + q ..
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(q + 2 * e) * TR_PITCH + j] | ((uint32_t)t[(q + 2 * e + 1) * TR_PITCH + j] << 16);
    if (c0 + j < C && r0 + q < R)
      *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + j) * ldd + r0 + q) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose(const uint16_t* src, int64_t lds, int R, int C, uint16_t* dst, int64_t ldd, int mode,
                            hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  // grid y is limited to 65535 row tiles: taller sources go in row bands of that many
  constexpr int BAND = 65535 * TR_ROWS;
  for (int rb = 0; rb < R; rb += BAND) {
    const int rn = R - rb < BAND ? R - rb : BAND;
    const dim3 g((unsigned)((C + TR_COLS - 1) / TR_COLS), (unsigned)((rn + TR_ROWS - 1) / TR_ROWS)), b(256);
    const uint16_t* sp = src + (int64_t)rb * lds;
    uint16_t* dp = dst + rb;                                 // the band's rows are output columns rb ..
    if (mode == TR_QDQ_FLOOR) hipLaunchKernelGGL(k_transpose<TR_QDQ_FLOOR>, g, b, 0, s, sp, lds, rn, C, dp, ldd);
    else if (mode == TR_QDQ_NOCLIP) hipLaunchKernelGGL(k_transpose<TR_QDQ_NOCLIP>, g, b, 0, s, sp, lds, rn, C, dp, ldd);
    else hipLaunchKernelGGL(k_transpose<TR_COPY>, g, b, 0, s, sp, lds, rn, C, dp, ldd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qf
