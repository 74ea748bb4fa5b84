// Dequantization of the engine-layout packed forms back to BF16: the read side of the
// export (QATFactory project page, "Method": weights leave training in the serving
// engine's own format; "Supported formats" table: the values each code and scale
// stand for).  Each kernel is the last step of the matching QDQ kernel applied to the
// stored bytes, so dequant(pack(x)) is bit for bit the QDQ'd bf16 of x.
//
// A lane handles 8 elements at a time: 4 code bytes in, one 16-byte bf16 store out (the
// Q4_K lane reads its 4 code bytes and the block's 16-byte header); consecutive lanes take
// consecutive elements of a row, so every load and store is coalesced.  The lanes of a
// block read its scale byte (or header) alike.
#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

constexpr int DQ_WG = 256;

// bf16 of E2M1 codes (8 per word, element e in nibble e) times s, then times s_t,
// each product rounded in fp32 (NVFP4: fl(fl(v s) s_t)).
__device__ __forceinline__ uint4 nvfp4_dequant8(uint32_t codes, float s, float s_t) {
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  uint4 o;
  o.x = pack_bf16x2((v0.x * s) * s_t, (v0.y * s) * s_t);
  o.y = pack_bf16x2((v1.x * s) * s_t, (v1.y * s) * s_t);
  o.z = pack_bf16x2((v2.x * s) * s_t, (v2.y * s) * s_t);
  o.w = pack_bf16x2((v3.x * s) * s_t, (v3.y * s) * s_t);
  return o;
}

// Chunk c (8 elements) of a contiguous [rows, cols] packed tensor has its codes at byte
// 4c and lies in row c / cpr; the output row has ldy elements.  A workgroup takes
// DQ_L x 256 chunks (Q4_K: DQ_L x 8 super-blocks), lane t the ones at t + 256 j, and
// issues all of its loads before the first store.  (Measured on the 8B layer: DQ_L = 2
// runs 2-4% faster than 4, and 1 or 8 slower.)
constexpr int DQ_L = 2;

template <bool NV>
__global__ __launch_bounds__(DQ_WG) void k_dequant_fp4(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, uint32_t nchunks,
                                                        uint32_t cpr, const float* __restrict__ d_scale,
                                                        uint16_t* __restrict__ y, int64_t ldy) {
  const uint32_t base = blockIdx.x * (DQ_WG * DQ_L) + threadIdx.x;
  uint32_t w[DQ_L], sb[DQ_L];
#pragma unroll
  for (int j = 0; j < DQ_L; ++j) {
    const uint32_t c = base + j * DQ_WG;
    w[j] = 0;
    sb[j] = 0;
    if (c < nchunks) {
      w[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes) + c);   // read once
      sb[j] = scales[NV ? c >> 1 : c >> 2];
    }
  }
  const float s_t = NV ? *d_scale : 0.0f;
#pragma unroll
  for (int j = 0; j < DQ_L; ++j) {
    const uint32_t c = base + j * DQ_WG;
    if (c >= nchunks) break;
    const uint32_t row = c / cpr, c8 = c - row * cpr;
    uint4 o;
    if constexpr (NV) {
      o = nvfp4_dequant8(w[j], e4m3_value(sb[j]), s_t);
    } else {
      // 2^(E - 127) with E in the scale operand's exponent field, as the QDQ kernel builds it
      const float sc = __uint_as_float(sb[j] << 23);
      o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 0));
      o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 1));
      o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 2));
      o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 3));
    }
    *reinterpret_cast<uint4*>(y + (int64_t)row * ldy + 8 * c8) = o;
  }
}

// Q4_K: lane l (0..31) of a super-block takes its elements 8l .. 8l+7, in sub-block l/4.
// Block bytes: 0-1 d and 2-3 dmin (fp16), 4-9 the eight 6-bit sc_j as one
// little-endian 48-bit field (sc_j at bit 6j), 10-15 the m_j likewise, then 128 bytes of
// codes with element 2i in the low nibble of byte 16+i.
__global__ __launch_bounds__(DQ_WG) void k_dequant_q4k(const uint8_t* __restrict__ blocks, uint32_t nsb_total,
                                                        uint32_t spr, uint16_t* __restrict__ y, int64_t ldy) {
  const uint32_t base = blockIdx.x * (DQ_WG * DQ_L) + threadIdx.x;
  const uint32_t l = threadIdx.x & 31u, j6 = 6u * (l >> 2);
  uint4 h[DQ_L];
  uint32_t q[DQ_L];
#pragma unroll
  for (int i = 0; i < DQ_L; ++i) {
    const uint32_t sb = (base + i * DQ_WG) >> 5;
    h[i] = make_uint4(0, 0, 0, 0);
    q[i] = 0;
    if (sb < nsb_total) {
      const uint8_t* blk = blocks + 144 * (int64_t)sb;
      h[i] = *reinterpret_cast<const uint4*>(blk);          // the 16-byte header
      q[i] = *reinterpret_cast<const uint32_t*>(blk + 16 + 4 * l);
    }
  }
#pragma unroll
  for (int i = 0; i < DQ_L; ++i) {
    const uint32_t sb = (base + i * DQ_WG) >> 5;
    if (sb >= nsb_total) break;
    // 6-bit field j of the 48-bit fields starting at header bits 32 (sc) and 80 (m)
    const uint64_t scf = ((uint64_t)h[i].y) | ((uint64_t)(h[i].z & 0xFFFFu) << 32);
    const uint64_t mf = ((uint64_t)(h[i].z >> 16)) | ((uint64_t)h[i].w << 16);
    const uint32_t sc = (uint32_t)(scf >> j6) & 63u, m = (uint32_t)(mf >> j6) & 63u;
    const float D = f16_value_hw(h[i].x & 0xFFFFu) * (float)sc;   // exact (<= 17 significant bits)
    const float M = f16_value_hw(h[i].x >> 16) * (float)m;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = D * (float)((q[i] >> (4 * e)) & 15u) - M;   // D q exact: one rounding
    const uint32_t row = sb / spr, s = sb - row * spr;
    uint4 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]);
    v.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(y + (int64_t)row * ldy + 256 * s + 8 * l) = v;
  }
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          const float* d_scale, uint16_t* y, int64_t ldy, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t per_wg = (int64_t)DQ_WG * DQ_L;
  if (fmt == QF_FMT_NVFP4 || fmt == QF_FMT_MXFP4) {
    const int64_t n = rows * (cols / 8);                  // < 2^32 - per_wg (checked by the caller)
    const dim3 g((unsigned)((n + per_wg - 1) / per_wg)), b(DQ_WG);
    if (fmt == QF_FMT_NVFP4)
      hipLaunchKernelGGL(k_dequant_fp4<true>, g, b, 0, s, codes, scales, (uint32_t)n, (uint32_t)(cols / 8), d_scale,
                         y, ldy);
    else
      hipLaunchKernelGGL(k_dequant_fp4<false>, g, b, 0, s, codes, scales, (uint32_t)n, (uint32_t)(cols / 8), d_scale,
                         y, ldy);
  } else {
    const int64_t nsb = rows * (cols / 256);
    hipLaunchKernelGGL(k_dequant_q4k, dim3((unsigned)((32 * nsb + per_wg - 1) / per_wg)), dim3(DQ_WG), 0, s, codes,
                       (uint32_t)nsb, (uint32_t)(cols / 256), y, ldy);
  }
  return hipGetLastError();
}

}  // namespace qf
