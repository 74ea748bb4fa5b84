// Clipped straight-through estimator for the FP4 grids: the gradient of the latent weight
// is the gradient of the QDQ'd weight where the quantizer kept the element inside its grid,
// and +0.0 where it saturated it (QATFactory project page, "Method", "Framework
// overview": the backward pass reaches the latent weights through an STE; the saturation
// follows from the "Supported formats" table's E2M1 grid, whose largest magnitude is 6).
//
// An element saturates when its scaled magnitude exceeds 6:
//   NVFP4: y = fl(|x| r) > 6 with the block's r = fl(1/d), d = fl(s s_t), the values the QDQ
//          kernel computes (a block with d = 0 and a zero element never saturate);
//   MXFP4: |x| > 6 * 2^(E-127) with the block's shared exponent E under the floor or the
//          noclip rule (y = |x| / 2^(E-127) is exact, so this is the QDQ's own decision).
//
// A wave takes 64 consecutive 8-element chunks (512 elements of the row-major [rows, cols]
// numbering) at a time, in two halves: in half h lane l takes elements 256h + 4l .. +3 of
// them (8-byte loads of x, row stride ldx, and of g_q; one 16-byte fp32 store), so every
// store instruction writes 1 KiB of contiguous output (8 elements per lane with two stores
// 32 bytes apart measured slower on the STE).  An NVFP4 block then sits in 4 adjacent
// lanes and an MXFP4 block in 8, and the block maximum is two or three DPP steps.
#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

constexpr int SC_WG = 256;
constexpr int SC_L = 1;                                    // 64-chunk segments per wave (2: 8% slower, 4: 16%)

template <int FMT, bool ACC, bool NOCLIP>
__global__ __launch_bounds__(SC_WG) void k_ste_clip(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                                    int64_t ldx, uint32_t nchunks, uint32_t cpr,
                                                    const float* __restrict__ d_scale, float* __restrict__ out) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wbase = blockIdx.x * (SC_WG * SC_L) + (threadIdx.x & ~63u);   // the wave's first chunk
  const float s_t = FMT == QF_FMT_NVFP4 ? *d_scale : 0.0f, k6 = 6.0f * s_t;
#pragma unroll
  for (int j = 0; j < SC_L; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = wbase + j * SC_WG + 32 * h + (lane >> 1), half = lane & 1u;
      if (c >= nchunks) break;                             // the same for all lanes of a quantization block
      const uint32_t row = c / cpr, c8 = c - row * cpr;
      // both read once: non-temporal
      const u32x2_t wn = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(x + (int64_t)row * ldx + 8 * c8 + 4 * half));
      const u32x2_t gn = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(g + (int64_t)c * 8 + 4 * half));
      const uint32_t wv[2] = {wn.x, wn.y};
      uint32_t m = amax_bits8(make_uint4(wn.x, wn.y, 0u, 0u));
      m = umax(m, dpp_xor1(m));
      m = umax(m, dpp_xor2(m));                            // NVFP4 block: 4 lanes
      bool sat[4];
      if constexpr (FMT == QF_FMT_NVFP4) {
        const float s = e4m3_value(e4m3_encode(__uint_as_float(m << 16) / k6));
        const float d = s * s_t;
        const float r = (d == 0.0f) ? 0.0f : 1.0f / d;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float lo = fabsf(bf16_lo(wv[e])), hi = fabsf(bf16_hi(wv[e]));
          sat[2 * e] = d != 0.0f && lo != 0.0f && lo * r > 6.0f;
          sat[2 * e + 1] = d != 0.0f && hi != 0.0f && hi * r > 6.0f;
        }
      } else {
        m = umax(m, dpp_hmirror(m));                       // MXFP4 block: 8 lanes
        // E = max(bf16 exponent field of the block maximum - 2 (+1 under noclip when its
        // significand exceeds 1.5, capped at 252), 0); the limit 6 * 2^(E-127) =
        // 1.5 * 2^(E-125) is exact for E <= 252 and beyond every finite bf16 above that
        const int ef = (int)(m >> 7);
        int E = ef - 2 + (NOCLIP && (m & 0x7Fu) > 0x40u ? 1 : 0);
        if (NOCLIP) E = E < MX_NOCLIP_E_MAX ? E : MX_NOCLIP_E_MAX;
        E = E < 0 ? 0 : E;
        const float lim = E + 2 >= 255 ? __builtin_inff() : __uint_as_float(((uint32_t)(E + 2) << 23) | 0x400000u);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          sat[2 * e] = fabsf(bf16_lo(wv[e])) > lim;
          sat[2 * e + 1] = fabsf(bf16_hi(wv[e])) > lim;
        }
      }
      float4 a = make_float4(sat[0] ? 0.0f : bf16_lo(gn.x), sat[1] ? 0.0f : bf16_hi(gn.x),
                             sat[2] ? 0.0f : bf16_lo(gn.y), sat[3] ? 0.0f : bf16_hi(gn.y));
      float4* o = reinterpret_cast<float4*>(out + (int64_t)c * 8 + 4 * half);
      if constexpr (ACC) {
        const float4 p = o[0];
        a.x += p.x; a.y += p.y; a.z += p.z; a.w += p.w;
      }
      o[0] = a;
    }
  }
}

hipError_t launch_ste_clip(int fmt, int mx_rule, const uint16_t* g, const uint16_t* x, int64_t rows, int64_t cols,
                           int64_t ldx, const float* d_scale, float* out, bool acc, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t n = rows * (cols / 8);                    // < 2^32 - 4096 (checked by the caller)
  const dim3 gr((unsigned)((n + SC_WG * SC_L - 1) / (SC_WG * SC_L))), b(SC_WG);
  const uint32_t nc = (uint32_t)n, cpr = (uint32_t)(cols / 8);
#define QF_STE_CLIP(F, A, N) hipLaunchKernelGGL((k_ste_clip<F, A, N>), gr, b, 0, s, g, x, ldx, nc, cpr, d_scale, out)
  if (fmt == QF_FMT_NVFP4) {
    if (acc) QF_STE_CLIP(QF_FMT_NVFP4, true, false);
    else QF_STE_CLIP(QF_FMT_NVFP4, false, false);
  } else if (mx_rule == QF_MX_RULE_NOCLIP) {
    if (acc) QF_STE_CLIP(QF_FMT_MXFP4, true, true);
    else QF_STE_CLIP(QF_FMT_MXFP4, false, true);
  } else {
    if (acc) QF_STE_CLIP(QF_FMT_MXFP4, true, false);
    else QF_STE_CLIP(QF_FMT_MXFP4, false, false);
  }
#undef QF_STE_CLIP
  return hipGetLastError();
}

}  // namespace qf
