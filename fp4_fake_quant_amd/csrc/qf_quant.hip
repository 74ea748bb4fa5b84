// Memory-bound kernels of the simulated-quantization hot path on gfx950:
// NVFP4 tensor amax (pass 1) and its reduction to tied-group FP32 scales,
// block QDQ + engine-layout packing for NVFP4 / MXFP4 / Q4_K (one pass over
// the input, any subset of {QDQ'd bf16, packed codes + scales}), the identity
// STE backward, and the device self-test of the conversion instructions.
//
// What is computed: QATFactory project page, "Method" (QDQ forward, STE
// backward, tied NVFP4 tensor scales for fused projections, engine-layout
// export) and the "Supported formats" table.  Bit-level rules: include/qf.h.
//
// Layout of the work: a workgroup of 256 lanes owns a tile of 256 * L chunks of
// 8 bf16 (16 bytes); lane t handles chunks t, t+256, ..., t+256(L-1) of the
// tile, issuing all L 128-bit loads before any arithmetic.  A quantization
// block therefore sits in 2 (NVFP4), 4 (MXFP4) or 32 (Q4_K) adjacent lanes and
// its statistics are reduced with DPP row operations (and one ds_swizzle for
// the 32-lane Q4_K super-block); no LDS and no barriers are needed.
#include <float.h>

#include "qf_device.h"
#include "qf_kernels.h"

namespace qf {

__device__ __forceinline__ int find_tensor(const QArgs& a, int b) {
  int i = 0;
#pragma unroll 1
  while (i + 1 < a.n && b >= a.t[i + 1].tile_begin) ++i;
  return i;
}

// Element offset of chunk c of a [rows, cols] tensor with row stride ld.
__device__ __forceinline__ uint64_t chunk_offset(uint32_t c, uint32_t cpr, int64_t ld, int contig) {
  if (contig) return (uint64_t)c * 8u;
  uint32_t row = c / cpr;
  uint32_t col8 = c - row * cpr;
  return (uint64_t)row * (uint64_t)ld + (uint64_t)col8 * 8u;
}

__device__ __forceinline__ uint4 load_chunk(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// Non-temporal, for the NVFP4 step's kernels (amax, QDQ+pack, STE; every input is read
// once).  Measured on the dense 8B step: 0.481 -> 0.456 ms; with plain loads the amax pass
// paid for writing back the previous kernel's dirty lines (121 us against 77 us now).  The
// MXFP4 and Q4_K kernels keep plain loads: nt measured 2-3% slower on their workloads.
__device__ __forceinline__ uint4 load_chunk_nt(const uint16_t* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// -------------------------------------------------- NVFP4 pass 1: amax -----
// Persistent grid: workgroup w walks tiles w, w + grid, ...; every wave folds
// its tile maximum into an LDS slot of the tile's tied group; at the end the
// workgroup writes one maximum per group to partial[g * grid + w].
__device__ __forceinline__ uint32_t wave_umax(uint32_t m) {
  m = umax(m, dpp_xor1(m));
  m = umax(m, dpp_xor2(m));
  m = umax(m, dpp_hmirror(m));
  m = umax(m, dpp_mirror(m));
  m = umax(m, swz_xor16(m));
  return umax((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 32));
}

template <int L>
__global__ __launch_bounds__(WG) void k_nvfp4_amax(QArgs a) {
  __shared__ uint32_t gmax[QF_MAX_GROUPS];
  for (int g = threadIdx.x; g < a.n_groups; g += WG) gmax[g] = 0;
  __syncthreads();
  for (int b = blockIdx.x; b < a.total_tiles; b += gridDim.x) {
    const int ti = find_tensor(a, b);
    const QTensor& T = a.t[ti];
    const uint32_t base = (uint32_t)(b - T.tile_begin) * (WG * L);
    uint4 w[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const uint32_t c = base + j * WG + threadIdx.x;
      w[j] = make_uint4(0, 0, 0, 0);
      if (c < T.nchunks) w[j] = load_chunk_nt(T.x + chunk_offset(c, T.cpr, T.ldx, T.contig_x));
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) m = umax(m, amax_bits8(w[j]));
    m = wave_umax(m);
    if ((threadIdx.x & 63) == 0 && m) atomicMax(&gmax[T.group], m);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < a.n_groups; g += WG) a.partial[g * gridDim.x + blockIdx.x] = gmax[g];
}

// One workgroup of 1024 lanes: per-group maximum of the partials (every load of
// a lane issued before any is used), then the tensor scale of every group.
constexpr int RED_WG = 1024;
__global__ __launch_bounds__(RED_WG) void k_nvfp4_scale_reduce(ReduceArgs a) {
  __shared__ uint32_t gmax[QF_MAX_GROUPS];
  for (int g = threadIdx.x; g < a.n_groups; g += RED_WG) gmax[g] = 0;
  __syncthreads();
  const int total = a.n_partial_groups * a.grid;
  for (int i0 = threadIdx.x; i0 < total; i0 += 8 * RED_WG) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k * RED_WG;
      v[k] = i < total ? a.partial[i] : 0u;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k * RED_WG;
      if (v[k]) atomicMax(&gmax[i / a.grid], v[k]);
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < a.n_groups; g += RED_WG) {
    const uint32_t bits = gmax[g];
    if (bits >= 0x7F80u && a.nonfinite) *a.nonfinite = 1u;
    uint32_t abits = bits << 16;                           // |x| max as fp32 bits (exact)
    if (a.tracked) {
      // running maximum over calls: the integer max of non-negative fp32 bit patterns is
      // their numeric max (a NaN pattern wins and stays, which the flag reports)
      const uint32_t prev = __float_as_uint(a.tracked[g]) & 0x7FFFFFFFu;
      abits = abits > prev ? abits : prev;
      a.tracked[g] = __uint_as_float(abits);
    }
    const float A = __uint_as_float(abits);
    a.tscale[g] = (A == 0.0f) ? 1.0f : A / 2688.0f;
  }
}

// ------------------------------------------------- NVFP4 pass 2: QDQ -------
// Lanes 2i and 2i+1 hold one 16-block.
template <bool WY, bool WP, int L>
__global__ __launch_bounds__(WG) void k_nvfp4(QArgs a) {
  // last tiles first: they are the ones the amax pass read last, so part of them
  // is still in the memory-side cache
  const int b = a.total_tiles - 1 - (int)blockIdx.x;
  const int ti = find_tensor(a, b);
  const QTensor& T = a.t[ti];
  const uint32_t base = (uint32_t)(b - T.tile_begin) * (WG * L);
  const float s_t = a.tscale[T.group];
  const float k = 6.0f * s_t;
  uint4 w[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    w[j] = make_uint4(0, 0, 0, 0);
    if (c < T.nchunks) w[j] = load_chunk_nt(T.x + chunk_offset(c, T.cpr, T.ldx, T.contig_x));
  }
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    const Nvfp4Chunk q = nvfp4_qdq_chunk(w[j], s_t, k);
    if (c < T.nchunks) {
      if (WY) *reinterpret_cast<uint4*>(T.y + chunk_offset(c, T.cpr, T.ldy, T.contig_y)) = q.y;
      if (WP) {
        reinterpret_cast<uint32_t*>(T.codes)[c] = q.codes;
        if ((threadIdx.x & 1) == 0) T.scales[c >> 1] = (uint8_t)q.S;
      }
    }
  }
}

// ---------------------------------------------------------------- MXFP4 ----
// Lanes 4i..4i+3 hold one 32-block.  NOCLIP selects the noclip shared-exponent rule.
template <bool WY, bool WP, int L, bool NOCLIP = false>
__global__ __launch_bounds__(WG) void k_mxfp4(QArgs a) {
  const int b = blockIdx.x;
  const int ti = find_tensor(a, b);
  const QTensor& T = a.t[ti];
  const uint32_t base = (uint32_t)(b - T.tile_begin) * (WG * L);
  uint4 w[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    w[j] = make_uint4(0, 0, 0, 0);
    if (c < T.nchunks) w[j] = load_chunk(T.x + chunk_offset(c, T.cpr, T.ldx, T.contig_x));
  }
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    uint32_t m = amax_bits8(w[j]);
    m = umax(m, dpp_xor1(m));
    m = umax(m, dpp_xor2(m));
    // E = floor(log2 amax) - 2 + 127 clamped to [0, 254]: the bf16 exponent field minus 2
    // (0 for zero and subnormal maxima, whose floor(log2) is below -126).  Noclip: the
    // smallest E with amax <= 6 * 2^(E-127), one more than that when the maximum's
    // significand exceeds 1.5 (mantissa field above 0x40), at most 252 (the last E whose
    // grid top 6 * 2^(E-127) is a finite bf16).
    const int ef = (int)(m >> 7);
    int e2 = NOCLIP ? ef - 2 + ((m & 0x7Fu) > 0x40u ? 1 : 0) : ef - 2;
    if (NOCLIP) e2 = e2 < MX_NOCLIP_E_MAX ? e2 : MX_NOCLIP_E_MAX;
    const uint32_t E = (uint32_t)(e2 > 0 ? e2 : 0);
    const float sc = __uint_as_float(E << 23);
    uint32_t codes = 0;
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w[j].x), sc, 0);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w[j].y), sc, 1);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w[j].z), sc, 2);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes, __builtin_bit_cast(bf16x2_t, w[j].w), sc, 3);
    if (c < T.nchunks) {
      if (WY) {
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
        *reinterpret_cast<uint4*>(T.y + chunk_offset(c, T.cpr, T.ldy, T.contig_y)) = o;
      }
      if (WP) {
        reinterpret_cast<uint32_t*>(T.codes)[c] = codes;
        if ((threadIdx.x & 3) == 0) T.scales[c >> 2] = (uint8_t)E;
      }
    }
  }
}

// ----------------------------------------------------------------- Q4_K ----
// Lanes 32i..32i+31 hold one 256 super-block; lanes 4j..4j+3 of it sub-block j.
__device__ __forceinline__ float fbits(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t ubits(float f) { return __float_as_uint(f); }

// MSE: the sub-block scale is the best of 8 shrunken min/max scales, base (1 - k/16) for
// k = 0..7, by the squared error of the sub-block quantized with it and the offset -mn:
// each lane sums its 8 elements' squared errors in index order, the quad adds the four
// partials as (lane 0 + lane 1) + (lane 2 + lane 3) (DPP xor 1, then xor 2; every lane
// gets the same total), and the first smallest total wins.  All steps are single fp32
// operations, so the choice is bit for bit the oracle's.
template <bool WY, bool WP, int L, bool MSE = false>
__global__ __launch_bounds__(WG) void k_q4k(QArgs a) {
  const int b = blockIdx.x;
  const int ti = find_tensor(a, b);
  const QTensor& T = a.t[ti];
  const uint32_t base = (uint32_t)(b - T.tile_begin) * (WG * L);
  const uint32_t lane32 = threadIdx.x & 31u;
  const uint32_t sub = lane32 >> 2;
  uint4 w[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    w[j] = make_uint4(0, 0, 0, 0);
    if (c < T.nchunks) w[j] = load_chunk(T.x + chunk_offset(c, T.cpr, T.ldx, T.contig_x));
  }
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const uint32_t c = base + j * WG + threadIdx.x;
    const uint32_t wv[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
    float xv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[2 * e] = bf16_lo(wv[e]);
      xv[2 * e + 1] = bf16_hi(wv[e]);
    }
    float mn = xv[0], mx = xv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      mn = fminf(mn, xv[e]);
      mx = fmaxf(mx, xv[e]);
    }
    mn = fminf(mn, fbits(dpp_xor1(ubits(mn))));
    mn = fminf(mn, fbits(dpp_xor2(ubits(mn))));
    mx = fmaxf(mx, fbits(dpp_xor1(ubits(mx))));
    mx = fmaxf(mx, fbits(dpp_xor2(ubits(mx))));
    mn = fminf(mn, 0.0f);
    if (mn == 0.0f) mn = 0.0f;        // a zero extreme counts as +0
    if (mx == 0.0f) mx = 0.0f;
    float scale = div15(mx - mn);
    if constexpr (MSE) {
      const float base = scale;
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = xv[e] - mn;
      float best = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float sk = base * (1.0f - (float)k / 16.0f);
        const float rk = (sk == 0.0f) ? 0.0f : 1.0f / sk;
        float p = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qe = fminf(fmaxf(__builtin_rintf(t[e] * rk), 0.0f), 15.0f);
          const float de = (qe * sk + mn) - xv[e];           // two roundings: no contraction
          p = e == 0 ? de * de : p + de * de;
        }
        float tot = p + fbits(dpp_xor1(ubits(p)));
        tot = tot + fbits(dpp_xor2(ubits(tot)));
        if (k == 0 || tot < best) {
          best = tot;
          scale = sk;
        }
      }
    }
    const float off = 0.0f - mn;
    // super-block maxima of the (non-negative) scales and offsets: unsigned max on bits
    uint32_t sb = ubits(scale), ob = ubits(off);
    sb = umax(sb, dpp_hmirror(sb));
    ob = umax(ob, dpp_hmirror(ob));
    sb = umax(sb, dpp_mirror(sb));
    ob = umax(ob, dpp_mirror(ob));
    sb = umax(sb, swz_xor16(sb));
    ob = umax(ob, swz_xor16(ob));
    // Lanes of a quad share the work: lane 0 derives d (from the largest scale), lane 1
    // dmin (from the largest offset), in one division and one fp16 conversion ...
    const bool odd = (threadIdx.x & 1u) != 0;
    const uint32_t h = f16_bits_sat_hw(div63(fbits(odd ? ob : sb)));
    const float d = f16_value_hw(quad_bcast0(h)), dmin = f16_value_hw(quad_bcast1(h));
    const uint32_t dh = f16_bits_of(d), dmh = f16_bits_of(dmin);
    // ... then lane 0 rounds scale / d to sc and lane 1 off / dmin to m, in one division.
    const float num = odd ? off : scale, den = odd ? dmin : d;
    const float t63 = (den == 0.0f) ? 0.0f : fminf(fmaxf(__builtin_rintf(num / den), 0.0f), 63.0f);
    const float scq = fbits(quad_bcast0(ubits(t63))), mq = fbits(quad_bcast1(ubits(t63)));
    const float D = d * scq, M = dmin * mq;
    const float r = (D == 0.0f) ? 0.0f : 1.0f / D;
    uint32_t qword = 0;
    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] = fminf(fmaxf(__builtin_rintf((xv[e] + M) * r), 0.0f), 15.0f);
      qword |= (uint32_t)q[e] << (4 * e);
    }
    if (WP) {
      // 96-bit scale stream: sc_j at bits 6j, m_j at bits 48 + 6j; OR over the super-block
      const uint64_t A = (uint64_t)(uint32_t)scq << (6 * sub);
      const uint64_t Bm = (uint64_t)(uint32_t)mq << (6 * sub);
      const uint64_t lo = A | (Bm << 48);
      uint32_t s0 = (uint32_t)lo, s1 = (uint32_t)(lo >> 32), s2 = (uint32_t)(Bm >> 16);
      s0 |= dpp_hmirror(s0); s1 |= dpp_hmirror(s1); s2 |= dpp_hmirror(s2);
      s0 |= dpp_mirror(s0);  s1 |= dpp_mirror(s1);  s2 |= dpp_mirror(s2);
      s0 |= swz_xor16(s0);   s1 |= swz_xor16(s1);   s2 |= swz_xor16(s2);
      if (c < T.nchunks) {
        uint8_t* blk = T.codes + (uint64_t)(c >> 5) * 144u;
        reinterpret_cast<uint32_t*>(blk + 16)[lane32] = qword;
        if (lane32 == 0) *reinterpret_cast<uint4*>(blk) = make_uint4(dh | (dmh << 16), s0, s1, s2);
      }
    }
    if (WY && c < T.nchunks) {
      uint4 o;
      o.x = pack_bf16x2(__builtin_fmaf(D, q[0], -M), __builtin_fmaf(D, q[1], -M));
      o.y = pack_bf16x2(__builtin_fmaf(D, q[2], -M), __builtin_fmaf(D, q[3], -M));
      o.z = pack_bf16x2(__builtin_fmaf(D, q[4], -M), __builtin_fmaf(D, q[5], -M));
      o.w = pack_bf16x2(__builtin_fmaf(D, q[6], -M), __builtin_fmaf(D, q[7], -M));
      *reinterpret_cast<uint4*>(T.y + chunk_offset(c, T.cpr, T.ldy, T.contig_y)) = o;
    }
  }
}

// ------------------------------------------------------------------ STE ----
// Identity STE: bf16 gradients -> fp32, optionally accumulated.  A wave owns 512
// consecutive elements; lane l takes elements 4l..4l+3 and 256+4l..256+4l+3 of them (two
// 8-byte loads, two 16-byte stores), so each store instruction writes 1 KiB of contiguous
// output.  With 8 elements per lane (one 16-byte load, two 16-byte stores 32 bytes apart)
// every store instruction covered half of each of 16 lines: 222 -> 208 us on the dense 8B
// layer (218 M elements).  The launcher gives each workgroup WG * 8 elements.
template <bool ACC, int L>
__global__ __launch_bounds__(WG) void k_ste(const uint16_t* __restrict__ g, float* __restrict__ out, int64_t n) {
  static_assert(L == 1, "one 512-element segment per wave");
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const int64_t ne = (n >> 3) << 3;                        // elements in whole 8-element chunks
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wbase = ((int64_t)blockIdx.x * WG + (threadIdx.x & ~63u)) * 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t e = wbase + 256 * h + 4 * lane;
    if (e < ne) {                                         // e + 4 <= ne: e and ne are multiples of 4
      const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(g + e));   // read once
      float4 v = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
      float4* o = reinterpret_cast<float4*>(out + e);
      if (ACC) {
        const float4 p = o[0];
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
      }
      o[0] = v;
    }
  }
  // ragged tail (n % 8 elements) handled by the first lanes of the first workgroup
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t i = ne + threadIdx.x;
    const float v = __uint_as_float((uint32_t)g[i] << 16);
    out[i] = ACC ? out[i] + v : v;
  }
}

// ------------------------------------------------------ conformance test ---
__device__ __forceinline__ uint32_t sw_e2m1(float y) {   // code of y (sign from y), RNE, saturating
  const float a = fabsf(y);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return m | ((__float_as_uint(y) >> 31) << 3);
}
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float v = m == 0 ? 0.f : m == 1 ? .5f : m == 2 ? 1.f : m == 3 ? 1.5f : m == 4 ? 2.f : m == 5 ? 3.f : m == 6 ? 4.f : 6.f;
  return (c & 8u) ? -v : v;
}

// counts[0]: v_cvt_pk_bf16_f32 over every finite fp32 (2^28 patterns per launch)
// counts[1]: v_cvt_scalef32_pk_fp4_f32 with scale 1.0 over every non-NaN fp32
__global__ __launch_bounds__(WG) void k_self_fp32(uint32_t base, unsigned long long* counts) {
  const uint32_t bits = base + blockIdx.x * WG + threadIdx.x;
  const float f = __uint_as_float(bits);
  uint32_t bad0 = 0, bad1 = 0;
  if (fabsf(f) <= 3.3895313e38f) {                          // finite, no bf16 overflow
    bad0 = pack_bf16x2(f, -f) != (bf16_rne_sw(f) | (bf16_rne_sw(-f) << 16));
  }
  if (f == f) bad1 = (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f, -f, 1.0f, 0) & 0xFFu) !=
                     (sw_e2m1(f) | (sw_e2m1(-f) << 4));
  if (bad0) atomicAdd(&counts[0], 1ull);
  if (bad1) atomicAdd(&counts[1], 1ull);
}

// counts[6]: v_cvt_f16_f32 with clamp vs the software fp16 conversion, every x >= 0 finite
// counts[7]: FMA-corrected division by 15 and by 63 vs IEEE division, every x >= 0 finite
__global__ __launch_bounds__(WG) void k_self_nonneg(uint32_t base, unsigned long long* counts) {
  const uint32_t bits = base + blockIdx.x * WG + threadIdx.x;     // base < 2^31: x >= 0
  const float x = __uint_as_float(bits);
  if (!(x <= FLT_MAX)) return;
  if (f16_bits_sat_hw(x) != f16_bits_sat(x)) atomicAdd(&counts[6], 1ull);
  if (bits < 0x7C00u && __float_as_uint(f16_value_hw(bits)) != __float_as_uint(f16_value(bits)))
    atomicAdd(&counts[6], 1ull);
  if (__float_as_uint(div15(x)) != __float_as_uint(x / 15.0f) ||
      __float_as_uint(div63(x)) != __float_as_uint(x / 63.0f)) atomicAdd(&counts[7], 1ull);
}

// counts[2], counts[3]: E8M0-scaled bf16 / f32 -> E2M1 over every bf16 and every E
// counts[4], counts[5]: E8M0-scaled E2M1 -> bf16 / f32 over every code and E
__global__ __launch_bounds__(WG) void k_self_scaled(unsigned long long* counts) {
  const uint32_t E = blockIdx.y;                           // 0..254
  const uint32_t hb = blockIdx.x * WG + threadIdx.x;       // 0..65535
  const float x = __uint_as_float(hb << 16);
  const float sc = __uint_as_float(E << 23);
  const float X = ldexpf(1.0f, (int)E - 127);
  if (x == x && fabsf(x) <= FLT_MAX) {
    const uint32_t want = sw_e2m1(x / X);
    const bf16x2_t v = __builtin_bit_cast(bf16x2_t, hb | (hb << 16));
    if ((__builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, v, sc, 0) & 15u) != want) atomicAdd(&counts[2], 1ull);
    if ((__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, x, sc, 0) & 15u) != want) atomicAdd(&counts[3], 1ull);
  }
  if (hb < 16) {
    const float want = e2m1_value(hb) * X;
    const uint32_t code = hb | (hb << 4);
    const uint32_t gb = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 0));
    if (gb != (bf16_rne_sw(want) * 0x10001u)) atomicAdd(&counts[4], 1ull);
    const f32x2_t gf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, sc, 0);
    if (__float_as_uint(gf.x) != __float_as_uint(want) || __float_as_uint(gf.y) != __float_as_uint(want))
      atomicAdd(&counts[5], 1ull);
    const f32x2_t g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
    if (__float_as_uint(g1.x) != __float_as_uint(e2m1_value(hb))) atomicAdd(&counts[5], 1ull);
  }
}

// ------------------------------------------------------------- launchers ---
hipError_t launch_nvfp4_amax(const QArgs& a, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_nvfp4_amax<L_AMAX>, dim3(amax_grid(a.total_tiles)), dim3(WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_nvfp4_scale_reduce(const ReduceArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_nvfp4_scale_reduce, dim3(1), dim3(RED_WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant(int fmt, bool wy, bool wp, const QArgs& a, hipStream_t s, int mx_rule) {
  // mx_rule: QF_MX_RULE_* for MXFP4, QF_Q4K_RULE_* for Q4_K
  if (a.total_tiles == 0) return hipSuccess;
  const dim3 g(a.total_tiles), blk(WG);
#define QF_DISPATCH(KERNEL, ...)                                                              \
  if (wy && wp) hipLaunchKernelGGL((KERNEL<true, true, __VA_ARGS__>), g, blk, 0, s, a);      \
  else if (wy) hipLaunchKernelGGL((KERNEL<true, false, __VA_ARGS__>), g, blk, 0, s, a);      \
  else hipLaunchKernelGGL((KERNEL<false, true, __VA_ARGS__>), g, blk, 0, s, a);
  switch (fmt) {
    case QF_FMT_NVFP4: QF_DISPATCH(k_nvfp4, L_NVFP4); break;
    case QF_FMT_MXFP4:
      if (mx_rule == QF_MX_RULE_NOCLIP) { QF_DISPATCH(k_mxfp4, L_MXFP4, true); }
      else { QF_DISPATCH(k_mxfp4, L_MXFP4); }
      break;
    case QF_FMT_Q4K:
      if (mx_rule == QF_Q4K_RULE_MSE) { QF_DISPATCH(k_q4k, L_Q4K, true); }
      else { QF_DISPATCH(k_q4k, L_Q4K); }
      break;
    default: return hipErrorInvalidValue;
  }
#undef QF_DISPATCH
  return hipGetLastError();
}

hipError_t launch_ste(const uint16_t* g, float* out, int64_t n, bool acc, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nv = n >> 3;
  int64_t tiles = (nv + WG * L_STE - 1) / (WG * L_STE);
  if (tiles == 0) tiles = 1;                                // tail-only input
  if (acc) hipLaunchKernelGGL((k_ste<true, L_STE>), dim3((uint32_t)tiles), dim3(WG), 0, s, g, out, n);
  else hipLaunchKernelGGL((k_ste<false, L_STE>), dim3((uint32_t)tiles), dim3(WG), 0, s, g, out, n);
  return hipGetLastError();
}

hipError_t launch_selftest_conversions(unsigned long long* counts, hipStream_t s) {
  for (uint32_t part = 0; part < 16; ++part) {
    hipLaunchKernelGGL(k_self_fp32, dim3((1u << 28) / WG), dim3(WG), 0, s, part << 28, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (uint32_t part = 0; part < 8; ++part) {
    hipLaunchKernelGGL(k_self_nonneg, dim3((1u << 28) / WG), dim3(WG), 0, s, part << 28, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_self_scaled, dim3(65536 / WG, 255), dim3(WG), 0, s, counts);
  return hipGetLastError();
}

}  // namespace qf
