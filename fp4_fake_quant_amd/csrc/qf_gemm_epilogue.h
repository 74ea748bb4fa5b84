// Output of a 256 x 256 tile of Y from the GEMM kernels whose 8 waves (2 x 4) each hold a
// 128 x 64 sub-tile as 4 x 2 MFMA 32 x 32 accumulator tiles: lane (frow, fhalf) of wave
// (wm, wn) holds row wm*128 + 32i + frow, columns wn*64 + 32j + 8g + 4 fhalf + 0..3 in
// elements 4g .. 4g+3 of acc[i][j].
//
// Stored straight from the accumulators, each store instruction covers 32 rows with 16
// bytes each: 32 partial cache lines, and the address unit takes that many cycles.  Here
// the tile is converted to bf16 into LDS instead (256 rows x 512 bytes, 16-byte chunks
// XOR-swizzled by the row's low 5 bits, so the 32 rows of one write instruction spread
// over all banks and a row's 32 chunks read back conflict-free), then leaves in 16-byte
// stores: one instruction writes two whole 512-byte row segments.  The bf16 values are
// the same (RNE of the same fp32), only the store pattern changes.  The stores are buffer
// stores over the tile's rows; those outside Y take an out-of-range offset instead of a
// branch, so every wave issues the same 16 stores (the persistent GEMM's waits for its
// next tile's loads rely on that count).
#pragma once
#include "qf_device.h"

namespace qf {

__device__ __forceinline__ uint32_t epi_off(uint32_t r, uint32_t c) { return r * 512u + ((c ^ (r & 31u)) << 4); }

// lds: 128 KiB that no wave reads any more once every wave has arrived here (the
// function starts with a barrier).  Y rows 16-byte aligned (Y and ldy * 2), N a multiple
// of 8 and ldy below 2^22 (y_store_mode's mode 2).
template <typename AccT>
__device__ __forceinline__ void store_tile_lds(const AccT (&acc)[4][2], uint8_t* lds, uint16_t* __restrict__ Y,
                                               int64_t ldy, int m0, int n0, int M, int N) {
  const uint32_t lane = threadIdx.x & 63u, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wave >> 2, wn = wave & 3u, frow = lane & 31u, fhalf = lane >> 5;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = wm * 128u + 32u * i + frow;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t c = 8u * wn + 4u * j + g;
        const uint32_t lo = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        const uint32_t hi = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        *reinterpret_cast<uint2*>(lds + epi_off(r, c) + 8u * fhalf) = make_uint2(lo, hi);
      }
  }
  __syncthreads();
  // wave w stores rows 32w .. 32w+31, two rows per instruction, lane l chunk l & 31; the
  // resource spans the tile's rows from (m0, n0) to the last row's column N
  const int rows = min(M - m0, 256);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      Y + (int64_t)m0 * ldy + n0, (short)0, (int)(((int64_t)(rows - 1) * ldy + (N - n0)) * 2), 0x00020000);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const uint32_t r = 32u * wave + 2u * t + (lane >> 5), c = lane & 31u;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + epi_off(r, c));
    const bool in = m0 + (int)r < M && n0 + 8 * (int)c < N;
    buf_store16(ry, in ? (uint32_t)(r * (uint32_t)ldy + 8u * c) * 2u : BUF_OOR, v);
  }
}

// The 16 stores of store_tile_lds, to no memory (a resource of no bytes): a kernel that
// loops over tiles issues them after its first tile's loads, so that the loop head sees
// loads followed by 16 stores in flight from either path.
__device__ __forceinline__ void epilogue_store_balance(uint16_t* Y) {
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(Y, (short)0, 0, 0x00020000);
#pragma unroll
  for (int t = 0; t < 16; ++t) buf_store16(none, 16u * t, make_uint4(0u, 0u, 0u, 0u));
}

// Store mode of Y for the launchers: 2 when rows are 16-byte aligned, N is a multiple of 8
// and a tile's rows span less than 2^31 bytes (store_tile_lds), 1 when rows are 8-byte
// aligned (8-byte stores from the accumulators), 0 otherwise (element stores).
inline int y_store_mode(const uint16_t* Y, int64_t ldy, int64_t N) {
  if (ldy % 8 == 0 && (uintptr_t)Y % 16 == 0 && N % 8 == 0 && ldy < (1ll << 22)) return 2;
  return (ldy % 4 == 0 && (uintptr_t)Y % 8 == 0) ? 1 : 0;
}

}  // namespace qf
