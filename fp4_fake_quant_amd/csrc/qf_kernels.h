// Host-side launch interface between the C ABI (qf_api.cpp) and the kernel
// translation units.  Plain structs of device pointers and sizes only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qf.h"

namespace qf {

// A quantization launch works on "chunks" of 8 consecutive bf16 (16 bytes):
// one 128-bit load per lane.  A workgroup of 256 lanes handles a tile of
// TILE_CHUNKS chunks (4 per lane, at stride 256 so that every load
// instruction of the workgroup covers 4 KiB of contiguous memory).  Tiles
// never straddle two tensors; a tensor's last tile may be partial.
constexpr int WG = 256;
constexpr int CHUNKS_PER_LANE = 4;
constexpr int TILE_CHUNKS = WG * CHUNKS_PER_LANE;   // 1024 chunks = 8192 elements

struct QTensor {
  const uint16_t* x;
  uint16_t* y;
  uint8_t* codes;      // NVFP4/MXFP4 packed codes, or Q4_K blocks
  uint8_t* scales;     // NVFP4/MXFP4 block-scale bytes
  int64_t ldx, ldy;
  uint32_t nchunks;    // rows * cols / 8
  uint32_t cpr;        // chunks per row = cols / 8
  int32_t tile_begin;  // first workgroup of this tensor
  int32_t group;       // NVFP4 tied group
  int32_t contig_x;    // ldx == cols
  int32_t contig_y;    // ldy == cols
};

struct QArgs {
  QTensor t[QF_MAX_GROUPED];
  int n;
  int total_tiles;
  const float* tscale;  // NVFP4: device float per group
  uint32_t* partial;    // NVFP4 pass 1: one uint32 per tile (amax bits | nonfinite << 31)
};

struct ReduceArgs {
  int32_t tile_begin[QF_MAX_GROUPED + 1];
  int32_t group[QF_MAX_GROUPED];
  int n;
  int n_groups;
  const uint32_t* partial;
  float* tscale;
  uint32_t* nonfinite;
};

hipError_t launch_nvfp4_amax(const QArgs& a, hipStream_t s);
hipError_t launch_nvfp4_scale_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_quant(int fmt, bool write_y, bool write_packed, const QArgs& a, hipStream_t s);
hipError_t launch_ste(const uint16_t* g, float* out, int64_t n, bool accumulate, hipStream_t s);
hipError_t launch_selftest_conversions(unsigned long long* counts, hipStream_t s);

}  // namespace qf
