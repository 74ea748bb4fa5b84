// Host-side launch interface between the C ABI (qf_api.cpp) and the kernel
// translation units.  Plain structs of device pointers and sizes only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qf.h"

namespace qf {

// QF_OK for hipSuccess; otherwise records e as the calling thread's last HIP error
// (qf_last_hip_error) and returns QF_ERR_HIP.
qf_status status_of(hipError_t e);
// Every argument check of the NVFP4 tensor-scale calls except the workspace.
qf_status check_tensor_scale(const qf_tensor_desc* d, int n, int n_groups, const float* d_scales);

// A quantization launch works on "chunks" of 8 consecutive bf16 (16 bytes):
// one 128-bit load per lane.  A workgroup of 256 lanes handles a tile of
// 256 * L chunks (L per lane, at stride 256 so that every load instruction of
// the workgroup covers 4 KiB of contiguous memory).  Tiles never straddle two
// tensors; a tensor's last tile may be partial.  L is chosen per kernel from
// measurements (more, smaller workgroups stream writes better on gfx950).
constexpr int WG = 256;
constexpr int L_AMAX = 2, L_NVFP4 = 1, L_MXFP4 = 1, L_Q4K = 2, L_STE = 1;
// The amax pass runs a persistent grid of at most AMAX_GRID workgroups, each
// keeping one maximum per tied group.
constexpr int AMAX_GRID = 2048;

inline int chunks_per_lane(int fmt) {
  return fmt == QF_FMT_NVFP4 ? L_NVFP4 : fmt == QF_FMT_MXFP4 ? L_MXFP4 : L_Q4K;
}

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
  uint32_t* partial;    // NVFP4 pass 1: [n_groups][grid] maxima (abs bf16 bits)
  int n_groups;         // NVFP4 pass 1: groups that own a partial row
};

struct ReduceArgs {
  int n_groups;         // groups to write
  int n_partial_groups; // groups with a row of partials (the others have no tensor)
  int grid;             // partials per group
  const uint32_t* partial;
  float* tscale;
  uint32_t* nonfinite;
  float* tracked;       // running maximum |x| per group, folded in and updated (null: none)
};

// ------------------------------------------------------------------ LoRA ---
constexpr int LORA_MAX_R = 16;      // adapter rank handled in registers
constexpr int LORA_SLAB = 512;      // gradient columns per workgroup unit
constexpr int LORA_MERGE_COLS = 64;     // pass-1 merge tile: 64 columns ...
constexpr int LORA_MERGE_ROWS = 32;     // ... of 32 rows
constexpr int LORA_MERGE_GRID_MAX = 768;    // pass-1 workgroups resident at once (3 per CU)
constexpr int LORA_MERGE_TILES_MIN = 4;     // tiles per wave below which the grid shrinks
constexpr int LORA_QDQ_ROWS = 32;       // rows per pass-2 unit (at most; fewer for small launches)
constexpr int LORA_DA_ROWS = 256;       // rows per gradient workgroup (one dA partial each), or
constexpr int LORA_DA_ROWS_MAX = 512;   // twice that when the launch still has a workgroup per CU

// A descriptor holds `count` experts of one shape, stacked: every tensor of expert e
// follows expert e - 1's contiguously (W [count][rows][ldw], A [count][r][cols], ...),
// and expert e's tied group is group + e * group_stride.  Pass 1 (merge + maximum):
// tiles numbered descriptor by descriptor, expert by expert, then by band of merge_band
// row tiles, column tile, row tile; each wave of the grid takes an equal contiguous run.
// Pass 2 without M in memory (merge + QDQ): a unit is one wave's LORA_SLAB-column slab of
// merge_rows rows, numbered row block major; every expert starts on a fresh workgroup of
// 4 waves.  A gradient unit is one workgroup's: a LORA_SLAB-column slab of da_rows rows.
struct LoraTensor {
  const uint16_t* W;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* M;          // merged weight; null: not stored (the QDQ pass merges again)
  uint16_t* y;          // merge-and-QDQ outputs (null: skipped)
  uint8_t* codes;
  uint8_t* scales;
  const uint16_t* G;
  float* dA;
  float* dB;
  float* dA_partial;   // workspace: [count][row blocks][LORA_MAX_R][cols]
  float* dB_partial;   // workspace: [count][slabs][rows][LORA_MAX_R]
  int64_t rows, cols, ldw;
  int32_t r, group;
  int32_t slabs;            // ceil(cols / LORA_SLAB), the gradient slabs
  int32_t merge_tile_begin;         // pass 1: first tile of the descriptor in the launch,
  int32_t merge_rtiles, merge_ctiles;  // its 32-row and 64-column tiles
  int32_t merge_units, merge_wg_begin;  // pass 2: units per expert and first workgroup
  int32_t grad_wg_begin;    // gradients: one workgroup per (expert, row block, slab)
  int32_t count, group_stride;  // stacked experts
  int32_t mat_begin;        // flat index of expert 0 among the launch's matrices
};

struct LoraArgs {
  LoraTensor d[QF_MAX_GROUPED];
  int n;
  int n_groups;        // rows of merge partials
  int n_mats;          // matrices of the launch (experts of all descriptors)
  int64_t merge_tiles; // pass-1 tiles of the launch
  int merge_band;      // row tiles per band of the pass-1 order (the longest wave run)
  int merge_rows;      // rows per pass-2 unit (32, 16 or 8)
  int qdq_wg;          // pass-2 workgroups (four units each)
  int da_rows;         // rows per gradient workgroup (LORA_DA_ROWS or LORA_DA_ROWS_MAX)
  uint32_t* partial;   // merge amax partials [n_groups][merge workgroups]
  const float* tscale; // merge-and-QDQ: NVFP4 tensor scale of every tied group
};

hipError_t launch_lora_merge(const LoraArgs& a, int grid, hipStream_t s);
hipError_t launch_lora_merge_qdq(const LoraArgs& a, int grid, hipStream_t s);
hipError_t launch_lora_grads(const LoraArgs& a, int grid, int accumulate, hipStream_t s);

// Workgroups of the amax pass for a launch with `tiles` tiles of 256 * L_AMAX chunks.
inline int amax_grid(int tiles) { return tiles < AMAX_GRID ? tiles : AMAX_GRID; }
hipError_t launch_nvfp4_amax(const QArgs& a, hipStream_t s);
hipError_t launch_nvfp4_scale_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_quant(int fmt, bool write_y, bool write_packed, const QArgs& a, hipStream_t s,
                        int mx_rule = QF_MX_RULE_FLOOR);
hipError_t launch_ste(const uint16_t* g, float* out, int64_t n, bool accumulate, hipStream_t s);
hipError_t launch_ste_clip(int fmt, int mx_rule, const uint16_t* g, const uint16_t* x, int64_t rows, int64_t cols,
                           int64_t ldx, const float* d_scale, float* out, bool acc, hipStream_t s);
hipError_t launch_selftest_conversions(unsigned long long* counts, hipStream_t s);
hipError_t launch_gemm_mx4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, const uint8_t* Wc,
                           const uint8_t* Ws, uint16_t* Y, int64_t ldy, int M, int N, int K, hipStream_t s);
hipError_t launch_gemm_mx4pp(const uint8_t* Xc, const uint8_t* Xs, const uint8_t* Wc, const uint8_t* Ws, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, hipStream_t s);
hipError_t launch_gemm_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, unsigned flags, hipStream_t s);
// codes: NVFP4/MXFP4 code bytes (scales their scale bytes), or Q4_K blocks (scales unused)
hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          const float* d_scale, uint16_t* y, int64_t ldy, hipStream_t s);
// dst [C, R] = src [R, C]^T, MXFP4-QDQ'd along C first (floor or noclip rule) unless mode is TR_COPY
enum { TR_COPY = 0, TR_QDQ_FLOOR = 1, TR_QDQ_NOCLIP = 2 };
hipError_t launch_transpose(const uint16_t* src, int64_t lds, int R, int C, uint16_t* dst, int64_t ldd, int mode,
                            hipStream_t s);
hipError_t launch_gemm_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                             int64_t ldy, int M, int N, int K, unsigned flags, const float* d_sx, const float* d_sw,
                             hipStream_t s);

}  // namespace qf
