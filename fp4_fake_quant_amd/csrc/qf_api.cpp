// C ABI of libqf: argument validation, descriptor marshalling and launches.
// Every operation and its error behaviour is specified in include/qf.h.
#include <algorithm>
#include <string.h>

#include "qf_kernels.h"

namespace {
int64_t round256(int64_t bytes) { return (bytes + 255) / 256 * 256; }

thread_local int g_last_hip_error = 0;

qf_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QF_OK;
  g_last_hip_error = (int)e;
  return QF_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
}  // namespace

qf_status qf::status_of(hipError_t e) { return hip_status(e); }

namespace {

int block_of(int fmt) {
  switch (fmt) {
    case QF_FMT_NVFP4: return 16;
    case QF_FMT_MXFP4: return 32;
    case QF_FMT_Q4K: return 256;
    default: return 0;
  }
}

// Validates one descriptor for format fmt; use_y / use_p: which outputs are written.
qf_status check_desc(const qf_tensor_desc& d, int fmt, bool use_y, bool use_p) {
  const int blk = block_of(fmt);
  if (d.rows < 0 || d.cols < 0) return QF_ERR_SHAPE;
  if (d.rows == 0 || d.cols == 0) return QF_OK;
  if (d.cols % blk != 0) return QF_ERR_SHAPE;
  if (!d.x) return QF_ERR_NULL;
  if (d.ldx < d.cols) return QF_ERR_SHAPE;
  if (!aligned(d.x, 16) || d.ldx % 8 != 0) return QF_ERR_ALIGN;
  const uint64_t chunks = (uint64_t)d.rows * (uint64_t)(d.cols / 8);
  if (chunks >= (1ull << 32) || (d.rows - 1) >= (1ll << 32)) return QF_ERR_SHAPE;
  if (use_y) {
    if (!d.y) return QF_ERR_NULL;
    if (d.ldy < d.cols) return QF_ERR_SHAPE;
    if (!aligned(d.y, 16) || d.ldy % 8 != 0) return QF_ERR_ALIGN;
  }
  if (use_p) {
    if (!d.codes) return QF_ERR_NULL;
    if (fmt == QF_FMT_Q4K) {
      if (!aligned(d.codes, 16)) return QF_ERR_ALIGN;
    } else {
      if (!d.scales) return QF_ERR_NULL;
      if (!aligned(d.codes, 4)) return QF_ERR_ALIGN;
    }
  }
  return QF_OK;
}

// Fills QArgs from descriptors; tiles of tile_chunks chunks are laid out tensor after tensor.
void fill_args(qf::QArgs& a, const qf_tensor_desc* d, int n, int tile_chunks) {
  memset(&a, 0, sizeof(a));
  int tiles = 0;
  int k = 0;
  for (int i = 0; i < n; ++i) {
    if (d[i].rows == 0 || d[i].cols == 0) continue;
    qf::QTensor& t = a.t[k++];
    t.x = d[i].x;
    t.y = d[i].y;
    t.codes = d[i].codes;
    t.scales = d[i].scales;
    t.ldx = d[i].ldx;
    t.ldy = d[i].y ? d[i].ldy : d[i].cols;
    t.cpr = (uint32_t)(d[i].cols / 8);
    t.nchunks = (uint32_t)((uint64_t)d[i].rows * t.cpr);
    t.tile_begin = tiles;
    t.group = d[i].group;
    t.contig_x = d[i].ldx == d[i].cols;
    t.contig_y = t.ldy == d[i].cols;
    tiles += (int)((t.nchunks + tile_chunks - 1) / tile_chunks);
  }
  a.n = k;
  a.total_tiles = tiles;
}

int64_t tiles_of(const qf_tensor_desc& d, int tile_chunks) {
  if (d.rows <= 0 || d.cols <= 0) return 0;
  const uint64_t chunks = (uint64_t)d.rows * (uint64_t)(d.cols / 8);
  return (int64_t)((chunks + tile_chunks - 1) / tile_chunks);
}

constexpr int AMAX_TILE = qf::WG * qf::L_AMAX;

// Rows of amax partials a tensor-scale call needs: highest group with a non-empty tensor, plus one.
int partial_groups(const qf_tensor_desc* d, int n) {
  int g = 0;
  for (int i = 0; i < n; ++i)
    if (d[i].rows > 0 && d[i].cols > 0 && d[i].group + 1 > g) g = d[i].group + 1;
  return g;
}

// Grouped quantization; each descriptor's NULL outputs are skipped.
qf_status quant_grouped(int fmt, const qf_tensor_desc* d, int n, const float* d_scales, hipStream_t s,
                        int mx_rule = QF_MX_RULE_FLOOR) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n > 0 && !d) return QF_ERR_NULL;
  if (fmt == QF_FMT_NVFP4 && !d_scales) return QF_ERR_NULL;
  const int tile_chunks = qf::WG * qf::chunks_per_lane(fmt);
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    const bool uy = d[i].y != nullptr, up = d[i].codes != nullptr;
    if (!uy && !up && d[i].rows > 0 && d[i].cols > 0) return QF_ERR_NULL;
    const qf_status st = check_desc(d[i], fmt, uy, up);
    if (st != QF_OK) return st;
    if (fmt == QF_FMT_NVFP4 && d[i].group < 0) return QF_ERR_ARG;
    tiles += tiles_of(d[i], tile_chunks);
  }
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  if (tiles == 0) return QF_OK;
  // one launch per distinct output combination (a grouped call normally has one)
  for (int combo = 0; combo < 3; ++combo) {
    const bool wy = combo != 2, wp = combo != 1;   // 0: both, 1: y only, 2: packed only
    qf_tensor_desc sel[QF_MAX_GROUPED];
    int k = 0;
    for (int i = 0; i < n; ++i) {
      const bool uy = d[i].y != nullptr, up = d[i].codes != nullptr;
      if (uy == wy && up == wp) sel[k++] = d[i];
    }
    if (k == 0) continue;
    qf::QArgs a;
    fill_args(a, sel, k, tile_chunks);
    a.tscale = d_scales;
    const hipError_t e = qf::launch_quant(fmt, wy, wp, a, s, mx_rule);
    if (e != hipSuccess) return hip_status(e);
  }
  return QF_OK;
}

qf_tensor_desc one(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                   uint8_t* codes, uint8_t* scales) {
  qf_tensor_desc d;
  d.x = x;
  d.rows = rows;
  d.cols = cols;
  d.ldx = ldx;
  d.y = y;
  d.ldy = ldy;
  d.codes = codes;
  d.scales = scales;
  d.group = 0;
  return d;
}

qf_status single(int fmt, const qf_tensor_desc& d, const float* d_scale, void* stream, bool wy, bool wp) {
  // the single-tensor calls require the outputs they name
  if (wy && d.rows > 0 && d.cols > 0 && !d.y) return QF_ERR_NULL;
  if (wp && d.rows > 0 && d.cols > 0 && !d.codes) return QF_ERR_NULL;
  return quant_grouped(fmt, &d, 1, d_scale, (hipStream_t)stream);
}

}  // namespace

// ------------------------------------------------------------ dequant ----
namespace {
qf_status dequant(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                  const float* d_scale, uint16_t* y, int64_t ldy, void* stream) {
  const int blk = block_of(fmt);
  if (rows < 0 || cols < 0 || cols % blk) return QF_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QF_OK;
  if (!codes || !y || (fmt != QF_FMT_Q4K && !scales) || (fmt == QF_FMT_NVFP4 && !d_scale)) return QF_ERR_NULL;
  if (ldy < cols) return QF_ERR_SHAPE;
  if ((uint64_t)rows * (uint64_t)(cols / 8) >= (1ull << 32) - 4096) return QF_ERR_SHAPE;   // 32-bit chunk index
  if (!aligned(y, 16) || ldy % 8 || !aligned(codes, fmt == QF_FMT_Q4K ? 16 : 4)) return QF_ERR_ALIGN;
  if (fmt == QF_FMT_NVFP4 && !aligned(d_scale, 4)) return QF_ERR_ALIGN;
  return hip_status(qf::launch_dequant(fmt, codes, scales, rows, cols, d_scale, y, ldy, (hipStream_t)stream));
}
}  // namespace

extern "C" {

uint32_t qf_version(void) { return (0u << 16) | (1u << 8) | 0u; }

const char* qf_status_str(qf_status s) {
  switch (s) {
    case QF_OK: return "ok";
    case QF_ERR_NULL: return "null pointer";
    case QF_ERR_SHAPE: return "invalid shape";
    case QF_ERR_ALIGN: return "misaligned pointer or stride";
    case QF_ERR_WORKSPACE: return "workspace missing or too small";
    case QF_ERR_HIP: return "HIP launch failed";
    case QF_ERR_NOT_IMPLEMENTED: return "not implemented";
    case QF_ERR_ARG: return "invalid argument";
    case QF_ERR_IO: return "file could not be written";
  }
  return "unknown status";
}

int qf_last_hip_error(void) { return g_last_hip_error; }

size_t qf_packed_bytes(int fmt, int64_t rows, int64_t cols) {
  const int blk = block_of(fmt);
  if (!blk || rows < 0 || cols < 0 || cols % blk) return 0;
  const size_t n = (size_t)rows * (size_t)cols;
  switch (fmt) {
    case QF_FMT_NVFP4: return n / 2 + n / 16;
    case QF_FMT_MXFP4: return n / 2 + n / 32;
    default: return n / 256 * 144;
  }
}

// ------------------------------------------------------ NVFP4 tensor scale --
size_t qf_nvfp4_tensor_scale_workspace(const qf_tensor_desc* d, int n) {
  if (n < 0 || (n > 0 && !d)) return 0;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) tiles += tiles_of(d[i], AMAX_TILE);
  const int64_t grid = tiles < qf::AMAX_GRID ? tiles : qf::AMAX_GRID;
  const int64_t words = grid * partial_groups(d, n);
  return (size_t)(words > 0 ? words : 1) * sizeof(uint32_t);
}

qf_status qf_nvfp4_tensor_scale_grouped(const qf_tensor_desc* d, int n, int n_groups, float* d_scales,
                                        uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream) {
  return qf_nvfp4_tensor_scale_tracked(d, n, n_groups, nullptr, d_scales, d_nonfinite, ws, ws_bytes, stream);
}

}  // extern "C"

// Every argument check of the tensor-scale calls except the workspace.
qf_status qf::check_tensor_scale(const qf_tensor_desc* d, int n, int n_groups, const float* d_scales) {
  if (n < 0 || n > QF_MAX_GROUPED || n_groups < 1 || n_groups > QF_MAX_GROUPS) return QF_ERR_ARG;
  if ((n > 0 && !d) || !d_scales) return QF_ERR_NULL;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    const qf_status st = check_desc(d[i], QF_FMT_NVFP4, false, false);
    if (st != QF_OK) return st;
    if (d[i].group < 0 || d[i].group >= n_groups) return QF_ERR_ARG;
    tiles += tiles_of(d[i], AMAX_TILE);
  }
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  return QF_OK;
}

extern "C" {

qf_status qf_nvfp4_tensor_scale_tracked(const qf_tensor_desc* d, int n, int n_groups, float* d_amax,
                                        float* d_scales, uint32_t* d_nonfinite, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (d_amax && !aligned(d_amax, 4)) return QF_ERR_ALIGN;
  const qf_status chk = qf::check_tensor_scale(d, n, n_groups, d_scales);
  if (chk != QF_OK) return chk;
  const size_t need = qf_nvfp4_tensor_scale_workspace(d, n);
  if (!ws || ws_bytes < need) return QF_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return QF_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  qf::QArgs a;
  fill_args(a, d, n, AMAX_TILE);
  a.partial = (uint32_t*)ws;
  a.n_groups = partial_groups(d, n);
  qf::ReduceArgs r;
  r.n_groups = n_groups;
  r.n_partial_groups = a.n_groups;
  r.grid = qf::amax_grid(a.total_tiles);
  r.partial = (const uint32_t*)ws;
  r.tscale = d_scales;
  r.nonfinite = d_nonfinite;
  r.tracked = d_amax;
  hipError_t e = qf::launch_nvfp4_amax(a, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(qf::launch_nvfp4_scale_reduce(r, s));
}

qf_status qf_nvfp4_tensor_scale(const uint16_t* const* x, const int64_t* numel, int n_tensors, float* d_scale,
                                uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream) {
  if (n_tensors < 0 || n_tensors > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n_tensors > 0 && (!x || !numel)) return QF_ERR_NULL;
  // each tensor is one contiguous row of numel elements, all in tied group 0
  qf_tensor_desc d[QF_MAX_GROUPED];
  for (int i = 0; i < n_tensors; ++i) {
    if (numel[i] < 0 || numel[i] % 16) return QF_ERR_SHAPE;
    d[i] = one(x[i], numel[i] ? 1 : 0, numel[i], numel[i], nullptr, 0, nullptr, nullptr);
  }
  return qf_nvfp4_tensor_scale_grouped(d, n_tensors, 1, d_scale, d_nonfinite, ws, ws_bytes, stream);
}

// -------------------------------------------------------------- NVFP4 QDQ --
qf_status qf_qdq_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const float* d_scale,
                       uint16_t* y, int64_t ldy, void* stream) {
  return single(QF_FMT_NVFP4, one(x, rows, cols, ldx, y, ldy, nullptr, nullptr), d_scale, stream, true, false);
}
qf_status qf_pack_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const float* d_scale,
                        uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows > 0 && cols > 0 && !scales) return QF_ERR_NULL;
  return single(QF_FMT_NVFP4, one(x, rows, cols, ldx, nullptr, 0, codes, scales), d_scale, stream, false, true);
}
qf_status qf_qdq_pack_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const float* d_scale,
                            uint16_t* y, int64_t ldy, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows > 0 && cols > 0 && !scales) return QF_ERR_NULL;
  return single(QF_FMT_NVFP4, one(x, rows, cols, ldx, y, ldy, codes, scales), d_scale, stream, true, true);
}
qf_status qf_qdq_pack_nvfp4_grouped(const qf_tensor_desc* d, int n, const float* d_scales, void* stream) {
  return quant_grouped(QF_FMT_NVFP4, d, n, d_scales, (hipStream_t)stream);
}

// -------------------------------------------------------------- MXFP4 QDQ --
qf_status qf_qdq_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                       void* stream) {
  return single(QF_FMT_MXFP4, one(x, rows, cols, ldx, y, ldy, nullptr, nullptr), nullptr, stream, true, false);
}
qf_status qf_pack_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                        uint8_t* scales, void* stream) {
  if (rows > 0 && cols > 0 && !scales) return QF_ERR_NULL;
  return single(QF_FMT_MXFP4, one(x, rows, cols, ldx, nullptr, 0, codes, scales), nullptr, stream, false, true);
}
qf_status qf_qdq_pack_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y,
                            int64_t ldy, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows > 0 && cols > 0 && !scales) return QF_ERR_NULL;
  return single(QF_FMT_MXFP4, one(x, rows, cols, ldx, y, ldy, codes, scales), nullptr, stream, true, true);
}
qf_status qf_qdq_pack_mxfp4_grouped(const qf_tensor_desc* d, int n, void* stream) {
  return quant_grouped(QF_FMT_MXFP4, d, n, nullptr, (hipStream_t)stream);
}
qf_status qf_qdq_pack_mxfp4_rule(const qf_tensor_desc* d, int n, int rule, void* stream) {
  if (rule != QF_MX_RULE_FLOOR && rule != QF_MX_RULE_NOCLIP) return QF_ERR_ARG;
  return quant_grouped(QF_FMT_MXFP4, d, n, nullptr, (hipStream_t)stream, rule);
}

// --------------------------------------------------------------- Q4_K QDQ --
qf_status qf_qdq_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                     void* stream) {
  return single(QF_FMT_Q4K, one(x, rows, cols, ldx, y, ldy, nullptr, nullptr), nullptr, stream, true, false);
}
qf_status qf_pack_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* blocks, void* stream) {
  return single(QF_FMT_Q4K, one(x, rows, cols, ldx, nullptr, 0, blocks, nullptr), nullptr, stream, false, true);
}
qf_status qf_qdq_pack_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                          uint8_t* blocks, void* stream) {
  return single(QF_FMT_Q4K, one(x, rows, cols, ldx, y, ldy, blocks, nullptr), nullptr, stream, true, true);
}
qf_status qf_qdq_pack_q4k_grouped(const qf_tensor_desc* d, int n, void* stream) {
  return quant_grouped(QF_FMT_Q4K, d, n, nullptr, (hipStream_t)stream);
}
qf_status qf_qdq_pack_q4k_rule(const qf_tensor_desc* d, int n, int rule, void* stream) {
  if (rule != QF_Q4K_RULE_MINMAX && rule != QF_Q4K_RULE_MSE) return QF_ERR_ARG;
  return quant_grouped(QF_FMT_Q4K, d, n, nullptr, (hipStream_t)stream, rule);
}

// -------------------------------------------------------------------- STE --
qf_status qf_ste_backward(const uint16_t* g_q, float* g_latent, int64_t n, int accumulate, void* stream) {
  if (n < 0) return QF_ERR_SHAPE;
  if (n == 0) return QF_OK;
  if (!g_q || !g_latent) return QF_ERR_NULL;
  if (!aligned(g_q, 16) || !aligned(g_latent, 16)) return QF_ERR_ALIGN;
  if (((n >> 3) + qf::WG * qf::L_STE - 1) / (qf::WG * qf::L_STE) >= (1ll << 31)) return QF_ERR_SHAPE;
  return hip_status(qf::launch_ste(g_q, g_latent, n, accumulate != 0, (hipStream_t)stream));
}

}  // extern "C"

namespace {
qf_status ste_clipped(int fmt, int rule, const uint16_t* g_q, const uint16_t* x, int64_t rows, int64_t cols,
                      int64_t ldx, const float* d_scale, float* g_latent, int accumulate, void* stream) {
  if (rows < 0 || cols < 0 || cols % block_of(fmt)) return QF_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QF_OK;
  if (!g_q || !x || !g_latent || (fmt == QF_FMT_NVFP4 && !d_scale)) return QF_ERR_NULL;
  if (ldx < cols) return QF_ERR_SHAPE;
  if ((uint64_t)rows * (uint64_t)(cols / 8) >= (1ull << 32) - 4096) return QF_ERR_SHAPE;   // 32-bit chunk index
  if (!aligned(g_q, 16) || !aligned(x, 16) || !aligned(g_latent, 16) || ldx % 8) return QF_ERR_ALIGN;
  if (fmt == QF_FMT_NVFP4 && !aligned(d_scale, 4)) return QF_ERR_ALIGN;
  return hip_status(qf::launch_ste_clip(fmt, rule, g_q, x, rows, cols, ldx, d_scale, g_latent, accumulate != 0,
                                        (hipStream_t)stream));
}
}  // namespace

extern "C" {
qf_status qf_ste_backward_clipped_nvfp4(const uint16_t* g_q, const uint16_t* x, int64_t rows, int64_t cols,
                                        int64_t ldx, const float* d_scale, float* g_latent, int accumulate,
                                        void* stream) {
  return ste_clipped(QF_FMT_NVFP4, QF_MX_RULE_FLOOR, g_q, x, rows, cols, ldx, d_scale, g_latent, accumulate, stream);
}
qf_status qf_ste_backward_clipped_mxfp4(const uint16_t* g_q, const uint16_t* x, int64_t rows, int64_t cols,
                                        int64_t ldx, int rule, float* g_latent, int accumulate, void* stream) {
  if (rule != QF_MX_RULE_FLOOR && rule != QF_MX_RULE_NOCLIP) return QF_ERR_ARG;
  return ste_clipped(QF_FMT_MXFP4, rule, g_q, x, rows, cols, ldx, nullptr, g_latent, accumulate, stream);
}
}  // extern "C"

// ------------------------------------------------------------------ LoRA --
namespace {

qf_status check_lora(const qf_lora_desc& d) {
  if (d.rows < 0 || d.cols < 0) return QF_ERR_SHAPE;
  if (d.rows == 0 || d.cols == 0) return QF_OK;
  if (d.cols % 32 != 0 || d.cols > QF_LORA_MAX_COLS || d.ldw < d.cols || d.ldw >= (1ll << 24)) return QF_ERR_SHAPE;
  if (d.r < 1 || d.r > qf::LORA_MAX_R) return QF_ERR_ARG;
  if (d.group < 0) return QF_ERR_ARG;
  if ((uint64_t)d.rows * (uint64_t)(d.cols / 8) >= (1ull << 32)) return QF_ERR_SHAPE;
  if ((uint64_t)d.rows * (uint64_t)d.r * 2u >= (1ull << 31)) return QF_ERR_SHAPE;   // B's byte offsets
  return QF_OK;
}

qf_status check_lora_merge_inputs(const qf_lora_desc& d) {
  if (!d.W || !d.A || !d.B) return QF_ERR_NULL;
  if (!aligned(d.W, 16) || !aligned(d.A, 16) || !aligned(d.B, 4) || d.ldw % 8) return QF_ERR_ALIGN;
  return QF_OK;
}

struct LoraCounts {
  int64_t merge_tiles = 0, merge_wg = 0, qdq_wg = 0, grad_wg = 0, dA_part = 0, dB_part = 0, mats = 0;
};

// A descriptor and the experts stacked behind it (count 1 for the grouped calls).
struct LoraIn {
  qf_lora_desc d;
  int64_t count;
  int64_t gs;
};

int64_t slabs_of(int64_t cols) { return (cols + qf::LORA_SLAB - 1) / qf::LORA_SLAB; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch sizes of a descriptor list for pass-2 units of qdq_rows rows and dA workgroups
// of da_rows rows; fills a (when given).  Pass 1: 32 x 64 tiles, descriptor by
// descriptor and expert by expert; its grid is the resident maximum of 3 workgroups per
// CU, or fewer so that every wave keeps at least LORA_MERGE_TILES_MIN tiles (one expert
// alone: 6,912 tiles, 432 workgroups).
LoraCounts lora_layout_with(const LoraIn* d, int n, int qdq_rows, int da_rows, qf::LoraArgs* a, float* dA_part) {
  LoraCounts c;
  if (a) memset(a, 0, sizeof(*a));
  int k = 0, groups = 0;
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    const int64_t cnt = d[i].count;
    if (x.rows <= 0 || x.cols <= 0 || cnt <= 0) continue;
    const int64_t slabs = slabs_of(x.cols);
    const int64_t rt = ceil_div(x.rows, qf::LORA_MERGE_ROWS), ct = ceil_div(x.cols, qf::LORA_MERGE_COLS);
    const int64_t qu = ceil_div(x.rows, qdq_rows) * slabs;
    const int64_t dblk = ceil_div(x.rows, da_rows);
    const int64_t du = dblk * slabs;
    if (a) {
      qf::LoraTensor& t = a->d[k];
      t.W = x.W; t.A = x.A; t.B = x.B; t.M = x.M; t.G = x.G;
      t.y = x.y; t.codes = x.codes; t.scales = x.scales;
      t.dA = x.dA; t.dB = x.dB;
      t.dA_partial = dA_part ? dA_part + c.dA_part : nullptr;
      t.dB_partial = nullptr;
      t.rows = x.rows; t.cols = x.cols; t.ldw = x.ldw;
      t.r = x.r; t.group = x.group;
      t.slabs = (int32_t)slabs;
      t.merge_tile_begin = (int32_t)c.merge_tiles;
      t.merge_rtiles = (int32_t)rt;
      t.merge_ctiles = (int32_t)ct;
      t.merge_units = (int32_t)qu;
      t.merge_wg_begin = (int32_t)c.qdq_wg;
      t.grad_wg_begin = (int32_t)c.grad_wg;
      t.count = (int32_t)cnt;
      t.group_stride = (int32_t)d[i].gs;
      t.mat_begin = (int32_t)c.mats;
    }
    ++k;
    const int64_t g_end = x.group + (cnt - 1) * d[i].gs + 1;
    if (g_end > groups) groups = (int)g_end;
    c.mats += cnt;
    c.merge_tiles += cnt * rt * ct;
    c.qdq_wg += cnt * ceil_div(qu, 4);
    c.grad_wg += cnt * du;
    c.dA_part += cnt * dblk * qf::LORA_MAX_R * x.cols;
  }
  c.merge_wg = std::min<int64_t>(qf::LORA_MERGE_GRID_MAX, ceil_div(c.merge_tiles, 4 * qf::LORA_MERGE_TILES_MIN));
  // dB partials follow all dA partials: [count][slabs][rows][LORA_MAX_R] per descriptor
  int k2 = 0;
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    if (x.rows <= 0 || x.cols <= 0 || d[i].count <= 0) continue;
    if (a) a->d[k2].dB_partial = dA_part ? dA_part + c.dA_part + c.dB_part : nullptr;
    ++k2;
    c.dB_part += d[i].count * slabs_of(x.cols) * x.rows * qf::LORA_MAX_R;
  }
  if (a) {
    a->n = k;
    a->n_groups = groups;
    a->n_mats = (int)c.mats;
    a->merge_tiles = c.merge_tiles;
    a->merge_band = (int)std::max<int64_t>(1, c.merge_wg > 0 ? ceil_div(c.merge_tiles, 4 * c.merge_wg) : 1);
    a->merge_rows = qdq_rows;
    a->qdq_wg = (int)c.qdq_wg;
    a->da_rows = da_rows;
  }
  return c;
}

// Pass-2 units shrink (32 -> 16 -> 8 rows) until a launch has at least two workgroups per
// CU, so that one expert alone still fills the chip.  Gradient workgroups take 512 rows
// when that still gives one workgroup per CU, else 256: fewer fp32 partials and all
// workgroups resident at once (8 experts per launch: 73.8 -> 69.0 us from cold caches);
// smaller ones multiply the partials, which cost more than the idle CUs (64 rows: grads
// 8.4 -> 10.1 ms).  A function of the descriptors only, so the workspace size and the
// launches agree.
LoraCounts lora_layout(const LoraIn* d, int n, qf::LoraArgs* a, float* dA_part) {
  constexpr int64_t FILL = 2 * 256;
  int qr = qf::LORA_QDQ_ROWS;
  int dr = qf::LORA_DA_ROWS_MAX;
  while (qr > 8 && lora_layout_with(d, n, qr, dr, nullptr, nullptr).qdq_wg < FILL) qr /= 2;
  if (lora_layout_with(d, n, qr, dr, nullptr, nullptr).grad_wg < 256) dr = qf::LORA_DA_ROWS;
  return lora_layout_with(d, n, qr, dr, a, dA_part);
}

int lora_groups(const LoraIn* d, int n) {
  int64_t g = 0;
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    if (x.rows > 0 && x.cols > 0 && d[i].count > 0) g = std::max<int64_t>(g, x.group + (d[i].count - 1) * d[i].gs + 1);
  }
  return (int)g;
}

// The grouped calls' descriptors as single experts.
int lora_in(const qf_lora_desc* d, int n, LoraIn* out) {
  for (int i = 0; i < n; ++i) {
    out[i].d = d[i];
    out[i].count = 1;
    out[i].gs = 0;
  }
  return n;
}

// Argument checks of the stacked-experts calls (each expert is checked as one
// descriptor by the shared code): count >= 1, group_stride >= 0, every expert's group
// below QF_MAX_GROUPS, at most 65,535 matrices per call, no merge scratch.
qf_status lora_experts_in(const qf_lora_experts* e, int n, LoraIn* out) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n > 0 && !e) return QF_ERR_NULL;
  int64_t mats = 0;
  for (int i = 0; i < n; ++i) {
    if (e[i].count < 1 || e[i].group_stride < 0 || e[i].d.group < 0) return QF_ERR_ARG;
    if (e[i].d.M) return QF_ERR_ARG;
    if (e[i].d.group + (int64_t)(e[i].count - 1) * e[i].group_stride >= QF_MAX_GROUPS) return QF_ERR_ARG;
    mats += e[i].count;
    out[i].d = e[i].d;
    out[i].count = e[i].count;
    out[i].gs = e[i].group_stride;
  }
  if (mats > 65535) return QF_ERR_ARG;
  return QF_OK;
}

size_t lora_workspace(const LoraIn* d, int n) {
  for (int i = 0; i < n; ++i)
    if (check_lora(d[i].d) != QF_OK) return 0;
  const LoraCounts c = lora_layout(d, n, nullptr, nullptr);
  const int64_t merge_words = c.merge_wg * lora_groups(d, n);
  const int64_t grad_words = c.dA_part + c.dB_part;
  const int64_t words = merge_words > grad_words ? merge_words : grad_words;
  return (size_t)(words > 0 ? words : 1) * 4;
}

qf_status lora_layout_out(const LoraIn* d, int n, int32_t* out) {
  if (!out) return QF_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const qf_status st = check_lora(d[i].d);
    if (st != QF_OK) return st;
  }
  qf::LoraArgs a;
  const LoraCounts c = lora_layout(d, n, &a, nullptr);
  out[0] = c.merge_wg > 0 ? (int32_t)ceil_div(c.merge_tiles, 4 * c.merge_wg) : 0;
  out[1] = (int32_t)c.merge_wg;
  out[2] = a.da_rows;
  out[3] = (int32_t)c.grad_wg;
  out[4] = a.merge_rows;
  out[5] = (int32_t)c.qdq_wg;
  return QF_OK;
}

qf_status lora_tensor_scale(const LoraIn* d, int n, int n_groups, float* d_scales, uint32_t* d_nonfinite, void* ws,
                            size_t ws_bytes, void* stream) {
  if (n_groups < 1 || n_groups > QF_MAX_GROUPS) return QF_ERR_ARG;
  if (!d_scales) return QF_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    const qf_status st = check_lora(x);
    if (st != QF_OK) return st;
    if (x.rows == 0 || x.cols == 0) continue;
    if (x.group + (d[i].count - 1) * d[i].gs >= n_groups) return QF_ERR_ARG;
    const qf_status sm = check_lora_merge_inputs(x);
    if (sm != QF_OK) return sm;
    if (x.M && !aligned(x.M, 16)) return QF_ERR_ALIGN;
  }
  if (!ws || ws_bytes < lora_workspace(d, n)) return QF_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return QF_ERR_ALIGN;
  qf::LoraArgs a;
  const LoraCounts c = lora_layout(d, n, &a, nullptr);
  if (c.merge_tiles >= (1ll << 31) || c.qdq_wg >= (1ll << 29)) return QF_ERR_SHAPE;
  a.partial = (uint32_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = qf::launch_lora_merge(a, (int)c.merge_wg, s);
  if (e != hipSuccess) return hip_status(e);
  qf::ReduceArgs r;
  r.n_groups = n_groups;
  r.n_partial_groups = a.n_groups;
  r.grid = (int)c.merge_wg;
  r.partial = (const uint32_t*)ws;
  r.tscale = d_scales;
  r.nonfinite = d_nonfinite;
  r.tracked = nullptr;
  return hip_status(qf::launch_nvfp4_scale_reduce(r, s));
}

qf_status lora_qdq_pack(const LoraIn* d, int n, const float* d_scales, void* stream) {
  if (!d_scales) return QF_ERR_NULL;
  // descriptors with M: QDQ + pack of M; without: merge again and QDQ in registers
  qf_tensor_desc t[QF_MAX_GROUPED];
  LoraIn fused[QF_MAX_GROUPED];
  int nt = 0, nf = 0;
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    const qf_status st = check_lora(x);
    if (st != QF_OK) return st;
    if (x.rows == 0 || x.cols == 0) continue;
    if (x.group < 0) return QF_ERR_ARG;
    const qf_tensor_desc q = one(x.M ? x.M : x.W, x.rows, x.cols, x.M ? x.cols : x.ldw, x.y, x.cols, x.codes,
                                 x.scales);
    const bool uy = x.y != nullptr, up = x.codes != nullptr;
    if (!uy && !up) return QF_ERR_NULL;
    const qf_status sq = check_desc(q, QF_FMT_NVFP4, uy, up);
    if (sq != QF_OK) return sq;
    if (x.M) {
      t[nt] = q;
      t[nt++].group = x.group;
    } else {
      const qf_status sm = check_lora_merge_inputs(x);
      if (sm != QF_OK) return sm;
      fused[nf++] = d[i];
    }
  }
  hipStream_t s = (hipStream_t)stream;
  if (nt > 0) {
    const qf_status st = quant_grouped(QF_FMT_NVFP4, t, nt, d_scales, s);
    if (st != QF_OK) return st;
  }
  if (nf == 0) return QF_OK;
  qf::LoraArgs a;
  const LoraCounts c = lora_layout(fused, nf, &a, nullptr);
  if (c.qdq_wg >= (1ll << 29)) return QF_ERR_SHAPE;
  a.tscale = d_scales;
  return hip_status(qf::launch_lora_merge_qdq(a, (int)c.qdq_wg, s));
}

qf_status lora_grads(const LoraIn* d, int n, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  for (int i = 0; i < n; ++i) {
    const qf_lora_desc& x = d[i].d;
    const qf_status st = check_lora(x);
    if (st != QF_OK) return st;
    if (x.rows == 0 || x.cols == 0) continue;
    if (!x.A || !x.B || !x.G || !x.dA || !x.dB) return QF_ERR_NULL;
    if (!aligned(x.A, 16) || !aligned(x.B, 4) || !aligned(x.G, 16) || !aligned(x.dB, 4) || !aligned(x.dA, 4))
      return QF_ERR_ALIGN;
  }
  if (!ws || ws_bytes < lora_workspace(d, n)) return QF_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return QF_ERR_ALIGN;
  qf::LoraArgs a;
  const LoraCounts c = lora_layout(d, n, &a, (float*)ws);
  if (c.grad_wg >= (1ll << 31)) return QF_ERR_SHAPE;
  return hip_status(qf::launch_lora_grads(a, (int)c.grad_wg, accumulate != 0, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t qf_lora_workspace(const qf_lora_desc* d, int n) {
  if (n < 0 || n > QF_MAX_GROUPED || (n > 0 && !d)) return 0;
  LoraIn in[QF_MAX_GROUPED];
  return lora_workspace(in, lora_in(d, n, in));
}

qf_status qf_lora_layout(const qf_lora_desc* d, int n, int32_t* out) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if ((n > 0 && !d) || !out) return QF_ERR_NULL;
  LoraIn in[QF_MAX_GROUPED];
  return lora_layout_out(in, lora_in(d, n, in), out);
}

qf_status qf_lora_merge_tensor_scale_nvfp4_grouped(const qf_lora_desc* d, int n, int n_groups, float* d_scales,
                                                   uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n > 0 && !d) return QF_ERR_NULL;
  LoraIn in[QF_MAX_GROUPED];
  return lora_tensor_scale(in, lora_in(d, n, in), n_groups, d_scales, d_nonfinite, ws, ws_bytes, stream);
}

qf_status qf_lora_merge_qdq_pack_nvfp4_grouped(const qf_lora_desc* d, int n, const float* d_scales, void* stream) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n > 0 && !d) return QF_ERR_NULL;
  LoraIn in[QF_MAX_GROUPED];
  return lora_qdq_pack(in, lora_in(d, n, in), d_scales, stream);
}

qf_status qf_lora_adapter_grads_grouped(const qf_lora_desc* d, int n, int accumulate, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (n < 0 || n > QF_MAX_GROUPED) return QF_ERR_ARG;
  if (n > 0 && !d) return QF_ERR_NULL;
  LoraIn in[QF_MAX_GROUPED];
  return lora_grads(in, lora_in(d, n, in), accumulate, ws, ws_bytes, stream);
}

size_t qf_lora_experts_workspace(const qf_lora_experts* e, int n) {
  LoraIn in[QF_MAX_GROUPED];
  if (lora_experts_in(e, n, in) != QF_OK) return 0;
  return lora_workspace(in, n);
}

qf_status qf_lora_experts_layout(const qf_lora_experts* e, int n, int32_t* out) {
  LoraIn in[QF_MAX_GROUPED];
  const qf_status st = lora_experts_in(e, n, in);
  if (st != QF_OK) return st;
  return lora_layout_out(in, n, out);
}

qf_status qf_lora_experts_merge_tensor_scale_nvfp4(const qf_lora_experts* e, int n, int n_groups, float* d_scales,
                                                   uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream) {
  LoraIn in[QF_MAX_GROUPED];
  const qf_status st = lora_experts_in(e, n, in);
  if (st != QF_OK) return st;
  return lora_tensor_scale(in, n, n_groups, d_scales, d_nonfinite, ws, ws_bytes, stream);
}

qf_status qf_lora_experts_merge_qdq_pack_nvfp4(const qf_lora_experts* e, int n, const float* d_scales,
                                               void* stream) {
  LoraIn in[QF_MAX_GROUPED];
  const qf_status st = lora_experts_in(e, n, in);
  if (st != QF_OK) return st;
  return lora_qdq_pack(in, n, d_scales, stream);
}

qf_status qf_lora_experts_adapter_grads(const qf_lora_experts* e, int n, int accumulate, void* ws, size_t ws_bytes,
                                        void* stream) {
  LoraIn in[QF_MAX_GROUPED];
  const qf_status st = lora_experts_in(e, n, in);
  if (st != QF_OK) return st;
  return lora_grads(in, n, accumulate, ws, ws_bytes, stream);
}

}  // extern "C"

// One contiguous matrix (ldw = cols) as a LoRA descriptor of tied group 0.
namespace {
qf_lora_desc lora_one(const uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t rows, int64_t cols, int r) {
  qf_lora_desc d;
  memset(&d, 0, sizeof(d));
  d.W = W;
  d.A = A;
  d.B = B;
  d.rows = rows;
  d.cols = cols;
  d.ldw = cols;
  d.r = r;
  d.group = 0;
  return d;
}
}  // namespace

extern "C" {

qf_status qf_lora_merge_tensor_scale_nvfp4(const uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t rows,
                                           int64_t cols, int r, float* d_scale, void* ws, size_t ws_bytes,
                                           void* stream) {
  const qf_lora_desc d = lora_one(W, A, B, rows, cols, r);
  return qf_lora_merge_tensor_scale_nvfp4_grouped(&d, 1, 1, d_scale, nullptr, ws, ws_bytes, stream);
}

qf_status qf_lora_merge_qdq_pack_nvfp4(const uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t rows,
                                       int64_t cols, int r, const float* d_scale, uint16_t* y_scratch,
                                       uint8_t* codes, uint8_t* scales, void* stream) {
  qf_lora_desc d = lora_one(W, A, B, rows, cols, r);
  d.y = y_scratch;
  d.codes = codes;
  d.scales = scales;
  return qf_lora_merge_qdq_pack_nvfp4_grouped(&d, 1, d_scale, stream);
}

qf_status qf_lora_adapter_grads(const uint16_t* G, const uint16_t* A, const uint16_t* B, int64_t rows, int64_t cols,
                                int r, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes,
                                void* stream) {
  qf_lora_desc d = lora_one(nullptr, A, B, rows, cols, r);
  d.G = G;
  d.dA = dA;
  d.dB = dB;
  return qf_lora_adapter_grads_grouped(&d, 1, accumulate, ws, ws_bytes, stream);
}

// ------------------------------------------------------------ W4A4 GEMM --

qf_status qf_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           const float* d_scale, uint16_t* y, int64_t ldy, void* stream) {
  return dequant(QF_FMT_NVFP4, codes, scales, rows, cols, d_scale, y, ldy, stream);
}
qf_status qf_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, uint16_t* y,
                           int64_t ldy, void* stream) {
  return dequant(QF_FMT_MXFP4, codes, scales, rows, cols, nullptr, y, ldy, stream);
}
qf_status qf_dequant_q4k(const uint8_t* blocks, int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, void* stream) {
  return dequant(QF_FMT_Q4K, blocks, nullptr, rows, cols, nullptr, y, ldy, stream);
}

}  // extern "C"

namespace {
// Operand checks shared by the BF16-core GEMM entry points (flags are checked by each).
qf_status check_gemm(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, const uint16_t* Y, int64_t ldy,
                     int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || M >= (1ll << 30) || N >= (1ll << 30)) return QF_ERR_SHAPE;
  if (M == 0 || N == 0) return QF_OK;
  if (!X || !W || !Y) return QF_ERR_NULL;
  if (ldx < K || ldw < K || ldy < N) return QF_ERR_SHAPE;
  if (ldx >= (1ll << 22) || ldw >= (1ll << 22)) return QF_ERR_SHAPE;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 2) || ldx % 8 || ldw % 8) return QF_ERR_ALIGN;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  return QF_OK;
}

// Two-pass forward: QDQ of each flagged operand into its caller buffer, then the BF16
// GEMM with no QDQ on what the matrix cores should see.  Every argument is checked
// before the first launch.
qf_status linear_forward(int fmt, const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                         int64_t ldy, int64_t M, int64_t N, int64_t K, unsigned flags, const float* d_sx,
                         const float* d_sw, uint16_t* Xq, int64_t ldxq, uint16_t* Wq, int64_t ldwq, hipStream_t s) {
  const bool qa = flags & QF_QDQ_A, qw = flags & QF_QDQ_W;
  qf_status st = check_gemm(X, ldx, W, ldw, Y, ldy, M, N, K);
  if (st != QF_OK || M == 0 || N == 0) return st;
  // the GEMM then reads the QDQ'd copies: the same constraints apply to them
  st = check_gemm(qa ? Xq : X, qa ? ldxq : ldx, qw ? Wq : W, qw ? ldwq : ldw, Y, ldy, M, N, K);
  if (st != QF_OK) return st;
  if (fmt == QF_FMT_NVFP4 && ((qa && !d_sx) || (qw && !d_sw))) return QF_ERR_NULL;
  if ((d_sx && !aligned(d_sx, 4)) || (d_sw && !aligned(d_sw, 4))) return QF_ERR_ALIGN;
  const qf_tensor_desc dx = one(X, M, K, ldx, Xq, ldxq, nullptr, nullptr);
  const qf_tensor_desc dw = one(W, N, K, ldw, Wq, ldwq, nullptr, nullptr);
  if (qa && (st = check_desc(dx, fmt, true, false)) != QF_OK) return st;
  if (qw && (st = check_desc(dw, fmt, true, false)) != QF_OK) return st;
  const int rule = (flags & QF_MX_NOCLIP) ? QF_MX_RULE_NOCLIP : QF_MX_RULE_FLOOR;
  if (qa && (st = quant_grouped(fmt, &dx, 1, d_sx, s, rule)) != QF_OK) return st;
  if (qw && (st = quant_grouped(fmt, &dw, 1, d_sw, s, rule)) != QF_OK) return st;
  return hip_status(qf::launch_gemm_mxfp4(qa ? Xq : X, qa ? ldxq : ldx, qw ? Wq : W, qw ? ldwq : ldw, Y, ldy, (int)M,
                                          (int)N, (int)K, 0, s));
}
}  // namespace

extern "C" {

qf_status qf_linear_forward_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                                  int64_t ldy, int64_t M, int64_t N, int64_t K, unsigned flags, uint16_t* Xq,
                                  int64_t ldxq, uint16_t* Wq, int64_t ldwq, void* stream) {
  if (flags & ~(QF_QDQ_A | QF_QDQ_W | QF_MX_NOCLIP)) return QF_ERR_ARG;
  if ((flags & QF_MX_NOCLIP) && !(flags & (QF_QDQ_A | QF_QDQ_W))) return QF_ERR_ARG;
  return linear_forward(QF_FMT_MXFP4, X, ldx, W, ldw, Y, ldy, M, N, K, flags, nullptr, nullptr, Xq, ldxq, Wq, ldwq,
                        (hipStream_t)stream);
}

qf_status qf_linear_forward_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y,
                                  int64_t ldy, int64_t M, int64_t N, int64_t K, unsigned flags,
                                  const float* d_scale_x, const float* d_scale_w, uint16_t* Xq, int64_t ldxq,
                                  uint16_t* Wq, int64_t ldwq, void* stream) {
  if ((flags & ~(QF_QDQ_A | QF_QDQ_W)) || flags == 0) return QF_ERR_ARG;
  return linear_forward(QF_FMT_NVFP4, X, ldx, W, ldw, Y, ldy, M, N, K, flags, d_scale_x, d_scale_w, Xq, ldxq, Wq,
                        ldwq, (hipStream_t)stream);
}

qf_status qf_gemm_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y, int64_t ldy,
                        int64_t M, int64_t N, int64_t K, unsigned flags, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || M >= (1ll << 30) || N >= (1ll << 30)) return QF_ERR_SHAPE;
  if (flags & ~(QF_QDQ_A | QF_QDQ_W | QF_FP4_CORES | QF_MX_NOCLIP)) return QF_ERR_ARG;
  if ((flags & QF_FP4_CORES) && (flags & (QF_QDQ_A | QF_QDQ_W)) != (QF_QDQ_A | QF_QDQ_W)) return QF_ERR_ARG;
  if ((flags & QF_MX_NOCLIP) && ((flags & QF_FP4_CORES) || !(flags & (QF_QDQ_A | QF_QDQ_W)))) return QF_ERR_ARG;
  if (M == 0 || N == 0) return QF_OK;
  if (!X || !W || !Y) return QF_ERR_NULL;
  if (ldx < K || ldw < K || ldy < N) return QF_ERR_SHAPE;
  if (ldx >= (1ll << 22) || ldw >= (1ll << 22)) return QF_ERR_SHAPE;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 2) || ldx % 8 || ldw % 8) return QF_ERR_ALIGN;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  if (flags & QF_FP4_CORES)
    return hip_status(qf::launch_gemm_mx4(X, ldx, W, ldw, nullptr, nullptr, Y, ldy, (int)M, (int)N, (int)K,
                                          (hipStream_t)stream));
  return hip_status(qf::launch_gemm_mxfp4(X, ldx, W, ldw, Y, ldy, (int)M, (int)N, (int)K, flags,
                                          (hipStream_t)stream));
}

qf_status qf_gemm_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* Y, int64_t ldy,
                        int64_t M, int64_t N, int64_t K, unsigned flags, const float* d_scale_x,
                        const float* d_scale_w, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || M >= (1ll << 30) || N >= (1ll << 30)) return QF_ERR_SHAPE;
  if ((flags & ~(QF_QDQ_A | QF_QDQ_W)) || flags == 0) return QF_ERR_ARG;
  if (M == 0 || N == 0) return QF_OK;
  if (!X || !W || !Y) return QF_ERR_NULL;
  if (((flags & QF_QDQ_A) && !d_scale_x) || ((flags & QF_QDQ_W) && !d_scale_w)) return QF_ERR_NULL;
  if (ldx < K || ldw < K || ldy < N) return QF_ERR_SHAPE;
  if (ldx >= (1ll << 22) || ldw >= (1ll << 22)) return QF_ERR_SHAPE;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 2) || ldx % 8 || ldw % 8) return QF_ERR_ALIGN;
  if ((d_scale_x && !aligned(d_scale_x, 4)) || (d_scale_w && !aligned(d_scale_w, 4))) return QF_ERR_ALIGN;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  return hip_status(qf::launch_gemm_nvfp4(X, ldx, W, ldw, Y, ldy, (int)M, (int)N, (int)K, flags, d_scale_x, d_scale_w,
                                          (hipStream_t)stream));
}

qf_status qf_transpose_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                            int qdq_mxfp4, void* stream) {
  if (qdq_mxfp4 < 0 || qdq_mxfp4 > 2) return QF_ERR_ARG;
  if (rows < 0 || cols < 0 || rows % 8 || cols % (qdq_mxfp4 ? 32 : 8) || rows >= (1ll << 22) || cols >= (1ll << 31))
    return QF_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QF_OK;
  if (!x || !y) return QF_ERR_NULL;
  if (ldx < cols || ldy < rows) return QF_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || ldx % 8 || ldy % 8) return QF_ERR_ALIGN;
  return hip_status(qf::launch_transpose(x, ldx, (int)rows, (int)cols, y, ldy, qdq_mxfp4, (hipStream_t)stream));
}

size_t qf_linear_backward_workspace(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  return (size_t)(round256(K * N * 2) + round256(N * M * 2) + round256(K * M * 2));
}

qf_status qf_linear_backward_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, const uint16_t* dY,
                                   int64_t lddy, uint16_t* dX, int64_t lddx, uint16_t* dW, int64_t lddw, int64_t M,
                                   int64_t N, int64_t K, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
  if (flags & ~(QF_QDQ_A | QF_QDQ_W | QF_MX_NOCLIP)) return QF_ERR_ARG;
  if ((flags & QF_MX_NOCLIP) && !(flags & (QF_QDQ_A | QF_QDQ_W))) return QF_ERR_ARG;
  if (M < 0 || N < 0 || K < 0 || M % 64 || N % 64 || K % 32) return QF_ERR_SHAPE;
  if (M >= (1ll << 22) || N >= (1ll << 22) || K >= (1ll << 22)) return QF_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0 || (!dX && !dW)) return QF_OK;
  if (!dY || (dX && !W) || (dW && !X)) return QF_ERR_NULL;
  if (lddy < N || (dX && (ldw < K || lddx < K)) || (dW && (ldx < K || lddw < K))) return QF_ERR_SHAPE;
  const int64_t big = 1ll << 22;                                            // tile offsets of the products
  if (lddy >= big || (dX && (ldw >= big || lddx >= big)) || (dW && (ldx >= big || lddw >= big))) return QF_ERR_SHAPE;
  if (!aligned(dY, 16) || lddy % 8) return QF_ERR_ALIGN;
  if (dX && (!aligned(W, 16) || !aligned(dX, 16) || ldw % 8 || lddx % 8)) return QF_ERR_ALIGN;
  if (dW && (!aligned(X, 16) || !aligned(dW, 16) || ldx % 8 || lddw % 8)) return QF_ERR_ALIGN;
  if (!ws || ws_bytes < qf_linear_backward_workspace(M, N, K)) return QF_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QF_ERR_ALIGN;
  uint16_t* wqt = (uint16_t*)ws;                                           // Wq^T [K, N]
  uint16_t* dyt = (uint16_t*)((char*)ws + round256(K * N * 2));             // dY^T [N, M]
  uint16_t* xqt = (uint16_t*)((char*)dyt + round256(N * M * 2));            // Xq^T [K, M]
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const int qdq = (flags & QF_MX_NOCLIP) ? qf::TR_QDQ_NOCLIP : qf::TR_QDQ_FLOOR;
  if (dX) {
    e = qf::launch_transpose(W, ldw, (int)N, (int)K, wqt, N, (flags & QF_QDQ_W) ? qdq : qf::TR_COPY, s);
    if (e == hipSuccess) e = qf::launch_gemm_mxfp4(dY, lddy, wqt, N, dX, lddx, (int)M, (int)K, (int)N, 0, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (dW) {
    e = qf::launch_transpose(dY, lddy, (int)M, (int)N, dyt, M, qf::TR_COPY, s);
    if (e == hipSuccess) e = qf::launch_transpose(X, ldx, (int)M, (int)K, xqt, M, (flags & QF_QDQ_A) ? qdq : qf::TR_COPY, s);
    if (e == hipSuccess) e = qf::launch_gemm_mxfp4(dyt, M, xqt, M, dW, lddw, (int)N, (int)K, (int)M, 0, s);
  }
  return hip_status(e);
}

qf_status qf_gemm_mxfp4_packed(const uint8_t* Xc, const uint8_t* Xs, const uint8_t* Wc, const uint8_t* Ws, uint16_t* Y,
                               int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || M >= (1ll << 30) || N >= (1ll << 30)) return QF_ERR_SHAPE;
  if (M == 0 || N == 0) return QF_OK;
  if (!Xc || !Xs || !Wc || !Ws || !Y) return QF_ERR_NULL;
  if (ldy < N) return QF_ERR_SHAPE;
  if (!aligned(Xc, 16) || !aligned(Wc, 16) || !aligned(Xs, 4) || !aligned(Ws, 4) || !aligned(Y, 2)) return QF_ERR_ALIGN;
  if (256 * (K / 2) >= (1ll << 31)) return QF_ERR_SHAPE;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  return hip_status(qf::launch_gemm_mx4pp(Xc, Xs, Wc, Ws, Y, ldy, (int)M, (int)N, (int)K, (hipStream_t)stream));
}

qf_status qf_gemm_mxfp4_packed_w(const uint16_t* X, int64_t ldx, const uint8_t* Wc, const uint8_t* Ws, uint16_t* Y,
                                 int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || M >= (1ll << 30) || N >= (1ll << 30)) return QF_ERR_SHAPE;
  if (M == 0 || N == 0) return QF_OK;
  if (!X || !Wc || !Ws || !Y) return QF_ERR_NULL;
  if (ldx < K || ldy < N) return QF_ERR_SHAPE;
  if (ldx >= (1ll << 22)) return QF_ERR_SHAPE;
  if (!aligned(X, 16) || !aligned(Wc, 16) || !aligned(Ws, 2) || !aligned(Y, 2) || ldx % 8) return QF_ERR_ALIGN;
  if ((N < 256 ? N : 256) * (K / 2) >= (1ll << 31)) return QF_ERR_SHAPE;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= (1ll << 31)) return QF_ERR_SHAPE;
  return hip_status(qf::launch_gemm_mx4(X, ldx, nullptr, 0, Wc, Ws, Y, ldy, (int)M, (int)N, (int)K,
                                        (hipStream_t)stream));
}

// ------------------------------------------------------ conformance test ---
qf_status qf_selftest_conversions(unsigned long long* d_counts, void* stream) {
  if (!d_counts) return QF_ERR_NULL;
  if (!aligned(d_counts, 8)) return QF_ERR_ALIGN;
  return hip_status(qf::launch_selftest_conversions(d_counts, (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

// --------------------------------------------------------- workspace query --
size_t qf_workspace_size(int op, int64_t rows, int64_t cols, int n) {
  if (rows < 0 || cols < 0 || n < 0) return 0;
  switch (op) {
    case QF_OP_NVFP4_TENSOR_SCALE: {
      if (n > QF_MAX_GROUPED) return 0;
      // partials: min(tiles, AMAX_GRID) per group with a tensor, group indices below QF_MAX_GROUPS
      const uint64_t chunks = (uint64_t)rows * (uint64_t)cols / 8;
      const uint64_t tiles = (uint64_t)n * ((chunks + AMAX_TILE - 1) / AMAX_TILE);
      const uint64_t grid = tiles < (uint64_t)qf::AMAX_GRID ? tiles : (uint64_t)qf::AMAX_GRID;
      const uint64_t words = grid * QF_MAX_GROUPS;
      return (size_t)(words > 0 ? words : 1) * sizeof(uint32_t);
    }
    case QF_OP_LORA: {
      if (n > QF_MAX_GROUPED || cols > QF_LORA_MAX_COLS) return 0;
      // the most any layout asks for: the full merge grid, 256-row gradient blocks, 64 groups
      const int64_t slabs = slabs_of(cols);
      const int64_t merge_words = (int64_t)qf::LORA_MERGE_GRID_MAX * QF_MAX_GROUPS;
      const int64_t grad_words = (int64_t)n * (ceil_div(rows, qf::LORA_DA_ROWS) * qf::LORA_MAX_R * cols +
                                               slabs * rows * qf::LORA_MAX_R);
      const int64_t words = merge_words > grad_words ? merge_words : grad_words;
      return (size_t)(words > 0 ? words : 1) * 4;
    }
    case QF_OP_LINEAR_BACKWARD:
      return qf_linear_backward_workspace(rows, cols, n);
    default:
      return 0;
  }
}

}  // extern "C"
