/*
 * qf.h -- C ABI of libqf, the MI355X (gfx950) simulated-quantization hot path.
 *
 * What the library computes is described on the QATFactory project page:
 *   - "Method" section, "Framework overview": the forward pass applies a lossy
 *     quantize-dequantize (QDQ) transform that reproduces inference numerics;
 *     the backward pass is a straight-through estimator (STE) onto the
 *     continuous latent weights.
 *   - "Method" section, "Deployment-aligned simulated quantization": the
 *     engine's values, block sizes and scaling rules; under NVFP4 the
 *     projections the engines fuse (QKV, gate/up) share one FP32 tensor scale.
 *   - "Supported formats" table: NVFP4 (E2M1, block 16, E4M3 block scale +
 *     FP32 tensor scale, 4.50 bpw), MXFP4 (E2M1, block 32, E8M0 block scale,
 *     4.25 bpw), Q4_K (unsigned INT4, 32-blocks in 256 super-blocks, 6-bit
 *     block scales, FP16 super-block scales, asymmetric, 4.50 bpw).
 *   - "Method" section, "Quantization-aware distillation": LoRA merges the
 *     adapters into the frozen base before quantization, one MoE expert at a
 *     time.
 *   - "Method" section, "Export" and "Quantization-aware reinforcement
 *     learning": codes and scales are packed into the engine's layout so the
 *     engine never requantizes.
 *   - "Overview": every matrix multiplication runs in BF16 (weights, and
 *     optionally activations, are QDQ'd first).
 * The bit-level rules (scale mapping, rounding, signed zeros, packed layouts)
 * are stated choices; they are written out next to each call below.
 *
 * Conventions for every call
 *   - Tensors are row-major [rows, cols]; blocks run along cols (the
 *     contiguous, input / K axis).  ld* are row strides in elements.
 *   - BF16 travels as uint16_t bit patterns.
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns.
 *     Descriptor arrays (qf_tensor_desc*) are HOST memory, read during the call.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work and return; results are ready when the stream reaches that point.
 *   - Argument errors are detected before anything is enqueued and return a
 *     status; nothing is written then.  A failed launch returns QF_ERR_HIP and
 *     qf_last_hip_error() gives the hipError_t of the calling thread.
 *   - Alignment: bf16 tensors (x, y) and their row strides must be 16-byte
 *     aligned (ld % 8 == 0); packed code arrays 4-byte aligned; Q4_K block
 *     arrays and fp32 gradient arrays 16-byte aligned.  Else QF_ERR_ALIGN.
 *   - Shapes: cols must be a multiple of the format's block (16 / 32 / 256),
 *     else QF_ERR_SHAPE; rows * cols / 8 must be below 2^32 per tensor.
 *     rows == 0 or cols == 0 is a valid no-op.
 *   - Inputs must be finite.  Results for Inf/NaN inputs are unspecified (the
 *     NVFP4 tensor-scale pass raises a flag when it sees one).
 *   - Calls are reentrant and keep no state between calls.
 */
#ifndef QF_H
#define QF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qf_status {
  QF_OK = 0,
  QF_ERR_NULL = 1,            /* a required pointer is NULL                        */
  QF_ERR_SHAPE = 2,           /* negative size, cols not a block multiple, ld < cols */
  QF_ERR_ALIGN = 3,           /* pointer or stride misaligned                      */
  QF_ERR_WORKSPACE = 4,       /* workspace missing or smaller than required         */
  QF_ERR_HIP = 5,             /* a HIP launch failed; see qf_last_hip_error()       */
  QF_ERR_NOT_IMPLEMENTED = 6, /* reserved                                           */
  QF_ERR_ARG = 7,             /* other invalid argument (count, flag, group index)  */
  QF_ERR_IO = 8               /* a file could not be created or written             */
} qf_status;

enum qf_format { QF_FMT_NVFP4 = 0, QF_FMT_MXFP4 = 1, QF_FMT_Q4K = 2 };

/* MXFP4 shared-exponent rules (the pages do not fix one).  FLOOR, the default of every
 * MXFP4 call: E = clamp(floor(log2 amax) - 2 + 127, 0, 254), which clips block maxima in
 * (6, 8) * 2^(E-127) to 6 (finite inputs never get past E = 252).  NOCLIP: the smallest
 * E in [0, 252] with amax <= 6 * 2^(E-127) (ceil(log2(amax / 6)) + 127), one more than
 * FLOOR exactly when the maximum's significand exceeds 1.5 and FLOOR's E is below 252;
 * nothing is clipped except block maxima above 6 * 2^125 = 1.5 * 2^127.  252 is the last
 * exponent whose whole grid (up to 6 * 2^(E-127)) bf16 can hold: at 253 a maximum in
 * [1.75, 2) * 2^127 would round to the code 4 and dequantize to 2^128 = Inf.  So every
 * finite input gives finite QDQ'd values under both rules.  amax == 0 gives E = 0. */
#define QF_MX_RULE_FLOOR 0
#define QF_MX_RULE_NOCLIP 1

/* Most tensors one grouped call accepts. */
#define QF_MAX_GROUPED 16
/* Most tied groups one grouped tensor-scale call accepts. */
#define QF_MAX_GROUPS 64

/* ------------------------------------------------------------ helpers ---- */
uint32_t qf_version(void);                 /* (major << 16) | (minor << 8) | patch */
const char* qf_status_str(qf_status s);
int qf_last_hip_error(void);               /* hipError_t of this thread's last failed launch */

/* Device workspace (bytes) that suffices for any call of operation `op` over at most n
 * tensors of at most rows x cols elements each (0 for an unknown op or invalid sizes):
 *   QF_OP_NVFP4_TENSOR_SCALE  the tensor-scale calls (any grouping below QF_MAX_GROUPS);
 *   QF_OP_LORA                the LoRA merge / tensor-scale and adapter-gradient calls
 *                             (n matrices, any rank 1..16, any grouping);
 *   QF_OP_LINEAR_BACKWARD     qf_linear_backward_mxfp4 with M = rows, N = cols, K = n.
 * The per-call queries (qf_nvfp4_tensor_scale_workspace, qf_lora_workspace,
 * qf_linear_backward_workspace) give the exact size for given descriptors. */
#define QF_OP_NVFP4_TENSOR_SCALE 0
#define QF_OP_LORA 1
#define QF_OP_LINEAR_BACKWARD 2
size_t qf_workspace_size(int op, int64_t rows, int64_t cols, int n);

/* Packed bytes of one [rows, cols] tensor (codes + block scales; Q4_K blocks).
 * NVFP4: rows*cols/2 + rows*cols/16 (the 4-byte FP32 tensor scale per group is
 * the caller's float).  MXFP4: rows*cols/2 + rows*cols/32.  Q4_K:
 * rows*cols/256*144.  These are the table's 4.50 / 4.25 / 4.50 bits per weight.
 * Returns 0 for invalid arguments. */
size_t qf_packed_bytes(int fmt, int64_t rows, int64_t cols);

/* One tensor of a grouped call.
 *   x      input bf16 [rows, ldx]
 *   y      QDQ'd bf16 output [rows, ldy], or NULL to skip it (x == y with
 *          ldx == ldy is allowed: in place)
 *   codes  NVFP4/MXFP4: packed codes [rows, cols/2] bytes, element 2i in the
 *          low nibble and 2i+1 in the high nibble; Q4_K: the 144-byte blocks
 *          [rows, cols/256, 144].  NULL skips packing.
 *   scales NVFP4: E4M3 bytes [rows, cols/16]; MXFP4: E8M0 bytes [rows, cols/32];
 *          unused for Q4_K (its scales live inside the blocks).  NULL iff codes is NULL.
 *   group  NVFP4 tied-group index (0 <= group < n_groups); ignored otherwise. */
typedef struct qf_tensor_desc {
  const uint16_t* x;
  int64_t rows, cols, ldx;
  uint16_t* y;
  int64_t ldy;
  uint8_t* codes;
  uint8_t* scales;
  int32_t group;
} qf_tensor_desc;

/* ------------------------------------------------- NVFP4 tensor scale ---- */
/* Pass 1 of NVFP4 ("Method", tying of fused projections; "Supported formats",
 * FP32 tensor scale).  For each tied group g: A_g = max |x| over every element
 * of every tensor with group == g; d_scales[g] = (A_g == 0) ? 1.0f :
 * fl(A_g / 2688.0f)  (2688 = 6 * 448: the group's largest block maps onto the
 * top of the E4M3 range).  d_scales is a device float[n_groups]; it stays on
 * the device for pass 2 (no host synchronisation).  d_nonfinite (device
 * uint32, may be NULL) is set to 1 if any element is Inf or NaN, and left
 * unchanged otherwise.  ws: device workspace of at least
 * qf_nvfp4_tensor_scale_workspace(d, n) bytes (no initialisation needed).
 * Only x, rows, cols, ldx and group of each descriptor are read. */
size_t qf_nvfp4_tensor_scale_workspace(const qf_tensor_desc* d, int n);
qf_status qf_nvfp4_tensor_scale_grouped(const qf_tensor_desc* d, int n, int n_groups,
                                        float* d_scales, uint32_t* d_nonfinite,
                                        void* ws, size_t ws_bytes, void* stream);
/* The same pass with a TRACKED scale ("Method", "Export": NVFP4 activation scales are
 * tracked during training and saved, so no calibration pass is needed).  The reading
 * taken: the tracked amax of group g is the running maximum of |x| over every call so far.
 * d_amax: device float[n_groups], 4-byte aligned, the state (the caller zeroes it to start
 * tracking and saves it with the checkpoint; non-negative finite values).  Each call sets
 * d_amax[g] = max(d_amax[g], A_g) with A_g this call's group maximum (a group with no
 * tensor keeps its value), then d_scales[g] = (d_amax[g] == 0) ? 1.0f :
 * fl(d_amax[g] / 2688.0f).  d_amax == NULL is qf_nvfp4_tensor_scale_grouped.  Everything
 * else as qf_nvfp4_tensor_scale_grouped. */
qf_status qf_nvfp4_tensor_scale_tracked(const qf_tensor_desc* d, int n, int n_groups, float* d_amax,
                                        float* d_scales, uint32_t* d_nonfinite,
                                        void* ws, size_t ws_bytes, void* stream);
/* One tied group given as a host array of n_tensors (<= QF_MAX_GROUPED, else QF_ERR_ARG)
 * device pointers to contiguous bf16 tensors of numel[i] elements each (the members the
 * engines fuse, e.g. Q, K and V): *d_scale = the group's tensor scale as above.  numel[i]
 * must be a non-negative multiple of 16 (the NVFP4 block; QF_ERR_SHAPE) below 2^35, each
 * x[i] 16-byte aligned (QF_ERR_ALIGN).  ws: at least
 * qf_workspace_size(QF_OP_NVFP4_TENSOR_SCALE, 1, max numel, n_tensors) bytes. */
qf_status qf_nvfp4_tensor_scale(const uint16_t* const* x, const int64_t* numel, int n_tensors,
                                float* d_scale, uint32_t* d_nonfinite,
                                void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- NVFP4 QDQ ---- */
/* Pass 2 of NVFP4, per 16-block of each row, with s_t = *d_scale:
 *   k = fl(6 s_t); a = max |x|; S = E4M3 RNE-satfinite(fl(a / k)); s = value(S);
 *   d = fl(s s_t); magnitude code = 0 if d == 0 else E2M1 RNE-saturating(fl(|x| fl(1/d)))
 *   (a zero element always gets magnitude 0); code sign = sign bit of x;
 *   y = sign | bf16(fl(fl(v s) s_t)).
 * qf_qdq_* writes only y; qf_pack_* writes only codes and scales; qf_qdq_pack_*
 * writes all three in one pass over x. */
qf_status qf_qdq_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                       const float* d_scale, uint16_t* y, int64_t ldy, void* stream);
qf_status qf_pack_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        const float* d_scale, uint8_t* codes, uint8_t* scales, void* stream);
qf_status qf_qdq_pack_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            const float* d_scale, uint16_t* y, int64_t ldy,
                            uint8_t* codes, uint8_t* scales, void* stream);
/* Grouped: one launch over up to QF_MAX_GROUPED tensors; tensor i uses
 * d_scales[d[i].group]. */
qf_status qf_qdq_pack_nvfp4_grouped(const qf_tensor_desc* d, int n, const float* d_scales,
                                    void* stream);

/* ----------------------------------------------------------- MXFP4 QDQ ---- */
/* Per 32-block: a = max |x|; E = 0 if a == 0 else clamp(floor(log2 a) - 2 + 127, 0, 254)
 * (largest element's exponent minus E2M1's largest exponent); X = 2^(E-127);
 * code = sign(x) | E2M1 RNE-saturating(|x| / X); y = sign | bf16(v X) (exact,
 * bf16 subnormals kept).  scales hold E. */
qf_status qf_qdq_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                       uint16_t* y, int64_t ldy, void* stream);
qf_status qf_pack_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* codes, uint8_t* scales, void* stream);
qf_status qf_qdq_pack_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            uint16_t* y, int64_t ldy, uint8_t* codes, uint8_t* scales,
                            void* stream);
qf_status qf_qdq_pack_mxfp4_grouped(const qf_tensor_desc* d, int n, void* stream);
/* qf_qdq_pack_mxfp4_grouped under a chosen shared-exponent rule (QF_MX_RULE_FLOOR or
 * QF_MX_RULE_NOCLIP, else QF_ERR_ARG).  The packed bytes mean the same under either
 * rule, so qf_dequant_mxfp4 and the packed GEMM inputs take them unchanged. */
qf_status qf_qdq_pack_mxfp4_rule(const qf_tensor_desc* d, int n, int rule, void* stream);

/* ------------------------------------------------------------ Q4_K QDQ ---- */
/* Per 256 super-block of eight 32-sub-blocks j (min/max round-to-nearest):
 *   mn_j = min(min x, 0), mx_j = max x (a zero extreme counts as +0);
 *   scale_j = fl(fl(mx_j - mn_j) / 15); off_j = fl(0 - mn_j);
 *   d = fp16(fl(max_j scale_j / 63)), dmin = fp16(fl(max_j off_j / 63)) (RNE, saturating);
 *   sc_j = d == 0 ? 0 : clamp(rint(fl(scale_j / d)), 0, 63); m_j likewise with off_j, dmin;
 *   D_j = d sc_j, M_j = dmin m_j; q = D_j == 0 ? 0 : clamp(rint(fl(fl(x + M_j) fl(1/D_j))), 0, 15);
 *   y = bf16(fl(D_j q - M_j)).
 * Block layout (144 bytes): d (fp16 LE) | dmin (fp16 LE) | 12 bytes holding a
 * 96-bit little-endian stream with sc_j at bits 6j.. and m_j at bits 48+6j.. |
 * 128 bytes of codes, element 2i low nibble, 2i+1 high nibble.  For the
 * single-tensor calls `blocks` is [rows, cols/256, 144]. */
qf_status qf_qdq_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                     uint16_t* y, int64_t ldy, void* stream);
qf_status qf_pack_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* blocks, void* stream);
qf_status qf_qdq_pack_q4k(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                          uint16_t* y, int64_t ldy, uint8_t* blocks, void* stream);
qf_status qf_qdq_pack_q4k_grouped(const qf_tensor_desc* d, int n, void* stream);

/* qf_qdq_pack_q4k_grouped under a sub-block scale rule: QF_Q4K_RULE_MINMAX (the rule above)
 * or QF_Q4K_RULE_MSE, a search of our own (the pages name an MSE-optimal quantizer only as a
 * PTQ baseline): each sub-block's scale is the best of the 8 candidates
 * s_k = fl(base (1 - k/16)), base = fl(fl(mx - mn)/15), by the squared error of the
 * sub-block quantized with s_k and the offset -mn (q = clamp(rint(fl(fl(x - mn) fl(1/s_k))),
 * 0, 15), error fl(fl(fl(q s_k) + mn) - x)), summed in float32 over each quarter of the
 * sub-block in index order and then as (quarter 0 + quarter 1) + (quarter 2 + quarter 3);
 * the first smallest sum wins.  The offsets, the two-level d / sc_j and dmin / m_j
 * quantization, the codes and the layout are as above.  Unknown rules give QF_ERR_ARG. */
#define QF_Q4K_RULE_MINMAX 0
#define QF_Q4K_RULE_MSE 1
qf_status qf_qdq_pack_q4k_rule(const qf_tensor_desc* d, int n, int rule, void* stream);

/* ---------------------------------------------------------------- STE ---- */
/* Identity straight-through estimator ("Method", "Framework overview"):
 * g_latent[i] = f32(g_q[i]) (accumulate == 0) or g_latent[i] += f32(g_q[i])
 * (accumulate != 0; one fp32 rounding).  g_q: device bf16[n], 16-byte aligned;
 * g_latent: device float[n], 16-byte aligned. */
qf_status qf_ste_backward(const uint16_t* g_q, float* g_latent, int64_t n, int accumulate,
                          void* stream);

/* Clipped STE on the FP4 grids (the second reading of the "Method", "Framework overview"
 * STE: the gradient reaches the latent weight only where the quantizer kept the element
 * inside the E2M1 grid of the "Supported formats" table).  For x [rows, ldx] (the latent
 * weight the forward quantized) an element saturates when its scaled magnitude exceeds 6:
 *   NVFP4: fl(|x| r) > 6 with the block's r = fl(1/d), d = fl(s s_t), s_t = *d_scale (the
 *          tensor scale the forward used); blocks with d = 0 and zero elements never do;
 *   MXFP4: |x| > 6 * 2^(E-127) with the block's shared exponent E under `rule`
 *          (QF_MX_RULE_FLOOR or QF_MX_RULE_NOCLIP; none saturates under the latter).
 * g_latent[i] = f32(g_q[i]), or +0.0 where x[i] saturated; with accumulate != 0 that value
 * is added (one fp32 rounding).  g_q bf16 and g_latent fp32 are contiguous [rows, cols],
 * 16-byte aligned; x 16-byte aligned with ldx a multiple of 8 and >= cols (QF_ERR_ALIGN /
 * QF_ERR_SHAPE); cols a multiple of 16 (NVFP4) or 32 (MXFP4), rows * cols / 8 < 2^32 - 4096
 * (QF_ERR_SHAPE); d_scale 4-byte aligned (QF_ERR_NULL if missing); an unknown rule gives
 * QF_ERR_ARG.  The masks are bit for bit the quantizers' own decisions. */
qf_status qf_ste_backward_clipped_nvfp4(const uint16_t* g_q, const uint16_t* x, int64_t rows, int64_t cols,
                                        int64_t ldx, const float* d_scale, float* g_latent, int accumulate,
                                        void* stream);
qf_status qf_ste_backward_clipped_mxfp4(const uint16_t* g_q, const uint16_t* x, int64_t rows, int64_t cols,
                                        int64_t ldx, int rule, float* g_latent, int accumulate, void* stream);

/* ---------------------------------------------- LoRA, one expert at a time */
/* "Method" section, "Quantization-aware distillation": LoRA keeps one frozen
 * base W, trains only the adapters A (r x cols) and B (rows x r), and quantizes
 * the merged weight; MoE models merge and quantize one expert at a time.  With
 * the identity STE the gradient G of the QDQ'd merged weight gives
 * dB = G . A^T and dA = B^T . G.
 *
 * One descriptor per matrix (an expert's fused gate/up or its down matrix):
 *   W  bf16 [rows, ldw] frozen base;  A bf16 [r, cols] and B bf16 [rows, r],
 *      both contiguous;  r in 1..16.
 *   M  bf16 [rows, cols] contiguous scratch for the merged weight (written by
 *      pass 1, read by pass 2; one expert's worth is the bounded scratch), or
 *      NULL: pass 1 then only takes the maximum and pass 2 merges again from W,
 *      A and B in registers (same bits, no scratch, one read of W instead of a
 *      write and a read of M).
 *   y, codes, scales  pass-2 outputs as in qf_qdq_pack_nvfp4 (y contiguous,
 *      ldy = cols; y or codes may be NULL to skip it).
 *   G  bf16 [rows, cols] contiguous; dA fp32 [r, cols]; dB fp32 [rows, r].
 *   group  tied-group index for the NVFP4 tensor scale (one per expert per
 *      fused matrix: experts never share a scale).
 * Shapes: cols a multiple of 32 and at most QF_LORA_MAX_COLS; rows >= 0 with rows * r
 * below 2^30; ldw a multiple of 8 and below 2^24.  W, A, M, G 16-byte aligned; B, dA, dB 4-byte aligned; the packed
 * arrays as in qf_qdq_pack_nvfp4.  With r odd, the row of B that ends the array
 * may be read as a whole 4-byte word (the 2 bytes after B, never used).
 * Empty descriptors (rows or cols 0) are skipped.  Errors: QF_ERR_SHAPE for a
 * shape outside these limits, QF_ERR_ARG for r outside 1..16, a negative group or
 * one >= n_groups, QF_ERR_NULL / QF_ERR_ALIGN for pointers, QF_ERR_WORKSPACE
 * when ws is smaller than qf_lora_workspace; nothing is launched then.
 *
 * Merge (bit-exact): acc = 0; for k = 0..r-1 in order, acc = fl(acc + B[i,k] A[k,j])
 * (the products are exact in fp32); M[i,j] = bf16(fl(W[i,j] + acc)); no alpha/r
 * factor.  Gradients are fp32 sums in an unspecified but fixed order: the same
 * inputs always give the same bits; with non-finite inputs they are unspecified. */
#define QF_LORA_MAX_COLS 65536

typedef struct qf_lora_desc {
  const uint16_t* W;
  int64_t rows, cols, ldw;
  const uint16_t* A;
  const uint16_t* B;
  int32_t r;
  int32_t group;
  uint16_t* M;
  uint16_t* y;
  uint8_t* codes;
  uint8_t* scales;
  const uint16_t* G;
  float* dA;
  float* dB;
} qf_lora_desc;

/* Device workspace (bytes) the LoRA calls need for these descriptors (0 when a
 * descriptor is invalid). */
size_t qf_lora_workspace(const qf_lora_desc* d, int n);
/* Host query of the launch layout the LoRA calls choose for these descriptors (nothing
 * is launched; only shapes, ranks and groups are read).  Pass 2 without M (merge again +
 * QDQ) works in units of a 512-column slab of 32 rows, shrinking to 16 or 8 until the
 * launch has 512 workgroups.  Pass 1 (merge + tensor scale) runs a grid of 768 4-wave
 * workgroups, or fewer so that a wave keeps at least 4 of the launch's 32-row x 64-column
 * tiles; with M, or when pass-2 units shrank below 32 rows, its waves take equal
 * contiguous runs of those tiles, and otherwise (no M, 32-row units) equal runs of the
 * pass-2 units, where they merge only the rows that may hold a new maximum.  out[0] most pass-1 tiles per
 * wave, out[1] pass-1 workgroups, out[2] rows per gradient workgroup (512 when that still
 * gives 256 workgroups, else 256), out[3] gradient workgroups, out[4] rows per pass-2
 * unit, out[5] pass-2 workgroups.  out is host int32[6].  Errors as the LoRA calls'
 * shape and argument checks. */
qf_status qf_lora_layout(const qf_lora_desc* d, int n, int32_t* out);
/* Pass 1: merge into M (skipped for M == NULL) and the NVFP4 tensor scale of
 * every tied group (d_scales[g] as in qf_nvfp4_tensor_scale_grouped, computed
 * from the merged values). */
qf_status qf_lora_merge_tensor_scale_nvfp4_grouped(const qf_lora_desc* d, int n, int n_groups, float* d_scales,
                                                   uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream);
/* Pass 2: NVFP4 QDQ + pack of the merged weight (exactly qf_qdq_pack_nvfp4 on M
 * with d_scales[group]); descriptors with M == NULL merge again from W, A, B. */
qf_status qf_lora_merge_qdq_pack_nvfp4_grouped(const qf_lora_desc* d, int n, const float* d_scales, void* stream);
/* STE to the adapters: dB = G . A^T, dA = B^T . G (fp32; accumulate != 0 adds). */
qf_status qf_lora_adapter_grads_grouped(const qf_lora_desc* d, int n, int accumulate, void* ws, size_t ws_bytes,
                                        void* stream);

/* The same three steps for one contiguous matrix (W [rows, cols], A [r, cols], B [rows, r],
 * G [rows, cols]; ldw = cols) with no merge scratch: pass 1 merges in registers and only
 * takes the maximum (*d_scale = the matrix's NVFP4 tensor scale, a tied group of one);
 * pass 2 merges again and writes the QDQ'd bf16 to y_scratch [rows, cols] (NULL: skipped)
 * and the packed codes [rows, cols/2] and E4M3 scales [rows, cols/16] (NULL: skipped; not
 * both NULL).  Bits, shapes, alignment and errors as the grouped calls with one descriptor
 * and M = NULL; ws of at least qf_workspace_size(QF_OP_LORA, rows, cols, 1) bytes. */
qf_status qf_lora_merge_tensor_scale_nvfp4(const uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t rows,
                                           int64_t cols, int r, float* d_scale, void* ws, size_t ws_bytes,
                                           void* stream);
qf_status qf_lora_merge_qdq_pack_nvfp4(const uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t rows,
                                       int64_t cols, int r, const float* d_scale, uint16_t* y_scratch,
                                       uint8_t* codes, uint8_t* scales, void* stream);
qf_status qf_lora_adapter_grads(const uint16_t* G, const uint16_t* A, const uint16_t* B, int64_t rows, int64_t cols,
                                int r, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes,
                                void* stream);

/* Stacked experts: one descriptor for `count` experts of one shape ("Method" section
 * of the QATFactory project page: MoE models merge and quantize expert by expert, each
 * expert with its own tied group).  d describes expert 0; every tensor of expert e
 * follows expert e - 1's contiguously: W [count][rows][ldw], A [count][r][cols],
 * B [count][rows][r], y [count][rows][cols], codes [count][rows][cols/2],
 * scales [count][rows][cols/16], G [count][rows][cols], dA [count][r][cols],
 * dB [count][rows][r].  Expert e's tied group is d.group + e * group_stride.
 * d.M must be NULL (no merge scratch: pass 1 only takes the maximum and pass 2 merges
 * again).  Every expert gives the bits the grouped calls give for it as a descriptor
 * of its own.  Shapes, alignment and errors as the grouped calls, plus QF_ERR_ARG for
 * count < 1, group_stride < 0, M not NULL, an expert's group at or above QF_MAX_GROUPS
 * (or n_groups), or more than 65,535 experts in one call.  Up to QF_MAX_GROUPED
 * descriptors per call: one launch of each kernel covers all their experts. */
typedef struct qf_lora_experts {
  qf_lora_desc d;
  int32_t count;
  int32_t group_stride;
} qf_lora_experts;

size_t qf_lora_experts_workspace(const qf_lora_experts* e, int n);
qf_status qf_lora_experts_layout(const qf_lora_experts* e, int n, int32_t* out);
qf_status qf_lora_experts_merge_tensor_scale_nvfp4(const qf_lora_experts* e, int n, int n_groups, float* d_scales,
                                                   uint32_t* d_nonfinite, void* ws, size_t ws_bytes, void* stream);
qf_status qf_lora_experts_merge_qdq_pack_nvfp4(const qf_lora_experts* e, int n, const float* d_scales,
                                               void* stream);
qf_status qf_lora_experts_adapter_grads(const qf_lora_experts* e, int n, int accumulate, void* ws, size_t ws_bytes,
                                        void* stream);

/* ------------------------------------------------------------ dequant ---- */
/* Packed engine layout -> BF16, the inverse direction of the pack calls ("Method":
 * weights leave training in the engine's own format; "Supported formats" table for
 * what each code and scale stands for).  Each call computes the dequant step of the
 * matching QDQ from the stored bytes, so dequant(pack(x)) is bit for bit the QDQ'd
 * bf16 of x:
 *   NVFP4  y = sign | bf16(fl(fl(E2M1(code) * E4M3(scale)) * s_t)), s_t = *d_scale;
 *   MXFP4  y = sign | bf16(E2M1(code) * 2^(E - 127))  (exact);
 *   Q4_K   y = bf16(fl(D_j q - M_j)), D_j = f32(d) sc_j, M_j = f32(dmin) m_j (exact).
 * Inputs are the contiguous arrays the pack calls write (codes [rows][cols/2], scales
 * [rows][cols/16] or [rows][cols/32], Q4_K blocks [rows][cols/256][144]); y is bf16
 * [rows, ldy], 16-byte aligned with ldy a multiple of 8 and >= cols.  Shapes as the pack
 * calls (cols a multiple of 16 / 32 / 256, rows * cols / 8 < 2^32 - 4096, QF_ERR_SHAPE).  Codes 4-byte aligned, Q4_K
 * blocks 16-byte aligned (QF_ERR_ALIGN).  Scale bytes must be ones a pack call can
 * write (E4M3 0x00..0x7E, E8M0 0x00..0xFE; Q4_K d and dmin finite and >= 0); others
 * give unspecified values. */
qf_status qf_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           const float* d_scale, uint16_t* y, int64_t ldy, void* stream);
qf_status qf_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           uint16_t* y, int64_t ldy, void* stream);
qf_status qf_dequant_q4k(const uint8_t* blocks, int64_t rows, int64_t cols, uint16_t* y, int64_t ldy,
                         void* stream);

/* ------------------------------------------------- W4A4 MXFP4 GEMM ---- */
/* Y = QDQ(X) . QDQ(W)^T with fp32 accumulation and one bf16 rounding of Y
 * ("Overview": weights and optionally activations rounded onto the grid, every
 * matmul in BF16; "Key findings" 02: MXFP4 trains best with W4A4).
 *   X  bf16 [M, ldx] (activations, tokens x hidden), W bf16 [N, ldw] (out x in),
 *   Y  bf16 [M, ldy] output.  QDQ is the MXFP4 rule of qf_qdq_mxfp4 along K,
 *   applied to X when flags has QF_QDQ_A and to W when flags has QF_QDQ_W;
 *   flags == 0 is a plain BF16 GEMM.  The QDQ happens on the way into the
 *   matrix cores: no QDQ'd copy of X or W is written.
 * Constraints: M, N >= 0 (any value; a zero extent is a no-op), K a positive
 * multiple of 64 (QF_ERR_SHAPE), ldx, ldw >= K and ldy >= N; X and W 16-byte
 * aligned with ldx, ldw multiples of 8, Y 2-byte aligned (QF_ERR_ALIGN);
 * M, N < 2^30; ldx, ldw < 2^22 (a 256-row tile's byte offsets stay below 2^31).
 * Output rows are written 8 bytes at a time when ldy is a multiple of 4 and Y is
 * 8-byte aligned, element by element otherwise.
 * Accuracy: fp32 accumulation in an unspecified order; every element obeys
 * |y - y_ref| <= 2^-8 |y_ref| + (1 + 2^-8) gamma_K sum_k |xq_k wq_k|,
 * gamma_K = K 2^-24 / (1 - K 2^-24), against the exact product of the QDQ'd
 * operands. */
#define QF_QDQ_A 1u
#define QF_QDQ_W 2u
/* QF_FP4_CORES (with QF_QDQ_A | QF_QDQ_W only, else QF_ERR_ARG): the same product
 * formed on gfx950's MXFP4 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).  Each
 * QDQ'd MXFP4 value is exactly E2M1(code) * 2^(E - 127), so the cores multiply the
 * very values the BF16 path multiplies, exactly, and accumulate in fp32: the
 * accuracy statement above holds unchanged.  The operands are quantized on the
 * way into LDS (codes and exponents only; nothing is dequantized). */
#define QF_FP4_CORES 4u
/* QF_MX_NOCLIP: quantize the operands under QF_MX_RULE_NOCLIP instead of the floor rule
 * (BF16 cores only, with at least one of QF_QDQ_A / QF_QDQ_W; else QF_ERR_ARG). */
#define QF_MX_NOCLIP 8u
qf_status qf_gemm_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                        uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                        unsigned flags, void* stream);

/* Y = QDQ(X) . dequant(Wc, Ws)^T on the MXFP4 matrix cores, with W already in the
 * packed MXFP4 layout that qf_pack_mxfp4 writes (codes [N][K/2], two per byte,
 * element 2i in the low nibble; E8M0 exponents [N][K/32]; both contiguous).  X is
 * quantized on the way into LDS as in qf_gemm_mxfp4.  With Wc, Ws from
 * qf_pack_mxfp4(W) the result is bit for bit that of qf_gemm_mxfp4(X, W, flags =
 * QF_QDQ_A | QF_QDQ_W | QF_FP4_CORES) and obeys the same bound.  This is the
 * deployment form: the engine-layout weights feed the matrix cores directly.
 * Constraints as qf_gemm_mxfp4; Wc 16-byte aligned, Ws 2-byte aligned. */
qf_status qf_gemm_mxfp4_packed_w(const uint16_t* X, int64_t ldx, const uint8_t* Wc, const uint8_t* Ws,
                                 uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream);

/* Y = dequant(Xc, Xs) . dequant(Wc, Ws)^T on the MXFP4 matrix cores, both operands in
 * the packed layout of qf_pack_mxfp4 (codes [rows][K/2], exponents [rows][K/32],
 * contiguous).  With the operands from qf_pack_mxfp4(X) and qf_pack_mxfp4(W) the result
 * is bit for bit that of qf_gemm_mxfp4_packed_w(X, Wc, Ws) and obeys the same bound.
 * Constraints: K a positive multiple of 128 (QF_ERR_SHAPE); code arrays 16-byte and
 * exponent arrays 4-byte aligned (QF_ERR_ALIGN); ldy >= N; M, N < 2^30. */
qf_status qf_gemm_mxfp4_packed(const uint8_t* Xc, const uint8_t* Xs, const uint8_t* Wc, const uint8_t* Ws,
                               uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream);

/* ------------------------------------------------- W4A4 NVFP4 GEMM ---- */
/* Y = QDQ(X) . QDQ(W)^T on the NVFP4 grid, the same product as qf_gemm_mxfp4 with
 * the NVFP4 rule of qf_qdq_nvfp4 along K ("Supported formats": E2M1 elements, an
 * E4M3 scale per 16-block, an FP32 tensor scale; "Overview": activations may be
 * quantized too).  X is quantized with the tensor scale *d_scale_x and W with
 * *d_scale_w (device fp32 each, e.g. from qf_nvfp4_tensor_scale over the operand, or
 * an activation scale the caller tracks across steps: the kernel reads whatever is
 * there when it runs).  flags: QF_QDQ_A and/or QF_QDQ_W, not 0 (QF_ERR_ARG); the
 * scale of each quantized operand must be given (QF_ERR_NULL).  Everything else as
 * qf_gemm_mxfp4 (constraints, the BF16 matrix cores, the accuracy statement); a scale
 * pointer that is given must be 4-byte aligned (QF_ERR_ALIGN).  There
 * is no FP4-core form: the cores' block scales are E8M0, and NVFP4's are E4M3. */
qf_status qf_gemm_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                        uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                        unsigned flags, const float* d_scale_x, const float* d_scale_w, void* stream);

/* ---------------------------------------- forward of the quantized linear ---- */
/* Y = QDQ(X) . QDQ(W)^T, the product of qf_gemm_mxfp4 / qf_gemm_nvfp4, in two passes
 * ("Overview": weights and optionally activations rounded onto the grid, every matmul
 * in BF16; "Method", "Framework overview": the forward applies the QDQ transform):
 *   1. Xq = QDQ(X) when flags has QF_QDQ_A and Wq = QDQ(W) when flags has QF_QDQ_W,
 *      written to the caller's bf16 buffers Xq [M, ldxq] and Wq [N, ldwq] by the
 *      streaming QDQ kernels (the rules of qf_qdq_mxfp4, or qf_qdq_nvfp4 with the
 *      tensor scales *d_scale_x / *d_scale_w);
 *   2. Y = Xq . Wq^T on the BF16 matrix cores (the kernel of qf_gemm_mxfp4 with
 *      flags 0; an operand that is not flagged is read as given).
 * Y is bit for bit that of qf_gemm_mxfp4 (qf_gemm_nvfp4) with the same flags and
 * obeys the same bound.  On MI355X this order is faster than quantizing inside the
 * GEMM: the fused kernel re-quantizes every operand tile for each tile of Y that
 * reads it, while here each element is quantized once, and Xq / Wq stay available
 * for the backward products (qf_linear_backward_mxfp4 with flags 0 on them).
 * Arguments: as qf_gemm_mxfp4 (flags QF_QDQ_A, QF_QDQ_W, QF_MX_NOCLIP there) or
 * qf_gemm_nvfp4 (flags QF_QDQ_A and/or QF_QDQ_W, not 0, and the flagged operands'
 * scales, 4-byte aligned); a flagged operand's buffer is required (QF_ERR_NULL),
 * 16-byte aligned with its leading dimension a multiple of 8 and >= K, < 2^22; an
 * unflagged one's buffer is ignored.  Xq may be X (ldxq == ldx: X is overwritten by
 * its QDQ), likewise Wq and W; no other overlap is allowed.  Every argument is
 * checked before the first of the three launches on `stream`. */
qf_status qf_linear_forward_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                  uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K, unsigned flags,
                                  uint16_t* Xq, int64_t ldxq, uint16_t* Wq, int64_t ldwq, void* stream);
qf_status qf_linear_forward_nvfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                  uint16_t* Y, int64_t ldy, int64_t M, int64_t N, int64_t K, unsigned flags,
                                  const float* d_scale_x, const float* d_scale_w,
                                  uint16_t* Xq, int64_t ldxq, uint16_t* Wq, int64_t ldwq, void* stream);

/* -------------------------------------- backward of the quantized linear ---- */
/* "Method", "Framework overview": the backward pass reaches the latent weights through
 * the STE, so the layer Y = Xq . Wq^T (Xq, Wq the MXFP4-QDQ'd operands, or the raw ones
 * for an operand the forward did not quantize) has dX = dY . Wq and dWq = dY^T . Xq;
 * qf_ste_backward then carries dWq to the fp32 latent weights.
 *
 * qf_transpose_bf16: y [cols, rows] = x [rows, cols]^T, MXFP4-QDQ'd along cols first
 * when qdq_mxfp4 is 1 (the floor rule of qf_qdq_mxfp4) or 2 (QF_MX_RULE_NOCLIP); 0 copies,
 * other values give QF_ERR_ARG.  rows and cols multiples of 8 (cols of 32 with
 * qdq_mxfp4), rows < 2^22, ldx >= cols, ldy >= rows (QF_ERR_SHAPE); x, y 16-byte aligned
 * with ldx, ldy multiples of 8 (QF_ERR_ALIGN); y must not overlap x.  The result is exact
 * (a copy, or QDQ values that are exactly those of qf_qdq_pack_mxfp4_rule). */
qf_status qf_transpose_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint16_t* y, int64_t ldy,
                            int qdq_mxfp4, void* stream);

/* dX [M, K] = dY [M, N] . Wq and dW [N, K] = dY^T . Xq for X [M, K], W [N, K], with Xq /
 * Wq = QDQ(X) / QDQ(W) when flags has QF_QDQ_A / QF_QDQ_W (the forward's flags), else
 * the operands themselves.  Five launches on `stream`: Wq^T, dY^T and Xq^T into the
 * workspace (qf_transpose_bf16), then the two products on the BF16 matrix cores
 * (qf_gemm_mxfp4 with flags 0).  QF_MX_NOCLIP (with QF_QDQ_A and/or QF_QDQ_W, else
 * QF_ERR_ARG) quantizes under the noclip rule, matching a forward run with that flag.
 * dX or dW may be NULL to skip it.  Shapes: M and N
 * multiples of 64 (the products' reduction lengths), K a multiple of 32, M, N, K and
 * the leading dimensions < 2^22; leading dimensions >= the row lengths, multiples of 8;
 * all arrays 16-byte aligned, the workspace 256-byte aligned.  Accuracy: each output element obeys the bound of qf_gemm_mxfp4 with the
 * reduction length N (dX) or M (dW). */
size_t qf_linear_backward_workspace(int64_t M, int64_t N, int64_t K);
qf_status qf_linear_backward_mxfp4(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                   const uint16_t* dY, int64_t lddy, uint16_t* dX, int64_t lddx,
                                   uint16_t* dW, int64_t lddw, int64_t M, int64_t N, int64_t K,
                                   unsigned flags, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- no-allocation variant ---- */
/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qf_nvfp4_tensor_scale_grouped with
 * its amax partials in a fixed array the library keeps on each GPU (allocated with the
 * code object, held until the process ends) instead of a caller workspace.  Same
 * arguments, checks, kernels and bits as qf_nvfp4_tensor_scale_grouped.  Limit: the call's
 * workspace need (qf_nvfp4_tensor_scale_workspace(d, n)) must not exceed
 * qf_noalloc_scratch_bytes() = 128 KiB, i.e. at most 16 groups with a tensor (group
 * indices below 16) for large launches, else QF_ERR_WORKSPACE before anything runs.  The
 * call allocates nothing; its first call on a device looks up that device's array.  Calls
 * on one GPU share the array: calls that overlap on the same GPU (different streams, or
 * host threads) race and must be serialized by the caller. */
size_t qf_noalloc_scratch_bytes(void);
qf_status qf_nvfp4_tensor_scale_grouped_noalloc(const qf_tensor_desc* d, int n, int n_groups, float* d_scales,
                                                uint32_t* d_nonfinite, void* stream);

/* ------------------------------------------------ checkpoint containers ---- */
/* "Method", "Export" on the project page: NVFP4 / MXFP4 checkpoints go to vLLM in the
 * compressed-tensors layout and Q4_K to llama.cpp as GGUF, so that the engine loads the
 * trained codes and scales with no extra lossy conversion (and the saved NVFP4 activation
 * scales need no calibration pass).  The pages fix neither container; these writers take
 * HOST buffers (copy the packed device arrays first) and write plain files.
 *
 * qf_write_safetensors: the safetensors container -- an 8-byte little-endian header
 * length N, N bytes of JSON {name: {"dtype", "shape", "data_offsets": [begin, end]}, ...,
 * "__metadata__": {key: value}} padded with spaces to a multiple of 8, then each tensor's
 * bytes in the order given (offsets relative to the end of the header).  dtype is a
 * safetensors dtype string: "U8", "I8", "BOOL", "F8_E4M3", "F8_E5M2", "F8_E8M0", "U16",
 * "I16", "F16", "BF16", "U32", "I32", "F32", "U64", "I64", "F64"; the data holds
 * product(shape) elements of it.  The metadata map (n_meta pairs, may be 0) holds strings.
 * Errors: QF_ERR_NULL (path, a name, dtype, key, value, or data of a non-empty tensor
 * missing), QF_ERR_ARG (unknown dtype, empty or repeated name, the name "__metadata__",
 * negative counts), QF_ERR_SHAPE (ndim outside 0..8, a negative extent), QF_ERR_IO (the file
 * cannot be written).  The file is only created once the arguments are checked.
 *
 * Names and the scale convention of the NVFP4 / MXFP4 tensors this library's binding
 * writes ("compressed-tensors-style"; byte compatibility with an engine's loader is
 * unpinned): <layer>.weight_packed U8 [rows, cols/2] (codes as qf_pack_*), <layer>.
 * weight_scale F8_E4M3 [rows, cols/16] or F8_E8M0 [rows, cols/32], <layer>.
 * weight_global_scale F32 [1] = the dequant multiplier s_t of the layer's tied group,
 * <layer>.input_global_scale F32 [1] = the tracked activation s_t (W4A4). */
typedef struct qf_st_tensor {
  const char* name;      /* UTF-8, unique within the file                   */
  const char* dtype;     /* safetensors dtype string                        */
  int32_t ndim;          /* 0..8                                            */
  const int64_t* shape;  /* host int64[ndim], row-major, outermost first    */
  const void* data;      /* HOST bytes, product(shape) * dtype size         */
} qf_st_tensor;
qf_status qf_write_safetensors(const char* path, const qf_st_tensor* t, int n, const char* const* meta_keys,
                               const char* const* meta_values, int n_meta);

/* qf_write_gguf: a GGUF-style container -- uint32 magic 0x46554747 ("GGUF"), uint32
 * version 3, uint64 tensor count, uint64 key-value count; each key-value pair as a string
 * key (uint64 length + bytes), uint32 type 8 (string) and a string value; each tensor info
 * as a string name, uint32 ndim (1..4), uint64 extents innermost first, uint32 type,
 * uint64 offset of its data; zero padding to a multiple of 32 bytes; then each tensor's
 * nbytes at its offset (multiples of 32, zero padded).  For this library's Q4_K blocks
 * (qf_pack_q4k, [rows, cols/256, 144]) the binding writes type 12 with extents {cols, rows}
 * and a key "qf.q4k.block_layout" describing the 144-byte block (d, dmin, the 96-bit
 * sc/m stream, element 2i in the low nibble): whether an engine reads these blocks the
 * same way is unpinned.  Errors as qf_write_safetensors (QF_ERR_SHAPE for ndim outside
 * 1..4 or a negative extent). */
typedef struct qf_gguf_tensor {
  const char* name;
  int32_t ndim;          /* 1..4                                            */
  const int64_t* dims;   /* host int64[ndim], innermost (contiguous) first  */
  uint32_t type;         /* the file's tensor type code                     */
  const void* data;      /* HOST bytes                                      */
  uint64_t nbytes;
} qf_gguf_tensor;
qf_status qf_write_gguf(const char* path, const qf_gguf_tensor* t, int n, const char* const* kv_keys,
                        const char* const* kv_values, int n_kv);

/* ---------------------------------------------------- conformance test ---- */
/* Checks on the device that the gfx950 instructions and shortcuts the kernels
 * rely on agree bit for bit with the software definitions above, over their
 * whole input domains:
 *   [0] v_cvt_pk_bf16_f32 vs bf16 RNE, every finite fp32
 *   [1] v_cvt_scalef32_pk_fp4_f32 (scale 1) vs E2M1 RNE-saturating, every non-NaN fp32
 *   [2] v_cvt_scalef32_pk_fp4_bf16 with an E8M0 scale, every bf16 x every E
 *   [3] v_cvt_scalef32_pk_fp4_f32 with an E8M0 scale, every bf16 x every E
 *   [4] v_cvt_scalef32_pk_bf16_fp4, every code x every E
 *   [5] v_cvt_scalef32_pk_f32_fp4, every code x every E, and with scale 1
 *   [6] v_cvt_f16_f32 after clamping to 65504 vs fp16 RNE-saturating, every fp32 >= 0;
 *       v_cvt_f32_f16 vs the exact fp16 value, every finite non-negative fp16
 *   [7] FMA-corrected division by 15 and by 63 vs IEEE division, every fp32 >= 0
 * d_counts: device uint64[8], zeroed by the caller; entry i receives the
 * number of mismatches of check i (all zero on a conforming device). */
qf_status qf_selftest_conversions(unsigned long long* d_counts, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QF_H */
