/*
 * rfpx.h -- C ABI of librfpx: one routed-MoE layer over block-quantized
 * experts on an AMD MI355X (gfx950), decode (q = 1..8 verify columns) and a
 * prefill chunk.
 *
 * Pages cited below:
 *   [P2] "APU 实现 token 自由：AMD Ryzen AI MAX+ 395 跑 DeepSeek V4 Flash，284B
 *        模型跑出 32 tok/s" (ainomam.com), section "Lucebox 的优化三板斧".
 *   [P3] "DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s"
 *        (taozi.news), sections "ROCmFPX：把 284B 权重压进 128 GB",
 *        "解码：32 tok/s" and "稀疏预填充：约 250 tok/s".
 *   [P5] "Lucebox专攻DeepSeek V4：DSpark草稿模型、MoE专家并行与ROCmFPX量化达成
 *        42 tok/s" (m.mzlw.cn), sections "MoE 专家并行" and "ROCmFPX 量化".
 *
 * ---------------------------------------------------------------- formats
 * [P3] "ROCmFPX": a family of block formats, each block holding the low-bit
 * codes of 32 weights and a scale; ROCmFP2 takes 10 bytes per block (2.50
 * bit/weight), ROCmFP3 about 3.50 bit/weight, ROCmFP4 ("fast path") about
 * 4.25 bit/weight.  The pages stop at block size; this library fixes the bit
 * layout of one canonical block as:
 *
 *   FP2, 10 B: bytes 0..7 = 32 2-bit codes, code j in bits 2(j%4)..2(j%4)+1
 *              of byte j/4; bytes 8..9 = IEEE fp16 scale s, little-endian.
 *              w_j = (code_j - 1.5) * s          codebook {-1.5,-0.5,0.5,1.5}
 *   FP3, 14 B: bytes 0..11 = one little-endian 96-bit integer, code j in its
 *              bits 3j..3j+2 (codes 10 and 21 straddle bytes); bytes 12..13 =
 *              fp16 scale s.   w_j = (code_j - 3.5) * s
 *   FP4, 17 B: bytes 0..15 = 32 4-bit codes, code j in the low nibble of byte
 *              j/2 for even j, the high nibble for odd j; byte 16 = E8M0
 *              exponent e.     w_j = (code_j - 7.5) * 2^(e-127)
 *
 * A row-major matrix of R rows and C columns (C a multiple of 32) is R*C/32
 * canonical blocks, block b of row r covering columns 32b..32b+31.  Every
 * dequantized weight is exact in fp32.
 *
 * [P3] "ROCmFPX" and [P2]: routed gate and up use FP2, routed down FP3,
 * dense or sensitive projections FP4 or wider; [P5] "ROCmFPX 量化": the width
 * may also be chosen per expert by routing hotness.  The library accepts any
 * of the three formats for any matrix, with gate and up of one expert in the
 * same format.
 *
 * ------------------------------------------------------------ the layer
 * [P5] "MoE 专家并行": each layer routes to 6 of 256 experts and adds 1
 * shared expert.  For every column c of x[q][d]:
 *   s[c][e]  = sum_i Wr[e][i] * x[c][i]                     (router, fp32)
 *   ids[c]   = the k experts of largest score, score descending, ties to the
 *              lower index                                    (TOP-K/ARGSORT, [P2])
 *   w[c][j]  = routed_scale * softmax over the k selected scores
 *   o_e      = Down_e ( silu(Gate_e x_c) * (Up_e x_c) )      (SiLU-gated FFN)
 *   y[c]     = sum_j w[c][j] * o_ids[c][j]  +  o_shared
 * Decode (q columns, [P3] "解码"): each packed block an expert needs is read
 * and decoded once per call and applied to every column that selected that
 * expert ([P2]: in the q=4 verify path each packed weight is decoded once
 * for all 4 columns).  Dequantized weights are exact.  bf16 activations
 * enter the products as they are; fp32 activations, and the hidden vector h
 * of every expert, enter as a bf16 hi + bf16 lo pair (relative residual
 * below 2^-16).  Every product is exact and sums are fp32, so results
 * differ from an exact evaluation by fp32 summation order and that
 * residual.
 *
 * ------------------------------------------------------------ conventions
 * - Every pointer named *_dev, and every pointer inside moe_layer except
 *   fmts, is device memory of the current HIP device, allocated and freed by
 *   the caller.  Host pointers are named *_host.
 * - The library never allocates or frees device memory, keeps no state
 *   between calls and never synchronizes the stream, except where a function
 *   says so.  Work is enqueued on `stream` (a hipStream_t; NULL = default).
 * - Every function validates its arguments on the host before enqueueing
 *   anything and returns an rfpx_status; nothing is launched on error.
 *   rfpx_last_error() then gives a message (thread-local).  A failed kernel
 *   launch returns RFPX_E_HIP.  Faults inside kernels surface at the caller's
 *   next synchronization.
 * - Calls that share a workspace must not overlap in time; calls with
 *   separate workspaces may run concurrently.
 */
#ifndef RFPX_H
#define RFPX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RFPX_FP2 = 2, RFPX_FP3 = 3, RFPX_FP4 = 4 } rfpx_fmt;
typedef enum { RFPX_X_F32 = 0, RFPX_X_BF16 = 1 } rfpx_xtype;
typedef enum {
  RFPX_OK = 0,
  RFPX_E_ARG = -1,       /* null pointer, bad enum, bad count */
  RFPX_E_SHAPE = -2,     /* unsupported d, f, E, k, q or T */
  RFPX_E_ALIGN = -3,     /* pointer not aligned as required */
  RFPX_E_FORMAT = -4,    /* bad format table or image header */
  RFPX_E_WORKSPACE = -5, /* workspace or output capacity too small */
  RFPX_E_HIP = -6        /* a HIP call failed */
} rfpx_status;

/* Compile-time limits of the library. */
#define RFPX_Q_MAX 8    /* verify columns per decode call */
#define RFPX_K_MAX 8    /* routed experts per column */
#define RFPX_E_MAX 1024 /* routed experts per layer */

/* Bytes of one canonical block: 10, 14, 17; 0 for an unknown format. */
size_t rfpx_block_bytes(int fmt);
/* rows * cols/32 * block bytes; 0 if cols is not a multiple of 32. */
size_t rfpx_matrix_bytes(int fmt, int rows, int cols);

/* Quantize w_dev[rows][cols] (fp32, finite) into canonical blocks at
 * out_dev (capacity cap bytes).  Per block: a = max|w|; FP2/FP3 scale s =
 * fp16 nearest-even of a/1.5 (a/3.5), 65504 on overflow, and if s rounds to
 * 0 (or a = 0) the block is all-zero bytes; codes = nearest-even integer of
 * w/s + offset, clamped.  FP4: e = clamp(127 + ceil(log2(a/7.5)), 1, 254),
 * codes = nearest-even of w*2^(127-e) + 7.5, clamped; a = 0 gives all-zero
 * bytes.  Divisions and roundings are done in double on the device.
 * Requires cols % 32 == 0, rows >= 0. */
rfpx_status rfpx_pack(int fmt, const float *w_dev, int rows, int cols,
                      uint8_t *out_dev, size_t cap, void *stream);
/* Importance-weighted quantizer ([P3] "ROCmFPX": weights are quantized with
 * an importance matrix).  imp_dev[cols] >= 0 (finite) is the importance of
 * each input column; block b of every row uses imp_dev[32b .. 32b+31].  Per
 * block, with a = max|w|, the stored scale is the candidate of least
 *     E(s) = sum_j imp_j * (w_j - (c_j - offset) * s)^2,
 * codes c_j = nearest-even of w_j/s + offset, clamped, from the stored s.
 * Candidates, tried in this order (a tie keeps the earlier one):
 *   FP2/FP3: s = fp16 nearest-even of a / (offset * t), 65504 on overflow,
 *            t = 1, 1+1/16, 1-1/16, 1+2/16, 1-2/16, ..., 1+8/16, 1-8/16
 *            (t = 1 is rfpx_pack's absmax scale); s = 0 and repeats skipped;
 *   FP4:     E8M0 e = e0, e0-1, e0+1 clamped to [1, 254], repeats skipped,
 *            e0 = rfpx_pack's exponent.
 * E is evaluated in double, term by term in column order, each operation
 * rounded on its own.  a = 0 (or no candidate) gives all-zero bytes.  With
 * every importance 0 the result equals rfpx_pack's. */
rfpx_status rfpx_pack_weighted(int fmt, const float *w_dev, const float *imp_dev,
                               int rows, int cols, uint8_t *out_dev, size_t cap,
                               void *stream);
/* Bit-pack codes_dev[rows][cols] (one code per byte, only the low 2/3/4
 * bits are used) and scale_bits_dev[rows][cols/32] (fp16 bit patterns for
 * FP2/FP3, E8M0 in the low byte for FP4) into canonical blocks.  Scale bits
 * are device data and are packed as given: a non-finite scale (fp16 Inf or
 * NaN, E8M0 = 255) is not rejected here; moe_image_validate reports every
 * such block of an image built from these blocks. */
rfpx_status rfpx_pack_codes(int fmt, const uint8_t *codes_dev,
                            const uint16_t *scale_bits_dev, int rows, int cols,
                            uint8_t *out_dev, size_t cap, void *stream);
/* Dequantize canonical blocks into w_dev[rows][cols] fp32 (exact). */
rfpx_status rfpx_unpack(int fmt, const uint8_t *in_dev, int rows, int cols,
                        float *w_dev, void *stream);

/* ------------------------------------------------------- device image
 * The layer's experts live in one device buffer, the image:
 *   header (64 B) | expert table (E+1) x 64 B | planes
 * Experts are stored expert-major (0..E-1 routed, E = shared).  Each matrix
 * (gate f x d, up f x d, down d x f) is split into a codes plane (rows x
 * cols/32 x 8|12|16 bytes, row-major) and a scales plane (rows x cols/32 x
 * 2|1 bytes); every plane starts on a 256-byte boundary.  The byte count of
 * the planes equals the canonical byte count: the image is a permutation of
 * the canonical blocks plus the header, table and alignment gaps. */
size_t moe_image_bytes(int d, int f, int n_experts, const int *fmts_host);

/* Build the image from canonical matrices.  fmts_host[3*e + m] is the format
 * of matrix m (0 gate, 1 up, 2 down) of expert e, e = 0..n_experts (the last
 * is the shared expert); canonical_host[3*e + m] is a host array of device
 * pointers to those canonical matrices.  image_dev must be 256-byte aligned
 * and hold moe_image_bytes().  Gate and up of an expert must share a format.
 * Enqueues one copy kernel per matrix; the canonical buffers may be freed
 * once the stream has passed this call. */
rfpx_status moe_image_build(int d, int f, int n_experts, const int *fmts_host,
                            const uint8_t *const *canonical_host,
                            uint8_t *image_dev, size_t cap, void *stream);

typedef struct {
  int d;              /* model width, a power of two from 256 to 4096 */
  int f;              /* expert width, a power of two from 64 to 4096 */
  int n_experts;      /* routed experts E, 1..RFPX_E_MAX */
  int top_k;          /* k, 1..min(E, RFPX_K_MAX) */
  float routed_scale; /* multiplies the k gating weights (1.0) */
  const float *router_w;  /* device, [E][d] fp32 */
  const uint8_t *image;   /* device, built by moe_image_build for fmts */
  const int *fmts;        /* host, [(E+1)*3], the table the image was built with */
  size_t image_bytes;     /* bytes of the image buffer: must equal
                             moe_image_bytes(d, f, n_experts, fmts) */
} moe_layer;

/* Checks made on the host by every call that takes a moe_layer (before
 * any launch): shapes and limits, the format table (known formats, gate
 * and up of an expert alike), 256-byte alignment of the image and
 * image_bytes == moe_image_bytes(d, f, n_experts, fmts) (RFPX_E_FORMAT
 * otherwise).  The contents of the image are not read on the host; they
 * are checked on the device by moe_image_validate, once per image.  Layer
 * kernels skip, and leave no output for, any expert whose device table
 * entry names a format absent from fmts. */

/* Check an image on the device against L: its header, its expert table and
 * every block scale ([P3] "ROCmFPX": FP2/FP3 blocks carry an fp16 scale, FP4
 * blocks an E8M0 power of two).  Writes report_dev[4] (uint32, device,
 * 4-byte aligned; overwritten, no initialization needed):
 *   [0] header faults, a bit set: 1 magic, 2 version, 4 d, f or E differ
 *       from L, 8 the recorded byte count differs from L->image_bytes;
 *   [1] expert-table entries (expert, matrix) whose format or plane offsets
 *       differ from the layout of L->fmts;
 *   [2] blocks whose scale is not a finite number: an fp16 Inf or NaN
 *       (FP2, FP3), or E8M0 = 255 (FP4; NaN in the OCP MX encoding);
 *   [3] 0.
 * All four zero: the layer kernels can use the image.  Two kernels on
 * `stream` (the scan reads every scales plane: about 2.5% of the image);
 * the report is valid once the stream has passed them.  Scales are read at
 * the offsets that L->fmts implies, never at offsets read from the image,
 * so a damaged table cannot send the scan outside the buffer. */
rfpx_status moe_image_validate(const moe_layer *L, uint32_t *report_dev, void *stream);

/* Dequantize matrix m of expert e straight from the image into w_dev
 * (rows x cols fp32) -- a check of the image layout. */
rfpx_status moe_image_unpack(const moe_layer *L, int expert, int matrix,
                             float *w_dev, void *stream);

/* Workspace for moe_route_topk / moe_layer_forward with q columns
 * (prefill = 0), or for moe_prefill_forward with T tokens (prefill = 1);
 * 0 if the shape is unsupported.  The workspace must be 256-byte aligned;
 * its contents need no initialization and are scratch between calls. */
size_t moe_workspace_bytes(const moe_layer *L, int q_or_T, int prefill);

/* Router scores, top-k and gating for q columns of x_dev ([q][d] fp32 or
 * bf16 per xtype): ids_dev[q][k] int32 (score descending, ties to the lower
 * index) and w_dev[q][k] fp32.  Reads only router_w: L->image and
 * L->image_bytes are neither read nor checked (either may be 0). */
rfpx_status moe_route_topk(const moe_layer *L, const void *x_dev, int xtype,
                           int q, int32_t *ids_dev, float *w_dev, void *ws_dev,
                           size_t ws_bytes, void *stream);

/* One decode step of the layer for q = 1..RFPX_Q_MAX columns: y_dev[q][d]
 * fp32.  Each column is routed independently; each expert block is read
 * once and applied to all columns that chose the expert. */
rfpx_status moe_layer_forward(const moe_layer *L, const void *x_dev, int xtype,
                              int q, float *y_dev, void *ws_dev,
                              size_t ws_bytes, void *stream);

/* moe_layer_forward that also stamps six caller-created hipEvent_t handles
 * (timing enabled, current device) with the start and end times of its
 * kernels, as hipExtLaunchKernel does: events[0] when the router-score
 * kernel starts, events[1] when the last routing kernel ends (the router
 * scores, or the route table of a step of several columns), events[2] and
 * events[3] when the gate/up kernel starts and ends, events[4] and events[5]
 * when the down-and-combine kernel starts and ends.  hipEventElapsedTime of
 * such a pair is the kernel's own duration, without launch gaps.  For
 * measuring each kernel of a step inside a timed loop; events may be NULL
 * (then it is moe_layer_forward). */
rfpx_status moe_layer_forward_timed(const moe_layer *L, const void *x_dev,
                                    int xtype, int q, float *y_dev,
                                    void *ws_dev, size_t ws_bytes,
                                    void *stream, void *const *events);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is the library's own device scratch of
 * moe_noalloc_scratch_bytes() bytes (8 MiB), one per GPU, held until the
 * process ends.  Nothing is allocated or freed; the caller passes x_dev and
 * y_dev as for moe_layer_forward.  A shape whose workspace
 * (moe_workspace_bytes for the given xtype) exceeds the scratch is rejected
 * with RFPX_E_WORKSPACE before any launch; the spec shapes (d = 4096,
 * f = 2048, E = 256, k = 6, q <= 8) fit, the largest shapes (d = f = 4096,
 * k = q = 8) do not.  The scratch needs no initialization (the step writes
 * everything it reads).  All calls on one GPU share its scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and must
 * be serialized by the caller. */
rfpx_status moe_layer_forward_noalloc(const moe_layer *L, const void *x_dev, int xtype,
                                      int q, float *y_dev, void *stream);
/* Bytes of the scratch moe_layer_forward_noalloc uses (8 MiB). */
size_t moe_noalloc_scratch_bytes(void);

/* One prefill chunk of T tokens (x_dev [T][d] bf16 or fp32): tokens are
 * grouped by expert and each expert runs as a dense grouped product on the
 * matrix cores.  y_dev[T][d] fp32.  ([P3] "稀疏预填充": prefill is batched per
 * layer.)  T in [1, 65536]; d a multiple of 128 and f of 64; the image at
 * most 4 GiB; x_dev and y_dev 16-byte aligned; ws_bytes at least
 * moe_workspace_bytes(L, T, 1).  A violated limit returns RFPX_E_SHAPE /
 * RFPX_E_ALIGN / RFPX_E_WORKSPACE before any launch. */
rfpx_status moe_prefill_forward(const moe_layer *L, const void *x_dev,
                                int xtype, int T, float *y_dev, void *ws_dev,
                                size_t ws_bytes, void *stream);

/* moe_prefill_forward that also stamps six caller-created hipEvent_t
 * handles (timing enabled, current device) as moe_layer_forward_timed does:
 * events[0] when the router-score kernel starts, events[1] when the
 * expert-grouping kernels end, events[2] and events[3] when the grouped
 * gate/up product starts and ends, events[4] when the grouped down product
 * starts and events[5] when the combine kernel ends.  events may be NULL
 * (then it is moe_prefill_forward). */
rfpx_status moe_prefill_forward_timed(const moe_layer *L, const void *x_dev,
                                      int xtype, int T, float *y_dev,
                                      void *ws_dev, size_t ws_bytes,
                                      void *stream, void *const *events);

/* ------------------------------------------------- dense projections
 * [P2] "Lucebox 的优化三板斧": in the q-column verify step each packed dense
 * weight is decoded once and applied to all columns; [P3] "ROCmFPX": dense
 * and sensitive projections stay ROCmFP4 or wider.  A dense matrix W of
 * rows x cols (rows a multiple of 64, cols a multiple of 32 -- of 64 for
 * FP2 -- and at most 65536) lives in a dense image, a permutation of its
 * canonical blocks: tiles of 64 rows; within a tile, chunk k (one block,
 * two for FP2) of the 64 rows stored contiguously, row r of the tile at
 * position r:
 *   codes plane  [rows/64][chunks][64][16 | 12 | 16 bytes]
 *   scales plane [rows/64][chunks][64][4 | 2 | 1 bytes], 256-byte aligned.
 * Bytes of that image; 0 for an unsupported shape or format. */
size_t rfpx_dense_image_bytes(int fmt, int rows, int cols);
/* Build the dense image from canonical blocks canonical_dev (rows x cols/32
 * blocks, row-major); image_dev 256-byte aligned, cap >= the image bytes. */
rfpx_status rfpx_dense_image_build(int fmt, const uint8_t *canonical_dev, int rows,
                                   int cols, uint8_t *image_dev, size_t cap, void *stream);
/* Dequantize W from its dense image into w_dev[rows][cols] fp32 (exact). */
rfpx_status rfpx_dense_image_unpack(int fmt, const uint8_t *image_dev, int rows, int cols,
                                    float *w_dev, void *stream);
/* Workspace of rfpx_dense_forward with q columns (any xtype); 0 if
 * unsupported.  256-byte aligned, no initialization needed. */
size_t rfpx_dense_workspace_bytes(int fmt, int rows, int cols, int q);
/* y_dev[c][r] = sum_j W[r][j] x_dev[c][j] for c < q (1..RFPX_Q_MAX): x_dev
 * [q][cols] bf16 or fp32 (16-byte aligned; fp32 enters as a bf16 hi + lo
 * pair), y_dev [q][rows] fp32.  Every block is read and decoded once and
 * applied to all q columns; products are exact, sums fp32 in a fixed
 * order (y is the same bit for bit from run to run). */
rfpx_status rfpx_dense_forward(int fmt, const uint8_t *image_dev, int rows, int cols,
                               const void *x_dev, int xtype, int q, float *y_dev,
                               void *ws_dev, size_t ws_bytes, void *stream);

/* ------------------------------------------------------- measurement
 * A plain streaming read of bytes at src_dev (16-byte aligned, a non-zero
 * multiple of 16 bytes): the achievable HBM ceiling for a read of that size,
 * launch included, which the layer kernels are compared with ([P5]
 * "新手常见疑问": decode is bound by memory bandwidth).  One kernel: eight
 * 16-byte loads in flight per thread, at most rfpx_stream_read_sink_words()
 * workgroups; workgroup w writes the XOR of the 32-bit words it read to
 * sink_dev[w] (the XOR of all written words is the XOR of the buffer's
 * words; sink_dev must hold rfpx_stream_read_sink_words() words). */
rfpx_status rfpx_stream_read(const void *src_dev, size_t bytes, uint32_t *sink_dev,
                             void *stream);
size_t rfpx_stream_read_sink_words(void);

const char *rfpx_status_str(int status);
const char *rfpx_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RFPX_H */
