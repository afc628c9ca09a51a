/*
 * oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU reference for one routed-MoE layer whose experts are
 * stored as ROCmFP2 / ROCmFP3 / ROCmFP4 blocks of 32 weights.  It exists so
 * that the GPU library can be checked against something written
 * independently: it shares no code, header, table or helper with the library
 * under block_quantized_expert_amd/, and the library never includes or links
 * it.  Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg may load it.
 *
 * Everything is computed in double and the layer output is rounded to fp32
 * exactly once.  Pages referred to in the comments:
 *   [P2] "APU 实现 token 自由：AMD Ryzen AI MAX+ 395 跑 DeepSeek V4 Flash，284B
 *        模型跑出 32 tok/s" (ainomam.com), section "Lucebox 的优化三板斧".
 *   [P3] "DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s"
 *        (taozi.news), sections "ROCmFPX：把 284B 权重压进 128 GB" and
 *        "解码：32 tok/s".
 *   [P5] "Lucebox专攻DeepSeek V4：DSpark草稿模型、MoE专家并行与ROCmFPX量化达成
 *        42 tok/s" (m.mzlw.cn), sections "MoE 专家并行" and "ROCmFPX 量化".
 *
 * Block formats (32 weights per block; sizes and bits/weight from [P3]
 * "ROCmFPX"; the bit layout is the one this project fixes):
 *   FP2 (10 B): bytes 0..7 hold 32 2-bit codes, code j in bits 2(j%4)..+1 of
 *               byte j/4; bytes 8..9 a little-endian IEEE fp16 scale s.
 *               weight_j = (code_j - 1.5) * s
 *   FP3 (14 B): bytes 0..11 are one little-endian 96-bit integer; code j is
 *               its bits 3j..3j+2; bytes 12..13 an fp16 scale s.
 *               weight_j = (code_j - 3.5) * s
 *   FP4 (17 B): bytes 0..15 hold 32 4-bit codes, code j in the low nibble of
 *               byte j/2 when j is even, the high nibble when odd; byte 16 is
 *               an E8M0 exponent e.
 *               weight_j = (code_j - 7.5) * 2^(e-127)
 * A matrix of R rows and C columns (C a multiple of 32) is R*C/32 blocks in
 * row-major order; block b of row r covers columns 32b..32b+31.
 */
#ifndef BQE_ORACLE_H
#define BQE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP2 = 2, ORC_FP3 = 3, ORC_FP4 = 4 };

/* Bytes in one block: 10, 14 or 17; 0 for an unknown format. */
int orc_block_bytes(int fmt);

/* fp16 bit pattern -> exact double (handles subnormals, inf, nan). */
double orc_half_to_double(uint16_t h);
/* bf16 bit pattern -> exact double. */
double orc_bf16_to_double(uint16_t b);
/* double -> fp16 bit pattern, round to nearest even, overflow -> inf. */
uint16_t orc_double_to_half_rne(double v);

/* Decode one block into its 32 codes and the block's scale multiplier. */
void orc_block_codes(int fmt, const uint8_t *blk, int codes[32], double *scale);
/* Decode one block into 32 weights. */
void orc_decode_block(int fmt, const uint8_t *blk, double w[32]);
/* Dequantize a whole row-major matrix into w[rows*cols]. */
void orc_unpack(int fmt, const uint8_t *bytes, int rows, int cols, double *w);

/* Bit-pack codes (one per byte, already in range) and per-block scale bits
 * (fp16 bits for FP2/FP3, the E8M0 byte for FP4) into canonical blocks. */
void orc_pack_codes(int fmt, const uint8_t *codes, const uint16_t *scale_bits,
                    int rows, int cols, uint8_t *out);
/* Quantize fp32 weights (finite) into canonical blocks: absmax scale per
 * block, codes rounded to nearest even from the rounded scale. */
void orc_pack(int fmt, const float *w, int rows, int cols, uint8_t *out);

/* Importance-weighted quantizer: per block the scale, among a fixed list
 * of candidates around the absmax scale, that minimizes
 * sum_j imp[col_j] * (w_j - dequantized w_j)^2 (oracle.c states the list
 * and the tie rule); codes nearest from the stored scale.  imp[cols] >= 0
 * is the importance of each input column. */
void orc_pack_weighted(int fmt, const float *w, const float *imp, int rows,
                       int cols, uint8_t *out);

/* Dense q-column product y[c][r] = sum_j W[r][j] x[c][j] for a row-major
 * block-quantized matrix W (rows x cols canonical blocks) and q columns of
 * x (fp32, xtype 0, or bf16 bits, xtype 1); y[q][rows] fp32. */
void orc_dense_forward(int fmt, const uint8_t *w, int rows, int cols,
                       const void *x, int xtype, int q, float *y);

/* Router scores s[c][e] = sum_i wr[e][i] * x[c][i]. */
void orc_router_scores(const double *x, int q, int d, const float *wr, int E,
                       double *s);
/* First k experts of the order (score descending, index ascending). */
void orc_topk(const double *s, int E, int k, int32_t *ids);
/* Softmax over the k selected scores, times routed_scale. */
void orc_gating(const double *s, const int32_t *ids, int k,
                double routed_scale, double *w);

/* One expert FFN on one column: g = G x, u = U x, h = silu(g) * u,
 * o = D h.  gate/up are f x d, down is d x f. */
void orc_expert_forward(const uint8_t *gate, int fmt_gate,
                        const uint8_t *up, int fmt_up,
                        const uint8_t *down, int fmt_down,
                        int d, int f, const double *x, double *o);

/* Activations given as fp32 (xtype 0) or bf16 bits (xtype 1). */
void orc_load_x(const void *x, int xtype, int n, double *out);

/* The whole layer for q columns (or q prefill tokens):
 *   mats[3*e + m] for expert e in 0..E (E = shared), m = 0 gate, 1 up, 2 down
 *   fmts[3*e + m] their formats
 * y[q][d] fp32; ids[q][k] and w[q][k] (may be NULL) report the routing. */
void orc_layer_forward(int d, int f, int E, int k, double routed_scale,
                       const float *wr, const uint8_t *const *mats,
                       const int *fmts, const void *x, int xtype, int q,
                       float *y, int32_t *ids, double *w);

#ifdef __cplusplus
}
#endif
#endif
