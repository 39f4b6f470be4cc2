/*
 * bq_oracle.h -- plain, slow, single-threaded CPU oracle for the block-quantized
 * wire codecs.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls it, and it includes nothing from the GPU library.
 *
 * Pages cited (the text of four web pages on block-quantized wire formats):
 *   P1 = sparkinfer pull request #46, "feat(pcie_dma): add block-INT8 wire modes
 *        for AG, ring, and A2A" (sections Summary, Implementation, Evidence).
 *   P2 = sparkinfer pull request #72, "feat(pcie_dma): add INT8 and MXFP8 wire
 *        modes" (PR body Summary / Modes, and the review comment that shows the
 *        device helper mxfp8_scale_byte).
 *   P4 = b12x pull request #241, "[II] Support staged MXFP8 linear inputs"
 *        (sections Behavior, Compatibility, Validation).
 *
 * Conventions shared by every function:
 *   - bf16 tensors are passed as uint16_t bit patterns;
 *   - n is the number of values, a multiple of 128; nb = n / 128 blocks;
 *   - all arithmetic is IEEE-754 binary32 with round-to-nearest-even, done one
 *     operation per C statement; the library is compiled with
 *     -ffp-contract=off -fno-fast-math on x86-64 SSE (no x87 excess precision);
 *   - inputs must be finite (non-finite inputs are outside the contract and
 *     abort the process).
 */
#ifndef BQ_ORACLE_H
#define BQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar conversions ------------------------------------------------ */
float    orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);          /* round to nearest, ties to even */
uint8_t  orc_e4m3_encode(float v);          /* OCP E4M3FN, RNE, finite saturation */
float    orc_e4m3_decode(uint8_t code);
uint8_t  orc_e8m0_scale(float amax);        /* MXFP8 shared-exponent byte */

/* ---- block-INT8 codec (P1 Summary / Implementation) ------------------- */
void orc_quant_i8(const uint16_t* x, int64_t n, int8_t* q, float* scale);
void orc_dequant_i8(const int8_t* q, const float* scale, int64_t n, uint16_t* y);
void orc_dequant_accum_i8(int nsrc, const int8_t* const* q, const float* const* scale,
                          int64_t n, uint16_t* y);
void orc_ring_hop_i8(const int8_t* q_in, const float* s_in, const uint16_t* local,
                     int64_t n, int8_t* q_out, float* s_out);

/* Fused all-to-all owner step: for each of nseg owners, the accumulate above over
 * values [j*seg_n, (j+1)*seg_n) of every source, its bf16 sum requantized with the
 * block-INT8 rule into q_out/s_out (segment j at j*seg_n), and the owner's own
 * materialization of that payload into y_out[j] (may be NULL); red (may be NULL)
 * receives the bf16 sums. */
void orc_a2a_reduce_i8(int nseg, int nsrc, const int8_t* const* q_srcs,
                       const float* const* s_srcs, int64_t seg_n, int8_t* q_out,
                       float* s_out, uint16_t* const* y_out, uint16_t* red);

/* ---- one-GPU simulation of the collectives (P1 Summary) --------------- */
/* Ring reduce-scatter + all-gather of `world` rank partials of n values each.
 * q_final/s_final receive the final payload of every chunk, chunk c at value
 * offset c*n/world; out[r] receives rank r's materialized bf16 tensor. */
void orc_ring_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                           int8_t* q_final, float* s_final, uint16_t* const* out);
/* Quantize-once all-to-all + broadcast.  red receives the owners' bf16 sums
 * (shard j at offset j*n/world), q_final/s_final the broadcast payloads. */
void orc_a2a_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                          uint16_t* red, int8_t* q_final, float* s_final,
                          uint16_t* const* out);

/* ---- MXFP8 codec (P2 Summary, P4 Behavior) ---------------------------- */
void orc_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                  uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds);
void orc_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                    int64_t rows, int64_t cols, uint16_t* y, int64_t ldy);
void orc_quant_mx_slice(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                        int64_t lds);
/* IEEE binary16 input (P4 Behavior: BF16 or FP16 slices). */
float orc_f16_to_f32(uint16_t h);
void orc_quant_mx_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds);
void orc_quant_mx_slice_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                            int64_t lds);

/* ---- MXFP8 scales in the order of the scaled matrix instruction ---------
 * P4 Behavior: the caller-owned staging holds the MXFP8 values and the scale layout
 * the dense GEMM consumes.  One K step of the gfx950 scaled MFMA covers 128 columns of
 * 16 rows; lane l of the wave supplies the scale byte of row l%16 and 32-column block
 * l/16.  A 256-byte tile holds 16 rows x 512 columns (four K steps): word l for lane l,
 * byte j of that word for K step j of the four.  Tiles are ordered by 512-column group
 * first, then by 16-row block; row_blocks is the number of 16-row blocks the array was
 * laid out for.  Offset of the byte of (row, 32-column group): */
int64_t orc_mx_mfma_offset(int64_t row, int64_t group, int64_t row_blocks);
/* Place row-major scales e8m0[rows][lds] (groups per row used) into that layout, group g
 * of the input at layout group group_off + g; bytes of other positions are not written. */
void orc_mx_scales_to_mfma(const uint8_t* e8m0, int64_t lds, int64_t rows, int64_t groups,
                           int64_t group_off, int64_t row_blocks, uint8_t* out);

/* ---- MXFP8 on the collective topologies (P2 Summary / Modes) ----------
 * Flat layout: n E4M3 bytes and n/32 E8M0 bytes; group g = values [32g, 32g+32). */
void orc_ring_hop_mx(const uint8_t* v_in, const uint8_t* e_in, const uint16_t* local,
                     int64_t n, uint8_t* v_out, uint8_t* e_out);
void orc_dequant_accum_mx(int nsrc, const uint8_t* const* v, const uint8_t* const* e8m0,
                          int64_t n, uint16_t* y);
void orc_a2a_reduce_mx(int nseg, int nsrc, const uint8_t* const* v_srcs,
                       const uint8_t* const* e_srcs, int64_t seg_n, uint8_t* v_out,
                       uint8_t* e_out, uint16_t* const* y_out, uint16_t* red);
void orc_ring_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                           uint8_t* v_final, uint8_t* e_final, uint16_t* const* out);
void orc_a2a_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                          uint16_t* red, uint8_t* v_final, uint8_t* e_final,
                          uint16_t* const* out);

/* ---- E4M3 128-block codec, the pre-existing format the INT8 codec
 *      replaces (P1 Summary / Why) ------------------------------------- */
void orc_quant_e4m3_b128(const uint16_t* x, int64_t n, uint8_t* v, float* scale);
void orc_dequant_e4m3_b128(const uint8_t* v, const float* scale, int64_t n, uint16_t* y);

#ifdef __cplusplus
}
#endif
#endif
