/*
 * blockq.h -- C ABI of libblockq, block-quantized wire codecs for AMD MI355X (gfx950).
 *
 * Pages cited:
 *   P1 = sparkinfer pull request #46, "feat(pcie_dma): add block-INT8 wire modes for AG,
 *        ring, and A2A" (sections Summary, Implementation, Evidence).
 *   P2 = sparkinfer pull request #72, "feat(pcie_dma): add INT8 and MXFP8 wire modes"
 *        (PR body Summary / Modes / Configuration; review comment showing mxfp8_scale_byte).
 *   P4 = b12x pull request #241, "[II] Support staged MXFP8 linear inputs" (sections
 *        Behavior, Compatibility, Validation).
 *
 * Conventions (every entry point):
 *   - Pointers named in a signature are DEVICE pointers unless marked "host array";
 *     a host array is a host-memory array of device pointers, read during the call only.
 *   - bf16 tensors are passed as uint16_t bit patterns.  INT8 payloads are int8_t, E4M3
 *     and E8M0 bytes are uint8_t, per-block scales are float (IEEE binary32).
 *   - n counts values; it must be a multiple of 128 (a block, P1 Summary; the per-rank
 *     shard rule of P2 Configuration).  n == 0 is valid and launches nothing, as are
 *     rows == 0 or cols == 0 (MXFP8) and M == 0 or N == 0 (GEMM); the counts and the other
 *     sizes are still validated first, and no pointer is read.
 *     Limits: n / 128 < 2^36 (else BQ_ERR_SIZE); a row-major operand of rows x cols with
 *     row stride ld spans at most 2^48 bytes, ((rows - 1) * ld + cols) * element size
 *     (else BQ_ERR_BOUNDS); the MXFP8 calls take rows * cols / 128 < 2^31 blocks, and
 *     the GEMM M, N, K < 2^31 (else BQ_ERR_SIZE).
 *   - Layout of an INT8 or E4M3 block payload is planar: n payload bytes, and nb = n/128
 *     scales in a separate array.  Together they are 132 bytes per 128 values (P1
 *     Summary); a caller may place the scale array right after the payload in one
 *     wire buffer.
 *   - Ownership: the caller allocates and owns every buffer.  The library never
 *     allocates, frees or synchronizes, holds no state between calls and is reentrant.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call enqueues its kernels and returns; inputs must stay unchanged until the stream
 *     reaches the work.  No call synchronizes, so calls may be captured in a HIP graph.
 *   - Errors: every argument is validated on the host before anything is launched; on
 *     an error the call returns a status, writes nothing and launches nothing.
 *     BQ_ERR_LAUNCH reports a failure of the launch itself (the status hipLaunchKernel
 *     returns for that launch).
 *   - Alignment: bf16 and payload pointers 16-byte aligned; float scale arrays 4-byte
 *     aligned; E8M0 scale arrays 4-byte aligned with a row stride divisible by 4.
 *   - Aliasing: outputs must not overlap inputs or each other, except where an entry
 *     point states an exact in-place form.  Partial overlap is BQ_ERR_ALIAS.
 *   - Arithmetic: IEEE binary32 with round-to-nearest-even; no fused multiply-add where
 *     the definitions below round a product; denormals are honoured.  Non-finite inputs
 *     are outside the contract.
 */
#ifndef BLOCKQ_H
#define BLOCKQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bq_status {
    BQ_OK = 0,
    BQ_ERR_NULL = 1,    /* a required pointer is NULL */
    BQ_ERR_SIZE = 2,    /* a count or shape is negative or not a multiple of its block */
    BQ_ERR_ALIGN = 3,   /* a pointer or leading dimension breaks the alignment rules */
    BQ_ERR_BOUNDS = 4,  /* a leading dimension, offset or capacity does not fit */
    BQ_ERR_NSRC = 5,    /* a source / rank / segment count is outside its range */
    BQ_ERR_ALIAS = 6,   /* an output overlaps an input or another output */
    BQ_ERR_LAUNCH = 7,  /* the HIP launch failed */
    BQ_ERR_SCRATCH = 8  /* the allocation-free entry point's scratch is too small */
} bq_status;

#define BQ_BLOCK 128        /* values per INT8 / E4M3 block */
#define BQ_MX_GROUP 32      /* values per MXFP8 scale group */
#define BQ_MAX_SRC 64       /* most sources of bq_dequant_accum_i8 */
#define BQ_MAX_BATCH 16     /* most segments of a batched call; most simulated ranks */

/* ==== Block-INT8 codec (P1 Summary, Implementation) ================================ */

/* BF16 -> signed INT8, one FP32 scale per 128 values.  For each block of 128 consecutive
 * values: amax = max |x|; scale = amax / 127 (binary32 division); q = round-half-even
 * (x / scale) clamped to [-127, 127].  An all-zero block stores scale +0 and payload 0.
 * x: bf16[n]; q: int8[n]; scale: float[n/128]. */
bq_status bq_quant_i8(const uint16_t* x, int64_t n, int8_t* q, float* scale, void* stream);

/* INT8 -> BF16 materialization: y = bf16_rne(fl32((float)q * scale)).
 * q: int8[n]; scale: float[n/128]; y: bf16[n]. */
bq_status bq_dequant_i8(const int8_t* q, const float* scale, int64_t n, uint16_t* y,
                        void* stream);

/* Multi-source INT8 dequantize with FP32 accumulation (the all-to-all reduce).
 * For each value: acc = +0; for s = 0 .. nsrc-1 in that order: acc = acc + fl32(q_s *
 * scale_s) (the product is rounded before the add); y = bf16_rne(acc).
 * q_srcs, s_srcs: host arrays of nsrc device pointers (int8[n], float[n/128]);
 * 1 <= nsrc <= BQ_MAX_SRC, else BQ_ERR_NSRC.  y: bf16[n]. */
bq_status bq_dequant_accum_i8(int nsrc, const int8_t* const* q_srcs, const float* const* s_srcs,
                              int64_t n, uint16_t* y, void* stream);

/* Batched form of the accumulate: `nseg` owners (1..BQ_MAX_BATCH) in one launch.  Owner j
 * sums shard j of every source: values [j*seg_n, (j+1)*seg_n) of q_srcs[k] (scales
 * likewise), k = 0 .. nsrc-1 in that order, into y + j*seg_n.  Each source holds
 * nseg*seg_n values; y holds nseg*seg_n values; seg_n a multiple of 128. */
bq_status bq_dequant_accum_i8_batch(int nseg, int nsrc, const int8_t* const* q_srcs,
                                    const float* const* s_srcs, int64_t seg_n, uint16_t* y,
                                    void* stream);

/* Fused all-to-all owner step, one pass, bit-identical to bq_dequant_accum_i8_batch ->
 * bq_quant_i8 -> bq_dequant_i8 (P1 Summary and Implementation: quantize-once A2A, owner
 * materializes from the payload it broadcasts).  Owner j (0 <= j < nseg) sums shard j --
 * values [j*seg_n, (j+1)*seg_n) -- of the nsrc sources in binary32 in source order, rounds
 * the sum to bf16, requantizes that bf16 sum with the bq_quant_i8 rule into q_out/s_out
 * (segment j at value offset j*seg_n), and materializes the owner's copy from that same
 * payload into y_out[j] (bf16[seg_n]).  red, if not NULL, receives the bf16 sums
 * (segment j at j*seg_n).  q_srcs, s_srcs: host arrays of nsrc device pointers to
 * nseg*seg_n values each; y_out: host array of nseg device pointers, or NULL to skip
 * the materialization.  1 <= nseg <= BQ_MAX_BATCH, 1 <= nsrc <= BQ_MAX_SRC. */
bq_status bq_a2a_reduce_i8(int nseg, int nsrc, const int8_t* const* q_srcs,
                           const float* const* s_srcs, int64_t seg_n, int8_t* q_out,
                           float* s_out, uint16_t* const* y_out, uint16_t* red, void* stream);

/* One fused ring reduce-scatter hop: per value sum = fl32(fl32(q_in * s_in) + local) in
 * binary32, then the binary32 sums of each block are requantized with the
 * bq_quant_i8 rule (no bf16 intermediate).  q_in: int8[n]; s_in: float[n/128];
 * local: bf16[n]; q_out: int8[n]; s_out: float[n/128].  In place is allowed when
 * q_out == q_in AND s_out == s_in exactly; any other overlap is BQ_ERR_ALIAS. */
bq_status bq_ring_hop_i8(const int8_t* q_in, const float* s_in, const uint16_t* local,
                         int64_t n, int8_t* q_out, float* s_out, void* stream);

/* Batched forms: `count` (1..BQ_MAX_BATCH) independent segments of n values each, one
 * launch -- the simulated ranks of one collective step.  Each array argument is a host
 * array of `count` device pointers; segment i is exactly the single call on element i.
 * The in-place rule of bq_ring_hop_i8 applies per segment; segments must not overlap
 * each other's outputs. */
bq_status bq_quant_i8_batch(int count, const uint16_t* const* x, int64_t n, int8_t* const* q,
                            float* const* scale, void* stream);
bq_status bq_dequant_i8_batch(int count, const int8_t* const* q, const float* const* scale,
                              int64_t n, uint16_t* const* y, void* stream);
bq_status bq_ring_hop_i8_batch(int count, const int8_t* const* q_in, const float* const* s_in,
                               const uint16_t* const* local, int64_t n, int8_t* const* q_out,
                               float* const* s_out, void* stream);

/* ==== Collectives simulated on one GPU: a "rank" is a separate HBM buffer ========== */

/* INT8 all-gather materialization (P1 Summary: every rank, the owner included,
 * materializes from the same final payload): each of `world` ranks materializes the
 * whole shared payload q (int8[n]) / s (float[n/128]) into out[r] (bf16[n]), one launch.
 * With skip_own != 0, rank r leaves its own shard -- values [r*n/W, (r+1)*n/W) --
 * untouched (an owner that materialized it in the fused owner step).  out: host array of
 * W device pointers.  n divisible by 128*world; 1 <= W <= BQ_MAX_BATCH. */
bq_status bq_allgather_dequant_i8(int world, const int8_t* q, const float* s, int64_t n,
                                  uint16_t* const* out, int skip_own, void* stream);

/* i8_ring all-reduce (P1 Summary): INT8 ring reduce-scatter, then INT8 all-gather of
 * the final payloads.  The n values of every rank are cut into `world` equal chunks
 * (n divisible by 128*world), chunk c owned by rank c.  Step 0: rank r quantizes its
 * chunk (r-1) mod W; steps k = 1..W-1: rank r folds its chunk (r-1-k) mod W into the
 * payload it received with one fused hop; every rank, owner included, then
 * materializes every chunk from that same final payload (the rank-consistency rule
 * of P1 Summary).  One launch per step covers all ranks.
 * partials: host array of W device pointers, bf16[n] each (read only);
 * q_wire: int8[n], s_wire: float[n/128] -- caller-owned wire buffers; on return (in
 * stream order) they hold the final payload of every chunk, chunk c at offset c*n/W;
 * out: host array of W device pointers, bf16[n] each.  1 <= W <= BQ_MAX_BATCH. */
bq_status bq_ring_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                               int8_t* q_wire, float* s_wire, uint16_t* const* out,
                               void* stream);

/* Allocation-free form of bq_ring_allreduce_i8, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Identical arguments, validation and results, except that the wire payload
 * lives in a library-owned device array of BQ_NOALLOC_SCRATCH_BYTES per GPU (held from
 * the first call on that GPU until the process ends) instead of caller buffers:
 * n + 4 * n/128 bytes must fit, else BQ_ERR_SCRATCH (nothing launched); that is at most
 * 65,075,200 values.  The call allocates nothing.  Every call on one GPU uses that GPU's
 * array: calls that overlap in time on one GPU (other streams, other threads) race on
 * it and must be ordered by the caller.  Nothing in the array needs to start at zero. */
#define BQ_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
bq_status bq_ring_allreduce_i8_noalloc(int world, int64_t n, const uint16_t* const* partials,
                                       uint16_t* const* out, void* stream);

/* i8_a2a all-reduce (P1 Summary, Implementation): every rank quantizes its partial
 * once into q_send[r]/s_send[r]; owner j dequantizes shard j of the W payloads and
 * accumulates them in binary32 in rank order (a bf16 sum, stored into red at offset
 * j*n/W when red is not NULL); it requantizes that bf16 sum once into q_bcast/s_bcast;
 * every rank materializes every shard from that broadcast payload into out[r].  The
 * owner step runs fused (bq_a2a_reduce_i8), the owner's own shard materialized in the
 * same pass.  partials, q_send, s_send, out: host arrays of W device pointers (bf16[n],
 * int8[n], float[n/128], bf16[n]); red: bf16[n] or NULL; q_bcast: int8[n];
 * s_bcast: float[n/128].  n divisible by 128*world; 1 <= W <= BQ_MAX_BATCH. */
bq_status bq_a2a_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                              int8_t* const* q_send, float* const* s_send, uint16_t* red,
                              int8_t* q_bcast, float* s_bcast, uint16_t* const* out,
                              void* stream);

/* ==== MXFP8 (P2 Summary; review comment showing mxfp8_scale_byte; P4 Behavior) ===== */

/* BF16 rows -> E4M3 values with one E8M0 scale per 32 consecutive columns of a row.
 * Scale byte of a group: 127 if amax == 0, else 127 + the smallest e with
 * 2^e >= fl32(amax / 448), clamped to [-127, 127].  Values: v = e4m3_rne_sat(x * 2^-(byte-127)),
 * OCP E4M3FN, round-half-even, saturating at +-448, sign of zero kept.
 * x: bf16[rows][ldx]; v: u8[rows][ldv]; e8m0: u8[rows][lds], scale (r, g) covers
 * columns [32g, 32g+32).  cols a multiple of 128; ldx >= cols, ldx % 8 == 0;
 * ldv >= cols, ldv % 16 == 0; lds >= cols/32, lds % 4 == 0. */
bq_status bq_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* v,
                      int64_t ldv, uint8_t* e8m0, int64_t lds, void* stream);

/* MXFP8 -> BF16: y = bf16_rne(fl32(e4m3 * 2^(byte-127))).  Same layout rules; y is
 * bf16[rows][ldy], ldy >= cols, ldy % 8 == 0. */
bq_status bq_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                        int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, void* stream);

/* Staged slice quantization (P4 Behavior, Compatibility): one BF16 slice of rows x cols
 * is quantized with the bq_quant_mx rule into columns [col_off, col_off+cols) of the
 * caller-owned staging buffer v (row stride ldv = total columns) and into scale
 * columns [col_off/32, (col_off+cols)/32) of e8m0 (row stride lds).  cols and col_off
 * must be multiples of 128; col_off + cols <= ldv; lds >= ldv/32; rows <=
 * capacity_rows (the staging buffer's row capacity).  Rows at or above `rows` and
 * columns outside the slice are not touched. */
bq_status bq_quant_mx_slice(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                            int64_t lds, int64_t capacity_rows, void* stream);

/* The same two calls on IEEE binary16 input (P4 Behavior: the slice quantizer takes BF16
 * or FP16 slices).  x holds binary16 bit patterns (finite); every binary16 value is exact
 * in binary32, and the group byte follows the rule above from that binary32 amax.
 * Arguments, layout and errors as bq_quant_mx / bq_quant_mx_slice. */
bq_status bq_quant_mx_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds, void* stream);
bq_status bq_quant_mx_slice_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                                int64_t lds, int64_t capacity_rows, void* stream);

/* Sizes of a staging buffer for `capacity_rows` rows of `total_cols` columns (the
 * allocation helper of P4 Behavior, as a host-side size query: the caller allocates).
 * total_cols must be a multiple of 128.  Host pointers. */
bq_status bq_mx_staging_bytes(int64_t capacity_rows, int64_t total_cols, int64_t* value_bytes,
                              int64_t* scale_bytes);

/* ==== MXFP8 on the collective topologies (P2 PR body Summary / Modes: mx_ring, mx_a2a) ====
 *
 * Flat layout of an MXFP8 wire payload of n values: v = u8[n] E4M3FN codes and
 * e8m0 = u8[n/32], byte g scaling values [32g, 32g+32) -- 132 bytes per 128 values, the
 * same spans as a block-INT8 payload.  A flat tensor quantizes and dequantizes with the
 * bq_quant_mx / bq_dequant_mx rules (rows = 1, cols = n).  The collectives below are
 * the INT8 ones with this codec, and carry the same canonical-payload rule: every rank,
 * the owner included, materializes from the payload that is forwarded. */

/* Batched flat quantize / dequantize: `count` (1..BQ_MAX_BATCH) segments of n values, one
 * launch; segment i is bq_quant_mx / bq_dequant_mx of x[i] / (v[i], e8m0[i]) with rows = 1.
 * Host arrays of device pointers.  v: 16-byte aligned; e8m0: 4-byte aligned. */
bq_status bq_quant_mx_batch(int count, const uint16_t* const* x, int64_t n, uint8_t* const* v,
                            uint8_t* const* e8m0, void* stream);
bq_status bq_dequant_mx_batch(int count, const uint8_t* const* v, const uint8_t* const* e8m0,
                              int64_t n, uint16_t* const* y, void* stream);

/* One fused mx_ring hop: per value sum = fl32(fl32(e4m3(v_in) * 2^(byte-127)) + local)
 * in binary32, then the binary32 sums of each 32-value group are requantized with the
 * MXFP8 rule (byte from the group's binary32 amax: 127 + the smallest e with 2^e >=
 * fl32(amax/448), clamped to [-127, 127], 0 when that quotient underflows; no bf16
 * intermediate).  In place is allowed when v_out == v_in AND e_out == e_in exactly. */
bq_status bq_ring_hop_mx(const uint8_t* v_in, const uint8_t* e_in, const uint16_t* local,
                         int64_t n, uint8_t* v_out, uint8_t* e_out, void* stream);
bq_status bq_ring_hop_mx_batch(int count, const uint8_t* const* v_in,
                               const uint8_t* const* e_in, const uint16_t* const* local,
                               int64_t n, uint8_t* const* v_out, uint8_t* const* e_out,
                               void* stream);

/* mx_a2a owner accumulate: acc = +0; for s = 0 .. nsrc-1 in that order acc = acc +
 * e4m3(v_s) * 2^(byte_s - 127) (each term exact in binary32); y = bf16_rne(acc).
 * 1 <= nsrc <= BQ_MAX_SRC. */
bq_status bq_dequant_accum_mx(int nsrc, const uint8_t* const* v_srcs,
                              const uint8_t* const* e_srcs, int64_t n, uint16_t* y,
                              void* stream);

/* Fused mx_a2a owner step, bit-identical to bq_dequant_accum_mx -> bq_quant_mx ->
 * bq_dequant_mx on each owner's shard.  Arguments as bq_a2a_reduce_i8, with v/e8m0 in
 * place of q/scale (owner j's scale bytes start at e_out + j*seg_n/32). */
bq_status bq_a2a_reduce_mx(int nseg, int nsrc, const uint8_t* const* v_srcs,
                           const uint8_t* const* e_srcs, int64_t seg_n, uint8_t* v_out,
                           uint8_t* e_out, uint16_t* const* y_out, uint16_t* red, void* stream);

/* MXFP8 all-gather materialization; arguments as bq_allgather_dequant_i8. */
bq_status bq_allgather_dequant_mx(int world, const uint8_t* v, const uint8_t* e8m0, int64_t n,
                                  uint16_t* const* out, int skip_own, void* stream);

/* mx_ring all-reduce: the i8_ring schedule with the MXFP8 codec.  v_wire: u8[n],
 * e_wire: u8[n/32]; on return they hold every chunk's final payload (chunk c at value
 * offset c*n/W, scale offset c*n/(32W)).  Other arguments as bq_ring_allreduce_i8. */
bq_status bq_ring_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                               uint8_t* v_wire, uint8_t* e_wire, uint16_t* const* out,
                               void* stream);

/* mx_a2a all-reduce: the i8_a2a schedule with the MXFP8 codec (the owner requantizes
 * its bf16 sum once).  v_send/e_send: host arrays of W device pointers (u8[n], u8[n/32]);
 * v_bcast: u8[n]; e_bcast: u8[n/32]; red: bf16[n] or NULL.  Other arguments as
 * bq_a2a_allreduce_i8. */
bq_status bq_a2a_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                              uint8_t* const* v_send, uint8_t* const* e_send, uint16_t* red,
                              uint8_t* v_bcast, uint8_t* e_bcast, uint16_t* const* out,
                              void* stream);

/* ==== The dense MXFP8 GEMM from staged inputs (P4 Behavior: mm_quantized_into) ========
 *
 * Y[m][n] = bf16_rne( sum over k of X[m][k] * W[n][k] ) for 0 <= m < M, 0 <= n < N:
 * X is MXFP8 activations (an assembled staging buffer: xv u8[M][ldxv] E4M3 values and
 * xe u8[M][ldxe] E8M0 bytes, byte g of a row scaling its columns [32g, 32g+32)), W is MXFP8
 * weights in the same layout (wv u8[N][ldwv], we u8[N][ldwe]), both contiguous along K.
 * Each product of two E4M3 values and their two scales is exact; the sums are binary32
 * (matrix-core accumulation, K in steps of 128) and are rounded to bf16 once into y
 * (bf16[M][ldy], caller-owned).  The summation order is fixed, so results are
 * deterministic: the same inputs give the same bits, whether the staging buffer was
 * filled by slices or by one call (P4 Validation).
 * K must be a positive multiple of 128; M == 0 or N == 0 launches nothing.  ldxv, ldwv
 * >= K and divisible by 16 with xv, wv 16-byte aligned; ldxe, ldwe >= K/32, divisible by
 * 4, with xe, we 4-byte aligned; ldy >= N; y must not overlap an input.
 * Speed, not results: when K is a multiple of 512 and xe, we are 16-byte aligned with ldxe,
 * ldwe divisible by 16, the kernel fetches four K steps' scale bytes per row at once (about
 * 7% faster at 4096 x 7168 x 43008); other layouts give the same bits.  Workgroup tiles are
 * 256 rows by 256 or 224 columns, whichever fills the device's compute units better
 * (bq_mm_tile_cols); both give the same bits. */
bq_status bq_mm_mx(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t ldxe,
                   const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t ldwe, int64_t M,
                   int64_t N, int64_t K, uint16_t* y, int64_t ldy, void* stream);

/* ==== MXFP8 scales laid out for the scaled matrix instruction (P4 Behavior) ==========
 *
 * P4 Behavior has the caller-owned staging hold the MXFP8 values and the scale layout the
 * dense GEMM consumes.  These entry points keep the values row-major as above and put the
 * E8M0 bytes in the order gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes them: one K
 * step of 128 columns of 16 rows takes from lane l the scale of row l%16 and 32-column
 * block l/16.  The layout of a matrix with R rows (its row capacity) and C columns is
 * ceil(R/16) * ceil(C/512) tiles of 256 bytes, tiles ordered by 512-column group first,
 * then by 16-row block; in a tile, word l (bytes 4l..4l+3) belongs to lane l and its byte j
 * to K step j of the group's four.  The scale of (row r, 32-column group g) therefore sits
 * at byte 256 * ((g/16) * ceil(R/16) + r/16) + 4 * (16 * (g%4) + r%16) + (g%16)/4.
 * Bytes of rows >= R or of columns >= C in a partial tile are never written or used.
 * Layout arrays must be 16-byte aligned. */

/* Bytes of the layout for rows x cols (cols a multiple of 128): 256 * ceil(rows/16) *
 * ceil(cols/512).  Returns -1 for a negative size, cols not a multiple of 128, or a size
 * beyond 2^40. */
int64_t bq_mx_scale_mfma_bytes(int64_t rows, int64_t cols);

/* Staged slice quantization with the scales in the layout: the bq_quant_mx_slice rule and
 * value placement (columns [col_off, col_off+cols) of v, row stride ldv), and the slice's
 * scale bytes at their layout positions in e8m0, a layout of capacity_rows rows and
 * total_cols columns (bq_mx_scale_mfma_bytes(capacity_rows, total_cols) bytes).  Staged
 * slices equal the one-call quantization of the concatenation in every byte (P4
 * Validation).  cols, col_off, total_cols multiples of 128; col_off + cols <= total_cols
 * <= ldv; rows <= capacity_rows; nothing outside the slice's values and scale bytes is
 * written.  _f16: IEEE binary16 input (P4 Behavior: BF16 or FP16 slices). */
bq_status bq_quant_mx_slice_mfma(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 int64_t col_off, uint8_t* v, int64_t ldv, int64_t total_cols,
                                 uint8_t* e8m0, int64_t capacity_rows, void* stream);
bq_status bq_quant_mx_slice_mfma_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                     int64_t col_off, uint8_t* v, int64_t ldv,
                                     int64_t total_cols, uint8_t* e8m0, int64_t capacity_rows,
                                     void* stream);

/* bq_dequant_mx with the scales read from the layout: rows x cols of v (row stride ldv)
 * whose scales are a layout of scale_rows (>= rows) rows starting at column 0. */
bq_status bq_dequant_mx_mfma(const uint8_t* v, int64_t ldv, const uint8_t* e8m0,
                             int64_t scale_rows, int64_t rows, int64_t cols, uint16_t* y,
                             int64_t ldy, void* stream);

/* bq_mm_mx with both operands' scales in the layout: xe laid out for xe_rows (>= M) rows,
 * we for we_rows (>= N) rows, each holding at least K columns.  Same result bits as
 * bq_mm_mx on the same values and scales.  The kernel brings four K steps' scales in as
 * whole tiles for any K that is a multiple of 128. */
bq_status bq_mm_mx_mfma(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t xe_rows,
                        const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t we_rows,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                        void* stream);

/* ==== E4M3 128-block codec: the format the INT8 codec replaces (P1 Summary, Why) ==== */

/* Same block and footprint as the INT8 codec (132 bytes per 128 values): scale =
 * fl32(amax / 448); v = e4m3_rne_sat(fl32(x / scale)); an all-zero block stores scale
 * +0 and every byte 0x00.  x: bf16[n]; v: u8[n]; scale: float[n/128]. */
bq_status bq_quant_e4m3_b128(const uint16_t* x, int64_t n, uint8_t* v, float* scale,
                             void* stream);

/* y = bf16_rne(fl32(e4m3(v) * scale)).  v: u8[n]; scale: float[n/128]; y: bf16[n]. */
bq_status bq_dequant_e4m3_b128(const uint8_t* v, const float* scale, int64_t n, uint16_t* y,
                               void* stream);

/* ==== Host helpers ================================================================ */

/* Wire/staging bytes of n values in any 128-value block format: 132 * n / 128
 * (P1 Summary; P2 Summary).  Returns -1 if n is negative or not a multiple of 128. */
int64_t bq_wire_bytes_b128(int64_t n);

/* Column count of the dense MXFP8 GEMM's workgroup tiles (bq_mm_mx, bq_mm_mx_mfma) for an
 * M x N product on a device with cus compute units: 224 or 256, whichever takes fewer
 * rounds of one tile per unit times the tile width (ties to 256; the launches read the
 * current device's count).  Returns -1 unless 1 <= M, N < 2^31 and cus >= 1. */
int bq_mm_tile_cols(int64_t M, int64_t N, int cus);

/* Static description of a status code. */
const char* bq_status_str(bq_status status);

/* Library version string. */
const char* bq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BLOCKQ_H */
