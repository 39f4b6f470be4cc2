/*
 * bq_oracle.c -- plain CPU oracle for the block-quantized wire codecs.
 *
 * TEST INFRASTRUCTURE ONLY (see bq_oracle.h).  Every function follows the
 * written definition step by step, one IEEE binary32 operation per statement,
 * with no blocking, fusion or reordering.  Page tags P1, P2, P4 are defined in
 * bq_oracle.h.
 *
 * Build: cc -std=c99 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include "bq_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define BLK 128          /* values per INT8 / E4M3 block (P1 Summary) */
#define MXG 32           /* values per MXFP8 scale group (P2 Summary) */
#define I8_QMAX 127.0f   /* symmetric INT8 range [-127, 127]; scale = amax/127 */
#define E4M3_MAX 448.0f  /* largest finite OCP E4M3FN value */

static void need_finite(float f) {
    if (!isfinite(f)) {
        fprintf(stderr, "bq_oracle: non-finite value is outside the contract\n");
        abort();
    }
}

static void need_blocks(int64_t n) {
    if (n < 0 || n % BLK != 0) {
        fprintf(stderr, "bq_oracle: n=%lld is not a multiple of 128\n", (long long)n);
        abort();
    }
}

/* ---------------------------------------------------------------------- */
/* BF16 <-> binary32.                                                       */
/* ---------------------------------------------------------------------- */

float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;   /* bf16 is the top half of a binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite binary32 to the nearest bf16, ties to the even bf16
 * significand.  A carry out of the significand moves into the exponent, so
 * the largest values round to infinity exactly as IEEE rounding does. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

/* ---------------------------------------------------------------------- */
/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;  */
/* 0x7F / 0xFF are NaN; largest finite 448; subnormal step 2^-9.           */
/* ---------------------------------------------------------------------- */

float orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int ex = (code >> 3) & 0xF;
    int man = code & 0x7;
    if (ex == 0xF && man == 0x7)
        return NAN;
    float mag;
    if (ex == 0)
        mag = ldexpf((float)man, -9);              /* subnormal: man * 2^-9 */
    else
        mag = ldexpf((float)(8 + man), ex - 10);   /* (1 + man/8) * 2^(ex-7) */
    return sign ? -mag : mag;
}

/* Nearest finite E4M3FN code to v, ties to the code with the even mantissa,
 * magnitudes at or above 448 saturate to 448, the sign (also of zero) kept.
 * The non-negative finite codes 0x00..0x7E are increasing in value, so the
 * nearest one is found by locating v between two neighbouring codes and
 * comparing against their midpoint (exactly representable). */
uint8_t orc_e4m3_encode(float v) {
    need_finite(v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= E4M3_MAX)
        return (uint8_t)(sign | 0x7E);
    /* largest code c in [0, 0x7D] with decode(c) <= a */
    int lo = 0, hi = 0x7E;            /* decode(lo) <= a < decode(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    float below = orc_e4m3_decode((uint8_t)lo);
    float above = orc_e4m3_decode((uint8_t)hi);
    float midpoint = (below + above) * 0.5f;      /* exact: 5 significant bits */
    int code;
    if (a < midpoint)
        code = lo;
    else if (a > midpoint)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;           /* tie: even mantissa bit */
    return (uint8_t)(sign | code);
}

/* ---------------------------------------------------------------------- */
/* MXFP8 shared scale (P2, review comment showing mxfp8_scale_byte):        */
/* an all-zero group gets byte 127 (scale 1.0); otherwise the scale is the  */
/* E8M0 value of amax/448 (binary32 division) rounded toward +infinity,     */
/* i.e. the smallest power of two 2^e >= amax/448, saturated to the finite  */
/* E8M0 range e in [-127, 127] (byte = e + 127, never the NaN byte 0xFF).   */
/* ---------------------------------------------------------------------- */

uint8_t orc_e8m0_scale(float amax) {
    need_finite(amax);
    if (amax == 0.0f)
        return 127;
    float d = amax / E4M3_MAX;
    if (d == 0.0f)               /* the quotient underflowed: saturate to the smallest */
        return 0;                /* finite E8M0 value, 2^-127                           */
    int k;
    float f = frexpf(d, &k);     /* d = f * 2^k, f in [0.5, 1) */
    int e = (f == 0.5f) ? k - 1 : k;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return (uint8_t)(e + 127);
}

/* ---------------------------------------------------------------------- */
/* Block-INT8 (P1 Summary, Implementation).                                 */
/* ---------------------------------------------------------------------- */

/* One 128-value block of binary32 values -> 128 signed bytes + FP32 scale.
 * amax = max |x|; scale = amax / 127; q = round-half-even(x / scale) clamped
 * to [-127, 127]; an all-zero block stores scale 0 and payload 0 (P1 Summary and
 * Implementation give the rule and the zero-block case). */
static void quant_block_f32(const float* x, int8_t* q, float* scale) {
    float amax = 0.0f;
    for (int i = 0; i < BLK; i++) {
        need_finite(x[i]);
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float s = amax / I8_QMAX;
    /* A nonzero amax below 127 * 2^-150 gives a scale that rounds to 0; only binary32
     * sums (a ring hop) can reach it.  Such a block dequantizes to 0 whatever its
     * payload, so it is stored exactly like an all-zero block. */
    if (amax == 0.0f || s == 0.0f) {
        *scale = 0.0f;
        for (int i = 0; i < BLK; i++)
            q[i] = 0;
        return;
    }
    *scale = s;
    for (int i = 0; i < BLK; i++) {
        float t = x[i] / s;
        float r = rintf(t);                 /* default mode: nearest, ties even */
        if (r > I8_QMAX)
            r = I8_QMAX;
        if (r < -I8_QMAX)
            r = -I8_QMAX;
        q[i] = (int8_t)r;
    }
}

void orc_quant_i8(const uint16_t* x, int64_t n, int8_t* q, float* scale) {
    need_blocks(n);
    float buf[BLK];
    for (int64_t b = 0; b < n / BLK; b++) {
        for (int i = 0; i < BLK; i++)
            buf[i] = orc_bf16_to_f32(x[b * BLK + i]);
        quant_block_f32(buf, q + b * BLK, scale + b);
    }
}

/* Materialization: y = bf16(fl32((float)q * scale)). */
void orc_dequant_i8(const int8_t* q, const float* scale, int64_t n, uint16_t* y) {
    need_blocks(n);
    for (int64_t i = 0; i < n; i++) {
        float v = (float)q[i] * scale[i / BLK];
        y[i] = orc_f32_to_bf16(v);
    }
}

/* A2A reduce: acc starts at +0 and adds the sources' dequantized values in
 * array order, each product rounded to binary32 before the add (no fused
 * multiply-add); the final sum is rounded once to bf16. */
void orc_dequant_accum_i8(int nsrc, const int8_t* const* q, const float* const* scale,
                          int64_t n, uint16_t* y) {
    need_blocks(n);
    for (int64_t i = 0; i < n; i++) {
        float acc = 0.0f;
        for (int s = 0; s < nsrc; s++) {
            float term = (float)q[s][i] * scale[s][i / BLK];
            acc = acc + term;
        }
        y[i] = orc_f32_to_bf16(acc);
    }
}

/* One fused ring reduce-scatter hop: sum = fl32(fl32(q * scale) + local) in
 * binary32, and the binary32 sums (no bf16 intermediate) are requantized with
 * the block-INT8 rule.  q_out/s_out may be the same buffers as q_in/s_in. */
void orc_ring_hop_i8(const int8_t* q_in, const float* s_in, const uint16_t* local,
                     int64_t n, int8_t* q_out, float* s_out) {
    need_blocks(n);
    float sum[BLK];
    for (int64_t b = 0; b < n / BLK; b++) {
        for (int i = 0; i < BLK; i++) {
            float deq = (float)q_in[b * BLK + i] * s_in[b];
            float loc = orc_bf16_to_f32(local[b * BLK + i]);
            sum[i] = deq + loc;
        }
        quant_block_f32(sum, q_out + b * BLK, s_out + b);
    }
}

/* The owner step of the quantize-once all-to-all (P1 Summary and Implementation):
 * accumulate the sources' shard in binary32 (bf16 result), requantize that bf16 sum
 * once, and materialize the owner's copy from the payload it broadcasts.  Written as
 * the composition of the three steps above, which is the definition. */
void orc_a2a_reduce_i8(int nseg, int nsrc, const int8_t* const* q_srcs,
                       const float* const* s_srcs, int64_t seg_n, int8_t* q_out,
                       float* s_out, uint16_t* const* y_out, uint16_t* red) {
    need_blocks(seg_n);
    const int8_t** qp = (const int8_t**)malloc((size_t)nsrc * sizeof(*qp));
    const float** sp = (const float**)malloc((size_t)nsrc * sizeof(*sp));
    uint16_t* sum = (uint16_t*)malloc((size_t)(seg_n ? seg_n : 1) * sizeof(uint16_t));
    if (!qp || !sp || !sum) {
        fprintf(stderr, "bq_oracle: out of memory\n");
        abort();
    }
    int64_t sb = seg_n / BLK;
    for (int j = 0; j < nseg; j++) {
        for (int k = 0; k < nsrc; k++) {
            qp[k] = q_srcs[k] + j * seg_n;
            sp[k] = s_srcs[k] + j * sb;
        }
        orc_dequant_accum_i8(nsrc, qp, sp, seg_n, sum);
        orc_quant_i8(sum, seg_n, q_out + j * seg_n, s_out + j * sb);
        if (y_out && y_out[j])
            orc_dequant_i8(q_out + j * seg_n, s_out + j * sb, seg_n, y_out[j]);
        if (red)
            memcpy(red + j * seg_n, sum, (size_t)seg_n * sizeof(uint16_t));
    }
    free(qp);
    free(sp);
    free(sum);
}

/* ---------------------------------------------------------------------- */
/* Collectives simulated on one host: a "rank" is only a separate buffer.   */
/* ---------------------------------------------------------------------- */

static void* xmalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "bq_oracle: out of memory\n");
        abort();
    }
    return p;
}

static int mod(int a, int w) { return ((a % w) + w) % w; }

/* i8_ring (P1 Summary): INT8 ring reduce-scatter, then an INT8 all-gather of
 * the final payloads.  The tensor is cut into `world` equal chunks, chunk c
 * owned by rank c.  Step 0: rank r quantizes its partial of chunk (r-1) mod W.
 * Step k = 1..W-1: rank r folds its partial of chunk (r-1-k) mod W into the
 * payload it received, with one fused hop.  Chunk c therefore collects ranks
 * c+1, c+2, ..., c (mod W) and finishes at its owner.  Every rank, the owner
 * included, then materializes each chunk from that same final payload
 * (P1 Summary, the rank-consistency rule). */
void orc_ring_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                           int8_t* q_final, float* s_final, uint16_t* const* out) {
    int W = world;
    need_blocks(n);
    if (W < 1 || n % ((int64_t)BLK * W) != 0) {
        fprintf(stderr, "bq_oracle: ring needs n divisible by 128*world\n");
        abort();
    }
    int64_t m = n / W;          /* values per chunk */
    int64_t mb = m / BLK;       /* blocks per chunk */
    /* payload "in flight" for each chunk; it stays with its chunk as it moves */
    for (int r = 0; r < W; r++) {
        int c = mod(r - 1, W);
        orc_quant_i8(partials[r] + c * m, m, q_final + c * m, s_final + c * mb);
    }
    for (int k = 1; k < W; k++) {
        for (int r = 0; r < W; r++) {
            int c = mod(r - 1 - k, W);
            orc_ring_hop_i8(q_final + c * m, s_final + c * mb, partials[r] + c * m, m,
                            q_final + c * m, s_final + c * mb);
        }
    }
    for (int r = 0; r < W; r++)
        for (int c = 0; c < W; c++)
            orc_dequant_i8(q_final + c * m, s_final + c * mb, m, out[r] + c * m);
}

/* i8_a2a (P1 Summary, Implementation): every rank quantizes its whole partial
 * once; shard j of each payload goes to owner j, which dequantizes the W
 * sources and accumulates them in binary32 in rank order (bf16 result);
 * the owner requantizes that bf16 sum once and broadcasts it; every rank,
 * the owner included, materializes shard j from that broadcast payload. */
void orc_a2a_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                          uint16_t* red, int8_t* q_final, float* s_final,
                          uint16_t* const* out) {
    int W = world;
    need_blocks(n);
    if (W < 1 || n % ((int64_t)BLK * W) != 0) {
        fprintf(stderr, "bq_oracle: a2a needs n divisible by 128*world\n");
        abort();
    }
    int64_t m = n / W, mb = m / BLK, nb = n / BLK;
    int8_t* qs = (int8_t*)xmalloc((size_t)W * (size_t)n);
    float* ss = (float*)xmalloc((size_t)W * (size_t)nb * sizeof(float));
    const int8_t** qp = (const int8_t**)xmalloc((size_t)W * sizeof(*qp));
    const float** sp = (const float**)xmalloc((size_t)W * sizeof(*sp));
    for (int s = 0; s < W; s++)
        orc_quant_i8(partials[s], n, qs + (size_t)s * n, ss + (size_t)s * nb);
    for (int j = 0; j < W; j++) {
        for (int s = 0; s < W; s++) {
            qp[s] = qs + (size_t)s * n + j * m;
            sp[s] = ss + (size_t)s * nb + j * mb;
        }
        orc_dequant_accum_i8(W, qp, sp, m, red + j * m);
        orc_quant_i8(red + j * m, m, q_final + j * m, s_final + j * mb);
    }
    for (int r = 0; r < W; r++)
        for (int j = 0; j < W; j++)
            orc_dequant_i8(q_final + j * m, s_final + j * mb, m, out[r] + j * m);
    free(qs);
    free(ss);
    free(qp);
    free(sp);
}

/* ---------------------------------------------------------------------- */
/* MXFP8 (P2 Summary; P4 Behavior).  Row-major; scale (r, g) covers columns */
/* [32g, 32g+32) of row r.                                                  */
/* ---------------------------------------------------------------------- */

/* One group of 32 binary32 values -> its scale byte and 32 E4M3 codes: the byte from
 * the group amax by the rule above, each value scaled by 2^-(byte-127) (ldexpf, exact
 * wherever the result is normal; below that the E4M3 code is a signed zero either way)
 * and encoded to E4M3FN. */
static void quant_group_mx(const float* x, uint8_t* v, uint8_t* byte_out) {
    float amax = 0.0f;
    for (int i = 0; i < MXG; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    uint8_t byte = orc_e8m0_scale(amax);
    *byte_out = byte;
    int e = (int)byte - 127;
    for (int i = 0; i < MXG; i++) {
        float scaled = ldexpf(x[i], -e);
        v[i] = orc_e4m3_encode(scaled);
    }
}

/* e4m3 * 2^(byte-127) in binary32 (exact for every code and byte whose product is
 * finite: E4M3 values are multiples of 2^-9 with 4 significant bits). */
static float mx_value(uint8_t code, uint8_t byte) {
    return ldexpf(orc_e4m3_decode(code), (int)byte - 127);
}

/* IEEE binary16 -> binary32, exact: sign, 5-bit exponent with bias 15, 10-bit
 * fraction; exponent 0 holds the subnormals fraction * 2^-24.  Infinities and NaNs
 * (exponent 31) are outside the contract. */
float orc_f16_to_f32(uint16_t h) {
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    if (ex == 0x1F) {
        fprintf(stderr, "bq_oracle: non-finite binary16 input is outside the contract\n");
        abort();
    }
    float mag = (ex == 0) ? ldexpf((float)man, -24) : ldexpf((float)(1024 + man), ex - 25);
    return (h & 0x8000u) ? -mag : mag;
}

/* MXFP8 quantization of rows of 16-bit inputs decoded by `to_f32`. */
static void quant_mx_rows(float (*to_f32)(uint16_t), const uint16_t* x, int64_t rows,
                          int64_t cols, int64_t ldx, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                          int64_t lds) {
    if (cols % MXG != 0) {
        fprintf(stderr, "bq_oracle: MX cols must be a multiple of 32\n");
        abort();
    }
    float xf[MXG];
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t g = 0; g < cols / MXG; g++) {
            const uint16_t* xg = x + r * ldx + g * MXG;
            for (int i = 0; i < MXG; i++)
                xf[i] = to_f32(xg[i]);
            quant_group_mx(xf, v + r * ldv + g * MXG, e8m0 + r * lds + g);
        }
    }
}

void orc_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                  uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds) {
    quant_mx_rows(orc_bf16_to_f32, x, rows, cols, ldx, v, ldv, e8m0, lds);
}

/* The same rule on IEEE binary16 input (P4 Behavior: the slice quantizer takes BF16 or
 * FP16 feature slices); every binary16 value is exact in binary32. */
void orc_quant_mx_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds) {
    quant_mx_rows(orc_f16_to_f32, x, rows, cols, ldx, v, ldv, e8m0, lds);
}

/* y = bf16(fl32(e4m3 * 2^(byte-127))). */
void orc_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                    int64_t rows, int64_t cols, uint16_t* y, int64_t ldy) {
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            float val = mx_value(v[r * ldv + c], e8m0[r * lds + c / MXG]);
            y[r * ldy + c] = orc_f32_to_bf16(val);
        }
    }
}

/* Staged slice (P4 Behavior / Compatibility): one 128-column-aligned slice is
 * quantized into columns [col_off, col_off+cols) and scale columns
 * [col_off/32, (col_off+cols)/32) of caller-owned storage.  A slice never
 * splits a 32-column group, so this equals the corresponding columns of the
 * one-call quantization of the concatenated tensor. */
void orc_quant_mx_slice(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                        int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                        int64_t lds) {
    if (col_off % 128 != 0 || cols % 128 != 0) {
        fprintf(stderr, "bq_oracle: slices and offsets must be multiples of 128\n");
        abort();
    }
    orc_quant_mx(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / MXG, lds);
}

void orc_quant_mx_slice_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                            int64_t lds) {
    if (col_off % 128 != 0 || cols % 128 != 0) {
        fprintf(stderr, "bq_oracle: slices and offsets must be multiples of 128\n");
        abort();
    }
    orc_quant_mx_f16(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / MXG, lds);
}

/* ---------------------------------------------------------------------- */
/* MXFP8 scales in the order of the scaled matrix instruction (P4 Behavior: */
/* the staging holds the scale layout the GEMM consumes).  One 256-byte     */
/* tile serves 16 rows x 512 columns: the four K steps of 128 columns, each */
/* needing per lane l the byte of row l%16 and 32-column block l/16.        */
/* ---------------------------------------------------------------------- */

int64_t orc_mx_mfma_offset(int64_t row, int64_t group, int64_t row_blocks) {
    int64_t kgroup = group / 16;          /* which 512 columns */
    int64_t step = (group % 16) / 4;      /* which K step of 128 among the four */
    int64_t block = group % 4;            /* which 32 columns within the K step */
    int64_t rblock = row / 16;
    int64_t lane = 16 * block + row % 16; /* the lane that supplies this byte */
    int64_t tile = kgroup * row_blocks + rblock;
    return 256 * tile + 4 * lane + step;
}

void orc_mx_scales_to_mfma(const uint8_t* e8m0, int64_t lds, int64_t rows, int64_t groups,
                           int64_t group_off, int64_t row_blocks, uint8_t* out) {
    if (rows > 16 * row_blocks) {
        fprintf(stderr, "bq_oracle: more rows than the layout's row blocks hold\n");
        abort();
    }
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < groups; g++)
            out[orc_mx_mfma_offset(r, group_off + g, row_blocks)] = e8m0[r * lds + g];
}

/* ---------------------------------------------------------------------- */
/* MXFP8 on the collective topologies (P2 PR body Summary / Modes: mx_ring  */
/* and mx_a2a carry the same 132-byte-per-128 payload over the ring and the */
/* all-to-all, with the INT8 modes' canonical-payload rule).  The tensor is */
/* flat: n E4M3 bytes and n/32 E8M0 bytes, group g = values [32g, 32g+32). */
/* ---------------------------------------------------------------------- */

static void quant_mx_flat(const uint16_t* x, int64_t n, uint8_t* v, uint8_t* e8m0) {
    orc_quant_mx(x, 1, n, n, v, n, e8m0, n / MXG);
}

static void dequant_mx_flat(const uint8_t* v, const uint8_t* e8m0, int64_t n, uint16_t* y) {
    orc_dequant_mx(v, n, e8m0, n / MXG, 1, n, y, n);
}

/* One mx_ring hop: per value the binary32 sum fl32(dequantized payload value +
 * local), then each group's 32 binary32 sums requantized with the MXFP8 rule (no
 * bf16 intermediate, as in the INT8 hop).  v_out/e_out may equal v_in/e_in. */
void orc_ring_hop_mx(const uint8_t* v_in, const uint8_t* e_in, const uint16_t* local,
                     int64_t n, uint8_t* v_out, uint8_t* e_out) {
    need_blocks(n);
    float sums[MXG];
    for (int64_t g = 0; g < n / MXG; g++) {
        for (int i = 0; i < MXG; i++) {
            float dq = mx_value(v_in[g * MXG + i], e_in[g]);
            float lp = orc_bf16_to_f32(local[g * MXG + i]);
            sums[i] = dq + lp;
        }
        quant_group_mx(sums, v_out + g * MXG, e_out + g);
    }
}

/* The mx_a2a owner accumulate: acc = +0, then acc = acc + (source value) for the
 * sources in array order, in binary32; y = bf16(acc). */
void orc_dequant_accum_mx(int nsrc, const uint8_t* const* v, const uint8_t* const* e8m0,
                          int64_t n, uint16_t* y) {
    need_blocks(n);
    for (int64_t i = 0; i < n; i++) {
        float total = 0.0f;
        for (int src = 0; src < nsrc; ++src) {
            float term = mx_value(v[src][i], e8m0[src][i / MXG]);
            total = total + term;
        }
        y[i] = orc_f32_to_bf16(total);
    }
}

/* The mx_a2a owner step for nseg owners: the accumulate above on each owner's shard,
 * the bf16 sum requantized with the MXFP8 rule into v_out/e_out, and the owner's copy
 * materialized from that payload (composition of the steps, which is the definition). */
void orc_a2a_reduce_mx(int nseg, int nsrc, const uint8_t* const* v_srcs,
                       const uint8_t* const* e_srcs, int64_t seg_n, uint8_t* v_out,
                       uint8_t* e_out, uint16_t* const* y_out, uint16_t* red) {
    need_blocks(seg_n);
    const uint8_t** vp = (const uint8_t**)xmalloc((size_t)nsrc * sizeof(*vp));
    const uint8_t** ep = (const uint8_t**)xmalloc((size_t)nsrc * sizeof(*ep));
    uint16_t* sum = (uint16_t*)xmalloc((size_t)seg_n * sizeof(uint16_t));
    int64_t sg = seg_n / MXG;
    for (int j = 0; j < nseg; j++) {
        for (int k = 0; k < nsrc; k++) {
            vp[k] = v_srcs[k] + j * seg_n;
            ep[k] = e_srcs[k] + j * sg;
        }
        orc_dequant_accum_mx(nsrc, vp, ep, seg_n, sum);
        quant_mx_flat(sum, seg_n, v_out + j * seg_n, e_out + j * sg);
        if (y_out && y_out[j])
            dequant_mx_flat(v_out + j * seg_n, e_out + j * sg, seg_n, y_out[j]);
        if (red)
            memcpy(red + j * seg_n, sum, (size_t)seg_n * sizeof(uint16_t));
    }
    free(vp);
    free(ep);
    free(sum);
}

/* mx_ring: the i8_ring schedule with the MXFP8 codec -- chunk c = values
 * [c*n/W, (c+1)*n/W), quantized at step 0 by rank c+1, folded in by one hop per
 * later step at ranks c+2, ..., c, then materialized by every rank from its final
 * payload. */
void orc_ring_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                           uint8_t* v_final, uint8_t* e_final, uint16_t* const* out) {
    int W = world;
    need_blocks(n);
    if (W < 1 || n % ((int64_t)BLK * W) != 0) {
        fprintf(stderr, "bq_oracle: ring needs n divisible by 128*world\n");
        abort();
    }
    int64_t m = n / W, mg = m / MXG;
    for (int r = 0; r < W; r++) {
        int c = mod(r - 1, W);
        quant_mx_flat(partials[r] + c * m, m, v_final + c * m, e_final + c * mg);
    }
    for (int k = 1; k < W; k++) {
        for (int r = 0; r < W; r++) {
            int chunk = mod(r - 1 - k, W);
            orc_ring_hop_mx(v_final + chunk * m, e_final + chunk * mg, partials[r] + chunk * m,
                            m, v_final + chunk * m, e_final + chunk * mg);
        }
    }
    for (int r = 0; r < W; r++)
        for (int c = 0; c < W; c++)
            dequant_mx_flat(v_final + c * m, e_final + c * mg, m, out[r] + c * m);
}

/* mx_a2a: every rank quantizes its partial once with the MXFP8 rule; owner j
 * accumulates shard j of the W payloads in rank order (bf16 sum into red), requantizes
 * that bf16 sum once and broadcasts it; every rank materializes from the broadcast. */
void orc_a2a_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                          uint16_t* red, uint8_t* v_final, uint8_t* e_final,
                          uint16_t* const* out) {
    int W = world;
    need_blocks(n);
    if (W < 1 || n % ((int64_t)BLK * W) != 0) {
        fprintf(stderr, "bq_oracle: a2a needs n divisible by 128*world\n");
        abort();
    }
    int64_t m = n / W, mg = m / MXG, ng = n / MXG;
    uint8_t* vs = (uint8_t*)xmalloc((size_t)W * (size_t)n);
    uint8_t* es = (uint8_t*)xmalloc((size_t)W * (size_t)ng);
    const uint8_t** vp = (const uint8_t**)xmalloc((size_t)W * sizeof(*vp));
    const uint8_t** ep = (const uint8_t**)xmalloc((size_t)W * sizeof(*ep));
    for (int r = 0; r < W; r++)
        quant_mx_flat(partials[r], n, vs + (size_t)r * n, es + (size_t)r * ng);
    for (int j = 0; j < W; j++) {
        for (int r = 0; r < W; r++) {
            vp[r] = vs + (size_t)r * n + j * m;
            ep[r] = es + (size_t)r * ng + j * mg;
        }
        orc_dequant_accum_mx(W, vp, ep, m, red + j * m);
        quant_mx_flat(red + j * m, m, v_final + j * m, e_final + j * mg);
    }
    for (int r = 0; r < W; r++)
        for (int j = 0; j < W; j++)
            dequant_mx_flat(v_final + j * m, e_final + j * mg, m, out[r] + j * m);
    free(vs);
    free(es);
    free(vp);
    free(ep);
}

/* ---------------------------------------------------------------------- */
/* E4M3 128-block codec: the INT8 rule with the E4M3 maximum in place of   */
/* 127 (P1 Summary / Why give only its 132-byte footprint).                */
/* ---------------------------------------------------------------------- */

void orc_quant_e4m3_b128(const uint16_t* x, int64_t n, uint8_t* v, float* scale) {
    need_blocks(n);
    for (int64_t b = 0; b < n / BLK; b++) {
        float amax = 0.0f;
        for (int i = 0; i < BLK; i++) {
            float a = fabsf(orc_bf16_to_f32(x[b * BLK + i]));
            if (a > amax)
                amax = a;
        }
        if (amax == 0.0f) {
            scale[b] = 0.0f;
            for (int i = 0; i < BLK; i++)
                v[b * BLK + i] = 0x00;
            continue;
        }
        float s = amax / E4M3_MAX;
        scale[b] = s;
        for (int i = 0; i < BLK; i++) {
            float t = orc_bf16_to_f32(x[b * BLK + i]) / s;
            v[b * BLK + i] = orc_e4m3_encode(t);
        }
    }
}

void orc_dequant_e4m3_b128(const uint8_t* v, const float* scale, int64_t n, uint16_t* y) {
    need_blocks(n);
    for (int64_t i = 0; i < n; i++) {
        float val = orc_e4m3_decode(v[i]) * scale[i / BLK];
        y[i] = orc_f32_to_bf16(val);
    }
}
