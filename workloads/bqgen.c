/*
 * bqgen.c -- seeded synthetic inputs for the block-quantized wire codecs.
 *
 * This module holds none of the codecs' arithmetic: it only draws numbers.
 * It is the one piece shared by the CPU oracle's tests and the GPU tests and
 * benchmark, which both call it for their inputs.
 *
 * Generators (published definitions, restated):
 *   - splitmix64 (Steele, Lea, Flood 2014) expands a 64-bit key into state;
 *   - xoshiro256** (Blackman, Vigna 2018) draws 64-bit words;
 *   - uniform doubles in (0, 1] from the top 53 bits;
 *   - standard normals by the Box-Muller transform (both branches used);
 *   - Student-t(nu) = Z / sqrt(chi2_nu / nu), chi2_nu a sum of nu squared normals.
 *
 * Every (config, rank, stream kind, row) has its own stream, so any row of
 * any rank can be regenerated on its own, in any order and on any number of
 * threads, with identical results.  Values are drawn in double, cast to
 * binary32 and then TRUNCATED to bf16 (the top 16 bits), or -- for the FP16
 * slice inputs -- truncated toward zero to IEEE binary16 from the double,
 * saturating at the binary16 maximum 65504 and keeping binary16 subnormals.
 * Truncation is a deliberate choice: the codecs round to nearest-even, and
 * the generator shares no rounding code with them.
 *
 * Build: cc -std=c99 -O2 -fopenmp -fPIC -shared -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { K_VALUE = 1, K_OUTLIER = 2, K_ZERO = 3, K_SPIKE = 4, K_GAIN = 5, K_SIGN = 6 };

typedef struct {
    uint64_t s[4];
    int have_spare;
    double spare;
} rng_t;

static uint64_t splitmix64(uint64_t* x) {
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void rng_init(rng_t* r, int cfg, int rank, int kind, int64_t row) {
    uint64_t key = ((uint64_t)(cfg & 0xFF) << 56) ^ ((uint64_t)(rank & 0xFF) << 48) ^
                   ((uint64_t)(kind & 0xFF) << 40) ^ ((uint64_t)row & 0xFFFFFFFFFFull);
    for (int i = 0; i < 4; i++)
        r->s[i] = splitmix64(&key);
    r->have_spare = 0;
    r->spare = 0.0;
}

static uint64_t rotl(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static uint64_t next_u64(rng_t* r) {
    uint64_t* s = r->s;
    uint64_t out = rotl(s[1] * 5u, 7) * 9u;
    uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl(s[3], 45);
    return out;
}

/* uniform in (0, 1] */
static double uniform(rng_t* r) { return (double)((next_u64(r) >> 11) + 1u) * 0x1.0p-53; }

static double normal(rng_t* r) {
    if (r->have_spare) {
        r->have_spare = 0;
        return r->spare;
    }
    double u1 = uniform(r), u2 = uniform(r);
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925 * u2;
    r->spare = rad * sin(ang);
    r->have_spare = 1;
    return rad * cos(ang);
}

static double student_t(rng_t* r, int nu) {
    double z = normal(r);
    double chi2 = 0.0;
    for (int i = 0; i < nu; i++) {
        double g = normal(r);
        chi2 += g * g;
    }
    return z / sqrt(chi2 / (double)nu);
}

static uint16_t to_bf16_trunc(double d) {
    float f = (float)d;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* binary16 bits of d truncated toward zero (finite d). */
static uint16_t to_f16_trunc(double d) {
    uint16_t sign = signbit(d) ? 0x8000u : 0u;
    double a = fabs(d);
    if (a >= 65504.0)
        return sign | 0x7BFFu;
    if (a < 0x1.0p-14)                                   /* subnormal: multiples of 2^-24 */
        return sign | (uint16_t)floor(a * 0x1.0p24);
    int e;
    double m = frexp(a, &e);                             /* a = m 2^e, m in [0.5, 1) */
    uint16_t man = (uint16_t)floor((m * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)((e - 1 + 15) << 10) | man;
}

/* output format of a generated value: 0 = bf16 (truncated), 1 = binary16 (truncated) */
static uint16_t enc(double d, int fmt) { return fmt == 1 ? to_f16_trunc(d) : to_bf16_trunc(d); }

/*
 * Config table.  Shapes are rows x cols of one rank's (or slice's) tensor.
 *   1: 512x7168, N(0,1); each element x50 with prob 1e-3; each 128-block
 *      zeroed with prob 0.02.
 *   2: 3072x7168 per rank, N(0,0.5).
 *   3: 3072x7168 per rank, 0.3 * t(4).
 *   4: 4096x7168 per slice, N(0,1) * g_row, g log-uniform in [1e-3, 1e2].
 *   5: 16384x7168 per rank, t(3); each 128-block zeroed with prob 0.01;
 *      each element replaced by +-1e3 with prob 1e-5.
 *   6: generic N(0,1) of any shape (edge-case tests).
 *   7: generic 0.3 * t(4) of any shape.
 * Zero-block positions are drawn from rank 0's stream for every rank, so
 * they coincide across ranks and survive the sums of a collective.
 */
int bqgen_shape(int cfg, int64_t* rows, int64_t* cols) {
    switch (cfg) {
    case 1: *rows = 512; *cols = 7168; return 0;
    case 2: *rows = 3072; *cols = 7168; return 0;
    case 3: *rows = 3072; *cols = 7168; return 0;
    case 4: *rows = 4096; *cols = 7168; return 0;
    case 5: *rows = 16384; *cols = 7168; return 0;
    default: return -1;
    }
}

static void gen_row(int cfg, int rank, int64_t row, int64_t cols, uint16_t* out, int fmt) {
    rng_t rv, ro, rz, rs, rg, rsg;
    rng_init(&rv, cfg, rank, K_VALUE, row);
    switch (cfg) {
    case 1: {
        rng_init(&ro, cfg, rank, K_OUTLIER, row);
        rng_init(&rz, cfg, 0, K_ZERO, row);
        for (int64_t b = 0; b < cols / 128; b++) {
            int zero = uniform(&rz) <= 0.02;
            for (int64_t i = b * 128; i < b * 128 + 128; i++) {
                double v = normal(&rv);
                if (uniform(&ro) <= 1e-3)
                    v *= 50.0;
                out[i] = zero ? 0 : enc(v, fmt);
            }
        }
        break;
    }
    case 2:
        for (int64_t i = 0; i < cols; i++)
            out[i] = enc(0.5 * normal(&rv), fmt);
        break;
    case 3:
    case 7:
        for (int64_t i = 0; i < cols; i++)
            out[i] = enc(0.3 * student_t(&rv, 4), fmt);
        break;
    case 4: {
        rng_init(&rg, cfg, rank, K_GAIN, row);
        double lg = log(1e-3) + (log(1e2) - log(1e-3)) * uniform(&rg);
        double g = exp(lg);
        for (int64_t i = 0; i < cols; i++)
            out[i] = enc(g * normal(&rv), fmt);
        break;
    }
    case 5: {
        rng_init(&rz, cfg, 0, K_ZERO, row);
        rng_init(&rs, cfg, rank, K_SPIKE, row);
        rng_init(&rsg, cfg, rank, K_SIGN, row);
        for (int64_t b = 0; b < cols / 128; b++) {
            int zero = uniform(&rz) <= 0.01;
            for (int64_t i = b * 128; i < b * 128 + 128; i++) {
                double v = student_t(&rv, 3);
                if (uniform(&rs) <= 1e-5)
                    v = (uniform(&rsg) <= 0.5) ? 1e3 : -1e3;
                out[i] = zero ? 0 : enc(v, fmt);
            }
        }
        break;
    }
    default: /* 6 */
        for (int64_t i = 0; i < cols; i++)
            out[i] = enc(normal(&rv), fmt);
        break;
    }
}

/* Rows [row0, row0+nrows) of `rank`'s tensor for config `cfg`, cols values
 * per row (cols a multiple of 128), written densely to out in format fmt
 * (0 = bf16, 1 = binary16). */
void bqgen_rows_fmt(int cfg, int rank, int64_t row0, int64_t nrows, int64_t cols, uint16_t* out,
                    int nthreads, int fmt) {
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t r = 0; r < nrows; r++)
        gen_row(cfg, rank, row0 + r, cols, out + r * cols, fmt);
    (void)nthreads;
}

void bqgen_rows(int cfg, int rank, int64_t row0, int64_t nrows, int64_t cols, uint16_t* out,
                int nthreads) {
    bqgen_rows_fmt(cfg, rank, row0, nrows, cols, out, nthreads, 0);
}
