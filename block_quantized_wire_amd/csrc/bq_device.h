// bq_device.h -- device building blocks of the libblockq kernels (gfx950, wave64).
//
// Work layouts of the codec kernels.  Kernels that write bf16 give a lane 8 consecutive
// values (one 16-byte bf16 vector): 16 lanes (one DPP row) own one 128-value block and a
// wave64 covers a "tile" of 4 blocks = 512 values per step (Lanes).  Kernels that write
// the one-byte side give a lane 16 values (one 16-byte payload vector): 8 lanes (half a
// DPP row) own a block and a tile is 8 blocks (Lanes16).  Per-block reductions therefore
// stay inside one DPP row and never touch LDS.
//
// Arithmetic follows the codec definitions bit for bit (IEEE binary32, round to
// nearest even, no contraction -- the library is compiled with -ffp-contract=off and
// denormals enabled).  Two shortcuts are used where they are provably exact:
//
//  * Block scales.  fl32(a/127) == fl32(fl64(a) * fl64(1/127)) for every finite
//    binary32 a: a/127 = M/127 * 2^k with M an integer, whose binary expansion is
//    purely periodic with period 7 (2^7 = 1 mod 127) unless exact.  The part beyond
//    the 24th significant bit is therefore p/127 of an ulp with p in 1..126, at least
//    1/254 ulp away from the rounding midpoint (also in the subnormal range, where
//    the grid is 2^-149), while the fp64 product is within 2^-52 relative.  The same
//    argument with period 3 covers a/448 = (a/7) * 2^-6 for bf16 a (no exact
//    midpoint is reachable from a bf16 numerator there either).
//
//  * Element quotients.  fl32(x/s) == fl32(fl64(x) * r) for fp32 x, s whenever r is
//    within 2^-52 (relative) of 1/s and x/s is a normal binary32: write x = X 2^a,
//    s = S 2^b with integer significands X, S < 2^24.  A binary32 rounding midpoint m
//    has an odd 25-bit significand, so x/s == m would need X's odd part to be a
//    multiple of a number >= 2^24 + 1, which it is not; otherwise |x/s - m| is at
//    least 2^-49 (relative), because the difference is a nonzero integer over S 2^25.
//    The fp64 product errs by less than 2^-51, so it rounds to the same binary32.
//    Quotients below the normal range round to 0 (INT8) or to a zero E4M3 code of the
//    right sign either way.  r is rcp(s) in fp64 refined by two Newton steps.
//    On MI355X non-packed fp32 and fp64 instructions issue at the same rate, so the
//    fp64 product costs little more than an fp32 one, with no branch.
//
// Conversions use gfx950's packed instructions, whose rounding is the codecs':
// v_cvt_pk_bf16_f32 rounds binary32 to bf16 to nearest even (subnormals kept, overflow
// to infinity); v_cvt_pk_fp8_f32 rounds to the nearest OCP E4M3FN code with ties to
// even and keeps the sign of zero, but turns magnitudes from 464 up into NaN, so its
// inputs stay below 449 in magnitude (see e4m3x4); v_cvt_pk_f32_fp8 decodes exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

constexpr int kBlock = 128;           // values per INT8 / E4M3 block
constexpr int kLaneVals = 8;          // values per lane per tile
constexpr int kTileBlocks = 4;        // blocks per wave64 tile
constexpr int kTileVals = 512;        // values per wave64 tile
constexpr int kWavesPerGroup = 4;     // 256-thread workgroups
constexpr int kGroupThreads = 256;
constexpr int kMaxBatch = 16;
constexpr int kMaxSrc = 64;
// Most workgroups of one launch before the waves start walking tiles grid-stride.
// Measured on MI355X (256 CUs): a grid that covers every tile once streams faster
// than a persistent grid of 4-16 groups per CU, so the cap only matters for the
// largest tensors.
constexpr int kMaxGroups = 256 * 64;

// ---- vector memory ----------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16- and 8-byte vector accesses.  Loads use the default cache policy, so a kernel that
// consumes what the previous kernel of a pipeline just wrote (a wire payload, a staged
// buffer) can be served by the 256 MB last-level cache; stores are non-temporal, since
// every output byte is written once and streamed out.  Measured on MI355X this beats
// non-temporal loads by 4-12% on the consumer kernels and costs at most 3% on cold
// inputs.
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
    return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st8(void* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// Write-through stores (device scope, the `sc1` policy): the data goes through the XCD's L2
// to the memory-side last-level cache at once instead of staying dirty in L2 until the end
// of the kernel.  A quantizer whose payload is read by the next kernel -- the ring's step 0
// before the first hop -- finishes sooner and its consumer finds the payload in the
// last-level cache: measured on MI355X (kernel trace), 4 x 768x7168 quantize 12.9 against
// 13.8 us and the hop after it 15.6 against 16.4 us.  Larger outputs stream faster with
// the non-temporal policy, so the launchers choose by output size (kWriteThroughBytes).
// The hop keeps non-temporal stores: written through, the next hop ran 0.8 us slower.
__device__ __forceinline__ void st16_wt(void* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st4_wt(void* p, uint32_t v) {
    asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
template <bool WT>
__device__ __forceinline__ void st16_out(void* p, u32x4 v) {
    if constexpr (WT)
        st16_wt(p, v);
    else
        st16(p, v);
}
// Largest payload output (all segments of a launch, payload and scales) written through.
// Measured on MI355X over three alternating runs of the benchmark: the ring's step-0
// quantize (23 MB out) plus three hops 5800 against 5586 GB/s; at a 128 MiB limit the
// 4-rank whole-tensor quantize (91 MB out) took 47.4 against 45.6 us and the whole step
// ran 1% slower, at 64 MiB the step is unchanged.
constexpr int64_t kWriteThroughBytes = (int64_t)64 << 20;

// ---- bf16 <-> binary32 --------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack_bf16x8(u32x4 w, float f[8]) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The 8 IEEE binary16 values of a 16-byte vector as binary32 (v_cvt_f32_f16 is exact,
// subnormals included: denormals are not flushed in this library).
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack_f16x8(u32x4 w, float f[8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h16x2 h = __builtin_bit_cast(h16x2, ws[i]);
        f[2 * i] = (float)h.x;
        f[2 * i + 1] = (float)h.y;
    }
}

// Round two binary32 values to bf16 (nearest, ties to even) and pack them, a in the
// low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float f[8]) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
}

// ---- DPP row reductions (16 lanes) -----------------------------------------------------

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
}

// Max of a non-negative binary32 (given as bits) over the 16 lanes of a DPP row.
// For non-negative floats the integer order of the bit patterns is the float order.
__device__ __forceinline__ uint32_t row_max16(uint32_t v) {
    v = max(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp<0x141>(v));   // row_half_mirror
    v = max(v, dpp<0x140>(v));   // row_mirror
    return v;
}

// Max of a non-negative binary32 (as bits) over the 8 lanes of a half DPP row: one block
// when a lane holds 16 values.
__device__ __forceinline__ uint32_t half_row_max8(uint32_t v) {
    v = max(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp<0x141>(v));   // row_half_mirror
    return v;
}

// Max over a pair of lanes (one MXFP8 group of 32 values when a lane holds 16).
__device__ __forceinline__ uint32_t pair_max2(uint32_t v) {
    return max(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
}

// The 4 E8M0 bytes of a block whose lanes hold 16 values -- one byte per lane pair of its
// half row -- packed into a word in the block's first lane, group 0 in byte 0.
__device__ __forceinline__ uint32_t gather_e8m0_pairs(uint32_t byte) {
    return byte | (dpp<0x102>(byte) << 8) | (dpp<0x104>(byte) << 16) | (dpp<0x106>(byte) << 24);
}

// Max over the 4 lanes of a quad (one MXFP8 group of 32 values).
__device__ __forceinline__ uint32_t quad_max4(uint32_t v) {
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    return v;
}

// ---- block INT8 ------------------------------------------------------------------------

// fl32(amax / 127) without an fp32 division (exact; see the header comment).
__device__ __forceinline__ float i8_scale(float amax) {
    return (float)((double)amax * (1.0 / 127.0));
}

// fl32(amax / 448) for a bf16 amax (exact; see the header comment).
__device__ __forceinline__ float e4m3_block_scale(float amax) {
    return (float)((double)amax * (1.0 / 448.0));
}

// round-half-even(t) for binary32 |t| < 2^22, as a bit pattern whose low byte is the
// result's two's-complement byte: t + 1.5 * 2^23 has ulp 1, so the binary32 sum (rounded to
// nearest even) is exactly 1.5 * 2^23 + rint(t), bit pattern 0x4B400000 + rint(t).  Ties go
// to even as rintf's do, and -0 and small negatives that round to zero give byte 0.
__device__ __forceinline__ uint32_t rint_low_byte(float t) { return __float_as_uint(t + 0x1.8p23f); }

// Pack the low bytes of four words into one word.
__device__ __forceinline__ uint32_t pack_lo_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);   // [a0, b0, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);   // [0, 0, c0, d0]
    return lo | hi;
}

// fl64(1/s) to within 2^-52 (relative) for a positive finite binary32 s: the hardware
// fp64 reciprocal refined by two Newton-Raphson steps (each squares the error).
__device__ __forceinline__ double recip64(float s) {
    const double d = (double)s;
    double r = __builtin_amdgcn_rcp(d);
    r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
    r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
    return r;
}

// fl32(x / s) exactly (see the header comment), given r = recip64(s).
__device__ __forceinline__ float quot32(float x, double r) { return (float)((double)x * r); }

// Quantize 8 binary32 values of one lane with its block's scale s = fl32(amax/127):
// q = round-half-even(fl32(x/s)) clamped to [-127, 127].  A block whose amax is 0 -- or
// whose scale underflows to 0, which only binary32 sums can reach -- is a zero block:
// scale 0, payload 0.
// The clamp can only bind when s is subnormal.  A normal s is within 2^-24 (relative) of
// amax/127, so |x/s| <= 127 (1 + 2^-23) rounds to at most 127.  A subnormal s keeps only
// the bits above 2^-149, and with few of them the quotient overshoots: amax = 190 * 2^-149
// (a ring hop's binary32 sums reach such values) gives s = 2^-149 and x/s = 190.  Below
// the normal range amax < 127 * 2^-126 and |x/s| <= 190 < 2^22, so rint_low_byte's range
// holds before the clamp too.  Blocks with a subnormal scale are rare, so the clamp sits
// behind a branch that waves skip when none of their lanes has one.
__device__ __forceinline__ u32x2 quant_i8x8(const float f[8], float s) {
    if (s == 0.0f)
        return u32x2{};
    const double r = recip64(s);
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        t[i] = quot32(f[i], r);
    if (s < 0x1p-126f) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = __builtin_fminf(__builtin_fmaxf(t[i], -127.0f), 127.0f);
    }
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        b[i] = rint_low_byte(t[i]);
    return u32x2{pack_lo_bytes(b[0], b[1], b[2], b[3]), pack_lo_bytes(b[4], b[5], b[6], b[7])};
}

// Dequantize the 8 signed payload bytes of a lane: f = fl32(q * s), the binary32 product of
// the definition, for every scale.  Each byte converts exactly (one sign-extending byte
// conversion), and one multiply rounds the product.
__device__ __forceinline__ void dequant_i8x8(u32x2 w, float s, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = (float)(int)(int8_t)((w.x >> (8 * i)) & 0xFFu) * s;
        f[i + 4] = (float)(int)(int8_t)((w.y >> (8 * i)) & 0xFFu) * s;
    }
}

// ---- OCP E4M3FN ------------------------------------------------------------------------

// E4M3FN codes of four binary32 values of magnitude below 449 packed into a word (a in byte
// 0): nearest code, ties to even, magnitudes above 448 saturate to 448, sign of zero kept.
// The hardware conversion does this without a clamp below 464 (it gives NaN from there), and
// every caller stays below 449: an MXFP8 group scale 2^e >= fl32(amax/448) leaves at most
// 448 / (1 - 2^-24), and an E4M3-b128 quotient x / fl32(amax/448) of bf16 data at most
// 2^16 / 146 = 448.88 (amax 2^-133, whose scale rounds down to 146 * 2^-149; a normal amax keeps it
// within 448 (1 + 2^-23)).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ u32x2 e4m3x8(const float f[8]) {
    return u32x2{e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7])};
}

// Exact binary32 values of the four E4M3FN codes of a word (byte 0 first).
__device__ __forceinline__ void e4m3_decode4(uint32_t w, float* f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
}

// E4M3FN codes of fl32(x / s) for the 8 values of a lane, s > 0 the block scale; the
// binary32 quotients are exact (see the header comment).
__device__ __forceinline__ u32x2 e4m3_quot8(const float f[8], float s) {
    const double r = recip64(s);
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        t[i] = quot32(f[i], r);
    return e4m3x8(t);
}

// MXFP8 shared-scale byte from a bf16 amax given as its 15 magnitude bits: 127 for an
// all-zero group; else 127 + (smallest e with 2^e >= fl32(amax/448)), clamped to
// [-127, 127].  For amax = m * 2^k (m in [1, 2)) that e is k - 8 + [m > 1.75], i.e.
// biased exponent - 8 plus one when the 7 stored significand bits exceed 96; bf16
// subnormals and anything below clamp to byte 0.
__device__ __forceinline__ uint32_t e8m0_from_bf16_amax(uint32_t h) {
    if (h == 0)
        return 127u;
    int e = (int)(h >> 7) - 8 + (((h & 0x7Fu) > 96u) ? 1 : 0);
    return (uint32_t)(e < 0 ? 0 : e);
}

// MXFP8 shared-scale byte from a binary32 amax >= 0 (the binary32 sums of a ring hop):
// 127 for amax == 0; else 127 + (smallest e with 2^e >= t), t = fl32(amax/448), clamped to
// [-127, 127].  t is taken from the fp64 product amax * fl64(1/448).  For a normal t that
// product rounds to fl32(amax/448) itself (the period-3 argument of the header holds for
// every binary32 numerator; an exact quotient stays exact), and the byte is the biased
// exponent plus one unless the significand bits are zero.  For t below 2^-126 the byte
// is 1 when t > 2^-127 and 0 otherwise; there the product can differ from fl32(amax/448)
// only at a tie between two subnormals, and no binary32 amax puts a tie next to 2^-127
// (it would need a 26-bit odd significand), so the byte is exact for every amax.
__device__ __forceinline__ uint32_t e8m0_from_f32_amax(float amax) {
    if (amax == 0.0f)
        return 127u;
    const uint32_t b = __float_as_uint((float)((double)amax * (1.0 / 448.0)));
    if (b >= 0x00800000u)
        return (b + 0x007FFFFFu) >> 23;
    return b > 0x00400000u ? 1u : 0u;
}

// 2^(byte - 127) as binary32: a normal number for byte >= 1, the subnormal 2^-127 for
// byte 0 (any E4M3 value times it is exact: the codes are multiples of 2^-9).
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
    return __uint_as_float(byte ? (byte << 23) : 0x00400000u);
}

// 2^(127 - byte) as binary32 for byte in [0, 254] (always a normal number here since
// the quantizer never produces a byte above 247).
__device__ __forceinline__ float e8m0_inv_scale(uint32_t byte) {
    return __uint_as_float((254u - byte) << 23);
}

// ---- MXFP8 scales in the scaled-MFMA operand order ----------------------------------------

// Byte offset of the E8M0 scale of (row, K step of 128 columns, 32-column block of that step)
// in the layout the GEMM's scaled matrix instruction reads: one K step of
// v_mfma_scale_f32_16x16x128_f8f6f4 takes from lane l the scale of row l%16 and 32-column
// block l/16, so a 256-byte tile holds 16 rows x 4 K steps as 64 words (word l for lane l,
// byte j for K step j of the four); tiles are ordered by group of 4 K steps, then by 16-row
// block, of `rb` row blocks.
__device__ __forceinline__ int64_t mfma_scale_offset(uint32_t row, uint32_t step, uint32_t block,
                                                     int64_t rb) {
    const int64_t tile = (int64_t)(step >> 2) * rb + (row >> 4);
    return tile * 256 + 4 * (16 * block + (row & 15)) + (step & 3);
}

// ---- lane walk -----------------------------------------------------------------------

// Lane bookkeeping of the flat kernels with 8 values per lane (one 128-value block per DPP
// row): the lane's block within a tile and its first value in that block.  Waves walk the
// tiles grid-stride, U adjacent tiles per step, so a launch needs no more workgroups than
// the chip holds at once.
// The wave index is read from the first lane, so the tile a wave works on is a uniform
// (scalar) value: each access is a scalar base of the step plus a small 32-bit lane
// offset, which keeps addresses out of the vector registers.
struct Lanes {
    uint32_t sub, off;
    bool leader;     // first lane of the row: stores the block's scale
    int64_t first;   // first tile of this wave
    int64_t step;    // tiles between successive steps of this wave
    __device__ explicit Lanes(int U) {
        const uint32_t lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        sub = lane >> 4;
        off = (lane & 15) * kLaneVals;
        leader = (lane & 15) == 0;
        first = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
        step = (int64_t)gridDim.x * kWavesPerGroup * U;
    }
    // MXFP8 group (0..3) of the lane's 8 values within its block: one quad per group
    __device__ __forceinline__ uint32_t grp() const { return off >> 5; }
    // block of tile u of a step, counted from the step's first block
    __device__ __forceinline__ uint32_t blk(int u) const { return (uint32_t)u * kTileBlocks + sub; }
    // first value of this lane in tile u of a step, counted from the step's first value
    __device__ __forceinline__ uint32_t val(int u) const { return blk(u) * kBlock + off; }
};

__device__ __forceinline__ int64_t tiles_of(int64_t nb) { return (nb + kTileBlocks - 1) / kTileBlocks; }

// The same walk with 16 values per lane: a block is the 8 lanes of a half DPP row and a
// wave64 tile is 8 blocks.  A lane then reads or writes its block's one-byte values as one
// 16-byte vector, which the kernels whose one-byte side is an output (quantize, ring hop)
// stream measurably faster; their bf16 side becomes two 16-byte vectors per lane.
constexpr int kLaneVals16 = 16;
constexpr int kTileBlocks16 = 8;
struct Lanes16 {
    uint32_t sub, off;
    bool leader;     // first lane of the block: stores its scale
    int64_t first;   // first tile of this wave
    int64_t step;    // tiles between successive steps of this wave
    __device__ explicit Lanes16(int U) {
        const uint32_t lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        sub = lane >> 3;
        off = (lane & 7) * kLaneVals16;
        leader = (lane & 7) == 0;
        first = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
        step = (int64_t)gridDim.x * kWavesPerGroup * U;
    }
    // block of tile u of a step, counted from the step's first block
    __device__ __forceinline__ uint32_t blk(int u) const { return (uint32_t)u * kTileBlocks16 + sub; }
    // first value of this lane in tile u of a step, counted from the step's first value
    __device__ __forceinline__ uint32_t val(int u) const { return blk(u) * kBlock + off; }
};

__device__ __forceinline__ int64_t tiles16_of(int64_t nb) {
    return (nb + kTileBlocks16 - 1) / kTileBlocks16;
}

// Launch shape of the flat kernels: 256-thread workgroups of 4 waves, U tiles of 4
// blocks per wave step; at most kMaxGroups workgroups in all (the `count` segments of a
// batch, grid.y, share them).
template <int U>
dim3 grid_for(int64_t nb, int count) {
    const int64_t per_group = (int64_t)kWavesPerGroup * U * kTileBlocks;
    const int64_t want = (nb + per_group - 1) / per_group;
    const int64_t cap = kMaxGroups / count > 0 ? kMaxGroups / count : 1;
    return dim3((unsigned)(want < cap ? want : cap), (unsigned)count, 1);
}

// Launch shape of the kernels on the 16-values-per-lane walk (tiles of 8 blocks).
template <int U>
dim3 grid16_for(int64_t nb, int count) {
    const int64_t per_group = (int64_t)kWavesPerGroup * U * kTileBlocks16;
    const int64_t want = (nb + per_group - 1) / per_group;
    const int64_t cap = kMaxGroups / count > 0 ? kMaxGroups / count : 1;
    return dim3((unsigned)(want < cap ? want : cap), (unsigned)count, 1);
}

}  // namespace bq
