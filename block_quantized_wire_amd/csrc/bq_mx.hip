// bq_mx.hip -- MXFP8 and E4M3 128-block codec kernels for gfx950.
//
// MXFP8 (sparkinfer pull request #72, "feat(pcie_dma): add INT8 and MXFP8 wire modes":
// PR body Summary, and the review comment showing the device helper mxfp8_scale_byte;
// b12x pull request #241, "[II] Support staged MXFP8 linear inputs": Behavior and
// Compatibility):
//   per 32 consecutive columns of a row, byte = 127 for an all-zero group, else
//   127 + the smallest e with 2^e >= fl32(amax/448), clamped to [-127, 127];
//   v = e4m3_rne_sat(x * 2^-(byte-127)); dequantize y = bf16_rne(fl32(e4m3 * 2^(byte-127))).
// E4M3 128-block codec (sparkinfer pull request #46, Summary and Why: the format that the
// INT8 codec replaces, 132 bytes per 128 values):
//   scale = fl32(amax/448), v = e4m3_rne_sat(fl32(x/scale)), all-zero block -> scale 0
//   and bytes 0x00; dequantize y = bf16_rne(fl32(e4m3 * scale)).
//
// Same lane layouts as the INT8 kernels.  The quantizers give a lane 16 values (a
// 128-column block per half DPP row; an MXFP8 group of 32 is a lane pair, its amax one DPP
// step) so that each lane stores its codes as one 16-byte vector; the dequantizers give it
// 8 (a block per DPP row, a group per quad) so that each lane stores one 16-byte bf16
// vector.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

namespace {

// Division by an invariant 32-bit divisor d >= 1 for numerators below 2^31
// (Granlund & Montgomery): q = (umulhi(n, m) + n) >> l, l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, l;
    static FastDiv make(uint32_t d) {
        FastDiv f{};
        f.d = d;
        uint32_t l = 0;
        while ((1ull << l) < d)
            ++l;
        f.l = l;
        f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
        return f;
    }
    __device__ uint32_t div(uint32_t n) const { return (__umulhi(n, m) + n) >> l; }
};

struct MxArgs {
    const uint16_t* x;   // quantize input / dequantize output (as bf16 bits)
    uint8_t* v;
    uint8_t* e;          // row-major scales; or, in the MFMA layout, the layout's base
    int64_t ldx, ldv, lds;
    int64_t rb;          // MFMA layout: its 16-row blocks
    uint32_t step0;      // MFMA layout: the K step of the matrix's column 0
    uint32_t nblocks;    // rows * (cols / 128)
    FastDiv per_row;     // cols / 128
};

struct MxLane {
    uint32_t row, cb;    // row and 128-column block of the lane's block
    bool in;
};

__device__ __forceinline__ MxLane mx_lane(const MxArgs& a, int64_t tile, int sub,
                                          int tile_blocks = kTileBlocks) {
    MxLane m;
    const int64_t b = tile * tile_blocks + sub;
    m.in = b < (int64_t)a.nblocks;
    const uint32_t bb = m.in ? (uint32_t)b : 0u;
    m.row = a.per_row.div(bb);
    m.cb = bb - m.row * a.per_row.d;
    return m;
}

// Grid-stride walk over tiles of 4 blocks (8 values per lane), U adjacent tiles per wave step.
struct Walk {
    int sub, off;
    int64_t first, step;
    __device__ explicit Walk(int U) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // uniform
        sub = lane >> 4;
        off = (lane & 15) * kLaneVals;
        first = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
        step = (int64_t)gridDim.x * kWavesPerGroup * U;
    }
};

// The same walk with 16 values per lane: tiles of 8 blocks, a block per half DPP row.
struct Walk16 {
    int sub, off;
    int64_t first, step;
    __device__ explicit Walk16(int U) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // uniform
        sub = lane >> 3;
        off = (lane & 7) * kLaneVals16;
        first = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
        step = (int64_t)gridDim.x * kWavesPerGroup * U;
    }
};

// A lane holds 16 values (Walk16): a 32-column group is a lane pair, and the block's codes
// are one 16-byte store per lane.
// F16: the input is IEEE binary16 (b12x pull request #241, Behavior: BF16 or FP16 slices);
// the group byte then comes from the binary32 amax rule, which is exact for any amax.
// Mfma: the scale bytes go to the scaled-MFMA layout (one byte store per lane pair) instead
// of four bytes per 128 columns of a row-major scale row.
template <int U, bool F16, bool Mfma = false>
__global__ __launch_bounds__(kGroupThreads) void k_quant_mx(MxArgs a) {
    const Walk16 w(U);
    const int lane = threadIdx.x & 63;
    const int64_t nt = ((int64_t)a.nblocks + kTileBlocks16 - 1) / kTileBlocks16;
    for (int64_t t0 = w.first; t0 < nt; t0 += w.step) {
        u32x4 xv[U][2];
        MxLane ml[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ml[u] = mx_lane(a, t0 + u, w.sub, kTileBlocks16);
            const uint16_t* src = a.x + ml[u].row * a.ldx + ml[u].cb * kBlock + w.off;
            xv[u][0] = ml[u].in ? ld16(src) : u32x4{};
            xv[u][1] = ml[u].in ? ld16(src + 8) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[16];
            if constexpr (F16) {
                unpack_f16x8(xv[u][0], f);
                unpack_f16x8(xv[u][1], f + 8);
            } else {
                unpack_bf16x8(xv[u][0], f);
                unpack_bf16x8(xv[u][1], f + 8);
            }
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
            const uint32_t amax_bits = pair_max2(__float_as_uint(m));
            const uint32_t byte = F16 ? e8m0_from_f32_amax(__uint_as_float(amax_bits))
                                      : e8m0_from_bf16_amax(amax_bits >> 16);
            const float inv = e8m0_inv_scale(byte);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                f[i] = f[i] * inv;                 // exact: a power of two
            const u32x2 lo = e4m3x8(f), hi = e4m3x8(f + 8);
            const uint32_t word = gather_e8m0_pairs(byte);
            if (ml[u].in) {
                st16(a.v + ml[u].row * a.ldv + ml[u].cb * kBlock + w.off, u32x4{lo.x, lo.y, hi.x, hi.y});
                if constexpr (Mfma) {
                    if ((lane & 1) == 0)
                        a.e[mfma_scale_offset(ml[u].row, a.step0 + ml[u].cb, (lane & 7) >> 1, a.rb)] =
                            (uint8_t)byte;
                } else if ((lane & 7) == 0) {
                    *reinterpret_cast<uint32_t*>(a.e + ml[u].row * a.lds + ml[u].cb * 4) = word;
                }
            }
        }
    }
}

// Mfma: the scales are read from the scaled-MFMA layout.
template <int U, bool Mfma = false>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_mx(MxArgs a) {
    const Walk w(U);
    const int grp = (threadIdx.x & 15) >> 2;
    const int64_t nt = ((int64_t)a.nblocks + kTileBlocks - 1) / kTileBlocks;
    uint16_t* y = const_cast<uint16_t*>(a.x);
    for (int64_t t0 = w.first; t0 < nt; t0 += w.step) {
        u32x2 vv[U];
        uint32_t ev[U];
        MxLane ml[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ml[u] = mx_lane(a, t0 + u, w.sub);
            vv[u] = ml[u].in ? ld8(a.v + ml[u].row * a.ldv + ml[u].cb * kBlock + w.off) : u32x2{};
            if constexpr (Mfma)
                ev[u] = ml[u].in ? a.e[mfma_scale_offset(ml[u].row, a.step0 + ml[u].cb, grp, a.rb)]
                                 : 127u;
            else
                ev[u] = ml[u].in ? a.e[ml[u].row * a.lds + ml[u].cb * 4 + grp] : 127u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float sc = e8m0_value(ev[u]);
            float f[8];
            e4m3_decode4(vv[u].x, f);
            e4m3_decode4(vv[u].y, f + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[i] = f[i] * sc;
            if (ml[u].in)
                st16(y + ml[u].row * a.ldx + ml[u].cb * kBlock + w.off, pack_bf16x8(f));
        }
    }
}

struct E4Args {
    const uint16_t* x;   // quantize input / dequantize output (as bf16 bits)
    uint8_t* v;
    float* s;
    int64_t nb;
};

// A lane holds 16 values (Walk16): the block's codes are one 16-byte store per lane.
template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_quant_e4m3_b128(E4Args a) {
    const uint16_t* __restrict__ x = a.x;
    uint8_t* __restrict__ v = a.v;
    float* __restrict__ s = a.s;
    const int64_t nb = a.nb;
    const Walk16 w(U);
    const bool leader = (threadIdx.x & 7) == 0;
    const int64_t nt = (nb + kTileBlocks16 - 1) / kTileBlocks16;
    for (int64_t t0 = w.first; t0 < nt; t0 += w.step) {
        u32x4 xv[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = (t0 + u) * kTileBlocks16 + w.sub;
            xv[u][0] = (b < nb) ? ld16(x + b * kBlock + w.off) : u32x4{};
            xv[u][1] = (b < nb) ? ld16(x + b * kBlock + w.off + 8) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = (t0 + u) * kTileBlocks16 + w.sub;
            float f[16];
            unpack_bf16x8(xv[u][0], f);
            unpack_bf16x8(xv[u][1], f + 8);
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
            const float amax = __uint_as_float(half_row_max8(__float_as_uint(m)));
            const float sc = e4m3_block_scale(amax);
            // zero block: every byte 0x00 (negative zeros included)
            const u32x2 lo = (sc == 0.0f) ? u32x2{} : e4m3_quot8(f, sc);
            const u32x2 hi = (sc == 0.0f) ? u32x2{} : e4m3_quot8(f + 8, sc);
            if (b < nb) {
                st16(v + b * kBlock + w.off, u32x4{lo.x, lo.y, hi.x, hi.y});
                if (leader)
                    s[b] = sc;
            }
        }
    }
}

template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_e4m3_b128(E4Args a) {
    const uint8_t* __restrict__ v = a.v;
    const float* __restrict__ s = a.s;
    uint16_t* __restrict__ y = const_cast<uint16_t*>(a.x);
    const int64_t nb = a.nb;
    const Walk w(U);
    const int64_t nt = (nb + kTileBlocks - 1) / kTileBlocks;
    for (int64_t t0 = w.first; t0 < nt; t0 += w.step) {
        u32x2 vv[U];
        float sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = (t0 + u) * kTileBlocks + w.sub;
            const bool in = b < nb;
            vv[u] = in ? ld8(v + b * kBlock + w.off) : u32x2{};
            sv[u] = in ? s[b] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = (t0 + u) * kTileBlocks + w.sub;
            float f[8];
            e4m3_decode4(vv[u].x, f);
            e4m3_decode4(vv[u].y, f + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[i] = f[i] * sv[u];
            if (b < nb)
                st16(y + b * kBlock + w.off, pack_bf16x8(f));
        }
    }
}

template <int U>
unsigned groups_for(int64_t nb) {
    const int64_t per_group = (int64_t)kWavesPerGroup * U * kTileBlocks;
    const int64_t want = (nb + per_group - 1) / per_group;
    return (unsigned)(want < kMaxGroups ? want : kMaxGroups);
}

template <int U>
unsigned groups16_for(int64_t nb) {
    const int64_t per_group = (int64_t)kWavesPerGroup * U * kTileBlocks16;
    const int64_t want = (nb + per_group - 1) / per_group;
    return (unsigned)(want < kMaxGroups ? want : kMaxGroups);
}

constexpr int kUMx = 2;        // dequantize (8 values per lane)
constexpr int kUE4 = 2;
constexpr int kUMxQ = 1;       // quantize (16 values per lane)
constexpr int kUE4Q = 1;

}  // namespace

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds,
                           hipStream_t stream, bool f16) {
    MxArgs a{};
    a.x = x;
    a.v = v;
    a.e = e8m0;
    a.ldx = ldx;
    a.ldv = ldv;
    a.lds = lds;
    a.nblocks = (uint32_t)(rows * (cols / kBlock));
    a.per_row = FastDiv::make((uint32_t)(cols / kBlock));
    const dim3 grid(groups16_for<kUMxQ>(a.nblocks));
    if (f16)
        return launch1(k_quant_mx<kUMxQ, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_quant_mx<kUMxQ, false>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                             int64_t rows, int64_t cols, uint16_t* y, int64_t ldy,
                             hipStream_t stream) {
    MxArgs a{};
    a.x = y;
    a.v = const_cast<uint8_t*>(v);
    a.e = const_cast<uint8_t*>(e8m0);
    a.ldx = ldy;
    a.ldv = ldv;
    a.lds = lds;
    a.nblocks = (uint32_t)(rows * (cols / kBlock));
    a.per_row = FastDiv::make((uint32_t)(cols / kBlock));
    return launch1(k_dequant_mx<kUMx>, dim3(groups_for<kUMx>(a.nblocks)), dim3(kGroupThreads), stream, a);
}

hipError_t launch_quant_mx_mfma(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* v, int64_t ldv, uint8_t* e_layout, int64_t rb,
                                int64_t step0, hipStream_t stream, bool f16) {
    MxArgs a{};
    a.x = x;
    a.v = v;
    a.e = e_layout;
    a.ldx = ldx;
    a.ldv = ldv;
    a.rb = rb;
    a.step0 = (uint32_t)step0;
    a.nblocks = (uint32_t)(rows * (cols / kBlock));
    a.per_row = FastDiv::make((uint32_t)(cols / kBlock));
    const dim3 grid(groups16_for<kUMxQ>(a.nblocks));
    if (f16)
        return launch1(k_quant_mx<kUMxQ, true, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_quant_mx<kUMxQ, false, true>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_dequant_mx_mfma(const uint8_t* v, int64_t ldv, const uint8_t* e_layout,
                                  int64_t rb, int64_t rows, int64_t cols, uint16_t* y,
                                  int64_t ldy, hipStream_t stream) {
    MxArgs a{};
    a.x = y;
    a.v = const_cast<uint8_t*>(v);
    a.e = const_cast<uint8_t*>(e_layout);
    a.ldx = ldy;
    a.ldv = ldv;
    a.rb = rb;
    a.nblocks = (uint32_t)(rows * (cols / kBlock));
    a.per_row = FastDiv::make((uint32_t)(cols / kBlock));
    return launch1(k_dequant_mx<kUMx, true>, dim3(groups_for<kUMx>(a.nblocks)), dim3(kGroupThreads),
                   stream, a);
}

hipError_t launch_quant_e4m3_b128(const uint16_t* x, uint8_t* v, float* s, int64_t n,
                                  hipStream_t stream) {
    const E4Args a{x, v, s, n / kBlock};
    return launch1(k_quant_e4m3_b128<kUE4Q>, dim3(groups16_for<kUE4Q>(a.nb)), dim3(kGroupThreads),
                   stream, a);
}

hipError_t launch_dequant_e4m3_b128(const uint8_t* v, const float* s, uint16_t* y, int64_t n,
                                    hipStream_t stream) {
    const E4Args a{y, const_cast<uint8_t*>(v), const_cast<float*>(s), n / kBlock};
    return launch1(k_dequant_e4m3_b128<kUE4>, dim3(groups_for<kUE4>(a.nb)), dim3(kGroupThreads),
                   stream, a);
}

}  // namespace bq
