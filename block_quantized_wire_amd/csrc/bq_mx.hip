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
// Same lane layout as the INT8 kernels: 8 values per lane, one 128-column block per DPP
// row, so an MXFP8 group of 32 is one quad of lanes and its amax takes two DPP steps.
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
    uint8_t* e;
    int64_t ldx, ldv, lds;
    uint32_t nblocks;    // rows * (cols / 128)
    FastDiv per_row;     // cols / 128
};

struct MxLane {
    uint32_t row, cb;    // row and 128-column block of the lane's block in tile u
    bool in;
};

__device__ __forceinline__ MxLane mx_lane(const MxArgs& a, int64_t tile, int sub) {
    MxLane m;
    const int64_t b = tile * kTileBlocks + sub;
    m.in = b < (int64_t)a.nblocks;
    const uint32_t bb = m.in ? (uint32_t)b : 0u;
    m.row = a.per_row.div(bb);
    m.cb = bb - m.row * a.per_row.d;
    return m;
}

template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_quant_mx(MxArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
    const int sub = lane >> 4;
    const int off = (lane & 15) * kLaneVals;
    u32x4 xv[U];
    MxLane ml[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ml[u] = mx_lane(a, tile0 + u, sub);
        xv[u] = ml[u].in ? ld16(a.x + ml[u].row * a.ldx + ml[u].cb * kBlock + off) : u32x4{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[8];
        unpack_bf16x8(xv[u], f);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
        const uint32_t amax_bits = quad_max4(__float_as_uint(m));
        const uint32_t byte = e8m0_from_bf16_amax(amax_bits >> 16);
        const float inv = e8m0_inv_scale(byte);
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c[i] = e4m3_encode(f[i] * inv);
        const u32x2 packed{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                           c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
        // gather the 4 group bytes of this 128-column block into the row's first lane
        const uint32_t word = byte | (dpp<0x104>(byte) << 8) | (dpp<0x108>(byte) << 16) |
                              (dpp<0x10C>(byte) << 24);
        if (ml[u].in) {
            st8(a.v + ml[u].row * a.ldv + ml[u].cb * kBlock + off, packed);
            if ((lane & 15) == 0)
                *reinterpret_cast<uint32_t*>(a.e + ml[u].row * a.lds + ml[u].cb * 4) = word;
        }
    }
}

template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_mx(MxArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
    const int sub = lane >> 4;
    const int off = (lane & 15) * kLaneVals;
    const int grp = (lane & 15) >> 2;
    u32x2 vv[U];
    uint32_t ev[U];
    MxLane ml[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ml[u] = mx_lane(a, tile0 + u, sub);
        vv[u] = ml[u].in ? ld8(a.v + ml[u].row * a.ldv + ml[u].cb * kBlock + off) : u32x2{};
        ev[u] = ml[u].in ? a.e[ml[u].row * a.lds + ml[u].cb * 4 + grp] : 127u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // 2^(byte-127): a normal binary32 for byte >= 1, the subnormal 2^-127 for byte 0
        const float sc = __uint_as_float(ev[u] ? (ev[u] << 23) : 0x00400000u);
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = e4m3_decode((vv[u].x >> (8 * i)) & 0xFFu) * sc;
            f[i + 4] = e4m3_decode((vv[u].y >> (8 * i)) & 0xFFu) * sc;
        }
        if (ml[u].in)
            st16(const_cast<uint16_t*>(a.x) + ml[u].row * a.ldx + ml[u].cb * kBlock + off,
                 pack_bf16x8(f));
    }
}

template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_quant_e4m3_b128(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ v,
                                                                  float* __restrict__ s,
                                                                  int64_t nb) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
    const int sub = lane >> 4;
    const int off = (lane & 15) * kLaneVals;
    u32x4 xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = (tile0 + u) * kTileBlocks + sub;
        xv[u] = (b < nb) ? ld16(x + b * kBlock + off) : u32x4{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = (tile0 + u) * kTileBlocks + sub;
        float f[8];
        unpack_bf16x8(xv[u], f);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
        const float amax = __uint_as_float(row_max16(__float_as_uint(m)));
        const float sc = e4m3_block_scale(amax);
        uint32_t c[8];
        if (sc == 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c[i] = 0u;                    // zero block: every byte 0x00
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c[i] = e4m3_encode(f[i] / sc);
        }
        const u32x2 packed{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                           c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
        if (b < nb) {
            st8(v + b * kBlock + off, packed);
            if ((lane & 15) == 0)
                s[b] = sc;
        }
    }
}

template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_e4m3_b128(const uint8_t* __restrict__ v,
                                                                    const float* __restrict__ s,
                                                                    uint16_t* __restrict__ y,
                                                                    int64_t nb) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = ((int64_t)blockIdx.x * kWavesPerGroup + wave) * U;
    const int sub = lane >> 4;
    const int off = (lane & 15) * kLaneVals;
    u32x2 vv[U];
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = (tile0 + u) * kTileBlocks + sub;
        const bool in = b < nb;
        vv[u] = in ? ld8(v + b * kBlock + off) : u32x2{};
        sv[u] = in ? s[b] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = (tile0 + u) * kTileBlocks + sub;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = e4m3_decode((vv[u].x >> (8 * i)) & 0xFFu) * sv[u];
            f[i + 4] = e4m3_decode((vv[u].y >> (8 * i)) & 0xFFu) * sv[u];
        }
        if (b < nb)
            st16(y + b * kBlock + off, pack_bf16x8(f));
    }
}

template <int U>
unsigned groups_for(int64_t nb) {
    const int64_t per_group = (int64_t)kWavesPerGroup * U * kTileBlocks;
    return (unsigned)((nb + per_group - 1) / per_group);
}

constexpr int kUMx = 4;
constexpr int kUE4 = 4;

}  // namespace

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds,
                           hipStream_t stream) {
    MxArgs a{};
    a.x = x;
    a.v = v;
    a.e = e8m0;
    a.ldx = ldx;
    a.ldv = ldv;
    a.lds = lds;
    a.nblocks = (uint32_t)(rows * (cols / kBlock));
    a.per_row = FastDiv::make((uint32_t)(cols / kBlock));
    hipLaunchKernelGGL(k_quant_mx<kUMx>, dim3(groups_for<kUMx>(a.nblocks)), dim3(kGroupThreads),
                       0, stream, a);
    return hipGetLastError();
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
    hipLaunchKernelGGL(k_dequant_mx<kUMx>, dim3(groups_for<kUMx>(a.nblocks)), dim3(kGroupThreads),
                       0, stream, a);
    return hipGetLastError();
}

hipError_t launch_quant_e4m3_b128(const uint16_t* x, uint8_t* v, float* s, int64_t n,
                                  hipStream_t stream) {
    const int64_t nb = n / kBlock;
    hipLaunchKernelGGL(k_quant_e4m3_b128<kUE4>, dim3(groups_for<kUE4>(nb)), dim3(kGroupThreads),
                       0, stream, x, v, s, nb);
    return hipGetLastError();
}

hipError_t launch_dequant_e4m3_b128(const uint8_t* v, const float* s, uint16_t* y, int64_t n,
                                    hipStream_t stream) {
    const int64_t nb = n / kBlock;
    hipLaunchKernelGGL(k_dequant_e4m3_b128<kUE4>, dim3(groups_for<kUE4>(nb)),
                       dim3(kGroupThreads), 0, stream, v, s, y, nb);
    return hipGetLastError();
}

}  // namespace bq
