// bq_mxc.hip -- MXFP8 on the collective topologies (flat layout) for gfx950.
//
// Definitions (sparkinfer pull request #72, "feat(pcie_dma): add INT8 and MXFP8 wire
// modes": PR body Summary and Modes name the mx, mx_ring and mx_a2a modes with the INT8
// modes' canonical-payload rule; the review comment showing mxfp8_scale_byte gives the
// scale rule):
//   layout        n E4M3FN codes and n/32 E8M0 bytes, byte g scaling values [32g, 32g+32);
//   quantize      byte = 127 + the smallest e with 2^e >= fl32(amax/448), clamped to
//                 [-127, 127] (127 for an all-zero group); v = e4m3_rne_sat(x * 2^-(byte-127));
//   materialize   y = bf16_rne(e4m3 * 2^(byte-127)) (the product is exact);
//   ring hop      sum = fl32(payload value + local) in binary32, and each group of binary32
//                 sums requantized directly (no bf16 intermediate);
//   accumulate    y = bf16_rne(the binary32 sum, from +0 and in source order, of the
//                 sources' values);
//   owner step    the accumulate, its bf16 sum requantized, and the owner's copy
//                 materialized from that payload.
//
// Lane layouts of the INT8 kernels.  Quantize and ring hop give a lane 16 values: a
// 128-value block per half DPP row, a 32-value group per lane pair (its amax one DPP step),
// the codes one 16-byte store per lane.  Dequantize and accumulate give it 8: a block per
// DPP row, a group per quad (two DPP steps).  Either way the 4 E8M0 bytes of a block are
// gathered into the block's first lane and stored as one dword.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

namespace {

struct MxfQuantArgs {
    const uint16_t* x[kMaxBatch];
    uint8_t* v[kMaxBatch];
    uint8_t* e[kMaxBatch];
    int64_t nb;   // blocks per segment
};

struct MxfDequantArgs {
    const uint8_t* v[kMaxBatch];
    const uint8_t* e[kMaxBatch];
    uint16_t* y[kMaxBatch];
    int64_t nb;
    int64_t skip_nb;   // SkipOwn: segment i leaves blocks [i*skip_nb, (i+1)*skip_nb) untouched
};

struct MxfHopArgs {
    const uint8_t* v_in[kMaxBatch];
    const uint8_t* e_in[kMaxBatch];
    const uint16_t* local[kMaxBatch];
    uint8_t* v_out[kMaxBatch];
    uint8_t* e_out[kMaxBatch];
    int64_t nb;
};

struct MxfAccumArgs {
    const uint8_t* v[kMaxSrc];
    const uint8_t* e[kMaxSrc];
    uint16_t* red;            // bf16 sums, segment j at j * seg_n (fused: may be null)
    uint8_t* v_out;           // fused: requantized codes, segment j at j * seg_n
    uint8_t* e_out;           // fused: its E8M0 bytes, segment j at j * seg_n / 32
    uint16_t* y[kMaxBatch];   // fused: the owner's materialization of segment j (or null)
    int nsrc;
    int64_t nb;               // blocks per segment
    int64_t seg_n;            // values per segment
};

// The 4 E8M0 bytes of a block whose lanes hold 8 values -- one per quad of its DPP row --
// packed into a word in the row's first lane, group 0 in byte 0.
__device__ __forceinline__ uint32_t gather_e8m0(uint32_t byte) {
    return byte | (dpp<0x104>(byte) << 8) | (dpp<0x108>(byte) << 16) | (dpp<0x10C>(byte) << 24);
}

// E4M3 codes of a lane's 8 values scaled by 2^-(byte-127).  The power-of-two product is
// exact wherever it is a normal number; below that the code is a signed zero either way.
__device__ __forceinline__ u32x2 mx_encode8(const float f[8], uint32_t byte) {
    const float inv = e8m0_inv_scale(byte);
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        t[i] = f[i] * inv;
    return e4m3x8(t);
}

// The exact binary32 values of a lane's 8 codes under scale byte `byte`.
__device__ __forceinline__ void mx_decode8(u32x2 w, uint32_t byte, float f[8]) {
    e4m3_decode4(w.x, f);
    e4m3_decode4(w.y, f + 4);
    const float sc = e8m0_value(byte);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = f[i] * sc;
}

__device__ __forceinline__ float abs_max8(const float f[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
    return m;
}

__device__ __forceinline__ void store_e8m0_word(uint8_t* p, uint32_t word) {
    __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(p));
}

// A lane holds 16 values (Lanes16): a group of 32 is a lane pair, and the block's codes
// are one 16-byte store per lane.  WT: written through to the last-level cache (st16_wt).
template <int U, bool WT>
__global__ __launch_bounds__(kGroupThreads) void k_quant_mxf(MxfQuantArgs a) {
    const uint16_t* __restrict__ x = a.x[blockIdx.y];
    uint8_t* __restrict__ v = a.v[blockIdx.y];
    uint8_t* __restrict__ e = a.e[blockIdx.y];
    const Lanes16 L(U);
    const int64_t nt = tiles16_of(a.nb);
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks16, left = a.nb - b0;   // uniform
        u32x4 xv[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = L.blk(u) < left;
            xv[u][0] = in ? ld16(x + b0 * kBlock + L.val(u)) : u32x4{};
            xv[u][1] = in ? ld16(x + b0 * kBlock + L.val(u) + 8) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[16];
            unpack_bf16x8(xv[u][0], f);
            unpack_bf16x8(xv[u][1], f + 8);
            const float m = __builtin_fmaxf(abs_max8(f), abs_max8(f + 8));
            const uint32_t amax_bits = pair_max2(__float_as_uint(m));
            const uint32_t byte = e8m0_from_bf16_amax(amax_bits >> 16);
            const u32x2 lo = mx_encode8(f, byte), hi = mx_encode8(f + 8, byte);
            const uint32_t word = gather_e8m0_pairs(byte);
            if (L.blk(u) < left) {
                st16_out<WT>(v + b0 * kBlock + L.val(u), u32x4{lo.x, lo.y, hi.x, hi.y});
                if (L.leader) {
                    if constexpr (WT)
                        st4_wt(e + (b0 + L.blk(u)) * 4, word);
                    else
                        store_e8m0_word(e + (b0 + L.blk(u)) * 4, word);
                }
            }
        }
    }
}

template <int U, bool SkipOwn>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_mxf(MxfDequantArgs a) {
    const uint8_t* __restrict__ v = a.v[blockIdx.y];
    const uint8_t* __restrict__ e = a.e[blockIdx.y];
    uint16_t* __restrict__ y = a.y[blockIdx.y];
    const Lanes L(U);
    const int64_t nt = tiles_of(a.nb);
    const int64_t skip_lo = (int64_t)blockIdx.y * a.skip_nb, skip_hi = skip_lo + a.skip_nb;
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks, left = a.nb - b0;   // uniform
        u32x2 vv[U];
        uint32_t ev[U];
        bool in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = L.blk(u);
            in[u] = r < left && !(SkipOwn && r >= skip_lo - b0 && r < skip_hi - b0);
            vv[u] = in[u] ? ld8(v + b0 * kBlock + L.val(u)) : u32x2{};
            ev[u] = in[u] ? (uint32_t)e[(b0 + L.blk(u)) * 4 + L.grp()] : 127u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[8];
            mx_decode8(vv[u], ev[u], f);
            if (in[u])
                st16(y + b0 * kBlock + L.val(u), pack_bf16x8(f));
        }
    }
}

// v_in/v_out and e_in/e_out may be the same buffers: every lane of a block loads its
// codes and its group's byte before the block's stores, which depend on those loads,
// and no other wave touches that block.
template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_ring_hop_mx(MxfHopArgs a) {
    const uint8_t* v_in = a.v_in[blockIdx.y];
    const uint8_t* e_in = a.e_in[blockIdx.y];
    const uint16_t* __restrict__ local = a.local[blockIdx.y];
    uint8_t* v_out = a.v_out[blockIdx.y];
    uint8_t* e_out = a.e_out[blockIdx.y];
    const Lanes16 L(U);
    const uint32_t grp = L.off >> 5;          // the lane's group within its block
    const int64_t nt = tiles16_of(a.nb);
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks16, left = a.nb - b0;   // uniform
        u32x4 vv[U], lv[U][2];
        uint32_t ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = L.blk(u) < left;
            vv[u] = in ? ld16(v_in + b0 * kBlock + L.val(u)) : u32x4{};
            ev[u] = in ? (uint32_t)e_in[(b0 + L.blk(u)) * 4 + grp] : 127u;
            lv[u][0] = in ? ld16(local + b0 * kBlock + L.val(u)) : u32x4{};
            lv[u][1] = in ? ld16(local + b0 * kBlock + L.val(u) + 8) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float deq[16], loc[16], sum[16];
            mx_decode8(u32x2{vv[u].x, vv[u].y}, ev[u], deq);
            mx_decode8(u32x2{vv[u].z, vv[u].w}, ev[u], deq + 8);
            unpack_bf16x8(lv[u][0], loc);
            unpack_bf16x8(lv[u][1], loc + 8);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sum[i] = deq[i] + loc[i];
            const float m = __builtin_fmaxf(abs_max8(sum), abs_max8(sum + 8));
            const float amax = __uint_as_float(pair_max2(__float_as_uint(m)));
            const uint32_t byte = e8m0_from_f32_amax(amax);
            const u32x2 lo = mx_encode8(sum, byte), hi = mx_encode8(sum + 8, byte);
            const uint32_t word = gather_e8m0_pairs(byte);
            if (L.blk(u) < left) {
                st16(v_out + b0 * kBlock + L.val(u), u32x4{lo.x, lo.y, hi.x, hi.y});
                if (L.leader)
                    store_e8m0_word(e_out + (b0 + L.blk(u)) * 4, word);
            }
        }
    }
}

// Sources are consumed in chunks of kMxSrcChunk whose loads are all issued before the
// chunk's ordered additions.  Fused: the mx_a2a owner step -- the bf16 sum is requantized
// with the MXFP8 rule into the broadcast payload and the owner's copy is materialized from
// that payload, all while the sum is in registers.
constexpr int kMxSrcChunk = 4;

template <int U, bool Fused>
__global__ __launch_bounds__(kGroupThreads) void k_accum_mx(MxfAccumArgs a) {
    const int64_t seg_off = (int64_t)blockIdx.y * a.seg_n;
    uint16_t* __restrict__ red = a.red ? a.red + seg_off : nullptr;
    const Lanes L(U);
    const int64_t nt = tiles_of(a.nb);
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks, left = a.nb - b0;   // uniform
        const int64_t v0 = seg_off + b0 * kBlock;                   // first value of the step
        const int64_t e0 = v0 / 32;                                  // its first E8M0 byte
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[u][i] = 0.0f;
        for (int k0 = 0; k0 < a.nsrc; k0 += kMxSrcChunk) {
            u32x2 vv[kMxSrcChunk][U];
            uint32_t ev[kMxSrcChunk][U];
#pragma unroll
            for (int j = 0; j < kMxSrcChunk; ++j) {
                if (k0 + j < a.nsrc) {
                    const uint8_t* v = a.v[k0 + j] + v0;
                    const uint8_t* e = a.e[k0 + j] + e0;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = L.blk(u) < left;
                        vv[j][u] = in ? ld8(v + L.val(u)) : u32x2{};
                        ev[j][u] = in ? (uint32_t)e[L.blk(u) * 4 + L.grp()] : 127u;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kMxSrcChunk; ++j) {
                if (k0 + j < a.nsrc) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float f[8];
                        mx_decode8(vv[j][u], ev[j][u], f);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[u][i] = acc[u][i] + f[i];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = L.blk(u) < left;
            const u32x4 rb = pack_bf16x8(acc[u]);       // the owner's bf16 sum
            if constexpr (!Fused) {
                if (in)
                    st16(red + b0 * kBlock + L.val(u), rb);
            } else {
                float f[8];
                unpack_bf16x8(rb, f);
                const uint32_t amax_bits = quad_max4(__float_as_uint(abs_max8(f)));
                const uint32_t byte = e8m0_from_bf16_amax(amax_bits >> 16);
                const u32x2 codes = mx_encode8(f, byte);
                const uint32_t word = gather_e8m0(byte);
                if (in) {
                    st8(a.v_out + v0 + L.val(u), codes);
                    if (L.leader)
                        store_e8m0_word(a.e_out + e0 + L.blk(u) * 4, word);
                    if (red)
                        st16(red + b0 * kBlock + L.val(u), rb);
                    uint16_t* y = a.y[blockIdx.y];
                    if (y) {
                        float g[8];
                        mx_decode8(codes, byte, g);
                        st16(y + b0 * kBlock + L.val(u), pack_bf16x8(g));
                    }
                }
            }
        }
    }
}

constexpr int kUMxf = 2;    // dequantize, accumulate (8 values per lane)
constexpr int kUMxfQ = 1;   // quantize, ring hop (16 values per lane)

}  // namespace

hipError_t launch_quant(int count, const uint16_t* const* x, uint8_t* const* v,
                        uint8_t* const* e, int64_t n, hipStream_t stream) {
    MxfQuantArgs a{};
    for (int i = 0; i < count; ++i) {
        a.x[i] = x[i];
        a.v[i] = v[i];
        a.e[i] = e[i];
    }
    a.nb = n / kBlock;
    const dim3 grid = grid16_for<kUMxfQ>(a.nb, count);
    if ((int64_t)count * a.nb * (kBlock + 4) <= kWriteThroughBytes)
        return launch1(k_quant_mxf<kUMxfQ, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_quant_mxf<kUMxfQ, false>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_dequant(int count, const uint8_t* const* v, const uint8_t* const* e,
                          uint16_t* const* y, int64_t n, hipStream_t stream,
                          int64_t skip_shard_n) {
    MxfDequantArgs a{};
    a.skip_nb = skip_shard_n / kBlock;
    for (int i = 0; i < count; ++i) {
        a.v[i] = v[i];
        a.e[i] = e[i];
        a.y[i] = y[i];
    }
    a.nb = n / kBlock;
    const dim3 grid = grid_for<kUMxf>(a.nb, count);
    if (a.skip_nb > 0)
        return launch1(k_dequant_mxf<kUMxf, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_dequant_mxf<kUMxf, false>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_ring_hop(int count, const uint8_t* const* v_in, const uint8_t* const* e_in,
                           const uint16_t* const* local, uint8_t* const* v_out,
                           uint8_t* const* e_out, int64_t n, hipStream_t stream) {
    MxfHopArgs a{};
    for (int i = 0; i < count; ++i) {
        a.v_in[i] = v_in[i];
        a.e_in[i] = e_in[i];
        a.local[i] = local[i];
        a.v_out[i] = v_out[i];
        a.e_out[i] = e_out[i];
    }
    a.nb = n / kBlock;
    return launch1(k_ring_hop_mx<kUMxfQ>, grid16_for<kUMxfQ>(a.nb, count), dim3(kGroupThreads), stream,
                   a);
}

hipError_t launch_accum(int nsrc, const uint8_t* const* v, const uint8_t* const* e, uint16_t* y,
                        int nseg, int64_t seg_n, hipStream_t stream) {
    MxfAccumArgs a{};
    for (int i = 0; i < nsrc; ++i) {
        a.v[i] = v[i];
        a.e[i] = e[i];
    }
    a.red = y;
    a.nsrc = nsrc;
    a.nb = seg_n / kBlock;
    a.seg_n = seg_n;
    return launch1(k_accum_mx<kUMxf, false>, grid_for<kUMxf>(a.nb, nseg), dim3(kGroupThreads),
                   stream, a);
}

hipError_t launch_a2a_reduce(int nsrc, const uint8_t* const* v, const uint8_t* const* e,
                             int nseg, int64_t seg_n, uint8_t* v_out, uint8_t* e_out,
                             uint16_t* const* y, uint16_t* red, hipStream_t stream) {
    MxfAccumArgs a{};
    for (int i = 0; i < nsrc; ++i) {
        a.v[i] = v[i];
        a.e[i] = e[i];
    }
    for (int j = 0; j < nseg; ++j)
        a.y[j] = y ? y[j] : nullptr;
    a.red = red;
    a.v_out = v_out;
    a.e_out = e_out;
    a.nsrc = nsrc;
    a.nb = seg_n / kBlock;
    a.seg_n = seg_n;
    return launch1(k_accum_mx<kUMxf, true>, grid_for<kUMxf>(a.nb, nseg), dim3(kGroupThreads),
                   stream, a);
}

}  // namespace bq
