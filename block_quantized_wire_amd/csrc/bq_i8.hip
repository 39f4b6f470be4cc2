// bq_i8.hip -- block-INT8 wire codec kernels for gfx950.
//
// Definitions (pages: sparkinfer pull request #46, "feat(pcie_dma): add block-INT8 wire
// modes for AG, ring, and A2A", sections Summary and Implementation):
//   quantize      per 128-value block: scale = fl32(amax/127), q = rne(fl32(x/scale)) in
//                 [-127, 127]; an all-zero block stores scale 0 and payload 0;
//   materialize   y = bf16_rne(fl32(q * scale));
//   accumulate    y = bf16_rne(sum over sources, in order, of fl32(q_s * scale_s)), summed
//                 in binary32 starting from +0 (the all-to-all reduce);
//   ring hop      requantize fl32(fl32(q * scale) + local) block by block (one fused
//                 reduce-scatter hop; the binary32 sums are requantized directly).
//
// All kernels are HBM streaming kernels with 16-byte vectors, per-block amax through DPP
// reductions (no LDS), no atomics, and a fixed order of every floating-point operation, so
// results are deterministic and bit-reproducible.  The kernels that write the INT8 payload
// (quantize, ring hop) give a lane 16 values -- one 16-byte payload vector, two of bf16 --
// and the others give it 8 (one 16-byte bf16 vector, 8 payload bytes): each side's
// stores then cover whole contiguous 1 KB runs per wave instruction.
// Every kernel takes a batch of equal-size segments (grid.y = segment) so that one
// launch covers all simulated ranks of a collective step.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

namespace {

struct QuantArgs {
    const uint16_t* x[kMaxBatch];
    int8_t* q[kMaxBatch];
    float* s[kMaxBatch];
    int64_t nb;   // blocks per segment
};

struct DequantArgs {
    const int8_t* q[kMaxBatch];
    const float* s[kMaxBatch];
    uint16_t* y[kMaxBatch];
    int64_t nb;
    int64_t skip_nb;   // > 0: segment i leaves blocks [i*skip_nb, (i+1)*skip_nb) untouched
};

struct HopArgs {
    const int8_t* q_in[kMaxBatch];
    const float* s_in[kMaxBatch];
    const uint16_t* local[kMaxBatch];
    int8_t* q_out[kMaxBatch];
    float* s_out[kMaxBatch];
    int64_t nb;
};

struct AccumArgs {
    const int8_t* q[kMaxSrc];
    const float* s[kMaxSrc];
    uint16_t* red;            // bf16 sums, segment j at j * seg_n (fused: may be null)
    int8_t* q_out;            // fused: requantized payload, segment j at j * seg_n
    float* s_out;             // fused: its scales, segment j at j * seg_n / 128
    uint16_t* y[kMaxBatch];   // fused: the owner's materialization of segment j (or null)
    int nsrc;
    int64_t nb;               // blocks per segment
    int64_t seg_n;            // values per segment
};

// A lane holds 16 values (Lanes16): its block's payload bytes are one 16-byte store.
// WT: the payload and scales are written through to the last-level cache (see st16_wt).
template <int U, bool WT>
__global__ __launch_bounds__(kGroupThreads) void k_quant_i8(QuantArgs a) {
    const uint16_t* __restrict__ x = a.x[blockIdx.y];
    int8_t* __restrict__ q = a.q[blockIdx.y];
    float* __restrict__ s = a.s[blockIdx.y];
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
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
            const float amax = __uint_as_float(half_row_max8(__float_as_uint(m)));
            const float sc = i8_scale(amax);
            const u32x2 lo = quant_i8x8(f, sc), hi = quant_i8x8(f + 8, sc);
            if (L.blk(u) < left) {
                st16_out<WT>(q + b0 * kBlock + L.val(u), u32x4{lo.x, lo.y, hi.x, hi.y});
                if (L.leader) {
                    if constexpr (WT)
                        st4_wt(s + b0 + L.blk(u), __float_as_uint(sc));
                    else
                        s[b0 + L.blk(u)] = sc;
                }
            }
        }
    }
}

// SkipOwn: segment i leaves its own shard of blocks [i*skip_nb, (i+1)*skip_nb) untouched.
template <int U, bool SkipOwn>
__global__ __launch_bounds__(kGroupThreads) void k_dequant_i8(DequantArgs a) {
    const int8_t* __restrict__ q = a.q[blockIdx.y];
    const float* __restrict__ s = a.s[blockIdx.y];
    uint16_t* __restrict__ y = a.y[blockIdx.y];
    const Lanes L(U);
    const int64_t nt = tiles_of(a.nb);
    const int64_t skip_lo = (int64_t)blockIdx.y * a.skip_nb, skip_hi = skip_lo + a.skip_nb;
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks, left = a.nb - b0;   // uniform
        u32x2 qv[U];
        float sv[U];
        bool in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = L.blk(u);
            in[u] = r < left && !(SkipOwn && r >= skip_lo - b0 && r < skip_hi - b0);
            qv[u] = in[u] ? ld8(q + b0 * kBlock + L.val(u)) : u32x2{};
            sv[u] = in[u] ? s[b0 + L.blk(u)] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[8];
            dequant_i8x8(qv[u], sv[u], f);
            if (in[u])
                st16(y + b0 * kBlock + L.val(u), pack_bf16x8(f));
        }
    }
}

// q_in/q_out and s_in/s_out may be the same buffers: the lanes of a block load all of
// it before any of its stores, and no other wave touches that block.
template <int U>
__global__ __launch_bounds__(kGroupThreads) void k_ring_hop_i8(HopArgs a) {
    const int8_t* q_in = a.q_in[blockIdx.y];
    const float* s_in = a.s_in[blockIdx.y];
    const uint16_t* __restrict__ local = a.local[blockIdx.y];
    int8_t* q_out = a.q_out[blockIdx.y];
    float* s_out = a.s_out[blockIdx.y];
    const Lanes16 L(U);
    const int64_t nt = tiles16_of(a.nb);
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks16, left = a.nb - b0;   // uniform
        u32x4 qv[U], lv[U][2];
        float sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = L.blk(u) < left;
            qv[u] = in ? ld16(q_in + b0 * kBlock + L.val(u)) : u32x4{};
            sv[u] = in ? s_in[b0 + L.blk(u)] : 0.0f;
            lv[u][0] = in ? ld16(local + b0 * kBlock + L.val(u)) : u32x4{};
            lv[u][1] = in ? ld16(local + b0 * kBlock + L.val(u) + 8) : u32x4{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float deq[16], loc[16], sum[16];
            dequant_i8x8(u32x2{qv[u].x, qv[u].y}, sv[u], deq);      // rounded products ...
            dequant_i8x8(u32x2{qv[u].z, qv[u].w}, sv[u], deq + 8);
            unpack_bf16x8(lv[u][0], loc);
            unpack_bf16x8(lv[u][1], loc + 8);
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sum[i] = deq[i] + loc[i];                            // ... then rounded adds
                m = __builtin_fmaxf(m, __builtin_fabsf(sum[i]));
            }
            const float amax = __uint_as_float(half_row_max8(__float_as_uint(m)));
            const float sc = i8_scale(amax);
            const u32x2 lo = quant_i8x8(sum, sc), hi = quant_i8x8(sum + 8, sc);
            if (L.blk(u) < left) {
                st16(q_out + b0 * kBlock + L.val(u), u32x4{lo.x, lo.y, hi.x, hi.y});
                if (L.leader)
                    s_out[b0 + L.blk(u)] = sc;
            }
        }
    }
}

// Sources are consumed in chunks of kSrcChunk whose loads are all issued before the
// chunk's ordered additions, so that many independent streams are in flight per lane.
// Fused: the owner step of the all-to-all -- the bf16 sum is requantized with the
// block-INT8 rule into the broadcast payload, and the owner's copy is materialized
// from that payload, all while the sum is in registers.
constexpr int kSrcChunk = 4;
template <int U, bool Fused>
__global__ __launch_bounds__(kGroupThreads) void k_accum_i8(AccumArgs a) {
    const int64_t seg_off = (int64_t)blockIdx.y * a.seg_n;
    const int64_t seg_sb = seg_off / kBlock;
    uint16_t* __restrict__ red = a.red ? a.red + seg_off : nullptr;
    const Lanes L(U);
    const int64_t nt = tiles_of(a.nb);
    for (int64_t t0 = L.first; t0 < nt; t0 += L.step) {
        const int64_t b0 = t0 * kTileBlocks, left = a.nb - b0;   // uniform
        const int64_t v0 = seg_off + b0 * kBlock, sb0 = seg_sb + b0;
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[u][i] = 0.0f;
        for (int k0 = 0; k0 < a.nsrc; k0 += kSrcChunk) {
            u32x2 qv[kSrcChunk][U];
            float sv[kSrcChunk][U];
#pragma unroll
            for (int j = 0; j < kSrcChunk; ++j) {
                if (k0 + j < a.nsrc) {
                    const int8_t* q = a.q[k0 + j] + v0;
                    const float* s = a.s[k0 + j] + sb0;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = L.blk(u) < left;
                        qv[j][u] = in ? ld8(q + L.val(u)) : u32x2{};
                        sv[j][u] = in ? s[L.blk(u)] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kSrcChunk; ++j) {
                if (k0 + j < a.nsrc) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float f[8];
                        dequant_i8x8(qv[j][u], sv[j][u], f);
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
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
                const float amax = __uint_as_float(row_max16(__float_as_uint(m)));
                const float sc = i8_scale(amax);
                const u32x2 qv = quant_i8x8(f, sc);
                if (in) {
                    st8(a.q_out + v0 + L.val(u), qv);
                    if (L.leader)
                        a.s_out[sb0 + L.blk(u)] = sc;
                    if (red)
                        st16(red + b0 * kBlock + L.val(u), rb);
                    uint16_t* y = a.y[blockIdx.y];
                    if (y) {
                        float g[8];
                        dequant_i8x8(qv, sc, g);
                        st16(y + b0 * kBlock + L.val(u), pack_bf16x8(g));
                    }
                }
            }
        }
    }
}

constexpr int kUQuant = 1;
constexpr int kUDequant = 2;
constexpr int kUHop = 1;
constexpr int kUAccum = 2;

}  // namespace

hipError_t launch_quant(int count, const uint16_t* const* x, int8_t* const* q,
                           float* const* s, int64_t n, hipStream_t stream) {
    QuantArgs a{};
    for (int i = 0; i < count; ++i) {
        a.x[i] = x[i];
        a.q[i] = q[i];
        a.s[i] = s[i];
    }
    a.nb = n / kBlock;
    const dim3 grid = grid16_for<kUQuant>(a.nb, count);
    if ((int64_t)count * a.nb * (kBlock + 4) <= kWriteThroughBytes)
        return launch1(k_quant_i8<kUQuant, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_quant_i8<kUQuant, false>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_dequant(int count, const int8_t* const* q, const float* const* s,
                             uint16_t* const* y, int64_t n, hipStream_t stream,
                             int64_t skip_shard_n) {
    DequantArgs a{};
    a.skip_nb = skip_shard_n / kBlock;
    for (int i = 0; i < count; ++i) {
        a.q[i] = q[i];
        a.s[i] = s[i];
        a.y[i] = y[i];
    }
    a.nb = n / kBlock;
    const dim3 grid = grid_for<kUDequant>(a.nb, count);
    if (a.skip_nb > 0)
        return launch1(k_dequant_i8<kUDequant, true>, grid, dim3(kGroupThreads), stream, a);
    return launch1(k_dequant_i8<kUDequant, false>, grid, dim3(kGroupThreads), stream, a);
}

hipError_t launch_ring_hop(int count, const int8_t* const* q_in, const float* const* s_in,
                              const uint16_t* const* local, int8_t* const* q_out,
                              float* const* s_out, int64_t n, hipStream_t stream) {
    HopArgs a{};
    for (int i = 0; i < count; ++i) {
        a.q_in[i] = q_in[i];
        a.s_in[i] = s_in[i];
        a.local[i] = local[i];
        a.q_out[i] = q_out[i];
        a.s_out[i] = s_out[i];
    }
    a.nb = n / kBlock;
    return launch1(k_ring_hop_i8<kUHop>, grid16_for<kUHop>(a.nb, count), dim3(kGroupThreads), stream, a);
}

hipError_t launch_accum(int nsrc, const int8_t* const* q, const float* const* s,
                           uint16_t* y, int nseg, int64_t seg_n, hipStream_t stream) {
    AccumArgs a{};
    for (int i = 0; i < nsrc; ++i) {
        a.q[i] = q[i];
        a.s[i] = s[i];
    }
    a.red = y;
    a.nsrc = nsrc;
    a.nb = seg_n / kBlock;
    a.seg_n = seg_n;
    return launch1(k_accum_i8<kUAccum, false>, grid_for<kUAccum>(a.nb, nseg),
                   dim3(kGroupThreads), stream, a);
}

hipError_t launch_a2a_reduce(int nsrc, const int8_t* const* q, const float* const* s,
                                int nseg, int64_t seg_n, int8_t* q_out, float* s_out,
                                uint16_t* const* y, uint16_t* red, hipStream_t stream) {
    AccumArgs a{};
    for (int i = 0; i < nsrc; ++i) {
        a.q[i] = q[i];
        a.s[i] = s[i];
    }
    for (int j = 0; j < nseg; ++j)
        a.y[j] = y ? y[j] : nullptr;
    a.red = red;
    a.q_out = q_out;
    a.s_out = s_out;
    a.nsrc = nsrc;
    a.nb = seg_n / kBlock;
    a.seg_n = seg_n;
    return launch1(k_accum_i8<kUAccum, true>, grid_for<kUAccum>(a.nb, nseg),
                   dim3(kGroupThreads), stream, a);
}

}  // namespace bq
