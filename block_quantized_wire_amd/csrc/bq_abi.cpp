// bq_abi.cpp -- the C ABI of libblockq: argument validation and kernel launches.
//
// Every entry point validates all of its arguments on the host before it launches
// anything (caller-owned staging whose bad shapes, layouts or capacity fail before a
// kernel runs: b12x pull request #241, "[II] Support staged MXFP8 linear inputs",
// Compatibility).  The library allocates nothing, keeps no state and never
// synchronizes, so every call may be captured in a HIP graph.
#include "blockq.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "bq_launch.h"

namespace {

constexpr int64_t kBlk = BQ_BLOCK;

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + (uintptr_t)bytes};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }
bool same(Span a, Span b) { return a.lo == b.lo && a.hi == b.hi; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bq_status launched(hipError_t e) { return e == hipSuccess ? BQ_OK : BQ_ERR_LAUNCH; }

// n must be a non-negative multiple of 128 (and fit the kernels' 32-bit grid).
bq_status check_n(int64_t n) {
    if (n < 0 || n % kBlk != 0 || n / kBlk >= ((int64_t)1 << 36))
        return BQ_ERR_SIZE;
    return BQ_OK;
}

// One segment of block-INT8 (or E4M3) data: bf16 values, payload bytes, scales.
bq_status check_bf16(const void* p) {
    if (!p)
        return BQ_ERR_NULL;
    return aligned(p, 16) ? BQ_OK : BQ_ERR_ALIGN;
}
bq_status check_payload(const void* p) { return check_bf16(p); }
bq_status check_scales(const void* p) {
    if (!p)
        return BQ_ERR_NULL;
    return aligned(p, 4) ? BQ_OK : BQ_ERR_ALIGN;
}

#define BQ_TRY(expr)                  \
    do {                              \
        const bq_status st_ = (expr); \
        if (st_ != BQ_OK)             \
            return st_;               \
    } while (0)

bool any_overlap(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j]))
                return true;
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return true;
    }
    return false;
}

// Largest number of spans any entry point checks at once (a2a: 4W+3 outputs, W inputs).
constexpr int kMaxSpans = 4 * BQ_MAX_BATCH + 4;

// ---- flat block formats on the wire ----------------------------------------------------
//
// Block INT8 and flat MXFP8 share one wire layout: n payload bytes (int8_t or uint8_t E4M3)
// and 4 scale bytes per 128-value block (one float, or four E8M0 bytes), 16- and 4-byte
// aligned.  The validation and the collective schedules below are therefore written once
// over the payload type P and scale type S; the launchers are overloaded per codec.

template <typename P, typename S>
bq_status quant_batch(int count, const uint16_t* const* x, int64_t n, P* const* q, S* const* s,
                      void* stream) {
    if (count < 1 || count > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n == 0)
        return BQ_OK;
    if (!x || !q || !s)
        return BQ_ERR_NULL;
    Span outs[2 * BQ_MAX_BATCH], ins[BQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        BQ_TRY(check_bf16(x[i]));
        BQ_TRY(check_payload(q[i]));
        BQ_TRY(check_scales(s[i]));
        ins[i] = span(x[i], 2 * n);
        outs[2 * i] = span(q[i], n);
        outs[2 * i + 1] = span(s[i], 4 * (n / kBlk));
    }
    if (any_overlap(outs, 2 * count, ins, count))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_quant(count, x, q, s, n, as_stream(stream)));
}

template <typename P, typename S>
bq_status dequant_batch(int count, const P* const* q, const S* const* s, int64_t n,
                        uint16_t* const* y, void* stream) {
    if (count < 1 || count > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n == 0)
        return BQ_OK;
    if (!q || !s || !y)
        return BQ_ERR_NULL;
    Span outs[BQ_MAX_BATCH], ins[2 * BQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        BQ_TRY(check_payload(q[i]));
        BQ_TRY(check_scales(s[i]));
        BQ_TRY(check_bf16(y[i]));
        ins[2 * i] = span(q[i], n);
        ins[2 * i + 1] = span(s[i], 4 * (n / kBlk));
        outs[i] = span(y[i], 2 * n);
    }
    if (any_overlap(outs, count, ins, 2 * count))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_dequant(count, q, s, y, n, as_stream(stream)));
}

template <typename P, typename S>
bq_status ring_hop_batch(int count, const P* const* q_in, const S* const* s_in,
                         const uint16_t* const* local, int64_t n, P* const* q_out,
                         S* const* s_out, void* stream) {
    if (count < 1 || count > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n == 0)
        return BQ_OK;
    if (!q_in || !s_in || !local || !q_out || !s_out)
        return BQ_ERR_NULL;
    const int64_t sb = 4 * (n / kBlk);
    Span outs[2 * BQ_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        BQ_TRY(check_payload(q_in[i]));
        BQ_TRY(check_scales(s_in[i]));
        BQ_TRY(check_bf16(local[i]));
        BQ_TRY(check_payload(q_out[i]));
        BQ_TRY(check_scales(s_out[i]));
        outs[2 * i] = span(q_out[i], n);
        outs[2 * i + 1] = span(s_out[i], sb);
    }
    // outputs: no overlap among themselves, none with any local partial; an output
    // may coincide exactly with its own segment's input (in place), nothing else.
    for (int i = 0; i < count; ++i) {
        const Span qo = outs[2 * i], so = outs[2 * i + 1];
        const Span qi = span(q_in[i], n), si = span(s_in[i], sb);
        const bool inplace_q = same(qo, qi), inplace_s = same(so, si);
        if (inplace_q != inplace_s)
            return BQ_ERR_ALIAS;
        for (int j = 0; j < 2 * count; ++j)
            if (j != 2 * i && j != 2 * i + 1 &&
                (overlaps(qo, outs[j]) || overlaps(so, outs[j])))
                return BQ_ERR_ALIAS;
        for (int j = 0; j < count; ++j) {
            const Span lj = span(local[j], 2 * n);
            if (overlaps(qo, lj) || overlaps(so, lj))
                return BQ_ERR_ALIAS;
            const Span qj = span(q_in[j], n), sj = span(s_in[j], sb);
            const bool own = (j == i);
            if (overlaps(qo, qj) && !(own && inplace_q))
                return BQ_ERR_ALIAS;
            if (overlaps(so, sj) && !(own && inplace_s))
                return BQ_ERR_ALIAS;
            if (overlaps(qo, sj) || overlaps(so, qj))
                return BQ_ERR_ALIAS;
        }
    }
    return launched(
        bq::launch_ring_hop(count, q_in, s_in, local, q_out, s_out, n, as_stream(stream)));
}

template <typename P, typename S>
bq_status accum_batch(int nseg, int nsrc, const P* const* q_srcs, const S* const* s_srcs,
                      int64_t seg_n, uint16_t* y, void* stream) {
    if (nsrc < 1 || nsrc > BQ_MAX_SRC || nseg < 1 || nseg > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(seg_n));
    if (seg_n == 0)
        return BQ_OK;
    if (!q_srcs || !s_srcs)
        return BQ_ERR_NULL;
    BQ_TRY(check_bf16(y));
    const int64_t n = seg_n * nseg;
    const Span ys = span(y, 2 * n);
    for (int i = 0; i < nsrc; ++i) {
        BQ_TRY(check_payload(q_srcs[i]));
        BQ_TRY(check_scales(s_srcs[i]));
        if (overlaps(ys, span(q_srcs[i], n)) || overlaps(ys, span(s_srcs[i], 4 * (n / kBlk))))
            return BQ_ERR_ALIAS;
    }
    return launched(bq::launch_accum(nsrc, q_srcs, s_srcs, y, nseg, seg_n, as_stream(stream)));
}

template <typename P, typename S>
bq_status a2a_reduce(int nseg, int nsrc, const P* const* q_srcs, const S* const* s_srcs,
                     int64_t seg_n, P* q_out, S* s_out, uint16_t* const* y_out, uint16_t* red,
                     void* stream) {
    if (nsrc < 1 || nsrc > BQ_MAX_SRC || nseg < 1 || nseg > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(seg_n));
    if (seg_n == 0)
        return BQ_OK;
    if (!q_srcs || !s_srcs)
        return BQ_ERR_NULL;
    const int64_t n = seg_n * nseg, sb = 4 * (n / kBlk);
    BQ_TRY(check_payload(q_out));
    BQ_TRY(check_scales(s_out));
    Span outs[BQ_MAX_BATCH + 3];
    int no = 0;
    outs[no++] = span(q_out, n);
    outs[no++] = span(s_out, sb);
    if (red) {
        BQ_TRY(check_bf16(red));
        outs[no++] = span(red, 2 * n);
    }
    if (y_out) {
        for (int j = 0; j < nseg; ++j) {
            BQ_TRY(check_bf16(y_out[j]));
            outs[no++] = span(y_out[j], 2 * seg_n);
        }
    }
    Span ins[2 * BQ_MAX_SRC];
    for (int k = 0; k < nsrc; ++k) {
        BQ_TRY(check_payload(q_srcs[k]));
        BQ_TRY(check_scales(s_srcs[k]));
        ins[2 * k] = span(q_srcs[k], n);
        ins[2 * k + 1] = span(s_srcs[k], sb);
    }
    if (any_overlap(outs, no, ins, 2 * nsrc))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_a2a_reduce(nsrc, q_srcs, s_srcs, nseg, seg_n, q_out, s_out, y_out,
                                          red, as_stream(stream)));
}

template <typename P, typename S>
bq_status allgather_dequant(int world, const P* q, const S* s, int64_t n, uint16_t* const* out,
                            int skip_own, void* stream) {
    const int W = world;
    if (W < 1 || W > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n % (kBlk * W) != 0)
        return BQ_ERR_SIZE;
    if (n == 0)
        return BQ_OK;
    if (!out)
        return BQ_ERR_NULL;
    BQ_TRY(check_payload(q));
    BQ_TRY(check_scales(s));
    Span outs[BQ_MAX_BATCH], ins[2] = {span(q, n), span(s, 4 * (n / kBlk))};
    for (int r = 0; r < W; ++r) {
        BQ_TRY(check_bf16(out[r]));
        outs[r] = span(out[r], 2 * n);
    }
    if (any_overlap(outs, W, ins, 2))
        return BQ_ERR_ALIAS;
    const P* qi[BQ_MAX_BATCH];
    const S* si[BQ_MAX_BATCH];
    for (int r = 0; r < W; ++r) {
        qi[r] = q;
        si[r] = s;
    }
    return launched(bq::launch_dequant(W, qi, si, out, n, as_stream(stream), skip_own ? n / W : 0));
}

// The ring all-reduce (P1 Summary; P2 Modes for the MXFP8 codec).  Chunk c of n/W values
// is quantized at step 0 by rank c+1, folded in by one hop per later step, and every rank
// materializes every chunk from its final payload.  Scale arrays hold 4 bytes per block,
// so a chunk's scales start at byte 4 * (c*n/W)/128 for either codec.
template <typename P, typename S>
bq_status ring_allreduce(int world, int64_t n, const uint16_t* const* partials, P* q_wire,
                         S* s_wire, uint16_t* const* out, void* stream) {
    const int W = world;
    if (W < 1 || W > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n % (kBlk * W) != 0)
        return BQ_ERR_SIZE;
    if (n == 0)
        return BQ_OK;
    if (!partials || !out)
        return BQ_ERR_NULL;
    BQ_TRY(check_payload(q_wire));
    BQ_TRY(check_scales(s_wire));
    Span outs[BQ_MAX_BATCH + 2], ins[BQ_MAX_BATCH];
    for (int r = 0; r < W; ++r) {
        BQ_TRY(check_bf16(partials[r]));
        BQ_TRY(check_bf16(out[r]));
        ins[r] = span(partials[r], 2 * n);
        outs[r] = span(out[r], 2 * n);
    }
    outs[W] = span(q_wire, n);
    outs[W + 1] = span(s_wire, 4 * (n / kBlk));
    if (any_overlap(outs, W + 2, ins, W))
        return BQ_ERR_ALIAS;

    const hipStream_t st = as_stream(stream);
    const int64_t m = n / W;
    const int64_t ms = (m / kBlk) * 4 / (int64_t)sizeof(S);   // scale elements per chunk
    const uint16_t* x[BQ_MAX_BATCH];
    const P* qi[BQ_MAX_BATCH];
    const S* si[BQ_MAX_BATCH];
    P* qo[BQ_MAX_BATCH];
    S* so[BQ_MAX_BATCH];
    // step 0: rank r quantizes its partial of chunk (r-1) mod W
    for (int r = 0; r < W; ++r) {
        const int c = (r - 1 + W) % W;
        x[r] = partials[r] + c * m;
        qo[r] = q_wire + c * m;
        so[r] = s_wire + c * ms;
    }
    bq_status stt = launched(bq::launch_quant(W, x, qo, so, m, st));
    // steps 1..W-1: rank r folds its partial of chunk (r-1-k) mod W into that payload
    for (int k = 1; k < W && stt == BQ_OK; ++k) {
        for (int r = 0; r < W; ++r) {
            const int c = ((r - 1 - k) % W + W) % W;
            x[r] = partials[r] + c * m;
            qi[r] = qo[r] = q_wire + c * m;
            si[r] = so[r] = s_wire + c * ms;
        }
        stt = launched(bq::launch_ring_hop(W, qi, si, x, qo, so, m, st));
    }
    // all-gather: every rank materializes every chunk from the same final payloads
    if (stt == BQ_OK) {
        for (int r = 0; r < W; ++r) {
            qi[r] = q_wire;
            si[r] = s_wire;
        }
        stt = launched(bq::launch_dequant(W, qi, si, out, n, st));
    }
    return stt;
}

// The quantize-once all-to-all (P1 Summary, Implementation; P2 Modes for MXFP8).
template <typename P, typename S>
bq_status a2a_allreduce(int world, int64_t n, const uint16_t* const* partials, P* const* q_send,
                        S* const* s_send, uint16_t* red, P* q_bcast, S* s_bcast,
                        uint16_t* const* out, void* stream) {
    const int W = world;
    if (W < 1 || W > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    BQ_TRY(check_n(n));
    if (n % (kBlk * W) != 0)
        return BQ_ERR_SIZE;
    if (n == 0)
        return BQ_OK;
    if (!partials || !q_send || !s_send || !out)
        return BQ_ERR_NULL;
    if (red)
        BQ_TRY(check_bf16(red));
    BQ_TRY(check_payload(q_bcast));
    BQ_TRY(check_scales(s_bcast));
    const int64_t sb = 4 * (n / kBlk);
    Span outs[kMaxSpans], ins[BQ_MAX_BATCH];
    int no = 0;
    for (int r = 0; r < W; ++r) {
        BQ_TRY(check_bf16(partials[r]));
        BQ_TRY(check_payload(q_send[r]));
        BQ_TRY(check_scales(s_send[r]));
        BQ_TRY(check_bf16(out[r]));
        ins[r] = span(partials[r], 2 * n);
        outs[no++] = span(q_send[r], n);
        outs[no++] = span(s_send[r], sb);
        outs[no++] = span(out[r], 2 * n);
    }
    if (red)
        outs[no++] = span(red, 2 * n);
    outs[no++] = span(q_bcast, n);
    outs[no++] = span(s_bcast, sb);
    if (any_overlap(outs, no, ins, W))
        return BQ_ERR_ALIAS;

    const hipStream_t st = as_stream(stream);
    const int64_t m = n / W;
    // quantize every partial once
    bq_status stt = launched(bq::launch_quant(W, partials, q_send, s_send, n, st));
    // owner j accumulates shard j of every payload in rank order, requantizes its bf16
    // sum once into the broadcast payload and materializes its own shard from it
    uint16_t* own[BQ_MAX_BATCH];
    for (int j = 0; j < W; ++j)
        own[j] = out[j] + j * m;
    if (stt == BQ_OK)
        stt = launched(bq::launch_a2a_reduce(W, q_send, s_send, W, m, q_bcast, s_bcast, own, red,
                                             st));
    // every rank materializes the other owners' shards from the broadcast payload
    if (stt == BQ_OK && W > 1) {
        const P* qi[BQ_MAX_BATCH];
        const S* si[BQ_MAX_BATCH];
        for (int r = 0; r < W; ++r) {
            qi[r] = q_bcast;
            si[r] = s_bcast;
        }
        stt = launched(bq::launch_dequant(W, qi, si, out, n, st, m));
    }
    return stt;
}

}  // namespace

extern "C" {

const char* bq_status_str(bq_status s) {
    switch (s) {
    case BQ_OK: return "ok";
    case BQ_ERR_NULL: return "a required pointer is NULL";
    case BQ_ERR_SIZE: return "a count or shape is negative or not a multiple of its block";
    case BQ_ERR_ALIGN: return "a pointer or leading dimension breaks the alignment rules";
    case BQ_ERR_BOUNDS: return "a leading dimension, offset or capacity does not fit";
    case BQ_ERR_NSRC: return "a source, rank or segment count is out of range";
    case BQ_ERR_ALIAS: return "an output overlaps an input or another output";
    case BQ_ERR_LAUNCH: return "the HIP kernel launch failed";
    case BQ_ERR_SCRATCH:
        return "the call needs more than the allocation-free entry point's scratch array";
    }
    return "unknown status";
}

const char* bq_version(void) { return "libblockq 0.1 (gfx950)"; }

int64_t bq_wire_bytes_b128(int64_t n) {
    if (n < 0 || n % kBlk != 0)
        return -1;
    return (n / kBlk) * 132;
}

bq_status bq_mx_staging_bytes(int64_t capacity_rows, int64_t total_cols, int64_t* value_bytes,
                              int64_t* scale_bytes) {
    if (!value_bytes || !scale_bytes)
        return BQ_ERR_NULL;
    if (capacity_rows < 0 || total_cols < 0 || total_cols % kBlk != 0)
        return BQ_ERR_SIZE;
    *value_bytes = capacity_rows * total_cols;
    *scale_bytes = capacity_rows * (total_cols / BQ_MX_GROUP);
    return BQ_OK;
}

// ---- block INT8 ----------------------------------------------------------------------

bq_status bq_quant_i8_batch(int count, const uint16_t* const* x, int64_t n, int8_t* const* q,
                            float* const* scale, void* stream) {
    return quant_batch(count, x, n, q, scale, stream);
}

bq_status bq_quant_i8(const uint16_t* x, int64_t n, int8_t* q, float* scale, void* stream) {
    return quant_batch(1, &x, n, &q, &scale, stream);
}

bq_status bq_dequant_i8_batch(int count, const int8_t* const* q, const float* const* scale,
                              int64_t n, uint16_t* const* y, void* stream) {
    return dequant_batch(count, q, scale, n, y, stream);
}

bq_status bq_dequant_i8(const int8_t* q, const float* scale, int64_t n, uint16_t* y,
                        void* stream) {
    return dequant_batch(1, &q, &scale, n, &y, stream);
}

bq_status bq_ring_hop_i8_batch(int count, const int8_t* const* q_in, const float* const* s_in,
                               const uint16_t* const* local, int64_t n, int8_t* const* q_out,
                               float* const* s_out, void* stream) {
    return ring_hop_batch(count, q_in, s_in, local, n, q_out, s_out, stream);
}

bq_status bq_ring_hop_i8(const int8_t* q_in, const float* s_in, const uint16_t* local,
                         int64_t n, int8_t* q_out, float* s_out, void* stream) {
    return ring_hop_batch(1, &q_in, &s_in, &local, n, &q_out, &s_out, stream);
}

bq_status bq_dequant_accum_i8_batch(int nseg, int nsrc, const int8_t* const* q_srcs,
                                    const float* const* s_srcs, int64_t seg_n, uint16_t* y,
                                    void* stream) {
    return accum_batch(nseg, nsrc, q_srcs, s_srcs, seg_n, y, stream);
}

bq_status bq_dequant_accum_i8(int nsrc, const int8_t* const* q_srcs, const float* const* s_srcs,
                              int64_t n, uint16_t* y, void* stream) {
    return accum_batch(1, nsrc, q_srcs, s_srcs, n, y, stream);
}

bq_status bq_a2a_reduce_i8(int nseg, int nsrc, const int8_t* const* q_srcs,
                           const float* const* s_srcs, int64_t seg_n, int8_t* q_out,
                           float* s_out, uint16_t* const* y_out, uint16_t* red, void* stream) {
    return a2a_reduce(nseg, nsrc, q_srcs, s_srcs, seg_n, q_out, s_out, y_out, red, stream);
}

bq_status bq_allgather_dequant_i8(int world, const int8_t* q, const float* s, int64_t n,
                                  uint16_t* const* out, int skip_own, void* stream) {
    return allgather_dequant(world, q, s, n, out, skip_own, stream);
}

bq_status bq_ring_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                               int8_t* q_wire, float* s_wire, uint16_t* const* out,
                               void* stream) {
    return ring_allreduce(world, n, partials, q_wire, s_wire, out, stream);
}

bq_status bq_a2a_allreduce_i8(int world, int64_t n, const uint16_t* const* partials,
                              int8_t* const* q_send, float* const* s_send, uint16_t* red,
                              int8_t* q_bcast, float* s_bcast, uint16_t* const* out,
                              void* stream) {
    return a2a_allreduce(world, n, partials, q_send, s_send, red, q_bcast, s_bcast, out, stream);
}

// ---- flat MXFP8 on the collective topologies ---------------------------------------------

bq_status bq_quant_mx_batch(int count, const uint16_t* const* x, int64_t n, uint8_t* const* v,
                            uint8_t* const* e8m0, void* stream) {
    return quant_batch(count, x, n, v, e8m0, stream);
}

bq_status bq_dequant_mx_batch(int count, const uint8_t* const* v, const uint8_t* const* e8m0,
                              int64_t n, uint16_t* const* y, void* stream) {
    return dequant_batch(count, v, e8m0, n, y, stream);
}

bq_status bq_ring_hop_mx_batch(int count, const uint8_t* const* v_in,
                               const uint8_t* const* e_in, const uint16_t* const* local,
                               int64_t n, uint8_t* const* v_out, uint8_t* const* e_out,
                               void* stream) {
    return ring_hop_batch(count, v_in, e_in, local, n, v_out, e_out, stream);
}

bq_status bq_ring_hop_mx(const uint8_t* v_in, const uint8_t* e_in, const uint16_t* local,
                         int64_t n, uint8_t* v_out, uint8_t* e_out, void* stream) {
    return ring_hop_batch(1, &v_in, &e_in, &local, n, &v_out, &e_out, stream);
}

bq_status bq_dequant_accum_mx(int nsrc, const uint8_t* const* v_srcs,
                              const uint8_t* const* e_srcs, int64_t n, uint16_t* y,
                              void* stream) {
    return accum_batch(1, nsrc, v_srcs, e_srcs, n, y, stream);
}

bq_status bq_a2a_reduce_mx(int nseg, int nsrc, const uint8_t* const* v_srcs,
                           const uint8_t* const* e_srcs, int64_t seg_n, uint8_t* v_out,
                           uint8_t* e_out, uint16_t* const* y_out, uint16_t* red, void* stream) {
    return a2a_reduce(nseg, nsrc, v_srcs, e_srcs, seg_n, v_out, e_out, y_out, red, stream);
}

bq_status bq_allgather_dequant_mx(int world, const uint8_t* v, const uint8_t* e8m0, int64_t n,
                                  uint16_t* const* out, int skip_own, void* stream) {
    return allgather_dequant(world, v, e8m0, n, out, skip_own, stream);
}

bq_status bq_ring_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                               uint8_t* v_wire, uint8_t* e_wire, uint16_t* const* out,
                               void* stream) {
    return ring_allreduce(world, n, partials, v_wire, e_wire, out, stream);
}

bq_status bq_a2a_allreduce_mx(int world, int64_t n, const uint16_t* const* partials,
                              uint8_t* const* v_send, uint8_t* const* e_send, uint16_t* red,
                              uint8_t* v_bcast, uint8_t* e_bcast, uint16_t* const* out,
                              void* stream) {
    return a2a_allreduce(world, n, partials, v_send, e_send, red, v_bcast, e_bcast, out, stream);
}

// ---- MXFP8 --------------------------------------------------------------------------------

namespace {

// rows x cols bf16 matrix with row stride ld (elements), 16-byte aligned rows.
bq_status check_mx_shape(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0 || cols % kBlk != 0)
        return BQ_ERR_SIZE;
    if (cols > 0 && rows > (((int64_t)1 << 31) - 1) / (cols / kBlk))
        return BQ_ERR_SIZE;
    return BQ_OK;
}

int64_t extent(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    return rows == 0 ? 0 : ((rows - 1) * ld + cols) * elem;
}

// A 2-D operand may span at most 2^48 bytes, far beyond any device's memory, so that extent()
// above and the kernels' 64-bit row * ld products cannot overflow.  Checked without overflow
// for rows, cols >= 0 and cols <= ld.
constexpr int64_t kMaxExtentBytes = (int64_t)1 << 48;
bool extent_fits(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    const int64_t lim = kMaxExtentBytes / elem;
    if (rows == 0)
        return true;
    if (ld > lim)
        return false;
    return rows == 1 || ld <= (lim - cols) / (rows - 1);
}

}  // namespace

namespace {

bq_status quant_mx_2d(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* v,
                      int64_t ldv, uint8_t* e8m0, int64_t lds, bool f16, void* stream) {
    BQ_TRY(check_mx_shape(rows, cols));
    if (rows == 0 || cols == 0)
        return BQ_OK;
    if (!x || !v || !e8m0)
        return BQ_ERR_NULL;
    if (ldx < cols || ldv < cols || lds < cols / BQ_MX_GROUP)
        return BQ_ERR_BOUNDS;
    if (!extent_fits(rows, cols, ldx, 2) || !extent_fits(rows, cols, ldv, 1) ||
        !extent_fits(rows, cols / BQ_MX_GROUP, lds, 1))
        return BQ_ERR_BOUNDS;
    if (!aligned(x, 16) || !aligned(v, 16) || !aligned(e8m0, 4) || ldx % 8 != 0 ||
        ldv % 16 != 0 || lds % 4 != 0)
        return BQ_ERR_ALIGN;
    const Span xs = span(x, extent(rows, cols, ldx, 2));
    const Span vs = span(v, extent(rows, cols, ldv, 1));
    const Span es = span(e8m0, extent(rows, cols / BQ_MX_GROUP, lds, 1));
    if (overlaps(xs, vs) || overlaps(xs, es) || overlaps(vs, es))
        return BQ_ERR_ALIAS;
    return launched(
        bq::launch_quant_mx(x, rows, cols, ldx, v, ldv, e8m0, lds, as_stream(stream), f16));
}

bq_status quant_mx_slice(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds,
                         int64_t capacity_rows, bool f16, void* stream) {
    BQ_TRY(check_mx_shape(rows, cols));
    if (col_off < 0 || col_off % kBlk != 0 || ldv < 0 || ldv % kBlk != 0)
        return BQ_ERR_SIZE;
    if (col_off > ldv || cols > ldv - col_off || lds < ldv / BQ_MX_GROUP || rows > capacity_rows)
        return BQ_ERR_BOUNDS;
    if (rows == 0 || cols == 0)
        return BQ_OK;
    if (!x || !v || !e8m0)
        return BQ_ERR_NULL;
    return quant_mx_2d(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / BQ_MX_GROUP, lds,
                       f16, stream);
}

}  // namespace

bq_status bq_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* v,
                      int64_t ldv, uint8_t* e8m0, int64_t lds, void* stream) {
    return quant_mx_2d(x, rows, cols, ldx, v, ldv, e8m0, lds, false, stream);
}

bq_status bq_quant_mx_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds, void* stream) {
    return quant_mx_2d(x, rows, cols, ldx, v, ldv, e8m0, lds, true, stream);
}

bq_status bq_quant_mx_slice(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                            int64_t lds, int64_t capacity_rows, void* stream) {
    return quant_mx_slice(x, rows, cols, ldx, col_off, v, ldv, e8m0, lds, capacity_rows, false,
                          stream);
}

bq_status bq_quant_mx_slice_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                int64_t col_off, uint8_t* v, int64_t ldv, uint8_t* e8m0,
                                int64_t lds, int64_t capacity_rows, void* stream) {
    return quant_mx_slice(x, rows, cols, ldx, col_off, v, ldv, e8m0, lds, capacity_rows, true,
                          stream);
}

bq_status bq_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                        int64_t rows, int64_t cols, uint16_t* y, int64_t ldy, void* stream) {
    BQ_TRY(check_mx_shape(rows, cols));
    if (rows == 0 || cols == 0)
        return BQ_OK;
    if (!v || !e8m0 || !y)
        return BQ_ERR_NULL;
    if (ldy < cols || ldv < cols || lds < cols / BQ_MX_GROUP)
        return BQ_ERR_BOUNDS;
    if (!extent_fits(rows, cols, ldy, 2) || !extent_fits(rows, cols, ldv, 1) ||
        !extent_fits(rows, cols / BQ_MX_GROUP, lds, 1))
        return BQ_ERR_BOUNDS;
    if (!aligned(y, 16) || !aligned(v, 16) || !aligned(e8m0, 4) || ldy % 8 != 0 ||
        ldv % 16 != 0 || lds % 4 != 0)
        return BQ_ERR_ALIGN;
    const Span ys = span(y, extent(rows, cols, ldy, 2));
    if (overlaps(ys, span(v, extent(rows, cols, ldv, 1))) ||
        overlaps(ys, span(e8m0, extent(rows, cols / BQ_MX_GROUP, lds, 1))))
        return BQ_ERR_ALIAS;
    return launched(
        bq::launch_dequant_mx(v, ldv, e8m0, lds, rows, cols, y, ldy, as_stream(stream)));
}

bq_status bq_mm_mx(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t ldxe,
                   const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t ldwe, int64_t M,
                   int64_t N, int64_t K, uint16_t* y, int64_t ldy, void* stream) {
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (M < 0 || N < 0 || K <= 0 || K % kBlk != 0 || M > lim || N > lim || K > lim)
        return BQ_ERR_SIZE;
    if (M == 0 || N == 0)
        return BQ_OK;
    if (!xv || !xe || !wv || !we || !y)
        return BQ_ERR_NULL;
    if (ldxv < K || ldwv < K || ldxe < K / BQ_MX_GROUP || ldwe < K / BQ_MX_GROUP || ldy < N)
        return BQ_ERR_BOUNDS;
    if (!extent_fits(M, K, ldxv, 1) || !extent_fits(M, K / BQ_MX_GROUP, ldxe, 1) ||
        !extent_fits(N, K, ldwv, 1) || !extent_fits(N, K / BQ_MX_GROUP, ldwe, 1) ||
        !extent_fits(M, N, ldy, 2))
        return BQ_ERR_BOUNDS;
    if (!aligned(xv, 16) || !aligned(wv, 16) || ldxv % 16 != 0 || ldwv % 16 != 0 ||
        !aligned(xe, 4) || !aligned(we, 4) || ldxe % 4 != 0 || ldwe % 4 != 0 || !aligned(y, 2))
        return BQ_ERR_ALIGN;
    const Span ys = span(y, extent(M, N, ldy, 2));
    if (overlaps(ys, span(xv, extent(M, K, ldxv, 1))) ||
        overlaps(ys, span(xe, extent(M, K / BQ_MX_GROUP, ldxe, 1))) ||
        overlaps(ys, span(wv, extent(N, K, ldwv, 1))) ||
        overlaps(ys, span(we, extent(N, K / BQ_MX_GROUP, ldwe, 1))))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_mm_mx(xv, ldxv, xe, ldxe, wv, ldwv, we, ldwe, M, N, K, y, ldy,
                                     as_stream(stream)));
}

int bq_mm_tile_cols(int64_t M, int64_t N, int cus) {
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (M < 1 || N < 1 || M > lim || N > lim || cus < 1)
        return -1;
    return bq::mm_tile_cols(M, N, cus);
}

// ---- MXFP8 scales in the scaled-MFMA layout --------------------------------------------------

namespace {

int64_t mfma_bytes(int64_t rows, int64_t cols) {
    return 256 * ((rows + 15) / 16) * ((cols + 511) / 512);
}

bq_status quant_mx_slice_mfma(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                              int64_t col_off, uint8_t* v, int64_t ldv, int64_t total_cols,
                              uint8_t* e8m0, int64_t capacity_rows, bool f16, void* stream) {
    BQ_TRY(check_mx_shape(rows, cols));
    if (col_off < 0 || col_off % kBlk != 0 || total_cols < 0 || total_cols % kBlk != 0 ||
        capacity_rows < 0)
        return BQ_ERR_SIZE;
    if (col_off > total_cols || cols > total_cols - col_off || total_cols > ldv ||
        rows > capacity_rows)
        return BQ_ERR_BOUNDS;
    if (rows == 0 || cols == 0)
        return BQ_OK;
    if (!x || !v || !e8m0)
        return BQ_ERR_NULL;
    if (ldx < cols || !extent_fits(rows, cols, ldx, 2) ||
        !extent_fits(rows, cols, ldv, 1) || !extent_fits(capacity_rows, total_cols, ldv, 1))
        return BQ_ERR_BOUNDS;
    if (!aligned(x, 16) || !aligned(v, 16) || !aligned(e8m0, 16) || ldx % 8 != 0 || ldv % 16 != 0)
        return BQ_ERR_ALIGN;
    const Span xs = span(x, extent(rows, cols, ldx, 2));
    const Span vs = span(v + col_off, extent(rows, cols, ldv, 1));
    const Span es = span(e8m0, mfma_bytes(capacity_rows, total_cols));
    if (overlaps(xs, vs) || overlaps(xs, es) || overlaps(vs, es))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_quant_mx_mfma(x, rows, cols, ldx, v + col_off, ldv, e8m0,
                                             (capacity_rows + 15) / 16, col_off / kBlk,
                                             as_stream(stream), f16));
}

}  // namespace

int64_t bq_mx_scale_mfma_bytes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0 || cols % kBlk != 0 || rows > ((int64_t)1 << 40) ||
        cols > ((int64_t)1 << 40))
        return -1;
    return mfma_bytes(rows, cols);
}

bq_status bq_quant_mx_slice_mfma(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 int64_t col_off, uint8_t* v, int64_t ldv, int64_t total_cols,
                                 uint8_t* e8m0, int64_t capacity_rows, void* stream) {
    return quant_mx_slice_mfma(x, rows, cols, ldx, col_off, v, ldv, total_cols, e8m0,
                               capacity_rows, false, stream);
}

bq_status bq_quant_mx_slice_mfma_f16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                     int64_t col_off, uint8_t* v, int64_t ldv,
                                     int64_t total_cols, uint8_t* e8m0, int64_t capacity_rows,
                                     void* stream) {
    return quant_mx_slice_mfma(x, rows, cols, ldx, col_off, v, ldv, total_cols, e8m0,
                               capacity_rows, true, stream);
}

bq_status bq_dequant_mx_mfma(const uint8_t* v, int64_t ldv, const uint8_t* e8m0,
                             int64_t scale_rows, int64_t rows, int64_t cols, uint16_t* y,
                             int64_t ldy, void* stream) {
    BQ_TRY(check_mx_shape(rows, cols));
    if (scale_rows < 0)
        return BQ_ERR_SIZE;
    if (rows > scale_rows)
        return BQ_ERR_BOUNDS;
    if (rows == 0 || cols == 0)
        return BQ_OK;
    if (!v || !e8m0 || !y)
        return BQ_ERR_NULL;
    if (ldy < cols || ldv < cols || !extent_fits(rows, cols, ldy, 2) ||
        !extent_fits(rows, cols, ldv, 1) || !extent_fits(scale_rows, cols, cols, 1))
        return BQ_ERR_BOUNDS;
    if (!aligned(y, 16) || !aligned(v, 16) || !aligned(e8m0, 16) || ldy % 8 != 0 || ldv % 16 != 0)
        return BQ_ERR_ALIGN;
    const Span ys = span(y, extent(rows, cols, ldy, 2));
    if (overlaps(ys, span(v, extent(rows, cols, ldv, 1))) ||
        overlaps(ys, span(e8m0, mfma_bytes(scale_rows, cols))))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_dequant_mx_mfma(v, ldv, e8m0, (scale_rows + 15) / 16, rows, cols,
                                               y, ldy, as_stream(stream)));
}

bq_status bq_mm_mx_mfma(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t xe_rows,
                        const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t we_rows,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                        void* stream) {
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (M < 0 || N < 0 || K <= 0 || K % kBlk != 0 || M > lim || N > lim || K > lim ||
        xe_rows < 0 || we_rows < 0 || xe_rows > lim || we_rows > lim)
        return BQ_ERR_SIZE;
    if (xe_rows < M || we_rows < N)
        return BQ_ERR_BOUNDS;
    if (M == 0 || N == 0)
        return BQ_OK;
    if (!xv || !xe || !wv || !we || !y)
        return BQ_ERR_NULL;
    if (ldxv < K || ldwv < K || ldy < N)
        return BQ_ERR_BOUNDS;
    if (!extent_fits(M, K, ldxv, 1) || !extent_fits(N, K, ldwv, 1) || !extent_fits(M, N, ldy, 2))
        return BQ_ERR_BOUNDS;
    if (!aligned(xv, 16) || !aligned(wv, 16) || ldxv % 16 != 0 || ldwv % 16 != 0 ||
        !aligned(xe, 16) || !aligned(we, 16) || !aligned(y, 2))
        return BQ_ERR_ALIGN;
    const Span ys = span(y, extent(M, N, ldy, 2));
    if (overlaps(ys, span(xv, extent(M, K, ldxv, 1))) ||
        overlaps(ys, span(xe, mfma_bytes(xe_rows, K))) ||
        overlaps(ys, span(wv, extent(N, K, ldwv, 1))) ||
        overlaps(ys, span(we, mfma_bytes(we_rows, K))))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_mm_mx_mfma(xv, ldxv, xe, (xe_rows + 15) / 16, wv, ldwv, we,
                                          (we_rows + 15) / 16, M, N, K, y, ldy,
                                          as_stream(stream)));
}

// ---- E4M3 128-block codec ------------------------------------------------------------------

bq_status bq_quant_e4m3_b128(const uint16_t* x, int64_t n, uint8_t* v, float* scale,
                             void* stream) {
    BQ_TRY(check_n(n));
    if (n == 0)
        return BQ_OK;
    BQ_TRY(check_bf16(x));
    BQ_TRY(check_payload(v));
    BQ_TRY(check_scales(scale));
    const Span xs = span(x, 2 * n), vs = span(v, n), ss = span(scale, 4 * (n / kBlk));
    if (overlaps(xs, vs) || overlaps(xs, ss) || overlaps(vs, ss))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_quant_e4m3_b128(x, v, scale, n, as_stream(stream)));
}

bq_status bq_dequant_e4m3_b128(const uint8_t* v, const float* scale, int64_t n, uint16_t* y,
                               void* stream) {
    BQ_TRY(check_n(n));
    if (n == 0)
        return BQ_OK;
    BQ_TRY(check_payload(v));
    BQ_TRY(check_scales(scale));
    BQ_TRY(check_bf16(y));
    const Span ys = span(y, 2 * n);
    if (overlaps(ys, span(v, n)) || overlaps(ys, span(scale, 4 * (n / kBlk))))
        return BQ_ERR_ALIAS;
    return launched(bq::launch_dequant_e4m3_b128(v, scale, y, n, as_stream(stream)));
}

}  // extern "C"
