// bq_launch.h -- internal launchers of the libblockq kernels (host side).
//
// Arguments are assumed valid: the public entry points in bq_abi.cpp validate every
// pointer, size, alignment and overlap before calling these.  Each launcher enqueues
// one kernel on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

// Launch `kernel` with its one by-value argument struct on `stream` and return the
// status of this launch itself (not the thread's sticky last error, which may hold
// an earlier failure of some unrelated runtime call).
template <typename Arg>
hipError_t launch1(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t stream, Arg arg) {
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

// Flat block formats on the wire, one overload per codec (selected by the payload and
// scale pointer types): block INT8 (int8_t payload, one float scale per 128 values)
// and flat MXFP8 (uint8_t E4M3 payload, one uint8_t E8M0 byte per 32 values).  Both
// are 132 bytes per 128 values.  Segment i of a batch is (x[i] -> q[i], s[i]), n values.
hipError_t launch_quant(int count, const uint16_t* const* x, int8_t* const* q, float* const* s,
                        int64_t n, hipStream_t stream);
hipError_t launch_quant(int count, const uint16_t* const* x, uint8_t* const* v,
                        uint8_t* const* e, int64_t n, hipStream_t stream);
// skip_shard_n > 0: segment i leaves values [i*skip_shard_n, (i+1)*skip_shard_n) of
// its output untouched (the shard an all-to-all owner has already materialized).
hipError_t launch_dequant(int count, const int8_t* const* q, const float* const* s,
                          uint16_t* const* y, int64_t n, hipStream_t stream,
                          int64_t skip_shard_n = 0);
hipError_t launch_dequant(int count, const uint8_t* const* v, const uint8_t* const* e,
                          uint16_t* const* y, int64_t n, hipStream_t stream,
                          int64_t skip_shard_n = 0);
hipError_t launch_ring_hop(int count, const int8_t* const* q_in, const float* const* s_in,
                           const uint16_t* const* local, int8_t* const* q_out,
                           float* const* s_out, int64_t n, hipStream_t stream);
hipError_t launch_ring_hop(int count, const uint8_t* const* v_in, const uint8_t* const* e_in,
                           const uint16_t* const* local, uint8_t* const* v_out,
                           uint8_t* const* e_out, int64_t n, hipStream_t stream);
// nseg segments of seg_n values: segment j reads q[k] + j*seg_n (scales likewise) for
// every source k in order and writes y + j*seg_n.
hipError_t launch_accum(int nsrc, const int8_t* const* q, const float* const* s, uint16_t* y,
                        int nseg, int64_t seg_n, hipStream_t stream);
hipError_t launch_accum(int nsrc, const uint8_t* const* v, const uint8_t* const* e, uint16_t* y,
                        int nseg, int64_t seg_n, hipStream_t stream);
// The fused all-to-all owner step: accumulate as above, requantize each owner's bf16
// sum into q_out/s_out (segment j at j*seg_n), materialize it into y[j] (y or y[j] may
// be null) and store the bf16 sums into red (may be null).
hipError_t launch_a2a_reduce(int nsrc, const int8_t* const* q, const float* const* s, int nseg,
                             int64_t seg_n, int8_t* q_out, float* s_out, uint16_t* const* y,
                             uint16_t* red, hipStream_t stream);
hipError_t launch_a2a_reduce(int nsrc, const uint8_t* const* v, const uint8_t* const* e,
                             int nseg, int64_t seg_n, uint8_t* v_out, uint8_t* e_out,
                             uint16_t* const* y, uint16_t* red, hipStream_t stream);

// MXFP8 (row-major with leading dimensions; cols a multiple of 128).
// f16: x holds IEEE binary16 values instead of bf16.
hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* v, int64_t ldv, uint8_t* e8m0, int64_t lds,
                           hipStream_t stream, bool f16 = false);
hipError_t launch_dequant_mx(const uint8_t* v, int64_t ldv, const uint8_t* e8m0, int64_t lds,
                             int64_t rows, int64_t cols, uint16_t* y, int64_t ldy,
                             hipStream_t stream);

// The same with the scales in the scaled-MFMA layout of `rb` 16-row blocks (base e_layout);
// the matrix's column 0 is K step `step0` of the layout.
hipError_t launch_quant_mx_mfma(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* v, int64_t ldv, uint8_t* e_layout, int64_t rb,
                                int64_t step0, hipStream_t stream, bool f16 = false);
hipError_t launch_dequant_mx_mfma(const uint8_t* v, int64_t ldv, const uint8_t* e_layout,
                                  int64_t rb, int64_t rows, int64_t cols, uint16_t* y,
                                  int64_t ldy, hipStream_t stream);

// The dense MXFP8 GEMM Y = bf16(X W^T) (M, N >= 1; K a positive multiple of 128).
hipError_t launch_mm_mx(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t ldxe,
                        const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t ldwe,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                        hipStream_t stream);
// The same GEMM with both operands' scales in the scaled-MFMA layout, of xrb and wrb
// 16-row blocks.
// The column count (256 or 224) of the GEMM's workgroup tiles for an M x N product on `cus`
// compute units.
int mm_tile_cols(int64_t M, int64_t N, int cus);
hipError_t launch_mm_mx_mfma(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t xrb,
                             const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t wrb,
                             int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                             hipStream_t stream);

// E4M3 128-block codec.
hipError_t launch_quant_e4m3_b128(const uint16_t* x, uint8_t* v, float* s, int64_t n,
                                  hipStream_t stream);
hipError_t launch_dequant_e4m3_b128(const uint8_t* v, const float* s, uint16_t* y, int64_t n,
                                    hipStream_t stream);

}  // namespace bq
