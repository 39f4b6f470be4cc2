// bq_mm.hip -- the dense MXFP8 GEMM from staged inputs, on gfx950's scaled MFMA.
//
// Definition (b12x pull request #241, "[II] Support staged MXFP8 linear inputs", Behavior:
// mm_quantized / mm_quantized_into run the dense GEMM on the assembled MXFP8 input):
//   Y[m][n] = bf16_rne( sum over k of X[m][k] * W[n][k] ),
// X the MXFP8 activations (E4M3 values, one E8M0 byte per 32 columns of a row), W the
// MXFP8 weights in the same layout, both K-contiguous; the products are exact and are
// summed in binary32 by the matrix cores, then rounded to bf16 once.
//
// Matrix-core mapping (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 operands): for a 16 x 128
// A block, lane l holds row l%16 and, with g = l/16, K bytes [16g, 16g+16) in its first
// 16 bytes and [64+16g, 64+16g+16) in its last 16; B likewise with column l%16.  The scale
// register of lane l supplies the E8M0 byte of row (column) l%16 and K-block l/16 of the
// 128 (byte 0 with opsel 0).  The 4 results of lane l are rows 4(l/16) + r, column l%16.
// (Measured on MI355X with exact small-integer operands before this kernel was written.)
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of Y; its 4 waves own 64 x 64
// quadrants, each 4 x 4 MFMA blocks.  Per K step of 128 the workgroup stages the X and W
// tiles (16 KB each) and their 128 x 4 scale bytes in LDS, double-buffered, so the
// global loads of step k+1 are in flight while step k computes; one barrier per step.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 128, kTN = 128, kTK = 128;   // workgroup tile
constexpr int kRowPad = kTK + 16;                 // LDS row stride of a staged tile (bytes)

struct MmArgs {
    const uint8_t* xv;
    const uint8_t* xe;
    const uint8_t* wv;
    const uint8_t* we;
    uint16_t* y;
    int64_t ldxv, ldxe, ldwv, ldwe, ldy;
    int32_t M, N, K;
    int32_t tiles_n;   // column tiles
};

struct Stage {
    uint8_t a[kTM * kRowPad];
    uint8_t b[kTN * kRowPad];
    uint32_t as[kTM];   // 4 E8M0 bytes (the 4 K-blocks of the step) per row
    uint32_t bs[kTN];
};

// The global loads of one K step: 4 16-byte chunks of the X tile and 4 of the W tile per
// thread (8 chunks per 128-byte row), and one scale word (threads 0-127: X rows,
// 128-255: W rows).  Rows beyond M (N) are clamped to the last row; their results are
// never stored.
struct Prefetch {
    u32x4 a[4], b[4];
    uint32_t s;
};

__device__ __forceinline__ void load_step(const MmArgs& p, int m0, int n0, int k0, int tid,
                                          Prefetch& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, col = (c & 7) * 16;
        const int ma = min(m0 + row, p.M - 1), nb = min(n0 + row, p.N - 1);
        f.a[i] = ld16(p.xv + (int64_t)ma * p.ldxv + k0 + col);
        f.b[i] = ld16(p.wv + (int64_t)nb * p.ldwv + k0 + col);
    }
    if (tid < kTM) {
        const int ma = min(m0 + tid, p.M - 1);
        f.s = *reinterpret_cast<const uint32_t*>(p.xe + (int64_t)ma * p.ldxe + k0 / 32);
    } else {
        const int nb = min(n0 + tid - kTM, p.N - 1);
        f.s = *reinterpret_cast<const uint32_t*>(p.we + (int64_t)nb * p.ldwe + k0 / 32);
    }
}

__device__ __forceinline__ void store_step(Stage& st, int tid, const Prefetch& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, col = (c & 7) * 16;
        *reinterpret_cast<u32x4*>(st.a + row * kRowPad + col) = f.a[i];
        *reinterpret_cast<u32x4*>(st.b + row * kRowPad + col) = f.b[i];
    }
    if (tid < kTM)
        st.as[tid] = f.s;
    else
        st.bs[tid - kTM] = f.s;
}

// One 16 x 128 operand fragment of a lane from a staged tile: row `r`, K bytes
// [16g, 16g+16) and [64+16g, 64+16g+16).
__device__ __forceinline__ i32x8 frag(const uint8_t* tile, int r, int g) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + r * kRowPad + 16 * g);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + r * kRowPad + 64 + 16 * g);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ __launch_bounds__(256) void k_mm_mx(MmArgs p) {
    __shared__ Stage stage[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int tile = blockIdx.x;
    const int m0 = (tile / p.tiles_n) * kTM, n0 = (tile % p.tiles_n) * kTN;
    const int r16 = lane & 15, g = lane >> 4;

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = p.K / kTK;
    Prefetch f;
    load_step(p, m0, n0, 0, tid, f);
    store_step(stage[0], tid, f);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more)
            load_step(p, m0, n0, (kt + 1) * kTK, tid, f);
        const Stage& st = stage[kt & 1];
        i32x8 bf[4];
        int bsc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = wn + 16 * b + r16;
            bf[b] = frag(st.b, n, g);
            bsc[b] = (int)((st.bs[n] >> (8 * g)) & 0xFFu);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int m = wm + 16 * a + r16;
            const i32x8 af = frag(st.a, m, g);
            const int asc = (int)((st.as[m] >> (8 * g)) & 0xFFu);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[b], acc[a][b], 0, 0, 0, asc, 0, bsc[b]);
        }
        if (more)
            store_step(stage[(kt + 1) & 1], tid, f);
        __syncthreads();
    }

    // epilogue: lane l holds rows 4(l/16) + r of column l%16 of each 16 x 16 block
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = n0 + wn + 16 * b + r16;
            const uint32_t lo = pack_bf16x2(acc[a][b].x, acc[a][b].y);
            const uint32_t hi = pack_bf16x2(acc[a][b].z, acc[a][b].w);
            const uint16_t v[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                   (uint16_t)(hi >> 16)};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + 16 * a + 4 * g + r;
                if (row < p.M && col < p.N)
                    p.y[(int64_t)row * p.ldy + col] = v[r];
            }
        }
    }
}

}  // namespace

hipError_t launch_mm_mx(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t ldxe,
                        const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t ldwe,
                        int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                        hipStream_t stream) {
    MmArgs a{};
    a.xv = xv;
    a.xe = xe;
    a.wv = wv;
    a.we = we;
    a.y = y;
    a.ldxv = ldxv;
    a.ldxe = ldxe;
    a.ldwv = ldwv;
    a.ldwe = ldwe;
    a.ldy = ldy;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    const int64_t tm = (M + kTM - 1) / kTM, tn = (N + kTN - 1) / kTN;
    a.tiles_n = (int32_t)tn;
    return launch1(k_mm_mx, dim3((unsigned)(tm * tn)), dim3(256), stream, a);
}

}  // namespace bq
