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
// Tiling: a 512-thread workgroup computes a 256 x TN tile of Y, TN = 256 or 224, whichever
// fills the compute units better for the shape (an N of 7168 makes 32 columns of 224 and
// 512 tiles, two full rounds on 256 units, where columns of 256 make 448 tiles and leave an
// eighth of the second round idle).  Its 8 waves (two per SIMD, so one can issue matrix
// instructions while the other waits on LDS) own 128 x 64 pieces (2 x 4 waves, TN = 256) or
// 64 x 112 pieces (4 x 2 waves, TN = 224): a wave reads 12 (11) operand fragments from LDS
// per 32 (28) MFMAs.
// Per K step of 128 the workgroup stages the X and W tiles (32 KB and TN x 128 bytes) in
// LDS, double-buffered, with gfx950's global-to-LDS loads (global_load_lds_dwordx4: each
// wave instruction fills 1 KB of LDS, lane i at byte 16i), so no registers hold the staged
// data and the loads of step k+1 are in flight while step k computes; every product of
// step k is issued before the wait that closes it, then one barrier.  A tile row is 128
// contiguous bytes; its 16-byte chunk c sits in slot c ^ ((row >> 1) & 7), so the 16 rows a
// fragment read touches at one chunk fall in 16 distinct 16-byte bank groups.
//
// Scales: a row's E8M0 bytes for one K step are 4 bytes, and fetching them as their own
// 4-byte request per row and step cost about 11% of the kernel's time (one request per row
// beside the row's two 64-byte operand requests).  When K is a multiple of 512 and the scale
// rows are 16-byte aligned, one 16-byte load per row brings the scales of 4 K steps into a
// double-buffered LDS area (2 x 8 KB), a quarter of the requests; otherwise each step stages
// its rows' 4 bytes with its operands.
//
// With the scales in the scaled-MFMA layout (256-byte tiles of 16 rows x 4 K steps, word l
// for lane l, byte j for step j), a group's scales for the workgroup are 32 whole tiles: one
// 16-byte global-to-LDS load per lane brings them in, for any K that is a multiple of 128,
// and each lane then reads its own word of its fragment's tile.
//
// Tiles are numbered in groups of 8 row tiles, a group walking down its 8 row tiles and
// then across the columns, and each XCD (every 8th workgroup) takes a contiguous run of that
// numbering: the 32 workgroups an XCD runs at once then share 8 X row tiles and 4 W column
// tiles in its L2, where a plain column-major run has them share 2 W tiles but need 16 X
// tiles, and fewer of their requests leave the L2.
#include "bq_device.h"
#include "bq_launch.h"

namespace bq {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 256, kTK = 128;                // workgroup tile rows, K step
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kWaveLoads = kTM * kTK / 1024 / kWaves;   // 1 KB X-tile loads per wave per step
constexpr int kScaleRows = kTM / kWaves;                 // scale rows per wave per operand
constexpr int kGroupSteps = 4;                           // K steps per grouped scale load
constexpr int kScaleSlots = 2 * kTM;                     // X rows, then W rows

// A workgroup tile of 256 rows by TN columns (TN = 256 or 224) and its split over the 8
// waves: 2 x 4 waves of 128 x 64 for TN = 256, 4 x 2 waves of 64 x 112 for TN = 224.
template <int TN>
struct Tiling {
    static_assert(TN == 256 || TN == 224, "tile widths");
    static constexpr int kWavesM = TN == 256 ? 2 : 4;
    static constexpr int kWavesN = kWaves / kWavesM;
    static constexpr int kWM = kTM / kWavesM, kWN = TN / kWavesN;
    static constexpr int kFA = kWM / 16, kFB = kWN / 16;    // MFMA blocks per wave tile side
    static constexpr int kPiecesB = TN * kTK / 1024;          // 1 KB pieces of a W tile
};

// How the E8M0 scales reach LDS: each K step its rows' 4 bytes from row-major rows; four
// K steps at once, 16 bytes per row-major row; or four K steps at once as whole tiles of
// the scaled-MFMA layout.
enum Scales { kStepRows = 0, kGroupRows = 1, kGroupMfma = 2 };

struct MmArgs {
    const uint8_t* xv;
    const uint8_t* xe;
    const uint8_t* wv;
    const uint8_t* we;
    uint16_t* y;
    int64_t ldxv, ldxe, ldwv, ldwe, ldy;   // MFMA layout: ldxe / ldwe are the 16-row blocks
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;   // row and column tiles
};

template <int TN>
struct Stage {
    uint8_t a[kTM * kTK];   // rows of 128 bytes, chunks swizzled (see chunk_slot)
    uint8_t b[TN * kTK];
    // the 4 E8M0 bytes (the step's 4 K blocks) of each row: word 64w + j holds X row
    // kScaleRows*w + j for j < 32 and W row kScaleRows*w + j - 32 for j >= 32
    uint32_t sc[kScaleSlots];
};

template <int TN>
struct Smem {
    Stage<TN> stage[2];
    // grouped scales: slot r (X row r, then W row r - kTM) holds the 16 E8M0 bytes of
    // kGroupSteps K steps, word j for step j of the group; in the MFMA layout the same
    // area holds 32 tiles of 64 words (X row blocks 0..15, then W row blocks 0..15)
    uint32_t scg[2][kScaleSlots * kGroupSteps];
};
static_assert(kScaleSlots * kGroupSteps == 32 * 64, "a group of MFMA-layout tiles fills the area");

template <int TN>
__device__ __forceinline__ uint32_t x_scale_word(const Stage<TN>& st, int row) {
    return st.sc[(row / kScaleRows) * 64 + row % kScaleRows];
}
template <int TN>
__device__ __forceinline__ uint32_t w_scale_word(const Stage<TN>& st, int row) {
    return st.sc[(row / kScaleRows) * 64 + 32 + row % kScaleRows];
}

__device__ __forceinline__ int chunk_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

// Issue the global-to-LDS loads of one K step into `st`: the X tile's 32 pieces of 1 KB go
// 4 to a wave (pieces 4w .. 4w+3), the W tile's TN/8 pieces are dealt round-robin (piece
// w + 8j); each piece is 64 lanes x 16 bytes, lane i landing at byte 16i of the piece and
// fetching the chunk that belongs in that slot.  In the per-step form the wave also loads
// the scale words of X and W rows [32w, 32w+32) (4 bytes per lane: lanes 0-31 X, 32-63 W).
// Rows beyond M (N) are clamped to the last row; their results are never stored.
template <int Sc, int TN>
__device__ __forceinline__ void load_step(const MmArgs& p, Stage<TN>& st, int m0, int n0, int k0,
                                          int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kWaveLoads; ++j) {
        const int piece = wave * kWaveLoads + j;
        const int u = piece * 64 + lane;              // 16-byte unit of the tile
        const int row = u >> 3;
        const int c = chunk_slot(row, u & 7);         // the slot's chunk (the map is an involution)
        const int ma = min(m0 + row, p.M - 1);
        __builtin_amdgcn_global_load_lds(p.xv + (int64_t)ma * p.ldxv + k0 + 16 * c,
                                         st.a + piece * 1024, 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < (Tiling<TN>::kPiecesB + kWaves - 1) / kWaves; ++j) {
        const int piece = wave + kWaves * j;
        if (piece < Tiling<TN>::kPiecesB) {
            const int u = piece * 64 + lane;
            const int row = u >> 3;
            const int c = chunk_slot(row, u & 7);
            const int nb = min(n0 + row, p.N - 1);
            __builtin_amdgcn_global_load_lds(p.wv + (int64_t)nb * p.ldwv + k0 + 16 * c,
                                             st.b + piece * 1024, 16, 0, 0);
        }
    }
    if (Sc != kStepRows)
        return;
    const int r = kScaleRows * wave + (lane & 31);
    const uint8_t* src = lane < 32
        ? p.xe + (int64_t)min(m0 + r, p.M - 1) * p.ldxe + k0 / 32
        : p.we + (int64_t)min(n0 + r, p.N - 1) * p.ldwe + k0 / 32;
    __builtin_amdgcn_global_load_lds(src, st.sc + 64 * wave, 4, 0, 0);
}

// The scales of K steps [4g, 4g+4), bytes [16g, 16g+16) of every E8M0 row, into `dst`:
// wave w fills slots [64w, 64w+64) (X rows for w < 4, W rows after), 16 bytes per lane,
// lane i at slot 64w + i.  Rows beyond M (N) are clamped to the last row.
__device__ __forceinline__ void load_scale_group(const MmArgs& p, uint32_t* dst, int m0, int n0,
                                                 int g, int wave, int lane) {
    const int slot = 64 * wave + lane;
    const uint8_t* src = slot < kTM
        ? p.xe + (int64_t)min(m0 + slot, p.M - 1) * p.ldxe + 16 * g
        : p.we + (int64_t)min(n0 + slot - kTM, p.N - 1) * p.ldwe + 16 * g;
    __builtin_amdgcn_global_load_lds(src, dst + 64 * kGroupSteps * wave, 16, 0, 0);
}

// The scales of K steps [4g, 4g+4) from the scaled-MFMA layout into `dst`: the workgroup's
// 16 X row blocks and 16 W row blocks are 32 tiles of 256 bytes; wave w fills tiles
// [4w, 4w+4), 16 bytes per lane, lane i at byte 16i of the wave's 1 KB (tile 4w + i/16,
// bytes [16(i%16), 16(i%16)+16) of it).  Row blocks beyond the last row are clamped to the
// last one; their results are never stored.
__device__ __forceinline__ void load_scale_group_mfma(const MmArgs& p, uint32_t* dst, int m0,
                                                      int n0, int g, int wave, int lane) {
    const int t = 4 * wave + (lane >> 4);
    const int part = 16 * (lane & 15);
    const uint8_t* src = t < 16
        ? p.xe + ((int64_t)g * p.ldxe + min(m0 / 16 + t, (p.M - 1) / 16)) * 256 + part
        : p.we + ((int64_t)g * p.ldwe + min(n0 / 16 + t - 16, (p.N - 1) / 16)) * 256 + part;
    __builtin_amdgcn_global_load_lds(src, dst + 256 * wave, 16, 0, 0);
}

// Wait for this wave's global-to-LDS loads (the barrier that follows publishes them).
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16 x 128 operand fragment of a lane from a staged tile: row `r`, K bytes
// [16g, 16g+16) and [64+16g, 64+16g+16) (chunks g and 4+g).
__device__ __forceinline__ i32x8 frag(const uint8_t* tile, int r, int g) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + r * kTK + 16 * chunk_slot(r, g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + r * kTK + 16 * chunk_slot(r, 4 + g));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// The tile of workgroup `bid` as its (row tile, column tile).  Tiles are numbered in groups
// of 8 row tiles, each group walking its 8 row tiles down one column of tiles, then the next
// column; with T tiles and T divisible by 8, XCD x (= bid % 8) takes the contiguous run
// [x T/8, (x+1) T/8) of that numbering, so the workgroups an XCD runs at once share a few
// row tiles (X) and column tiles (W) in its L2.
__device__ __forceinline__ int2 tile_of(int bid, int tiles_m, int tiles_n) {
    constexpr int kGroupM = 8;
    const int tiles = tiles_m * tiles_n;
    const int t = tiles % 8 != 0 ? bid : (bid % 8) * (tiles / 8) + bid / 8;
    const int first = t / (kGroupM * tiles_n) * kGroupM;   // the group's first row tile
    const int rows = min(tiles_m - first, kGroupM);
    const int u = t % (kGroupM * tiles_n);
    return int2{first + u % rows, u / rows};
}

template <int Sc, int TN>
__global__ __launch_bounds__(kThreads) void k_mm_mx(MmArgs p) {
    constexpr bool Grouped = Sc != kStepRows;
    constexpr int kWavesN = Tiling<TN>::kWavesN, kWM = Tiling<TN>::kWM, kWN = Tiling<TN>::kWN;
    constexpr int kFA = Tiling<TN>::kFA, kFB = Tiling<TN>::kFB;
    __shared__ Smem<TN> sm;
    Stage<TN>* stage = sm.stage;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / kWavesN) * kWM, wn = (wave % kWavesN) * kWN;
    const int2 tile = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
    const int m0 = tile.x * kTM, n0 = tile.y * TN;
    const int r16 = lane & 15, g = lane >> 4;

    f32x4 acc[kFA][kFB];
#pragma unroll
    for (int a = 0; a < kFA; ++a)
#pragma unroll
        for (int b = 0; b < kFB; ++b)
            acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Pipeline: two stages; the loads of step k+1 are issued as step k starts and have
    // landed, in every wave, by the barrier that closes step k.
    const int nk = p.K / kTK;
    load_step<Sc, TN>(p, stage[0], m0, n0, 0, wave, lane);
    if (Sc == kGroupRows)
        load_scale_group(p, sm.scg[0], m0, n0, 0, wave, lane);
    if (Sc == kGroupMfma)
        load_scale_group_mfma(p, sm.scg[0], m0, n0, 0, wave, lane);
    wait_loads();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk)
            load_step<Sc, TN>(p, stage[(kt + 1) & 1], m0, n0, (kt + 1) * kTK, wave, lane);
        // the next group's scales go into the buffer the previous group used; they land by
        // this step's closing wait, three steps before they are read
        if (Grouped && (kt & (kGroupSteps - 1)) == 0 && kt + kGroupSteps < nk) {
            uint32_t* next = sm.scg[(kt / kGroupSteps + 1) & 1];
            if (Sc == kGroupRows)
                load_scale_group(p, next, m0, n0, kt / kGroupSteps + 1, wave, lane);
            else
                load_scale_group_mfma(p, next, m0, n0, kt / kGroupSteps + 1, wave, lane);
        }
        const Stage<TN>& st = stage[kt & 1];
        const uint32_t* scg = sm.scg[(kt / kGroupSteps) & 1] + (kt & (kGroupSteps - 1));
        // MFMA layout: lane l's word of a fragment's tile, byte kt % 4
        const uint32_t* tiles = sm.scg[(kt / kGroupSteps) & 1] + lane;
        const int shift = 8 * (kt & (kGroupSteps - 1));
        i32x8 bf[kFB];
        int bsc[kFB];
#pragma unroll
        for (int b = 0; b < kFB; ++b) {
            const int n = wn + 16 * b + r16;
            bf[b] = frag(st.b, n, g);
            if constexpr (Sc == kGroupMfma) {
                bsc[b] = (int)((tiles[64 * (16 + wn / 16 + b)] >> shift) & 0xFFu);
            } else {
                const uint32_t ww = Grouped ? scg[(kTM + n) * kGroupSteps] : w_scale_word(st, n);
                bsc[b] = (int)((ww >> (8 * g)) & 0xFFu);
            }
        }
#pragma unroll
        for (int a = 0; a < kFA; ++a) {
            const int m = wm + 16 * a + r16;
            const i32x8 af = frag(st.a, m, g);
            int asc;
            if constexpr (Sc == kGroupMfma) {
                asc = (int)((tiles[64 * (wm / 16 + a)] >> shift) & 0xFFu);
            } else {
                const uint32_t xw = Grouped ? scg[m * kGroupSteps] : x_scale_word(st, m);
                asc = (int)((xw >> (8 * g)) & 0xFFu);
            }
#pragma unroll
            for (int b = 0; b < kFB; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[b], acc[a][b], 0, 0, 0, asc, 0, bsc[b]);
        }
        // every product of the step is issued before the wait (left to itself the compiler
        // moves half of them after the barrier, which leaves the loads half a step to land)
        __builtin_amdgcn_sched_barrier(0);
        wait_loads();
        __syncthreads();
    }

    // epilogue: lane l holds rows 4(l/16) + r of column l%16 of each 16 x 16 block
#pragma unroll
    for (int a = 0; a < kFA; ++a) {
#pragma unroll
        for (int b = 0; b < kFB; ++b) {
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

// The tile width the launches use on the current device (its compute-unit count read each
// launch; 256 if it cannot be read).
int pick_tile_n(int64_t M, int64_t N) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return mm_tile_cols(M, N, cus);
}

template <int Sc>
hipError_t launch_tiled(const MmArgs& a0, hipStream_t stream) {
    MmArgs a = a0;
    const int64_t tm = (a.M + kTM - 1) / kTM;
    const int tn_w = pick_tile_n(a.M, a.N);
    const int64_t tn = (a.N + tn_w - 1) / tn_w;
    a.tiles_m = (int32_t)tm;
    a.tiles_n = (int32_t)tn;
    const dim3 grid((unsigned)(tm * tn));
    if (tn_w == 224)
        return launch1(k_mm_mx<Sc, 224>, grid, dim3(kThreads), stream, a);
    return launch1(k_mm_mx<Sc, 256>, grid, dim3(kThreads), stream, a);
}

}  // namespace

// The tile width for an M x N product on `cus` compute units: the one whose tiles fill the
// units in the least time, counted as rounds of one workgroup per unit times the tile's
// width (a 256 x 256 tile keeps a unit for 8/7 of a 256 x 224 tile's time); ties go to 256.
int mm_tile_cols(int64_t M, int64_t N, int cus) {
    const int64_t tm = (M + kTM - 1) / kTM;
    const auto cost = [&](int64_t tn) {
        const int64_t tiles = tm * ((N + tn - 1) / tn);
        return (tiles + cus - 1) / cus * tn;
    };
    return cost(224) < cost(256) ? 224 : 256;
}

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
    const bool grouped = K % (kTK * kGroupSteps) == 0 && reinterpret_cast<uintptr_t>(xe) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(we) % 16 == 0 && ldxe % 16 == 0 && ldwe % 16 == 0;
    if (grouped)
        return launch_tiled<kGroupRows>(a, stream);
    return launch_tiled<kStepRows>(a, stream);
}

hipError_t launch_mm_mx_mfma(const uint8_t* xv, int64_t ldxv, const uint8_t* xe, int64_t xrb,
                             const uint8_t* wv, int64_t ldwv, const uint8_t* we, int64_t wrb,
                             int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                             hipStream_t stream) {
    MmArgs a{};
    a.xv = xv;
    a.xe = xe;
    a.wv = wv;
    a.we = we;
    a.y = y;
    a.ldxv = ldxv;
    a.ldxe = xrb;
    a.ldwv = ldwv;
    a.ldwe = wrb;
    a.ldy = ldy;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    return launch_tiled<kGroupMfma>(a, stream);
}

}  // namespace bq
