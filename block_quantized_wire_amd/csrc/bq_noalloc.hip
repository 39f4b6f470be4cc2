// bq_noalloc.hip -- the allocation-free form of the INT8 ring all-reduce.
//
// The ring all-reduce needs one wire payload of 132 bytes per 128 values besides the
// caller's partials and outputs.  bq_ring_allreduce_i8 takes it as caller-owned
// buffers; bq_ring_allreduce_i8_noalloc keeps it in a file-scope device array instead,
// for callers that cannot allocate.  The array's device address is looked up once per
// GPU with that GPU current and cached; kernels only ever see that address.
#include "blockq.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = BQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// One copy per GPU, at its own address on each.  In host code `scratch` is only a
// registration handle: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];

// The device address of the scratch array on the GPU that `stream` runs on (the current
// GPU for the null stream), looked up on the first call for that GPU.
bq_status scratch_for(hipStream_t stream, uint8_t** out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return BQ_ERR_LAUNCH;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess)
        return BQ_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices)
        return BQ_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return BQ_ERR_LAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess)
            return BQ_ERR_LAUNCH;
        if (e != hipSuccess || p == nullptr)
            return BQ_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch[dev]);
    return BQ_OK;
}

}  // namespace

extern "C" bq_status bq_ring_allreduce_i8_noalloc(int world, int64_t n,
                                                  const uint16_t* const* partials,
                                                  uint16_t* const* out, void* stream) {
    // Sizes first, so that a call that cannot fit fails before anything else happens;
    // every other check is the ring driver's own.
    if (world < 1 || world > BQ_MAX_BATCH)
        return BQ_ERR_NSRC;
    if (n < 0 || n % BQ_BLOCK != 0 || n % ((int64_t)BQ_BLOCK * world) != 0)
        return BQ_ERR_SIZE;
    if (n / BQ_BLOCK > kScratchBytes / (BQ_BLOCK + 4))
        return BQ_ERR_SCRATCH;
    if (n == 0)
        return BQ_OK;
    if (partials == nullptr || out == nullptr)
        return BQ_ERR_NULL;
    uint8_t* base = nullptr;
    const bq_status st = scratch_for(reinterpret_cast<hipStream_t>(stream), &base);
    if (st != BQ_OK)
        return st;
    // payload: n bytes at the start (256-byte aligned); scales: 4 bytes per block right
    // after it (n is a multiple of 128, so 4-byte aligned)
    return bq_ring_allreduce_i8(world, n, partials, reinterpret_cast<int8_t*>(base),
                                reinterpret_cast<float*>(base + n), out, stream);
}
