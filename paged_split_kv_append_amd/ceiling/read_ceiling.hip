// Read-only probe kernel that bounds what a decode read can reach on this
// GPU: a buffer read as 4 KB blocks (one 16-position page of one KV head at
// D = 128, bf16), one wave per block, in the order a caller gives: address
// order for a plain stream, a random permutation for the decode's page order.
// It does no arithmetic beyond folding the loaded words into a value that is
// stored only if it equals a fixed constant, so the loads cannot be dropped.
// Used by bench.py to report the decode's fraction of the practical ceiling
// beside its fraction of the HBM peak; not part of libnbx_paged.
//
// 16-byte non-temporal loads, as the decode kernels stream K/V; 256-thread
// workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;       // the folded value is stored only if equal

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Blocks order[0 .. nblocks) of 4 KB each from `base`, one wave per block at a
// time (four 1 KB loads of 64 lanes x 16 bytes), two blocks in flight per wave;
// wave w takes blocks w, w + Wt, ... (Wt waves in the grid).
__global__ void __launch_bounds__(kThreads) block_read_kernel(const uint8_t *base,
                                                              const int32_t *order,
                                                              int32_t nblocks, uint32_t *sink)
{
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (kThreads / 64);
    int w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    uint32_t acc = 0;
    for (; w < nblocks; w += 2 * waves) {
        const u32x4 *x = (const u32x4 *)(base + (int64_t)order[w] * 4096) + lane;
        const bool two = w + waves < nblocks;
        const u32x4 *y = (const u32x4 *)(base + (int64_t)order[two ? w + waves : w] * 4096) + lane;
        u32x4 r[8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = __builtin_nontemporal_load(x + 64 * j);
        if (two) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[4 + j] = __builtin_nontemporal_load(y + 64 * j);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[4 + j] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc ^= fold(r[j]);
    }
    if (acc == kNever)
        sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

int launch_status(hipError_t e) { return e == hipSuccess ? 0 : -7; }

}  // namespace

extern "C" {

// Reads the 4 KB blocks order[0 .. nblocks) of device buffer base (4 KB
// aligned, every order[i] in [0, nblocks) so the buffer holds nblocks * 4096
// bytes: the caller passes a permutation) with `workgroups` workgroups of 256
// threads; sink is a device uint32 array of at least workgroups * 256 entries.
int nbx_ceiling_block_read(const void *base, const int32_t *order, int32_t nblocks,
                           int32_t workgroups, uint32_t *sink, hipStream_t stream)
{
    if (!base || !order || !sink)
        return -1;
    if (nblocks < 1 || ((uintptr_t)base & 4095u) || workgroups < 1)
        return -3;
    block_read_kernel<<<workgroups, kThreads, 0, stream>>>((const uint8_t *)base, order, nblocks,
                                                           sink);
    return launch_status(hipGetLastError());
}

}  // extern "C"
