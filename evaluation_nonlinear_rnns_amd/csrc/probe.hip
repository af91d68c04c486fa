// Measurement utility: the HBM rate a plain streaming kernel reaches on this
// device for a given read / write mix, the reference the bench reports next to
// the datasheet peak.  One contiguous read stream and one write stream: output
// group g (64 vectors of 16 bytes, one per lane of a wavefront) is the XOR of
// the k input groups k g .. k g + k - 1 taken lane by lane (every load and
// store is 1 KB per wavefront, contiguous), U groups per wavefront in flight
// (4 for a copy, 8 otherwise), non-temporal loads and stores, one workgroup of
// four wavefronts per compute unit (the fastest of the grid sizes and depths
// measured for this probe).  A last partial group of r < 64 vectors reads its k
// partial input groups of r vectors the same way.
#include "internal.h"

namespace deer {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int K, int U>
__global__ __launch_bounds__(256) void stream_probe_kernel(const v4i *__restrict__ src, v4i *__restrict__ dst,
                                                           size_t n)
{
    const size_t ngroups = n / 64;
    const size_t nw = static_cast<size_t>(gridDim.x) * (blockDim.x / 64);     // wavefronts in the grid
    const int lane = threadIdx.x & 63;
    size_t g = static_cast<size_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
    for (; g + (U - 1) * nw < ngroups; g += U * nw) {
        v4i r[U] = {};
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int u = 0; u < U; ++u)
                r[u] ^= __builtin_nontemporal_load(src + ((g + u * nw) * K + k) * 64 + lane);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(r[u], dst + (g + u * nw) * 64 + lane);
    }
    for (; g < ngroups; g += nw) {
        v4i r = {};
#pragma unroll
        for (int k = 0; k < K; ++k) r ^= __builtin_nontemporal_load(src + (g * K + k) * 64 + lane);
        __builtin_nontemporal_store(r, dst + g * 64 + lane);
    }
    const size_t rem = n - ngroups * 64;
    if (rem && blockIdx.x == 0 && threadIdx.x < rem) {
        v4i r = {};
#pragma unroll
        for (int k = 0; k < K; ++k) r ^= src[ngroups * 64 * K + k * rem + threadIdx.x];
        dst[ngroups * 64 + threadIdx.x] = r;
    }
}

template <int K>
void launch_probe(const void *src, void *dst, size_t n, hipStream_t stream)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    constexpr int U = K == 1 ? 4 : 8;
    DEER_LAUNCH((stream_probe_kernel<K, U>), dim3(static_cast<unsigned>(cus)), dim3(256), 0, stream,
                static_cast<const v4i *>(src), static_cast<v4i *>(dst), n);
}

}  // namespace
}  // namespace deer

extern "C" int deer_bandwidth_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes, void *stream)
{
    using namespace deer;
    if (dst_bytes == 0 && src_bytes == 0) return DEER_OK;
    if (!src || !dst) return fail(DEER_ERR_INVALID, "deer_bandwidth_probe: null pointer");
    if (dst_bytes == 0 || dst_bytes % 16 || src_bytes % dst_bytes || reinterpret_cast<uintptr_t>(src) % 16 ||
        reinterpret_cast<uintptr_t>(dst) % 16)
        return fail(DEER_ERR_INVALID,
                    "deer_bandwidth_probe: dst_bytes and the addresses must be multiples of 16 bytes and "
                    "src_bytes a multiple of dst_bytes");
    const size_t k = src_bytes / dst_bytes;
    if (k != 1 && k != 2 && k != 4 && k != 8)
        return fail(DEER_ERR_INVALID, "deer_bandwidth_probe: src_bytes / dst_bytes must be 1, 2, 4 or 8");
    const char *s = static_cast<const char *>(src);
    const char *d = static_cast<const char *>(dst);
    if (s < d + dst_bytes && d < s + src_bytes) return fail(DEER_ERR_INVALID, "deer_bandwidth_probe: buffers overlap");
    const size_t n = dst_bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (k) {
    case 1: launch_probe<1>(src, dst, n, st); break;
    case 2: launch_probe<2>(src, dst, n, st); break;
    case 4: launch_probe<4>(src, dst, n, st); break;
    default: launch_probe<8>(src, dst, n, st); break;
    }
    DEER_HIP(hipGetLastError());
    return DEER_OK;
}
