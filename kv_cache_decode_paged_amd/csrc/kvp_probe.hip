// kvp_probe.hip -- achievable HBM read bandwidth: a plain streaming read of a buffer, the
// yardstick for the decode kernels' rates (decode is bound by the bytes it reads: neuralialabs
// "Tornar a inferencia barata", prefill vs decode passage).
//
// Each wave reads 16-byte vectors, 8 in flight per lane, striding over the buffer by the
// whole grid; the lanes fold what they read into a word that is stored only when it holds
// one fixed bit pattern, so the loads cannot be removed and nothing is written in practice.
#include <hip/hip_runtime.h>

#include "kvp_internal.h"

namespace kvp {

typedef int i32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const i32x4v *__restrict__ buf, long long n16,
                                                         int *__restrict__ sink)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    int acc = 0;
    // eight independent loads per trip keep 128 bytes per lane in flight
    for (; i + 7 * stride < n16; i += 8 * stride) {
        i32x4v a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            acc ^= a[k].x ^ a[k].y ^ a[k].z ^ a[k].w;
    }
    for (; i < n16; i += stride) {
        const i32x4v a = __builtin_nontemporal_load(buf + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x5eed1e55)
        sink[0] = acc;
}

} // namespace kvp

using namespace kvp;

extern "C" kvp_status kvp_read_bandwidth_probe(const void *d_buf, size_t bytes, int32_t waves, int32_t *d_sink,
                                               kvp_stream stream)
{
    if (!d_buf || !d_sink || bytes == 0 || (bytes & 15) || ((uintptr_t)d_buf & 15) || waves < 0)
        return fail(KVP_ERR_INVALID, "kvp_read_bandwidth_probe: bad arguments (buf %p, %zu bytes, %d waves)", d_buf,
                    bytes, waves);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                  hipSuccess)
        cus = 256; // the MI355X's compute units
    const long long w = waves > 0 ? waves : 8LL * cus;
    const long long blocks = (w + 3) / 4; // 4 waves of 64 lanes per workgroup
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const i32x4v *)d_buf, (long long)(bytes / 16), d_sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "kvp_read_bandwidth_probe: %s", hipGetErrorString(e));
    return KVP_OK;
}
