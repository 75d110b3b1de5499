// capi.hip -- library-wide entry points: version, status strings, the
// workspace fill, and the plain streaming read that serves as the measured
// HBM read ceiling.
#include "common.h"

namespace mv {

__global__ void fill_zero_kernel(u32x4 *__restrict__ p, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = u32x4{0, 0, 0, 0};
}

// A plain streaming read: grid-stride 16-byte non-temporal loads, eight in
// flight per thread; every 32-bit word is folded into a running XOR, so the
// loads cannot be dropped and the result can be checked. Workgroup b
// writes the XOR of the words it read to out[b].
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const u32x4 *__restrict__ src,
                                                                 size_t n,
                                                                 uint32_t *__restrict__ out)
{
    __shared__ uint32_t s_w[kProbeThreads / kWave];
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = load_stream(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = load_stream(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int m = kWave / 2; m >= 1; m >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, m);
    if ((threadIdx.x & (kWave - 1)) == 0)
        s_w[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kProbeThreads / kWave; ++w)
            t ^= s_w[w];
        out[blockIdx.x] = t;
    }
}

} // namespace mv

using namespace mv;

extern "C" int32_t moe_abi_version(void) { return 1; }

extern "C" const char *moe_status_str(moe_status_t s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "size out of range or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "size not supported by this library";
    case MOE_ERR_ALIGN: return "pointer not aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

extern "C" moe_status_t moe_workspace_clear(void *workspace, size_t bytes, void *stream)
{
    if (!workspace)
        return MOE_ERR_NULL;
    if (!aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (bytes % 16 != 0)
        return MOE_ERR_SHAPE;
    const size_t n = bytes / 16;
    if (n == 0)
        return MOE_OK;
    size_t grid = (n + 255) / 256;
    if (grid > 1024)
        grid = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, (u32x4 *)workspace, n);
    return check_launch();
}

extern "C" moe_status_t moe_hbm_read_probe(const void *src, size_t bytes, uint32_t *checksums,
                                           void *stream)
{
    if (!src || !checksums)
        return MOE_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0)
        return MOE_ERR_SHAPE;
    if (!aligned16(src) || !aligned4(checksums))
        return MOE_ERR_ALIGN;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(MOE_HBM_PROBE_GROUPS), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, (const u32x4 *)src, bytes / 16, checksums);
    return check_launch();
}
