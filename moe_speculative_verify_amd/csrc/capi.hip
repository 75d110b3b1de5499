// capi.hip -- library-wide entry points: version, status strings and the
// workspace fill.
#include "common.h"

namespace mv {

__global__ void fill_zero_kernel(u32x4 *__restrict__ p, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = u32x4{0, 0, 0, 0};
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
