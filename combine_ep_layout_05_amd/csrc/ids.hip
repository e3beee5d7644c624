// ids.hip -- int64 expert ids to the int32 ids the layout kernels take
// (gfx950).  A framework's top-k returns int64 indices; the layouts read
// int32.  One grid-strided pass, 8 bytes read and 4 written per id.
#include <cstdint>

#include "ep_device.h"
#include "ep_launch.h"

namespace ep {
namespace {

// int64 expert ids -> the int32 ids every layout takes: a negative id (a
// dropped entry) becomes -1, one above INT32_MAX becomes INT32_MAX (at least
// E, so the layout reports it as bad), the rest keep their value.
__global__ __launch_bounds__(256) void idx_narrow_kernel(const int64_t* __restrict__ in, int64_t n,
                                                         int32_t* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride) {
        const int64_t v = in[j];
        out[j] = v < 0 ? -1 : (v > (int64_t)INT32_MAX ? INT32_MAX : (int32_t)v);
    }
}

}  // namespace

hipError_t launch_idx_narrow(const int64_t* in, int64_t n, int32_t* out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(idx_narrow_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, n, out);
    return hipGetLastError();
}

}  // namespace ep
