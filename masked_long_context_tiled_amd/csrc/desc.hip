// Column-interval mask descriptor on the device: one thread per key column runs the same
// per-column rule as the host builder (desc.h), so a step that rebuilds the descriptor needs
// no host work and no copy (the document boundaries, if any, are read from device memory).
#include "common.h"
#include "desc.h"

namespace mlct {

__global__ __launch_bounds__(256) void desc_kernel(attn_mask_params mp, int32_t T, int4* __restrict__ out) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= T) return;
    int32_t d[4];
    desc_column(&mp, T, 0, 0, T, j, d);
    out[j] = int4{d[0], d[1], d[2], d[3]};
}

int launch_desc(const attn_mask_params& mp, int32_t T, int32_t* desc, void* stream) {
    hipLaunchKernelGGL(desc_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       mp, T, reinterpret_cast<int4*>(desc));
    return (int)hipGetLastError();
}

}  // namespace mlct
