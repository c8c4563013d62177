// Empty-tensor result: out = 0 and lse = +inf for every row.
// aclnnFusedInferAttentionScoreV4, Constraints, processing when the input parameter is
// empty: with key/value of zero elements the output is all 0 and the lse all inf.
// A plain kernel rather than hipMemsetAsync, so the op stays capture-friendly.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

__global__ void __launch_bounds__(256) fill_kernel(FillArgs a) {
    const int64_t row_elems = a.head_num * a.head_size;
    const int64_t total = a.n_tokens * row_elems;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += stride) {
        const int64_t t = i / row_elems, e = i - t * row_elems;
        const int64_t h = e / a.head_size, d = e - h * a.head_size;
        static_cast<uint16_t*>(a.out)[t * a.out_tok_stride + h * a.out_head_stride + d] = 0;  // +0.0
    }
    if (a.lse != nullptr) {
        const int64_t nl = a.n_tokens * a.head_num;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nl;
             i += stride) {
            const int64_t t = i / a.head_num, h = i - t * a.head_num;
            a.lse[t * a.lse_tok_stride + h] = INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_fill(const FillArgs& a, hipStream_t stream) {
    const int64_t total = a.n_tokens * a.head_num * a.head_size;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
