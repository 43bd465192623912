// Pooler distillation from dense attention, for gfx950 (RecSA, abstract, sentence
// on the pooler: each layer's pooler learns from full attention as its teacher).  Two small kernels of one
// training step; the step's other parts are the library's decode, backward and
// tree build.
//   loss = (1 / rows) sum ||out - teacher||^2,  dO = 2 (out - teacher) / rows;
//   vel <- mu vel + dw,  w <- w - lr vel  (SGD with momentum).
#include "recsa_internal.hpp"

namespace recsa {
namespace {

// One workgroup: the loss (a deterministic tree reduction) and dO.
__global__ __launch_bounds__(1024) void distill_loss_kernel(const float *out, const float *teacher,
                                                            float *dout, float *loss, int64_t n,
                                                            int64_t rows) {
    __shared__ float part[1024];
    const float inv = 1.f / (float)rows;
    float acc = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
        const float d = out[i] - teacher[i];
        dout[i] = 2.f * d * inv;
        acc += d * d;
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 512; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *loss = part[0] * inv;
}

__global__ void distill_update_kernel(float *w, float *vel, const float *dw, int64_t n, float lr,
                                      float mu) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float v = mu * vel[i] + dw[i];
        vel[i] = v;
        w[i] -= lr * v;
    }
}

}  // namespace

hipError_t launch_distill_loss(const float *out, const float *teacher, float *dout, float *loss,
                               int64_t n, int64_t rows, hipStream_t s) {
    hipLaunchKernelGGL(distill_loss_kernel, dim3(1), dim3(1024), 0, s, out, teacher, dout, loss, n, rows);
    return hipGetLastError();
}

hipError_t launch_distill_update(float *w, float *vel, const float *dw, int64_t n, float lr, float mu,
                                 hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(distill_update_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                       s, w, vel, dw, n, lr, mu);
    return hipGetLastError();
}

}  // namespace recsa
