// pool_fwd.hip -- pooling forward pass: one thread per output element.
//
//   max:                  y = alpha * max over the window positions inside the plane + beta * y
//   average (with pad):   y = alpha * (sum inside) / (R * S)                        + beta * y
//   average (no pad):     y = alpha * (sum inside) / (positions inside)             + beta * y
//
// (cuDNN page, "Proposed Method": pooling among the library's forward
// routines; the window geometry is the convolution's: R x S window, strides
// u, v, per-side zero padding, floor output size.)  Padding never wins a
// max; a window with no position inside gives 0.  The pass is bound by HBM
// bandwidth: x is read once from memory (overlapping windows hit in cache)
// and y written once.  Consecutive threads take consecutive outputs along
// y's unit stride: along q, or along c for channels-innermost y.
//
// Parameters: x, its strides sx*; y, its strides sy*; N, C, H, W; window
// R x S; P, Q; u, v; pad_top, pad_left; M = N*P*Q; div_pq, div_q divide by
// P*Q and Q; Kred = the mode (0 max, 1 average over R*S, 2 average over the
// positions inside).
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"

namespace miconv {

namespace {

struct Bf16Pool { uint16_t bits; };

__device__ __forceinline__ float widen_pool(float v) { return v; }
__device__ __forceinline__ double widen_pool(double v) { return v; }
__device__ __forceinline__ float widen_pool(Bf16Pool v) { return __uint_as_float((uint32_t)v.bits << 16); }

}  // namespace

template <class In, class Acc, class Out>
__global__ void __launch_bounds__(256) pool_fwd_kernel(const ConvParams p)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * p.C) return;
    int c, m;
    if (p.syk == 1) {
        m = (int)(idx / p.C);
        c = (int)(idx - (int64_t)m * p.C);
    } else {
        c = (int)(idx / p.M);
        m = (int)(idx - (int64_t)c * p.M);
    }
    uint32_t n, pq, pp, q;
    p.div_pq.divmod((uint32_t)m, n, pq);
    p.div_q.divmod(pq, pp, q);
    const int h0 = (int)pp * p.u - p.pad_top;
    const int w0 = (int)q * p.v - p.pad_left;
    const In* x = static_cast<const In*>(p.x) + (int)n * p.sxn + c * p.sxc;
    Acc best = 0, sum = 0;
    int inside = 0;
    for (int r = 0; r < p.R; ++r) {
        const int h = h0 + r;
        if ((unsigned)h >= (unsigned)p.H) continue;
        for (int s = 0; s < p.S; ++s) {
            const int w = w0 + s;
            if ((unsigned)w >= (unsigned)p.W) continue;
            const Acc v = widen_pool(x[h * p.sxh + w * p.sxw]);
            best = (inside == 0 || v > best) ? v : best;
            sum += v;
            ++inside;
        }
    }
    Acc acc;
    if (p.Kred == 0)
        acc = inside ? best : Acc(0);
    else if (p.Kred == 1)
        acc = sum / (Acc)(p.R * p.S);
    else
        acc = inside ? sum / (Acc)inside : Acc(0);
    Out* y = static_cast<Out*>(p.y);
    const int off = (int)n * p.syn + c * p.syk + (int)pp * p.syp + (int)q * p.syq;
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Acc val = alpha * acc;
    if (beta != Acc(0)) val += beta * (Acc)y[off];
    y[off] = (Out)val;
}

template <class In, class Acc, class Out>
static hipError_t launch_pool_t(const ConvParams& p, hipStream_t stream)
{
    const int64_t total = (int64_t)p.M * p.C;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL((pool_fwd_kernel<In, Acc, Out>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_pool_forward(DType dt, const ConvParams& p, hipStream_t stream)
{
    switch (dt) {
    case DType::F32: return launch_pool_t<float, float, float>(p, stream);
    case DType::F64: return launch_pool_t<double, double, double>(p, stream);
    case DType::BF16: return launch_pool_t<Bf16Pool, float, float>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace miconv
