// conv_fwd_direct.hip -- plain direct convolution, one thread per output.
//
// No tiling, no MFMA: each thread sums its receptive field times its filter
// (maxDNN page, "Proposed Method": an output coordinate is the receptive
// field times the filter) in the accumulation type.  It serves shapes and
// strides of any kind and is the library's variant of last resort; the
// MFMA variants are the fast path.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"

namespace miconv {

struct Bf16Bits { uint16_t bits; };

// Exact widening of one input element to the accumulation type.
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ double widen(double v) { return v; }
__device__ __forceinline__ float widen(Bf16Bits v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <class In, class Acc, class Out>
__global__ void __launch_bounds__(256) conv_fwd_direct_kernel(const ConvParams p)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * p.K) return;
    // consecutive threads take consecutive output rows m for one filter k
    const int k = (int)(idx / p.M);
    const int m = (int)(idx - (int64_t)k * p.M);
    uint32_t n, pq, pp, q;
    p.div_pq.divmod((uint32_t)m, n, pq);
    p.div_q.divmod(pq, pp, q);
    const int hb = (int)pp * p.u - p.pad_top;
    const int wb = (int)q * p.v - p.pad_left;
    const In* x = static_cast<const In*>(p.x);
    const In* w = static_cast<const In*>(p.w);
    const int rs = p.R * p.S;
    // filter F[k, c, tap] at wc + tap * wt: packed KCRS, or blocked
    // [K/kb][C/cb][R][S][cb][kb] (taps cb*kb apart)
    const int wt = p.wkb > 0 ? p.wcb * p.wkb : 1;
    Acc acc = 0;
    for (int c = 0; c < p.C; ++c) {
        const int xc = (int)n * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, c);
        const int wc = p.wkb > 0 ? wblk_off(k, c, 0, p.C, rs, p.wkb, p.wcb) : k * p.Kred + c * rs;
        for (int r = 0; r < p.R; ++r) {
            const int h = hb + r;
            if ((unsigned)h >= (unsigned)p.H) continue;
            for (int s = 0; s < p.S; ++s) {
                const int ww = wb + s;
                if ((unsigned)ww >= (unsigned)p.W) continue;
                const Acc xv = widen(x[xc + h * p.sxh + ww * p.sxw]);
                const Acc fv = widen(w[wc + (r * p.S + s) * wt]);
                acc += xv * fv;
            }
        }
    }
    Out* y = static_cast<Out*>(p.y);
    const int off = (int)n * p.syn + blk_off(p.div_ycb, p.sycb, p.syk, k) + (int)pp * p.syp + (int)q * p.syq;
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Acc val = alpha * acc;
    if (beta != Acc(0)) val += beta * (Acc)y[off];
    y[off] = (Out)val;
}

template <class In, class Acc, class Out>
static hipError_t launch_direct_t(const ConvParams& p, hipStream_t stream)
{
    const int64_t total = (int64_t)p.M * p.K;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL((conv_fwd_direct_kernel<In, Acc, Out>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_direct(DType dt, const ConvParams& p, hipStream_t stream)
{
    switch (dt) {
    case DType::F32: return launch_direct_t<float, float, float>(p, stream);
    case DType::F64: return launch_direct_t<double, double, double>(p, stream);
    case DType::BF16: return launch_direct_t<Bf16Bits, float, float>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace miconv
