// conv_bwd_data.hip -- data gradient of the convolution (backward pass with
// respect to x), plain direct form: one thread per dx element.
//
//   dx[n,c,h,w] = alpha * sum over k, and the (p, r), (q, s) pairs with
//                 p*u + r - pad_top = h and q*v + s - pad_left = w
//                 (0 <= p < P, 0 <= r < R, 0 <= q < Q, 0 <= s < S),
//                 of dy[n,k,p,q] * F[k,c,r,s]
//               + beta * dx[n,c,h,w]
//
// the adjoint of the forward sum in x (the cuDNN page, "Proposed Method",
// names forward and backward routines; the maxDNN page, Abstract and RQ4,
// expects its forward techniques to carry over to the backward pass).  For a
// given h the contributing rows p run over an interval, so no division by
// the stride happens per term.  This kernel serves every shape, stride and
// type; stride-1 problems of the halo shapes take the tap-batched MFMA
// kernels instead (conv_fwd_halo.hip, filter read flipped and transposed).
//
// Parameters come in a ConvParams laid out for this direction: x = dy with
// sx* its (n, k, p, q) strides, y = dx with sy* its (n, c, h, w) strides;
// N, C, H, W are dx's dims, P, Q dy's; M = N*H*W; div_pq divides by H*W and
// div_q by W; Kred = C*R*S (one filter's length).
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"

namespace miconv {

namespace {

struct Bf16Raw { uint16_t bits; };

__device__ __forceinline__ float widen_dg(float v) { return v; }
__device__ __forceinline__ double widen_dg(double v) { return v; }
__device__ __forceinline__ float widen_dg(Bf16Raw v) { return __uint_as_float((uint32_t)v.bits << 16); }

// rows p (and taps r = i + pad - p*stride) that reach input row i:
// p in [lo, hi], both clipped to [0, n_out - 1]
__device__ __forceinline__ void contrib_range(int i, int pad, int f, int stride, int n_out, int& lo, int& hi)
{
    const int top = i + pad;                 // r = top - p*stride must lie in [0, f)
    const int first = top - (f - 1);
    lo = first <= 0 ? 0 : (first + stride - 1) / stride;
    hi = top < 0 ? -1 : top / stride;
    if (hi > n_out - 1) hi = n_out - 1;
}

}  // namespace

template <class In, class Acc, class Out>
__global__ void __launch_bounds__(256) conv_bwd_data_direct_kernel(const ConvParams p)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * p.C) return;
    // consecutive threads take consecutive (n, h, w) rows for one channel c,
    // or, when dx is channel-innermost, consecutive channels of one row: the
    // stores run along dx's unit stride and the threads of a row share dy
    int c, m;
    if (p.syk == 1) {
        m = (int)(idx / p.C);
        c = (int)(idx - (int64_t)m * p.C);
    } else {
        c = (int)(idx / p.M);
        m = (int)(idx - (int64_t)c * p.M);
    }
    uint32_t n, hw, h, w;
    p.div_pq.divmod((uint32_t)m, n, hw);
    p.div_q.divmod(hw, h, w);
    int p_lo, p_hi, q_lo, q_hi;
    contrib_range((int)h, p.pad_top, p.R, p.u, p.P, p_lo, p_hi);
    contrib_range((int)w, p.pad_left, p.S, p.v, p.Q, q_lo, q_hi);
    const In* dy = static_cast<const In*>(p.x);
    const In* f = static_cast<const In*>(p.w);
    Acc acc = 0;
    for (int k = 0; k < p.K; ++k) {
        const In* fk = f + ((size_t)k * p.C + c) * (p.R * p.S);
        const In* dyk = dy + (int)n * p.sxn + k * p.sxc;
        for (int pp = p_lo; pp <= p_hi; ++pp) {
            const int r = (int)h + p.pad_top - pp * p.u;
            for (int qq = q_lo; qq <= q_hi; ++qq) {
                const int s = (int)w + p.pad_left - qq * p.v;
                acc += widen_dg(dyk[pp * p.sxh + qq * p.sxw]) * widen_dg(fk[r * p.S + s]);
            }
        }
    }
    Out* dx = static_cast<Out*>(p.y);
    const int off = (int)n * p.syn + c * p.syk + (int)h * p.syp + (int)w * p.syq;
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Acc val = alpha * acc;
    if (beta != Acc(0)) val += beta * (Acc)dx[off];
    dx[off] = (Out)val;
}

template <class In, class Acc, class Out>
static hipError_t launch_t(const ConvParams& p, hipStream_t stream)
{
    const int64_t total = (int64_t)p.M * p.C;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL((conv_bwd_data_direct_kernel<In, Acc, Out>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_data_direct(DType dt, const ConvParams& p, hipStream_t stream)
{
    switch (dt) {
    case DType::F32: return launch_t<float, float, float>(p, stream);
    case DType::F64: return launch_t<double, double, double>(p, stream);
    case DType::BF16: return launch_t<Bf16Raw, float, float>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace miconv
