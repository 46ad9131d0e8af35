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
// Index arithmetic is 32-bit (the plan keeps N*C*P*Q below 2^30) with
// multiply-shift division.  A 3x3 window (AlexNet's) has an instance per
// mode with the window unrolled, so its nine loads (clamped to the plane's
// first element where they fall outside it) issue together and only the
// mode's own arithmetic runs; other windows loop.
//
// Parameters: x, its strides sx*; y, its strides sy*; N, C, H, W; window
// R x S; P, Q; u, v; pad_top, pad_left; M = N*P*Q; div_pq, div_q divide by
// P*Q and Q, div_rs by C and div_s by M; Kred = the mode (0 max, 1 average
// over R*S, 2 average over the positions inside).
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

// MODE: the pooling mode as a compile-time constant (0 max, 1 average over
// R*S, 2 average over the positions inside), or -1 to read it from Kred.
template <class In, class Acc, class Out, int RT, int ST, int MODE>
__global__ void __launch_bounds__(256) pool_fwd_kernel(const ConvParams p)
{
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
    if (idx >= (uint32_t)p.M * (uint32_t)p.C) return;
    // consecutive threads take consecutive outputs along y's unit stride
    uint32_t c, m;
    if (p.syk == 1)
        p.div_rs.divmod(idx, m, c);
    else
        p.div_s.divmod(idx, c, m);
    uint32_t n, pq, pp, q;
    p.div_pq.divmod(m, n, pq);
    p.div_q.divmod(pq, pp, q);
    const int h0 = (int)pp * p.u - p.pad_top;
    const int w0 = (int)q * p.v - p.pad_left;
    const In* x = static_cast<const In*>(p.x) + (int)n * p.sxn + (int)c * p.sxc;
    Acc best = 0, sum = 0;
    int inside = 0;
    // positions in row order; padding never counts, and max takes the first
    // inside value, then any larger one
    auto take = [&](Acc v) {
        best = (inside == 0 || v > best) ? v : best;
        sum += v;
        ++inside;
    };
    if constexpr (RT > 0) {
        // the window's rows and columns tested once each; a position outside
        // the plane reads x's first element and is left out by its mask
        uint32_t rok = 0, cok = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) rok |= ((unsigned)(h0 + r) < (unsigned)p.H ? 1u : 0u) << r;
#pragma unroll
        for (int s = 0; s < ST; ++s) cok |= ((unsigned)(w0 + s) < (unsigned)p.W ? 1u : 0u) << s;
        const In* xw = x + h0 * p.sxh + w0 * p.sxw;
        Acc vals[RT][ST];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int s = 0; s < ST; ++s) {
                const bool ok = ((rok >> r) & (cok >> s) & 1u) != 0;
                vals[r][s] = widen_pool((ok ? xw : x)[ok ? r * p.sxh + s * p.sxw : 0]);
            }
        if constexpr (MODE == 0) {
            // max: the first inside value, then any larger one
            bool any = false;
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int s = 0; s < ST; ++s) {
                    const bool ok = ((rok >> r) & (cok >> s) & 1u) != 0;
                    best = ok && (!any || vals[r][s] > best) ? vals[r][s] : best;
                    any = any || ok;
                }
            inside = any ? 1 : 0;
        } else if constexpr (MODE == 1 || MODE == 2) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int s = 0; s < ST; ++s) {
                    const bool ok = ((rok >> r) & (cok >> s) & 1u) != 0;
                    sum += ok ? vals[r][s] : Acc(0);
                }
            if constexpr (MODE == 2) inside = __builtin_popcount(rok) * __builtin_popcount(cok);
        } else {
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int s = 0; s < ST; ++s)
                    if (((rok >> r) & (cok >> s) & 1u) != 0) take(vals[r][s]);
        }
    } else {
        for (int r = 0; r < p.R; ++r) {
            const int h = h0 + r;
            if ((unsigned)h >= (unsigned)p.H) continue;
            for (int s = 0; s < p.S; ++s) {
                const int w = w0 + s;
                if ((unsigned)w >= (unsigned)p.W) continue;
                take(widen_pool(x[h * p.sxh + w * p.sxw]));
            }
        }
    }
    Acc acc;
    const int mode = MODE >= 0 ? MODE : p.Kred;
    if (mode == 0)
        acc = inside ? best : Acc(0);
    else if (mode == 1)
        acc = sum / (Acc)(p.R * p.S);
    else
        acc = inside ? sum / (Acc)inside : Acc(0);
    Out* y = static_cast<Out*>(p.y);
    const int off = (int)n * p.syn + (int)c * p.syk + (int)pp * p.syp + (int)q * p.syq;
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
    if (p.R == 3 && p.S == 3 && p.Kred == 0)
        hipLaunchKernelGGL((pool_fwd_kernel<In, Acc, Out, 3, 3, 0>), grid, dim3(256), 0, stream, p);
    else if (p.R == 3 && p.S == 3 && p.Kred == 1)
        hipLaunchKernelGGL((pool_fwd_kernel<In, Acc, Out, 3, 3, 1>), grid, dim3(256), 0, stream, p);
    else if (p.R == 3 && p.S == 3)
        hipLaunchKernelGGL((pool_fwd_kernel<In, Acc, Out, 3, 3, 2>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((pool_fwd_kernel<In, Acc, Out, 0, 0, -1>), grid, dim3(256), 0, stream, p);
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
