// conv_bwd_filter_rows.hip -- filter gradient of a first layer: few input
// channels, wide strided filter rows, a reduction over hundreds of
// thousands of output positions.
//
//   dw[k,c,r,s] = alpha * sum_{n,p,q} dy[n,k,p,q] * X(n, c, p*u + r - pad_top, q*v + s - pad_left)
//               + beta * dw[k,c,r,s]
//
// (the backward routine in F that the cuDNN page, "Proposed Method", lists
// beside the forward one).  Such a dw is small (32 x 1 x 41 x 11 for the
// speech network's first layer, 96 x 3 x 11 x 11 for Overfeat's), and with
// no workspace one workgroup must own each output it writes, so the matrix
// kernels' 16 x 16 or larger tiles leave most compute units idle.  Here a
// workgroup owns the KT x S outputs dw[k0 .. k0+KT-1, c, r, 0 .. S-1] of one
// channel and filter row, and reduces them on the vector ALU from output
// rows staged in LDS:
//
//  * its NW waves take the output rows (n, p) whose input row
//    p*u + r - pad_top lies inside x, in turn (wave w: rows w, w + NW, ...);
//  * per row a wave stages, in an LDS region of its own, dy[n, k0+kk, p, q]
//    for its KT filters and q < 64*NQ (zero past Q and K), and the input row
//    X(n, c, p*u + r - pad_top, col - pad_left) for col < 64*NX (zero outside
//    x), the latter split by column phase: column j*V + b at b*WPH + j, so
//    that lanes at consecutive q read consecutive words for every tap;
//  * lane l takes positions q = l + 64*j (j < NQ): KT dy values and S
//    input values from LDS, KT*S fused multiply-adds into registers;
//  * the next row's loads go to registers while the current row is
//    computed, and are written to the wave's region after it (the wave's
//    own LDS accesses complete in order, so no barrier is needed);
//  * at the end each wave adds its 64 lanes by a fixed butterfly and the
//    NW wave sums are added in wave order: the result does not depend on
//    timing.
//
// Parameters as in conv_bwd_filter.hip: x and its strides sx*; w = dy and
// its strides sd*; y = dw packed K,C,R,S; N, C, H, W, R, S, P, Q, u, v and
// the padding of the forward geometry; M = K.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"

namespace miconv {
namespace {

constexpr int kBufWord3 = 0x00020000;        // raw 32-bit buffer, range-checked per dword
constexpr int kOutside = (int)0x80000000u;   // an offset past any buffer here (rows are < 2^31 bytes)

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, kBufWord3);
}
__device__ __forceinline__ float row_load(__amdgpu_buffer_rsrc_t r, int voff)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

template <int KT, int S, int V, int NQ, int NX, int NW>
__global__ void __launch_bounds__(64 * NW)
conv_bwd_filter_rows_kernel(const ConvParams p)
{
    constexpr int KTP = (KT + 3) / 4 * 4;            // a lane's dy values, padded to whole 16-byte words
    constexpr int WPH = 64 * NX / V;                 // words per column phase
    constexpr int DY = NQ * 64 * KTP;                // staged dy words [j][lane][kk]
    constexpr int REGION = DY + 64 * NX;             // one wave's LDS words
    static_assert(64 % V == 0, "column phases of a 64-column load group");
    static_assert(64 * NQ - 1 + (S - 1) / V < WPH, "taps of the last position inside the staged row");
    static_assert((NW * REGION + NW * KT * S) * 4 <= 64 * 1024, "LDS");

    __shared__ __attribute__((aligned(16))) float stage[NW * REGION];
    __shared__ float wsum[NW * KT * S];

    const int lane = threadIdx.x & 63;
    // wave-uniform, so that the row and its buffer descriptors live in scalar
    // registers (a descriptor the compiler cannot prove uniform costs a loop
    // over the lanes around every load)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float* const dys = stage + wave * REGION;
    float* const xs = dys + DY;

    // tile = (k block, c, r), consecutive tiles share dy's k block
    const int ncr = p.C * p.R;
    const int tile = (int)blockIdx.x;
    const int kb = tile / ncr;
    const int cr = tile - kb * ncr;
    const int c = cr / p.R;
    const int r = cr - c * p.R;
    const int k0 = kb * KT;

    // output rows p whose input row p*u + r - pad_top is inside x
    const int off = r - p.pad_top;                   // input row = p*u + off
    const int p_lo = off >= 0 ? 0 : (-off + p.u - 1) / p.u;
    const int p_hi = min(p.P - 1, (p.H - 1 - off) >= 0 ? (p.H - 1 - off) / p.u : -1);
    const int pv = p_hi >= p_lo ? p_hi - p_lo + 1 : 0;
    const int nrows = p.N * pv;

    const float* __restrict__ x = static_cast<const float*>(p.x);
    const float* __restrict__ dy = static_cast<const float*>(p.w);

    // Loads through one range-checked buffer per staged row (unit stride
    // along q and w): dy row (n, k0+kk, p) of Q words, none past K; x row
    // (n, c, h) of W words.  Offsets past a row read zero, so positions
    // q >= Q and columns outside x need no select.  Column col - pad_left of
    // group i is at byte 4*(lane + 64 i - pad_left); only group 0 can be left
    // of the row (pad_left < 64), and goes to kOutside there.
    const int dq_bytes = 4 * p.Q;
    const int x_bytes = 4 * p.W;
    const int dv0 = 4 * lane;
    const int xv0 = lane >= p.pad_left ? 4 * (lane - p.pad_left) : kOutside;
    const int xv1 = 4 * (lane + 64 - p.pad_left);
    const int x_dst = (lane % V) * WPH + lane / V;   // LDS word of column lane (+ 64/V per group i)

    float dv[KT][NQ], xv[NX];
    auto load_row = [&](int t) {
        const int n = t / pv;
        const int pp = p_lo + (t - n * pv);
        const float* drow = dy + (n * p.sdn + pp * p.sdp + k0 * p.sdk);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            const __amdgpu_buffer_rsrc_t dr = row_rsrc(drow + kk * p.sdk, k0 + kk < p.M ? dq_bytes : 0);
#pragma unroll
            for (int j = 0; j < NQ; ++j) dv[kk][j] = row_load(dr, dv0 + 256 * j);
        }
        const __amdgpu_buffer_rsrc_t xr = row_rsrc(x + (n * p.sxn + c * p.sxc + (pp * p.u + off) * p.sxh), x_bytes);
        xv[0] = row_load(xr, xv0);
#pragma unroll
        for (int i = 1; i < NX; ++i) xv[i] = row_load(xr, xv1 + 256 * (i - 1));
    };
    auto store_row = [&]() {
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int v4 = 0; v4 < KTP / 4; ++v4) {
                f32x4v w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = 4 * v4 + e < KT ? dv[4 * v4 + e][j] : 0.0f;
                *reinterpret_cast<f32x4v*>(dys + (j * 64 + lane) * KTP + 4 * v4) = w;
            }
#pragma unroll
        for (int i = 0; i < NX; ++i) xs[x_dst + (64 / V) * i] = xv[i];
    };

    float acc[KT][S];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk)
#pragma unroll
        for (int s = 0; s < S; ++s) acc[kk][s] = 0.0f;

    int t = wave;
    if (t < nrows) load_row(t);
    for (; t < nrows; t += NW) {
        store_row();
        if (t + NW < nrows) load_row(t + NW);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float d[KTP];
#pragma unroll
            for (int v4 = 0; v4 < KTP / 4; ++v4) {
                const f32x4v w = *reinterpret_cast<const f32x4v*>(dys + (j * 64 + lane) * KTP + 4 * v4);
#pragma unroll
                for (int e = 0; e < 4; ++e) d[4 * v4 + e] = w[e];
            }
            const int q = lane + 64 * j;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float xq = xs[(s % V) * WPH + q + s / V];
#pragma unroll
                for (int kk = 0; kk < KT; ++kk) acc[kk][s] = __builtin_fmaf(d[kk], xq, acc[kk][s]);
            }
        }
    }

    // lanes of a wave by a fixed butterfly, then the waves in order
#pragma unroll
    for (int kk = 0; kk < KT; ++kk)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            float v = acc[kk][s];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
            acc[kk][s] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int s = 0; s < S; ++s) wsum[wave * KT * S + kk * S + s] = acc[kk][s];
    }
    __syncthreads();
    float* __restrict__ dw = static_cast<float*>(p.y);
    for (int e = (int)threadIdx.x; e < KT * S; e += 64 * NW) {
        const int kk = e / S, s = e - (e / S) * S;
        if (k0 + kk >= p.M || s >= p.S) continue;
        float sum = 0.0f;
        for (int w = 0; w < NW; ++w) sum += wsum[w * KT * S + e];
        const int o = (k0 + kk) * p.syn + (c * p.R + r) * p.S + s;
        float val = (float)p.alpha * sum;
        if (p.beta != 0.0) val += (float)p.beta * dw[o];
        dw[o] = val;
    }
}

// instance: KT filters, S taps, column stride V, positions q < 64*NQ,
// staged columns 64*NX, NW waves
template <int KT, int S, int V, int NQ, int NX, int NW>
bool rows_fits(const ConvParams& p)
{
    // unit stride along q and w (one buffer per row), left padding inside
    // the first 64-column group
    return p.S == S && p.v == V && p.Q <= 64 * NQ && (int64_t)(p.Q - 1) * V + S <= 64 * NX && p.sdq == 1 &&
           p.sxw == 1 && p.pad_left < 64;
}

template <int KT, int S, int V, int NQ, int NX, int NW>
hipError_t rows_launch(const ConvParams& p, hipStream_t stream)
{
    if (!rows_fits<KT, S, V, NQ, NX, NW>(p)) return hipErrorInvalidValue;
    const int64_t tiles = (int64_t)((p.M + KT - 1) / KT) * p.C * p.R;
    if (tiles <= 0 || tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv_bwd_filter_rows_kernel<KT, S, V, NQ, NX, NW>), dim3((unsigned)tiles),
                       dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

//                name               KT  S  V NQ NX NW
#define MICONV_WGR_VARIANTS(X)                  \
    X(WGR_F32_S11_V2, 3, 11, 2, 6, 13, 4)       \
    X(WGR_F32_S11_V4, 7, 11, 4, 1, 5, 4)

bool bwd_filter_rows_fits(Variant v, const ConvParams& p)
{
    switch (v) {
#define X(name, kt, s, vv, nq, nx, nw) \
    case Variant::name: return rows_fits<kt, s, vv, nq, nx, nw>(p);
        MICONV_WGR_VARIANTS(X)
#undef X
    default: return false;
    }
}

hipError_t launch_bwd_filter_rows(Variant v, const ConvParams& p, hipStream_t stream)
{
    switch (v) {
#define X(name, kt, s, vv, nq, nx, nw) \
    case Variant::name: return rows_launch<kt, s, vv, nq, nx, nw>(p, stream);
        MICONV_WGR_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
