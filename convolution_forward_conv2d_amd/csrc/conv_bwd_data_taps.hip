// conv_bwd_data_taps.hip -- data gradient of a strided layer onto few input
// channels (a first layer: the speech network's 41 x 11 bank at stride 2 onto
// one channel) on gfx950 MFMA, with the filter's column taps as the GEMM's
// columns.
//
//   dx[n,c,h,w] = alpha * sum_{k,r,s: h + pt - r = u p, w + pl - s = v q} dy[n,k,p,q] * F[k,c,r,s] + beta * dx
//
// (the backward routine in x that the cuDNN page, "Proposed Method", lists
// beside the forward one; the maxDNN page, Abstract and RQ4, expects the
// forward techniques to carry over to it).  Onto one channel the usual
// implicit GEMM has a single column; here the columns are the S taps of a
// filter row instead.  For the row phase a = (h + pt) mod u, with
// h + pt = u P' + a, the rows reaching h are r = a + u i at p = P' - i, so
//
//   Z[P', q, s] = sum_k sum_i dy[n, k, P' - i, q] * F[k, c, a + u i, s]
//   dx[n, c, h, w] = sum over s with (w + pl - s) = v q, 0 <= q < Q, of Z[P', q, s]
//
// Z is an implicit GEMM -- rows (P', q), columns s, reduction (k, i) -- whose
// operands are plain dy rows and filter taps; the second sum, a handful of
// terms per output, runs from LDS in the epilogue.  No multiply-add falls off
// the stride grid; the waste is the column padding (S of 16) and the rows'
// q padding to whole 16-blocks.
//
// A workgroup takes one image n, channel c, phase a and a band of TB
// consecutive phase rows P'.  The reduction runs channel by channel of dy:
// a chunk stages the TB + 4*IS - 1 dy rows P'_0 + TB - 1 - i (zeros outside
// dy) of QP = 16*QB columns in LDS, double-buffered; 16x16x4 fp32 MFMA blocks
// (PolF32x16), the four lane groups taking four consecutive i, each lane's
// filter tap F[k, c, a + u i, s] read straight from memory (zero for i past
// the phase's taps or s past S).  The 4 waves split the TB * QB row blocks.
//
// Parameters (direct layout, as conv_bwd_data_phase.hip): x = dy and its
// strides sx*, w = F (packed K,C,R,S), y = dx and its strides sy*; N, C, H, W
// dx's dims; K, P, Q dy's; R, S, u, v, pad_top, pad_left the forward
// geometry.  The host checks: fp32, S <= 16, Q <= QP, ceil(R/u) <= 4*IS.
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

namespace {
constexpr int kTapsBufWord3 = 0x00020000;         // raw 32-bit buffer, range-checked per dword
constexpr int kTapsOutside = (int)0x80000000u;    // an offset past dy and F (both under 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t taps_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kTapsBufWord3);
}
template <class T>
__device__ __forceinline__ T taps_load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    if constexpr (std::is_same<T, float4>::value) {
        typedef unsigned int u4 __attribute__((ext_vector_type(4)));
        const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
    } else if constexpr (std::is_same<T, float2>::value) {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return float2{__uint_as_float(v[0]), __uint_as_float(v[1])};
    } else {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
}

// dy's and the filters' element counts
__host__ __device__ __forceinline__ int64_t taps_dy_elems(const ConvParams& p)
{
    return (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.K - 1) * p.sxc + (int64_t)(p.P - 1) * p.sxh +
           (int64_t)(p.Q - 1) * p.sxw + 1;
}
__host__ __device__ __forceinline__ int64_t taps_f_elems(const ConvParams& p)
{
    return (int64_t)p.K * p.C * p.R * p.S;
}
}  // namespace

// V: dy values per staging load (1, 2 or 4 consecutive columns; V > 1 needs
// unit column stride, Q and the row, channel and image strides multiples of
// V and dy's address aligned to V values)
template <int TB, int QB, int IS, int V>
__global__ void __launch_bounds__(256)
conv_bwd_data_taps_kernel(const ConvParams p, int bands)
{
    using Pol = PolF32x16;
    using AccV = Pol::AccV;
    constexpr int NT = 256;
    constexpr int QP = 16 * QB;                  // staged columns per dy row
    constexpr int NI = 4 * IS;                   // taps i per chunk (zero past the phase's)
    constexpr int ROWS = TB + NI - 1;            // staged dy rows per chunk
    constexpr int BUF = ROWS * QP;               // floats
    constexpr int NBLK = TB * QB;                // 16-row blocks of the tile
    constexpr int FM = (NBLK + 3) / 4;           // blocks per wave
    constexpr int NU = BUF / V;                  // staging units of V columns per chunk
    constexpr int NL = (NU + NT - 1) / NT;       // staging units per thread per chunk
    static_assert(QP % V == 0, "whole units per staged row");
    constexpr int ZP = 17;                       // epilogue: floats per (P', q) row of Z (16 taps + pad)
    constexpr int ZR0 = 2 * BUF / (QP * ZP);     // phase rows of Z the chunk buffers hold
    constexpr int ZR = ZR0 < TB ? ZR0 : TB;
    static_assert(ZR >= 1, "one phase row of Z fits in the chunk buffers");
    static_assert(NL <= 64, "staging mask");

    __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // workgroup -> (band, phase a, channel c, image n), band fastest, in runs
    // of consecutive ids per XCD: the bands of one phase, which stage
    // overlapping dy rows, share an L2
    int bid = xcd_logical_tile((int)blockIdx.x, (int)gridDim.x, p.tile_rev);
    const int band = bid % bands;
    bid /= bands;
    const int a = bid % p.u;
    bid /= p.u;
    const int c = bid % p.C;
    const int n = bid / p.C;
    // phase rows P' of dx rows h = u P' + a - pt inside [0, H)
    const int h_first = ((a - p.pad_top) % p.u + p.u) % p.u;     // smallest h >= 0 of the phase
    if (h_first >= p.H) return;
    const int P_lo = (h_first + p.pad_top - a) / p.u;
    const int P_hi = (p.H - 1 - ((p.H - 1 - h_first) % p.u) + p.pad_top - a) / p.u;
    const int P0 = P_lo + band * TB;
    if (P0 > P_hi) return;                        // uniform: the band lies past the phase's rows
    const int Ia = (p.R - a + p.u - 1) / p.u;     // taps i of the phase (a + u i < R)

    // Loads go through range-checked buffer descriptors: a unit outside dy,
    // or a tap past the filter, reads past the buffer and gets zero, so the
    // stores and products need no masks; channel k is the scalar offset.
    const __amdgpu_buffer_rsrc_t dr = taps_rsrc(p.x, 4 * taps_dy_elems(p));
    const __amdgpu_buffer_rsrc_t fr = taps_rsrc(p.w, 4 * taps_f_elems(p));

    // ---- staging: unit e = (staged row j, columns q ... q + V - 1): dy row
    // P0 + TB - 1 - j (the host keeps Q a multiple of V: a unit lies in one row)
    using VT = typename std::conditional<V == 4, float4, typename std::conditional<V == 2, float2, float>::type>::type;
    int st_voff[NL];                              // byte offset in dy at channel 0
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = tid + NT * i;
        const int j = e / (QP / V);
        const int q = V * (e - j * (QP / V));
        const int prow = P0 + TB - 1 - j;
        const bool ok = e < NU && prow >= 0 && prow < p.P && q < p.Q;
        st_voff[i] = ok ? 4 * (n * p.sxn + prow * p.sxh + q * p.sxw) : kTapsOutside;
    }
    VT sv[NL];
    auto load_chunk = [&](int k) {
#pragma unroll
        for (int i = 0; i < NL; ++i) sv[i] = taps_load<VT>(dr, st_voff[i], 4 * k * p.sxc);
    };
    auto store_chunk = [&](int buf) {
        VT* dst = reinterpret_cast<VT*>(smem + buf * BUF);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int e = tid + NT * i;
            if (NU % NT == 0 || e < NU) dst[e] = sv[i];
        }
    };

    // ---- MFMA geometry: wave w takes blocks w, w + 4, ... of the TB x QB grid;
    // lane l: A row (position) l % 16 of the block, lane group g = l / 16 takes tap i = 4t + g
    const int g = lane >> 4;
    const int l16 = lane & 15;
    int a_base[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int b = wave + 4 * f;
        const int pb = b / QB;                    // phase row within the band
        const int qb = b - pb * QB;
        // staged row of (P0 + pb) - i is TB - 1 - pb + i
        a_base[f] = (b < NBLK ? (TB - 1 - pb + g) * QP + qb * 16 + l16 : 0);
    }
    // B: F[k, c, a + u i, s] with i = 4t + g and s = l16 (zero past the taps)
    const bool s_ok = l16 < p.S;
    int b_voff[IS];                               // byte offset in F at k = 0
#pragma unroll
    for (int t = 0; t < IS; ++t) {
        const int i = 4 * t + g;
        const int r = a + p.u * i;
        const bool ok = s_ok && i < Ia && r < p.R;
        b_voff[t] = ok ? 4 * ((c * p.R + r) * p.S + l16) : kTapsOutside;
    }
    const int fk = p.C * p.R * p.S;               // filter stride between k

    AccV acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = AccV{};

    float bv[IS];
    auto load_b = [&](int k) {
#pragma unroll
        for (int t = 0; t < IS; ++t) bv[t] = taps_load<float>(fr, b_voff[t], 4 * k * fk);
    };
    auto blk_ok = [&](int f) { return NBLK % 4 == 0 || wave + 4 * f < NBLK; };

    load_chunk(0);
    store_chunk(0);
    load_b(0);
    __syncthreads();
    for (int k = 0; k < p.K; ++k) {
        const int cur = k & 1;
        const bool more = k + 1 < p.K;
        load_chunk(more ? k + 1 : k);
        const float* buf = smem + cur * BUF;
        float bcur[IS];
#pragma unroll
        for (int t = 0; t < IS; ++t) bcur[t] = bv[t];
        load_b(more ? k + 1 : k);
        // keep the next chunk's loads ahead of this chunk's products
        __builtin_amdgcn_sched_barrier(0);
        // operands of step t + 1 read from LDS while step t's products issue
        float av[FM], an[FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) av[f] = blk_ok(f) ? buf[a_base[f]] : 0.0f;
#pragma unroll
        for (int t = 0; t < IS; ++t) {
            if (t + 1 < IS) {
#pragma unroll
                for (int f = 0; f < FM; ++f) an[f] = blk_ok(f) ? buf[a_base[f] + 4 * (t + 1) * QP] : 0.0f;
            }
#pragma unroll
            for (int f = 0; f < FM; ++f)
                if (blk_ok(f)) acc[f] = Pol::mfma_s(av[f], bcur[t], acc[f]);
            if (t + 1 < IS) {
#pragma unroll
                for (int f = 0; f < FM; ++f) av[f] = an[f];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) store_chunk(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: Z -> LDS as [pb][q][s] (17 floats per (pb, q)), ZR phase
    // rows at a time, then each output of those rows sums its taps
    float* Z = smem;
    float* dx = static_cast<float*>(p.y);
    const float alpha = (float)p.alpha;
    const float beta = (float)p.beta;
#pragma unroll
    for (int pb0 = 0; pb0 < TB; pb0 += ZR) {
        if (pb0 > 0) __syncthreads();             // the previous rows' sums are read
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const int b = wave + 4 * f;
            const int pb = b / QB;
            if (b < NBLK && pb >= pb0 && pb < pb0 + ZR) {
                const int qb = b - pb * QB;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = Pol::row(e, lane);          // position within the block
                    const int s = Pol::col(e, lane);          // tap
                    Z[((pb - pb0) * QP + qb * 16 + m) * ZP + s] = acc[f][e];
                }
            }
        }
        __syncthreads();
        const int nr = min(ZR, TB - pb0);
        for (int e = tid; e < nr * p.W; e += NT) {
            const int zr = e / p.W;
            const int w = e - zr * p.W;
            const int Pp = P0 + pb0 + zr;
            const int h = p.u * Pp + a - p.pad_top;
            if (Pp > P_hi || h < 0 || h >= p.H) continue;
            const int wp = w + p.pad_left;
            float sum = 0.0f;
            // taps s = wp - v q for q = floor(wp / v) down to the first with s >= S
            for (int q = wp / p.v; q >= 0; --q) {
                const int s = wp - p.v * q;
                if (s >= p.S) break;
                if (q < p.Q) sum += Z[(zr * QP + q) * ZP + s];
            }
            float* o = dx + (int64_t)n * p.syn + (int64_t)c * p.syk + (int64_t)h * p.syp + (int64_t)w * p.syq;
            *o = beta != 0.0f ? alpha * sum + beta * *o : alpha * sum;
        }
    }
}

// phase rows of the phase with the most rows (bands per phase)
static int taps_rows_per_phase(const ConvParams& p)
{
    return (p.H + p.u - 1) / p.u;
}

constexpr int kTapsTB = 2, kTapsQB = 22, kTapsIS = 6;

bool bwd_data_taps_fits(const ConvParams& p)
{
    return p.S <= 16 && p.Q <= 16 * kTapsQB && (p.R + p.u - 1) / p.u <= 4 * kTapsIS && p.K >= 1 && p.v >= 1 &&
           p.u >= 1 && 4 * taps_dy_elems(p) < ((int64_t)1 << 31) && 4 * taps_f_elems(p) < ((int64_t)1 << 31);
}

// dy values per staging load: V consecutive columns at V-aligned addresses
static int taps_vector_width(const ConvParams& p)
{
    for (int v = 4; v > 1; v /= 2)
        if (p.sxw == 1 && p.Q % v == 0 && p.sxh % v == 0 && p.sxc % v == 0 && p.sxn % v == 0 &&
            reinterpret_cast<uintptr_t>(p.x) % (4 * v) == 0)
            return v;
    return 1;
}

template <int V>
static void launch_taps_v(const ConvParams& p, int bands, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((conv_bwd_data_taps_kernel<kTapsTB, kTapsQB, kTapsIS, V>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p, bands);
}

hipError_t launch_bwd_data_taps(const ConvParams& p, hipStream_t stream)
{
    if (!bwd_data_taps_fits(p)) return hipErrorInvalidValue;
    const int bands = (taps_rows_per_phase(p) + kTapsTB - 1) / kTapsTB;
    const int64_t grid = (int64_t)p.N * p.C * p.u * bands;
    if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (taps_vector_width(p)) {
    case 4: launch_taps_v<4>(p, bands, grid, stream); break;
    case 2: launch_taps_v<2>(p, bands, grid, stream); break;
    default: launch_taps_v<1>(p, bands, grid, stream); break;
    }
    return hipGetLastError();
}

}  // namespace miconv
