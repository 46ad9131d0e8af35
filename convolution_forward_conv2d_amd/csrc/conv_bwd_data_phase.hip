// conv_bwd_data_phase.hip -- data gradient onto few channels (a network's
// first layer: 1-4 input channels under a large, strided filter bank).
//
//   dx[n,c,h,w] = alpha * sum over k, and the (p, r), (q, s) pairs with
//                 p*u + r = h + pad_top and q*v + s = w + pad_left,
//                 of dy[n,k,p,q] * F[k,c,r,s]
//               + beta * dx[n,c,h,w]
//
// (the backward routine in x that the cuDNN page, "Proposed Method", lists
// beside the forward one).  With one to four output channels a matrix-core
// tile would be almost empty in that dimension, so this kernel uses the
// vector ALU, organised by stride phase: for a = (h + pad_top) mod u and
// b = (w + pad_left) mod v the contributing taps are r = a + i*u and
// s = b + t*v, with p = P0(h) - i and q = Q0(w) - t where
// P0 = (h + pad_top - a) / u, Q0 = (w + pad_left - b) / v.  A workgroup
// works on one phase pair (a, b) -- grid.y -- so the filter values of every
// step are the same for all its lanes and come in as scalar loads.  A lane
// owns one output row h of that phase and WT consecutive positions of the
// phase along w (w = w0 + v*j), for all C channels: per filter k and tap row
// i it loads the WT + NSM - 1 dy values its positions reach (a sliding
// window along q) once and makes C * WT * NSM multiply-adds from them.
//
// Loads are range-checked buffer loads: a dy row outside [0, P) reads from
// an offset past the tensor and gets zero; window positions outside
// [0, Q) are zeroed by a select that is fixed for the lane.  Taps t with
// b + t*v >= S contribute a zero filter value.
//
// Parameters in the direct kernel's layout (conv_bwd_data.hip): x = dy with
// sx* its (n, k, p, q) strides, y = dx with sy* its (n, c, h, w) strides,
// w = F packed K,C,R,S; N, C, H, W are dx's dims, K, P, Q dy's.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"

namespace miconv {

namespace {

constexpr int kBufWord3 = 0x00020000;        // raw 32-bit buffer, range-checked
constexpr int kOutside = (int)0x80000000u;    // an offset past any dy under 1 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dg_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}
__device__ __forceinline__ float dg_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, float)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ double dg_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, double)
{
    typedef unsigned int u32x2_t __attribute__((__vector_size__(2 * sizeof(unsigned int))));
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return __hiloint2double((int)v[1], (int)v[0]);
}

// first index >= 0 of the phase class: (i + pad) mod stride == ph
__device__ __forceinline__ int phase_first(int ph, int pad, int stride)
{
    return ((ph - pad) % stride + stride) % stride;
}

}  // namespace

template <class T, int CT, int NSM, int WT>
__global__ void __launch_bounds__(256) conv_bwd_data_phase_kernel(const ConvParams p)
{
    constexpr int ES = (int)sizeof(T);
    constexpr int NWIN = WT + NSM - 1;
    const int u = p.u, v = p.v;
    const int a = (int)blockIdx.y / v;
    const int b = (int)blockIdx.y - a * v;
    // the phase's rows and columns: h = h0 + u*h', w = w0 + v*w'
    const int h0 = phase_first(a, p.pad_top, u);
    const int w0 = phase_first(b, p.pad_left, v);
    const int hph = h0 < p.H ? (p.H - h0 + u - 1) / u : 0;
    const int wph = w0 < p.W ? (p.W - w0 + v - 1) / v : 0;
    const int wb = (wph + WT - 1) / WT;          // WT-position blocks per row
    const int items = p.N * hph * wb;
    const int item = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (item >= items) return;
    const int ns = b < p.S ? (p.S - b + v - 1) / v : 0;   // taps s = b + t*v (<= NSM)
    // taps r = a + i*u; a phase with no tap in either direction adds nothing
    const int nr = a < p.R && ns > 0 ? (p.R - a + u - 1) / u : 0;

    const int n = item / (hph * wb);
    const int rem = item - n * hph * wb;
    const int hq = rem / wb;
    const int wq0 = (rem - hq * wb) * WT;       // first phase column of the lane
    const int h = h0 + u * hq;
    const int P0 = (h + p.pad_top - a) / u;
    const int Q0 = (w0 + v * wq0 + p.pad_left - b) / v;
    const int qlo = Q0 - (NSM - 1);             // window element e is dy column qlo + e

    const int d_bytes = ((p.N - 1) * p.sxn + (p.K - 1) * p.sxc + (p.P - 1) * p.sxh + (p.Q - 1) * p.sxw + 1) * ES;
    const __amdgpu_buffer_rsrc_t dr = dg_rsrc(p.x, d_bytes);
    const T* __restrict__ f = static_cast<const T*>(p.w);

    // window columns inside [0, Q): fixed for the lane
    uint32_t colmask = 0;
#pragma unroll
    for (int e = 0; e < NWIN; ++e) colmask |= (unsigned)(qlo + e) < (unsigned)p.Q ? 1u << e : 0u;
    uint32_t coloff[NWIN];
#pragma unroll
    for (int e = 0; e < NWIN; ++e) coloff[e] = (uint32_t)((qlo + e) * p.sxw * ES);

    T acc[CT][WT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int j = 0; j < WT; ++j) acc[c][j] = T(0);

    const int rs = p.R * p.S;
    for (int i = 0; i < nr; ++i) {
        const int pr = P0 - i;
        const int r = a + i * u;
        // the lane's dy row, or an offset past the tensor (the sums below
        // wrap modulo 2^32 like the buffer unit's offset arithmetic)
        const uint32_t rowoff = (unsigned)pr < (unsigned)p.P ? (uint32_t)((n * p.sxn + pr * p.sxh) * ES)
                                                              : (uint32_t)kOutside;
        for (int k = 0; k < p.K; ++k) {
            const int soff = k * p.sxc * ES;
            T win[NWIN];
#pragma unroll
            for (int e = 0; e < NWIN; ++e) win[e] = dg_load(dr, (int)(rowoff + coloff[e]), soff, T{});
            // filter taps (k, c, r, b + t*v): the same for every lane; taps
            // past the filter's edge read the last one and count zero
            T fv[CT][NSM];
            const T* fk = f + (k * p.C) * rs + r * p.S + b;
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int t = 0; t < NSM; ++t) {
                    const T fval = fk[c * rs + min(t, ns - 1) * v];
                    fv[c][t] = t < ns ? fval : T(0);
                }
#pragma unroll
            for (int e = 0; e < NWIN; ++e) win[e] = (colmask >> e) & 1u ? win[e] : T(0);
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int j = 0; j < WT; ++j)
#pragma unroll
                    for (int t = 0; t < NSM; ++t) acc[c][j] += win[NSM - 1 + j - t] * fv[c][t];
        }
    }

    T* __restrict__ dx = static_cast<T*>(p.y);
    const T alpha = (T)p.alpha;
    const T beta = (T)p.beta;
#pragma unroll
    for (int j = 0; j < WT; ++j) {
        if (wq0 + j >= wph) break;
        const int w = w0 + v * (wq0 + j);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            if (c >= p.C) break;
            const int off = n * p.syn + c * p.syk + h * p.syp + w * p.syq;
            T val = alpha * acc[c][j];
            if (beta != T(0)) val += beta * dx[off];
            dx[off] = val;
        }
    }
}

// Row-staged form of the same phase decomposition, for one to four
// channels under a tall filter (speech layer 1: 41 x 11, stride 2, onto one
// channel), where per-lane windows from global memory would touch many
// cache lines per load.  A workgroup takes one image, one phase pair and a
// band of HB output rows of that phase; for each filter k it stages the dy
// rows and columns the band reaches -- HB + nr - 1 rows of wph + NSM - 1
// values, zero outside dy -- in LDS with coalesced loads, double-buffered:
// filter k + 1's values are loaded into registers before filter k is
// computed and stored to the other buffer after it.  A lane owns WT
// consecutive phase columns of one row (the host checks that 256 / HB lanes
// cover a row) and reads its window from LDS with 16-byte reads; window
// values past the staged row feed only columns that are not stored, and
// the allocation has room for them.  Filter values are the workgroup's and
// come in as scalars, as above.
template <int CT, int NSM, int WT, int HB, int PER>
__global__ void __launch_bounds__(256) conv_bwd_data_rows_kernel(const ConvParams p, int buf_elems)
{
    constexpr int NT = 256;
    constexpr int TPR = NT / HB;                       // lanes per output row
    constexpr int NWIN = WT + NSM - 1;
    constexpr int NWV = (NWIN + 3) / 4;                // 16-byte window reads
    static_assert(WT % 4 == 0 && NT % HB == 0, "lane shapes");
    const int u = p.u, v = p.v;
    const int a = (int)blockIdx.y / v;
    const int b = (int)blockIdx.y - a * v;
    const int h0 = phase_first(a, p.pad_top, u);
    const int w0 = phase_first(b, p.pad_left, v);
    const int hph = h0 < p.H ? (p.H - h0 + u - 1) / u : 0;
    const int wph = w0 < p.W ? (p.W - w0 + v - 1) / v : 0;
    const int nbands = (hph + HB - 1) / HB;
    if ((int)blockIdx.x >= p.N * nbands) return;      // whole workgroup: the grid covers the largest phase
    const int n = (int)blockIdx.x / nbands;
    const int band = (int)blockIdx.x - n * nbands;
    const int ns = b < p.S ? (p.S - b + v - 1) / v : 0;
    const int nr = a < p.R && ns > 0 ? (p.R - a + u - 1) / u : 0;

    // output row h' = band*HB + hr reads dy rows P0(h') - i, P0(h') = P0f + h';
    // staged row sr holds dy row prow0 + sr, staged column sc dy column qcol0 + sc
    const int P0f = (h0 + p.pad_top - a) / u;
    const int Q0f = (w0 + p.pad_left - b) / v;
    const int hq0 = band * HB;
    const int nrr = nr > 0 ? nr : 1;
    const int prow0 = P0f + hq0 - (nrr - 1);
    const int qcol0 = Q0f - (NSM - 1);
    const int srows = HB + nrr - 1;
    const int scols = wph + NSM - 1;
    const int pitch = (scols + 3) & ~3;
    const int selems = srows * pitch;                  // <= buf_elems (host-sized for every phase)

    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    float* const stage = reinterpret_cast<float*>(dsm);

    const float* __restrict__ dy = static_cast<const float*>(p.x);
    const float* __restrict__ f = static_cast<const float*>(p.w);
    const int tid = threadIdx.x;
    const int hr = tid / TPR;
    const int wq = (tid - hr * TPR) * WT;              // first phase column of the lane

    // staging: element e = tid + 256*i of the band's window, column fastest;
    // loads unconditional at a valid address, zeros chosen at the store
    int soff[PER];
    uint64_t sok = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + NT * i;
        const int r = e / pitch;
        const int c = e - r * pitch;
        const int pr = prow0 + r;
        const int qc = qcol0 + c;
        const bool ok = e < selems && c < scols && (unsigned)pr < (unsigned)p.P && (unsigned)qc < (unsigned)p.Q;
        soff[i] = ok ? n * p.sxn + pr * p.sxh + qc * p.sxw : 0;
        sok |= (uint64_t)(ok ? 1u : 0u) << i;
    }
    float sval[PER];
    auto stage_load = [&](int k) {
#pragma unroll
        for (int i = 0; i < PER; ++i) sval[i] = dy[soff[i] + k * p.sxc];
    };
    auto stage_store = [&](int buf) {
        float* dst = stage + buf * buf_elems;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + NT * i;
            if (e < selems) dst[e] = (sok >> i) & 1 ? sval[i] : 0.0f;
        }
    };

    float acc[CT][WT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int j = 0; j < WT; ++j) acc[c][j] = 0.0f;

    const int rs = p.R * p.S;
    if (nr > 0) {
        stage_load(0);
        stage_store(0);
        __syncthreads();
        for (int k = 0; k < p.K; ++k) {
            const int cur = k & 1;
            stage_load(k + 1 < p.K ? k + 1 : k);
            const float* src = stage + cur * buf_elems;
            if (wq < wph) {
                for (int i = 0; i < nr; ++i) {
                    const float* row = src + (hr + (nr - 1) - i) * pitch + wq;
                    float win[NWV * 4];
#pragma unroll
                    for (int vv = 0; vv < NWV; ++vv) {
                        const float4 q4 = *reinterpret_cast<const float4*>(row + 4 * vv);
                        win[4 * vv] = q4.x;
                        win[4 * vv + 1] = q4.y;
                        win[4 * vv + 2] = q4.z;
                        win[4 * vv + 3] = q4.w;
                    }
                    const float* fk = f + (k * p.C) * rs + (a + i * u) * p.S + b;
                    float fv[CT][NSM];
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int t = 0; t < NSM; ++t) {
                            const float fval = fk[c * rs + min(t, ns - 1) * v];
                            fv[c][t] = t < ns ? fval : 0.0f;
                        }
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int j = 0; j < WT; ++j)
#pragma unroll
                            for (int t = 0; t < NSM; ++t) acc[c][j] += win[NSM - 1 + j - t] * fv[c][t];
                }
            }
            stage_store(cur ^ 1);
            __syncthreads();
        }
    }

    if (hq0 + hr >= hph) return;
    const int h = h0 + u * (hq0 + hr);
    float* __restrict__ dx = static_cast<float*>(p.y);
    const float alpha = (float)p.alpha;
    const float beta = (float)p.beta;
#pragma unroll
    for (int j = 0; j < WT; ++j) {
        if (wq + j >= wph) break;
        const int w = w0 + v * (wq + j);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            if (c >= p.C) break;
            const int off = n * p.syn + c * p.syk + h * p.syp + w * p.syq;
            float val = alpha * acc[c][j];
            if (beta != 0.0f) val += beta * dx[off];
            dx[off] = val;
        }
    }
}

// Row-staged instance onto one channel: 8-row bands, 12 columns per lane
// (so 32 lanes cover 384 phase columns), up to 6 column taps per phase.
constexpr int kRowsHB = 8, kRowsWT = 12, kRowsNSM = 6, kRowsPER = 48;

bool bwd_data_rows_fits(const ConvParams& p, size_t* lds_bytes)
{
    if (p.C != 1 || (p.S + p.v - 1) / p.v > kRowsNSM) return false;
    const int wph = (p.W + p.v - 1) / p.v;
    if (wph > (256 / kRowsHB) * kRowsWT) return false;
    const int nrmax = (p.R + p.u - 1) / p.u;
    const int pitch = (wph + kRowsNSM - 1 + 3) & ~3;
    const int64_t elems = (int64_t)(kRowsHB + nrmax - 1) * pitch;
    if (elems > 256 * kRowsPER) return false;
    // two buffers, and room for the last lane's window past the last row
    const int64_t bytes = (2 * elems + 16) * 4;
    if (bytes > 160 * 1024) return false;
    if (lds_bytes) *lds_bytes = (size_t)bytes;
    return true;
}

hipError_t launch_bwd_data_rows(const ConvParams& p, hipStream_t stream)
{
    size_t lds = 0;
    if (!bwd_data_rows_fits(p, &lds)) return hipErrorInvalidValue;
    const int wph = (p.W + p.v - 1) / p.v;
    const int nrmax = (p.R + p.u - 1) / p.u;
    const int pitch = (wph + kRowsNSM - 1 + 3) & ~3;
    const int buf_elems = (kRowsHB + nrmax - 1) * pitch;
    const int hph = (p.H + p.u - 1) / p.u;
    const dim3 grid((unsigned)(p.N * ((hph + kRowsHB - 1) / kRowsHB)), (unsigned)(p.u * p.v));
    auto kern = conv_bwd_data_rows_kernel<1, kRowsNSM, kRowsWT, kRowsHB, kRowsPER>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, p, buf_elems);
    return hipGetLastError();
}

template <class T, int CT, int NSM, int WT>
static hipError_t launch_phase_t(const ConvParams& p, hipStream_t stream)
{
    // grid.x covers the largest phase class: ceil(H/u) rows by ceil(W/v) columns
    const int hph = (p.H + p.u - 1) / p.u;
    const int wph = (p.W + p.v - 1) / p.v;
    const int64_t items = (int64_t)p.N * hph * ((wph + WT - 1) / WT);
    const dim3 grid((unsigned)((items + 255) / 256), (unsigned)(p.u * p.v));
    hipLaunchKernelGGL((conv_bwd_data_phase_kernel<T, CT, NSM, WT>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class T>
static hipError_t launch_phase_dt(const ConvParams& p, hipStream_t stream)
{
    const int nsm = (p.S + p.v - 1) / p.v;
    if (p.C < 1 || p.C > 4 || nsm > 6) return hipErrorInvalidValue;
    if (nsm <= 3) {
        switch (p.C) {
        case 1: return launch_phase_t<T, 1, 3, 8>(p, stream);
        case 2: return launch_phase_t<T, 2, 3, 4>(p, stream);
        case 3: return launch_phase_t<T, 3, 3, 4>(p, stream);
        default: return launch_phase_t<T, 4, 3, 4>(p, stream);
        }
    }
    switch (p.C) {
    case 1: return launch_phase_t<T, 1, 6, 8>(p, stream);
    case 2: return launch_phase_t<T, 2, 6, 4>(p, stream);
    case 3: return launch_phase_t<T, 3, 6, 4>(p, stream);
    default: return launch_phase_t<T, 4, 6, 4>(p, stream);
    }
}

hipError_t launch_bwd_data_phase(DType dt, const ConvParams& p, hipStream_t stream)
{
    switch (dt) {
    case DType::F32: return launch_phase_dt<float>(p, stream);
    case DType::F64: return launch_phase_dt<double>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
