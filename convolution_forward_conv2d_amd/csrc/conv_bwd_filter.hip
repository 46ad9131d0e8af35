// conv_bwd_filter.hip -- filter gradient of the convolution (backward pass
// with respect to F) as an implicit GEMM on gfx950 MFMA.
//
//   dw[k,c,r,s] = alpha * sum_{n,p,q} dy[n,k,p,q] * X(n, c, p*u + r - pad_top, q*v + s - pad_left)
//               + beta * dw[k,c,r,s]
//
// the adjoint of the forward sum in F (the cuDNN page, "Proposed Method",
// names forward and backward routines; the maxDNN page, Abstract and RQ4,
// expects its forward techniques to carry over to the backward pass).  As a
// matrix product, never formed:
//
//   rows     k = filter                 M = K
//   columns  j = (c, r, s)              Kred = C * R * S
//   reduce   t = (n, p, q)              L = N * P * Q
//   A[k, t] = dy[n, k, p, q]
//   B[t, j] = X(n, c, p*u + r - pad_top, q*v + s - pad_left)   (0 outside the plane)
//
// A workgroup of 4 waves owns a TM x TN tile of dw and runs the whole
// reduction over the positions in chunks of TK: each chunk of A (dy rows)
// and B (receptive-field gathers of x) goes global -> VGPR -> LDS,
// double-buffered, and feeds MFMA blocks as in conv_fwd_mfma.hip.  Lanes
// next to each other take consecutive positions, which run along q in
// memory for NCHW-like dy and x.  No workspace: the reduction is not split
// across workgroups (that would need a buffer or order-dependent atomics),
// so the grid is the tile count.  dw is packed K,C,R,S; the epilogue stores
// along j.
//
// Parameters: x, its strides sx*; w = dy, its strides sd*; y = dw with
// syn = C*R*S, syk = 1; M = K and K = C*R*S (the GEMM's rows and columns),
// div_pq = div_q = 1 (a row is one filter); div_opq, div_oq divide by P*Q
// and Q, div_rs and div_s by R*S and S; Kred = N*P*Q (the reduction length).
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
__global__ void __launch_bounds__(256)
conv_bwd_filter_kernel(const ConvParams p)
{
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using AccV = typename Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int SEG = TK / Pol::G;
    constexpr int FRAG_VECS = SEG * (int)sizeof(In) / 16;
    constexpr int STEPS = SEG / Pol::V;
    constexpr int PITCH = TK * (int)sizeof(In) + 16;
    constexpr int A_TPR = NT / TM;               // loader threads per A row (a filter)
    constexpr int A_EPT = TK / A_TPR;            // consecutive positions per thread
    constexpr int B_TPR = NT / TN;
    constexpr int B_EPT = TK / B_TPR;
    constexpr int A_BYTES = TM * PITCH;
    constexpr int B_BYTES = TN * PITCH;
    constexpr int BUF_BYTES = A_BYTES + B_BYTES;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WM % BM == 0 && WN % BM == 0, "wave tile must hold whole MFMA blocks");
    static_assert(NT % TM == 0 && NT % TN == 0 && A_EPT >= 1 && B_EPT >= 1, "loader shapes");
    static_assert(SEG * (int)sizeof(In) % 16 == 0, "lane slice must be whole 16-byte vectors");
    static_assert((A_EPT * (int)sizeof(In)) % 4 == 0 && (B_EPT * (int)sizeof(In)) % 4 == 0,
                  "loader slices must be whole words");
    static_assert(4 * BM * (BM + 1) * (int)sizeof(Acc) <= 2 * BUF_BYTES, "epilogue stage fits");
    constexpr int A_WORDS = A_EPT * (int)sizeof(In) / 4;
    constexpr int B_WORDS = B_EPT * (int)sizeof(In) / 4;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TM;
    const int n0 = nt * TN;

    const In* __restrict__ x = static_cast<const In*>(p.x);
    const In* __restrict__ dy = static_cast<const In*>(p.w);
    const int L = p.Kred;

    // ---- A loader: thread -> filter row, A_EPT consecutive positions
    const int a_row = tid / A_TPR;
    const int a_seg = tid % A_TPR;
    const bool a_ok = m0 + a_row < p.M;
    const In* __restrict__ dyk = dy + (a_ok ? m0 + a_row : 0) * p.sdk;
    // ---- B loader: thread -> column (c, r, s), B_EPT consecutive positions
    const int b_row = tid / B_TPR;
    const int b_seg = tid % B_TPR;
    int bc = 0, br = 0, bs = 0;
    const bool b_ok = n0 + b_row < p.K;
    if (b_ok) {
        uint32_t c, rs, r, s;
        p.div_rs.divmod((uint32_t)(n0 + b_row), c, rs);
        p.div_s.divmod(rs, r, s);
        bc = (int)c;
        br = (int)r - p.pad_top;
        bs = (int)s - p.pad_left;
    }
    const In* __restrict__ xc = x + bc * p.sxc;

    In a_val[A_EPT];
    In b_val[B_EPT];

    auto pos_of = [&](int t, int& n, int& pp, int& q) {
        uint32_t un, pq, up, uq;
        p.div_opq.divmod((uint32_t)t, un, pq);
        p.div_oq.divmod(pq, up, uq);
        n = (int)un;
        pp = (int)up;
        q = (int)uq;
    };

    auto load_chunk = [&](int ch) {
        {
            int t = ch * TK + a_seg * A_EPT, n, pp, q;
            pos_of(t, n, pp, q);
#pragma unroll
            for (int j = 0; j < A_EPT; ++j) {
                const bool ok = a_ok && t + j < L;
                a_val[j] = ok ? load_elem(dyk + n * p.sdn + pp * p.sdp + q * p.sdq) : In(0);
                if (++q == p.Q) {
                    q = 0;
                    if (++pp == p.P) { pp = 0; ++n; }
                }
            }
        }
        {
            int t = ch * TK + b_seg * B_EPT, n, pp, q;
            pos_of(t, n, pp, q);
#pragma unroll
            for (int j = 0; j < B_EPT; ++j) {
                const int h = pp * p.u + br;
                const int w = q * p.v + bs;
                const bool ok = b_ok && t + j < L && (unsigned)h < (unsigned)p.H && (unsigned)w < (unsigned)p.W;
                b_val[j] = ok ? load_elem(xc + n * p.sxn + h * p.sxh + w * p.sxw) : In(0);
                if (++q == p.Q) {
                    q = 0;
                    if (++pp == p.P) { pp = 0; ++n; }
                }
            }
        }
    };

    auto store_tiles = [&](int buf) {
        unsigned char* a_dst = smem + buf * BUF_BYTES + a_row * PITCH + a_seg * A_EPT * (int)sizeof(In);
        unsigned char* b_dst = smem + buf * BUF_BYTES + A_BYTES + b_row * PITCH + b_seg * B_EPT * (int)sizeof(In);
        uint32_t aw[A_WORDS];
        uint32_t bw[B_WORDS];
        Pack<In>::to_words(a_val, aw);
        Pack<In>::to_words(b_val, bw);
        lds_store_words<A_WORDS>(a_dst, aw);
        lds_store_words<B_WORDS>(b_dst, bw);
    };

    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane % BM;
    const int lgrp = lane / BM;

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    const int nchunks = (L + TK - 1) / TK;
    load_chunk(0);
    store_tiles(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nchunks;
        if (more) load_chunk(ch + 1);
        const unsigned char* a_src = smem + cur * BUF_BYTES;
        const unsigned char* b_src = a_src + A_BYTES;
        u32x4 fa[FM][FRAG_VECS];
        u32x4 fb[FN][FRAG_VECS];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4* src = reinterpret_cast<const u32x4*>(
                a_src + (wm * WM + i * BM + lrow) * PITCH + lgrp * SEG * (int)sizeof(In));
#pragma unroll
            for (int v = 0; v < FRAG_VECS; ++v) fa[i][v] = src[v];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4* src = reinterpret_cast<const u32x4*>(
                b_src + (wn * WN + j * BM + lrow) * PITCH + lgrp * SEG * (int)sizeof(In));
#pragma unroll
            for (int v = 0; v < FRAG_VECS; ++v) fb[j][v] = src[v];
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Pol::mfma(fa[i], fb[j], t, acc[i][j]);
            if (t == STEPS / 2 && more) store_tiles(cur ^ 1);
        }
        __syncthreads();
    }

    store_acc_tile<Pol, FM, FN>(p, smem, acc, m0 + wm * WM, n0 + wn * WN, p.M, wave, lane);
}

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
static hipError_t launch_wg_variant(const ConvParams& p0, hipStream_t stream)
{
    ConvParams p = p0;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    hipLaunchKernelGGL((conv_bwd_filter_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

//        name              policy   TM   TN  waves  TK
#define MICONV_WG_VARIANTS(X)                          \
    X(WG_F32_128x128, PolF32, 128, 128, 2, 2, 32)      \
    X(WG_F32_64x128, PolF32, 64, 128, 2, 2, 32)        \
    X(WG_F32_128x64, PolF32, 128, 64, 2, 2, 32)        \
    X(WG_F32_64x64, PolF32, 64, 64, 2, 2, 32)          \
    X(WG_F64_128x64, PolF64, 128, 64, 2, 2, 16)        \
    X(WG_F64_64x64, PolF64, 64, 64, 2, 2, 16)          \
    X(WG_BF16_128x128, PolBF16, 128, 128, 2, 2, 32)    \
    X(WG_BF16_64x64, PolBF16, 64, 64, 2, 2, 32)

hipError_t launch_bwd_filter(Variant v, const ConvParams& p, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, tk) \
    case Variant::name: return launch_wg_variant<pol, tm, tn, wmm, wnn, tk>(p, stream);
        MICONV_WG_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
