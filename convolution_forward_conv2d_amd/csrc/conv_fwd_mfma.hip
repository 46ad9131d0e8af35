// conv_fwd_mfma.hip -- implicit-GEMM convolution forward pass on gfx950 MFMA.
//
// The convolution is read as a matrix product without ever forming the
// matrices (maxDNN page, "Proposed Method": each output coordinate is the
// receptive field times the filter; batch-reduce GEMM page, "Proposed
// Method": a batch of sub-block products reduced into one output block):
//
//   rows     m = (n, p, q)            M    = N * P * Q
//   columns  k = filter               K
//   reduce   kappa = (c, r, s)        Kred = C * R * S
//   A[m, kappa] = X(n, c, p*u + r - pad_top, q*v + s - pad_left)   (0 outside)
//   B[kappa, k] = F[k, c, r, s]                 (packed KCRS; WB: blocked filters)
//
// A workgroup of 4 waves owns a TM x TN output tile.  The reduction runs in
// chunks of TK: each chunk of A (input receptive fields, gathered straight
// from x through its strides) and of B (filter rows) goes global -> VGPR ->
// LDS, double-buffered so the next chunk's global loads fly while the
// matrix cores work on the current one (maxDNN page, "Proposed Method":
// double buffering through shared memory).  Each wave runs MFMA blocks over
// its WM x WN sub-tile.  The epilogue stages every accumulator block through
// LDS and writes y along its unit-stride direction (maxDNN page, "Proposed
// Method": outputs reorganised in shared memory for coalesced writes).
// Nothing but x, w and y is touched in device memory: no workspace
// (zero-memory direct-convolution page, Abstract).
//
// DG = true computes the data gradient (the adjoint of the forward sum in
// x) for any stride, in tap order: rows m = (n, h, w) of dx, columns c,
// reduction (k, r, s) with
//   A[m, (k,r,s)] = dy[n, k, p, q] where p*u = h + pad_top - r and
//                   q*v = w + pad_left - s (0 outside or off the stride grid)
//   B[(k,r,s), c] = F[k, c, r, s]
// The host passes C = the filter count, K = the channel count of dx,
// H, W = dy's dims, P, Q = dx's dims, x = dy, y = dx.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

// ------------------------------------------------------------------ the kernel

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK, bool BVEC, bool TAP, bool DG, bool WB>
__global__ void __launch_bounds__(256)
conv_fwd_mfma_kernel(const ConvParams p)
{
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using AccV = typename Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;                 // MFMA blocks per wave along m
    constexpr int FN = WN / BM;                 // ... along k
    constexpr int SEG = TK / Pol::G;            // reduction elements per lane group per chunk
    constexpr int FRAG_VECS = SEG * (int)sizeof(In) / 16;
    constexpr int STEPS = SEG / Pol::V;         // MFMA instructions per block per chunk
    constexpr int PITCH = TK * (int)sizeof(In) + 16;   // LDS row pitch in bytes (bank skew)
    constexpr int A_TPR = NT / TM;              // loader threads per A row
    constexpr int A_EPT = TK / A_TPR;           // A elements per thread per chunk
    constexpr int B_TPR = NT / TN;
    constexpr int B_EPT = TK / B_TPR;
    constexpr int A_BYTES = TM * PITCH;
    constexpr int B_BYTES = TN * PITCH;
    constexpr int BUF_BYTES = A_BYTES + B_BYTES;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WM % BM == 0 && WN % BM == 0, "wave tile must hold whole MFMA blocks");
    static_assert(TM >= 64 && NT % TM == 0, "A loader needs wave-uniform segments");
    static_assert(NT % TN == 0 && B_EPT >= 1, "B loader shape");
    static_assert(SEG * (int)sizeof(In) % 16 == 0, "lane slice must be whole 16-byte vectors");
    static_assert((A_EPT * (int)sizeof(In)) % 4 == 0 && (B_EPT * (int)sizeof(In)) % 4 == 0,
                  "loader slices must be whole words");
    static_assert(4 * BM * (BM + 1) * (int)sizeof(Acc) <= 2 * BUF_BYTES, "epilogue stage fits");
    static_assert(!DG || TAP, "the data gradient runs in tap order");
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
    const In* __restrict__ w = static_cast<const In*>(p.w);

    // ---- A loader: thread -> one output row m, one wave-uniform reduction segment
    const int a_row = tid % TM;
    const int a_seg = __builtin_amdgcn_readfirstlane(tid / TM);
    int hb, wb, abase;
    {
        const int m = m0 + a_row;
        if (m < p.M) {
            uint32_t n, pq, pp, q;
            p.div_pq.divmod((uint32_t)m, n, pq);
            p.div_q.divmod(pq, pp, q);
            if constexpr (DG) {
                // (pp, q) is the dx position (h, w): keep h + pad_top, w + pad_left
                hb = (int)pp + p.pad_top;
                wb = (int)q + p.pad_left;
                abase = (int)n * p.sxn;
            } else {
                hb = (int)pp * p.u - p.pad_top;
                wb = (int)q * p.v - p.pad_left;
                abase = (int)n * p.sxn + hb * p.sxh + wb * p.sxw;
            }
        } else {
            hb = -0x40000000;      // every h = hb + r falls outside [0, H): row reads as zeros
            wb = 0;
            abase = 0;
        }
    }
    // ---- B loader: thread -> one filter k, one reduction segment
    const int b_row = tid % TN;
    const int b_seg = tid / TN;
    const bool b_ok = (n0 + b_row) < p.K;
    // (DG: column c's filter values F[k, c, :, :] start at c*R*S, filter k at k*K*R*S)
    const In* __restrict__ wrow = w + (size_t)(b_ok ? n0 + b_row : 0) * (size_t)(DG ? p.R * p.S : p.Kred);

    In a_val[A_EPT];
    In b_val[B_EPT];

    // Reduction order.  Flat: chunk ch = kappa in [ch*TK, ch*TK + TK), kappa
    // = (c, r, s) in KCRS order, decoded per element.  Tap: chunk ch = TK
    // consecutive channels at one filter tap, ch = channel_block * R*S + tap;
    // one bounds check per chunk and a plain channel stride per element.
    auto tap_of = [&](int ch, int& c0, int& r, int& s) {
        uint32_t cb, rs, rr, ss;
        p.div_rs.divmod((uint32_t)ch, cb, rs);
        p.div_s.divmod(rs, rr, ss);
        c0 = (int)cb * TK;
        r = (int)rr;
        s = (int)ss;
    };

    auto load_a = [&](int ch) {
        if constexpr (DG) {
            int k0, r, s;
            tap_of(ch, k0, r, s);
            k0 += a_seg * A_EPT;                     // wave-uniform
            const int hh = hb - r, ww = wb - s;      // p*u and q*v if on the stride grid
            uint32_t pp = 0, qq = 0;
            bool tap_ok = hh >= 0 && ww >= 0;
            if (tap_ok) {
                pp = p.div_u.div((uint32_t)hh);
                qq = p.div_v.div((uint32_t)ww);
                tap_ok = (int)pp * p.u == hh && (int)qq * p.v == ww && (int)pp < p.H && (int)qq < p.W;
            }
            const In* src = x + (abase + k0 * p.sxc + (int)pp * p.sxh + (int)qq * p.sxw);
#pragma unroll
            for (int j = 0; j < A_EPT; ++j)
                a_val[j] = (tap_ok && k0 + j < p.C) ? load_elem(src + j * p.sxc) : In(0);
            return;
        }
        if constexpr (TAP) {
            int c0, r, s;
            tap_of(ch, c0, r, s);
            c0 += a_seg * A_EPT;                     // wave-uniform
            const bool tap_ok = ((unsigned)(hb + r) < (unsigned)p.H) && ((unsigned)(wb + s) < (unsigned)p.W);
            // (channel-blocked x: the chunk's channels lie in one block)
            const In* src = x + (abase + blk_off(p.div_xcb, p.sxcb, p.sxc, c0) + r * p.sxh + s * p.sxw);
#pragma unroll
            for (int j = 0; j < A_EPT; ++j)
                a_val[j] = (tap_ok && c0 + j < p.C) ? load_elem(src + j * p.sxc) : In(0);
            return;
        }
        const int kap = ch * TK + a_seg * A_EPT;    // wave-uniform
        uint32_t c, rs, r, s;
        p.div_rs.divmod((uint32_t)kap, c, rs);
        p.div_s.divmod(rs, r, s);
#pragma unroll
        for (int j = 0; j < A_EPT; ++j) {
            const bool ok = (kap + j < p.Kred) &&
                            ((unsigned)(hb + (int)r) < (unsigned)p.H) &&
                            ((unsigned)(wb + (int)s) < (unsigned)p.W);
            const int off = abase + blk_off(p.div_xcb, p.sxcb, p.sxc, (int)c) + (int)r * p.sxh + (int)s * p.sxw;
            a_val[j] = ok ? load_elem(x + off) : In(0);
            if (++s == (uint32_t)p.S) {
                s = 0;
                if (++r == (uint32_t)p.R) { r = 0; ++c; }
            }
        }
    };

    auto load_b = [&](int ch) {
        if constexpr (DG) {
            int k0, r, s;
            tap_of(ch, k0, r, s);
            k0 += b_seg * B_EPT;
            const int rs = p.R * p.S;
            const In* src = wrow + (size_t)k0 * p.K * rs + r * p.S + s;
#pragma unroll
            for (int j = 0; j < B_EPT; ++j)
                b_val[j] = (b_ok && k0 + j < p.C) ? load_elem(src + (size_t)j * p.K * rs) : In(0);
            return;
        }
        if constexpr (TAP) {
            int c0, r, s;
            tap_of(ch, c0, r, s);
            c0 += b_seg * B_EPT;
            const int rs = p.R * p.S;
            if constexpr (WB) {
                // blocked filters [K/kb][C/cb][R][S][cb][kb]: consecutive channels
                // of one block kb apart, consecutive filters (lanes) adjacent
                const int k = b_ok ? n0 + b_row : 0;
                const In* src = w + wblk_off(k, c0, r * p.S + s, p.C, rs, p.wkb, p.wcb);
#pragma unroll
                for (int j = 0; j < B_EPT; ++j)
                    b_val[j] = (b_ok && c0 + j < p.C) ? load_elem(src + j * p.wkb) : In(0);
                return;
            }
            const In* src = wrow + (c0 * p.R + r) * p.S + s;
#pragma unroll
            for (int j = 0; j < B_EPT; ++j)
                b_val[j] = (b_ok && c0 + j < p.C) ? load_elem(src + j * rs) : In(0);
            return;
        }
        const int kap = ch * TK + b_seg * B_EPT;
        if constexpr (BVEC) {
            // the host guarantees Kred % (16 / sizeof(In)) == 0 and a 16-byte aligned w
            constexpr int VE = 16 / (int)sizeof(In);
            static_assert(B_EPT % VE == 0, "vector B loads need whole vectors");
#pragma unroll
            for (int vi = 0; vi < B_EPT / VE; ++vi) {
                const bool ok = b_ok && (kap + vi * VE < p.Kred);
                u32x4 t = ok ? *reinterpret_cast<const u32x4*>(wrow + kap + vi * VE) : u32x4{0, 0, 0, 0};
                __builtin_memcpy(&b_val[vi * VE], &t, 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < B_EPT; ++j) {
                const bool ok = b_ok && (kap + j < p.Kred);
                b_val[j] = ok ? load_elem(wrow + kap + j) : In(0);
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

    // ---- per-wave MFMA geometry
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane % BM;            // row (m or k) this lane feeds within a block
    const int lgrp = lane / BM;            // reduction group of this lane

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    const int nchunks = TAP ? (p.C + TK - 1) / TK * p.R * p.S : (p.Kred + TK - 1) / TK;

    load_a(0);
    load_b(0);
    store_tiles(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nchunks;
        if (more) {
            load_a(ch + 1);
            load_b(ch + 1);
        }
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
            // store the next chunk into the other buffer halfway through (its
            // last readers finished before the previous barrier)
            if (t == STEPS / 2 && more) store_tiles(cur ^ 1);
        }
        __syncthreads();
    }

    // ---- epilogue
    store_acc_tile<Pol, FM, FN>(p, smem, acc, m0 + wm * WM, n0 + wn * WN, p.M, wave, lane);
}

// ------------------------------------------------------------------ instances and launch

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
static hipError_t launch_variant(const ConvParams& p0, bool bvec, bool tap, bool dgrad, hipStream_t stream)
{
    ConvParams p = p0;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    // vector filter loads need each thread's slice to be whole 16-byte vectors
    constexpr int B_EPT = TK * TN / 256;
    constexpr bool CAN_VEC = (B_EPT * (int)sizeof(typename Pol::In)) % 16 == 0;
    if constexpr (!CAN_VEC) bvec = false;
    if (p.wkb > 0) {
        // blocked filters: tap order only, a chunk's TK channels in one block
        if (dgrad || !tap || p.wcb % TK != 0 || p.K % p.wkb != 0 || p.C % p.wcb != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false, true, false, true>),
                           grid, dim3(256), 0, stream, p);
    } else if (dgrad)
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false, true, true, false>),
                           grid, dim3(256), 0, stream, p);
    else if (tap)
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false, true, false, false>),
                           grid, dim3(256), 0, stream, p);
    else if (bvec)
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, CAN_VEC, false, false, false>),
                           grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false, false, false, false>),
                           grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

//        name               policy   TM   TN  waves  TK
#define MICONV_VARIANTS(X)                                   \
    X(MFMA_F32_128x128, PolF32, 128, 128, 2, 2, 16)          \
    X(MFMA_F32_128x64, PolF32, 128, 64, 2, 2, 16)            \
    X(MFMA_F32_256x32, PolF32, 256, 32, 4, 1, 16)            \
    X(MFMA_F32_64x128, PolF32, 64, 128, 2, 2, 16)            \
    X(MFMA_F64_128x128, PolF64, 128, 128, 2, 2, 16)          \
    X(MFMA_F64_128x64, PolF64, 128, 64, 2, 2, 16)            \
    X(MFMA_F64_64x64, PolF64, 64, 64, 2, 2, 16)              \
    X(MFMA_BF16_128x128, PolBF16, 128, 128, 2, 2, 32)        \
    X(MFMA_BF16_128x64, PolBF16, 128, 64, 2, 2, 32)          \
    X(MFMA_BF16_256x32, PolBF16, 256, 32, 4, 1, 32)

hipError_t launch_mfma(Variant v, const ConvParams& p, bool bvec, bool tap, bool dgrad, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, tk) \
    case Variant::name: return launch_variant<pol, tm, tn, wmm, wnn, tk>(p, bvec, tap, dgrad, stream);
        MICONV_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
