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
//   B[kappa, k] = F[k, c, r, s]                                     (packed KCRS)
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
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "tile_map.h"

namespace miconv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ MFMA policies
//
// A policy fixes the element types, the MFMA instruction, its block shape
// BM x BM, how the 64 lanes split the reduction (G lane groups, V values per
// lane per instruction) and where accumulator value i of a lane sits in the
// block.  A lane's slice of one reduction chunk must be whole 16-byte
// vectors of LDS.

struct PolF32 {
    using In = float;
    using Acc = float;
    using Out = float;
    using AccV = f32x16;
    static constexpr int BM = 32, G = 2, V = 1, NACC = 16;
    // v_mfma_f32_32x32x2_f32: lane l gives A[l%32][l/32], B[l/32][l%32].
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        float a = __uint_as_float(fa[t >> 2][t & 3]);
        float b = __uint_as_float(fb[t >> 2][t & 3]);
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
    __device__ static int col(int, int lane) { return lane & 31; }
};

struct PolF64 {
    using In = double;
    using Acc = double;
    using Out = double;
    using AccV = f64x4;
    static constexpr int BM = 16, G = 4, V = 1, NACC = 4;
    // v_mfma_f64_16x16x4_f64: lane l gives A[l%16][l/16], B[l/16][l%16].
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        const u32x4 va = fa[t >> 1], vb = fb[t >> 1];
        const int h = (t & 1) * 2;
        double a = __hiloint2double((int)va[h + 1], (int)va[h]);
        double b = __hiloint2double((int)vb[h + 1], (int)vb[h]);
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // accumulator value i of lane l is D[l/16 + 4 i][l % 16] (checked on gfx950)
    __device__ static int row(int i, int lane) { return (lane >> 4) + 4 * i; }
    __device__ static int col(int, int lane) { return lane & 15; }
};

struct PolBF16 {
    using In = uint16_t;        // raw bf16 bits
    using Acc = float;
    using Out = float;
    using AccV = f32x16;
    static constexpr int BM = 32, G = 2, V = 8, NACC = 16;
    // v_mfma_f32_32x32x16_bf16: lane l gives A[l%32][8*(l/32) .. +8], B likewise.
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        bf16x8 a = __builtin_bit_cast(bf16x8, fa[t]);
        bf16x8 b = __builtin_bit_cast(bf16x8, fb[t]);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
    __device__ static int col(int, int lane) { return lane & 31; }
};

// ------------------------------------------------------------------ element <-> word packing

template <class In> struct Pack;

template <> struct Pack<float> {
    template <int E>
    __device__ static void to_words(const float (&v)[E], uint32_t (&w)[E]) {
#pragma unroll
        for (int i = 0; i < E; ++i) w[i] = __float_as_uint(v[i]);
    }
};

template <> struct Pack<double> {
    template <int E>
    __device__ static void to_words(const double (&v)[E], uint32_t (&w)[2 * E]) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            w[2 * i] = (uint32_t)__double2loint(v[i]);
            w[2 * i + 1] = (uint32_t)__double2hiint(v[i]);
        }
    }
};

template <> struct Pack<uint16_t> {
    template <int E>
    __device__ static void to_words(const uint16_t (&v)[E], uint32_t (&w)[E / 2]) {
#pragma unroll
        for (int i = 0; i < E / 2; ++i) w[i] = (uint32_t)v[2 * i] | ((uint32_t)v[2 * i + 1] << 16);
    }
};

// Store NW 32-bit words to 16-byte-aligned LDS with the widest ds_write.
template <int NW>
__device__ __forceinline__ void lds_store_words(unsigned char* dst, const uint32_t (&w)[NW])
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i)
            reinterpret_cast<u32x4*>(dst)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 2; ++i)
            reinterpret_cast<u32x2*>(dst)[i] = u32x2{w[2 * i], w[2 * i + 1]};
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) reinterpret_cast<uint32_t*>(dst)[i] = w[i];
    }
}

template <class In> __device__ __forceinline__ In load_elem(const In* p) { return *p; }

// ------------------------------------------------------------------ the kernel

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK, bool BVEC>
__global__ void __launch_bounds__(256)
conv_fwd_mfma_kernel(const ConvParams p)
{
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using Out = typename Pol::Out;
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
    constexpr int STAGE_PITCH = BM + 1;         // epilogue staging pitch (elements)
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WM % BM == 0 && WN % BM == 0, "wave tile must hold whole MFMA blocks");
    static_assert(TM >= 64 && NT % TM == 0, "A loader needs wave-uniform segments");
    static_assert(NT % TN == 0 && B_EPT >= 1, "B loader shape");
    static_assert(SEG * (int)sizeof(In) % 16 == 0, "lane slice must be whole 16-byte vectors");
    static_assert((A_EPT * (int)sizeof(In)) % 4 == 0 && (B_EPT * (int)sizeof(In)) % 4 == 0,
                  "loader slices must be whole words");
    static_assert(4 * BM * STAGE_PITCH * (int)sizeof(Acc) <= 2 * BUF_BYTES, "staging fits");
    constexpr int A_WORDS = A_EPT * (int)sizeof(In) / 4;
    constexpr int B_WORDS = B_EPT * (int)sizeof(In) / 4;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles);
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
            hb = (int)pp * p.u - p.pad_top;
            wb = (int)q * p.v - p.pad_left;
            abase = (int)n * p.sxn + hb * p.sxh + wb * p.sxw;
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
    const In* __restrict__ wrow = w + (size_t)(b_ok ? n0 + b_row : 0) * (size_t)p.Kred;

    In a_val[A_EPT];
    In b_val[B_EPT];

    auto load_a = [&](int kc0) {
        const int kap = kc0 + a_seg * A_EPT;        // wave-uniform
        uint32_t c, rs, r, s;
        p.div_rs.divmod((uint32_t)kap, c, rs);
        p.div_s.divmod(rs, r, s);
#pragma unroll
        for (int j = 0; j < A_EPT; ++j) {
            const bool ok = (kap + j < p.Kred) &&
                            ((unsigned)(hb + (int)r) < (unsigned)p.H) &&
                            ((unsigned)(wb + (int)s) < (unsigned)p.W);
            const int off = abase + (int)c * p.sxc + (int)r * p.sxh + (int)s * p.sxw;
            a_val[j] = ok ? load_elem(x + off) : In(0);
            if (++s == (uint32_t)p.S) {
                s = 0;
                if (++r == (uint32_t)p.R) { r = 0; ++c; }
            }
        }
    };

    auto load_b = [&](int kc0) {
        const int kap = kc0 + b_seg * B_EPT;
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

    const int nchunks = (p.Kred + TK - 1) / TK;

    load_a(0);
    load_b(0);
    store_tiles(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nchunks;
        if (more) {
            load_a((ch + 1) * TK);
            load_b((ch + 1) * TK);
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
        for (int t = 0; t < STEPS; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Pol::mfma(fa[i], fb[j], t, acc[i][j]);
        if (more) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: y = alpha * acc + beta * y, through a per-wave LDS stage
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Out* __restrict__ y = static_cast<Out*>(p.y);
    Acc* stage = reinterpret_cast<Acc*>(smem) + wave * BM * STAGE_PITCH;
    constexpr int LG = 64 / BM;                 // lanes sharing one staged column index
    const bool k_fast = (p.syk == 1);           // NHWC-like output: k is the unit-stride direction

#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int e = 0; e < Pol::NACC; ++e)
                stage[Pol::col(e, lane) * STAGE_PITCH + Pol::row(e, lane)] = acc[i][j][e];
            __syncthreads();
            const int bm0 = m0 + wm * WM + i * BM;
            const int bk0 = n0 + wn * WN + j * BM;
#pragma unroll
            for (int t = 0; t < BM / LG; ++t) {
                const int ml = k_fast ? (lane / BM + LG * t) : (lane % BM);
                const int kl = k_fast ? (lane % BM) : (lane / BM + LG * t);
                const int gm = bm0 + ml;
                const int gk = bk0 + kl;
                if (gm < p.M && gk < p.K) {
                    uint32_t n, pq, pp, q;
                    p.div_pq.divmod((uint32_t)gm, n, pq);
                    p.div_q.divmod(pq, pp, q);
                    const int off = (int)n * p.syn + gk * p.syk + (int)pp * p.syp + (int)q * p.syq;
                    Acc val = alpha * stage[kl * STAGE_PITCH + ml];
                    if (beta != Acc(0)) val += beta * (Acc)y[off];
                    y[off] = (Out)val;
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------ instances and launch

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
static hipError_t launch_variant(const ConvParams& p0, bool bvec, hipStream_t stream)
{
    ConvParams p = p0;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    // vector filter loads need each thread's slice to be whole 16-byte vectors
    constexpr int B_EPT = TK * TN / 256;
    constexpr bool CAN_VEC = (B_EPT * (int)sizeof(typename Pol::In)) % 16 == 0;
    if constexpr (!CAN_VEC) bvec = false;
    if (bvec)
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, CAN_VEC>),
                           grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((conv_fwd_mfma_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false>),
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

hipError_t launch_mfma(Variant v, const ConvParams& p, bool bvec, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, tk) \
    case Variant::name: return launch_variant<pol, tm, tn, wmm, wnn, tk>(p, bvec, stream);
        MICONV_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
