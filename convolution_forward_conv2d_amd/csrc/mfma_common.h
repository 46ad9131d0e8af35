// mfma_common.h -- pieces shared by the MFMA convolution kernels: vector
// types, the per-element-type MFMA policies, register packing and the
// LDS-staged output epilogue.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"

namespace miconv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ MFMA policies
//
// A policy fixes the element types, the MFMA instruction, its block shape
// BM x BM, how the 64 lanes split the reduction (G lane groups, V values per
// lane per instruction) and where accumulator value i of a lane sits in the
// block.  mfma() takes a lane's operands from 16-byte LDS vectors (step t of
// a chunk); mfma_s() takes one scalar operand each (V = 1 policies only).

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
    __device__ static AccV mfma_s(float a, float b, AccV c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // accumulator value i of lane l is D[8 (i/4) + 4 (l/32) + i%4][l % 32]
    __device__ static int row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
    __device__ static int col(int, int lane) { return lane & 31; }
};

// fp32 on 16x16 blocks: finer tile granularity (multiples of 16 rows) at
// the same rate as the 32x32x2 instruction.
struct PolF32x16 {
    using In = float;
    using Acc = float;
    using Out = float;
    using AccV = f32x4;
    static constexpr int BM = 16, G = 4, V = 1, NACC = 4;
    // v_mfma_f32_16x16x4_f32: lane l gives A[l%16][l/16], B[l/16][l%16].
    __device__ static AccV mfma_s(float a, float b, AccV c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // accumulator value i of lane l is D[4 (l/16) + i][l % 16] (checked on gfx950)
    __device__ static int row(int i, int lane) { return 4 * (lane >> 4) + i; }
    __device__ static int col(int, int lane) { return lane & 15; }
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
    __device__ static AccV mfma_s(double a, double b, AccV c) {
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

// ------------------------------------------------------------------ epilogue
//
// y = alpha * acc + beta * y for one wave's FM x FN accumulator blocks whose
// top-left output is (row mw0, filter nw0), with the global stores running
// along y's unit-stride direction (maxDNN page, "Proposed Method": outputs
// reorganised in shared memory for coalesced writes):
//  * along k (NHWC-like y, syk == 1): the lanes of an accumulator register
//    already hold consecutive filters of one output row, so they store
//    straight from registers;
//  * otherwise along m: each block goes through a per-wave LDS stage
//    (BM x (BM + 1) accumulators at smem + wave * BM * (BM + 1)), and a lane
//    then stores consecutive rows of one filter.
// Rows at or past m_end belong to no output (tile padding) and are dropped.
// The stage is private to the wave, so no workgroup barrier is needed; the
// caller guarantees that every wave has finished reading the main loop's
// LDS buffers (a barrier after the loop).  With beta == 0, y is never read.
// Waves with active == false store nothing.
template <class Pol, int FM, int FN>
__device__ __forceinline__ void store_acc_tile(const ConvParams& p, unsigned char* smem,
                                               typename Pol::AccV (&acc)[FM][FN],
                                               int mw0, int nw0, int m_end, int wave, int lane,
                                               bool active = true)
{
    using Acc = typename Pol::Acc;
    using Out = typename Pol::Out;
    constexpr int BM = Pol::BM;
    constexpr int STAGE_PITCH = BM + 1;
    constexpr int LG = 64 / BM;                 // lanes sharing one staged column index
    if (!active) return;
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Out* __restrict__ y = static_cast<Out*>(p.y);

    auto row_offset = [&](int gm) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)gm, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * p.syn + (int)pp * p.syp + (int)q * p.syq;
    };
    auto put = [&](int off, Acc v) {
        Acc val = alpha * v;
        if (beta != Acc(0)) val += beta * (Acc)y[off];
        y[off] = (Out)val;
    };

    if (p.syk == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int e = 0; e < Pol::NACC; ++e) {
                const int gm = mw0 + i * BM + Pol::row(e, lane);
                if (gm >= m_end) continue;
                const int moff = row_offset(gm);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int gk = nw0 + j * BM + Pol::col(e, lane);
                    if (gk < p.K) put(moff + blk_off(p.div_ycb, p.sycb, 1, gk), acc[i][j][e]);
                }
            }
        }
        return;
    }

    Acc* stage = reinterpret_cast<Acc*>(smem) + wave * BM * STAGE_PITCH;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        // a lane stores rows ml = lane % BM of the block, for LG-strided filters
        const int gm = mw0 + i * BM + lane % BM;
        const bool row_ok = gm < m_end;
        const int moff = row_ok ? row_offset(gm) : 0;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int e = 0; e < Pol::NACC; ++e)
                stage[Pol::col(e, lane) * STAGE_PITCH + Pol::row(e, lane)] = acc[i][j][e];
            const int bk0 = nw0 + j * BM;
#pragma unroll
            for (int t = 0; t < BM / LG; ++t) {
                const int kl = lane / BM + LG * t;
                const int gk = bk0 + kl;
                if (row_ok && gk < p.K)
                    put(moff + blk_off(p.div_ycb, p.sycb, p.syk, gk), stage[kl * STAGE_PITCH + lane % BM]);
            }
        }
    }
}

}  // namespace miconv
