// conv_bwd_filter_cl.hip -- bf16 filter gradient for channels-last x and dy
// (channel stride 1, e.g. NHWC), on gfx950 MFMA with transposing LDS reads.
//
//   dw[k,c,r,s] = alpha * sum_{n,p,q} dy[n,k,p,q] * X(n, c, p*u + r - pad_top, q*v + s - pad_left)
//               + beta * dw[k,c,r,s]
//
// (the backward routine in F that the cuDNN page, "Proposed Method", lists
// beside the forward one; the maxDNN page, Abstract and RQ4, expects the
// forward techniques to carry over).  For one filter tap (r, s) this is a
// matrix product over the positions t = (n, p, q):
//
//   dw[k0.., c0.., r, s] = A^T B,  A[t, k] = dy[n, k, p, q],  B[t, c] = X(n, c, p*u + r - pt, q*v + s - pl)
//
// With channels contiguous, a 16-byte load takes 8 consecutive filters (or
// channels) of one position, so a chunk of TK positions is staged in LDS as
// TK rows of TM filters and TK rows of TN channels -- the tap's shift is
// applied when a position's x address is formed, and taps in the padding
// read zeros.  The MFMA wants, per lane, consecutive positions of one filter
// (or channel): ds_read_b64_tr_b16 delivers exactly that from the row layout
// (a 16-lane group reads a 4-position x 16-column block, lane i receiving
// column i's 4 positions), two reads per operand.  Rows are padded by 32
// bytes so that a group's four rows hit disjoint banks.
//
// A workgroup owns a TM x TN = 64 x 64 block of dw at one tap.  Each of its
// KS groups of 4 waves -- 2 x 2 waves of one 32 x 32 block each
// (v_mfma_f32_32x32x16_bf16) -- runs every KS-th chunk of TK positions of the
// reduction through its own double buffer; at the end groups 1..KS-1 hand
// their partial sums to group 0 through LDS, added in group order, so the
// result does not depend on timing.  With about one tile per compute unit
// (these layers have 200-330 tiles) KS = 2 or 3 keeps two or three waves on
// each SIMD.  No
// workspace: the grid is ceil(K/64) x ceil(C/64) x R*S tiles.
//
// Parameters as in conv_bwd_filter.hip: x and its strides sx*; w = dy and its
// strides sd*; y = dw packed K,C,R,S; M = K, K = C*R*S, Kred = N*P*Q; div_opq,
// div_oq divide by P*Q and Q, div_s by S.  The host checks: bf16; sxc == sdk
// == 1; K, C and every other x and dy stride multiples of 8; x and dy 16-byte
// aligned.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 4 positions x one column for each lane of a 16-lane group (see above)
__device__ __forceinline__ u32x2 read_tr(const unsigned char* p)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)p);
    return __builtin_bit_cast(u32x2, v);
}

}  // namespace

template <int TM, int TN, int TK, int KS>
__global__ void __launch_bounds__(256 * KS)
conv_bwd_filter_cl_kernel(const ConvParams p)
{
    constexpr int NT = 256;
    constexpr int RA = TM * 2 + 32;          // LDS bytes per position row of dy
    constexpr int RB = TN * 2 + 32;          // ... and of x
    constexpr int A_BYTES = TK * RA;
    constexpr int B_BYTES = TK * RB;
    constexpr int BUF = A_BYTES + B_BYTES;
    constexpr int PA = TM / 8;               // 16-byte pieces per position row
    constexpr int PB = TN / 8;
    constexpr int NPA = TK * PA / NT;        // pieces per thread per chunk
    constexpr int NPB = TK * PB / NT;
    constexpr int KSTEPS = TK / 16;
    static_assert(TM == 64 && TN == 64, "2 x 2 waves of one 32 x 32 block");
    static_assert(TK % 16 == 0 && (TK * PA) % NT == 0 && (TK * PB) % NT == 0, "loader shapes");
    static_assert((KS - 1) * 4 * 16 * 64 * 4 <= KS * 2 * BUF, "partial sums fit in the chunk buffers");

    __shared__ __attribute__((aligned(16))) unsigned char smem_all[KS * 2 * BUF];

    const int grp = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255;           // thread within its group
    const int lane = tid & 63;
    const int wave = tid >> 6;                   // wave within its group
    unsigned char* const smem = smem_all + grp * 2 * BUF;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int ctiles = (p.C + TN - 1) / TN;
    const int tap = nt / ctiles;
    const int k0 = mt * TM;
    const int c0 = (nt - tap * ctiles) * TN;
    uint32_t ur, us;
    p.div_s.divmod((uint32_t)tap, ur, us);
    const int rr = (int)ur - p.pad_top;
    const int ss = (int)us - p.pad_left;

    const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
    const uint16_t* __restrict__ dy = static_cast<const uint16_t*>(p.w);
    const int L = p.Kred;

    // loader: piece e = tid + NT*i is position e / P* of the chunk, 8 columns (e % P*) * 8
    u32x4 va[NPA], vb[NPB];
    auto load_chunk = [&](int ch) {
#pragma unroll
        for (int i = 0; i < NPA; ++i) {
            const int e = tid + NT * i;
            const int t = ch * TK + e / PA;
            const int col = k0 + (e % PA) * 8;
            bool ok = t < L && col < p.M;
            int off = 0;
            if (ok) {
                uint32_t n, pq, pp, q;
                p.div_opq.divmod((uint32_t)t, n, pq);
                p.div_oq.divmod(pq, pp, q);
                off = (int)n * p.sdn + (int)pp * p.sdp + (int)q * p.sdq + col;
            }
            va[i] = ok ? *reinterpret_cast<const u32x4*>(dy + off) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < NPB; ++i) {
            const int e = tid + NT * i;
            const int t = ch * TK + e / PB;
            const int col = c0 + (e % PB) * 8;
            bool ok = t < L && col < p.C;
            int off = 0;
            if (ok) {
                uint32_t n, pq, pp, q;
                p.div_opq.divmod((uint32_t)t, n, pq);
                p.div_oq.divmod(pq, pp, q);
                const int h = (int)pp * p.u + rr;
                const int w = (int)q * p.v + ss;
                ok = (unsigned)h < (unsigned)p.H && (unsigned)w < (unsigned)p.W;
                off = (int)n * p.sxn + h * p.sxh + w * p.sxw + col;
            }
            vb[i] = ok ? *reinterpret_cast<const u32x4*>(x + off) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_chunk = [&](int buf) {
        unsigned char* a = smem + buf * BUF;
        unsigned char* b = a + A_BYTES;
#pragma unroll
        for (int i = 0; i < NPA; ++i) {
            const int e = tid + NT * i;
            *reinterpret_cast<u32x4*>(a + (e / PA) * RA + (e % PA) * 16) = va[i];
        }
#pragma unroll
        for (int i = 0; i < NPB; ++i) {
            const int e = tid + NT * i;
            *reinterpret_cast<u32x4*>(b + (e / PB) * RB + (e % PB) * 16) = vb[i];
        }
    };

    // transposing reads: in 16-lane group G, lane j reads the 8 bytes of
    // columns 16*(G%2) + 4*(j%4) .. +3 of the block at position 8*(G/2) + j/4
    // (+4 for the second read), which hands lane i of the group the k-th
    // position of column i for k = 0..3
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int G = lane >> 4;
    const int j = lane & 15;
    const int prow = 8 * (G >> 1) + (j >> 2);
    const int a_off = prow * RA + (wm * 32 + 16 * (G & 1) + 4 * (j & 3)) * 2;
    const int b_off = A_BYTES + prow * RB + (wn * 32 + 16 * (G & 1) + 4 * (j & 3)) * 2;

    f32x16 acc = f32x16{};
    // group grp takes chunks grp, grp + KS, ...; every group runs the same
    // number of iterations (the barrier is shared), idling past the end
    const int nchunks = (L + TK - 1) / TK;
    const int iters = (nchunks + KS - 1) / KS;
    if (grp < nchunks) {
        load_chunk(grp);
        store_chunk(0);
    }
    __syncthreads();
    for (int it = 0; it < iters; ++it) {
        const int ch = it * KS + grp;
        const int cur = it & 1;
        const bool mine = ch < nchunks;          // uniform per group
        const bool more = ch + KS < nchunks;
        if (more) load_chunk(ch + KS);
        if (!mine) {
            __syncthreads();
            continue;
        }
        const unsigned char* buf = smem + cur * BUF;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const u32x2 a0 = read_tr(buf + a_off + (16 * ks) * RA);
            const u32x2 a1 = read_tr(buf + a_off + (16 * ks + 4) * RA);
            const u32x2 b0 = read_tr(buf + b_off + (16 * ks) * RB);
            const u32x2 b1 = read_tr(buf + b_off + (16 * ks + 4) * RB);
            const bf16x8 fa = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
            const bf16x8 fb = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
            if (ks == KSTEPS / 2 - 1 && more) store_chunk(cur ^ 1);
        }
        __syncthreads();
    }

    if constexpr (KS > 1) {
        // groups 1..KS-1 -> LDS -> added by group 0 in group order
        float* red = reinterpret_cast<float*>(smem_all);
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) red[(((grp - 1) * 4 + wave) * 16 + i) * 64 + lane] = acc[i];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int g = 1; g < KS; ++g)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] += red[(((g - 1) * 4 + wave) * 16 + i) * 64 + lane];
        }
        if (grp > 0) return;
    }

    // dw[k, c, r, s] = alpha * acc + beta * dw: lane l holds column c0 + wn*32 + l%32
    // (one channel) and rows PolBF16::row(i, l) of the wave's 32 filters
    float* dw = static_cast<float*>(p.y);
    const float alpha = (float)p.alpha;
    const float beta = (float)p.beta;
    const int RS = p.R * p.S;
    const int c = c0 + wn * 32 + (lane & 31);
    if (c < p.C) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = k0 + wm * 32 + PolBF16::row(i, lane);
            if (k < p.M) {
                float* o = dw + (int64_t)k * p.K + c * RS + tap;
                *o = beta != 0.0f ? alpha * acc[i] + beta * *o : alpha * acc[i];
            }
        }
    }
}

hipError_t launch_bwd_filter_cl(Variant v, const ConvParams& p0, hipStream_t stream)
{
    ConvParams p = p0;
    constexpr int TM = 64, TN = 64, TK = 64;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.C + TN - 1) / TN * p.R * p.S;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    if (v == Variant::WGC_BF16_64x64_KS3)
        hipLaunchKernelGGL((conv_bwd_filter_cl_kernel<TM, TN, TK, 3>), grid, dim3(768), 0, stream, p);
    else if (v == Variant::WGC_BF16_64x64_KS2)
        hipLaunchKernelGGL((conv_bwd_filter_cl_kernel<TM, TN, TK, 2>), grid, dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((conv_bwd_filter_cl_kernel<TM, TN, TK, 1>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace miconv
