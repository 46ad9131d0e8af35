// conv_bwd_data_subpixel.hip -- data gradient of a strided convolution as a
// stride-1 implicit GEMM over dy whose columns are dx's stride phases.
//
//   dx[n,c,h,w] = alpha * sum over k, and the (p, r), (q, s) pairs with
//                 p*u + r = h + pad_top and q*v + s = w + pad_left,
//                 of dy[n,k,p,q] * F[k,c,r,s]
//               + beta * dx[n,c,h,w]
//
// (the backward routine in x that the cuDNN page, "Proposed Method", lists
// beside the forward one).  Write h + pad_top = u*P' + a (0 <= a < u) and
// w + pad_left = v*Q' + b (0 <= b < v).  The taps reaching (h, w) are then
// r = u*i + a and s = v*j + b for i, j >= 0 with r < R, s < S, and
// p = P' - i, q = Q' - j.  So the u x v block (P', Q') of dx is
//
//   dx[n, c, u*P' + a - pad_top, v*Q' + b - pad_left]
//     = sum over k, i < D, j < E of dy[n, k, P' - i, Q' - j] * F[k, c, u*i + a, v*j + b]
//
// with D = ceil(R / u), E = ceil(S / v) and F read as zero past R and S: a
// stride-1 correlation of dy (K channels, a D x E window) onto C*u*v
// output columns (c, a, b).  Every multiply-add of it belongs to the data
// gradient except those on the zero taps past R, S, where the adjoint taken
// over all R x S taps per dx element (conv_fwd_mfma.hip's DG mode) meets the
// stride grid on one tap in u*v.  As an implicit GEMM on the matrix cores
// (batch-reduce GEMM page, "Proposed Method": sub-block products reduced
// into one output block):
//
//   rows     m = (n, P'', Q'')   dx blocks, P' = P'' + P0, Q' = Q'' + Q0,
//                                 P0 = floor(pad_top / u), Q0 = floor(pad_left / v)
//   columns  z = (c, a, b)       C*u*v, b fastest
//   reduce   (k, i, j)           in tap order: a chunk is TK channels at one (i, j)
//   A[m, (k,i,j)] = dy[n, k, P' - i, Q' - j]      (0 outside dy)
//   B[(k,i,j), z] = F[k, c, u*i + a, v*j + b]     (0 past R, S)
//
// The block grid covers dx exactly: P'' runs over the P' of rows 0 .. H-1,
// so every dx element is one (block, column) pair and is written once.  A
// workgroup of 4 waves owns a TM x TN tile; chunks go global -> VGPR -> LDS,
// double-buffered, the next chunk stored halfway through the current one's
// MFMA steps (the gather kernel's pipeline).  The epilogue stages each
// accumulator block through LDS and stores column (c, a, b) of block
// (P', Q') to dx[n, c, u*P' + a - pad_top, v*Q' + b - pad_left] where that
// lies inside dx; along m the stores step v elements of a dx row.  No
// workspace: nothing but dy, F and dx is touched in device memory.
//
// Host parameters in the direct kernel's layout (conv_bwd_data.hip): x = dy
// with sx* its (n, k, p, q) strides, y = dx with sy* its (n, c, h, w)
// strides, w = F packed K,C,R,S; N, C, H, W are dx's dims, K, P, Q dy's.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

namespace {

// fp32 16x16x4 blocks with operands taken from 16-byte LDS vectors, as
// PolF32 does for 32x32x2: column tiles of 48 fit 3 channels x 4 x 4 phases
struct PolF32x16V : PolF32x16 {
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        const float a = __uint_as_float(fa[t >> 2][t & 3]);
        const float b = __uint_as_float(fb[t >> 2][t & 3]);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// largest power of two p with p * tn <= nt: B loader threads per tile column
constexpr int b_threads_per_col(int nt, int tn)
{
    int p = 1;
    while (2 * p * tn <= nt) p *= 2;
    return p;
}

struct SubpixelArgs {
    const void* dy;
    const void* w;
    void* dx;
    int N, K, C;            // images, dy channels (reduction), dx channels
    int P, Q;               // dy rows, columns
    int H, W;               // dx rows, columns
    int R, S, u, v;
    int P0, Q0;             // block row / column of dx block 0
    int h_off, w_off;       // pad_top mod u, pad_left mod v: dx row of block row P'' is u*P'' - h_off + a
    int sdn, sdk, sdp, sdq; // dy element strides
    int sxn, sxc, sxh, sxw; // dx element strides
    int M, Z;               // rows N * HB * WB, columns C*u*v
    int m_tiles, n_tiles;
    FastDiv div_blk, div_wb;    // by HB * WB and by WB
    FastDiv div_de, div_e;      // by D * E and by E (tap decode)
    FastDiv div_uv, div_v;      // column z -> (c, a, b)
    double alpha, beta;
    int tile_rev;               // tiles in reverse order (xcd_logical_tile)
};

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
__global__ void __launch_bounds__(256)
conv_bwd_data_subpixel_kernel(const SubpixelArgs p)
{
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using Out = typename Pol::Out;
    using AccV = typename Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int SEG = TK / Pol::G;            // reduction elements per lane group per chunk
    constexpr int FRAG_VECS = SEG * (int)sizeof(In) / 16;
    constexpr int STEPS = SEG / Pol::V;
    constexpr int PITCH = TK * (int)sizeof(In) + 16;   // LDS row pitch in bytes (bank skew)
    constexpr int A_TPR = NT / TM;              // loader threads per A row
    constexpr int A_EPT = TK / A_TPR;
    constexpr int B_TPR = b_threads_per_col(NT, TN);   // the first B_TPR * TN threads load B
    constexpr int B_EPT = TK / B_TPR;
    constexpr int A_BYTES = TM * PITCH;
    constexpr int B_BYTES = TN * PITCH;
    constexpr int BUF_BYTES = A_BYTES + B_BYTES;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WM % BM == 0 && WN % BM == 0, "wave tile must hold whole MFMA blocks");
    static_assert(TM >= 64 && NT % TM == 0 && TK % B_TPR == 0 && A_EPT >= 1 && B_EPT >= 1, "loader shapes");
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

    const In* __restrict__ dy = static_cast<const In*>(p.dy);
    const In* __restrict__ f = static_cast<const In*>(p.w);

    // ---- A loader: thread -> one block row m, one wave-uniform channel segment
    const int a_row = tid % TM;
    const int a_seg = __builtin_amdgcn_readfirstlane(tid / TM);
    int pb, qb, abase;                          // P', Q' of the block, dy image offset
    {
        const int m = m0 + a_row;
        if (m < p.M) {
            uint32_t n, pq, pp, q;
            p.div_blk.divmod((uint32_t)m, n, pq);
            p.div_wb.divmod(pq, pp, q);
            pb = (int)pp + p.P0;
            qb = (int)q + p.Q0;
            abase = (int)n * p.sdn;
        } else {
            pb = -0x40000000;   // every dy row pb - i is negative: the row reads as zeros
            qb = 0;
            abase = 0;
        }
    }
    // ---- B loader: thread -> one column z = (c, a, b), one channel segment
    const bool b_loader = tid < B_TPR * TN;
    const int b_row = tid % TN;
    const int b_seg = b_loader ? tid / TN : 0;
    int b_cbase = 0, b_a = 0, b_b = 0;
    const bool b_ok = b_loader && n0 + b_row < p.Z;
    {
        uint32_t c, ab, a, b;
        p.div_uv.divmod((uint32_t)(b_ok ? n0 + b_row : 0), c, ab);
        p.div_v.divmod(ab, a, b);
        b_cbase = (int)c * p.R * p.S;
        b_a = (int)a;
        b_b = (int)b;
    }
    const int krs = p.C * p.R * p.S;            // filter k's stride in F

    In a_val[A_EPT];
    In b_val[B_EPT];

    // chunk ch = channel_block * (D*E) + tap, tap = i * E + j
    auto chunk_of = [&](int ch, int& k0, int& i, int& j) {
        uint32_t kb, t, ti, tj;
        p.div_de.divmod((uint32_t)ch, kb, t);
        p.div_e.divmod(t, ti, tj);
        k0 = (int)kb * TK;
        i = (int)ti;
        j = (int)tj;
    };

    auto load_a = [&](int ch) {
        int k0, i, j;
        chunk_of(ch, k0, i, j);
        k0 += a_seg * A_EPT;                    // wave-uniform
        const int pr = pb - i, qc = qb - j;
        const bool ok = (unsigned)pr < (unsigned)p.P && (unsigned)qc < (unsigned)p.Q;
        const In* src = dy + (ok ? abase + k0 * p.sdk + pr * p.sdp + qc * p.sdq : 0);
#pragma unroll
        for (int e = 0; e < A_EPT; ++e)
            a_val[e] = (ok && k0 + e < p.K) ? load_elem(src + e * p.sdk) : In(0);
    };

    auto load_b = [&](int ch) {
        int k0, i, j;
        chunk_of(ch, k0, i, j);
        k0 += b_seg * B_EPT;
        const int r = p.u * i + b_a, s = p.v * j + b_b;
        const bool ok = b_ok && r < p.R && s < p.S;
        const In* src = f + (ok ? k0 * krs + b_cbase + r * p.S + s : 0);
#pragma unroll
        for (int e = 0; e < B_EPT; ++e)
            b_val[e] = (ok && k0 + e < p.K) ? load_elem(src + e * krs) : In(0);
    };

    auto store_tiles = [&](int buf) {
        unsigned char* a_dst = smem + buf * BUF_BYTES + a_row * PITCH + a_seg * A_EPT * (int)sizeof(In);
        unsigned char* b_dst = smem + buf * BUF_BYTES + A_BYTES + b_row * PITCH + b_seg * B_EPT * (int)sizeof(In);
        uint32_t aw[A_WORDS];
        uint32_t bw[B_WORDS];
        Pack<In>::to_words(a_val, aw);
        Pack<In>::to_words(b_val, bw);
        lds_store_words<A_WORDS>(a_dst, aw);
        if (B_TPR * TN == NT || b_loader) lds_store_words<B_WORDS>(b_dst, bw);
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

    const int nchunks = (p.K + TK - 1) / TK * (int)p.div_de.d;

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
            for (int t = 0; t < FRAG_VECS; ++t) fa[i][t] = src[t];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4* src = reinterpret_cast<const u32x4*>(
                b_src + (wn * WN + j * BM + lrow) * PITCH + lgrp * SEG * (int)sizeof(In));
#pragma unroll
            for (int t = 0; t < FRAG_VECS; ++t) fb[j][t] = src[t];
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma(fa[i], fb[j], t, acc[i][j]);
            // the other buffer's last readers finished before the previous barrier
            if (t == STEPS / 2 && more) store_tiles(cur ^ 1);
        }
        __syncthreads();
    }

    // ---- epilogue: depth-to-space through a per-wave LDS stage; a lane
    // stores rows m = lane % BM of a block for LG-strided columns
    constexpr int STAGE_PITCH = BM + 1;
    constexpr int LG = 64 / BM;
    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Out* __restrict__ dx = static_cast<Out*>(p.dx);
    Acc* stage = reinterpret_cast<Acc*>(smem) + wave * BM * STAGE_PITCH;
    const int mw0 = m0 + wm * WM;
    const int nw0 = n0 + wn * WN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int gm = mw0 + i * BM + lane % BM;
        const bool row_ok = gm < p.M;
        int hb = 0, wb = 0, moff = 0;
        if (row_ok) {
            uint32_t n, pq, pp, q;
            p.div_blk.divmod((uint32_t)gm, n, pq);
            p.div_wb.divmod(pq, pp, q);
            hb = p.u * (int)pp - p.h_off;       // dx row of phase a = 0
            wb = p.v * (int)q - p.w_off;
            moff = (int)n * p.sxn + hb * p.sxh + wb * p.sxw;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int e = 0; e < Pol::NACC; ++e)
                stage[Pol::col(e, lane) * STAGE_PITCH + Pol::row(e, lane)] = acc[i][j][e];
            const int bk0 = nw0 + j * BM;
#pragma unroll
            for (int t = 0; t < BM / LG; ++t) {
                const int kl = lane / BM + LG * t;
                const int z = bk0 + kl;
                if (!row_ok || z >= p.Z) continue;
                uint32_t c, ab, a, b;
                p.div_uv.divmod((uint32_t)z, c, ab);
                p.div_v.divmod(ab, a, b);
                const int h = hb + (int)a, w = wb + (int)b;
                if ((unsigned)h >= (unsigned)p.H || (unsigned)w >= (unsigned)p.W) continue;
                const int off = moff + (int)c * p.sxc + (int)a * p.sxh + (int)b * p.sxw;
                Acc val = alpha * stage[kl * STAGE_PITCH + lane % BM];
                if (beta != Acc(0)) val += beta * (Acc)dx[off];
                dx[off] = (Out)val;
            }
        }
    }
}

constexpr int kSpTM = 128;

// D x E taps per phase, the block grid and the decode constants; tn, the
// column tile (64, or 48 where that pads the C*u*v columns less)
bool subpixel_args(const ConvParams& p, SubpixelArgs& a, int tn)
{
    if (p.u < 1 || p.v < 1) return false;
    const int D = (p.R + p.u - 1) / p.u, E = (p.S + p.v - 1) / p.v;
    a.dy = p.x;
    a.w = p.w;
    a.dx = p.y;
    a.N = p.N;
    a.K = p.K;
    a.C = p.C;
    a.P = p.P;
    a.Q = p.Q;
    a.H = p.H;
    a.W = p.W;
    a.R = p.R;
    a.S = p.S;
    a.u = p.u;
    a.v = p.v;
    a.P0 = p.pad_top / p.u;
    a.Q0 = p.pad_left / p.v;
    a.h_off = p.pad_top - a.P0 * p.u;
    a.w_off = p.pad_left - a.Q0 * p.v;
    const int HB = (p.H - 1 + p.pad_top) / p.u - a.P0 + 1;
    const int WB = (p.W - 1 + p.pad_left) / p.v - a.Q0 + 1;
    a.sdn = p.sxn;
    a.sdk = p.sxc;
    a.sdp = p.sxh;
    a.sdq = p.sxw;
    a.sxn = p.syn;
    a.sxc = p.syk;
    a.sxh = p.syp;
    a.sxw = p.syq;
    const int64_t M = (int64_t)p.N * HB * WB;
    const int64_t Z = (int64_t)p.C * p.u * p.v;
    if (M >= (int64_t(1) << 31) || Z >= (int64_t(1) << 30) || (int64_t)D * E * ((p.K + 15) / 16) >= (int64_t(1) << 30))
        return false;
    a.M = (int)M;
    a.Z = (int)Z;
    a.div_blk = FastDiv((uint32_t)(HB * WB));
    a.div_wb = FastDiv((uint32_t)WB);
    a.div_de = FastDiv((uint32_t)(D * E));
    a.div_e = FastDiv((uint32_t)E);
    a.div_uv = FastDiv((uint32_t)(p.u * p.v));
    a.div_v = FastDiv((uint32_t)p.v);
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.m_tiles = (a.M + kSpTM - 1) / kSpTM;
    a.tile_rev = p.tile_rev;
    a.n_tiles = (a.Z + tn - 1) / tn;
    return true;
}

// fp32: 48-wide column tiles of 16x16 blocks when they pad the columns less
// than 64-wide ones of 32x32 blocks
int subpixel_tn(DType dt, const ConvParams& p)
{
    const int64_t z = (int64_t)p.C * p.u * p.v;
    if (dt != DType::F32) return 64;
    return (z + 47) / 48 * 48 < (z + 63) / 64 * 64 ? 48 : 64;
}

}  // namespace

bool bwd_data_subpixel_fits(const ConvParams& p)
{
    SubpixelArgs a;
    return subpixel_args(p, a, 64);
}

hipError_t launch_bwd_data_subpixel(DType dt, const ConvParams& p, hipStream_t stream)
{
    SubpixelArgs a;
    const int tn = subpixel_tn(dt, p);
    if (!subpixel_args(p, a, tn)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.m_tiles * a.n_tiles));
    if (dt == DType::F32 && tn == 48)
        hipLaunchKernelGGL((conv_bwd_data_subpixel_kernel<PolF32x16V, kSpTM, 48, 4, 1, 16>), grid, dim3(256), 0,
                           stream, a);
    else if (dt == DType::F32)
        hipLaunchKernelGGL((conv_bwd_data_subpixel_kernel<PolF32, kSpTM, 64, 2, 2, 16>), grid, dim3(256), 0,
                           stream, a);
    else if (dt == DType::F64)
        hipLaunchKernelGGL((conv_bwd_data_subpixel_kernel<PolF64, kSpTM, 64, 2, 2, 8>), grid, dim3(256), 0,
                           stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace miconv
