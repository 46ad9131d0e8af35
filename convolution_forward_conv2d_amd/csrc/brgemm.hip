// brgemm.hip -- the batch-reduce GEMM as a standalone primitive on gfx950
// MFMA (single-building-block page, "Proposed Method": the products of a
// batch of input sub-tensor blocks reduced into one output block):
//
//   C[m, n] = alpha * sum_{i < batch} sum_{k < K} A_i[m, k] * B_i[k, n] + beta * C[m, n]
//
// A_i[m, k] = a[i*sa_i + m*sa_m + k*sa_k], B_i[k, n] = b[i*sb_i + k*sb_k + n*sb_n],
// C[m, n] = c[m*sc_m + n*sc_n].  A fully-connected layer is one block
// product (batch 1) or its input features cut into blocks (batch > 1).
// The reduction index t = i*k + kk runs over all blocks; a chunk of it may
// span several blocks.
//
// Two kernels, no workspace (the reduction is never split across
// workgroups, so the result does not depend on timing):
//   brgemm_kernel    -- large products: 4 waves share a TM x TN tile through
//                       double-buffered LDS, as the convolution kernels do;
//   brgemm_ws_kernel -- skinny products: the waves split the reduction.
//
// Parameters in a ConvParams: x = a with sxn = sa_i, sxh = sa_m, sxw = sa_k;
// w = b with sdn = sb_i, sdk = sb_k, sdq = sb_n; y = c with syn = sc_m,
// syk = sc_n (div_pq = div_q = 1: a row is one m); M = the rows, K = the
// columns (n), Kred = the per-block reduction length k, N = batch,
// div_rs divides by k.
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

// fp32 on 16x16 blocks, operands taken from 16-byte LDS vectors like PolF32
struct PolF32x16V : PolF32x16 {
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        float a = __uint_as_float(fa[t >> 2][t & 3]);
        float b = __uint_as_float(fb[t >> 2][t & 3]);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// bf16 on 16x16 blocks (v_mfma_f32_16x16x32_bf16): lane l gives A[l%16][8*(l/16) .. +8]
// and B likewise; the accumulator layout is that of every 16x16 fp32 block.
struct PolBF16x16 {
    using In = uint16_t;
    using Acc = float;
    using Out = float;
    using AccV = f32x4;
    static constexpr int BM = 16, G = 4, V = 8, NACC = 4;
    __device__ static AccV mfma(const u32x4* fa, const u32x4* fb, int t, AccV c) {
        bf16x8 a = __builtin_bit_cast(bf16x8, fa[t]);
        bf16x8 b = __builtin_bit_cast(bf16x8, fb[t]);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static int row(int i, int lane) { return 4 * (lane >> 4) + i; }
    __device__ static int col(int, int lane) { return lane & 15; }
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Consecutive logical tiles share an XCD's L2.  With few m tiles (a skinny
// product) the m tiles of one n tile run together, so the large B columns
// are fetched from HBM once per XCD; otherwise the n tiles of one m tile do.
struct TileMN {
    int mt, nt;
};

__device__ __forceinline__ TileMN tile_coords(int m_tiles, int n_tiles, int rev)
{
    const int tile = xcd_logical_tile((int)blockIdx.x, m_tiles * n_tiles, rev);
    TileMN t;
    if (m_tiles <= n_tiles) {
        t.nt = tile / m_tiles;
        t.mt = tile - t.nt * m_tiles;
    } else {
        t.mt = tile / n_tiles;
        t.nt = tile - t.mt * n_tiles;
    }
    return t;
}

// Large products.  A workgroup of 4 waves owns a TM x TN block of C and
// runs the whole reduction in chunks of TK: the chunk's A rows and B
// columns go global -> VGPR -> LDS (double-buffered) and feed the MFMA
// policies of the convolution kernels, WAVES_M x WAVES_N waves each taking a
// sub-tile.  VEC (A and B contiguous along k, a chunk row one 128-byte
// line): thread (r, s) of each group of 8 loads 16-byte segment s of row r,
// so a load instruction covers 8 whole lines; loads are unconditional (the
// last chunk re-read past the end) and out-of-range values are zeroed when
// stored to LDS.  Otherwise each thread gathers a run of elements one by one
// through the general strides.
template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK, bool VEC>
__global__ void __launch_bounds__(256)
brgemm_kernel(const ConvParams p)
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
    constexpr int A_BYTES = TM * PITCH;
    constexpr int B_BYTES = TN * PITCH;
    constexpr int BUF_BYTES = A_BYTES + B_BYTES;
    constexpr int VE = 16 / (int)sizeof(In);
    // gather path: a thread's run of A_EPT (B_EPT) consecutive reduction elements
    constexpr int A_TPR = NT / TM;
    constexpr int A_EPT = TK / A_TPR;
    constexpr int B_TPR = NT / TN;
    constexpr int B_EPT = TK / B_TPR;
    constexpr int A_WORDS = A_EPT * (int)sizeof(In) / 4;
    constexpr int B_WORDS = B_EPT * (int)sizeof(In) / 4;
    // vector path: rows per thread
    constexpr int AV = TM / 32;
    constexpr int BV = TN / 32;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WM % BM == 0 && WN % BM == 0, "wave tile must hold whole MFMA blocks");
    static_assert(NT % TM == 0 && NT % TN == 0 && A_EPT >= 1 && B_EPT >= 1, "loader shapes");
    static_assert(SEG * (int)sizeof(In) % 16 == 0, "lane slice must be whole 16-byte vectors");
    static_assert((A_EPT * (int)sizeof(In)) % 4 == 0 && (B_EPT * (int)sizeof(In)) % 4 == 0,
                  "loader slices must be whole words");
    static_assert(!VEC || (TK * (int)sizeof(In) == 128 && TM % 32 == 0 && TN % 32 == 0),
                  "vector path: a chunk row is one 128-byte line, 32 rows per 256 threads");
    static_assert(4 * BM * (BM + 1) * (int)sizeof(Acc) <= 2 * BUF_BYTES, "epilogue stage fits");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const TileMN tc = tile_coords(p.m_tiles, p.n_tiles, p.tile_rev);
    const int m0 = tc.mt * TM;
    const int n0 = tc.nt * TN;

    const In* __restrict__ a = static_cast<const In*>(p.x);
    const In* __restrict__ b = static_cast<const In*>(p.w);
    const int kb = p.Kred;
    const int L = p.N * kb;
    const int nchunks = (L + TK - 1) / TK;

    // ---- vector path state
    const int vr = tid >> 3;
    const int vs = tid & 7;
    const In* avp[AV];
    bool avok[AV];
    const In* bvp[BV];
    bool bvok[BV];
    u32x4 ar[AV];
    u32x4 br[BV];
    bool cin = false;
    // ---- gather path state
    const int a_row = tid / A_TPR;
    const int a_seg = tid % A_TPR;
    const bool a_ok = m0 + a_row < p.M;
    const In* __restrict__ arow = a + (a_ok ? m0 + a_row : 0) * p.sxh;
    const int b_row = tid / B_TPR;
    const int b_seg = tid % B_TPR;
    const bool b_ok = n0 + b_row < p.K;
    const In* __restrict__ bcol = b + (b_ok ? n0 + b_row : 0) * p.sdq;
    In a_val[VEC ? 1 : A_EPT];
    In b_val[VEC ? 1 : B_EPT];

    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int r = m0 + j * 32 + vr;
            avok[j] = r < p.M;
            avp[j] = a + (avok[j] ? r : 0) * p.sxh;
        }
#pragma unroll
        for (int j = 0; j < BV; ++j) {
            const int c = n0 + j * 32 + vr;
            bvok[j] = c < p.K;
            bvp[j] = b + (bvok[j] ? c : 0) * p.sdq;
        }
    }

    // chunk ch (clamped by the caller to an existing one) into registers
    auto load_chunk = [&](int ch) {
        if constexpr (VEC) {
            const int t = ch * TK + vs * VE;
            cin = t < L;
            uint32_t i, kk;
            p.div_rs.divmod((uint32_t)(cin ? t : 0), i, kk);
            const int aoff = (int)i * p.sxn + (int)kk;
            const int boff = (int)i * p.sdn + (int)kk;
#pragma unroll
            for (int j = 0; j < AV; ++j) ar[j] = *reinterpret_cast<const u32x4*>(avp[j] + aoff);
#pragma unroll
            for (int j = 0; j < BV; ++j) br[j] = *reinterpret_cast<const u32x4*>(bvp[j] + boff);
        } else {
            auto run = [&](const In* __restrict__ base, bool ok, int t0, int s_i, int s_k, auto& val) {
                constexpr int E = sizeof(val) / sizeof(In);
                uint32_t i, kk;
                p.div_rs.divmod((uint32_t)t0, i, kk);
                int ii = (int)i, k2 = (int)kk;
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    val[j] = (ok && t0 + j < L) ? load_elem(base + ii * s_i + k2 * s_k) : In(0);
                    if (++k2 == kb) {
                        k2 = 0;
                        ++ii;
                    }
                }
            };
            run(arow, a_ok, ch * TK + a_seg * A_EPT, p.sxn, p.sxw, a_val);
            run(bcol, b_ok, ch * TK + b_seg * B_EPT, p.sdn, p.sdk, b_val);
        }
    };

    auto store_tiles = [&](int buf) {
        unsigned char* base = smem + buf * BUF_BYTES;
        if constexpr (VEC) {
            const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < AV; ++j)
                *reinterpret_cast<u32x4*>(base + (j * 32 + vr) * PITCH + vs * 16) = (cin && avok[j]) ? ar[j] : zero;
#pragma unroll
            for (int j = 0; j < BV; ++j)
                *reinterpret_cast<u32x4*>(base + A_BYTES + (j * 32 + vr) * PITCH + vs * 16) =
                    (cin && bvok[j]) ? br[j] : zero;
        } else {
            uint32_t aw[A_WORDS];
            uint32_t bw[B_WORDS];
            Pack<In>::to_words(a_val, aw);
            Pack<In>::to_words(b_val, bw);
            lds_store_words<A_WORDS>(base + a_row * PITCH + a_seg * A_EPT * (int)sizeof(In), aw);
            lds_store_words<B_WORDS>(base + A_BYTES + b_row * PITCH + b_seg * B_EPT * (int)sizeof(In), bw);
        }
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

    if (nchunks > 0) {
        load_chunk(0);
        store_tiles(0);
        __syncthreads();
    }
    for (int ch = 0; ch < nchunks; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nchunks;
        // unconditional: a load under a branch makes the compiler's wait
        // counts assume the path without it and stall on the chunk just issued
        load_chunk(more ? ch + 1 : ch);
        __builtin_amdgcn_sched_barrier(0);
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

// End of a wave-split tile: the NW waves' partial TM x TN tiles meet in
// LDS (stage, NW * TM * SP elements) and every thread sums, in wave order,
// the partials of the outputs it stores (consecutive threads, consecutive
// columns of a row).  C <- alpha * sum + beta * C, C not read when beta == 0.
template <class Pol, int TM, int TN, int NW, class AccV, int FM, int FN>
__device__ __forceinline__ void ws_reduce_store(const ConvParams& p, typename Pol::Acc* stage,
                                                AccV (&acc)[FM][FN], int m0, int n0, int wave, int lane)
{
    using Acc = typename Pol::Acc;
    constexpr int BM = Pol::BM;
    constexpr int SP = TN + 16 / (int)sizeof(Acc);
    Acc* mine = stage + wave * TM * SP;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < Pol::NACC; ++e)
                mine[(i * BM + Pol::row(e, lane)) * SP + j * BM + Pol::col(e, lane)] = acc[i][j][e];
    __syncthreads();

    const Acc alpha = (Acc)p.alpha;
    const Acc beta = (Acc)p.beta;
    Acc* __restrict__ y = static_cast<Acc*>(p.y);
#pragma unroll
    for (int q = 0; q < TM * TN / (NW * 64); ++q) {
        const int e = q * NW * 64 + (int)threadIdx.x;
        const int r = e / TN;
        const int c = e - r * TN;
        Acc sum = stage[r * SP + c];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += stage[w * TM * SP + r * SP + c];
        const int gm = m0 + r, gn = n0 + c;
        if (gm < p.M && gn < p.K) {
            const int off = gm * p.syn + gn * p.syk;
            Acc val = alpha * sum;
            if (beta != Acc(0)) val += beta * y[off];
            y[off] = val;
        }
    }
}

// Skinny products (few output tiles, long reduction: a fully-connected
// layer at small minibatch).  The NW waves of a workgroup split every chunk
// of TK = NW * TKW reduction elements, wave w taking [w*TKW, (w+1)*TKW), and
// own the whole TM x TN tile each; the partial tiles are summed at the end
// (ws_reduce_store).  No operand is shared between waves.  A wave loads its
// rows of the chunk whole, a row's TKW elements being one 128-byte line:
// 8 lanes per row, 8 rows (8 lines) per load instruction.  (Loading MFMA
// fragments straight into registers gives a row only 4 lanes per
// instruction and touches twice the lines; measured on MI355X it halves the
// bf16 throughput.)  The wave writes its rows to its own LDS region,
// 16-byte segment s of row r at segment s ^ (r % 8), and reads its MFMA
// fragments back from there: the region is private to the wave (LDS
// operations of one wave complete in order), so the main loop has no
// workgroup barrier.  Loads run NBUF - 1 chunks ahead in registers.  A and
// B must be contiguous along k with k a multiple of a 16-byte vector and
// every vector aligned (brgemm_ws_run).
namespace {
constexpr int kBrBufWord3 = 0x00020000;           // raw 32-bit buffer, range-checked per dword

__device__ __forceinline__ __amdgpu_buffer_rsrc_t br_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBrBufWord3);
}
__device__ __forceinline__ u32x4 br_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
    return u32x4{v[0], v[1], v[2], v[3]};
}
}  // namespace

template <class Pol, int TM, int TN, int NW, int TKW, int NBUF>
__global__ void __launch_bounds__(NW * 64)
brgemm_ws_kernel(const ConvParams p)
{
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using AccV = typename Pol::AccV;
    constexpr int BM = Pol::BM;
    constexpr int FM = TM / BM;
    constexpr int FN = TN / BM;
    constexpr int SEG = TKW / Pol::G;
    constexpr int FV = SEG * (int)sizeof(In) / 16;
    constexpr int STEPS = SEG / Pol::V;
    constexpr int TK = NW * TKW;
    constexpr int VE = 16 / (int)sizeof(In);
    constexpr int RB = TKW * (int)sizeof(In);          // bytes of one row's chunk
    constexpr int AI = TM / 8;                          // load instructions per chunk, A
    constexpr int BI = TN / 8;                          // and B
    constexpr int WBYTES = (TM + TN) * RB;              // a wave's transposition region
    constexpr int SP = TN + 16 / (int)sizeof(Acc);
    constexpr int STAGE_BYTES = NW * TM * SP * (int)sizeof(Acc);
    constexpr int SMEM = NW * WBYTES > STAGE_BYTES ? NW * WBYTES : STAGE_BYTES;
    static_assert(TM % BM == 0 && TN % BM == 0 && TM % 8 == 0 && TN % 8 == 0, "whole MFMA blocks");
    static_assert(RB == 128 && FV * Pol::G == 8, "a row's chunk is one 128-byte line of 8 segments");
    static_assert(TM * TN % (NW * 64) == 0, "reduction split");
    static_assert(SMEM <= 160 * 1024, "LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const TileMN tc = tile_coords(p.m_tiles, p.n_tiles, p.tile_rev);
    const int m0 = tc.mt * TM;
    const int n0 = tc.nt * TN;

    const int kb = p.Kred;
    const int L = p.N * kb;
    // A and B through range-checked buffer descriptors (host: each under
    // 2^30 bytes): a row past M or N, or a chunk past the reduction, reads at
    // an offset of at least 2^30 and gets zeros, so nothing is selected when
    // the chunk is written to LDS and no load waits on a test
    constexpr uint32_t OUT = 0x40000000u;
    constexpr int ES = (int)sizeof(In);
    const int64_t a_elems = (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.M - 1) * p.sxh + (int64_t)(kb - 1) * p.sxw + 1;
    const int64_t b_elems = (int64_t)(p.N - 1) * p.sdn + (int64_t)(p.K - 1) * p.sdq + (int64_t)(kb - 1) * p.sdk + 1;
    const __amdgpu_buffer_rsrc_t ar = br_rsrc(p.x, a_elems * ES);
    const __amdgpu_buffer_rsrc_t brs = br_rsrc(p.w, b_elems * ES);

    // loader coordinates: row lr (+ 8 per instruction), 16-byte segment sg
    const int lr = lane >> 3;
    const int sg = lane & 7;
    uint32_t arow[AI];                                  // byte offset of the row (OUT: none)
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int r = m0 + j * 8 + lr;
        arow[j] = r < p.M ? (uint32_t)(r * p.sxh * ES) : OUT;
    }
    uint32_t bcol[BI];
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int c = n0 + j * 8 + lr;
        bcol[j] = c < p.K ? (uint32_t)(c * p.sdq * ES) : OUT;
    }

    // The loaded values stay raw in the ring until the chunk is due.
    u32x4 sa[NBUF][AI];
    u32x4 sb[NBUF][BI];
    auto load = [&](auto buf_c, int ch) {
        constexpr int B = decltype(buf_c)::value;
        const int t = ch * TK + wave * TKW + sg * VE;
        const bool in = t < L;
        uint32_t i, kk;
        if (p.N == 1) {                                 // one product: no batch index
            i = 0;
            kk = (uint32_t)t;
        } else {
            p.div_rs.divmod((uint32_t)(in ? t : 0), i, kk);
        }
        const uint32_t aoff = in ? (uint32_t)(((int)i * p.sxn + (int)kk) * ES) : OUT;
        const uint32_t boff = in ? (uint32_t)(((int)i * p.sdn + (int)kk) * ES) : OUT;
#pragma unroll
        for (int j = 0; j < AI; ++j) sa[B][j] = br_load16(ar, arow[j] + aoff);
#pragma unroll
        for (int j = 0; j < BI; ++j) sb[B][j] = br_load16(brs, bcol[j] + boff);
    };

    unsigned char* region = smem + wave * WBYTES;
    const int lrow = lane % BM;
    const int lgrp = lane / BM;
    u32x4 fa[FM][FV];
    u32x4 fb[FN][FV];
    // staged chunk -> the wave's LDS region -> MFMA fragments
    auto transpose = [&](auto buf_c) {
        constexpr int B = decltype(buf_c)::value;
#pragma unroll
        for (int j = 0; j < AI; ++j)
            *reinterpret_cast<u32x4*>(region + (j * 8 + lr) * RB + ((sg ^ lr) << 4)) = sa[B][j];
#pragma unroll
        for (int j = 0; j < BI; ++j)
            *reinterpret_cast<u32x4*>(region + (TM + j * 8 + lr) * RB + ((sg ^ lr) << 4)) = sb[B][j];
        // vector v of lane group g is segment v*G + g of its row
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int v = 0; v < FV; ++v)
                fa[f][v] = *reinterpret_cast<const u32x4*>(
                    region + (f * BM + lrow) * RB + (((v * Pol::G + lgrp) ^ (lrow & 7)) << 4));
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int v = 0; v < FV; ++v)
                fb[f][v] = *reinterpret_cast<const u32x4*>(
                    region + (TM + f * BM + lrow) * RB + (((v * Pol::G + lgrp) ^ (lrow & 7)) << 4));
    };

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};
    auto compute = [&]() {
#pragma unroll
        for (int t = 0; t < STEPS; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma(fa[i], fb[j], t, acc[i][j]);
    };

    // Every load in the pipeline is issued unconditionally (chunks past the
    // end re-read the last chunk, into a slot that is never consumed): a
    // load under a branch makes the compiler's wait counts assume the path
    // without it and stall on the chunk just issued.
    const int nch = (L + TK - 1) / TK;
    if (nch > 0) {
        static_for<0, NBUF - 1>([&](auto bc) {
            constexpr int c = decltype(bc)::value;
            load(bc, c < nch ? c : nch - 1);
        });
        int ch = 0;
        for (; ch + NBUF <= nch; ch += NBUF) {
            static_for<0, NBUF>([&](auto bc) {
                constexpr int cur = decltype(bc)::value;
                const int nxt = ch + cur + NBUF - 1;
                load(std::integral_constant<int, (cur + NBUF - 1) % NBUF>{}, nxt < nch ? nxt : nch - 1);
                // keep the loads ahead of this chunk's work (the scheduler
                // would sink them next to their use a chunk later)
                __builtin_amdgcn_sched_barrier(0);
                transpose(bc);
                compute();
            });
        }
        static_for<0, NBUF - 1>([&](auto bc) {
            if (ch + decltype(bc)::value < nch) {
                transpose(bc);
                compute();
            }
        });
    }

    __syncthreads();     // the stage below reuses the transposition regions
    ws_reduce_store<Pol, TM, TN, NW>(p, reinterpret_cast<Acc*>(smem), acc, m0, n0, wave, lane);
}

// An operand can be read as 16-byte vectors along the reduction when it is
// contiguous along k, k is a multiple of E elements (a vector never crosses
// into the next batch entry or past the end) and every vector is aligned.
template <class In>
static bool vec_ok(int E, const void* base, int s_i, int s_mn, int s_k, int k, int batch, int rows)
{
    constexpr int VE = 16 / (int)sizeof(In);
    return E % VE == 0 && s_k == 1 && k % E == 0 && (batch <= 1 || s_i % VE == 0) &&
           (rows <= 1 || s_mn % VE == 0) && (uintptr_t)base % 16 == 0;
}

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int TK>
static hipError_t launch_br_variant(const ConvParams& p0, hipStream_t stream)
{
    using In = typename Pol::In;
    ConvParams p = p0;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    constexpr int VE = 16 / (int)sizeof(In);
    constexpr bool CAN = TK * (int)sizeof(In) == 128 && TM % 32 == 0 && TN % 32 == 0;
    const bool vec = CAN && vec_ok<In>(VE, p.x, p.sxn, p.sxh, p.sxw, p.Kred, p.N, p.M) &&
                     vec_ok<In>(VE, p.w, p.sdn, p.sdq, p.sdk, p.Kred, p.N, p.K);
    if (vec)
        hipLaunchKernelGGL((brgemm_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, CAN>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((brgemm_kernel<Pol, TM, TN, WAVES_M, WAVES_N, TK, false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class Pol, int TM, int TN, int NW, int TKW, int NBUF>
static hipError_t launch_ws_variant(const ConvParams& p0, hipStream_t stream)
{
    using In = typename Pol::In;
    ConvParams p = p0;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    constexpr int VE = 16 / (int)sizeof(In);
    const bool vec = vec_ok<In>(VE, p.x, p.sxn, p.sxh, p.sxw, p.Kred, p.N, p.M) &&
                     vec_ok<In>(VE, p.w, p.sdn, p.sdq, p.sdk, p.Kred, p.N, p.K);
    if (!vec) return hipErrorInvalidValue;     // the host picks these variants only for such operands
    // the buffer descriptors' range: A and B under 2^30 bytes
    const int64_t es = (int64_t)sizeof(In);
    const int64_t a_elems = (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.M - 1) * p.sxh + (int64_t)(p.Kred - 1) * p.sxw + 1;
    const int64_t b_elems = (int64_t)(p.N - 1) * p.sdn + (int64_t)(p.K - 1) * p.sdq + (int64_t)(p.Kred - 1) * p.sdk + 1;
    if (es * a_elems >= ((int64_t)1 << 30) || es * b_elems >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((brgemm_ws_kernel<Pol, TM, TN, NW, TKW, NBUF>), grid, dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

//        name              policy      TM   TN  waves  TK
#define MICONV_BR_VARIANTS(X)                            \
    X(BR_F32_128x128, PolF32, 128, 128, 2, 2, 32)        \
    X(BR_F32_64x64, PolF32, 64, 64, 2, 2, 32)            \
    X(BR_F32_32x64, PolF32x16V, 32, 64, 2, 2, 32)        \
    X(BR_F64_64x64, PolF64, 64, 64, 2, 2, 16)            \
    X(BR_F64_32x64, PolF64, 32, 64, 2, 2, 16)            \
    X(BR_BF16_128x128, PolBF16, 128, 128, 2, 2, 64)      \
    X(BR_BF16_64x64, PolBF16, 64, 64, 2, 2, 64)          \
    X(BR_BF16_32x128, PolBF16, 32, 128, 1, 4, 64)

//        name              policy      TM  TN  waves  per-wave TK  ring
#define MICONV_WS_VARIANTS(X)                            \
    X(WS_F32_64x64, PolF32, 64, 64, 8, 32, 2)            \
    X(WS_F32_32x64, PolF32, 32, 64, 8, 32, 2)            \
    X(WS_F32_16x32, PolF32x16V, 16, 32, 8, 32, 2)        \
    X(WS_F64_32x64, PolF64, 32, 64, 8, 16, 2)            \
    X(WS_F64_16x32, PolF64, 16, 32, 8, 16, 2)            \
    X(WS_BF16_32x64, PolBF16x16, 32, 64, 8, 64, 2)       \
    X(WS_BF16_16x32, PolBF16x16, 16, 32, 8, 64, 2)

hipError_t launch_brgemm(Variant v, const ConvParams& p, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, tk) \
    case Variant::name: return launch_br_variant<pol, tm, tn, wmm, wnn, tk>(p, stream);
        MICONV_BR_VARIANTS(X)
#undef X
#define X(name, pol, tm, tn, nw, tkw, nbuf) \
    case Variant::name: return launch_ws_variant<pol, tm, tn, nw, tkw, nbuf>(p, stream);
        MICONV_WS_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

int brgemm_ws_run(Variant v)
{
    switch (v) {
#define X(name, pol, tm, tn, nw, tkw, nbuf) \
    case Variant::name: return 16 / (int)sizeof(pol::In);
        MICONV_WS_VARIANTS(X)
#undef X
    default: return 0;
    }
}

}  // namespace miconv
