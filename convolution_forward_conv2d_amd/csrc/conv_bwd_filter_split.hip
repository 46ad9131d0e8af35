// conv_bwd_filter_split.hip -- filter gradient of the convolution for layers
// whose dw is too small to give every compute unit a tile of its own.
//
//   dw[k,c,r,s] = alpha * sum_{n,p,q} dy[n,k,p,q] * X(n, c, p*u + r - pad_top, q*v + s - pad_left)
//               + beta * dw[k,c,r,s]
//
// (the backward routine in F that the cuDNN page, "Proposed Method", lists
// beside the forward one), as the matrix product of conv_bwd_filter.hip:
// rows k (M = K), columns j = (c, r, s) (C*R*S), reduction over the
// positions t = (n, p, q) (L = N*P*Q), A[k, t] = dy, B[t, j] = gathered x.
//
// A first layer has few filters and few input channels -- 96 x 363 for an
// 11x11 filter bank on 3 channels, 32 x 451 for a 41x11 bank on one -- so
// 64 x 64 tiles of dw number 12 or 8 and the rest of the 256 compute units
// idle through a reduction over hundreds of thousands of positions.  With no
// workspace the reduction cannot be split across workgroups (partial sums
// need a buffer; atomics break the bit-identical rerun), so it is split
// inside one: a workgroup owns a small TM x TN tile (32 x 32 or 16 x 16, so
// that there are several times more tiles) and KS groups of waves take
// disjoint parts of every chunk of positions.  At the end groups 1..KS-1
// hand their partial sums to group 0 through LDS, which adds them in group
// order: the result does not depend on timing.
//
// A chunk of TK = KS * TKG positions is staged in LDS for A (TM rows) and B
// (TN rows), double-buffered.  The loader gives each wave one 64-position
// segment of the chunk and a set of rows; a lane loads one position of each
// of those rows, so every load instruction reads 64 consecutive positions of
// one row -- contiguous along q for dy, a stride-v gather of x -- and the
// column (c, r, s) of a B row is a wave-uniform (scalar) quantity.  The
// loads are range-checked buffer loads: positions past the reduction and
// taps in the padding read an offset outside the tensor and get zero, with
// no select on the loaded value.  A chunk is loaded two MFMA phases before
// it is stored to LDS.  Group g's waves then read positions
// [g*TKG, (g+1)*TKG) of their rows as MFMA fragments.
//
// Parameters as in conv_bwd_filter.hip: x and its strides sx*; w = dy and
// its strides sd*; y = dw packed K,C,R,S (syn = C*R*S, syk = 1); M = K,
// K = C*R*S, Kred = N*P*Q; div_opq, div_oq divide by P*Q and Q, div_rs and
// div_s by R*S and S.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {
namespace {

// element t of a lane's fragment slice (t is a compile-time index after
// unrolling).  The vector element is copied to a scalar before the bit
// cast: a bit cast applied to the element expression itself read the
// vector's first element on this compiler.
__device__ __forceinline__ float frag_elem(const u32x4* f, int t, float)
{
    const uint32_t w = f[t >> 2][t & 3];
    return __uint_as_float(w);
}
__device__ __forceinline__ double frag_elem(const u32x4* f, int t, double)
{
    const uint64_t lo = f[t >> 1][2 * (t & 1)];
    const uint64_t hi = f[t >> 1][2 * (t & 1) + 1];
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Raw buffer loads: with a buffer resource whose record count is the
// tensor's size in bytes, a load at an offset past it returns zero and
// touches no memory.  Positions past the reduction and taps in the padding
// are loaded from offset kOutside; valid offsets are below 2^31 (the plan
// admits only tensors smaller than that), so kOutside plus any scalar
// offset stays out of range without wrapping.
constexpr int kBufWord3 = 0x00020000;        // raw 32-bit buffer, range-checked
constexpr int kOutside = (int)0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, float)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ uint16_t buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint16_t)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ double buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, double)
{
    typedef unsigned int u32x2_t __attribute__((__vector_size__(2 * sizeof(unsigned int))));
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return __hiloint2double((int)v[1], (int)v[0]);
}

}  // namespace

template <class Pol, int TM, int TN, int NW, int NSLOT, int TMV>
__global__ void __launch_bounds__(64 * NW)
conv_bwd_filter_split_kernel(const ConvParams p)
{
    // TMV <= TM filters per tile are loaded and stored; with TMV < TM the
    // MFMA block's other rows read the B rows that follow in LDS and their
    // results are dropped (8-filter tiles: twice the tiles of a 16-row block)
    using In = typename Pol::In;
    using Acc = typename Pol::Acc;
    using AccV = typename Pol::AccV;
    constexpr int ES = (int)sizeof(In);
    constexpr int BM = Pol::BM;
    constexpr int FM = TM / BM;
    constexpr int FN = TN / BM;
    constexpr int SEG = 64 / Pol::G;            // positions per lane per segment
    constexpr int FRAG_VECS = SEG * ES / 16;
    constexpr int STEPS = SEG / Pol::V;         // MFMA steps per segment
    constexpr int PITCH = 64 * ES + 16;         // one 64-position row, padded
    constexpr int WAVE_BYTES = (TMV + TN) * PITCH;
    constexpr int RED_BYTES = (NW - 1) * FM * FN * Pol::NACC * 64 * (int)sizeof(Acc);
    constexpr int SMEM = NW * WAVE_BYTES > RED_BYTES ? NW * WAVE_BYTES : RED_BYTES;
    static_assert(SEG % Pol::V == 0, "whole MFMA steps per segment");
    static_assert(TM % BM == 0 && TN % BM == 0, "tile must hold whole MFMA blocks");
    static_assert(TMV <= TM && (TMV == TM || TMV + TN >= TM), "valid rows; the block's other rows stay in LDS");
    static_assert(SEG * ES % 16 == 0, "lane slice must be whole 16-byte vectors");
    static_assert(NSLOT == 1 || NSLOT == 2, "one or two register slots");
    static_assert(BM * (BM + 1) * (int)sizeof(Acc) <= SMEM, "epilogue stage fits");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TMV;
    const int n0 = nt * TN;
    const int L = p.Kred;

    const int x_bytes = ((p.N - 1) * p.sxn + (p.C - 1) * p.sxc + (p.H - 1) * p.sxh + (p.W - 1) * p.sxw + 1) * ES;
    const int d_bytes = ((p.N - 1) * p.sdn + (p.M - 1) * p.sdk + (p.P - 1) * p.sdp + (p.Q - 1) * p.sdq + 1) * ES;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, x_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(p.w, d_bytes);
    // A rows: byte offset of filter k; B rows: byte offset of column
    // (c, r, s) and its tap.  Rows past the tile's edge are clamped to the
    // last: they feed only rows and columns of the MFMA block that are never
    // stored.
    int a_off[TMV];
#pragma unroll
    for (int e = 0; e < TMV; ++e) a_off[e] = min(m0 + e, p.M - 1) * p.sdk * ES;
    int b_off[TN], b_r[TN], b_s[TN];
#pragma unroll
    for (int e = 0; e < TN; ++e) {
        const int j = min(n0 + e, p.K - 1);
        uint32_t c, rs, r, s;
        p.div_rs.divmod((uint32_t)j, c, rs);
        p.div_s.divmod(rs, r, s);
        b_off[e] = ((int)c * p.sxc + (int)r * p.sxh + (int)s * p.sxw) * ES;
        b_r[e] = (int)r;
        b_s[e] = (int)s;
    }

    struct Slot {
        In a[TMV];
        In b[TN];
    };
    // one 64-position segment: lane = position, every row of the tile
    auto load_seg = [&](int sg, Slot& sl) {
        const int t = sg * 64 + lane;
        const bool pos_ok = t < L;
        uint32_t n, pq, pp, q;
        p.div_opq.divmod((uint32_t)(pos_ok ? t : 0), n, pq);
        p.div_oq.divmod(pq, pp, q);
        const int dvoff = pos_ok ? ((int)n * p.sdn + (int)pp * p.sdp + (int)q * p.sdq) * ES : kOutside;
        const int hp = (int)pp * p.u - p.pad_top;
        const int wq = (int)q * p.v - p.pad_left;
        const int xbase = ((int)n * p.sxn + hp * p.sxh + wq * p.sxw) * ES;
#pragma unroll
        for (int e = 0; e < TMV; ++e) sl.a[e] = buf_load(dr, dvoff, a_off[e], In{});
#pragma unroll
        for (int e = 0; e < TN; ++e) {
            const bool ok = pos_ok && (unsigned)(hp + b_r[e]) < (unsigned)p.H &&
                            (unsigned)(wq + b_s[e]) < (unsigned)p.W;
            sl.b[e] = buf_load(xr, ok ? xbase + b_off[e] : kOutside, 0, In{});
        }
    };

    // this wave's private transpose region: rows A 0..TMV-1, then B
    unsigned char* const mine = smem + wave * WAVE_BYTES;
    auto store_seg = [&](const Slot& sl) {
        unsigned char* base = mine + lane * ES;
#pragma unroll
        for (int e = 0; e < TMV; ++e) *reinterpret_cast<In*>(base + e * PITCH) = sl.a[e];
#pragma unroll
        for (int e = 0; e < TN; ++e) *reinterpret_cast<In*>(base + (TMV + e) * PITCH) = sl.b[e];
    };

    const int lrow = lane % BM;
    const int lgrp = lane / BM;
    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    // the segment just stored -> fragments (registers) -> SEG MFMA steps.
    // LDS operations of one wave run in order, so the fragment reads see the
    // stores before them and finish before the next segment's stores.
    u32x4 fa[FM][FRAG_VECS];
    u32x4 fb[FN][FRAG_VECS];
    auto read_frags = [&]() {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4* src = reinterpret_cast<const u32x4*>(mine + (i * BM + lrow) * PITCH + lgrp * SEG * ES);
#pragma unroll
            for (int v = 0; v < FRAG_VECS; ++v) fa[i][v] = src[v];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4* src = reinterpret_cast<const u32x4*>(mine + (TMV + j * BM + lrow) * PITCH + lgrp * SEG * ES);
#pragma unroll
            for (int v = 0; v < FRAG_VECS; ++v) fb[j][v] = src[v];
        }
    };
    auto mfma_seg = [&]() {
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (Pol::V == 1)
                        acc[i][j] = Pol::mfma_s(frag_elem(fa[i], t, In{}), frag_elem(fb[j], t, In{}), acc[i][j]);
                    else   // V consecutive positions per lane: one 16-byte fragment vector
                        acc[i][j] = Pol::mfma(fa[i], fb[j], t, acc[i][j]);
                }
        }
    };

    // wave w takes segments w, w + NW, w + 2 NW, ... (neighbouring waves on
    // neighbouring positions); its i-th segment is w + i * NW
    const int nseg = (L + 63) / 64;
    const int cnt = nseg > wave ? (nseg - wave + NW - 1) / NW : 0;
    auto seg_of = [&](int i) { return wave + min(i, cnt - 1) * NW; };
    if (cnt > 0) {
        if constexpr (NSLOT == 1) {
            Slot s0;
            load_seg(seg_of(0), s0);
            for (int i = 0; i < cnt; ++i) {
                store_seg(s0);
                read_frags();
                load_seg(seg_of(i + 1), s0);
                __builtin_amdgcn_sched_barrier(0);
                mfma_seg();
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            Slot s0, s1;
            load_seg(seg_of(0), s0);
            load_seg(seg_of(1), s1);
            for (int i = 0;; i += 2) {
                store_seg(s0);
                read_frags();
                load_seg(seg_of(i + 2), s0);
                __builtin_amdgcn_sched_barrier(0);
                mfma_seg();
                __builtin_amdgcn_sched_barrier(0);
                if (i + 1 >= cnt) break;
                store_seg(s1);
                read_frags();
                load_seg(seg_of(i + 3), s1);
                __builtin_amdgcn_sched_barrier(0);
                mfma_seg();
                __builtin_amdgcn_sched_barrier(0);
                if (i + 2 >= cnt) break;
            }
        }
    }

    // waves 1..NW-1 -> LDS -> added by wave 0 in wave order
    Acc* red = reinterpret_cast<Acc*>(smem);
    auto red_at = [&](int w, int i, int j, int e) {
        return ((((w - 1) * FM + i) * FN + j) * Pol::NACC + e) * 64 + lane;
    };
    __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < Pol::NACC; ++e) red[red_at(wave, i, j, e)] = acc[i][j][e];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 1; w < NW; ++w) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < Pol::NACC; ++e) acc[i][j][e] += red[red_at(w, i, j, e)];
        }
    }
    __syncthreads();
    store_acc_tile<Pol, FM, FN>(p, smem, acc, m0, n0, min(m0 + TMV, p.M), 0, lane, wave == 0);
}

template <class Pol, int TM, int TN, int NW, int NSLOT, int TMV>
static hipError_t launch_wgs_variant(const ConvParams& p0, hipStream_t stream)
{
    ConvParams p = p0;
    p.m_tiles = (p.M + TMV - 1) / TMV;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    hipLaunchKernelGGL((conv_bwd_filter_split_kernel<Pol, TM, TN, NW, NSLOT, TMV>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

//        name              policy     TM  TN  waves slots valid rows
#define MICONV_WGS_VARIANTS(X)                         \
    X(WGS_F32_32x32, PolF32, 32, 32, 8, 1, 32)         \
    X(WGS_F32_16x16, PolF32x16, 16, 16, 8, 2, 16)      \
    X(WGS_F32_8x16, PolF32x16, 16, 16, 8, 2, 8)        \
    X(WGS_F64_32x32, PolF64, 32, 32, 4, 1, 32)         \
    X(WGS_F64_16x16, PolF64, 16, 16, 8, 2, 16)         \
    X(WGS_BF16_32x32, PolBF16, 32, 32, 8, 1, 32)

hipError_t launch_bwd_filter_split(Variant v, const ConvParams& p, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, nw, ns, tmv) \
    case Variant::name: return launch_wgs_variant<pol, tm, tn, nw, ns, tmv>(p, stream);
        MICONV_WGS_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
