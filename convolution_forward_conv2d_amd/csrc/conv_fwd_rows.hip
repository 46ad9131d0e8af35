// conv_fwd_rows.hip -- fp32 convolution forward pass for tall filter banks
// with few filters (the speech network's second layer: 32 filters of
// 32 x 21 x 11, stride (2, 1), on 81 x 350 inputs), as an implicit GEMM whose
// reduction is streamed one filter row at a time.
//
//   y[n,k,p,q] = alpha * sum_{c,r,s} x[n,c,p*u+r-pad_top,q*v+s-pad_left] * F[k,c,r,s] + beta * y
//
// (the convolution of the cuDNN page, "Proposed Method"; batch-reduce GEMM
// over the filter taps as on the single-building-block page, read from x
// with no packed copy as on the zero-memory direct-convolution page).
//
// The tap-batched halo kernel stages, per channel block, every input row a
// tile touches and the whole R x S filter slab; with R = 21 and only 32
// filters that slab and halo outgrow LDS, and the gather kernel's
// per-element receptive-field loads then bound the layer.  Here a chunk of
// the reduction is (CB-channel block, filter row r): a tile of TM output
// positions spans at most NSL output rows (the host checks Q >= TM for
// NSL = 2), so the chunk stages NSL input rows -- row p*u + r - pad_top of
// each output row p -- of WP columns for CB channels, zero-padded, plus the
// S taps x CB channels x TN filters of row r.  The MFMA operand of position
// (slot, q) at tap s and channel c is then halo[c][slot][q*v + s]: a per-lane
// base plus a tap offset, no per-element gather.  v_mfma_f32_32x32x2_f32
// takes two channels per step (one per lane group), so a chunk is S * CB / 2
// steps; operands are read from LDS one step ahead, and chunk ch + 1 moves
// global -> registers during chunk ch and registers -> the other LDS buffer
// after its steps (one barrier per chunk).  Small chunks are the point: at
// CB = 4 a block holds 35 KB of LDS and 128 registers a lane, so four blocks
// share a CU and cover each other's chunk-edge waits (CB = 8: two blocks,
// 4% slower on the speech layer; CB = 2: 6% slower).
//
// Parameters as for the forward kernels (conv_params.h): x, w, y and their
// strides; M = N*P*Q; div_pq, div_q divide by P*Q and Q.
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

namespace {
constexpr int kRowsBufWord3 = 0x00020000;         // raw 32-bit buffer, range-checked per dword
constexpr int kRowsOutside = (int)0x80000000u;    // an offset past any buffer (host: x, w < 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRowsBufWord3);
}
template <class T>
__device__ __forceinline__ T rows_load(__amdgpu_buffer_rsrc_t r, int voff, int soff = 0)
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
// elements x spans: its last element's offset + 1 (every index at its
// largest; blocked x: the last channel lies in the last block)
__host__ __device__ __forceinline__ int64_t rows_x_elems(const ConvParams& p)
{
    return (int64_t)(p.N - 1) * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) + (int64_t)(p.H - 1) * p.sxh +
           (int64_t)(p.W - 1) * p.sxw + 1;
}

// x and w within the range a buffer descriptor checks (an offset of 2^31
// then lies past both)
static bool rows_buffers_fit(const ConvParams& p)
{
    return 4 * rows_x_elems(p) < ((int64_t)1 << 31) && 4 * (int64_t)p.K * p.Kred < ((int64_t)1 << 31);
}
}  // namespace

// XB: x channel-blocked ([N][C/cb][H][W][cb], cb a multiple of CB, 16-byte
// aligned): a chunk's CB = 4 channels lie side by side, so the halo moves as
// one 16-byte load per (slot, column).  WB: blocked filters
// ([K/kb][C/cb][R][S][cb][kb]).  Both false: NCHW x and packed KCRS filters.
// XV (unblocked x): the halo moves XV = 1, 2 or 4 consecutive columns per
// load; the host picks XV > 1 when W, pad_left and x's strides are multiples
// of XV (a unit then lies wholly inside or wholly outside the row) and x is
// aligned to XV values (speech layer 2: XV = 2, 2264 -> about 2100 us).
template <int TM, int TN, int WAVES_M, int WAVES_N, int S, int CB, int NSL, int WP, bool XB, bool WB, int XV>
__global__ void __launch_bounds__(256)
conv_fwd_rows_kernel(const ConvParams p)
{
    using Pol = PolF32;
    using AccV = Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int G = Pol::G;                       // channels per MFMA step (one per lane group)
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int PLANE = NSL * WP;                 // one channel's staged rows
    constexpr int HALO = CB * PLANE;                // floats
    constexpr int SLAB = S * CB * TN;               // floats: [s][c][k]
    constexpr int BUF = HALO + SLAB;
    // halo units per thread per chunk (XB: 4-channel groups; else XV columns)
    static_assert(XV == 1 || XV == 2 || XV == 4, "column units");
    static_assert(!XB || XV == 1, "blocked x moves channel groups");
    static_assert(WP % XV == 0, "whole units per staged row");
    constexpr int HE = XB ? PLANE : HALO / XV;      // halo units per chunk
    constexpr int NH = (HE + NT - 1) / NT;
    constexpr int STEPS = S * (CB / G);
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    static_assert(!XB || CB == 4, "blocked x: one 16-byte load per chunk column");
    constexpr int SROWS = TN * CB;                  // slab rows (filter, channel) of S taps
    constexpr int SPLIT = NT / SROWS;               // threads sharing a slab row
    constexpr int SH = (S + SPLIT - 1) / SPLIT;     // taps per thread
    static_assert(CB % G == 0 && NT % SROWS == 0, "whole slab rows per thread group");
    static_assert(NH <= 32, "halo validity mask");
    static_assert(2 * BUF * 4 <= 160 * 1024, "two chunk buffers fit the LDS");
    static_assert(4 * BM * (BM + 1) <= 2 * BUF, "epilogue stage fits");

    __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TM;
    const int m_end = min(m0 + TM, p.M);
    const int n0 = nt * TN;

    const float* __restrict__ x = static_cast<const float*>(p.x);
    const float* __restrict__ w = static_cast<const float*>(p.w);

    // the tile's first output row (n * P + p) and the slot of a position
    auto out_row = [&](int m) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * p.P + (int)pp;
    };
    const int row0 = out_row(m0);
    const int nrows = p.N * p.P;

    // Loads go through range-checked buffer descriptors (as in the one-channel
    // kernel below): a unit outside x, or a filter past K, reads at an offset
    // past the buffer and gets zeros (speech layer 2: 2148 -> 1897 us against
    // masked global loads).
    const int64_t x_elems = rows_x_elems(p);
    const __amdgpu_buffer_rsrc_t xr = rows_rsrc(p.x, (int)(4 * x_elems));

    // ---- halo loader: unit e = (channel, slot, XV columns), columns fastest
    // (XB: e = (slot, column) carrying the chunk's four channels)
    uint32_t h_voff[NH];                             // byte offset of (n, channel, row p*u - pad_top, column)
    int h_row[NH];                                   // input row p*u - pad_top (far negative: no unit)
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int e = tid + NT * i;
        const int el = XB ? e : e * XV;              // first staged element of the unit
        const int cl = el / PLANE;
        const int rem = el - cl * PLANE;
        const int sl = rem / WP;
        const int col = rem - sl * WP;
        const int orow = row0 + sl;
        const int n = orow / p.P;
        const int pp = orow - n * p.P;
        const int wc = col - p.pad_left;
        const bool ok = e < HE && orow < nrows && (unsigned)wc < (unsigned)p.W;
        const int hr = pp * p.u - p.pad_top;
        h_row[i] = ok ? hr : -(1 << 30);
        h_voff[i] = 4u * (uint32_t)(n * p.sxn + cl * p.sxc + wc * p.sxw + hr * p.sxh);   // (wraps; valid with a row)
    }
    // ---- slab loader: thread -> (filter k, channel c, taps sh*SH ... sh*SH + SH - 1) of row r
    const int sk = tid % TN;
    const int sc = (tid / TN) % CB;
    const int sh = tid / SROWS;
    const bool s_ok = n0 + sk < p.K;
    // packed KCRS: filter k's row of C*R*S; blocked: its block row and place in the block
    const int kk = s_ok ? n0 + sk : 0;
    const int s_base = WB ? (kk / p.wkb) * (p.C / p.wcb) * (p.R * S * p.wcb * p.wkb) + kk % p.wkb : kk * p.Kred;
    const __amdgpu_buffer_rsrc_t wr = rows_rsrc(p.w, 4 * p.K * p.Kred);
    // packed: byte offset of tap 0 of (filter, channel sc, row 0); a chunk adds (c0 R + r) S
    const int s_voff = s_ok ? 4 * (s_base + sc * p.R * S) : kRowsOutside;

    using HV = typename std::conditional<
        XB || XV == 4, float4, typename std::conditional<XV == 2, float2, float>::type>::type;
    HV hv[NH];
    float sv[SH];
    const int ncb = p.C / CB;
    const int nch = ncb * p.R;
    auto load_chunk = [&](int c0, int r) {
        // x offset of the chunk's first channel (blocked x: the chunk lies in one block)
        const int xo = XB ? blk_off(p.div_xcb, p.sxcb, p.sxc, c0) : c0 * p.sxc;
        const uint32_t chunk_off = 4u * (uint32_t)(xo + r * p.sxh);
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const bool ok = (unsigned)(h_row[i] + r) < (unsigned)p.H;
            hv[i] = rows_load<HV>(xr, ok ? (int)(h_voff[i] + chunk_off) : kRowsOutside);
        }
        if (WB) {
            // the channel's block once per chunk, then the taps at a stride of cb*kb
            // (a filter past K reads past w: zero)
            const int c = c0 + sc;
            const int wo = s_base + (c / p.wcb) * (p.R * S * p.wcb * p.wkb) + (c % p.wcb) * p.wkb +
                           r * S * p.wcb * p.wkb;
            const int vo = s_ok ? 4 * wo : kRowsOutside;
#pragma unroll
            for (int i = 0; i < SH; ++i) sv[i] = rows_load<float>(wr, vo + 4 * min(sh * SH + i, S - 1) * p.wcb * p.wkb);
        } else {
            const int s_chunk = 4 * (c0 * p.R + r) * S;
#pragma unroll
            for (int i = 0; i < SH; ++i) sv[i] = rows_load<float>(wr, s_voff + 4 * min(sh * SH + i, S - 1), s_chunk);
        }
    };
    auto store_chunk = [&](int buf) {
        float* dst = smem + buf * BUF;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int e = tid + NT * i;
            if constexpr (XB) {
                if (PLANE % NT == 0 || e < PLANE) {
                    const float4 v = hv[i];
                    dst[e] = v.x;
                    dst[PLANE + e] = v.y;
                    dst[2 * PLANE + e] = v.z;
                    dst[3 * PLANE + e] = v.w;
                }
            } else {
                if (HE % NT == 0 || e < HE) reinterpret_cast<HV*>(dst)[e] = hv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < SH; ++i) {
            const int s = sh * SH + i;
            if (SPLIT * SH == S || s < S) dst[HALO + (s * CB + sc) * TN + sk] = sv[i];
        }
    };

    // ---- per-lane operand bases (floats)
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane & 31;
    const int lgrp = lane >> 5;                      // channel within a step's pair
    int a_base[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = min(m0 + wm * WM + i * BM + lrow, p.M - 1);
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        const int sl = (int)n * p.P + (int)pp - row0;
        a_base[i] = lgrp * PLANE + sl * WP + (int)q * p.v;
    }
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_base[j] = HALO + lgrp * TN + wn * WN + j * BM + lrow;

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    // step t = (tap s, channel pair cp): A = halo[(2cp + g) PLANE + base + s],
    // B = slab[(s CB + 2cp + g) TN + k]
    auto a_off = [](int t) { const int s = t / (CB / G), cp = t % (CB / G); return G * cp * PLANE + s; };
    auto b_off = [](int t) { const int s = t / (CB / G), cp = t % (CB / G); return (s * CB + G * cp) * TN; };

    int lc0 = 0, lr = 0;                             // the chunk last loaded: channel block, filter row
    load_chunk(lc0, lr);
    store_chunk(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nch;
        if (more && (lc0 += CB) == p.C) {
            lc0 = 0;
            ++lr;
        }
        load_chunk(lc0, lr);
        __builtin_amdgcn_sched_barrier(0);
        const float* buf = smem + cur * BUF;
        float a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = buf[a_base[i] + a_off(0)];
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = buf[b_base[j] + b_off(0)];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            float an[FM], bn[FN];
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) an[i] = buf[a_base[i] + a_off(t + 1)];
#pragma unroll
                for (int j = 0; j < FN; ++j) bn[j] = buf[b_base[j] + b_off(t + 1)];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma_s(a[i], b[j], acc[i][j]);
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) a[i] = an[i];
#pragma unroll
                for (int j = 0; j < FN; ++j) b[j] = bn[j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) store_chunk(cur ^ 1);
        __syncthreads();
    }

    store_acc_tile<Pol, FM, FN>(p, reinterpret_cast<unsigned char*>(smem), acc, m0 + wm * WM, n0 + wn * WN, m_end,
                                wave, lane);
}

// ------------------------------------------------------------------ one input channel
//
// The same streaming for one to four input channels (the speech network's
// first layer: 32 filters of 41 x 11, stride 2, on one channel; Overfeat's:
// 96 filters of 3 x 11 x 11, stride 4): with no channel pair to give the
// MFMA's two lane groups, they take adjacent taps (s, s+1) of a filter row
// (S rounded up to SP = S + 1, the extra tap zero), and a chunk is one
// channel and RB filter rows, so that it holds RB * SP / 2 steps.  The chunk
// stages, per filter row j and output-row slot, one input row of WP
// columns; the operand of (slot, q) at (j, s) is halo[j][slot][q*v + s].
//
// waves_per_eu(6): the register allocator keeps a lane under 85 registers, so
// six workgroups share a CU and cover each other's chunk edges (measured on
// MI355X: 5-6% faster on speech layer 1 and Overfeat layer 1 than the four
// workgroups that 109 registers allow).  Measured and not kept: the next
// chunk's loads and LDS stores spread over the MFMA steps (3% slower), two
// filter rows per chunk (6-12% slower), the row stored by column phase so
// that stride-v operand reads hit distinct banks (6% slower with the loader
// gathering x at stride v; 8% slower with coalesced loads scattered into the
// phases, Overfeat layer 1 342 -> 369 us, although the LDS bank conflicts
// fell to zero and the LDS-active cycles by half), one tap per step on
// v_mfma_f32_32x32x1_2b_f32 (two 32-row blocks per instruction: 11 MFMAs a
// filter row instead of 12, no padding tap; 343 -> 345 us, speech layer 1
// 274 -> 282 us), 96 filters a tile (256 x 96 at three waves per SIMD: 353
// us; 128 x 96 at four or five: 381-388 us).  Neither the operand reads nor
// the MFMA count bounds this kernel; its vector-ALU work does: the loads
// through range-checked buffer descriptors (one add and one compare per unit
// and chunk, no store masks, no division per chunk) halved the loop's VALU
// and SALU instructions and took Overfeat layer 1 343 -> 284 us, speech
// layer 1 274 -> 246 us.
//
// XV: consecutive columns per halo load, as for the multi-channel kernel
// (speech layer 1: XV = 4).
template <int TM, int TN, int WAVES_M, int WAVES_N, int S, int RB, int NSL, int WP, int XV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6)))
conv_fwd_rows1_kernel(const ConvParams p)
{
    using Pol = PolF32;
    using AccV = Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int G = Pol::G;
    constexpr int SP = (S + G - 1) / G * G;         // taps rounded up to whole pairs
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int ROWP = NSL * WP;                  // one filter row's staged input rows
    constexpr int HALO = RB * ROWP;
    constexpr int SLAB = RB * SP * TN;              // [j][s][k]
    constexpr int BUF = HALO + SLAB;
    static_assert((XV == 1 || XV == 2 || XV == 4) && WP % XV == 0, "column units");
    constexpr int HE = HALO / XV;                   // halo units of XV columns
    constexpr int NH = (HE + NT - 1) / NT;
    constexpr int NS = (SLAB + NT - 1) / NT;
    constexpr int STEPS = RB * (SP / G);
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    static_assert(NH <= 32 && NS <= 32, "validity masks");
    static_assert(2 * BUF * 4 <= 160 * 1024, "two chunk buffers fit the LDS");
    constexpr int SMEM = 2 * BUF > 4 * BM * (BM + 1) ? 2 * BUF : 4 * BM * (BM + 1);   // chunk buffers / epilogue stage

    __shared__ __attribute__((aligned(16))) float smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TM;
    const int m_end = min(m0 + TM, p.M);
    const int n0 = nt * TN;

    const float* __restrict__ x = static_cast<const float*>(p.x);
    const float* __restrict__ w = static_cast<const float*>(p.w);

    auto out_row = [&](int m) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * p.P + (int)pp;
    };
    const int row0 = out_row(m0);
    const int nrows = p.N * p.P;

    // Loads go through range-checked buffer descriptors: a unit outside x (or
    // a filter outside w) reads at an offset past the buffer and gets zeros,
    // so the stores need no masks and a chunk's offsets are one add each.
    const int64_t x_elems = rows_x_elems(p);
    const __amdgpu_buffer_rsrc_t xr = rows_rsrc(p.x, (int)(4 * x_elems));
    const __amdgpu_buffer_rsrc_t wr = rows_rsrc(p.w, 4 * p.K * p.Kred);

    // ---- halo loader: unit e = (filter row j, slot, XV columns), columns fastest
    uint32_t h_voff[NH];                             // byte offset at channel 0, filter row 0
    int h_row[NH];                                   // input row of filter row j at chunk row 0 (far negative: no unit)
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int e = tid + NT * i;
        const int el = e * XV;                       // the unit's first staged element
        const int j = el / ROWP;
        const int rem = el - j * ROWP;
        const int sl = rem / WP;
        const int col = rem - sl * WP;
        const int orow = row0 + sl;
        const int n = orow / p.P;
        const int pp = orow - n * p.P;
        const int wc = col - p.pad_left;
        const bool ok = e < HE && orow < nrows && (unsigned)wc < (unsigned)p.W;
        const int hr = pp * p.u - p.pad_top + j;
        h_row[i] = ok ? hr : -(1 << 30);
        h_voff[i] = 4u * (uint32_t)(n * p.sxn + wc * p.sxw + hr * p.sxh);   // (wraps; valid once a chunk's row is added)
    }
    // ---- slab loader: element e = (filter row j, tap s, filter k), k fastest
    int s_voff[NS];
    int s_row[NS];                                   // filter row j of the element
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int e = tid + NT * i;
        const int j = e / (SP * TN);
        const int rem = e - j * (SP * TN);
        const int ss = rem / TN;
        const int k = rem - ss * TN;
        const bool ok = e < SLAB && ss < S && n0 + k < p.K;
        s_voff[i] = ok ? 4 * ((n0 + k) * p.Kred + j * S + ss) : kRowsOutside;   // packed K,C,R,S
        s_row[i] = j;
    }

    using HV = typename std::conditional<XV == 4, float4, typename std::conditional<XV == 2, float2, float>::type>::type;
    HV hv[NH];
    float sv[NS];
    // chunk = (filter row block, channel), channel fastest
    auto load_chunk = [&](int c, int r0) {
        const uint32_t chunk_off = 4u * (uint32_t)(c * p.sxc + r0 * p.sxh);
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const bool ok = (unsigned)(h_row[i] + r0) < (unsigned)p.H;
            hv[i] = rows_load<HV>(xr, ok ? (int)(h_voff[i] + chunk_off) : kRowsOutside);
        }
        const int s_chunk = 4 * (c * p.R + r0) * S;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int vo = RB == 1 || r0 + s_row[i] < p.R ? s_voff[i] : kRowsOutside;
            sv[i] = rows_load<float>(wr, vo, s_chunk);
        }
    };
    auto store_chunk = [&](int buf) {
        float* dst = smem + buf * BUF;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int e = tid + NT * i;
            if (HE % NT == 0 || e < HE) reinterpret_cast<HV*>(dst)[e] = hv[i];
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int e = tid + NT * i;
            if (SLAB % NT == 0 || e < SLAB) dst[HALO + e] = sv[i];
        }
    };

    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane & 31;
    const int lgrp = lane >> 5;                      // tap within a step's pair
    int a_base[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = min(m0 + wm * WM + i * BM + lrow, p.M - 1);
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        const int sl = (int)n * p.P + (int)pp - row0;
        a_base[i] = sl * WP + (int)q * p.v + lgrp;
    }
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_base[j] = HALO + lgrp * TN + wn * WN + j * BM + lrow;

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    // step t = (filter row j, tap pair sp): A = halo[j ROWP + base + 2 sp], B = slab[(j SP + 2 sp + g) TN + k]
    auto a_off = [](int t) { const int j = t / (SP / G), sp = t % (SP / G); return j * ROWP + G * sp; };
    auto b_off = [](int t) { const int j = t / (SP / G), sp = t % (SP / G); return (j * SP + G * sp) * TN; };

    const int nch = p.C * ((p.R + RB - 1) / RB);
    int lc = 0, lr0 = 0;                             // the chunk last loaded
    load_chunk(lc, lr0);
    store_chunk(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nch;
        if (more && ++lc == p.C) {
            lc = 0;
            lr0 += RB;
        }
        load_chunk(lc, lr0);
        __builtin_amdgcn_sched_barrier(0);
        const float* buf = smem + cur * BUF;
        float av[FM], bv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) av[i] = buf[a_base[i] + a_off(0)];
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = buf[b_base[j] + b_off(0)];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            float an[FM], bn[FN];
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) an[i] = buf[a_base[i] + a_off(t + 1)];
#pragma unroll
                for (int j = 0; j < FN; ++j) bn[j] = buf[b_base[j] + b_off(t + 1)];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma_s(av[i], bv[j], acc[i][j]);
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) av[i] = an[i];
#pragma unroll
                for (int j = 0; j < FN; ++j) bv[j] = bn[j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) store_chunk(cur ^ 1);
        __syncthreads();
    }

    store_acc_tile<Pol, FM, FN>(p, reinterpret_cast<unsigned char*>(smem), acc, m0 + wm * WM, n0 + wn * WN, m_end,
                                wave, lane);
}

// ------------------------------------------------------------------ data gradient
//
// dx[n,c,h,w] = alpha * sum over k, r, s with h + pad_top - r = p*u
// (0 <= p < P) and q = w + pad_left - s (0 <= q < Q; horizontal stride 1)
// of dy[n,k,p,q] * F[k,c,r,s] + beta * dx.  For the rows of one phase
// a = (h + pad_top) mod u the taps are r = a + u*i and p = P0(h) - i: a
// stride-1 correlation of dy with filter rows a, a + u, ... and the columns
// reversed.  One launch per phase (the host folds the phase's first row
// into y and u into its row stride, so the epilogue is the forward one);
// a chunk is (8 dy channels, tap row i), staging the dy rows P0 + h' - i of
// the tile's two output rows, columns q = w + pad_left - (S - 1) ... ;
// the operand of (w, s) is halo[k][slot][w + S - 1 - s] and the slab holds
// F[k][c][a + u*i][s] with the output channel c as the MFMA column.
//
// Parameters (per launch): x = dy with sx* its (n, k, p, q) strides, w = F,
// y = dx at row h0 of the phase, syp = u * dx's row stride; N, P, Q dy's
// dims; H = the phase's row count h', W = dx's width; K = dx's channels
// (the MFMA columns), C = dy's channels (the reduction), R = the phase's
// tap rows; pad_top carries P0(h0), pad_left the column pad, u the filter
// row step, Hp the phase a; M = N * h' * W, div_pq / div_q by h'*W and W.
//
// XV: consecutive dy columns per halo load (1, 2 or 4), as for the forward
// kernel: the host picks XV > 1 when Q, the first staged column and dy's
// strides are multiples of it and dy is aligned to it.
template <int TM, int TN, int WAVES_M, int WAVES_N, int S, int CB, int NSL, int WP, int XV>
__global__ void __launch_bounds__(256)
conv_bwd_data_rows_mfma_kernel(const ConvParams p)
{
    using Pol = PolF32;
    using AccV = Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int G = Pol::G;
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int PLANE = NSL * WP;
    constexpr int HALO = CB * PLANE;
    constexpr int SLAB = S * CB * TN;
    constexpr int BUF = HALO + SLAB;
    static_assert((XV == 1 || XV == 2 || XV == 4) && WP % XV == 0, "column units");
    constexpr int HE = HALO / XV;                    // halo units of XV columns
    constexpr int NH = (HE + NT - 1) / NT;
    constexpr int STEPS = S * (CB / G);
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    constexpr int SROWS = TN * CB;                   // slab rows (output channel, dy channel) of S taps
    constexpr int SPLIT = NT / SROWS;                // threads sharing a slab row
    constexpr int SH = (S + SPLIT - 1) / SPLIT;      // taps per thread
    static_assert(CB % G == 0 && NT % SROWS == 0, "whole slab rows per thread group");
    static_assert(NH <= 32, "halo validity mask");
    static_assert(2 * BUF * 4 <= 160 * 1024, "two chunk buffers fit the LDS");
    static_assert(4 * BM * (BM + 1) <= 2 * BUF, "epilogue stage fits");

    __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TM;
    const int m_end = min(m0 + TM, p.M);
    const int n0 = nt * TN;

    const float* __restrict__ dy = static_cast<const float*>(p.x);
    const float* __restrict__ f = static_cast<const float*>(p.w);
    const int hq = p.H;                               // output rows of the phase
    const int P0f = p.pad_top;                        // dy row of tap row 0 at h' = 0
    const int a = p.Hp;                               // the phase: filter rows a + u*i
    const int qoff = p.pad_left - (S - 1);            // dy column of halo column 0 at w = 0

    auto out_row = [&](int m) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * hq + (int)pp;
    };
    const int row0 = out_row(m0);
    const int nrows = p.N * hq;

    // Loads go through range-checked buffer descriptors (as in the forward
    // kernels above): a unit outside dy, or an output channel past K, reads
    // past the buffer and gets zeros.
    const int64_t dy_elems = (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.C - 1) * p.sxc + (int64_t)(p.P - 1) * p.sxh +
                             (int64_t)(p.Q - 1) * p.sxw + 1;
    const __amdgpu_buffer_rsrc_t dr = rows_rsrc(p.x, (int)(4 * dy_elems));
    const int RS = p.R * S;                           // p.R here: the filter's full row count
    const __amdgpu_buffer_rsrc_t fr = rows_rsrc(p.w, 4 * p.C * p.K * RS);

    // ---- halo loader: unit e = (dy channel, slot, XV columns), columns fastest
    uint32_t h_voff[NH];                              // byte offset at dy channel 0, tap row 0
    int h_row[NH];                                    // dy row of tap row 0 (i subtracted per chunk; far negative: no unit)
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int e = tid + NT * i;
        const int el = e * XV;                        // the unit's first staged element
        const int cl = el / PLANE;
        const int rem = el - cl * PLANE;
        const int sl = rem / WP;
        const int col = rem - sl * WP;
        const int orow = row0 + sl;
        const int n = orow / hq;
        const int hh = orow - n * hq;
        const int qc = col + qoff;
        const bool ok = e < HE && orow < nrows && (unsigned)qc < (unsigned)p.Q;
        h_row[i] = ok ? P0f + hh : -(1 << 30);
        h_voff[i] = 4u * (uint32_t)(n * p.sxn + cl * p.sxc + qc * p.sxw + (P0f + hh) * p.sxh);   // (wraps)
    }
    // ---- slab loader: thread -> (output channel c, dy channel k, taps sh*SH ...) of row a + u*i
    const int sk = tid % TN;                          // output channel within the tile
    const int sc = (tid / TN) % CB;                   // dy channel within the block
    const int sh = tid / SROWS;
    // F[k0 + sc][n0 + sk][a + u*i][s], packed K,C,R,S: this thread's part (past w for a channel past K)
    const int s_voff = n0 + sk < p.K ? 4 * ((sc * p.K + n0 + sk) * RS + a * S) : kRowsOutside;

    using HV = typename std::conditional<XV == 4, float4, typename std::conditional<XV == 2, float2, float>::type>::type;
    HV hv[NH];
    float sv[SH];
    const int ncb = p.C / CB;
    const int nri = p.Kred;                           // tap rows of the phase
    const int nch = ncb * nri;
    auto load_chunk = [&](int k0, int i) {
        const uint32_t chunk_off = 4u * (uint32_t)(k0 * p.sxc - i * p.sxh);
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            const bool ok = (unsigned)(h_row[e] - i) < (unsigned)p.P;
            hv[e] = rows_load<HV>(dr, ok ? (int)(h_voff[e] + chunk_off) : kRowsOutside);
        }
        const int s_chunk = 4 * (k0 * p.K * RS + p.u * i * S);
#pragma unroll
        for (int j = 0; j < SH; ++j) sv[j] = rows_load<float>(fr, s_voff + 4 * min(sh * SH + j, S - 1), s_chunk);
    };
    auto store_chunk = [&](int buf) {
        float* dst = smem + buf * BUF;
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            const int ee = tid + NT * e;
            if (HE % NT == 0 || ee < HE) reinterpret_cast<HV*>(dst)[ee] = hv[e];
        }
#pragma unroll
        for (int j = 0; j < SH; ++j) {
            const int s = sh * SH + j;
            if (SPLIT * SH == S || s < S) dst[HALO + (s * CB + sc) * TN + sk] = sv[j];
        }
    };

    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane & 31;
    const int lgrp = lane >> 5;
    int a_base[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = min(m0 + wm * WM + i * BM + lrow, p.M - 1);
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        const int sl = (int)n * hq + (int)pp - row0;
        a_base[i] = lgrp * PLANE + sl * WP + (int)q + (S - 1);
    }
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_base[j] = HALO + lgrp * TN + wn * WN + j * BM + lrow;

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    // step t = (tap s, dy channel pair cp): A = halo[(2cp + g) PLANE + base - s]
    auto a_off = [](int t) { const int s = t / (CB / G), cp = t % (CB / G); return G * cp * PLANE - s; };
    auto b_off = [](int t) { const int s = t / (CB / G), cp = t % (CB / G); return (s * CB + G * cp) * TN; };

    int lk0 = 0, li = 0;                              // the chunk last loaded: dy channel block, tap row
    if (nch > 0) {
        load_chunk(lk0, li);
        store_chunk(0);
        __syncthreads();
    }
    for (int ch = 0; ch < nch; ++ch) {
        const int cur = ch & 1;
        const bool more = ch + 1 < nch;
        if (more && (lk0 += CB) == p.C) {
            lk0 = 0;
            ++li;
        }
        load_chunk(lk0, li);
        __builtin_amdgcn_sched_barrier(0);
        const float* buf = smem + cur * BUF;
        float av[FM], bv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) av[i] = buf[a_base[i] + a_off(0)];
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = buf[b_base[j] + b_off(0)];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            float an[FM], bn[FN];
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) an[i] = buf[a_base[i] + a_off(t + 1)];
#pragma unroll
                for (int j = 0; j < FN; ++j) bn[j] = buf[b_base[j] + b_off(t + 1)];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma_s(av[i], bv[j], acc[i][j]);
            if (t + 1 < STEPS) {
#pragma unroll
                for (int i = 0; i < FM; ++i) av[i] = an[i];
#pragma unroll
                for (int j = 0; j < FN; ++j) bv[j] = bn[j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) store_chunk(cur ^ 1);
        __syncthreads();
    }

    store_acc_tile<Pol, FM, FN>(p, reinterpret_cast<unsigned char*>(smem), acc, m0 + wm * WM, n0 + wn * WN, m_end,
                                wave, lane);
}

// The data gradient's instance: the forward geometry (dy = P x Q, filters
// K x C x R x S, dx = N x C x H x W) with horizontal stride 1, S = 11, K a
// multiple of 8, W >= 256 (a tile within two output rows of a phase) and
// W + S - 1 <= 368.  Params in the direct kernel's layout.
constexpr int kDgRowsTM = 256, kDgRowsTN = 32, kDgRowsS = 11, kDgRowsCB = 8, kDgRowsWP = 368;

bool bwd_data_rows_mfma_fits(const ConvParams& p)
{
    return p.v == 1 && p.S == kDgRowsS && p.K % kDgRowsCB == 0 && p.W >= kDgRowsTM &&
           p.W + kDgRowsS - 1 <= kDgRowsWP;
}

hipError_t launch_bwd_data_rows_mfma(const ConvParams& p0, hipStream_t stream)
{
    if (!bwd_data_rows_mfma_fits(p0)) return hipErrorInvalidValue;
    // buffer descriptor ranges: dy and the filters under 2^31 bytes
    const int64_t dy_elems = (int64_t)(p0.N - 1) * p0.sxn + (int64_t)(p0.K - 1) * p0.sxc + (int64_t)(p0.P - 1) * p0.sxh +
                             (int64_t)(p0.Q - 1) * p0.sxw + 1;
    if (4 * dy_elems >= ((int64_t)1 << 31) || 4 * (int64_t)p0.K * p0.C * p0.R * p0.S >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    // dy columns per halo load: the first staged column pad_left - (S - 1),
    // Q and dy's strides multiples of it, unit column stride, dy aligned
    int xv = 1;
    const int qoff = p0.pad_left - (kDgRowsS - 1);
    for (int v = 4; v > 1; v /= 2)
        if (p0.sxw == 1 && p0.Q % v == 0 && ((qoff % v) + v) % v == 0 && p0.sxh % v == 0 && p0.sxc % v == 0 &&
            p0.sxn % v == 0 && reinterpret_cast<uintptr_t>(p0.x) % (4 * v) == 0) {
            xv = v;
            break;
        }
    const int u = p0.u;
    for (int a = 0; a < u; ++a) {
        // rows h with (h + pad_top) mod u == a: h = h0 + u*h'
        const int h0 = ((a - p0.pad_top) % u + u) % u;
        const int hq = h0 < p0.H ? (p0.H - h0 + u - 1) / u : 0;
        if (hq == 0) continue;
        const int nr = a < p0.R ? (p0.R - a + u - 1) / u : 0;
        ConvParams p = p0;
        p.y = static_cast<float*>(p0.y) + (int64_t)h0 * p0.syp;
        p.syp = u * p0.syp;
        p.H = hq;
        p.K = p0.C;                                  // MFMA columns: dx's channels
        p.C = p0.K;                                  // reduction: dy's channels (blocks of 8)
        p.R = p0.R;                                  // the filter's rows (for its strides)
        p.Kred = nr;                                 // tap rows a, a + u, ...
        p.Hp = a;
        p.pad_top = (h0 + p0.pad_top - a) / u;       // P0 at h' = 0
        p.M = p0.N * hq * p0.W;
        p.div_pq = FastDiv((uint32_t)(hq * p0.W));
        p.div_q = FastDiv((uint32_t)p0.W);
        p.Q = p0.Q;
        p.m_tiles = (p.M + kDgRowsTM - 1) / kDgRowsTM;
        p.n_tiles = (p.K + kDgRowsTN - 1) / kDgRowsTN;
        const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
        if (nr == 0 && p.beta == 1.0) continue;      // nothing to add (alpha * 0 + dx)
        if (xv == 4)
            hipLaunchKernelGGL((conv_bwd_data_rows_mfma_kernel<kDgRowsTM, kDgRowsTN, 4, 1, kDgRowsS, kDgRowsCB, 2,
                                                               kDgRowsWP, 4>),
                               grid, dim3(256), 0, stream, p);
        else if (xv == 2)
            hipLaunchKernelGGL((conv_bwd_data_rows_mfma_kernel<kDgRowsTM, kDgRowsTN, 4, 1, kDgRowsS, kDgRowsCB, 2,
                                                               kDgRowsWP, 2>),
                               grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((conv_bwd_data_rows_mfma_kernel<kDgRowsTM, kDgRowsTN, 4, 1, kDgRowsS, kDgRowsCB, 2,
                                                               kDgRowsWP, 1>),
                               grid, dim3(256), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Columns per halo load of unblocked x: 4 or 2 when W, pad_left and x's
// strides are multiples of it (a unit of consecutive columns then lies
// wholly inside or wholly outside the row, at an aligned address), with unit
// column stride and x aligned to it; else 1.
static int rows_column_unit(const ConvParams& p)
{
    for (int v = 4; v > 1; v /= 2)
        if (p.sxw == 1 && p.W % v == 0 && p.pad_left % v == 0 && p.sxh % v == 0 && p.sxc % v == 0 &&
            p.sxn % v == 0 && reinterpret_cast<uintptr_t>(p.x) % (4 * v) == 0)
            return v;
    return 1;
}

// Eligibility: fp32, S and the filter row length of the instance, C a
// multiple of the channel block, every tile inside NSL output rows
// (Q >= TM), the staged row width (Q - 1) * v + S <= WP.
template <int TM, int TN, int WAVES_M, int WAVES_N, int S, int CB, int NSL, int WP>
static bool rows_variant_fits(const ConvParams& p)
{
    static_assert(NSL >= 2, "a tile within two output rows");
    return p.S == S && p.C % CB == 0 && p.Q >= TM && (int64_t)(p.Q - 1) * p.v + S <= WP && rows_buffers_fit(p);
}

template <int TM, int TN, int WAVES_M, int WAVES_N, int S, int CB, int NSL, int WP>
static hipError_t launch_rows_variant(const ConvParams& p0, hipStream_t stream)
{
    ConvParams p = p0;
    if (!rows_variant_fits<TM, TN, WAVES_M, WAVES_N, S, CB, NSL, WP>(p)) return hipErrorInvalidValue;
    const bool xb = p.div_xcb.d != kOneBlock;
    const bool wb = p.wkb > 0;
    if (xb) {
        // the chunk's channels side by side, 16-byte aligned: packed blocks of
        // a multiple of CB channels, strides in whole 16-byte units
        const int cb = (int)p.div_xcb.d;
        if (cb % CB || p.sxc != 1 || p.sxw % 4 || p.sxh % 4 || p.sxn % 4 || p.sxcb % 4 ||
            reinterpret_cast<uintptr_t>(p.x) % 16)
            return hipErrorInvalidValue;
    }
    if (wb && (p.C % p.wcb || p.K % p.wkb)) return hipErrorInvalidValue;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    const int xv = xb ? 1 : rows_column_unit(p);
#define MICONV_ROWS_LAUNCH(XBV, WBV, XVV)                                                                        \
    hipLaunchKernelGGL((conv_fwd_rows_kernel<TM, TN, WAVES_M, WAVES_N, S, CB, NSL, WP, XBV, WBV, XVV>), grid,     \
                       dim3(256), 0, stream, p)
    if (xb && wb)
        MICONV_ROWS_LAUNCH(true, true, 1);
    else if (xb)
        MICONV_ROWS_LAUNCH(true, false, 1);
    else if (wb && xv == 4)
        MICONV_ROWS_LAUNCH(false, true, 4);
    else if (wb && xv == 2)
        MICONV_ROWS_LAUNCH(false, true, 2);
    else if (wb)
        MICONV_ROWS_LAUNCH(false, true, 1);
    else if (xv == 4)
        MICONV_ROWS_LAUNCH(false, false, 4);
    else if (xv == 2)
        MICONV_ROWS_LAUNCH(false, false, 2);
    else
        MICONV_ROWS_LAUNCH(false, false, 1);
#undef MICONV_ROWS_LAUNCH
    return hipGetLastError();
}

//        name                policy TM  TN  waves  S  CB NSL WP
#define MICONV_ROWS_VARIANTS(X)                        \
    X(ROWS_F32_S11_256x32, 256, 32, 4, 1, 11, 4, 2, 368)

// one to four input channels: S = 11 taps as 6 pairs, one filter row per
// chunk (14-18 KB of LDS, at most 116 registers a lane: four or more
// blocks a CU; four filter rows, two blocks a CU, took 1.3-1.4x as long);
// two output-row slots of 712 staged columns (a 256-position tile
// within two output rows: Q >= 256), or six of 232 (Q >= 51, as Overfeat
// layer 1's 56); (Q - 1) * v + 12 <= the staged width
constexpr int kRows1TM = 256, kRows1TN = 32, kRows1S = 11, kRows1RB = 1;

template <int NSL, int WP>
static bool rows1_variant_fits(const ConvParams& p)
{
    const int spanned = (kRows1TM - 1 + p.Q - 1) / p.Q + 1;    // output rows a tile can touch
    return p.C >= 1 && p.C <= 4 && p.S == kRows1S && spanned <= NSL &&
           (int64_t)(p.Q - 1) * p.v + kRows1S + 1 <= WP && rows_buffers_fit(p);
}

template <int NSL, int WP>
static hipError_t launch_rows1_variant(const ConvParams& p0, hipStream_t stream)
{
    if (!rows1_variant_fits<NSL, WP>(p0)) return hipErrorInvalidValue;
    ConvParams p = p0;
    p.m_tiles = (p.M + kRows1TM - 1) / kRows1TM;
    p.n_tiles = (p.K + kRows1TN - 1) / kRows1TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    switch (rows_column_unit(p)) {
    case 4:
        hipLaunchKernelGGL((conv_fwd_rows1_kernel<kRows1TM, kRows1TN, 4, 1, kRows1S, kRows1RB, NSL, WP, 4>), grid,
                           dim3(256), 0, stream, p);
        break;
    case 2:
        hipLaunchKernelGGL((conv_fwd_rows1_kernel<kRows1TM, kRows1TN, 4, 1, kRows1S, kRows1RB, NSL, WP, 2>), grid,
                           dim3(256), 0, stream, p);
        break;
    default:
        hipLaunchKernelGGL((conv_fwd_rows1_kernel<kRows1TM, kRows1TN, 4, 1, kRows1S, kRows1RB, NSL, WP, 1>), grid,
                           dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

bool rows_fits(Variant v, const ConvParams& p)
{
    if (v == Variant::ROWS1_F32_S11_256x32) return rows1_variant_fits<2, 712>(p);
    if (v == Variant::ROWS1N6_F32_S11_256x32) return rows1_variant_fits<6, 232>(p);
    switch (v) {
#define X(name, tm, tn, wmm, wnn, s, cb, nsl, wp) \
    case Variant::name: return rows_variant_fits<tm, tn, wmm, wnn, s, cb, nsl, wp>(p);
        MICONV_ROWS_VARIANTS(X)
#undef X
    default: return false;
    }
}

hipError_t launch_rows(Variant v, const ConvParams& p, hipStream_t stream)
{
    if (v == Variant::ROWS1_F32_S11_256x32) return launch_rows1_variant<2, 712>(p, stream);
    if (v == Variant::ROWS1N6_F32_S11_256x32) return launch_rows1_variant<6, 232>(p, stream);
    switch (v) {
#define X(name, tm, tn, wmm, wnn, s, cb, nsl, wp) \
    case Variant::name: return launch_rows_variant<tm, tn, wmm, wnn, s, cb, nsl, wp>(p, stream);
        MICONV_ROWS_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
