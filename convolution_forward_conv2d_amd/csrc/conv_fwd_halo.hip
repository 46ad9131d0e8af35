// conv_fwd_halo.hip -- convolution forward pass as a batch-reduce GEMM over
// the R x S filter taps, with the input read once per channel block.
//
// Same implicit GEMM as conv_fwd_mfma.hip (rows m = (n, p, q), columns k,
// reduction kappa = (c, r, s)), but the reduction is cut into chunks of CB
// whole channels with all R*S taps, kappa = (c_local, r, s) in KCRS order.
// Per chunk a workgroup stages in LDS:
//
//  * the input halo: for each of the CB channels, every zero-padded input
//    row ("slot") that the tile's TM output rows touch, WP columns wide
//    (padding positions hold zeros), loaded once along W;
//  * the filter slab: for each of its TN filters, the CB*R*S contiguous
//    values F[k, c0 .. c0+CB, :, :] (plain 16-byte loads of packed KCRS).
//
// Tap (r, s) of output row m then reads its A operand from LDS at
// slot(m, r) * WP + q*v + s: a per-lane base plus a compile-time offset,
// so the gather costs one LDS read per MFMA operand and no index math.
// This is the batch-reduce GEMM of the single-building-block page
// ("Proposed Method": a batch of sub-tensor block products reduced into one
// output block; here one block product per filter tap), computed directly
// from x with no packed copy (zero-memory direct-convolution page, Abstract
// and "Proposed Method"), double-buffered through LDS (maxDNN page,
// "Proposed Method").
//
// Eligibility (checked by the host): R, S equal to the instance's; the
// padded width W + pad_left + pad_right <= WP; every tile's slot span
// <= SL; C a multiple of CB; the filter 8- or 16-byte aligned as the
// instance's vector loads need.
//
// DG = true computes the data gradient of a stride-1 convolution as the
// forward pass of dy with the filter transposed (K <-> C) and flipped
// (r -> R-1-r, s -> S-1-s), the padding becoming R-1-pad_top and
// S-1-pad_left: the adjoint of the forward sum in x.  The host passes the
// parameters of that forward problem (x = dy, y = dx, C and K exchanged);
// only the slab loader differs, reading for each slab row (a channel of dx)
// and chunk channel (a filter of the real problem) the run of R*S taps of
// F[k, c, :, :] and storing it reversed.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

namespace {
constexpr int kHaloBufWord3 = 0x00020000;         // raw 32-bit buffer, range-checked per dword
constexpr int kHaloOutside = (int)0x80000000u;    // an offset past x and w (both under 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t halo_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kHaloBufWord3);
}
__device__ __forceinline__ u32x4 halo_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return u32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ u32x2 halo_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return u32x2{v[0], v[1]};
}
__device__ __forceinline__ void halo_load_elem(float& v, __amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void halo_load_elem(double& v, __amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    const u32x2 t = halo_load8(r, voff, soff);
    v = __hiloint2double((int)t[1], (int)t[0]);
}
}  // namespace

// WPE: the fewest waves per SIMD the register allocation must leave room for
// (1: no constraint).  Two for instances whose LDS admits two workgroups per
// CU but whose unconstrained allocation would not (Overfeat L2 on 208 x 64
// tiles: 603 -> 520 us; AlexNet conv2-conv4 and the fp64 128 x 64 tiles
// 1-2% faster); a cap would hurt the instances that run three.
//
// XR: x rows with unit column stride, 16-byte aligned, whole VX-pixel
// segments inside every row's storage (VX = 16 / sizeof(element): W a
// multiple of VX, or a row pitch reaching the last segment's end): the halo
// moves as 16-byte loads of VX consecutive pixels of one (channel, slot)
// row, stored at their padded columns; pixels outside the plane (padding
// columns, pixels past W, rows outside x, slots past the tile) are never
// written -- the halo starts zeroed.  XR = 1: W a multiple of VX (whole
// segments only).  XR = 2: a padded row pitch; the tensor's last row ends
// x's storage, so a segment reaching past W there is read pixel by pixel
// (the forward pass only: on the data gradient's dy it measured slower).
template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int CB, int WP, int SL, int KS,
          bool DG, bool WB, int WPE, int XR, bool BL>
__global__ void __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(WPE)))
conv_fwd_halo_kernel(const ConvParams p)
{
    using In = typename Pol::In;
    using AccV = typename Pol::AccV;
    constexpr int NT = 256;
    constexpr int BM = Pol::BM;
    constexpr int ES = (int)sizeof(In);
    constexpr int RS = R * S;
    constexpr int TK = CB * RS;                  // reduction elements per chunk
    constexpr int CPG = CB / Pol::G;             // channels per lane group
    constexpr int SEG = CPG * RS;                // reduction elements per lane group = MFMA steps
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    // halo: CB planes of SL slots x WP columns; the plane pitch is skewed by
    // 16 elements so the lane groups (one channel set each) hit other banks
    constexpr int PLANE = SL * WP + 16;
    constexpr int HALO_BYTES = CB * PLANE * ES;
    constexpr int HE = (CB * SL * WP) / NT;      // halo elements per thread per chunk
    constexpr int VX = 16 / ES;                  // XR: pixels per 16-byte load
    constexpr int NSX = WP / VX;                 // ... segments per staged row (W <= WP)
    constexpr int HUX = CB * SL * NSX;           // ... units per chunk
    constexpr int HXT = XR ? (HUX + NT - 1) / NT : 0;
    static_assert(!XR || ((SL * WP + 16) * ES) % 16 == 0 && (WP * ES) % 16 == 0, "16-byte aligned rows and planes");
    // filter slab: TN rows of TK values; row pitch an odd number of 8-byte units
    constexpr int ROW8 = (TK * ES + 7) / 8;
    constexpr int BROW = 8 * (ROW8 % 2 ? ROW8 : ROW8 + 1);
    constexpr int B_BYTES = TN * BROW;
    constexpr int VB = (TK * ES) % 16 == 0 ? 16 : 8;   // global vector width for the slab
    constexpr int VPR = TK * ES / VB;                   // vectors per filter row
    constexpr int NVB = (TN * VPR + NT - 1) / NT;       // slab vectors per thread per chunk
    constexpr int BUF_BYTES = ((HALO_BYTES + B_BYTES) + 15) / 16 * 16;
    // WB (blocked filters [K/kb][C/cb][R][S][cb][kb]): a 16-byte load takes VK
    // consecutive filters of one (channel, tap) slab column; units are
    // (column e, filter quad kq) with 8 consecutive quads on 8 consecutive lanes
    constexpr int VK = 16 / ES;
    constexpr int QT = (TN + VK - 1) / VK;              // filter quads per slab
    constexpr int QG = (QT + 7) / 8;                    // groups of 8 quads
    constexpr int NWU = QG * 8 * TK;                    // units (some past QT)
    constexpr int NWB = WB ? (NWU + NT - 1) / NT : 1;   // units per thread per chunk
    static_assert(!(DG && WB), "blocked filters in the forward pass only");
    static_assert(Pol::V == 1, "scalar-operand MFMA policies only");
    static_assert(CB % Pol::G == 0, "whole channels per lane group");
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    static_assert((CB * SL * WP) % NT == 0, "halo elements split evenly over the threads");
    static_assert((TK * ES) % 8 == 0, "slab rows are whole 8-byte vectors");
    static_assert(4 * BM * (BM + 1) * (int)sizeof(typename Pol::Acc) <= 2 * BUF_BYTES, "epilogue stage fits");
    static_assert(((CPG - 1) * PLANE + (R - 1) * WP + S) * ES < 65536, "LDS immediate offsets");
    // KS = 2: two 4-wave halves share one output tile and split its
    // reduction (alternate channel blocks); half 1 hands its partial sums to
    // half 0 through LDS at the end, so each SIMD holds two waves of the tile
    static_assert(KS == 1 || KS == 2, "one or two halves");
    constexpr int RED_BYTES = KS == 2 ? 4 * FM * FN * Pol::NACC * 64 * (int)sizeof(typename Pol::Acc) : 0;
    static_assert(RED_BYTES <= KS * 2 * BUF_BYTES, "partial sums fit in the chunk buffers");

    __shared__ __attribute__((aligned(16))) unsigned char smem_all[KS * 2 * BUF_BYTES];

    const int half = KS == 2 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255;           // thread within its half
    const int lane = tid & 63;
    const int wave = tid >> 6;                   // wave within its half
    unsigned char* smem = smem_all + half * 2 * BUF_BYTES;
    if constexpr (XR) {
        // every halo buffer starts zeroed: the row loader writes only pixels inside x
        for (int i = (int)threadIdx.x; i < KS * 2 * BUF_BYTES / 16; i += NT * KS)
            reinterpret_cast<u32x4*>(smem_all)[i] = u32x4{0, 0, 0, 0};
        __syncthreads();
    }

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const TileRC rc = grouped_tile(tile, p.m_tiles, p.n_tiles, p.n_group);
    const int mt = rc.mt;
    const int nt = rc.nt;
    // a tile covers rows m0 .. m_end-1: TM consecutive rows, or one output
    // image (m_step = P*Q <= TM, the rest of the tile idle)
    const int m0 = mt * p.m_step;
    const int m_end = min(m0 + p.m_step, p.M);
    const int n0 = nt * TN;

    const In* __restrict__ x = static_cast<const In*>(p.x);
    const In* __restrict__ w = static_cast<const In*>(p.w);
    // x and w through range-checked buffer descriptors: a unit outside x or
    // past the filters reads at an offset past the buffer and gets zeros, so
    // no load sits in a branch or needs a select; a chunk's channel offset is
    // the scalar offset (host: x, w under 2^31 bytes)
    const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) +
                            (int64_t)(p.H - 1) * p.sxh + (int64_t)(p.W - 1) * p.sxw + 1;
    const __amdgpu_buffer_rsrc_t xr = halo_rsrc(p.x, x_elems * ES);
    const __amdgpu_buffer_rsrc_t wr = halo_rsrc(p.w, (int64_t)p.C * p.K * RS * ES);

    // virtual padded row of output row m (tap r adds r): n * Hp + p * u
    auto vrow = [&](int m) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * p.Hp + (int)pp * p.u;
    };
    const int vr_first = vrow(m0);
    const int nslots = vrow(m_end - 1) + R - vr_first;  // <= SL (host-checked)

    // ---- halo loader: thread -> HE (channel, slot, column) positions, fixed for the tile
    int h_voff[HE];                                  // byte offsets at channel 0 (past x: none)
#pragma unroll
    for (int i = 0; i < HE; ++i) {
        const int e = tid + NT * i;
        const int col = e % WP;
        const int slot = (e / WP) % SL;
        const int cl = e / (WP * SL);
        uint32_t n, hp;
        p.div_hp.divmod((uint32_t)(vr_first + slot), n, hp);
        const int h = (int)hp - p.pad_top;
        const int wcol = col - p.pad_left;
        const bool ok = slot < nslots && (int)n < p.N && h >= 0 && h < p.H && wcol >= 0 && wcol < p.W;
        const int off = (int)n * p.sxn + cl * p.sxc + h * p.sxh + wcol * p.sxw;
        h_voff[i] = BL ? (ok ? off * ES : kHaloOutside) : (ok ? off : -1);   // (!BL: elements, -1 none)
    }

    // XR: unit u = (channel, slot, segment): pixels w0 .. w0 + VX - 1, w0 = VX * segment
    int x_off[XR ? HXT : 1], x_dst[XR ? HXT : 1], x_np[XR ? HXT : 1];
    uint32_t x_ok = 0, x_last = 0;
    if constexpr (XR) {
#pragma unroll
        for (int i = 0; i < HXT; ++i) {
            const int u = tid + NT * i;
            const int seg = u % NSX;
            const int slot = (u / NSX) % SL;
            const int cl = u / (NSX * SL);
            uint32_t n, hp;
            p.div_hp.divmod((uint32_t)(vr_first + slot), n, hp);
            const int h = (int)hp - p.pad_top;
            const int w0 = VX * seg;
            const bool ok = u < HUX && slot < nslots && (int)n < p.N && h >= 0 && h < p.H && w0 < p.W;
            const int off = (int)n * p.sxn + cl * p.sxc + h * p.sxh + w0;
            x_off[i] = BL ? (ok ? off * ES : kHaloOutside) : (ok ? off : 0);   // bytes (!BL: elements)
            x_dst[i] = cl * PLANE + slot * WP + w0 + p.pad_left;     // element index of pixel w0
            x_np[i] = ok ? min(VX, p.W - w0) : 0;                      // pixels inside the row
            x_ok |= (ok ? 1u : 0u) << i;
            // the last row: image N-1, row H-1, channel C-1 (the last chunk's channel CB-1)
            const bool last = ok && (int)n == p.N - 1 && h == p.H - 1 && cl == CB - 1 && w0 + VX > p.W;
            x_last |= (last ? 1u : 0u) << i;
        }
    }
    u32x4 x_val[XR ? HXT : 1];

    // ---- slab loader: thread -> NVB (filter row, vector) positions
    // (DG: thread -> NDU (slab row, channel) runs of R*S taps instead)
    constexpr int DU = TN * CB;
    constexpr int NDU = DG ? (DU + NT - 1) / NT : 1;
    int d_off[NDU];                                  // byte offsets at chunk 0 (past w: none)
    if constexpr (DG) {
#pragma unroll
        for (int i = 0; i < NDU; ++i) {
            const int e = tid + NT * i;
            const int row = e % TN;
            const int cl = e / TN;
            const bool ok = e < DU && n0 + row < p.K;
            const int off = (cl * p.K + n0 + row) * RS;
            d_off[i] = BL ? (ok ? off * ES : kHaloOutside) : (ok ? off : -1);
        }
    }
    int b_off[WB ? 1 : NVB];                         // byte offsets at chunk 0 (past w: none)
    if constexpr (!WB) {
#pragma unroll
        for (int i = 0; i < NVB; ++i) {
            const int e = tid + NT * i;
            const int row = e / VPR;
            const int vec = e - row * VPR;
            const bool ok = e < TN * VPR && n0 + row < p.K;
            const int off = (n0 + row) * p.Kred + vec * (VB / ES);
            b_off[i] = BL ? (ok ? off * ES : kHaloOutside) : (ok ? off : -1);
        }
    }
    // WB: unit u -> slab column e = (channel cl, tap t), quad kq; its element
    // offset is w_off[i] plus the chunk's (c0 / cb) * R*S*cb*kb + (c0 % cb) * kb
    // (a chunk lies in one channel block; K is a multiple of kb, kb of VK)
    int w_off[WB ? NWB : 1];
    uint32_t w_ok = 0;
    if constexpr (WB) {
        const int blk = RS * p.wcb * p.wkb;
#pragma unroll
        for (int i = 0; i < NWB; ++i) {
            const int u = tid + NT * i;
            const int kq = (u / (8 * TK)) * 8 + (u & 7);
            const int e = (u >> 3) % TK;
            const int k = n0 + kq * VK;
            const bool ok = u < NWU && kq < QT && k < p.K;
            const int cl = e / RS, t = e - cl * RS;
            const int off = (k / p.wkb) * (p.C / p.wcb) * blk + (t * p.wcb + cl) * p.wkb + k % p.wkb;
            w_off[i] = BL ? (ok ? off * ES : kHaloOutside) : (ok ? off : 0);   // (BL: bytes)
            w_ok |= (ok ? 1u : 0u) << i;
        }
    }

    In h_val[HE];
    u32x4 b_val[DG ? 1 : (WB ? NWB : NVB)];
    In d_val[NDU][DG ? RS : 1];

    auto load_chunk = [&](int c0) {
        const int xo = blk_off(p.div_xcb, p.sxcb, p.sxc, c0);
        if constexpr (XR) {
#pragma unroll
            for (int i = 0; i < HXT; ++i) {
                if (XR == 2 && ((x_last >> i) & 1) && c0 + CB == p.C) {
                    const In* src = x + (BL ? x_off[i] / ES : x_off[i]) + xo;
                    In v[VX] = {};
                    for (int e = 0; e < x_np[i]; ++e) v[e] = src[e];
                    __builtin_memcpy(&x_val[i], v, 16);
                } else if constexpr (BL) {
                    x_val[i] = halo_load16(xr, x_off[i], xo * ES);
                } else {
                    x_val[i] = *reinterpret_cast<const u32x4*>(x + x_off[i] + xo);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < HE; ++i) {
                if constexpr (BL)
                    halo_load_elem(h_val[i], xr, h_voff[i], xo * ES);
                else
                    h_val[i] = h_voff[i] >= 0 ? load_elem(x + h_voff[i] + xo) : In(0);
            }
        }
        if constexpr (DG) {
            const int wo = c0 * p.K * RS * ES;
#pragma unroll
            for (int i = 0; i < NDU; ++i) {
#pragma unroll
                for (int t = 0; t < RS; ++t) {
                    if constexpr (BL)
                        halo_load_elem(d_val[i][t], wr, d_off[i] + t * ES, wo);
                    else
                        d_val[i][t] = d_off[i] >= 0 ? load_elem(w + d_off[i] + wo / ES + t) : In(0);
                }
            }
        } else if constexpr (WB) {
            const int wo = (c0 / p.wcb) * (RS * p.wcb * p.wkb) + (c0 % p.wcb) * p.wkb;
#pragma unroll
            for (int i = 0; i < NWB; ++i) {
                if constexpr (BL)
                    b_val[i] = halo_load16(wr, w_off[i], wo * ES);
                else
                    b_val[i] = *reinterpret_cast<const u32x4*>(w + w_off[i] + wo);
            }
        } else {
            const int wo = c0 * RS * ES;
#pragma unroll
            for (int i = 0; i < NVB; ++i) {
                if constexpr (!BL) {
                    const In* src = w + b_off[i] + wo / ES;
                    if constexpr (VB == 16) {
                        b_val[i] = b_off[i] >= 0 ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
                    } else {
                        const u32x2 t = b_off[i] >= 0 ? *reinterpret_cast<const u32x2*>(src) : u32x2{0, 0};
                        b_val[i] = u32x4{t[0], t[1], 0, 0};
                    }
                } else if constexpr (VB == 16) {
                    b_val[i] = halo_load16(wr, b_off[i], wo);
                } else {
                    const u32x2 t = halo_load8(wr, b_off[i], wo);
                    b_val[i] = u32x4{t[0], t[1], 0, 0};
                }
            }
        }
    };

    auto store_chunk = [&](int buf) {
        unsigned char* hb = smem + buf * BUF_BYTES;
        if constexpr (XR) {
            // a segment starts on a 16-byte LDS boundary when pad_left is a
            // multiple of VX (the plane and row pitches are): one 16-byte store
            const bool whole = p.pad_left % VX == 0;
#pragma unroll
            for (int i = 0; i < HXT; ++i) {
                if ((x_ok >> i) & 1) {
                    if (whole && (XR == 1 || x_np[i] == VX)) {
                        *reinterpret_cast<u32x4*>(hb + x_dst[i] * ES) = x_val[i];
                    } else {
                        In v[VX];
                        __builtin_memcpy(v, &x_val[i], 16);
#pragma unroll
                        for (int e = 0; e < VX; ++e)
                            if (XR == 1 || e < x_np[i]) reinterpret_cast<In*>(hb)[x_dst[i] + e] = v[e];
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < HE; ++i) {
                const int e = tid + NT * i;
                const int col = e % WP;
                const int slot = (e / WP) % SL;
                const int cl = e / (WP * SL);
                reinterpret_cast<In*>(hb)[cl * PLANE + slot * WP + col] = h_val[i];
            }
        }
        unsigned char* bb = hb + HALO_BYTES;
        if constexpr (DG) {
            // run element t is tap RS-1-t of the slab row (the filter flipped)
#pragma unroll
            for (int i = 0; i < NDU; ++i) {
                const int e = tid + NT * i;
                if (DU % NT == 0 || e < DU) {
                    const int row = e % TN;
                    const int cl = e / TN;
                    In* dst = reinterpret_cast<In*>(bb + row * BROW) + cl * RS;
#pragma unroll
                    for (int t = 0; t < RS; ++t) dst[RS - 1 - t] = d_val[i][t];
                }
            }
        } else if constexpr (WB) {
            // a quad's VK filters are VK slab rows of column e (zeros outside)
#pragma unroll
            for (int i = 0; i < NWB; ++i) {
                const int u = tid + NT * i;
                const int kq = (u / (8 * TK)) * 8 + (u & 7);
                const int e = (u >> 3) % TK;
                if (NWU % NT == 0 || u < NWU) {
                    if (kq < QT) {
                        const bool ok = BL || ((w_ok >> i) & 1);   // (BL: zeros read past w)
                        In v[VK];
                        __builtin_memcpy(v, &b_val[i], 16);
#pragma unroll
                        for (int j = 0; j < VK; ++j)
                            if (kq * VK + j < TN)
                                *reinterpret_cast<In*>(bb + (kq * VK + j) * BROW + e * ES) = ok ? v[j] : In(0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NVB; ++i) {
                const int e = tid + NT * i;
                if (e < TN * VPR) {
                    const int row = e / VPR;
                    const int vec = e - row * VPR;
                    u32x2* dst = reinterpret_cast<u32x2*>(bb + row * BROW + vec * VB);
                    dst[0] = u32x2{b_val[i][0], b_val[i][1]};
                    if constexpr (VB == 16) dst[1] = u32x2{b_val[i][2], b_val[i][3]};
                }
            }
        }
    };

    // ---- per-wave MFMA geometry
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane % BM;
    const int lgrp = lane / BM;
    int a_base[FM];                     // element offset of tap (0,0) of this lane's row, per block
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + i * BM + lrow;
        int base = 0;
        if (m < m_end) {
            uint32_t n, pq, pp, q;
            p.div_pq.divmod((uint32_t)m, n, pq);
            p.div_q.divmod(pq, pp, q);
            base = ((int)n * p.Hp + (int)pp * p.u - vr_first) * WP + (int)q * p.v;
        }
        a_base[i] = base + lgrp * CPG * PLANE;
    }
    int b_row[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_row[j] = (wn * WN + j * BM + lrow) * BROW + lgrp * SEG * ES;

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    // MFMAs of the chunk in LDS buffer `cur`.  Halfway through, the next
    // chunk (already in registers) is parked in the other buffer: its last
    // readers finished before the previous barrier, and the store's wait on
    // the global loads and its LDS latency overlap the second half.
    auto compute = [&](int cur, bool park) {
        const In* halo = reinterpret_cast<const In*>(smem + cur * BUF_BYTES);
        const unsigned char* slab = smem + cur * BUF_BYTES + HALO_BYTES;
        In bf[FN][SEG];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const In* src = reinterpret_cast<const In*>(slab + b_row[j]);
#pragma unroll
            for (int t = 0; t < SEG; ++t) bf[j][t] = src[t];
        }
#pragma unroll
        for (int t = 0; t < SEG; ++t) {
            const int off = (t / RS) * PLANE + ((t % RS) / S) * WP + (t % RS) % S;
            In a[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) a[i] = halo[a_base[i] + off];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Pol::mfma_s(a[i], bf[j][t], acc[i][j]);
            if (t == SEG / 2 && park) store_chunk(cur ^ 1);
        }
    };

    // chunk j of this half is channel block j*KS + half
    const int nblocks = p.C / CB;
    const int iters = (nblocks + KS - 1) / KS;
    auto chunk_of = [&](int j) { return j * KS + half; };
    if (chunk_of(0) < nblocks) {
        load_chunk(chunk_of(0) * CB);
        store_chunk(0);
    }
    __syncthreads();

    for (int it = 0; it < iters; ++it) {
        const int cur = it & 1;
        const bool mine = chunk_of(it) < nblocks;          // uniform per half
        const bool more = chunk_of(it + 1) < nblocks;
        if (more) load_chunk(chunk_of(it + 1) * CB);
        if (mine) compute(cur, more);
        __syncthreads();
    }

    if constexpr (KS == 2) {
        // half 1's partial sums -> LDS -> added by half 0 in a fixed order
        typename Pol::Acc* red = reinterpret_cast<typename Pol::Acc*>(smem_all);
        auto red_at = [&](int i, int j, int e) { return ((((wave * FM + i) * FN + j) * Pol::NACC + e) << 6) + lane; };
        if (half == 1) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < Pol::NACC; ++e) red[red_at(i, j, e)] = acc[i][j][e];
        }
        __syncthreads();
        if (half == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < Pol::NACC; ++e) acc[i][j][e] += red[red_at(i, j, e)];
        }
        __syncthreads();
    }

    store_acc_tile<Pol, FM, FN>(p, smem_all, acc, m0 + wm * WM, n0 + wn * WN, m_end, wave, lane, half == 0);
}

// ------------------------------------------------------------------ instances and launch

// BLM: loads through buffer descriptors (BL) always (1), never (0: masked
// global loads), or in the forward pass only (2) -- per instance, as measured
// on MI355X: the 16x16-block tiles of 144 and 176 rows, whose registers are
// full, ran 4-10% slower with them (their SGPRs spill), fp64 176x64 in the
// data gradient 6% slower; every other instance 2-9% faster.
template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int CB, int WP, int SL, int KS, int WPE,
          int BLM>
static hipError_t launch_halo_variant(const ConvParams& p0, bool dgrad, hipStream_t stream)
{
    ConvParams p = p0;
    {
        // the buffer descriptors' range: x (dy) and the filters under 2^31 bytes
        constexpr int64_t ES = (int64_t)sizeof(typename Pol::In);
        const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) +
                                (int64_t)(p.H - 1) * p.sxh + (int64_t)(p.W - 1) * p.sxw + 1;
        if (BLM != 0 && (ES * x_elems >= ((int64_t)1 << 31) || ES * p.C * (int64_t)p.K * R * S >= ((int64_t)1 << 31)))
            return hipErrorInvalidValue;
    }
    if (p.m_step <= 0 || p.m_step > TM) p.m_step = TM;   // the host sets P*Q for image tiles
    p.m_tiles = (p.M + p.m_step - 1) / p.m_step;
    p.n_tiles = (p.K + TN - 1) / TN;
    {
        // workgroups per CU as the LDS allows (the chunk buffers of every half)
        constexpr int ES = (int)sizeof(typename Pol::In);
        constexpr int TK = CB * R * S;
        constexpr int ROW8 = (TK * ES + 7) / 8;
        constexpr int BROW = 8 * (ROW8 % 2 ? ROW8 : ROW8 + 1);
        constexpr int BUF = ((CB * (SL * WP + 16) * ES + TN * BROW) + 15) / 16 * 16;
        constexpr int WG_PER_CU = (160 * 1024) / (KS * 2 * BUF) > 0 ? (160 * 1024) / (KS * 2 * BUF) : 1;
        p.n_group = choose_n_group(p, (int64_t)p.N * p.C * p.H * p.W * ES, (int64_t)p.K * p.Kred * ES, WG_PER_CU);
    }
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    constexpr int VK = 16 / (int)sizeof(typename Pol::In);
    if (p.wkb > 0) {
        // blocked filters: the host checked cb % CB == 0, kb % VK == 0, K % kb == 0,
        // C % cb == 0 and a 16-byte aligned w
        if (dgrad || p.wcb % CB != 0 || p.wkb % VK != 0 || p.K % p.wkb != 0 || p.C % p.wcb != 0 ||
            (uintptr_t)p.w % 16 != 0)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(
            (conv_fwd_halo_kernel<Pol, TM, TN, WAVES_M, WAVES_N, R, S, CB, WP, SL, KS, false, true, WPE, 0, BLM != 0>), grid,
            dim3(256 * KS), 0, stream, p);
        return hipGetLastError();
    }
    // 16-byte row segments of x: unit column stride, x's strides multiples of
    // the segment, x aligned; whole segments (W a multiple of one), or in the
    // forward pass every row's storage holding its last segment whole (a
    // padded row pitch) with NCHW nesting, so that only the tensor's last row
    // ends x's storage
    constexpr int VX = 16 / (int)sizeof(typename Pol::In);
    const bool xv = p.div_xcb.d == kOneBlock && p.sxw == 1 && (uintptr_t)p.x % 16 == 0 && p.sxh % VX == 0 &&
                    p.sxc % VX == 0 && p.sxn % VX == 0;
    const bool xr1 = xv && p.W % VX == 0;
    const bool xr2 = xv && !xr1 && !dgrad && p.sxh >= (p.W + VX - 1) / VX * VX &&
                     (int64_t)p.sxc >= (int64_t)p.sxh * p.H && (int64_t)p.sxn >= (int64_t)p.sxc * p.C;
#define MICONV_HALO_LAUNCH(DGV, XRV)                                                                              \
    hipLaunchKernelGGL((conv_fwd_halo_kernel<Pol, TM, TN, WAVES_M, WAVES_N, R, S, CB, WP, SL, KS, DGV, false, WPE, \
                                             XRV, BLM == 1 || (BLM == 2 && !DGV)>),                               \
                       grid, dim3(256 * KS), 0, stream, p)
    if (dgrad && xr1)
        MICONV_HALO_LAUNCH(true, 1);
    else if (dgrad)
        MICONV_HALO_LAUNCH(true, 0);
    else if (xr1)
        MICONV_HALO_LAUNCH(false, 1);
    else if (xr2)
        MICONV_HALO_LAUNCH(false, 2);
    else
        MICONV_HALO_LAUNCH(false, 0);
#undef MICONV_HALO_LAUNCH
    return hipGetLastError();
}

//        name                     policy     TM   TN  waves  R  S  CB  WP  SL  KS  WPE  BLM
#define MICONV_HALO_VARIANTS(X)                                                 \
    X(HALO_F32_3x3_128x128, PolF32, 128, 128, 2, 2, 3, 3, 4, 16, 16, 1, 2, 1)          \
    X(HALO_F32_3x3_128x64, PolF32, 128, 64, 2, 2, 3, 3, 4, 16, 16, 1, 1, 1)            \
    X(HALO_F32_3x3_64x128, PolF32, 64, 128, 2, 2, 3, 3, 4, 16, 16, 1, 1, 1)            \
    X(HALO_F32_3x3_96x128, PolF32, 96, 128, 1, 4, 3, 3, 4, 16, 16, 1, 1, 1)            \
    X(HALO_F32_5x5_128x128, PolF32, 128, 128, 2, 2, 5, 5, 4, 32, 16, 1, 1, 1)          \
    X(HALO_F32_5x5_128x128_C2, PolF32, 128, 128, 2, 2, 5, 5, 2, 32, 16, 1, 2, 1)       \
    X(HALO_F32_5x5_128x96_C2, PolF32, 128, 96, 4, 1, 5, 5, 2, 32, 16, 1, 1, 1)         \
    X(HALO_F32x16_5x5_208x64, PolF32x16, 208, 64, 1, 4, 5, 5, 4, 32, 24, 1, 2, 1)      \
    X(HALO_F32x16_3x3_176x128, PolF32x16, 176, 128, 1, 4, 3, 3, 4, 16, 16, 1, 1, 1)    \
    X(HALO_F32x16_3x3_144x128, PolF32x16, 144, 128, 1, 4, 3, 3, 4, 16, 16, 1, 1, 0)    \
    X(HALO_F32x16_5x5_128x96, PolF32x16, 128, 96, 2, 2, 5, 5, 4, 32, 16, 1, 1, 1)      \
    X(HALO_F32x16_3x3_176x128_KS2, PolF32x16, 176, 128, 1, 4, 3, 3, 4, 16, 16, 2, 1, 0) \
    X(HALO_F32_3x3_128x128_KS2, PolF32, 128, 128, 2, 2, 3, 3, 4, 16, 16, 2, 1, 1)      \
    X(HALO_F64_3x3_128x128, PolF64, 128, 128, 2, 2, 3, 3, 4, 16, 16, 1, 1, 1)          \
    X(HALO_F64_3x3_64x64, PolF64, 64, 64, 2, 2, 3, 3, 4, 16, 16, 1, 1, 1)               \
    X(HALO_F64_3x3_128x64, PolF64, 128, 64, 2, 2, 3, 3, 4, 16, 16, 1, 2, 1)            \
    X(HALO_F64_3x3_176x64_KS2, PolF64, 176, 64, 1, 4, 3, 3, 4, 16, 16, 2, 1, 2)

hipError_t launch_halo(Variant v, const ConvParams& p, bool dgrad, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, r, s, cb, wp, sl, ks, wpe, blm) \
    case Variant::name:                                                \
        return launch_halo_variant<pol, tm, tn, wmm, wnn, r, s, cb, wp, sl, ks, wpe, blm>(p, dgrad, stream);
        MICONV_HALO_VARIANTS(X)
#undef X
    default: return dgrad ? hipErrorInvalidValue : launch_halo_bf16(v, p, stream);
    }
}

}  // namespace miconv
