// conv_fwd_halo_bf16.hip -- bf16 convolution forward pass (fp32 accumulate,
// fp32 output) as a batch-reduce GEMM over the R x S filter taps.
//
// The tap-batched scheme of conv_fwd_halo.hip, laid out for the
// v_mfma_f32_32x32x16_bf16 instruction, whose lanes each supply eight
// consecutive reduction elements.  With the reduction ordered as
// (channel block, tap, 16 channels), eight consecutive elements are eight
// channels at one tap, so both operands are stored channel-innermost in LDS
// and every MFMA operand is one 16-byte LDS read:
//
//  * input halo: the zero-padded input rows ("slots") that the tile's output
//    rows touch, WP pixels per slot; per pixel the chunk's 16 channels as two
//    8-channel groups of 16 bytes, on a 48-byte pixel pitch (the odd number
//    of 16-byte units keeps a wave's reads of consecutive pixels on distinct
//    banks);
//  * filter slab: per tap, per filter, the same two 8-channel groups, the
//    group order swapped for filters with ((n >> 2) ^ (n >> 3)) odd, which
//    spreads 8 or 16 consecutive filters over all banks without padding.
//
// The filter arrives in packed KCRS order, where a filter's 8 channels x R*S
// taps form one contiguous run: a thread loads that run with 16-byte loads
// and regroups it by tap in registers (byte permutes) before its LDS stores,
// so no separate transpose pass or buffer exists.  Input halo pixels come in
// as eight 2-byte loads per 8-channel group, or as one 16-byte load when the
// channels of x are contiguous and aligned (NHWC-like layouts).
//
// Batch-reduce GEMM of the single-building-block page ("Proposed Method"),
// read directly from x with no packed copy (zero-memory direct-convolution
// page, "Proposed Method"), double-buffered through LDS (maxDNN page,
// "Proposed Method").
//
// DG = true computes the data gradient of a stride-1 convolution as the
// forward pass of dy with the filter transposed (K <-> C) and flipped, as
// the fp32 halo kernel does (the host passes that forward problem: x = dy,
// y = dx, C and K exchanged).  Only the slab differs: a unit (dx channel n,
// 8-channel group g) needs, per tap, the 8 values F[c0 + 8g + j, n, tap]
// of 8 filters of the real problem, which lie C*R*S apart.  Two threads
// share a unit: each loads 4 of the runs F[c0 + 8g + j, n, 0 .. RS-1] with
// 2-byte loads (consecutive lanes take consecutive n, whose runs are
// adjacent in memory) and packs tap RS-1-t of its runs into 8 bytes of slab
// tap t.
//
// WB = true reads blocked filters [K/kb][C/cb][R][S][cb][kb] (the forward
// pass; kb a multiple of 8, cb of 16): there 8 consecutive filters of one
// (channel, tap) are one 16-byte load.  A thread takes blocks of (tap, 8-channel
// group, 8 filters): 8 loads, one per channel, and an 8 x 8 transpose of the
// 16-bit values in registers (byte permutes) gives each filter's 8 channels,
// stored as the same slab units the KCRS loader writes.
//
// Eligibility (checked by the host): R and S equal to the instance's; C a
// multiple of 16; W + pad_left + pad_right <= WP; every tile's slot span
// <= SL; w 16-byte aligned (the forward pass).
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

// filter n of a tile keeps group g of a tap at 16-byte unit 2n + (g ^ swz(n))
__device__ __forceinline__ int slab_swz(int n) { return ((n >> 2) ^ (n >> 3)) & 1; }

namespace {
constexpr int kBf16BufWord3 = 0x00020000;         // raw 32-bit buffer, range-checked per dword
constexpr int kBf16Outside = (int)0x80000000u;    // an offset past x and w (both under 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bf16_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBf16BufWord3);
}
__device__ __forceinline__ u32x4 bf16_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return u32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint32_t bf16_load2(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
}  // namespace

template <int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int WP, int SL, bool CVEC, bool DG, bool WB,
          bool RV>
__global__ void __launch_bounds__(256)
conv_fwd_halo_bf16_kernel(const ConvParams p)
{
    using Pol = PolBF16;
    constexpr int NT = 256;
    constexpr int BM = 32;
    constexpr int RS = R * S;
    constexpr int CB = 16;                        // channels per chunk = one MFMA k-step per tap
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int PIX = 48;                       // bytes per halo pixel: two 16-byte groups + pad
    constexpr int HALO_BYTES = SL * WP * PIX;
    constexpr int HU = 2 * SL * WP;               // halo units (8-channel group, pixel) per chunk
    constexpr int HUT = (HU + NT - 1) / NT;       // per thread
    constexpr int TAP_BYTES = TN * 32;            // one tap of the slab: TN filters x 16 channels
    constexpr int SLAB_BYTES = RS * TAP_BYTES;
    constexpr int SU = 2 * TN;                    // slab units (filter, 8-channel group) per chunk
    constexpr int SUD = DG ? 2 * SU : SU;         // DG: two threads per unit, 4 filter runs each
    constexpr int SUT = (SUD + NT - 1) / NT;
    constexpr int NV = RS;                        // 16-byte vectors per slab unit: 8 channels x RS taps
    constexpr int ND = DG ? 4 * RS : 1;           // DG: 2-byte loads per half unit (4 runs of RS taps)
    constexpr int BUF_BYTES = HALO_BYTES + SLAB_BYTES;
    // WB: transpose blocks (tap, group, filter octet) per chunk, per thread
    constexpr int OCT = TN / 8;
    constexpr int NB = RS * 2 * OCT;
    constexpr int WBT = WB ? (NB + NT - 1) / NT : 0;
    static_assert(!(WB && DG), "blocked filters in the forward pass only");
    // RV: blocks (group g, slot, 8-pixel segment) of 8 channels x 8 pixels
    constexpr int NSEG = (WP + 7) / 8;
    constexpr int NBX = 2 * SL * NSEG;
    constexpr int NBT = RV ? (NBX + NT - 1) / NT : 0;
    static_assert(!(RV && CVEC), "one input loader");
    constexpr int HSP = RV ? 8 * NBT : HUT;          // halo store pieces per chunk
    static_assert(TN % 8 == 0, "whole filter octets");
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    static_assert(BUF_BYTES % 16 == 0, "16-byte aligned buffers");
    static_assert(4 * BM * (BM + 1) * 4 <= 2 * BUF_BYTES, "epilogue stage fits");
    static_assert(((R - 1) * WP + S - 1) * PIX + 16 < 65536 && (RS - 1) * TAP_BYTES < 65536,
                  "LDS immediate offsets");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tile = xcd_logical_tile((int)blockIdx.x, p.m_tiles * p.n_tiles, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * p.m_step;
    const int m_end = min(m0 + p.m_step, p.M);
    const int n0 = nt * TN;

    const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
    const uint16_t* __restrict__ w = static_cast<const uint16_t*>(p.w);
    // x (and the packed filters of the forward pass) through range-checked
    // buffer descriptors: a unit outside x or past K reads at an offset past
    // the buffer and gets zeros, so the stores need no masks and a chunk's
    // channel offset is the scalar offset (host: x, w under 2^31 bytes)
    const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) +
                            (int64_t)(p.H - 1) * p.sxh + (int64_t)(p.W - 1) * p.sxw + 1;
    const __amdgpu_buffer_rsrc_t xr = bf16_rsrc(p.x, 2 * x_elems);
    const __amdgpu_buffer_rsrc_t wr = bf16_rsrc(p.w, 2 * (int64_t)p.K * p.Kred);

    if constexpr (RV) {
        // both halo buffers start zeroed: the row loader writes only pixels inside x
        for (int i = tid; i < HALO_BYTES / 16; i += NT) {
            reinterpret_cast<u32x4*>(smem)[i] = u32x4{0, 0, 0, 0};
            reinterpret_cast<u32x4*>(smem + BUF_BYTES)[i] = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
    }

    auto vrow = [&](int m) {
        uint32_t n, pq, pp, q;
        p.div_pq.divmod((uint32_t)m, n, pq);
        p.div_q.divmod(pq, pp, q);
        return (int)n * p.Hp + (int)pp * p.u;
    };
    const int vr_first = vrow(m0);
    const int nslots = vrow(m_end - 1) + R - vr_first;   // <= SL (host-checked)

    // ---- halo loader: unit e = (group g, pixel), pixel fastest along the lanes
    int h_voff[HUT];                                 // byte offset at the chunk's first channel
#pragma unroll
    for (int i = 0; i < HUT; ++i) {
        const int e = tid + NT * i;
        const int pix = e % (SL * WP);
        const int g = e / (SL * WP);
        const int col = pix % WP;
        const int slot = pix / WP;
        uint32_t n, hp;
        p.div_hp.divmod((uint32_t)(vr_first + slot), n, hp);
        const int h = (int)hp - p.pad_top;
        const int wcol = col - p.pad_left;
        const bool ok = e < HU && slot < nslots && (int)n < p.N && h >= 0 && h < p.H && wcol >= 0 &&
                        wcol < p.W;
        h_voff[i] = ok ? 2 * ((int)n * p.sxn + 8 * g * p.sxc + h * p.sxh + wcol * p.sxw) : kBf16Outside;
    }

    // RV (x with unit column stride, 16-byte aligned rows): block b = (group g,
    // slot, segment) takes pixels w0 .. w0 + 7 (w0 = 8 * segment) of the
    // slot's input row for the group's 8 channels: one 16-byte load per
    // channel, an 8 x 8 transpose of the 16-bit values in registers, one
    // 16-byte LDS unit per pixel inside the row.  Pixels outside the plane
    // (padding columns, rows outside x, slots past the tile) are never
    // written: the halo starts zeroed.  (Measured on the 13x13 layers at a
    // 16-element pitch: 1-3% faster than eight 2-byte loads per pixel group;
    // the blocks spread over all four waves instead of the first: 5-7% slower.)
    int rv_voff[RV ? NBT : 1], rv_pix[RV ? NBT : 1], rv_np[RV ? NBT : 1];
    uint32_t rv_last = 0;
    if constexpr (RV) {
#pragma unroll
        for (int i = 0; i < NBT; ++i) {
            const int b = tid + NT * i;
            const int seg = b % NSEG;
            const int slot = (b / NSEG) % SL;
            const int g = b / (NSEG * SL);
            uint32_t n, hp;
            p.div_hp.divmod((uint32_t)(vr_first + slot), n, hp);
            const int h = (int)hp - p.pad_top;
            const int w0 = 8 * seg;
            const bool ok = b < NBX && slot < nslots && (int)n < p.N && h >= 0 && h < p.H && w0 < p.W;
            rv_voff[i] = ok ? 2 * ((int)n * p.sxn + 8 * g * p.sxc + h * p.sxh + w0) : kBf16Outside;
            rv_pix[i] = (slot * WP + w0 + p.pad_left) * PIX + 16 * g;   // LDS byte offset of pixel w0
            rv_np[i] = ok ? min(8, p.W - w0) : 0;                      // pixels inside the row
            // the tensor's last row (channel C-1 is group 1, channel 7 of the
            // last chunk) ends x's storage: a segment reaching past W there
            // is read pixel by pixel
            const bool last = ok && (int)n == p.N - 1 && h == p.H - 1 && g == 1 && w0 + 8 > p.W;
            rv_last |= (last ? 1u : 0u) << i;
        }
    }
    u32x4 rv_val[RV ? NBT : 1][8];

    // ---- slab loader: unit e = (filter row, 8-channel group)
    int s_off[SUT];                                  // DG: elements (masked); else byte offsets (past w: none)
    uint32_t s_ok = 0;
#pragma unroll
    for (int i = 0; i < SUT; ++i) {
        const int e = tid + NT * i;
        const int half = DG ? e / SU : 0;
        const int ue = DG ? e % SU : e;
        const int row = ue >> 1;
        const int g = ue & 1;
        const bool ok = e < SUD && n0 + row < p.K;
        // DG: F[c0 + 8g + 4half + j, n, t] at ((c0 + 8g + 4half + j) * K + n) * RS + t,
        // K the channel count of dx here
        if constexpr (DG)
            s_off[i] = ok ? ((8 * g + 4 * half) * p.K + n0 + row) * RS : 0;
        else
            s_off[i] = ok ? 2 * ((n0 + row) * p.Kred + 8 * g * RS) : kBf16Outside;
        s_ok |= (ok ? 1u : 0u) << i;
    }

    // WB: block b = (tap t, group g, octet o), octet fastest (consecutive lanes
    // read consecutive 16-byte pieces of one (channel, tap) filter row)
    int wb_voff[WB ? WBT : 1];                      // byte offsets (past w: none)
    if constexpr (WB) {
        const int cblk = RS * p.wcb * p.wkb;             // elements of one (filter block, channel block)
#pragma unroll
        for (int i = 0; i < WBT; ++i) {
            const int b = tid + NT * i;
            const int o = b % OCT;
            const int tg = b / OCT;
            const int g = tg & 1;
            const int t = tg >> 1;
            const int k = n0 + 8 * o;
            const bool ok = b < NB && k < p.K;
            wb_voff[i] = ok ? 2 * ((k / p.wkb) * (p.C / p.wcb) * cblk + (t * p.wcb + 8 * g) * p.wkb + k % p.wkb)
                            : kBf16Outside;
        }
    }
    u32x4 wb_val[WB ? WBT : 1][8];

    // registers of the chunk in flight
    uint32_t h_raw[CVEC ? 1 : HUT][8];
    u32x4 h_vec[CVEC ? HUT : 1];
    u32x4 s_val[SUT][DG ? 1 : NV];
    uint16_t s_raw[SUT][ND];

    // A chunk moves global -> registers -> LDS in pieces: load piece q is
    // one global load (a 2-byte channel value or a 16-byte vector), store
    // piece q one 16-byte LDS write (a halo unit, or one tap of a slab unit).
    constexpr int NLH = RV ? 8 * NBT : CVEC ? HUT : 8 * HUT;    // halo load pieces
    constexpr int NL = NLH + (WB ? 8 * WBT : SUT * (DG ? ND : NV));   // load pieces per chunk
    constexpr int NS = HSP + (WB ? 8 * WBT : SUT * RS);              // store pieces per chunk

    // No load sits in a branch: the halo and the forward pass's filters come
    // through the buffer descriptors (zeros outside); the data gradient's
    // filter loads are unconditional at a valid address and their values are
    // replaced by zeros at the store.
    // x offset of a chunk's first channel (channel-blocked x: the chunk lies in one block)
    auto x_chunk = [&](int c0) { return blk_off(p.div_xcb, p.sxcb, p.sxc, c0); };
    auto load_piece = [&](int q, int c0) {
        if (q < NLH) {
            if constexpr (RV) {
                // block i, channel j (unconditional: an empty block reads the chunk's first row)
                const int i = q / 8, j = q % 8;
                if (j == 7 && ((rv_last >> i) & 1) && c0 + CB == p.C) {
                    const uint16_t* src = x + rv_voff[i] / 2 + x_chunk(c0) + j * p.sxc;
                    uint32_t v[4] = {0, 0, 0, 0};
                    for (int f = 0; f < rv_np[i]; ++f) v[f >> 1] |= (uint32_t)src[f] << (16 * (f & 1));
                    rv_val[i][j] = u32x4{v[0], v[1], v[2], v[3]};
                } else {
                    rv_val[i][j] = bf16_load16(xr, rv_voff[i], 2 * (x_chunk(c0) + j * p.sxc));
                }
            } else if constexpr (CVEC) {
                h_vec[q] = bf16_load16(xr, h_voff[q], 2 * x_chunk(c0));
            } else {
                const int i = q / 8, j = q % 8;
                h_raw[i][j] = bf16_load2(xr, h_voff[i], 2 * (x_chunk(c0) + j * p.sxc));
            }
        } else if constexpr (WB) {
            // the chunk's 16 channels lie in one channel block
            const int i = (q - NLH) / 8, j = (q - NLH) % 8;
            const int co = (c0 / p.wcb) * (RS * p.wcb * p.wkb) + (c0 % p.wcb) * p.wkb;
            wb_val[i][j] = bf16_load16(wr, wb_voff[i], 2 * (co + j * p.wkb));
        } else if constexpr (DG) {
            const int i = (q - NLH) / ND, v = (q - NLH) % ND;
            const int j = v / RS, t = v % RS;
            s_raw[i][v] = w[s_off[i] + (c0 + j) * p.K * RS + t];
        } else {
            const int i = (q - NLH) / NV, v = (q - NLH) % NV;
            s_val[i][v] = bf16_load16(wr, s_off[i] + 16 * v, 2 * c0 * RS);
        }
    };

    auto store_piece = [&](int q, int buf) {
        unsigned char* hb = smem + buf * BUF_BYTES;
        if constexpr (RV) {
            if (q < HSP) {
                // pixel f of block i: dword d holds channels 2d and 2d+1, the 16-bit
                // half f%2 of word f/2 of those channels' loads
                const int i = q / 8, f = q % 8;
                if (f < rv_np[i]) {
                    u32x4 out;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t lo = rv_val[i][2 * d][f >> 1];
                        const uint32_t hi = rv_val[i][2 * d + 1][f >> 1];
                        out[d] = (f & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                    }
                    *reinterpret_cast<u32x4*>(hb + rv_pix[i] + f * PIX) = out;
                }
                return;
            }
        }
        if (!RV && q < HUT) {
            const int i = q;
            const int e = tid + NT * i;
            if (HU % NT == 0 || e < HU) {
                const int pix = e % (SL * WP);
                const int g = e / (SL * WP);
                u32x4 val;
                if constexpr (CVEC) {
                    val = h_vec[i];
                } else {
                    // the empty asm keeps the packing at this point of the
                    // compute; hoisted next to the loads it would wait for them
#pragma unroll
                    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(h_raw[i][j]));
#pragma unroll
                    for (int d = 0; d < 4; ++d) val[d] = h_raw[i][2 * d] | (h_raw[i][2 * d + 1] << 16);
                }
                *reinterpret_cast<u32x4*>(hb + pix * PIX + 16 * g) = val;
            }
        } else if constexpr (WB) {
            // filter f of block i: dword d holds channels 2d, 2d+1, i.e. the
            // 16-bit half f%2 of word f/2 of channel rows 2d and 2d+1
            const int i = (q - HSP) / 8, f = (q - HSP) % 8;
            const int b = tid + NT * i;
            if (NB % NT == 0 || b < NB) {
                const int o = b % OCT;
                const int tg = b / OCT;
                const int g = tg & 1;
                const int t = tg >> 1;
                const int row = 8 * o + f;
                u32x4 out;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t lo = wb_val[i][2 * d][f >> 1];
                    const uint32_t hi = wb_val[i][2 * d + 1][f >> 1];
                    out[d] = (f & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                *reinterpret_cast<u32x4*>(hb + HALO_BYTES + t * TAP_BYTES + 16 * (2 * row + (g ^ slab_swz(row)))) = out;
            }
        } else {
            const int i = (q - HSP) / RS, t = (q - HSP) % RS;
            const int e = tid + NT * i;
            if (SUD % NT == 0 || e < SUD) {
                const int half = DG ? e / SU : 0;
                const int ue = DG ? e % SU : e;
                const int row = ue >> 1;
                const int g = ue & 1;
                const bool ok = (s_ok >> i) & 1;
                unsigned char* dst = hb + HALO_BYTES + 16 * (2 * row + (g ^ slab_swz(row)));
                if constexpr (DG) {
                    // slab tap t is tap RS-1-t of the runs (the filter flipped);
                    // dword 2half + d holds runs 4half + 2d and 4half + 2d + 1
                    u32x2 o2;
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const uint32_t lo = s_raw[i][(2 * d) * RS + RS - 1 - t];
                        const uint32_t hi = s_raw[i][(2 * d + 1) * RS + RS - 1 - t];
                        o2[d] = ok ? (lo | (hi << 16)) : 0u;
                    }
                    *reinterpret_cast<u32x2*>(dst + 8 * half + t * TAP_BYTES) = o2;
                } else {
                    // element k of the unit's run is channel k / RS at tap k % RS:
                    // dword d of tap t holds channels 2d and 2d+1 of that tap
                    const uint32_t* words = reinterpret_cast<const uint32_t*>(&s_val[i][0]);
                    u32x4 out;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int klo = (2 * d) * RS + t;
                        const int khi = (2 * d + 1) * RS + t;
                        const uint32_t wlo = words[klo >> 1];
                        const uint32_t whi = words[khi >> 1];
                        const uint32_t lo = (klo & 1) ? (wlo >> 16) : (wlo & 0xffffu);
                        const uint32_t hi = (khi & 1) ? (whi & 0xffff0000u) : (whi << 16);
                        out[d] = lo | hi;
                    }
                    *reinterpret_cast<u32x4*>(dst + t * TAP_BYTES) = out;
                }
            }
        }
    };

    // ---- per-wave MFMA geometry
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane & 31;
    const int lgrp = lane >> 5;
    int a_base[FM];                      // byte offset of tap (0,0), channel group lgrp, per block
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + i * BM + lrow;
        int pix = 0;
        if (m < m_end) {
            uint32_t n, pq, pp, q;
            p.div_pq.divmod((uint32_t)m, n, pq);
            p.div_q.divmod(pq, pp, q);
            pix = ((int)n * p.Hp + (int)pp * p.u - vr_first) * WP + (int)q * p.v;
        }
        a_base[i] = pix * PIX + 16 * lgrp;
    }
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = wn * WN + j * BM + lrow;
        b_base[j] = HALO_BYTES + 16 * (2 * n + (lgrp ^ slab_swz(n)));
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // One MFMA k-step per tap; the operands of step t + PFD are read from
    // LDS during step t.  The chunk held in registers (the next one) is
    // written to the other LDS buffer over steps 0 .. SPLIT-1 (that buffer's
    // last readers finished before the previous barrier), then the loads of
    // the chunk after it are issued over the remaining steps.  Each step's
    // memory instructions stay between its MFMAs, so no step waits on a
    // burst; one barrier ends each chunk.
    constexpr int SPLIT = RS / 2;
    constexpr int PFD = 1;
    bf16x8 fa[PFD + 1][FM], fb[PFD + 1][FN];
    auto frags = [&](const unsigned char* buf, int t, int k) {
        const int aoff = ((t / S) * WP + (t % S)) * PIX;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[k][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + a_base[i] + aoff));
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[k][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + b_base[j] + t * TAP_BYTES));
    };
    // STORE / LOAD are compile-time so that a step is straight-line code the
    // scheduler can interleave with the MFMAs
    auto compute = [&](auto store_c, auto load_c, int cur, int c_load) {
        constexpr bool STORE = decltype(store_c)::value;
        constexpr bool LOAD = decltype(load_c)::value;
        const unsigned char* buf = smem + cur * BUF_BYTES;
#pragma unroll
        for (int t = 0; t < PFD; ++t) frags(buf, t, t);
#pragma unroll
        for (int t = 0; t < RS; ++t) {
            if (t + PFD < RS) frags(buf, t + PFD, (t + PFD) % (PFD + 1));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t % (PFD + 1)][i], fb[t % (PFD + 1)][j],
                                                                        acc[i][j], 0, 0, 0);
            if constexpr (STORE) {
#pragma unroll
                for (int q = 0; q < NS; ++q)
                    if (q * SPLIT / NS == t) store_piece(q, cur ^ 1);
            }
            if constexpr (LOAD) {
#pragma unroll
                for (int q = 0; q < NL; ++q)
                    if (SPLIT + q * (RS - SPLIT) / NL == t) load_piece(q, c_load);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };
    using yes = std::true_type;
    using no = std::false_type;

    const int nblocks = p.C / CB;
#pragma unroll
    for (int q = 0; q < NL; ++q) load_piece(q, 0);
#pragma unroll
    for (int q = 0; q < NS; ++q) store_piece(q, 0);
    if (nblocks > 1) {
#pragma unroll
        for (int q = 0; q < NL; ++q) load_piece(q, CB);
    }
    __syncthreads();
    int it = 0;
    for (; it + 2 < nblocks; ++it) compute(yes{}, yes{}, it & 1, (it + 2) * CB);
    if (it + 1 < nblocks) compute(yes{}, no{}, (it++) & 1, 0);
    compute(no{}, no{}, it & 1, 0);

    store_acc_tile<Pol, FM, FN>(p, smem, acc, m0 + wm * WM, n0 + wn * WN, m_end, wave, lane);
}

// ------------------------------------------------------------------ instances and launch

template <int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int WP, int SL, bool DGOK>
static hipError_t launch_halo_bf16_variant(const ConvParams& p0, bool dgrad, hipStream_t stream)
{
    ConvParams p = p0;
    // blocked filters: the host checked kb % 8 == 0, cb % 16 == 0, K % kb == 0,
    // C % cb == 0 and a 16-byte aligned w (forward pass only)
    if (p.wkb > 0 && (dgrad || p.wkb % 8 != 0 || p.wcb % 16 != 0 || p.K % p.wkb != 0 || p.C % p.wcb != 0 ||
                      (uintptr_t)p.w % 16 != 0))
        return hipErrorInvalidValue;
    if (p.m_step <= 0 || p.m_step > TM) p.m_step = TM;   // the host sets P*Q for image tiles
    p.m_tiles = (p.M + p.m_step - 1) / p.m_step;
    p.n_tiles = (p.K + TN - 1) / TN;
    const dim3 grid((unsigned)(p.m_tiles * p.n_tiles));
    // 16-byte input loads when the 8 channels of a group are contiguous and
    // every group starts on a 16-byte boundary
    const bool cvec = p.sxc == 1 && (uintptr_t)p.x % 16 == 0 && p.sxn % 8 == 0 && p.sxh % 8 == 0 &&
                      p.sxw % 8 == 0 && p.sxcb % 8 == 0;
    // 16-byte loads of 8 pixels per channel when x's rows have unit column
    // stride, start on 16-byte boundaries and hold whole 8-pixel segments
    // (a padded row pitch: the last segment stays inside the row's storage)
    // (and NCHW nesting, so that only the tensor's last row ends its storage)
    const bool rvec = !cvec && p.div_xcb.d == kOneBlock && p.sxw == 1 && (uintptr_t)p.x % 16 == 0 &&
                      p.sxn % 8 == 0 && p.sxc % 8 == 0 && p.sxh % 8 == 0 && p.sxh >= (p.W + 7) / 8 * 8 &&
                      (int64_t)p.sxc >= (int64_t)p.sxh * p.H && (int64_t)p.sxn >= (int64_t)p.sxc * p.C;
#define MICONV_BF16_LAUNCH(CV, DGV, WBV, RVV)                                                                      \
    hipLaunchKernelGGL((conv_fwd_halo_bf16_kernel<TM, TN, WAVES_M, WAVES_N, R, S, WP, SL, CV, DGV, WBV, RVV>), grid, \
                       dim3(256), 0, stream, p)
    if (dgrad) {
        if constexpr (DGOK) {
            if (cvec)
                MICONV_BF16_LAUNCH(true, true, false, false);
            else if (rvec)
                MICONV_BF16_LAUNCH(false, true, false, true);
            else
                MICONV_BF16_LAUNCH(false, true, false, false);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (p.wkb > 0) {
        if (cvec)
            MICONV_BF16_LAUNCH(true, false, true, false);
        else if (rvec)
            MICONV_BF16_LAUNCH(false, false, true, true);
        else
            MICONV_BF16_LAUNCH(false, false, true, false);
    } else if (cvec) {
        MICONV_BF16_LAUNCH(true, false, false, false);
    } else if (rvec) {
        MICONV_BF16_LAUNCH(false, false, false, true);
    } else {
        MICONV_BF16_LAUNCH(false, false, false, false);
    }
#undef MICONV_BF16_LAUNCH
    return hipGetLastError();
}

// (DG: the data-gradient slab holds 36 more registers per 256 slab half units)
//        name                     TM   TN  waves  R  S  WP  SL  DG
#define MICONV_HALO_BF16_VARIANTS(X)                              \
    X(HALO_BF16_3x3_128x128, 128, 128, 2, 2, 3, 3, 16, 16, true)   \
    X(HALO_BF16_3x3_128x64, 128, 64, 2, 2, 3, 3, 16, 16, true)     \
    X(HALO_BF16_3x3_192x128, 192, 128, 2, 2, 3, 3, 16, 16, false)

static hipError_t launch_halo_bf16_any(Variant v, const ConvParams& p, bool dgrad, hipStream_t stream)
{
    switch (v) {
#define X(name, tm, tn, wmm, wnn, r, s, wp, sl, dg) \
    case Variant::name: return launch_halo_bf16_variant<tm, tn, wmm, wnn, r, s, wp, sl, dg>(p, dgrad, stream);
        MICONV_HALO_BF16_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

// the buffer descriptors' range: x (dy) and the filters under 2^31 bytes
static bool bf16_buffers_fit(const ConvParams& p)
{
    const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) +
                            (int64_t)(p.H - 1) * p.sxh + (int64_t)(p.W - 1) * p.sxw + 1;
    return 2 * x_elems < ((int64_t)1 << 31) && 2 * (int64_t)p.C * p.K * p.R * p.S < ((int64_t)1 << 31);
}

hipError_t launch_halo_bf16(Variant v, const ConvParams& p, hipStream_t stream)
{
    if (!bf16_buffers_fit(p)) return hipErrorInvalidValue;
    return launch_halo_bf16_any(v, p, false, stream);
}

hipError_t launch_halo_bf16_dgrad(Variant v, const ConvParams& p, hipStream_t stream)
{
    if (!bf16_buffers_fit(p)) return hipErrorInvalidValue;
    return launch_halo_bf16_any(v, p, true, stream);
}

}  // namespace miconv
