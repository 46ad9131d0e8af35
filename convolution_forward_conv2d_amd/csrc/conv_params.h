// conv_params.h -- kernel arguments shared by the host dispatcher and the
// HIP kernels of libmiconv.  Plain data, passed by value as kernel arguments.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace miconv {

// Unsigned division by a run-time constant through a multiply-high, valid
// for numerators below 2^31 (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, the round-up variant):
//   shift = ceil(log2(d)), mul = floor(2^32 * (2^shift - d) / d) + 1,
//   n / d = (umulhi(n, mul) + n) >> shift.
struct FastDiv {
    uint32_t d;
    uint32_t mul;
    uint32_t shift;

    FastDiv() : d(1), mul(1), shift(0) {}
    explicit FastDiv(uint32_t divisor) : d(divisor) {
        shift = 0;
        while ((uint64_t(1) << shift) < divisor) ++shift;
        mul = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << shift) - divisor)) / divisor + 1);
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(n, mul);
#else
        uint32_t hi = uint32_t((uint64_t(n) * mul) >> 32);
#endif
        return (hi + n) >> shift;
    }
    __host__ __device__ __forceinline__ void divmod(uint32_t n, uint32_t& q, uint32_t& r) const {
        q = div(n);
        r = n - q * d;
    }
};

// One forward convolution, everything the kernels need.  Element offsets are
// 32-bit: the dispatcher rejects tensors whose highest offset reaches 2^31.
struct ConvParams {
    const void* x;
    const void* w;
    void* y;
    int N, C, H, W;
    int K, R, S;
    int P, Q;
    int u, v;            // strides along H and W
    int pad_top, pad_left;
    int sxn, sxc, sxh, sxw;   // input element strides
    int syn, syk, syp, syq;   // output element strides
    int Hp;              // H + pad_top + pad_bottom (rows of the zero-padded input)
    int M;               // N * P * Q   (rows of the implicit GEMM)
    int Kred;            // C * R * S   (reduction length)
    int m_tiles, n_tiles;
    int m_step;          // output rows per m tile (halo kernel: TM, or P*Q for one image per tile)
    FastDiv div_pq, div_q, div_rs, div_s, div_hp;
    FastDiv div_u, div_v;   // by the strides (data-gradient gather kernel)
    // filter gradient: dy's element strides and division by P*Q and by Q
    int sdn, sdk, sdp, sdq;
    FastDiv div_opq, div_oq;
    // Channel-blocked layouts: channel c of x lies at (c / xcb) * sxcb +
    // (c % xcb) * sxc, output channel k of y at (k / ycb) * sycb + (k % ycb) * syk
    // (blk_off); an unblocked tensor is one block of 2^30 channels.  Filters
    // are packed KCRS when wkb == 0, else blocked [K/wkb][C/wcb][R][S][wcb][wkb].
    FastDiv div_xcb, div_ycb;
    int sxcb, sycb;
    int wkb, wcb;
    double alpha, beta;  // converted to the accumulation type inside the kernel
    int tile_rev;        // 1: tiles run in reverse order (xcd_logical_tile); tests only
    int n_group;         // n tiles per group of the logical tile order (grouped_tile); 0: one group
};

// Element offset of channel c in a channel-blocked dimension (block size
// d.d, block stride sblk, stride inside a block sc).
__host__ __device__ __forceinline__ int blk_off(const FastDiv& d, int sblk, int sc, int c)
{
    uint32_t b, i;
    d.divmod((uint32_t)c, b, i);
    return (int)b * sblk + (int)i * sc;
}

// Element offset of F[k, c, r*S + s] in blocked filters [K/kb][C/cb][R][S][cb][kb].
__host__ __device__ __forceinline__ int wblk_off(int k, int c, int tap, int C, int RS, int kb, int cb)
{
    return ((k / kb) * (C / cb) + c / cb) * (RS * cb * kb) + (tap * cb + c % cb) * kb + k % kb;
}

constexpr uint32_t kOneBlock = 1u << 30;   // block size of an unblocked channel dimension

}  // namespace miconv
