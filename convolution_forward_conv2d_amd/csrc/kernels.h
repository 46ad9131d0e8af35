// kernels.h -- kernel variants of libmiconv and their launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "conv_params.h"

namespace miconv {

enum class Variant : int {
    DIRECT = 0,          // one thread per output, any dtype/layout (plain loop, no MFMA)
    DG_PHASE,            // data gradient onto 1-4 channels by stride phase (conv_bwd_data_phase.hip)
    DG_ROWS,             // ... onto one channel, dy rows staged in LDS (same file)
    ROWS_F32_S11_256x32, // forward pass, reduction streamed by filter row (conv_fwd_rows.hip)
    ROWS1_F32_S11_256x32, // ... onto one input channel, tap pairs (same file)
    ROWS1N6_F32_S11_256x32, // ... six output-row slots (short output rows)
    DG_ROWS_MFMA,        // data gradient, the same streaming per stride phase (conv_fwd_rows.hip)
    DG_SUBPIXEL,         // strided data gradient as a stride-1 GEMM onto the stride phases (conv_bwd_data_subpixel.hip)
    DG_TAPS,             // strided data gradient onto few channels, filter column taps as GEMM columns (conv_bwd_data_taps.hip)
    WGR_F32_S11_V2,      // filter gradient of a first layer on the vector ALU, staged output rows (conv_bwd_filter_rows.hip)
    WGR_F32_S11_V4,
    MFMA_F32_128x128,
    MFMA_F32_128x64,
    MFMA_F32_256x32,
    MFMA_F32_64x128,
    MFMA_F64_128x128,
    MFMA_F64_128x64,
    MFMA_F64_64x64,
    MFMA_BF16_128x128,
    MFMA_BF16_128x64,
    MFMA_BF16_256x32,
    HALO_F32_3x3_128x128,   // tap-batched kernel with an LDS input halo (conv_fwd_halo.hip)
    HALO_F32_3x3_128x64,
    HALO_F32_3x3_64x128,
    HALO_F32_3x3_96x128,
    HALO_F32_5x5_128x128,
    HALO_F32_5x5_128x128_C2,
    HALO_F32x16_3x3_176x128,
    HALO_F32x16_3x3_144x128,
    HALO_F32x16_5x5_128x96,        // 96 filters per tile (K = 96, e.g. a data gradient onto 96 channels)
    HALO_F32_5x5_128x96_C2,        // ... on 32x32 blocks, 2-channel chunks, four waves of 32 rows x 96
    HALO_F32x16_5x5_208x64,        // 208 rows x 64 filters on 16x16 blocks, 1x4 waves (two workgroups per CU)
    HALO_F32x16_3x3_176x128_KS2,   // two halves split the reduction of one tile
    HALO_F32_3x3_128x128_KS2,
    HALO_F64_3x3_128x128,
    HALO_F64_3x3_64x64,
    HALO_F64_3x3_128x64,           // fp64, 64 filters: two or three workgroups per CU
    HALO_F64_3x3_176x64_KS2,       // fp64, one output image per tile, the reduction split over two halves
    HALO_BF16_3x3_128x128,  // bf16 halo kernel, channel-innermost LDS (conv_fwd_halo_bf16.hip)
    HALO_BF16_3x3_128x64,
    HALO_BF16_3x3_192x128,
    WG_F32_128x128,         // filter gradient (conv_bwd_filter.hip)
    WG_F32_64x128,
    WG_F32_128x64,
    WG_F32_64x64,
    WG_F64_128x64,
    WG_F64_64x64,
    WG_BF16_128x128,
    WG_BF16_64x64,
    WGH_F32_3x3_W16,        // filter gradient, stride 1, halo in LDS (conv_bwd_filter_halo.hip)
    WGH_F32_5x5_W24,
    WGH_F32_5x5_W36,
    WGH_F32_3x3_W16_64x96,
    WGH_F32X16_3x3_W16,
    WGH_F32X16_5x5_W24,
    WGH_F64_3x3_W16,
    WGH_F32_3x3_Q12_64x96,   // ... stepping along output rows of exactly 12 columns
    WGH_F32_3x3_Q13,         // ... 13 columns (32x32 blocks)
    WGH_F32X16_5x5_Q20,      // ... 5x5, 20 columns
    WGH_F32X16_5x5_Q27,      // ... 5x5, 27 columns
    WGH_F32X16_5x5_Q20_64x48,  // ... 5x5, 20 columns, 64 filters x 48 columns (more tiles)
    WGH_F32X16_5x5_Q27_64x48,  // ... 5x5, 27 columns, 64 filters x 48 columns
    WGH_F32_3x3_Q13_KS4,       // 3x3, 13 columns, four groups of waves per tile
    WGH_F32_3x3_W16_64x96_KS4, // 3x3, 64 x 96, four groups of waves per tile
    WGH_F32_3x3_Q12_64x96_KS4, // 3x3, 12 columns, 64 x 96, four groups of waves per tile
    WGH_F32X16_5x5_Q20_64x48_KS4,  // 5x5, 20 columns, 64 x 48, four groups of waves per tile
    WGH_F32X16_5x5_Q27_64x48_KS4,  // 5x5, 27 columns, 64 x 48, four groups of waves per tile
    WGH_F32X16_PAIRS_S11_32x32,     // 11-wide filter rows, any height and row stride: (c, r) pairs staged
    WGH_F32X16_PAIRS_S11_32x32_KS4, // ... four groups of waves per tile
    WGH_F32X16_PAIRS_S11_32x64,     // ... 32 filters x 64 columns
    WGH_F64_3x3_W16_KS4,            // fp64 3x3 64x64, four groups of waves per tile
    WGH_F64_3x3_W16_64x96,          // fp64 3x3 64x96
    WGH_BF16_3x3_W16,               // bf16 x and dy staged as fp32: 3x3 64x64
    WGH_BF16_3x3_Q13,               // ... 13 columns
    WGH_BF16_3x3_W16_64x96_KS4,     // ... 64x96, four groups of waves per tile
    WGC_BF16_64x64,         // filter gradient, bf16, channels-last x and dy (conv_bwd_filter_cl.hip)
    WGC_BF16_64x64_KS2,     // ... two groups of waves split the reduction
    WGC_BF16_64x64_KS3,     // ... three groups
    WGS_F32_32x32,          // filter gradient, reduction split over waves (conv_bwd_filter_split.hip)
    WGS_F32_16x16,
    WGS_F32_8x16,
    WGS_F64_32x32,
    WGS_F64_16x16,
    WGS_BF16_32x32,
    BR_F32_128x128,         // batch-reduce GEMM, shared-LDS tiles (brgemm.hip)
    BR_F32_64x64,
    BR_F32_32x64,
    BR_F64_64x64,
    BR_F64_32x64,
    BR_BF16_128x128,
    BR_BF16_64x64,
    BR_BF16_32x128,
    WS_F32_64x64,           // batch-reduce GEMM, waves split the reduction (brgemm.hip)
    WS_F32_32x64,
    WS_F32_16x32,
    WS_F64_32x64,
    WS_F64_16x32,
    WS_BF16_32x64,
    WS_BF16_16x32,
    COUNT
};

enum class DType : int { F32 = 0, F64 = 1, BF16 = 2 };

// Launch an implicit-GEMM MFMA variant.  bvec: the filter may be read with
// 16-byte loads (w 16-byte aligned and C*R*S a multiple of the vector).
// tap: reduction in channel blocks per filter tap instead of flat KCRS order.
// dgrad: the data gradient, any stride (p laid out as conv_fwd_mfma.hip
// describes).
hipError_t launch_mfma(Variant v, const ConvParams& p, bool bvec, bool tap, bool dgrad, hipStream_t stream);

// Launch a tap-batched halo variant (the host has checked its eligibility).
// dgrad: p describes the forward problem equivalent to a stride-1 data
// gradient (conv_fwd_halo.hip); fp32 and fp64 instances only.
hipError_t launch_halo(Variant v, const ConvParams& p, bool dgrad, hipStream_t stream);
hipError_t launch_halo_bf16(Variant v, const ConvParams& p, hipStream_t stream);
hipError_t launch_halo_bf16_dgrad(Variant v, const ConvParams& p, hipStream_t stream);

// Launch the plain direct kernel (one thread per output element).
hipError_t launch_direct(DType dt, const ConvParams& p, hipStream_t stream);

// Filter gradient (implicit GEMM over the output positions); p laid out as
// conv_bwd_filter.hip describes.
// Filter gradient of a stride-1 layer through an LDS halo (R, S, dtype and
// Q + S - 1 <= the variant's row pitch, host-checked).  split_k > 0 (beta = 0
// only): dw is zeroed and each tile's reduction runs as two workgroups, the
// first taking k / (k + 1) of it, both adding into dw atomically.
hipError_t launch_bwd_filter_halo(Variant v, const ConvParams& p, int split_k, hipStream_t stream);
hipError_t launch_bwd_filter(Variant v, const ConvParams& p, hipStream_t stream);
hipError_t launch_bwd_filter_split(Variant v, const ConvParams& p, hipStream_t stream);
hipError_t launch_bwd_filter_cl(Variant v, const ConvParams& p, hipStream_t stream);

// Batch-reduce GEMM; p laid out as brgemm.hip describes.  16-byte operand
// loads are chosen inside when strides, k and alignment allow them.
hipError_t launch_brgemm(Variant v, const ConvParams& p, hipStream_t stream);
// Wave-split variants: the reduction elements one 16-byte load reads (A and
// B must be contiguous along k, k a multiple of it, loads 16-byte aligned);
// 0 for every other variant.
int brgemm_ws_run(Variant v);

// Pooling forward pass (one thread per output); p laid out as pool_fwd.hip describes.
hipError_t launch_pool_forward(DType dt, const ConvParams& p, hipStream_t stream);

// Data gradient, plain direct kernel (one thread per dx element); p is laid
// out as conv_bwd_data.hip describes.
hipError_t launch_bwd_data_direct(DType dt, const ConvParams& p, hipStream_t stream);
hipError_t launch_bwd_data_phase(DType dt, const ConvParams& p, hipStream_t stream);
bool bwd_data_rows_fits(const ConvParams& p, size_t* lds_bytes);
hipError_t launch_bwd_data_rows(const ConvParams& p, hipStream_t stream);
bool rows_fits(Variant v, const ConvParams& p);
hipError_t launch_rows(Variant v, const ConvParams& p, hipStream_t stream);
bool bwd_data_rows_mfma_fits(const ConvParams& p);
hipError_t launch_bwd_data_rows_mfma(const ConvParams& p, hipStream_t stream);
bool bwd_data_subpixel_fits(const ConvParams& p);
bool bwd_data_taps_fits(const ConvParams& p);
hipError_t launch_bwd_data_taps(const ConvParams& p, hipStream_t stream);
hipError_t launch_bwd_data_subpixel(DType dt, const ConvParams& p, hipStream_t stream);
bool bwd_filter_rows_fits(Variant v, const ConvParams& p);
hipError_t launch_bwd_filter_rows(Variant v, const ConvParams& p, hipStream_t stream);

}  // namespace miconv
