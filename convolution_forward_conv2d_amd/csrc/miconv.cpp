// miconv.cpp -- host side of the libmiconv C ABI: descriptors, validation,
// output size, kernel-variant choice and launch.
//
// Descriptor model: cuDNN page (Chetlur et al.), "Proposed Method": opaque
// tensor and filter descriptors with arbitrary strides, user-owned device
// memory, no auxiliary buffers, asymmetric padding.  Variant choice: the
// zero-memory direct-convolution page, "Proposed Method": blocking
// parameters chosen per shape by an analytical model.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <new>

#include <hip/hip_runtime.h>

#include "miconv.h"
#include "conv_params.h"
#include "kernels.h"

struct mic_handle_st {
    int device;
    int num_cu;
    hipStream_t stream;
};

struct mic_tensor_desc_st {
    bool set;
    mic_dtype dtype;
    int n, c, h, w;
    int64_t sn, sc, sh, sw;
    int cb;          // channel block (0: unblocked); channel c at (c / cb) * scb + (c % cb) * sc
    int64_t scb;
};

struct mic_filter_desc_st {
    bool set;
    mic_dtype dtype;
    int k, c, r, s;
    int kb, cb;      // 0, 0: packed KCRS; else blocked [K/kb][C/cb][R][S][cb][kb]
};

struct mic_conv_desc_st {
    bool set;
    int pad_top, pad_bottom, pad_left, pad_right;
    int u, v;
};

struct mic_pool_desc_st {
    bool set;
    mic_pool_mode mode;
    int r, s;
    int pad_top, pad_bottom, pad_left, pad_right;
    int u, v;
};

namespace {

using miconv::ConvParams;
using miconv::DType;
using miconv::FastDiv;
using miconv::Variant;

constexpr int64_t kMaxOffset = int64_t(1) << 30;   // element offsets stay far below 2^31
constexpr int kDefaultCUs = 256;                   // MI355X

bool valid_dtype(mic_dtype d) { return d == MIC_DTYPE_F32 || d == MIC_DTYPE_F64 || d == MIC_DTYPE_BF16; }

size_t dtype_size(mic_dtype d)
{
    switch (d) {
    case MIC_DTYPE_F32: return 4;
    case MIC_DTYPE_F64: return 8;
    case MIC_DTYPE_BF16: return 2;
    }
    return 0;
}

// Highest element offset a strided N,C,H,W tensor reaches, plus one.
int64_t extent(const mic_tensor_desc_st& d)
{
    const int64_t chan = d.cb > 0 ? (int64_t)(d.c / d.cb - 1) * d.scb + (int64_t)(d.cb - 1) * d.sc
                                  : (int64_t)(d.c - 1) * d.sc;
    return (int64_t)(d.n - 1) * d.sn + chan + (int64_t)(d.h - 1) * d.sh + (int64_t)(d.w - 1) * d.sw + 1;
}

bool blocked(const mic_tensor_desc_st* d) { return d && d->cb > 0; }
bool blocked(const mic_filter_desc_st* d) { return d && d->kb > 0; }

// Channel blocking of x, y and the filters into the kernel parameters
// (unblocked: one block of 2^30 channels, packed KCRS filters).
void set_blocks(ConvParams& p, const mic_tensor_desc_st* xd, const mic_tensor_desc_st* yd,
                const mic_filter_desc_st* wd)
{
    p.div_xcb = FastDiv(blocked(xd) ? (uint32_t)xd->cb : miconv::kOneBlock);
    p.sxcb = blocked(xd) ? (int)xd->scb : 0;
    p.div_ycb = FastDiv(blocked(yd) ? (uint32_t)yd->cb : miconv::kOneBlock);
    p.sycb = blocked(yd) ? (int)yd->scb : 0;
    p.wkb = blocked(wd) ? wd->kb : 0;
    p.wcb = blocked(wd) ? wd->cb : 0;
}

mic_status output_dims(const mic_conv_desc_st* cd, const mic_tensor_desc_st* xd,
                       const mic_filter_desc_st* wd, int* n, int* k, int* p, int* q)
{
    if (!cd || !xd || !wd || !cd->set || !xd->set || !wd->set) return MIC_STATUS_BAD_PARAM;
    if (xd->c != wd->c) return MIC_STATUS_BAD_PARAM;
    const int64_t hspan = (int64_t)xd->h + cd->pad_top + cd->pad_bottom - wd->r;
    const int64_t wspan = (int64_t)xd->w + cd->pad_left + cd->pad_right - wd->s;
    if (hspan < 0 || wspan < 0) return MIC_STATUS_BAD_PARAM;   // filter exceeds padded input
    const int64_t P = hspan / cd->u + 1;                          // floor: spans are >= 0
    const int64_t Q = wspan / cd->v + 1;
    if (P > INT32_MAX || Q > INT32_MAX) return MIC_STATUS_NOT_SUPPORTED;
    *n = xd->n;
    *k = wd->k;
    *p = (int)P;
    *q = (int)Q;
    return MIC_STATUS_SUCCESS;
}

struct Candidate {
    Variant v;
    int tm, tn;
    const char* name;
};

const Candidate kF32[] = {
    {Variant::MFMA_F32_128x128, 128, 128, "mfma_f32_128x128"},
    {Variant::MFMA_F32_128x64, 128, 64, "mfma_f32_128x64"},
    {Variant::MFMA_F32_64x128, 64, 128, "mfma_f32_64x128"},
    {Variant::MFMA_F32_256x32, 256, 32, "mfma_f32_256x32"},
};
const Candidate kF64[] = {
    {Variant::MFMA_F64_128x128, 128, 128, "mfma_f64_128x128"},
    {Variant::MFMA_F64_128x64, 128, 64, "mfma_f64_128x64"},
    {Variant::MFMA_F64_64x64, 64, 64, "mfma_f64_64x64"},
};
const Candidate kBF16[] = {
    {Variant::MFMA_BF16_128x128, 128, 128, "mfma_bf16_128x128"},
    {Variant::MFMA_BF16_128x64, 128, 64, "mfma_bf16_128x64"},
    {Variant::MFMA_BF16_256x32, 256, 32, "mfma_bf16_256x32"},
};
const Candidate kDirect = {Variant::DIRECT, 0, 0, "direct"};
const Candidate kDgPhase = {Variant::DG_PHASE, 0, 0, "phase"};
const Candidate kDgRows = {Variant::DG_ROWS, 0, 0, "rows"};
// forward pass with the reduction streamed by filter row (conv_fwd_rows.hip)
const Candidate kRowsF32 = {Variant::ROWS_F32_S11_256x32, 256, 32, "rows_f32_s11_256x32"};
const Candidate kDgRowsMfma = {Variant::DG_ROWS_MFMA, 256, 32, "rows_mfma_f32_s11_256x32"};
const Candidate kDgSubpixel = {Variant::DG_SUBPIXEL, 128, 64, "subpixel"};
const Candidate kDgTaps = {Variant::DG_TAPS, 0, 0, "taps"};
const Candidate kRows1F32 = {Variant::ROWS1_F32_S11_256x32, 256, 32, "rows1_f32_s11_256x32"};
const Candidate kRows1N6F32 = {Variant::ROWS1N6_F32_S11_256x32, 256, 32, "rows1n6_f32_s11_256x32"};
// Filter-gradient kernels: the gather kernel (conv_bwd_filter.hip, any
// geometry), the LDS-halo kernel (conv_bwd_filter_halo.hip: stride 1, fixed
// R x S, Q + S - 1 <= the row pitch wph) and the kernel that splits the
// reduction over the waves of one workgroup (conv_bwd_filter_split.hip:
// small tiles, tensors under 2 GiB).  ns is the measured time of one tile
// per reduction position (N*P*Q) on MI355X with per_cu workgroups resident
// on a compute unit; the plan picks the least rounds * ns.
enum class WgKind { GATHER, HALO, SPLIT, ROWS, CL };
struct WgCandidate {
    Candidate c;
    DType dt;
    WgKind kind;
    int r, s, wph;      // halo kernel only
    double ns;
    int per_cu;
    int qd;             // halo kernel: output rows of exactly qd columns (0: any width)
    int res2;           // halo kernel: two workgroups fit on a CU (LDS, registers)
};
const WgCandidate kWg[] = {
    {{Variant::WG_F32_128x128, 128, 128, "wg_f32_128x128"}, DType::F32, WgKind::GATHER, 0, 0, 0, 170.0, 1},
    {{Variant::WG_F32_64x128, 64, 128, "wg_f32_64x128"}, DType::F32, WgKind::GATHER, 0, 0, 0, 90.0, 1},
    {{Variant::WG_F32_128x64, 128, 64, "wg_f32_128x64"}, DType::F32, WgKind::GATHER, 0, 0, 0, 90.0, 1},
    {{Variant::WG_F32_64x64, 64, 64, "wg_f32_64x64"}, DType::F32, WgKind::GATHER, 0, 0, 0, 60.0, 1},
    {{Variant::WG_F64_128x64, 128, 64, "wg_f64_128x64"}, DType::F64, WgKind::GATHER, 0, 0, 0, 157.0, 1},
    {{Variant::WG_F64_64x64, 64, 64, "wg_f64_64x64"}, DType::F64, WgKind::GATHER, 0, 0, 0, 93.0, 1},
    {{Variant::WG_BF16_128x128, 128, 128, "wg_bf16_128x128"}, DType::BF16, WgKind::GATHER, 0, 0, 0, 190.0, 1},
    {{Variant::WG_BF16_64x64, 64, 64, "wg_bf16_64x64"}, DType::BF16, WgKind::GATHER, 0, 0, 0, 75.0, 1},
    {{Variant::WGH_F32_3x3_W16, 64, 64, "wgh_f32_3x3_64x64"}, DType::F32, WgKind::HALO, 3, 3, 16, 21.5, 1},
    {{Variant::WGH_F32_5x5_W24, 64, 64, "wgh_f32_5x5_w24_64x64"}, DType::F32, WgKind::HALO, 5, 5, 24, 22, 1},
    {{Variant::WGH_F32_5x5_W36, 64, 64, "wgh_f32_5x5_w36_64x64"}, DType::F32, WgKind::HALO, 5, 5, 36, 23.7, 1},
    {{Variant::WGH_F32_3x3_W16_64x96, 64, 96, "wgh_f32_3x3_64x96"}, DType::F32, WgKind::HALO, 3, 3, 16, 29.9, 1},
    {{Variant::WGH_F32X16_3x3_W16, 64, 64, "wgh_f32x16_3x3_64x64"}, DType::F32, WgKind::HALO, 3, 3, 16, 21.6, 1},
    {{Variant::WGH_F32X16_5x5_W24, 64, 64, "wgh_f32x16_5x5_w24_64x64"}, DType::F32, WgKind::HALO, 5, 5, 24, 22.4, 1},
    {{Variant::WGH_F64_3x3_W16, 64, 64, "wgh_f64_3x3_64x64"}, DType::F64, WgKind::HALO, 3, 3, 16, 52.0, 1},
    {{Variant::WGH_F32_3x3_Q12_64x96, 64, 96, "wgh_f32_3x3_q12_64x96"}, DType::F32, WgKind::HALO, 3, 3, 16, 25.1, 1, 12},
    {{Variant::WGH_F32_3x3_Q13, 64, 64, "wgh_f32_3x3_q13_64x64"}, DType::F32, WgKind::HALO, 3, 3, 16, 18, 1, 13},
    {{Variant::WGH_F32X16_5x5_Q20, 64, 64, "wgh_f32x16_5x5_q20_64x64"}, DType::F32, WgKind::HALO, 5, 5, 24, 19, 1, 20},
    {{Variant::WGH_F32X16_5x5_Q27, 64, 64, "wgh_f32x16_5x5_q27_64x64"}, DType::F32, WgKind::HALO, 5, 5, 32, 20.2, 1, 27},
    {{Variant::WGH_F32X16_5x5_Q20_64x48, 64, 48, "wgh_f32x16_5x5_q20_64x48"}, DType::F32, WgKind::HALO, 5, 5, 24, 16.8, 1, 20, 1},
    {{Variant::WGH_F32X16_5x5_Q27_64x48, 64, 48, "wgh_f32x16_5x5_q27_64x48"}, DType::F32, WgKind::HALO, 5, 5, 40, 18.6, 1, 27},
    // four groups of waves per tile (16 waves a CU, latency hidden within the
    // tile; measured on MI355X: AlexNet conv3/conv5 616 -> 576 us, conv4 952 -> 834)
    {{Variant::WGH_F32_3x3_Q13_KS4, 64, 64, "wgh_f32_3x3_q13_64x64_ks4"}, DType::F32, WgKind::HALO, 3, 3, 16, 19.2, 1, 13},
    {{Variant::WGH_F32_3x3_W16_64x96_KS4, 64, 96, "wgh_f32_3x3_64x96_ks4"}, DType::F32, WgKind::HALO, 3, 3, 16, 29.7, 1},
    {{Variant::WGH_F32_3x3_Q12_64x96_KS4, 64, 96, "wgh_f32_3x3_q12_64x96_ks4"}, DType::F32, WgKind::HALO, 3, 3, 16, 26.2, 1, 12},
    {{Variant::WGH_F32X16_5x5_Q20_64x48_KS4, 64, 48, "wgh_f32x16_5x5_q20_64x48_ks4"}, DType::F32, WgKind::HALO, 5, 5, 24, 17.6, 1, 20},
    {{Variant::WGH_F32X16_5x5_Q27_64x48_KS4, 64, 48, "wgh_f32x16_5x5_q27_64x48_ks4"}, DType::F32, WgKind::HALO, 5, 5, 32, 20.2, 1, 27},
    // r = 0: the (channel, filter row) pairs of the tile's columns staged, any
    // filter height and row stride (speech layer 2: 21 x 11 at stride (2, 1))
    {{Variant::WGH_F32X16_PAIRS_S11_32x32, 32, 32, "wgh_f32x16_pairs_s11_32x32"}, DType::F32, WgKind::HALO, 0, 11, 368, 7.4, 1},
    {{Variant::WGH_F32X16_PAIRS_S11_32x32_KS4, 32, 32, "wgh_f32x16_pairs_s11_32x32_ks4"}, DType::F32, WgKind::HALO, 0, 11, 384, 8.0, 1},
    // 32 x 64: half the tiles, so that a two-part split fits one round (speech
    // L2: 116 tiles, 4232 us in one part, 2135 at k = 1; 231 of 32 x 32: 2877)
    {{Variant::WGH_F32X16_PAIRS_S11_32x64, 32, 64, "wgh_f32x16_pairs_s11_32x64"}, DType::F32, WgKind::HALO, 0, 11, 368, 9.2, 1},
    // fp64: four wave groups (AlexNet-shape conv3 / conv5 560 -> 519 us); 64x96
    // tiles where 64x64 would take a second round (conv4: 324 -> 216 tiles, 1110 -> 765 us)
    {{Variant::WGH_F64_3x3_W16_KS4, 64, 64, "wgh_f64_3x3_64x64_ks4"}, DType::F64, WgKind::HALO, 3, 3, 16, 48.1, 1},
    {{Variant::WGH_F64_3x3_W16_64x96, 64, 96, "wgh_f64_3x3_64x96"}, DType::F64, WgKind::HALO, 3, 3, 16, 71.7, 1},
    // bf16 x and dy widened to fp32 as they are staged, fp32 MFMA (the
    // fp32 forms' instances; times from AlexNet conv3 at N = 64 in one part)
    {{Variant::WGH_BF16_3x3_W16, 64, 64, "wgh_bf16_3x3_64x64"}, DType::BF16, WgKind::HALO, 3, 3, 16, 29.5, 1},
    {{Variant::WGH_BF16_3x3_Q13, 64, 64, "wgh_bf16_3x3_q13_64x64"}, DType::BF16, WgKind::HALO, 3, 3, 16, 32.8, 1, 13},
    {{Variant::WGH_BF16_3x3_W16_64x96_KS4, 64, 96, "wgh_bf16_3x3_64x96_ks4"}, DType::BF16, WgKind::HALO, 3, 3, 16, 31.3, 1},
    {{Variant::WGS_F32_32x32, 32, 32, "wgs_f32_32x32"}, DType::F32, WgKind::SPLIT, 0, 0, 0, 12.5, 1},
    {{Variant::WGS_F32_16x16, 16, 16, "wgs_f32_16x16"}, DType::F32, WgKind::SPLIT, 0, 0, 0, 7.1, 2},
    {{Variant::WGS_F32_8x16, 8, 16, "wgs_f32_8x16"}, DType::F32, WgKind::SPLIT, 0, 0, 0, 4.5, 2},
    {{Variant::WGS_F64_32x32, 32, 32, "wgs_f64_32x32"}, DType::F64, WgKind::SPLIT, 0, 0, 0, 28.0, 1},
    {{Variant::WGS_F64_16x16, 16, 16, "wgs_f64_16x16"}, DType::F64, WgKind::SPLIT, 0, 0, 0, 5.7, 1},
    {{Variant::WGS_BF16_32x32, 32, 32, "wgs_bf16_32x32"}, DType::BF16, WgKind::SPLIT, 0, 0, 0, 15.8, 2},
    // bf16 with channels-last x and dy: 64 filters x 64 channels of one tap,
    // operands transposed on their way out of LDS
    {{Variant::WGC_BF16_64x64, 64, 64, "wgc_bf16_64x64"}, DType::BF16, WgKind::CL, 0, 0, 0, 15.0, 2},
    {{Variant::WGC_BF16_64x64_KS3, 64, 64, "wgc_bf16_64x64_ks3"}, DType::BF16, WgKind::CL, 0, 0, 0, 6.0, 1},
    {{Variant::WGC_BF16_64x64_KS2, 64, 64, "wgc_bf16_64x64_ks2"}, DType::BF16, WgKind::CL, 0, 0, 0, 8.0, 2},
    // first layers on the vector ALU: tiles of KT filters x S taps of one
    // (c, r); ns here is the time of one output row per tile, the cost that
    // time over Q (measured on MI355X: speech L1 770 us, Overfeat L1 855 us)
    {{Variant::WGR_F32_S11_V2, 3, 11, "wgr_f32_s11_v2"}, DType::F32, WgKind::ROWS, 0, 0, 0, 298.0, 2},
    {{Variant::WGR_F32_S11_V4, 7, 11, "wgr_f32_s11_v4"}, DType::F32, WgKind::ROWS, 0, 0, 0, 119.0, 2},
};
// the split kernel's loads run along the positions: with x or dy strided
// along q (channels-last) they gather (measured 2.6x slower for fp64,
// 4.1-4.6x for bf16, whose 2-byte gathers use less of each cache line)
double split_strided_penalty(DType dt) { return dt == DType::BF16 ? 4.5 : 2.6; }

bool is_wgh(Variant v)
{
    return v == Variant::WGH_F32_3x3_W16 || v == Variant::WGH_F32_5x5_W24 || v == Variant::WGH_F32_5x5_W36 ||
           v == Variant::WGH_F32_3x3_W16_64x96 || v == Variant::WGH_F32X16_3x3_W16 ||
           v == Variant::WGH_F32X16_5x5_W24 || v == Variant::WGH_F64_3x3_W16 || v == Variant::WGH_F32_3x3_Q12_64x96 ||
           v == Variant::WGH_F32_3x3_Q13 || v == Variant::WGH_F32X16_5x5_Q20 ||
           v == Variant::WGH_F32X16_5x5_Q27 || v == Variant::WGH_F32X16_5x5_Q20_64x48 ||
           v == Variant::WGH_F32X16_5x5_Q27_64x48 || v == Variant::WGH_F32_3x3_Q13_KS4 ||
           v == Variant::WGH_F32_3x3_W16_64x96_KS4 || v == Variant::WGH_F32_3x3_Q12_64x96_KS4 ||
           v == Variant::WGH_F32X16_5x5_Q20_64x48_KS4 || v == Variant::WGH_F32X16_5x5_Q27_64x48_KS4 ||
           v == Variant::WGH_F32X16_PAIRS_S11_32x32 || v == Variant::WGH_F32X16_PAIRS_S11_32x32_KS4 ||
           v == Variant::WGH_F32X16_PAIRS_S11_32x64 ||
           v == Variant::WGH_F64_3x3_W16_KS4 || v == Variant::WGH_F64_3x3_W16_64x96 ||
           v == Variant::WGH_BF16_3x3_W16 || v == Variant::WGH_BF16_3x3_Q13 || v == Variant::WGH_BF16_3x3_W16_64x96_KS4;
}

bool is_wgr(Variant v) { return v == Variant::WGR_F32_S11_V2 || v == Variant::WGR_F32_S11_V4; }

bool is_wgc(Variant v)
{
    return v == Variant::WGC_BF16_64x64 || v == Variant::WGC_BF16_64x64_KS2 || v == Variant::WGC_BF16_64x64_KS3;
}

bool is_wgs(Variant v)
{
    return v == Variant::WGS_F32_32x32 || v == Variant::WGS_F32_16x16 || v == Variant::WGS_F32_8x16 ||
           v == Variant::WGS_F64_32x32 ||
           v == Variant::WGS_F64_16x16 || v == Variant::WGS_BF16_32x32;
}

// batch-reduce GEMM (brgemm.hip): shared-LDS tiles for large products
const Candidate kBrF32[] = {
    {Variant::BR_F32_128x128, 128, 128, "br_f32_128x128"},
    {Variant::BR_F32_64x64, 64, 64, "br_f32_64x64"},
    {Variant::BR_F32_32x64, 32, 64, "br_f32_32x64"},
};
const Candidate kBrF64[] = {
    {Variant::BR_F64_64x64, 64, 64, "br_f64_64x64"},
    {Variant::BR_F64_32x64, 32, 64, "br_f64_32x64"},
};
const Candidate kBrBF16[] = {
    {Variant::BR_BF16_128x128, 128, 128, "br_bf16_128x128"},
    {Variant::BR_BF16_64x64, 64, 64, "br_bf16_64x64"},
    {Variant::BR_BF16_32x128, 32, 128, "br_bf16_32x128"},
};
// ... and the wave-split kernel for skinny ones (contiguous k only), largest tile first
const Candidate kWsF32[] = {
    {Variant::WS_F32_64x64, 64, 64, "ws_f32_64x64"},
    {Variant::WS_F32_32x64, 32, 64, "ws_f32_32x64"},
    {Variant::WS_F32_16x32, 16, 32, "ws_f32_16x32"},
};
const Candidate kWsF64[] = {
    {Variant::WS_F64_32x64, 32, 64, "ws_f64_32x64"},
    {Variant::WS_F64_16x32, 16, 32, "ws_f64_16x32"},
};
const Candidate kWsBF16[] = {
    {Variant::WS_BF16_32x64, 32, 64, "ws_bf16_32x64"},
    {Variant::WS_BF16_16x32, 16, 32, "ws_bf16_16x32"},
};

// Tap-batched halo kernels (conv_fwd_halo.hip): fixed R x S, CB channels per
// chunk, padded input width <= WP, per-tile slot span <= SL.
struct HaloCandidate {
    Candidate c;
    DType dt;
    int r, s, cb, wp, sl;
    double eff;   // relative per-tile efficiency, measured on MI355X (128x128 = 1)
    int ks;       // 2: a 512-thread workgroup whose halves split one tile's reduction
};

const HaloCandidate kHalo[] = {
    {{Variant::HALO_F32_3x3_128x128, 128, 128, "halo_f32_3x3_128x128"}, DType::F32, 3, 3, 4, 16, 16, 1.0, 1},
    {{Variant::HALO_F32_3x3_128x64, 128, 64, "halo_f32_3x3_128x64"}, DType::F32, 3, 3, 4, 16, 16, 0.93, 1},
    {{Variant::HALO_F32_3x3_64x128, 64, 128, "halo_f32_3x3_64x128"}, DType::F32, 3, 3, 4, 16, 16, 0.8, 1},
    {{Variant::HALO_F32_3x3_96x128, 96, 128, "halo_f32_3x3_96x128"}, DType::F32, 3, 3, 4, 16, 16, 0.97, 1},
    {{Variant::HALO_F32_5x5_128x128, 128, 128, "halo_f32_5x5_128x128"}, DType::F32, 5, 5, 4, 32, 16, 0.93, 1},
    {{Variant::HALO_F32_5x5_128x128_C2, 128, 128, "halo_f32_5x5_128x128_c2"}, DType::F32, 5, 5, 2, 32, 16, 1.0, 1},
    {{Variant::HALO_F32x16_3x3_176x128, 176, 128, "halo_f32x16_3x3_176x128"}, DType::F32, 3, 3, 4, 16, 16, 0.9, 1},
    {{Variant::HALO_F32x16_3x3_144x128, 144, 128, "halo_f32x16_3x3_144x128"}, DType::F32, 3, 3, 4, 16, 16, 0.95, 1},
    {{Variant::HALO_F32x16_5x5_128x96, 128, 96, "halo_f32x16_5x5_128x96"}, DType::F32, 5, 5, 4, 32, 16, 0.85, 1},
    {{Variant::HALO_F32_5x5_128x96_C2, 128, 96, "halo_f32_5x5_128x96_c2"}, DType::F32, 5, 5, 2, 32, 16, 0.98, 1},
    {{Variant::HALO_F32x16_5x5_208x64, 208, 64, "halo_f32x16_5x5_208x64"}, DType::F32, 5, 5, 4, 32, 24, 0.9, 1},
    {{Variant::HALO_F32x16_3x3_176x128_KS2, 176, 128, "halo_f32x16_3x3_176x128_ks2"}, DType::F32, 3, 3, 4, 16, 16, 0.95, 2},
    {{Variant::HALO_F32_3x3_128x128_KS2, 128, 128, "halo_f32_3x3_128x128_ks2"}, DType::F32, 3, 3, 4, 16, 16, 0.9, 2},
    {{Variant::HALO_F64_3x3_128x128, 128, 128, "halo_f64_3x3_128x128"}, DType::F64, 3, 3, 4, 16, 16, 1.0, 1},
    {{Variant::HALO_F64_3x3_64x64, 64, 64, "halo_f64_3x3_64x64"}, DType::F64, 3, 3, 4, 16, 16, 0.8, 1},
    // (1.03: ahead of 128x128 on one tile per CU, measured 1.11-1.13x; behind
    // 64x64 on conv5's 170 tiles, measured 0.92x)
    {{Variant::HALO_F64_3x3_128x64, 128, 64, "halo_f64_3x3_128x64"}, DType::F64, 3, 3, 4, 16, 16, 1.03, 1},
    // one 13x13 output image (169 of 176 rows) x 64 filters, two halves per tile:
    // K = 256 at N = 64 gives exactly one tile per CU
    {{Variant::HALO_F64_3x3_176x64_KS2, 176, 64, "halo_f64_3x3_176x64_ks2"}, DType::F64, 3, 3, 4, 16, 16, 0.95, 2},
    {{Variant::HALO_BF16_3x3_128x128, 128, 128, "halo_bf16_3x3_128x128"}, DType::BF16, 3, 3, 16, 16, 16, 1.0, 1},
    {{Variant::HALO_BF16_3x3_128x64, 128, 64, "halo_bf16_3x3_128x64"}, DType::BF16, 3, 3, 16, 16, 16, 0.8, 1},
    {{Variant::HALO_BF16_3x3_192x128, 192, 128, "halo_bf16_3x3_192x128"}, DType::BF16, 3, 3, 16, 16, 16, 1.0, 1},
};

// MIC_TILE_ORDER=reverse (environment) makes every tiled kernel run its
// output tiles in the opposite order; the result must not change (the tests
// compare both orders bit for bit).
int tile_order_reversed()
{
    const char* e = getenv("MIC_TILE_ORDER");
    return e && strcmp(e, "reverse") == 0 ? 1 : 0;
}

struct Plan {
    mic_status status;
    DType dt;
    ConvParams p;
    Candidate cand;
    bool bvec;
    bool tap;          // gather kernel: reduction in channel blocks per filter tap
    int split_k;       // filter-gradient halo kernel: reduction in two parts, k : 1 (0: one part)
    char name[64];     // variant name as reported and as MIC_FORCE_VARIANT spells it
};

// Reduction chunk of the gather kernel (elements of kappa).
int gather_tk(DType dt) { return dt == DType::BF16 ? 32 : 16; }

// Tap order pays when whole channel blocks fill the chunks: at least one
// block, and at most 1/8 of the chunk slots left empty by a ragged C.
// Measured on MI355X for fp32 (speech layer 2: 45.6 -> 75.0 TFLOP/s); for
// bf16 its 2-byte filter gathers cost more than the flat decode saves.
bool prefer_tap(DType dt, int C)
{
    if (dt != DType::F32) return false;
    const int tk = gather_tk(dt);
    const int padded = (C + tk - 1) / tk * tk;
    return C >= tk && padded * 8 <= C * 9;
}

int max_tile_slots(const ConvParams& p, int step);

// Cheapest way to run halo instance hc on p: tiles of hc.c.tm consecutive
// output rows, or one output image per tile (P*Q <= tm).  Returns false if
// neither fits; else the cost (busiest CU's tile count x tile area /
// efficiency) and the rows per tile.
bool halo_cost(const HaloCandidate& hc, const ConvParams& p, int Wp, int num_cu, double* cost, int* step)
{
    if (Wp > hc.wp) return false;
    const int pq = p.P * p.Q;
    const int steps[2] = {hc.c.tm, pq <= hc.c.tm ? pq : 0};
    bool ok = false;
    for (int st : steps) {
        if (st <= 0 || max_tile_slots(p, st) > hc.sl) continue;
        const int64_t tiles = (int64_t)((p.M + st - 1) / st) * ((p.K + hc.c.tn - 1) / hc.c.tn);
        const int64_t rounds = (tiles + num_cu - 1) / num_cu;
        // a split workgroup fills a CU: only worth it with at most one tile per CU;
        // a plain one alone on its CU has no second workgroup to hide latency
        if (hc.ks == 2 && tiles > num_cu) continue;
        const double occ = (hc.ks == 1 && tiles <= num_cu) ? 0.92 : 1.0;
        const double c = (double)rounds * hc.c.tm * hc.c.tn / (hc.eff * occ);
        if (!ok || c < *cost) {
            *cost = c;
            *step = st;
            ok = true;
        }
    }
    return ok;
}

void candidates(DType dt, const Candidate** list, int* count)
{
    switch (dt) {
    case DType::F32: *list = kF32; *count = (int)(sizeof(kF32) / sizeof(kF32[0])); return;
    case DType::F64: *list = kF64; *count = (int)(sizeof(kF64) / sizeof(kF64[0])); return;
    case DType::BF16: *list = kBF16; *count = (int)(sizeof(kBF16) / sizeof(kBF16[0])); return;
    }
    *list = nullptr;
    *count = 0;
}

// Analytical tile choice: the busiest compute unit runs ceil(tiles / CUs)
// tiles; a tile costs its MFMA work divided by a reuse factor that drops
// for thin tiles (fewer MACs per loaded element).
Candidate choose_tile(DType dt, int M, int K, int num_cu)
{
    const Candidate* list;
    int count;
    candidates(dt, &list, &count);
    double best = 0;
    int best_i = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t tiles = (int64_t)((M + list[i].tm - 1) / list[i].tm) * ((K + list[i].tn - 1) / list[i].tn);
        const int64_t rounds = (tiles + num_cu - 1) / num_cu;
        const double reuse = (double)list[i].tm * list[i].tn / (list[i].tm + list[i].tn);
        const double eff = reuse >= 48.0 ? 1.0 : reuse / 48.0;
        const double cost = (double)rounds * list[i].tm * list[i].tn / eff;
        if (i == 0 || cost < best) {
            best = cost;
            best_i = i;
        }
    }
    return list[best_i];
}

bool is_halo(Variant v)
{
    for (const HaloCandidate& hc : kHalo)
        if (hc.c.v == v) return true;
    return false;
}

// Largest number of padded input rows ("slots") one tile of `step`
// consecutive output rows touches: rows n*Hp + p*u .. of its first and last
// output row.
int max_tile_slots(const ConvParams& p, int step)
{
    int worst = 0;
    for (int64_t m0 = 0; m0 < p.M; m0 += step) {
        const int64_t m1 = (m0 + step < p.M ? m0 + step : p.M) - 1;
        const int64_t pq = (int64_t)p.P * p.Q;
        const int64_t v0 = (m0 / pq) * p.Hp + ((m0 % pq) / p.Q) * p.u;
        const int64_t v1 = (m1 / pq) * p.Hp + ((m1 % pq) / p.Q) * p.u;
        const int64_t slots = v1 + p.R - v0;
        if (slots > worst) worst = (int)(slots > INT32_MAX ? INT32_MAX : slots);
    }
    return worst;
}

bool halo_eligible(const HaloCandidate& h, DType dt, const ConvParams& p, const void* w, bool check_ptr,
                   bool dgrad = false)
{
    if (h.dt != dt || h.r != p.R || h.s != p.S) return false;
    {
        // the halo kernels' buffer descriptors: x (dy) and the filters under 2^31 bytes
        const int64_t es = dt == DType::F64 ? 8 : dt == DType::BF16 ? 2 : 4;
        const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + miconv::blk_off(p.div_xcb, p.sxcb, p.sxc, p.C - 1) +
                                (int64_t)(p.H - 1) * p.sxh + (int64_t)(p.W - 1) * p.sxw + 1;
        if (es * x_elems >= (int64_t(1) << 31) || es * p.C * (int64_t)p.K * p.R * p.S >= (int64_t(1) << 31))
            return false;
    }
    if (p.C % h.cb != 0) return false;
    // channel-blocked x: a chunk of h.cb channels must lie in one block
    if (p.div_xcb.d != miconv::kOneBlock && p.div_xcb.d % h.cb != 0) return false;
    // scalar filter loads: no alignment needed.  bf16 with packed KCRS
    // filters: 64-filter tiles, 128-filter ones where dy is read 2 bytes at a
    // time (channels not innermost; with 16-byte dy loads they run slower)
    if (dgrad)
        return dt != DType::BF16 ||
               (p.wkb == 0 && (h.c.v == Variant::HALO_BF16_3x3_128x64 ||
                               (h.c.v == Variant::HALO_BF16_3x3_128x128 && p.sxc != 1)));
    if (p.wkb > 0) {
        // blocked filters: 16-byte loads of kb-contiguous filters (4 fp32, 2 fp64
        // or 8 bf16 filters; bf16 transposes 8 x 8 blocks, a chunk's 16 channels in one block)
        const int vk = dt == DType::F64 ? 2 : dt == DType::BF16 ? 8 : 4;
        if (p.wcb % h.cb != 0 || p.wkb % vk != 0) return false;
    }
    if (check_ptr && (uintptr_t)w % 16 != 0) return false;
    return true;
}

Plan make_plan(const mic_handle_st* h, const mic_tensor_desc_st* xd, const void* x,
               const mic_filter_desc_st* wd, const void* w, const mic_conv_desc_st* cd,
               const mic_tensor_desc_st* yd, const void* y, double alpha, double beta,
               bool need_pointers)
{
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.status = MIC_STATUS_BAD_PARAM;
    if (!xd || !wd || !cd || !yd) return pl;
    if (!xd->set || !wd->set || !cd->set || !yd->set) return pl;
    if (need_pointers && (!x || !w || !y)) return pl;
    int n, k, P, Q;
    mic_status st = output_dims(cd, xd, wd, &n, &k, &P, &Q);
    if (st != MIC_STATUS_SUCCESS) {
        pl.status = st;
        return pl;
    }
    if (yd->n != n || yd->c != k || yd->h != P || yd->w != Q) return pl;

    // dtype combination
    if (xd->dtype == MIC_DTYPE_F32 && wd->dtype == MIC_DTYPE_F32 && yd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::F32;
    else if (xd->dtype == MIC_DTYPE_F64 && wd->dtype == MIC_DTYPE_F64 && yd->dtype == MIC_DTYPE_F64)
        pl.dt = DType::F64;
    else if (xd->dtype == MIC_DTYPE_BF16 && wd->dtype == MIC_DTYPE_BF16 && yd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::BF16;
    else {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }

    // size limits: 32-bit element offsets with headroom
    const int64_t M = (int64_t)n * P * Q;
    const int64_t Kred = (int64_t)wd->c * wd->r * wd->s;
    const int64_t wsize = (int64_t)wd->k * Kred;
    if (extent(*xd) >= kMaxOffset || extent(*yd) >= kMaxOffset || wsize >= kMaxOffset ||
        M >= kMaxOffset || Kred >= kMaxOffset || xd->sn >= kMaxOffset || xd->sc >= kMaxOffset ||
        xd->sh >= kMaxOffset || xd->sw >= kMaxOffset || yd->sn >= kMaxOffset ||
        yd->sc >= kMaxOffset || yd->sh >= kMaxOffset || yd->sw >= kMaxOffset) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    // element alignment of the data pointers
    if (need_pointers) {
        const size_t ie = dtype_size(xd->dtype), oe = dtype_size(yd->dtype);
        if ((uintptr_t)x % ie || (uintptr_t)w % ie || (uintptr_t)y % oe) return pl;
    }

    ConvParams& p = pl.p;
    p.x = x;
    p.w = w;
    p.y = const_cast<void*>(y);
    p.N = n;
    p.C = xd->c;
    p.H = xd->h;
    p.W = xd->w;
    p.K = k;
    p.R = wd->r;
    p.S = wd->s;
    p.P = P;
    p.Q = Q;
    p.u = cd->u;
    p.v = cd->v;
    p.pad_top = cd->pad_top;
    p.pad_left = cd->pad_left;
    p.sxn = (int)xd->sn;
    p.sxc = (int)xd->sc;
    p.sxh = (int)xd->sh;
    p.sxw = (int)xd->sw;
    p.syn = (int)yd->sn;
    p.syk = (int)yd->sc;
    p.syp = (int)yd->sh;
    p.syq = (int)yd->sw;
    p.M = (int)M;
    p.Kred = (int)Kred;
    p.div_pq = FastDiv((uint32_t)(P * Q));
    p.div_q = FastDiv((uint32_t)Q);
    p.div_rs = FastDiv((uint32_t)(wd->r * wd->s));
    p.div_s = FastDiv((uint32_t)wd->s);
    p.Hp = xd->h + cd->pad_top + cd->pad_bottom;
    p.div_hp = FastDiv((uint32_t)p.Hp);
    p.div_u = FastDiv((uint32_t)p.u);
    p.div_v = FastDiv((uint32_t)p.v);
    set_blocks(p, xd, yd, wd);
    p.alpha = alpha;
    p.beta = beta;
    const int Wp = xd->w + cd->pad_left + cd->pad_right;

    const int num_cu = h ? h->num_cu : kDefaultCUs;
    pl.cand = choose_tile(pl.dt, p.M, p.K, num_cu);
    // prefer a tap-batched halo kernel where one fits: the busiest compute unit
    // runs ceil(tiles / CUs) tiles, each costing its area over its efficiency
    {
        double best = 0;
        bool found = false;
        for (const HaloCandidate& hc : kHalo) {
            double cost;
            int step;
            if (!halo_eligible(hc, pl.dt, p, w, need_pointers)) continue;
            if (!halo_cost(hc, p, Wp, num_cu, &cost, &step)) continue;
            if (!found || cost < best) {
                best = cost;
                pl.cand = hc.c;
                p.m_step = step;
                found = true;
            }
        }
    }

    // no halo instance: tall filter banks with few filters stream the
    // reduction by filter row (speech layer 2: 2.9 ms through the gather kernel)
    // the row-streamed kernel reads channel-blocked x when a block holds its
    // 4-channel chunks (one 16-byte load per chunk column: x 16-byte aligned),
    // blocked filters tap by tap, blocked y in the epilogue
    const bool rows_blocks_ok =
        !blocked(xd) || (xd->cb % 4 == 0 && (!need_pointers || (uintptr_t)x % 16 == 0));
    const bool rows_ok = pl.dt == DType::F32 && rows_blocks_ok && miconv::rows_fits(kRowsF32.v, p);
    // ... and onto 1-4 input channels with adjacent taps paired (speech
    // layer 1: two output-row slots; Overfeat layer 1: six)
    // ... and the one-channel forms blocked y (their x and filter loaders read plain layouts)
    const bool rows1_layout_ok = !blocked(xd) && !blocked(wd);
    const bool rows1_ok = pl.dt == DType::F32 && rows1_layout_ok && miconv::rows_fits(kRows1F32.v, p);
    const bool rows1n6_ok = pl.dt == DType::F32 && rows1_layout_ok && miconv::rows_fits(kRows1N6F32.v, p);
    if (!is_halo(pl.cand.v) && rows_ok) pl.cand = kRowsF32;
    if (!is_halo(pl.cand.v) && rows1n6_ok) pl.cand = kRows1N6F32;
    if (!is_halo(pl.cand.v) && rows1_ok) pl.cand = kRows1F32;

    pl.tap = prefer_tap(pl.dt, p.C);
    bool forced_gather = false;
    // MIC_FORCE_VARIANT=<name> pins a variant (tests walk every variant with it)
    if (const char* force = getenv("MIC_FORCE_VARIANT")) {
        if (force[0]) {
            bool halo_forced = false;
            for (const HaloCandidate& hc : kHalo) {
                if (strcmp(force, hc.c.name) != 0) continue;
                double cost;
                int step;
                if (!halo_eligible(hc, pl.dt, p, w, need_pointers) ||
                    !halo_cost(hc, p, Wp, num_cu, &cost, &step)) {
                    pl.status = MIC_STATUS_NOT_SUPPORTED;
                    return pl;
                }
                pl.cand = hc.c;
                p.m_step = step;
                halo_forced = true;
            }
            if (!halo_forced) p.m_step = 0;
            if (halo_forced) {
            } else if (strcmp(force, kDirect.name) == 0) {
                pl.cand = kDirect;
            } else if (strcmp(force, kRowsF32.name) == 0 || strcmp(force, kRows1F32.name) == 0 ||
                       strcmp(force, kRows1N6F32.name) == 0) {
                const Candidate& c = strcmp(force, kRowsF32.name) == 0    ? kRowsF32
                                     : strcmp(force, kRows1F32.name) == 0 ? kRows1F32
                                                                          : kRows1N6F32;
                const bool ok = c.v == kRowsF32.v ? rows_ok : c.v == kRows1F32.v ? rows1_ok : rows1n6_ok;
                if (!ok) {
                    pl.status = MIC_STATUS_NOT_SUPPORTED;
                    return pl;
                }
                pl.cand = c;
            } else {
                const Candidate* list;
                int count;
                candidates(pl.dt, &list, &count);
                int found = -1;
                bool tap = false;
                for (int i = 0; i < count; ++i) {
                    const size_t n = strlen(list[i].name);
                    if (strcmp(force, list[i].name) == 0) {
                        found = i;
                        tap = false;
                    } else if (strncmp(force, list[i].name, n) == 0 && strcmp(force + n, "_tap") == 0) {
                        found = i;
                        tap = true;
                    }
                }
                if (found < 0) {
                    pl.status = MIC_STATUS_NOT_SUPPORTED;
                    return pl;
                }
                pl.cand = list[found];
                pl.tap = tap;
                forced_gather = true;
            }
        }
    }
    const size_t ie = dtype_size(xd->dtype);
    pl.bvec = ((Kred * (int64_t)ie) % 16 == 0) && ((uintptr_t)w % 16 == 0) && !blocked(wd);
    const bool gather = pl.cand.v != Variant::DIRECT && pl.cand.v != kRowsF32.v && pl.cand.v != kRows1F32.v &&
                        pl.cand.v != kRows1N6F32.v && !is_halo(pl.cand.v);
    if (!gather) pl.tap = false;
    if (gather && (blocked(xd) || blocked(wd))) {
        // Tap order reads a chunk of TK channels at one tap: with blocked x or
        // filters the chunk must lie in one block.  Blocked filters need tap
        // order; blocked x alone can also go through the flat order.
        const int tk = gather_tk(pl.dt);
        const bool tap_ok = (!blocked(xd) || xd->cb % tk == 0) && (!blocked(wd) || wd->cb % tk == 0);
        if (forced_gather && pl.tap && !tap_ok) {
            pl.status = MIC_STATUS_NOT_SUPPORTED;
            return pl;
        }
        if (blocked(wd)) {
            if (forced_gather && !pl.tap) {
                pl.status = MIC_STATUS_NOT_SUPPORTED;
                return pl;
            }
            if (tap_ok)
                pl.tap = true;
            else
                pl.cand = kDirect;       // any blocking, one output per thread
        } else if (!tap_ok) {
            pl.tap = false;
        }
        if (pl.cand.v == Variant::DIRECT) pl.tap = false;
    }
    snprintf(pl.name, sizeof(pl.name), "%s%s", pl.cand.name, pl.tap ? "_tap" : "");
    pl.status = MIC_STATUS_SUCCESS;
    return pl;
}

// ---------------------------------------------------------------- data gradient

// dx <- alpha * dgrad(dy, w) + beta * dx.  The forward geometry is (dx, w,
// conv); dy must have the forward output's dims.  Stride-1 problems of the
// halo shapes (fp32, fp64) run as the forward pass of dy with the filter
// transposed and flipped (conv_fwd_halo.hip, DG instances); strided ones as
// a stride-1 GEMM over dy onto dx's stride phases (conv_bwd_data_subpixel.hip)
// or one of the kernels below; the rest the gather kernel in data-gradient
// mode or the direct kernel (conv_bwd_data.hip).
Plan make_dgrad_plan(const mic_handle_st* h, const mic_tensor_desc_st* dyd, const void* dy,
                     const mic_filter_desc_st* wd, const void* w, const mic_conv_desc_st* cd,
                     const mic_tensor_desc_st* dxd, const void* dx, double alpha, double beta,
                     bool need_pointers)
{
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.status = MIC_STATUS_BAD_PARAM;
    if (!dyd || !wd || !cd || !dxd) return pl;
    if (!dyd->set || !wd->set || !cd->set || !dxd->set) return pl;
    if (blocked(dyd) || blocked(wd) || blocked(dxd)) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;     // channel-blocked layouts: forward pass only
        return pl;
    }
    if (need_pointers && (!dy || !w || !dx)) return pl;
    int n, k, P, Q;
    mic_status st = output_dims(cd, dxd, wd, &n, &k, &P, &Q);
    if (st != MIC_STATUS_SUCCESS) {
        pl.status = st;
        return pl;
    }
    if (dyd->n != n || dyd->c != k || dyd->h != P || dyd->w != Q) return pl;

    if (dyd->dtype == MIC_DTYPE_F32 && wd->dtype == MIC_DTYPE_F32 && dxd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::F32;
    else if (dyd->dtype == MIC_DTYPE_F64 && wd->dtype == MIC_DTYPE_F64 && dxd->dtype == MIC_DTYPE_F64)
        pl.dt = DType::F64;
    else if (dyd->dtype == MIC_DTYPE_BF16 && wd->dtype == MIC_DTYPE_BF16 && dxd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::BF16;
    else {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }

    const int64_t M = (int64_t)dxd->n * dxd->h * dxd->w;
    const int64_t RS = (int64_t)wd->r * wd->s;
    const int64_t wsize = (int64_t)wd->k * wd->c * RS;
    if (extent(*dyd) >= kMaxOffset || extent(*dxd) >= kMaxOffset || wsize >= kMaxOffset ||
        M >= kMaxOffset || (int64_t)wd->k * RS >= kMaxOffset || dyd->sn >= kMaxOffset ||
        dyd->sc >= kMaxOffset || dyd->sh >= kMaxOffset || dyd->sw >= kMaxOffset ||
        dxd->sn >= kMaxOffset || dxd->sc >= kMaxOffset || dxd->sh >= kMaxOffset || dxd->sw >= kMaxOffset) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    if (need_pointers) {
        const size_t ie = dtype_size(dyd->dtype), oe = dtype_size(dxd->dtype);
        if ((uintptr_t)dy % ie || (uintptr_t)w % ie || (uintptr_t)dx % oe) return pl;
    }

    const int R = wd->r, S = wd->s, C = dxd->c, H = dxd->h, W = dxd->w;
    const int pt = cd->pad_top, pl_ = cd->pad_left;
    ConvParams& p = pl.p;
    set_blocks(p, nullptr, nullptr, nullptr);
    p.x = dy;
    p.w = w;
    p.y = const_cast<void*>(dx);
    p.sxn = (int)dyd->sn;
    p.sxc = (int)dyd->sc;
    p.sxh = (int)dyd->sh;
    p.sxw = (int)dyd->sw;
    p.syn = (int)dxd->sn;
    p.syk = (int)dxd->sc;
    p.syp = (int)dxd->sh;
    p.syq = (int)dxd->sw;
    p.N = n;
    p.R = R;
    p.S = S;
    p.M = (int)M;
    p.div_pq = FastDiv((uint32_t)(H * W));
    p.div_q = FastDiv((uint32_t)W);
    p.div_rs = FastDiv((uint32_t)RS);
    p.div_s = FastDiv((uint32_t)S);
    p.alpha = alpha;
    p.beta = beta;
    pl.cand = kDirect;
    const char* forced_dgrad_name = getenv("MIC_FORCE_DGRAD_VARIANT");
    if (forced_dgrad_name && !forced_dgrad_name[0]) forced_dgrad_name = nullptr;

    // the equivalent forward problem of a stride-1 data gradient: input dy
    // (C' = K channels, H' x W' = P x Q), K' = C filters, padding R-1-pad_top
    // on top and H-P+pad_top below (S-1-pad_left, W-Q+pad_left across), output
    // H x W
    const int pb2 = H - P + pt, pr2 = W - Q + pl_;
    const bool halo_ok = cd->u == 1 && cd->v == 1 && pt <= R - 1 && pl_ <= S - 1 && pb2 >= 0 && pr2 >= 0;
    if (halo_ok) {
        ConvParams v = p;
        v.C = k;
        v.H = P;
        v.W = Q;
        v.K = C;
        v.P = H;
        v.Q = W;
        v.u = 1;
        v.v = 1;
        v.pad_top = R - 1 - pt;
        v.pad_left = S - 1 - pl_;
        v.Hp = P + v.pad_top + pb2;
        v.div_hp = FastDiv((uint32_t)v.Hp);
        v.Kred = (int)((int64_t)k * RS);
        const int Wp = Q + v.pad_left + pr2;
        const int num_cu = h ? h->num_cu : kDefaultCUs;
        double best = 0;
        bool found = false;
        for (const HaloCandidate& hc : kHalo) {
            double cost;
            int step;
            if (forced_dgrad_name && strcmp(forced_dgrad_name, hc.c.name) != 0) continue;
            if (!halo_eligible(hc, pl.dt, v, w, need_pointers, true)) continue;
            if (!halo_cost(hc, v, Wp, num_cu, &cost, &step)) continue;
            if (!found || cost < best) {
                best = cost;
                pl.cand = hc.c;
                v.m_step = step;
                found = true;
            }
        }
        if (found) p = v;
    }
    if (pl.cand.v == Variant::DIRECT) {
        // no halo instance: the gather kernel in data-gradient mode (any
        // stride), laid out as conv_fwd_mfma.hip describes; onto fewer than 16
        // channels, where the gather kernel's tiles would be almost empty
        // (measured on MI355X: 1 channel 5.2 ms direct vs 36 ms gathered,
        // 3 channels 8 vs 53), a vector-ALU kernel in the direct layout: the
        // stride-phase kernel (conv_bwd_data_phase.hip) onto 2-4 channels with
        // at most 6 column taps per phase and dy under 1 GiB (fp32, fp64),
        // else the one-thread-per-element kernel (conv_bwd_data.hip).  Onto
        // one channel the phase kernel's dy window yields too few
        // multiply-adds per load (measured on MI355X, speech layer 1: 6.6 ms
        // against 5.2 direct; Overfeat layer 1, 3 channels: 2.1 against 8.2);
        // it runs there only when forced.
        const bool phase_ok = C <= 4 && (S + cd->v - 1) / cd->v <= 6 && pl.dt != DType::BF16 &&
                              extent(*dyd) * (int64_t)dtype_size(dyd->dtype) <= (int64_t(1) << 30);
        const bool phase = forced_dgrad_name ? strcmp(forced_dgrad_name, kDgPhase.name) == 0 && phase_ok
                                             : C >= 2 && phase_ok;
        // onto one channel (fp32): the row-staged form of the phase kernel
        // when its staged window fits (speech layer 1: 5.2 ms direct)
        bool rows_ok = false;
        if (C == 1 && pl.dt == DType::F32) {
            ConvParams q = p;
            q.C = C;
            q.H = H;
            q.W = W;
            q.R = R;
            q.S = S;
            q.u = cd->u;
            q.v = cd->v;
            rows_ok = miconv::bwd_data_rows_fits(q, nullptr);
        }
        const bool rows = forced_dgrad_name ? strcmp(forced_dgrad_name, kDgRows.name) == 0 && rows_ok : rows_ok;
        // horizontal stride 1 and an 11-wide filter onto wide rows: the
        // forward pass's row-streamed kernel per stride phase (speech layer 2:
        // 5.0 ms through the gather kernel)
        bool rows_mfma_ok = false;
        // (its buffer loads: dy and the filters under 2^31 bytes)
        if (pl.dt == DType::F32 && C >= 16 && extent(*dyd) * 4 < (int64_t(1) << 31) &&
            (int64_t)k * C * R * S * 4 < (int64_t(1) << 31)) {
            ConvParams q = p;
            q.K = k;
            q.W = W;
            q.S = S;
            q.v = cd->v;
            rows_mfma_ok = miconv::bwd_data_rows_mfma_fits(q);
        }
        const bool rows_mfma = forced_dgrad_name ? strcmp(forced_dgrad_name, kDgRowsMfma.name) == 0 && rows_mfma_ok
                                                 : rows_mfma_ok;
        // a stride above 1 with at least 32 columns (channel, row phase,
        // column phase): the stride-1 GEMM over dy onto dx's stride phases,
        // which spends no multiply-adds off the stride grid (Overfeat layer 1,
        // 3 channels at stride 4: 48 columns)
        bool subpixel_ok = false;
        if ((cd->u > 1 || cd->v > 1) && pl.dt != DType::BF16 && (int64_t)C * cd->u * cd->v >= 32) {
            ConvParams q = p;
            q.C = C;
            q.H = H;
            q.W = W;
            q.K = k;
            q.P = P;
            q.Q = Q;
            q.R = R;
            q.S = S;
            q.u = cd->u;
            q.v = cd->v;
            q.pad_top = pt;
            q.pad_left = pl_;
            subpixel_ok = miconv::bwd_data_subpixel_fits(q);
        }
        const bool subpixel = forced_dgrad_name ? strcmp(forced_dgrad_name, kDgSubpixel.name) == 0 && subpixel_ok
                                                : subpixel_ok && !rows_mfma;
        // a strided layer onto 1-4 channels with too few (channel, phase)
        // columns for the stride-phase GEMM and filter rows of at most 16
        // taps: the GEMM whose columns are the taps of a filter row, the
        // stride grid's column sum done from LDS (conv_bwd_data_taps.hip;
        // speech layer 1 onto one channel)
        bool taps_ok = false;
        if ((cd->u > 1 || cd->v > 1) && pl.dt == DType::F32 && C <= 4) {
            ConvParams q = p;
            q.C = C;
            q.H = H;
            q.W = W;
            q.K = k;
            q.P = P;
            q.Q = Q;
            q.R = R;
            q.S = S;
            q.u = cd->u;
            q.v = cd->v;
            taps_ok = miconv::bwd_data_taps_fits(q);
        }
        const bool taps = forced_dgrad_name ? strcmp(forced_dgrad_name, kDgTaps.name) == 0 && taps_ok
                                            : taps_ok && !subpixel && !rows_mfma;
        const bool direct = forced_dgrad_name
                                ? strcmp(forced_dgrad_name, kDirect.name) == 0 || phase || rows || rows_mfma || subpixel ||
                                      taps
                                : C < 16 || rows_mfma || subpixel || taps;
        if (!direct) {
            p.C = k;
            p.K = C;
            p.H = P;
            p.W = Q;
            p.P = H;
            p.Q = W;
            p.u = cd->u;
            p.v = cd->v;
            p.div_u = FastDiv((uint32_t)cd->u);
            p.div_v = FastDiv((uint32_t)cd->v);
            p.pad_top = pt;
            p.pad_left = pl_;
            p.Kred = (int)((int64_t)k * RS);
            const int num_cu = h ? h->num_cu : kDefaultCUs;
            pl.cand = choose_tile(pl.dt, p.M, p.K, num_cu);
            if (forced_dgrad_name) {
                const Candidate* list;
                int count;
                candidates(pl.dt, &list, &count);
                for (int i = 0; i < count; ++i)
                    if (strcmp(forced_dgrad_name, list[i].name) == 0) pl.cand = list[i];
            }
        } else {
            // direct kernel layout (conv_bwd_data.hip, conv_bwd_data_phase.hip)
            if (phase) pl.cand = kDgPhase;
            if (rows) pl.cand = kDgRows;
            if (rows_mfma) pl.cand = kDgRowsMfma;
            if (subpixel) pl.cand = kDgSubpixel;
            if (taps) pl.cand = kDgTaps;
            p.C = C;
            p.H = H;
            p.W = W;
            p.K = k;
            p.P = P;
            p.Q = Q;
            p.u = cd->u;
            p.v = cd->v;
            p.pad_top = pt;
            p.pad_left = pl_;
            p.Kred = (int)((int64_t)C * RS);
        }
    }
    if (forced_dgrad_name && strcmp(forced_dgrad_name, pl.cand.name) != 0) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;   // the forced variant does not fit this problem
        return pl;
    }
    snprintf(pl.name, sizeof(pl.name), "dgrad_%s", pl.cand.name);
    pl.status = MIC_STATUS_SUCCESS;
    return pl;
}

// ---------------------------------------------------------------- filter gradient

// dw <- alpha * wgrad(x, dy) + beta * dw for the forward geometry (x, dw,
// conv); dy must have the forward output's dims.  Stride-1 layers whose
// rows fit a halo variant take conv_bwd_filter_halo.hip; the others the
// gather kernel (conv_bwd_filter.hip) or, for a dw of few tiles, the kernel
// that splits the reduction over the waves of one workgroup
// (conv_bwd_filter_split.hip), by a quantisation cost model over the dw
// tiles.  The reduction is never split across workgroups: no workspace.
Plan make_wgrad_plan(const mic_handle_st* h, const mic_tensor_desc_st* xd, const void* x,
                     const mic_tensor_desc_st* dyd, const void* dy, const mic_conv_desc_st* cd,
                     const mic_filter_desc_st* wd, const void* dw, double alpha, double beta,
                     bool need_pointers)
{
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.status = MIC_STATUS_BAD_PARAM;
    if (!xd || !dyd || !cd || !wd) return pl;
    if (!xd->set || !dyd->set || !cd->set || !wd->set) return pl;
    if (blocked(xd) || blocked(dyd) || blocked(wd)) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;     // channel-blocked layouts: forward pass only
        return pl;
    }
    if (need_pointers && (!x || !dy || !dw)) return pl;
    int n, k, P, Q;
    mic_status st = output_dims(cd, xd, wd, &n, &k, &P, &Q);
    if (st != MIC_STATUS_SUCCESS) {
        pl.status = st;
        return pl;
    }
    if (dyd->n != n || dyd->c != k || dyd->h != P || dyd->w != Q) return pl;
    if (xd->dtype == MIC_DTYPE_F32 && dyd->dtype == MIC_DTYPE_F32 && wd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::F32;
    else if (xd->dtype == MIC_DTYPE_F64 && dyd->dtype == MIC_DTYPE_F64 && wd->dtype == MIC_DTYPE_F64)
        pl.dt = DType::F64;
    else if (xd->dtype == MIC_DTYPE_BF16 && dyd->dtype == MIC_DTYPE_BF16 && wd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::BF16;
    else {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    const int64_t L = (int64_t)n * P * Q;
    const int64_t CRS = (int64_t)wd->c * wd->r * wd->s;
    if (extent(*xd) >= kMaxOffset || extent(*dyd) >= kMaxOffset || (int64_t)wd->k * CRS >= kMaxOffset ||
        L >= kMaxOffset || xd->sn >= kMaxOffset || xd->sc >= kMaxOffset || xd->sh >= kMaxOffset ||
        xd->sw >= kMaxOffset || dyd->sn >= kMaxOffset || dyd->sc >= kMaxOffset || dyd->sh >= kMaxOffset ||
        dyd->sw >= kMaxOffset) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    if (need_pointers) {
        const size_t ie = dtype_size(xd->dtype), oe = dtype_size(wd->dtype);
        if ((uintptr_t)x % ie || (uintptr_t)dy % ie || (uintptr_t)dw % oe) return pl;
    }
    ConvParams& p = pl.p;
    set_blocks(p, nullptr, nullptr, nullptr);
    p.x = x;
    p.w = dy;
    p.y = const_cast<void*>(dw);
    p.N = n;
    p.C = xd->c;
    p.H = xd->h;
    p.W = xd->w;
    p.R = wd->r;
    p.S = wd->s;
    p.P = P;
    p.Q = Q;
    p.u = cd->u;
    p.v = cd->v;
    p.pad_top = cd->pad_top;
    p.pad_left = cd->pad_left;
    p.sxn = (int)xd->sn;
    p.sxc = (int)xd->sc;
    p.sxh = (int)xd->sh;
    p.sxw = (int)xd->sw;
    p.sdn = (int)dyd->sn;
    p.sdk = (int)dyd->sc;
    p.sdp = (int)dyd->sh;
    p.sdq = (int)dyd->sw;
    p.syn = (int)CRS;       // dw packed K,C,R,S: row k, column (c, r, s)
    p.syk = 1;
    p.syp = 0;
    p.syq = 0;
    p.M = k;
    p.K = (int)CRS;
    p.Kred = (int)L;
    p.div_pq = FastDiv(1);
    p.div_q = FastDiv(1);
    p.div_rs = FastDiv((uint32_t)(wd->r * wd->s));
    p.div_s = FastDiv((uint32_t)wd->s);
    p.div_opq = FastDiv((uint32_t)(P * Q));
    p.div_oq = FastDiv((uint32_t)Q);
    p.alpha = alpha;
    p.beta = beta;

    const int num_cu = h ? h->num_cu : kDefaultCUs;
    const char* force = getenv("MIC_FORCE_WGRAD_VARIANT");
    if (force && !force[0]) force = nullptr;
    // the split kernel addresses x and dy with 32-bit byte offsets and reads
    // zeros at offset 2^31 (range-checked buffer loads)
    const int64_t es = (int64_t)dtype_size(xd->dtype);
    const bool split_fits = extent(*xd) * es < INT32_MAX && extent(*dyd) * es < INT32_MAX;
    // the halo kernels' buffer loads: x and dy under 2^30 bytes (an offset of
    // 2^30 lies past both, and three such offsets still fit 32 bits)
    const bool halo_bufs_fit = extent(*xd) * es < (int64_t(1) << 30) && extent(*dyd) * es < (int64_t(1) << 30);
    const bool unit_q = xd->sw == 1 && dyd->sw == 1;
    // The halo kernel's reduction split in two (beta = 0: both parts add into
    // a zeroed dw) when its tiles leave compute units idle in a single round.
    // MIC_WGRAD_SPLIT=off keeps one part (tests compare the two); =k (1-15)
    // sets the ratio k : 1 wherever the split is allowed (measurements).
    const char* split_env = getenv("MIC_WGRAD_SPLIT");
    const int split_force = split_env ? atoi(split_env) : 0;
    const bool split_allowed = beta == 0.0 && L >= 2 && !(split_env && strcmp(split_env, "off") == 0);
    double best = 0;
    bool found = false;
    for (const WgCandidate& wc : kWg) {
        if (wc.dt != pl.dt) continue;
        if (force && strcmp(force, wc.c.name) != 0) continue;
        bool ok = true;
        if (wc.kind == WgKind::HALO)
            // (r = 0: any filter height and row stride)
            ok = (wc.r == 0 || (wc.r == wd->r && cd->u == 1)) && wc.s == wd->s && cd->v == 1 &&
                 Q + wc.s - 1 <= wc.wph && (wc.qd == 0 || Q == wc.qd) && halo_bufs_fit;
        else if (wc.kind == WgKind::SPLIT)
            ok = split_fits;
        else if (wc.kind == WgKind::ROWS)
            ok = miconv::bwd_filter_rows_fits(wc.c.v, p);
        else if (wc.kind == WgKind::CL)
            // 16-byte loads of 8 consecutive filters / channels at every position
            ok = xd->sc == 1 && dyd->sc == 1 && wd->k % 8 == 0 && wd->c % 8 == 0 && xd->sn % 8 == 0 &&
                 xd->sh % 8 == 0 && xd->sw % 8 == 0 && dyd->sn % 8 == 0 && dyd->sh % 8 == 0 &&
                 dyd->sw % 8 == 0 && (!need_pointers || ((uintptr_t)x % 16 == 0 && (uintptr_t)dy % 16 == 0));
        // 8-filter split tiles double the tile count at 1.5x the loads per
        // position: worth it only when 16x16 tiles leave most CUs idle
        // (measured: speech L1, 58 tiles, 4.7 -> 4.1 ms; Overfeat L1, 138
        // tiles, 2.4 -> 3.0 ms)
        // (a preference of the automatic choice: forced, the kernel takes any shape)
        if (wc.c.v == Variant::WGS_F32_8x16 && !force)
            ok = ok && (int64_t)((p.M + 15) / 16) * ((p.K + 15) / 16) * 4 <= num_cu;
        if (!ok) {
            if (force) {
                pl.status = MIC_STATUS_NOT_SUPPORTED;   // forced onto a layer it cannot take
                return pl;
            }
            continue;
        }
        const int64_t tiles = (int64_t)((p.M + wc.c.tm - 1) / wc.c.tm) * ((p.K + wc.c.tn - 1) / wc.c.tn);
        const int64_t slots = (int64_t)num_cu * wc.per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        double cost = (double)rounds * wc.ns;
        if (wc.kind == WgKind::SPLIT && !unit_q) cost *= split_strided_penalty(pl.dt);
        if (wc.kind == WgKind::ROWS) cost /= Q;
        // split: T tiles, U slots; the long parts (k / (k + 1) of the
        // reduction) on T units, the short ones about T / (U - T) at a time on
        // the other U - T.  Each short part also pays a fixed cost (prologue,
        // first chunk, atomic epilogue: about 12 us measured), so past three
        // short parts per unit k takes two more.  Where two workgroups fit on
        // a CU the halves share the units: k = 1.  Measured on MI355X (AlexNet
        // conv2, 200 tiles: 1746 us in one part, 1713 at k = 4, 1498 at k = 6;
        // conv3, 216 tiles: 408 / 411 at k = 6 / 376 at k = 8; 144 tiles of
        // 64 x 96: 654 / 447 at k = 2 / 523 at k = 4; Overfeat L2, 200 tiles
        // two to a CU: 867 / 717 at k = 1 / 802 at k = 6).
        int split_k = 0;
        if (wc.kind == WgKind::HALO && split_allowed && tiles > 0 && tiles < slots) {
            // the 5x5 forms on 64 x 64 tiles gain far less than k / (k + 1)
            // (AlexNet conv2, 152 tiles: 1859 -> 1646 us at k = 2, where 200
            // tiles of 64 x 48 at k = 6 take 1498; Overfeat L2: 981 -> 844):
            // not chosen split
            if (wc.r == 5 && wc.c.tn == 64 && !force) continue;
            const double r = (double)tiles / (double)(slots - tiles);
            split_k = 2 * tiles <= slots || wc.res2 ? 1 : (int)std::ceil(r) + (r > 3.0 ? 2 : 0);
            // past six short parts per idle CU the fixed costs eat the gain
            // (speech L2, 231 tiles of 32 x 32: 2896 -> 2881 us at k = 12)
            if (split_k > 8 && !(split_force >= 1 && split_force <= 15)) split_k = 0;
            if (split_k > 0) cost *= (double)split_k / (split_k + 1);
            if (split_force >= 1 && split_force <= 15) split_k = split_force;
        }
        if (!found || cost < best) {
            best = cost;
            pl.cand = wc.c;
            pl.split_k = split_k;
            found = true;
        }
    }
    if (!found) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;   // a forced variant of another type
        return pl;
    }
    snprintf(pl.name, sizeof(pl.name), "%s", pl.cand.name);
    pl.status = MIC_STATUS_SUCCESS;
    return pl;
}

// ---------------------------------------------------------------- batch-reduce GEMM

// Highest element offset of an operand with the given extents and strides
// (all >= 0), or -1 when a stride is negative.
int64_t operand_extent(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2)
{
    if (s0 < 0 || s1 < 0 || s2 < 0) return -1;
    return (n0 - 1) * s0 + (n1 - 1) * s1 + (n2 - 1) * s2;
}

// C[m, n] <- alpha sum_i A_i B_i + beta C (single-building-block page,
// "Proposed Method"): rows m map to the kernel's M, columns n to its K,
// the per-block reduction k to Kred and the batch to N.
Plan make_brgemm_plan(const mic_handle_st* h, mic_dtype dtype, int m, int n, int k, int batch, double alpha,
                      const void* a, int64_t sa_i, int64_t sa_m, int64_t sa_k, const void* b, int64_t sb_i,
                      int64_t sb_k, int64_t sb_n, double beta, const void* c, int64_t sc_m, int64_t sc_n,
                      bool need_pointers)
{
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.status = MIC_STATUS_BAD_PARAM;
    if (m < 0 || n < 0 || k < 0 || batch < 0) return pl;
    if (sa_i < 0 || sa_m < 0 || sa_k < 0 || sb_i < 0 || sb_k < 0 || sb_n < 0 || sc_m < 0 || sc_n < 0) return pl;
    if (!valid_dtype(dtype)) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    pl.dt = dtype == MIC_DTYPE_F32 ? DType::F32 : dtype == MIC_DTYPE_F64 ? DType::F64 : DType::BF16;
    const bool empty_c = m == 0 || n == 0;
    const bool empty_red = k == 0 || batch == 0;
    if (need_pointers && !empty_c && (!c || (!empty_red && (!a || !b)))) return pl;
    // C's elements must not alias: distinct (m, n) need distinct offsets
    if (!empty_c && ((m > 1 && sc_m == 0) || (n > 1 && sc_n == 0))) return pl;
    const int64_t ea = empty_c || empty_red ? 0 : operand_extent(batch, sa_i, m, sa_m, k, sa_k);
    const int64_t eb = empty_c || empty_red ? 0 : operand_extent(batch, sb_i, k, sb_k, n, sb_n);
    const int64_t ec = empty_c ? 0 : operand_extent(1, 0, m, sc_m, n, sc_n);
    if (ea >= kMaxOffset || eb >= kMaxOffset || ec >= kMaxOffset || (int64_t)batch * k >= kMaxOffset) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    if (need_pointers && !empty_c) {
        const size_t ie = dtype_size(dtype), oe = pl.dt == DType::F64 ? 8 : 4;
        if ((uintptr_t)c % oe) return pl;
        if (!empty_red && ((uintptr_t)a % ie || (uintptr_t)b % ie)) return pl;
    }
    ConvParams& p = pl.p;
    set_blocks(p, nullptr, nullptr, nullptr);
    p.x = a;
    p.w = b;
    p.y = const_cast<void*>(c);
    p.N = batch;
    p.M = m;
    p.K = n;
    p.Kred = k;
    p.sxn = (int)sa_i;
    p.sxh = (int)sa_m;
    p.sxw = (int)sa_k;
    p.sdn = (int)sb_i;
    p.sdk = (int)sb_k;
    p.sdq = (int)sb_n;
    p.syn = (int)sc_m;
    p.syk = (int)sc_n;
    p.div_pq = FastDiv(1);
    p.div_q = FastDiv(1);
    p.div_rs = FastDiv((uint32_t)(k > 0 ? k : 1));
    p.alpha = alpha;
    p.beta = beta;

    const Candidate* list = kBrF32;
    int count = (int)(sizeof(kBrF32) / sizeof(kBrF32[0]));
    const Candidate* ws = kWsF32;
    int ws_count = (int)(sizeof(kWsF32) / sizeof(kWsF32[0]));
    if (pl.dt == DType::F64) {
        list = kBrF64;
        count = (int)(sizeof(kBrF64) / sizeof(kBrF64[0]));
        ws = kWsF64;
        ws_count = (int)(sizeof(kWsF64) / sizeof(kWsF64[0]));
    } else if (pl.dt == DType::BF16) {
        list = kBrBF16;
        count = (int)(sizeof(kBrBF16) / sizeof(kBrBF16[0]));
        ws = kWsBF16;
        ws_count = (int)(sizeof(kWsBF16) / sizeof(kWsBF16[0]));
    }
    // the wave-split kernel reads the reduction with 16-byte loads: A and B
    // contiguous along k, k a multiple of a load's elements, every load
    // 16-byte aligned (pointer alignment is known only at a call)
    const int ve = 16 / (int)dtype_size(dtype);
    auto ws_ok = [&](const Candidate& cd) {
        const int run = brgemm_ws_run(cd.v);
        if (run == 0 || k == 0 || batch == 0 || sa_k != 1 || sb_k != 1 || k % run) return false;
        if (batch > 1 && (sa_i % ve || sb_i % ve)) return false;
        if ((m > 1 && sa_m % ve) || (n > 1 && sb_n % ve)) return false;
        // its buffer descriptors: A and B under 2^30 bytes
        const int64_t es = (int64_t)dtype_size(dtype);
        if ((operand_extent(batch, sa_i, m, sa_m, k, sa_k) + 1) * es >= (int64_t(1) << 30) ||
            (operand_extent(batch, sb_i, n, sb_n, k, sb_k) + 1) * es >= (int64_t(1) << 30))
            return false;
        return !need_pointers || ((uintptr_t)a % 16 == 0 && (uintptr_t)b % 16 == 0);
    };
    const int num_cu = h ? h->num_cu : kDefaultCUs;
    const char* force = getenv("MIC_FORCE_BRGEMM_VARIANT");
    if (force && !force[0]) force = nullptr;
    bool found = false;
    if (force) {
        for (int i = 0; i < count && !found; ++i)
            if (strcmp(force, list[i].name) == 0) {
                pl.cand = list[i];
                found = true;
            }
        for (int i = 0; i < ws_count && !found; ++i)
            if (strcmp(force, ws[i].name) == 0) {
                if (!ws_ok(ws[i])) {
                    pl.status = MIC_STATUS_NOT_SUPPORTED;   // forced onto operands it cannot read
                    return pl;
                }
                pl.cand = ws[i];
                found = true;
            }
    } else {
        // Products whose 128 x 128 tiles cannot fill the chip go to the
        // wave-split kernel (measured on MI355X: faster there, the shared-LDS
        // tiles faster once 128 x 128 tiles fill every compute unit): its
        // largest tile that still gives every compute unit one, else its
        // smallest.
        const int64_t big = (int64_t)((m + 127) / 128) * ((n + 127) / 128);
        if (big < num_cu) {
            for (int i = 0; i < ws_count && !found; ++i) {
                const int64_t tiles = (int64_t)((m + ws[i].tm - 1) / ws[i].tm) * ((n + ws[i].tn - 1) / ws[i].tn);
                if (ws_ok(ws[i]) && (tiles >= num_cu || i == ws_count - 1)) {
                    pl.cand = ws[i];
                    found = true;
                }
            }
        }
        double best = 0;
        for (int i = 0; i < count && !found; ++i) {
            const int64_t tiles = (int64_t)((m + list[i].tm - 1) / list[i].tm) * ((n + list[i].tn - 1) / list[i].tn);
            const int64_t rounds = (tiles + num_cu - 1) / num_cu;
            const double reuse = (double)list[i].tm * list[i].tn / (list[i].tm + list[i].tn);
            const double eff = reuse >= 48.0 ? 1.0 : reuse / 48.0;
            const double cost = (double)rounds * list[i].tm * list[i].tn / eff;
            if (i == 0 || cost < best) {
                best = cost;
                pl.cand = list[i];
            }
        }
        found = true;
    }
    if (!found) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;   // a forced variant of another type
        return pl;
    }
    snprintf(pl.name, sizeof(pl.name), "%s", pl.cand.name);
    pl.status = MIC_STATUS_SUCCESS;
    return pl;
}

// ---------------------------------------------------------------- pooling

// Output dims of pooling: the convolution's floor rule over the window.
mic_status pool_output_dims(const mic_pool_desc_st* pd, const mic_tensor_desc_st* xd, int* n, int* c, int* p,
                            int* q)
{
    if (!pd || !xd || !pd->set || !xd->set) return MIC_STATUS_BAD_PARAM;
    const int64_t hspan = (int64_t)xd->h + pd->pad_top + pd->pad_bottom - pd->r;
    const int64_t wspan = (int64_t)xd->w + pd->pad_left + pd->pad_right - pd->s;
    if (hspan < 0 || wspan < 0) return MIC_STATUS_BAD_PARAM;
    const int64_t P = hspan / pd->u + 1;
    const int64_t Q = wspan / pd->v + 1;
    if (P > INT32_MAX || Q > INT32_MAX) return MIC_STATUS_NOT_SUPPORTED;
    *n = xd->n;
    *c = xd->c;
    *p = (int)P;
    *q = (int)Q;
    return MIC_STATUS_SUCCESS;
}

Plan make_pool_plan(const mic_pool_desc_st* pd, const mic_tensor_desc_st* xd, const void* x,
                    const mic_tensor_desc_st* yd, const void* y, double alpha, double beta, bool need_pointers)
{
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.status = MIC_STATUS_BAD_PARAM;
    if (!yd || !yd->set) return pl;
    if (blocked(xd) || blocked(yd)) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;     // channel-blocked layouts: forward pass only
        return pl;
    }
    if (need_pointers && (!x || !y)) return pl;
    int n, c, P, Q;
    mic_status st = pool_output_dims(pd, xd, &n, &c, &P, &Q);
    if (st != MIC_STATUS_SUCCESS) {
        pl.status = st;
        return pl;
    }
    if (yd->n != n || yd->c != c || yd->h != P || yd->w != Q) return pl;
    if (xd->dtype == MIC_DTYPE_F32 && yd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::F32;
    else if (xd->dtype == MIC_DTYPE_F64 && yd->dtype == MIC_DTYPE_F64)
        pl.dt = DType::F64;
    else if (xd->dtype == MIC_DTYPE_BF16 && yd->dtype == MIC_DTYPE_F32)
        pl.dt = DType::BF16;
    else {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    const int64_t M = (int64_t)n * P * Q;
    // the kernel visits the R*S window positions of every output with int
    // arithmetic: the window stays below the offset limit too
    if ((int64_t)pd->r * pd->s >= kMaxOffset || extent(*xd) >= kMaxOffset || extent(*yd) >= kMaxOffset ||
        M * c >= kMaxOffset ||
        xd->sn >= kMaxOffset || xd->sc >= kMaxOffset || xd->sh >= kMaxOffset || xd->sw >= kMaxOffset ||
        yd->sn >= kMaxOffset || yd->sc >= kMaxOffset || yd->sh >= kMaxOffset || yd->sw >= kMaxOffset) {
        pl.status = MIC_STATUS_NOT_SUPPORTED;
        return pl;
    }
    if (need_pointers) {
        const size_t ie = dtype_size(xd->dtype), oe = dtype_size(yd->dtype);
        if ((uintptr_t)x % ie || (uintptr_t)y % oe) return pl;
    }
    ConvParams& p = pl.p;
    set_blocks(p, nullptr, nullptr, nullptr);
    p.x = x;
    p.y = const_cast<void*>(y);
    p.N = n;
    p.C = c;
    p.H = xd->h;
    p.W = xd->w;
    p.R = pd->r;
    p.S = pd->s;
    p.P = P;
    p.Q = Q;
    p.u = pd->u;
    p.v = pd->v;
    p.pad_top = pd->pad_top;
    p.pad_left = pd->pad_left;
    p.sxn = (int)xd->sn;
    p.sxc = (int)xd->sc;
    p.sxh = (int)xd->sh;
    p.sxw = (int)xd->sw;
    p.syn = (int)yd->sn;
    p.syk = (int)yd->sc;
    p.syp = (int)yd->sh;
    p.syq = (int)yd->sw;
    p.M = (int)M;
    p.Kred = (int)pd->mode;    // pool_fwd.hip reads the mode here
    p.div_pq = FastDiv((uint32_t)(P * Q));
    p.div_q = FastDiv((uint32_t)Q);
    p.div_rs = FastDiv((uint32_t)c);      // pool_fwd.hip: the channel count
    p.div_s = FastDiv((uint32_t)M);       // and N*P*Q
    p.alpha = alpha;
    p.beta = beta;
    snprintf(pl.name, sizeof(pl.name), "pool_direct");
    pl.status = MIC_STATUS_SUCCESS;
    return pl;
}

}  // namespace

extern "C" {

const char* mic_status_string(mic_status status)
{
    switch (status) {
    case MIC_STATUS_SUCCESS: return "success";
    case MIC_STATUS_BAD_PARAM: return "bad parameter";
    case MIC_STATUS_NOT_SUPPORTED: return "not supported";
    case MIC_STATUS_LAUNCH_FAILED: return "kernel launch failed";
    case MIC_STATUS_INTERNAL_ERROR: return "internal error";
    case MIC_STATUS_ALLOC_FAILED: return "host allocation failed";
    }
    return "unknown status";
}

mic_status mic_get_version(int* major, int* minor, int* patch)
{
    if (major) *major = MICONV_VERSION_MAJOR;
    if (minor) *minor = MICONV_VERSION_MINOR;
    if (patch) *patch = MICONV_VERSION_PATCH;
    return MIC_STATUS_SUCCESS;
}

// ---------------------------------------------------------------- handle

mic_status mic_create(mic_handle* handle)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    *handle = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MIC_STATUS_INTERNAL_ERROR;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MIC_STATUS_INTERNAL_ERROR;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MIC_STATUS_NOT_SUPPORTED;
    mic_handle_st* h = new (std::nothrow) mic_handle_st;
    if (!h) return MIC_STATUS_ALLOC_FAILED;
    h->device = dev;
    h->num_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCUs;
    h->stream = nullptr;
    *handle = h;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_destroy(mic_handle handle)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    delete handle;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_set_stream(mic_handle handle, void* stream)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    handle->stream = static_cast<hipStream_t>(stream);
    return MIC_STATUS_SUCCESS;
}

mic_status mic_get_stream(mic_handle handle, void** stream)
{
    if (!handle || !stream) return MIC_STATUS_BAD_PARAM;
    *stream = handle->stream;
    return MIC_STATUS_SUCCESS;
}

// ---------------------------------------------------------------- tensor descriptor

mic_status mic_tensor_desc_create(mic_tensor_desc* desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    *desc = new (std::nothrow) mic_tensor_desc_st();
    return *desc ? MIC_STATUS_SUCCESS : MIC_STATUS_ALLOC_FAILED;
}

mic_status mic_tensor_desc_destroy(mic_tensor_desc desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    delete desc;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_tensor_desc_set(mic_tensor_desc desc, mic_dtype dtype, int n, int c, int h, int w,
                               int64_t sn, int64_t sc, int64_t sh, int64_t sw)
{
    if (!desc || !valid_dtype(dtype)) return MIC_STATUS_BAD_PARAM;
    if (n < 1 || c < 1 || h < 1 || w < 1) return MIC_STATUS_BAD_PARAM;
    if (sn < 1 || sc < 1 || sh < 1 || sw < 1) return MIC_STATUS_BAD_PARAM;
    desc->set = true;
    desc->dtype = dtype;
    desc->n = n;
    desc->c = c;
    desc->h = h;
    desc->w = w;
    desc->sn = sn;
    desc->sc = sc;
    desc->sh = sh;
    desc->sw = sw;
    desc->cb = 0;
    desc->scb = 0;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_tensor_desc_set_blocked(mic_tensor_desc desc, mic_dtype dtype, int n, int c, int h, int w, int cb)
{
    if (!desc || !valid_dtype(dtype)) return MIC_STATUS_BAD_PARAM;
    if (n < 1 || c < 1 || h < 1 || w < 1 || cb < 1 || c % cb != 0) return MIC_STATUS_BAD_PARAM;
    const int64_t H = h, W = w, CB = cb;
    mic_status st = mic_tensor_desc_set(desc, dtype, n, c, h, w, (int64_t)c * H * W, 1, W * CB, CB);
    if (st != MIC_STATUS_SUCCESS) return st;
    desc->cb = cb;
    desc->scb = H * W * CB;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_tensor_desc_get_block(mic_tensor_desc desc, int* cb, int64_t* block_stride)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (cb) *cb = desc->cb;
    if (block_stride) *block_stride = desc->scb;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_tensor_desc_set_packed(mic_tensor_desc desc, mic_dtype dtype, mic_layout layout,
                                      int n, int c, int h, int w)
{
    if (n < 1 || c < 1 || h < 1 || w < 1) return MIC_STATUS_BAD_PARAM;
    const int64_t C = c, H = h, W = w;
    switch (layout) {
    case MIC_LAYOUT_NCHW: return mic_tensor_desc_set(desc, dtype, n, c, h, w, C * H * W, H * W, W, 1);
    case MIC_LAYOUT_NHWC: return mic_tensor_desc_set(desc, dtype, n, c, h, w, H * W * C, 1, W * C, C);
    }
    return MIC_STATUS_BAD_PARAM;
}

mic_status mic_tensor_desc_get(mic_tensor_desc desc, mic_dtype* dtype, int* n, int* c, int* h,
                               int* w, int64_t* strides)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (dtype) *dtype = desc->dtype;
    if (n) *n = desc->n;
    if (c) *c = desc->c;
    if (h) *h = desc->h;
    if (w) *w = desc->w;
    if (strides) {
        strides[0] = desc->sn;
        strides[1] = desc->sc;
        strides[2] = desc->sh;
        strides[3] = desc->sw;
    }
    return MIC_STATUS_SUCCESS;
}

// ---------------------------------------------------------------- filter descriptor

mic_status mic_filter_desc_create(mic_filter_desc* desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    *desc = new (std::nothrow) mic_filter_desc_st();
    return *desc ? MIC_STATUS_SUCCESS : MIC_STATUS_ALLOC_FAILED;
}

mic_status mic_filter_desc_destroy(mic_filter_desc desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    delete desc;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_filter_desc_set(mic_filter_desc desc, mic_dtype dtype, int k, int c, int r, int s)
{
    if (!desc || !valid_dtype(dtype)) return MIC_STATUS_BAD_PARAM;
    if (k < 1 || c < 1 || r < 1 || s < 1) return MIC_STATUS_BAD_PARAM;
    desc->set = true;
    desc->dtype = dtype;
    desc->k = k;
    desc->c = c;
    desc->r = r;
    desc->s = s;
    desc->kb = 0;
    desc->cb = 0;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_filter_desc_set_blocked(mic_filter_desc desc, mic_dtype dtype, int k, int c, int r, int s, int kb,
                                       int cb)
{
    if (!desc || kb < 1 || cb < 1 || k % kb != 0 || c % cb != 0) return MIC_STATUS_BAD_PARAM;
    mic_status st = mic_filter_desc_set(desc, dtype, k, c, r, s);
    if (st != MIC_STATUS_SUCCESS) return st;
    desc->kb = kb;
    desc->cb = cb;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_filter_desc_get_block(mic_filter_desc desc, int* kb, int* cb)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (kb) *kb = desc->kb;
    if (cb) *cb = desc->cb;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_filter_desc_get(mic_filter_desc desc, mic_dtype* dtype, int* k, int* c, int* r, int* s)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (dtype) *dtype = desc->dtype;
    if (k) *k = desc->k;
    if (c) *c = desc->c;
    if (r) *r = desc->r;
    if (s) *s = desc->s;
    return MIC_STATUS_SUCCESS;
}

// ---------------------------------------------------------------- convolution descriptor

mic_status mic_conv_desc_create(mic_conv_desc* desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    *desc = new (std::nothrow) mic_conv_desc_st();
    return *desc ? MIC_STATUS_SUCCESS : MIC_STATUS_ALLOC_FAILED;
}

mic_status mic_conv_desc_destroy(mic_conv_desc desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    delete desc;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_conv_desc_set(mic_conv_desc desc, int pad_top, int pad_bottom, int pad_left,
                             int pad_right, int stride_h, int stride_w)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    if (pad_top < 0 || pad_bottom < 0 || pad_left < 0 || pad_right < 0) return MIC_STATUS_BAD_PARAM;
    if (stride_h < 1 || stride_w < 1) return MIC_STATUS_BAD_PARAM;
    desc->set = true;
    desc->pad_top = pad_top;
    desc->pad_bottom = pad_bottom;
    desc->pad_left = pad_left;
    desc->pad_right = pad_right;
    desc->u = stride_h;
    desc->v = stride_w;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_conv_desc_get(mic_conv_desc desc, int* pad_top, int* pad_bottom, int* pad_left,
                             int* pad_right, int* stride_h, int* stride_w)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (pad_top) *pad_top = desc->pad_top;
    if (pad_bottom) *pad_bottom = desc->pad_bottom;
    if (pad_left) *pad_left = desc->pad_left;
    if (pad_right) *pad_right = desc->pad_right;
    if (stride_h) *stride_h = desc->u;
    if (stride_w) *stride_w = desc->v;
    return MIC_STATUS_SUCCESS;
}

// ---------------------------------------------------------------- forward

mic_status mic_conv_forward_output_dim(mic_conv_desc conv, mic_tensor_desc x_desc,
                                       mic_filter_desc w_desc, int* n, int* k, int* p, int* q)
{
    if (!n || !k || !p || !q) return MIC_STATUS_BAD_PARAM;
    return output_dims(conv, x_desc, w_desc, n, k, p, q);
}

mic_status mic_conv_forward(mic_handle handle, double alpha, mic_tensor_desc x_desc, const void* x,
                            mic_filter_desc w_desc, const void* w, mic_conv_desc conv, double beta,
                            mic_tensor_desc y_desc, void* y)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_plan(handle, x_desc, x, w_desc, w, conv, y_desc, y, alpha, beta, true);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    pl.p.tile_rev = tile_order_reversed();
    hipError_t err;
    if (pl.cand.v == Variant::DIRECT)
        err = miconv::launch_direct(pl.dt, pl.p, handle->stream);
    else if (pl.cand.v == kRowsF32.v || pl.cand.v == kRows1F32.v || pl.cand.v == kRows1N6F32.v)
        err = miconv::launch_rows(pl.cand.v, pl.p, handle->stream);
    else if (is_halo(pl.cand.v))
        err = miconv::launch_halo(pl.cand.v, pl.p, false, handle->stream);
    else
        err = miconv::launch_mfma(pl.cand.v, pl.p, pl.bvec, pl.tap, false, handle->stream);
    return err == hipSuccess ? MIC_STATUS_SUCCESS : MIC_STATUS_LAUNCH_FAILED;
}

mic_status mic_conv_backward_data(mic_handle handle, double alpha, mic_filter_desc w_desc, const void* w,
                                  mic_tensor_desc dy_desc, const void* dy, mic_conv_desc conv, double beta,
                                  mic_tensor_desc dx_desc, void* dx)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_dgrad_plan(handle, dy_desc, dy, w_desc, w, conv, dx_desc, dx, alpha, beta, true);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    pl.p.tile_rev = tile_order_reversed();
    hipError_t err;
    if (pl.cand.v == Variant::DIRECT)
        err = miconv::launch_bwd_data_direct(pl.dt, pl.p, handle->stream);
    else if (pl.cand.v == Variant::DG_PHASE)
        err = miconv::launch_bwd_data_phase(pl.dt, pl.p, handle->stream);
    else if (pl.cand.v == Variant::DG_ROWS)
        err = miconv::launch_bwd_data_rows(pl.p, handle->stream);
    else if (pl.cand.v == Variant::DG_ROWS_MFMA)
        err = miconv::launch_bwd_data_rows_mfma(pl.p, handle->stream);
    else if (pl.cand.v == Variant::DG_TAPS)
        err = miconv::launch_bwd_data_taps(pl.p, handle->stream);
    else if (pl.cand.v == Variant::DG_SUBPIXEL)
        err = miconv::launch_bwd_data_subpixel(pl.dt, pl.p, handle->stream);
    else if (is_halo(pl.cand.v) && pl.dt == DType::BF16)
        err = miconv::launch_halo_bf16_dgrad(pl.cand.v, pl.p, handle->stream);
    else if (is_halo(pl.cand.v))
        err = miconv::launch_halo(pl.cand.v, pl.p, true, handle->stream);
    else
        err = miconv::launch_mfma(pl.cand.v, pl.p, false, true, true, handle->stream);
    return err == hipSuccess ? MIC_STATUS_SUCCESS : MIC_STATUS_LAUNCH_FAILED;
}

mic_status mic_conv_backward_data_kernel_name(mic_handle handle, mic_filter_desc w_desc,
                                              mic_tensor_desc dy_desc, mic_conv_desc conv,
                                              mic_tensor_desc dx_desc, char* buf, size_t buflen)
{
    if (!buf) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_dgrad_plan(handle, dy_desc, nullptr, w_desc, nullptr, conv, dx_desc, nullptr, 1.0, 0.0, false);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    const size_t len = strlen(pl.name);
    if (len + 1 > buflen) return MIC_STATUS_BAD_PARAM;
    memcpy(buf, pl.name, len + 1);
    return MIC_STATUS_SUCCESS;
}

mic_status mic_conv_backward_filter(mic_handle handle, double alpha, mic_tensor_desc x_desc, const void* x,
                                    mic_tensor_desc dy_desc, const void* dy, mic_conv_desc conv, double beta,
                                    mic_filter_desc dw_desc, void* dw)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_wgrad_plan(handle, x_desc, x, dy_desc, dy, conv, dw_desc, dw, alpha, beta, true);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    pl.p.tile_rev = tile_order_reversed();
    const hipError_t err = is_wgh(pl.cand.v)
                               ? miconv::launch_bwd_filter_halo(pl.cand.v, pl.p, pl.split_k, handle->stream)
                           : is_wgc(pl.cand.v) ? miconv::launch_bwd_filter_cl(pl.cand.v, pl.p, handle->stream)
                           : is_wgs(pl.cand.v) ? miconv::launch_bwd_filter_split(pl.cand.v, pl.p, handle->stream)
                           : is_wgr(pl.cand.v) ? miconv::launch_bwd_filter_rows(pl.cand.v, pl.p, handle->stream)
                                               : miconv::launch_bwd_filter(pl.cand.v, pl.p, handle->stream);
    return err == hipSuccess ? MIC_STATUS_SUCCESS : MIC_STATUS_LAUNCH_FAILED;
}

mic_status mic_conv_backward_filter_kernel_name(mic_handle handle, mic_tensor_desc x_desc,
                                                mic_tensor_desc dy_desc, mic_conv_desc conv,
                                                mic_filter_desc dw_desc, char* buf, size_t buflen)
{
    if (!buf) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_wgrad_plan(handle, x_desc, nullptr, dy_desc, nullptr, conv, dw_desc, nullptr, 1.0, 0.0, false);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    const size_t len = strlen(pl.name);
    if (len + 1 > buflen) return MIC_STATUS_BAD_PARAM;
    memcpy(buf, pl.name, len + 1);
    return MIC_STATUS_SUCCESS;
}

mic_status mic_pool_desc_create(mic_pool_desc* desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    *desc = new (std::nothrow) mic_pool_desc_st();
    return *desc ? MIC_STATUS_SUCCESS : MIC_STATUS_ALLOC_FAILED;
}

mic_status mic_pool_desc_destroy(mic_pool_desc desc)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    delete desc;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_pool_desc_set(mic_pool_desc desc, mic_pool_mode mode, int window_h, int window_w, int pad_top,
                             int pad_bottom, int pad_left, int pad_right, int stride_h, int stride_w)
{
    if (!desc) return MIC_STATUS_BAD_PARAM;
    if (mode != MIC_POOL_MAX && mode != MIC_POOL_AVG_INCLUDE_PAD && mode != MIC_POOL_AVG_EXCLUDE_PAD)
        return MIC_STATUS_BAD_PARAM;
    if (window_h < 1 || window_w < 1 || stride_h < 1 || stride_w < 1) return MIC_STATUS_BAD_PARAM;
    if (pad_top < 0 || pad_bottom < 0 || pad_left < 0 || pad_right < 0) return MIC_STATUS_BAD_PARAM;
    desc->set = true;
    desc->mode = mode;
    desc->r = window_h;
    desc->s = window_w;
    desc->pad_top = pad_top;
    desc->pad_bottom = pad_bottom;
    desc->pad_left = pad_left;
    desc->pad_right = pad_right;
    desc->u = stride_h;
    desc->v = stride_w;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_pool_desc_get(mic_pool_desc desc, mic_pool_mode* mode, int* window_h, int* window_w, int* pad_top,
                             int* pad_bottom, int* pad_left, int* pad_right, int* stride_h, int* stride_w)
{
    if (!desc || !desc->set) return MIC_STATUS_BAD_PARAM;
    if (mode) *mode = desc->mode;
    if (window_h) *window_h = desc->r;
    if (window_w) *window_w = desc->s;
    if (pad_top) *pad_top = desc->pad_top;
    if (pad_bottom) *pad_bottom = desc->pad_bottom;
    if (pad_left) *pad_left = desc->pad_left;
    if (pad_right) *pad_right = desc->pad_right;
    if (stride_h) *stride_h = desc->u;
    if (stride_w) *stride_w = desc->v;
    return MIC_STATUS_SUCCESS;
}

mic_status mic_pool_forward_output_dim(mic_pool_desc pool, mic_tensor_desc x_desc, int* n, int* c, int* p, int* q)
{
    if (!n || !c || !p || !q) return MIC_STATUS_BAD_PARAM;
    return pool_output_dims(pool, x_desc, n, c, p, q);
}

mic_status mic_pool_forward(mic_handle handle, double alpha, mic_pool_desc pool, mic_tensor_desc x_desc,
                            const void* x, double beta, mic_tensor_desc y_desc, void* y)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_pool_plan(pool, x_desc, x, y_desc, y, alpha, beta, true);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    const hipError_t err = miconv::launch_pool_forward(pl.dt, pl.p, handle->stream);
    return err == hipSuccess ? MIC_STATUS_SUCCESS : MIC_STATUS_LAUNCH_FAILED;
}

mic_status mic_brgemm(mic_handle handle, mic_dtype dtype, int m, int n, int k, int batch, double alpha,
                      const void* a, int64_t a_stride_batch, int64_t a_stride_m, int64_t a_stride_k,
                      const void* b, int64_t b_stride_batch, int64_t b_stride_k, int64_t b_stride_n,
                      double beta, void* c, int64_t c_stride_m, int64_t c_stride_n)
{
    if (!handle) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_brgemm_plan(handle, dtype, m, n, k, batch, alpha, a, a_stride_batch, a_stride_m, a_stride_k,
                               b, b_stride_batch, b_stride_k, b_stride_n, beta, c, c_stride_m, c_stride_n, true);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    if (m == 0 || n == 0) return MIC_STATUS_SUCCESS;
    pl.p.tile_rev = tile_order_reversed();
    const hipError_t err = miconv::launch_brgemm(pl.cand.v, pl.p, handle->stream);
    return err == hipSuccess ? MIC_STATUS_SUCCESS : MIC_STATUS_LAUNCH_FAILED;
}

mic_status mic_brgemm_kernel_name(mic_handle handle, mic_dtype dtype, int m, int n, int k, int batch,
                                  int64_t a_stride_batch, int64_t a_stride_m, int64_t a_stride_k,
                                  int64_t b_stride_batch, int64_t b_stride_k, int64_t b_stride_n,
                                  int64_t c_stride_m, int64_t c_stride_n, char* buf, size_t buflen)
{
    if (!buf) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_brgemm_plan(handle, dtype, m, n, k, batch, 1.0, nullptr, a_stride_batch, a_stride_m, a_stride_k,
                               nullptr, b_stride_batch, b_stride_k, b_stride_n, 0.0, nullptr, c_stride_m, c_stride_n,
                               false);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    const size_t len = strlen(pl.name);
    if (len + 1 > buflen) return MIC_STATUS_BAD_PARAM;
    memcpy(buf, pl.name, len + 1);
    return MIC_STATUS_SUCCESS;
}

mic_status mic_conv_forward_kernel_name(mic_handle handle, mic_tensor_desc x_desc,
                                        mic_filter_desc w_desc, mic_conv_desc conv,
                                        mic_tensor_desc y_desc, char* buf, size_t buflen)
{
    if (!buf) return MIC_STATUS_BAD_PARAM;
    Plan pl = make_plan(handle, x_desc, nullptr, w_desc, nullptr, conv, y_desc, nullptr, 1.0, 0.0, false);
    if (pl.status != MIC_STATUS_SUCCESS) return pl.status;
    const size_t len = strlen(pl.name);
    if (len + 1 > buflen) return MIC_STATUS_BAD_PARAM;
    memcpy(buf, pl.name, len + 1);
    return MIC_STATUS_SUCCESS;
}

}  // extern "C"
