// conv_bwd_filter_halo.hip -- filter gradient of a stride-1 convolution with
// the receptive fields read from an LDS halo (gfx950 MFMA).
//
//   dw[k,c,r,s] = alpha * sum_{n,p,q} dy[n,k,p,q] * X(n, c, p + r - pad_top, q + s - pad_left)
//               + beta * dw[k,c,r,s]
//
// (the adjoint of the forward sum in F; cuDNN page, "Proposed Method":
// forward and backward routines; maxDNN page, Abstract and RQ4: the forward
// techniques carry over to the backward pass).  The matrix product is the
// one of conv_bwd_filter.hip -- rows k (TM per tile), columns j = (c, r, s)
// (TN per tile), reduction over the positions (n, p, q) -- but the
// reduction runs in chunks of PR output rows of one image n, and each chunk
// is staged in LDS once:
//
//   DY[k][pos]           dy[n, k, p0 + pos / WPH, pos % WPH]   (0 for q >= Q or p >= P)
//   HALO[c - c_lo][h][w] X(n, c, p0 + h - pad_top, w - pad_left)  (0 outside the plane)
//
// with the position index pos = (p - p0) * WPH + q over a compile-time row
// pitch WPH >= Q + S - 1.  Then B[pos, (c, r, s)] = HALO[c - c_lo][p - p0 + r][q + s]
// = HALO_flat[base(c, r, s) + pos]: both MFMA operands are LDS reads at a
// per-lane base plus the compile-time step, and the MFMA loop carries no
// address arithmetic (the same device the forward halo kernel uses for its
// input operand, with the roles of positions and taps exchanged).  Padding
// positions (q >= Q, p >= P) have dy = 0 and cost MFMA steps only: Q / WPH
// of the work is useful.  Lane group g of an MFMA takes positions
// [g * SEGP, (g + 1) * SEGP).
//
// QD > 0 (instances for a compile-time output width Q = QD, with PR a
// multiple of G): lane group g takes the output rows g, g + G, ... of the
// chunk and steps along their QD real columns only, so no step lands on a
// padding column; step u of the group is row G * (u / QD) + g, column
// u % QD, at the compile-time offset G * WPH * (u / QD) + u % QD from the
// group's base g * WPH.  With KS groups of 4 waves ("halves", KS = 1, 2 or
// 4), group h takes steps [h * SEGH, (h + 1) * SEGH) (the last may take fewer)
// (one fewer when SEGP is odd), each in its own unrolled copy of the steps.
//
// R = 0 ("pairs"; any filter height, any row stride u, column stride 1):
// instead of every input row of CH whole channels, a chunk stages, for each
// (channel c, filter row r) pair the tile's columns touch (at most
// (TN - 2 + S) / S + 1 of them), the input rows (p0 + pr) * u + r - pad_top
// of its PR output rows, WPH columns each, at PLANE >= PR * WPH + S - 1 per
// pair.  B[pos, (c, r, s)] is then PAIR[(c, r)][pos + s] with the same
// position index as DY: tall filters (21 rows onto 32 channels at stride 2,
// the speech network's second layer) whose channel planes would not fit.
//
// No workspace.  The epilogue stores dw (packed K,C,R,S) along j as
// conv_bwd_filter.hip does; or, with split_ch > 0 (beta = 0 only), the
// launch runs every tile twice: workgroup b < T (T tiles) takes the chunks
// [0, split_ch) of its tile, workgroup T + b the chunks [split_ch, end),
// and both add alpha times their sum into dw, zeroed beforehand, with
// atomic adds.  Two terms added onto zero give the same bits in either
// order (fp addition commutes), so the result does not depend on which
// workgroup lands first.  This fills the compute units a one-round launch
// leaves idle: with T tiles on U units and k = ceil(T / (U - T)), the long
// parts (a fraction k / (k + 1) of the chunks) run on T units while the
// other U - T units take the short ones k at a time.
//
// Parameters as for conv_bwd_filter.hip: x, strides sx*; w = dy, strides
// sd*; y = dw with syn = C*R*S, syk = 1; M = K, K = C*R*S; div_pq = div_q = 1;
// u = v = 1 (host-checked), Q + S - 1 <= WPH.
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "conv_params.h"
#include "kernels.h"
#include "mfma_common.h"
#include "tile_map.h"

namespace miconv {

namespace {
constexpr int kWghBufWord3 = 0x00020000;         // raw 32-bit buffer, range-checked per dword
// an offset past any buffer here (x and dy are under 2^30 bytes, host-checked);
// a sum of up to three of them and a valid offset stays below 2^32
constexpr uint32_t kWghOutside = 0x40000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wgh_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kWghBufWord3);
}
__device__ __forceinline__ void wgh_load(float& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, int soff)
{
    v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0));
}
__device__ __forceinline__ void wgh_load(double& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, int soff)
{
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, soff, 0);
    v = __hiloint2double((int)t[1], (int)t[0]);
}

// a global element of type G into a staged register: bf16 (the upper half of
// an fp32) widened exactly, fp32 / fp64 as they are
template <class G, class T>
__device__ __forceinline__ void wgh_gload(T& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, int soff)
{
    if constexpr (std::is_same<G, uint16_t>::value)
        v = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, soff, 0) << 16);
    else
        wgh_load(v, r, voff, soff);
}

template <class Pol, class = void>
struct wgh_gin {
    using type = typename Pol::In;
};
template <class Pol>
struct wgh_gin<Pol, std::void_t<typename Pol::GIn>> {
    using type = typename Pol::GIn;
};

template <int B, int E, class F>
__device__ __forceinline__ void unroll_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        unroll_for<B + 1, E>(f);
    }
}
}  // namespace

// bf16 x and dy (GIn: their 2-byte storage) widened to fp32 as they are
// staged, then the fp32 MFMA of P: products and sums in fp32, as the pages'
// fp32 filter gradient, from inputs that are exact in fp32
template <class P>
struct WghBf16 : P {
    using GIn = uint16_t;
    static_assert(std::is_same<typename P::In, float>::value, "fp32 staging");
};

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int WPH, int PR, int PLANE, int KS,
          int QD>
__global__ void __launch_bounds__(256 * KS)
conv_bwd_filter_halo_kernel(const ConvParams p, int split_ch)
{
    using In = typename Pol::In;                     // staged (LDS) element
    using GIn = typename wgh_gin<Pol>::type;         // stored element of x and dy
    using AccV = typename Pol::AccV;
    constexpr int NT = 256;                          // threads per half
    constexpr int NTT = NT * KS;                     // threads of the workgroup
    constexpr int BM = Pol::BM;
    constexpr int G = Pol::G;
    constexpr int ES = (int)sizeof(In);
    constexpr int GES = (int)sizeof(GIn);
    constexpr int RS = R * S;
    constexpr int RS1 = RS > 0 ? RS : 1;             // (pairs: R = 0; divisions by RS not taken)
    constexpr int WM = TM / WAVES_M;
    constexpr int WN = TN / WAVES_N;
    constexpr int FM = WM / BM;
    constexpr int FN = WN / BM;
    constexpr int NPOS = PR * WPH;                   // positions per chunk
    constexpr int SEGP = QD > 0 ? PR / G * QD : NPOS / G;   // MFMA steps per chunk
    constexpr int SEGH = (SEGP + KS - 1) / KS;       // ... of half 0 (QD > 0: the last half may take fewer)
    static_assert(QD == 0 || (PR % G == 0 && QD + S - 1 <= WPH), "whole rows per lane group");
    constexpr int DYP = NPOS + 1;                    // DY row pitch (odd: rows fall on other banks)
    constexpr bool PAIRS = R == 0;                   // staged rows: the tile's (channel, filter row) pairs
    constexpr int HROWS = PAIRS ? PR : PR + R - 1;
    // A padding position's tap (q + s up to WPH + S - 2) reads up to S - 1
    // elements past the plane's last row: PLANE >= HROWS * WPH + S - 1 leaves
    // spare elements, zeroed once, so such reads see finite zeros.  Beyond
    // that, WPH and PLANE are chosen so the 32 columns (c, r, s) a half-wave
    // reads land on distinct LDS banks but for at most two-way conflicts.
    static_assert(PLANE >= HROWS * WPH + S - 1, "plane spare");   // (pairs: HROWS = PR)
    // channels (pairs) TN consecutive columns can touch
    constexpr int CH = PAIRS ? (TN - 2 + S) / S + 1 : (RS - 1 + TN - 1) / RS1 + 1;
    constexpr int DY_ELEMS = TM * DYP;
    constexpr int BUF_BYTES = ((DY_ELEMS + CH * PLANE) * ES + 15) / 16 * 16;
    // DY loader: in each half TPK threads per filter row; half h takes rows
    // pr = h + KS * i, a thread positions q0 + TPK * j of them.  With fewer
    // rows than halves (DY_ALL) all threads share every row instead: TPK =
    // the workgroup's threads per filter row.
    constexpr bool DY_ALL = PR < KS;
    constexpr int TPK = (DY_ALL ? NTT : NT) / TM;
    constexpr int QPT = WPH / TPK;                   // q values a thread visits per row
    constexpr int PRH = DY_ALL ? PR : (PR + KS - 1) / KS;   // rows per thread
    constexpr int RSTEP = DY_ALL ? 1 : KS;           // between a thread's rows
    constexpr int NDY = PRH * QPT;                   // DY elements per thread per chunk
    // halo loader: units (channel, row, column), column fastest, over all threads
    constexpr int HU = CH * HROWS * WPH;
    constexpr int NH = (HU + NTT - 1) / NTT;
    static_assert(Pol::V == 1, "scalar-operand MFMA policies only");
    static_assert(WAVES_M * WAVES_N == 4 && WM % BM == 0 && WN % BM == 0, "wave tiling");
    static_assert(NPOS % G == 0 && NT % TM == 0 && WPH % TPK == 0, "loader shapes");
    static_assert(PLANE >= (PAIRS ? PR * WPH : 0) + S - 1, "pair spare");
    static_assert((KS == 1 || KS == 2 || KS == 4) && (QD > 0 || SEGP % KS == 0) && SEGP > (KS - 1) * SEGH,
                  "one, two or four halves split the steps");
    static_assert(NDY <= 64 && NH <= 32, "validity masks");
    static_assert(2 * BUF_BYTES <= 160 * 1024, "two chunk buffers fit the LDS");
    static_assert((SEGP + DYP) * ES < 65536, "LDS immediate offsets");
    static_assert(4 * BM * (BM + 1) * (int)sizeof(typename Pol::Acc) <= 2 * BUF_BYTES, "epilogue stage fits");

    static_assert((KS - 1) * 4 * FM * FN * Pol::NACC * 64 * (int)sizeof(typename Pol::Acc) <= 2 * BUF_BYTES,
                  "partial sums fit in the chunk buffers");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    const int half = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255;               // thread within its half
    const int lane = tid & 63;
    const int wave = tid >> 6;                       // wave within its half
    const int ntl = p.m_tiles * p.n_tiles;
    const int part = split_ch > 0 && (int)blockIdx.x >= ntl ? 1 : 0;   // the reduction part (split launches)
    const int tile = xcd_logical_tile((int)blockIdx.x - part * ntl, ntl, p.tile_rev);
    const int mt = tile / p.n_tiles;
    const int nt = tile - mt * p.n_tiles;
    const int m0 = mt * TM;
    const int n0 = nt * TN;
    const int c_lo = PAIRS ? n0 / S : n0 / RS1;     // first channel (pair) the tile's columns touch

    const int PB = (p.P + PR - 1) / PR;              // row blocks per image
    const int nch_all = p.N * PB;                    // chunks of the whole reduction
    const int ch0 = part ? split_ch : 0;             // this workgroup's chunks [ch0, ch0 + nch)
    const int nch = split_ch > 0 ? (part ? nch_all - split_ch : split_ch) : nch_all;

    // both chunk buffers start zeroed (the planes' spare elements stay so)
    for (int i = (int)threadIdx.x; i < 2 * BUF_BYTES / 16; i += NTT)
        reinterpret_cast<u32x4*>(smem)[i] = u32x4{0, 0, 0, 0};
    __syncthreads();

    // Loads go through range-checked buffer descriptors at 32-bit byte
    // offsets: a piece outside dy or x reads at kWghOutside and gets zero, so
    // the stores carry no masks, and a chunk adds its uniform part as the
    // scalar offset.  (Against masked global loads whose offsets were
    // recomputed per piece and chunk: 4-5x fewer VALU instructions in the
    // step loop; AlexNet conv3 585 -> 418 us, conv4 838 -> 648 us.)
    const int64_t dy_elems = (int64_t)(p.N - 1) * p.sdn + (int64_t)(p.M - 1) * p.sdk + (int64_t)(p.P - 1) * p.sdp +
                             (int64_t)(p.Q - 1) * p.sdq + 1;
    const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.C - 1) * p.sxc + (int64_t)(p.H - 1) * p.sxh +
                            (int64_t)(p.W - 1) * p.sxw + 1;
    const __amdgpu_buffer_rsrc_t dr = wgh_rsrc(p.w, dy_elems * GES);
    const __amdgpu_buffer_rsrc_t xr = wgh_rsrc(p.x, x_elems * GES);

    // ---- DY loader geometry: filter row kr, first position q0, first row rh
    const int ltid = DY_ALL ? (int)threadIdx.x : tid;
    const int kr = ltid / TPK;
    const int q0 = ltid % TPK;
    const int rh = DY_ALL ? 0 : half;
    const bool k_ok = m0 + kr < p.M;
    // piece (row pr, column qj): dy_tb + dy_rowc[pr] + dy_col[qj], each past dy where invalid
    const uint32_t dy_tb = k_ok ? (uint32_t)(((m0 + kr) * p.sdk + rh * p.sdp + q0 * p.sdq) * GES) : kWghOutside;
    uint32_t dy_row[PRH], dy_col[QPT];
#pragma unroll
    for (int i = 0; i < PRH; ++i)
        dy_row[i] = rh + RSTEP * i < PR ? (uint32_t)(RSTEP * i * p.sdp * GES) : kWghOutside;
#pragma unroll
    for (int j = 0; j < QPT; ++j) dy_col[j] = q0 + TPK * j < p.Q ? (uint32_t)(TPK * j * p.sdq * GES) : kWghOutside;

    In dy_val[NDY];
    In h_val[NH];

    // halo pieces, fixed for the tile: byte offset at image 0 and chunk row 0,
    // input row at chunk row 0 (far negative: no piece) and LDS index
    uint32_t h_voff[NH];
    int h_row[NH], h_lds[NH];
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int e = (int)threadIdx.x + NTT * i;
        const int hc = e % WPH;
        const int rowi = e / WPH;
        const int chl = rowi / HROWS;
        const int hr = rowi - chl * HROWS;
        const int w = hc - p.pad_left;
        int c, row;
        if constexpr (PAIRS) {
            const int cr = c_lo + chl;
            c = cr / p.R;
            row = hr * p.u + cr - c * p.R - p.pad_top;       // (p0 * u added per chunk)
        } else {
            c = c_lo + chl;
            row = hr - p.pad_top;                            // (p0 added per chunk)
        }
        const bool ok = e < HU && c < p.C && (unsigned)w < (unsigned)p.W;
        h_row[i] = ok ? row : -(1 << 30);
        h_voff[i] = (uint32_t)((c * p.sxc + w * p.sxw + row * p.sxh) * GES);   // (wraps; valid with a chunk's row)
        h_lds[i] = DY_ELEMS + chl * PLANE + hr * WPH + hc;
    }

    // The next chunk moves global -> registers -> LDS in NL pieces (one
    // element each) spread over the current chunk's MFMA steps: loads over
    // the first half, LDS stores over the second.
    constexpr int NL = NDY + NH;
    int cn = 0, cp0 = 0;                             // the chunk the pieces in flight belong to (image, first row)
    int dy_soff = 0, x_soff = 0, crow = 0;
    uint32_t x_rowoff = 0;
    uint32_t dy_rowc[PRH];
    auto set_chunk = [&](int n, int pr0) {
        cn = n;
        cp0 = pr0;
        dy_soff = (cn * p.sdn + cp0 * p.sdp) * GES;
        x_soff = cn * p.sxn * GES;
        crow = PAIRS ? cp0 * p.u : cp0;
        x_rowoff = (uint32_t)(crow * p.sxh * GES);
#pragma unroll
        for (int i = 0; i < PRH; ++i) dy_rowc[i] = cp0 + rh + RSTEP * i < p.P ? dy_row[i] : kWghOutside;
    };
    auto load_piece = [&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q < NDY) {
            wgh_gload<GIn>(dy_val[q], dr, dy_tb + dy_rowc[q / QPT] + dy_col[q % QPT], dy_soff);
        } else {
            constexpr int i = q - NDY;
            const bool ok = (unsigned)(h_row[i] + crow) < (unsigned)p.H;
            wgh_gload<GIn>(h_val[i], xr, ok ? h_voff[i] + x_rowoff : kWghOutside, x_soff);
        }
    };
    auto store_piece = [&](auto qc, int buf) {
        constexpr int q = decltype(qc)::value;
        In* dyl = reinterpret_cast<In*>(smem + buf * BUF_BYTES);
        if constexpr (q < NDY) {
            constexpr int prs = RSTEP * (q / QPT);
            constexpr int qj = q % QPT;
            // (PR not a multiple of KS leaves the last halves a row short)
            if (DY_ALL || PR % KS == 0 || rh + prs < PR)
                dyl[kr * DYP + rh * WPH + q0 + prs * WPH + TPK * qj] = dy_val[q];
        } else {
            constexpr int i = q - NDY;
            if (HU % NTT == 0 || (int)threadIdx.x + NTT * i < HU) dyl[h_lds[i]] = h_val[i];
        }
    };

    // ---- per-lane operand bases (elements): A = DY row, B = the halo tap of a column
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int lrow = lane % BM;
    const int lgrp = lane / BM;
    // half h takes steps [h * SEGH, (h + 1) * SEGH) of every lane group's segment
    // (QD > 0: the group's first row; the half's steps are compile-time offsets)
    const int pos_base = QD > 0 ? lgrp * WPH : lgrp * SEGP + half * SEGH;
    int a_base[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) a_base[i] = (wm * WM + i * BM + lrow) * DYP + pos_base;
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * BM + lrow;        // past C*R*S: a zero region, masked at the store
        if constexpr (PAIRS) {
            uint32_t cr, s;
            p.div_s.divmod((uint32_t)col, cr, s);
            b_base[j] = DY_ELEMS + ((int)cr - c_lo) * PLANE + (int)s + pos_base;
        } else {
            uint32_t c, rs, r, s;
            p.div_rs.divmod((uint32_t)col, c, rs);
            p.div_s.divmod(rs, r, s);
            b_base[j] = DY_ELEMS + ((int)c - c_lo) * PLANE + (int)r * WPH + (int)s + pos_base;
        }
    }

    AccV acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccV{};

    if (nch > 0) {
        set_chunk(ch0 / PB, (ch0 % PB) * PR);
        unroll_for<0, NL>([&](auto qc) { load_piece(qc); });
        unroll_for<0, NL>([&](auto qc) { store_piece(qc, 0); });
        __syncthreads();
    }
    // offset of step t of half H from the lane's base
    auto step_off = [](auto hc, int t) constexpr {
        constexpr int H = decltype(hc)::value;
        if constexpr (QD > 0) {
            const int u = H * SEGH + t;
            return G * WPH * (u / QD) + u % QD;
        } else {
            return t;
        }
    };
    // operands are read PD steps ahead of their MFMA: more where a step has
    // few MFMAs to cover an LDS read's latency (measured: AlexNet conv2, three
    // per step, 1492 us one step ahead, 1469 two, 1430 three)
    constexpr int PD = FM * FN <= 3 ? 3 : FM * FN <= 4 ? 2 : 1;
    auto run_steps = [&](auto hc, const In* buf, int cur) {
        constexpr int H = decltype(hc)::value;
        constexpr int NSTEP = SEGP - H * SEGH < SEGH ? SEGP - H * SEGH : SEGH;   // this half's steps
        In a[PD + 1][FM], b[PD + 1][FN];             // step t's operands in slot t % (PD + 1)
        auto read_step = [&](auto uc) {
            constexpr int u = decltype(uc)::value;
            if constexpr (u < NSTEP) {
#pragma unroll
                for (int i = 0; i < FM; ++i) a[u % (PD + 1)][i] = buf[a_base[i] + step_off(hc, u)];
#pragma unroll
                for (int j = 0; j < FN; ++j) b[u % (PD + 1)][j] = buf[b_base[j] + step_off(hc, u)];
            }
        };
        unroll_for<0, PD>([&](auto uc) { read_step(uc); });
        unroll_for<0, NSTEP>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            unroll_for<0, NL>([&](auto qc) {
                if constexpr (decltype(qc)::value * (NSTEP / 2) / NL == t) load_piece(qc);
            });
            read_step(std::integral_constant<int, t + PD>{});
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Pol::mfma_s(a[t % (PD + 1)][i], b[t % (PD + 1)][j], acc[i][j]);
            unroll_for<0, NL>([&](auto qc) {
                if constexpr (NSTEP / 2 + decltype(qc)::value * (NSTEP - NSTEP / 2) / NL == t) store_piece(qc, cur ^ 1);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int ch = 0; ch < nch; ++ch) {
        const int cur = ch & 1;
        // the next chunk (past the end: reload, written where nothing reads)
        if (ch + 1 < nch) {
            if (cp0 + PR < p.P)
                set_chunk(cn, cp0 + PR);
            else
                set_chunk(cn + 1, 0);
        }
        const In* buf = reinterpret_cast<const In*>(smem + cur * BUF_BYTES);
        if (QD == 0 || half == 0)
            run_steps(std::integral_constant<int, 0>{}, buf, cur);
        else if (KS == 2 || half == 1)
            run_steps(std::integral_constant<int, 1>{}, buf, cur);
        else if constexpr (KS == 4) {
            if (half == 2)
                run_steps(std::integral_constant<int, 2>{}, buf, cur);
            else
                run_steps(std::integral_constant<int, 3>{}, buf, cur);
        }
        __syncthreads();
    }

    if constexpr (KS > 1) {
        // halves 1 .. KS-1 hand their partial sums to half 0 through LDS,
        // which adds them in half order (a fixed order: no timing dependence)
        typename Pol::Acc* red = reinterpret_cast<typename Pol::Acc*>(smem);
        constexpr int PART = 4 * FM * FN * Pol::NACC * 64;     // one half's partial sums
        auto red_at = [&](int i, int j, int e) { return ((((wave * FM + i) * FN + j) * Pol::NACC + e) << 6) + lane; };
        if (half > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < Pol::NACC; ++e) red[(half - 1) * PART + red_at(i, j, e)] = acc[i][j][e];
        }
        __syncthreads();
        if (half == 0) {
#pragma unroll
            for (int h = 1; h < KS; ++h)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int e = 0; e < Pol::NACC; ++e) acc[i][j][e] += red[(h - 1) * PART + red_at(i, j, e)];
        }
        __syncthreads();
    }
    if (split_ch > 0) {
        // a part's sum times alpha, added into the zeroed packed dw
        static_assert(std::is_same<typename Pol::Acc, typename Pol::Out>::value, "atomic adds in the sum's type");
        using Acc = typename Pol::Acc;
        if (half == 0) {
            Acc* dw = static_cast<Acc*>(p.y);
            const Acc alpha = (Acc)p.alpha;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < Pol::NACC; ++e) {
                    const int gm = m0 + wm * WM + i * BM + Pol::row(e, lane);
                    if (gm >= p.M) continue;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int gk = n0 + wn * WN + j * BM + Pol::col(e, lane);
                        if (gk < p.K) unsafeAtomicAdd(dw + (int64_t)gm * p.syn + gk, alpha * acc[i][j][e]);
                    }
                }
        }
        return;
    }
    store_acc_tile<Pol, FM, FN>(p, smem, acc, m0 + wm * WM, n0 + wn * WN, p.M, wave, lane, half == 0);
}

// dw <- 0 ahead of a split launch (a kernel rather than a memset: callers may
// capture the launch in a graph)
template <class T>
__global__ void __launch_bounds__(256) wgh_zero_kernel(T* __restrict__ y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) y[i] = T(0);
}

template <class Pol, int TM, int TN, int WAVES_M, int WAVES_N, int R, int S, int WPH, int PR, int PLANE, int KS,
          int QD>
static hipError_t launch_wgh_variant(const ConvParams& p0, int split_k, hipStream_t stream)
{
    ConvParams p = p0;
    // R = 0 (pairs): any filter height and row stride
    if ((R > 0 && (p.u != 1 || p.R != R)) || p.v != 1 || p.S != S || p.Q + S - 1 > WPH || (QD > 0 && p.Q != QD))
        return hipErrorInvalidValue;
    // the buffer descriptors' range: x and dy under 2^30 bytes
    constexpr int64_t ES = (int64_t)sizeof(typename wgh_gin<Pol>::type);
    const int64_t dy_elems = (int64_t)(p.N - 1) * p.sdn + (int64_t)(p.M - 1) * p.sdk + (int64_t)(p.P - 1) * p.sdp +
                             (int64_t)(p.Q - 1) * p.sdq + 1;
    const int64_t x_elems = (int64_t)(p.N - 1) * p.sxn + (int64_t)(p.C - 1) * p.sxc + (int64_t)(p.H - 1) * p.sxh +
                            (int64_t)(p.W - 1) * p.sxw + 1;
    if (ES * dy_elems >= ((int64_t)1 << 30) || ES * x_elems >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
    p.m_tiles = (p.M + TM - 1) / TM;
    p.n_tiles = (p.K + TN - 1) / TN;
    const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
    // split_k > 0: the first part takes k / (k + 1) of the chunks (at least
    // one each); with beta = 0 only, and at least two chunks
    if (split_k < 0 || (split_k > 0 && p.beta != 0.0)) return hipErrorInvalidValue;
    const int64_t nch = (int64_t)p.N * ((p.P + PR - 1) / PR);
    int split_ch = 0;
    if (split_k > 0 && nch >= 2 && tiles > 0) {
        const int64_t c = (nch * split_k + (split_k + 1) / 2) / (split_k + 1);
        split_ch = (int)(c < 1 ? 1 : c > nch - 1 ? nch - 1 : c);
        using Acc = typename Pol::Acc;
        const int64_t n = (int64_t)p.M * p.K;
        const int64_t blocks = (n + 255) / 256;
        hipLaunchKernelGGL(wgh_zero_kernel<Acc>, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0,
                           stream, static_cast<Acc*>(p.y), n);
    }
    const dim3 grid((unsigned)(tiles * (split_ch > 0 ? 2 : 1)));
    hipLaunchKernelGGL((conv_bwd_filter_halo_kernel<Pol, TM, TN, WAVES_M, WAVES_N, R, S, WPH, PR, PLANE, KS, QD>),
                       grid, dim3(256 * KS), 0, stream, p, split_ch);
    return hipGetLastError();
}

// row pitch WPH and plane pitch PLANE: the smallest with at most two-way
// (fp64 three-way) bank conflicts on the halo reads, searched offline
// (QD: output rows of exactly QD columns, the steps along them only).
// The 27-column 5x5 form on 64 x 48 tiles takes pitch 40 / plane 333: at
// 32 / 261 its B reads ran up to 5-way conflicts (73% of the LDS cycles
// conflict cycles, measured), and once the loads had stopped bounding the
// kernel the wider rows won (AlexNet conv2 1878 -> 1737 us); pitch 20 on
// the 12-column 3x3 form (2-way -> mostly conflict-free) ran 4% slower.
// 64 x 48 tiles: 256 filters x 2400 columns (96 channels, 5x5) make 200
// tiles instead of 152 of 64 x 64 on the 256 compute units.
//        name                     policy   TM  TN  waves  R  S  WPH  PR  PLANE  KS  QD
#define MICONV_WGH_VARIANTS(X)                                              \
    X(WGH_F32_3x3_W16, PolF32, 64, 64, 2, 2, 3, 3, 16, 13, 243, 2, 0)       \
    X(WGH_F32_5x5_W24, PolF32, 64, 64, 2, 2, 5, 5, 24, 7, 269, 2, 0)        \
    X(WGH_F32_5x5_W36, PolF32, 64, 64, 2, 2, 5, 5, 36, 7, 401, 2, 0)        \
    X(WGH_F32_3x3_W16_64x96, PolF32x16, 64, 96, 2, 2, 3, 3, 16, 13, 247, 2, 0) \
    X(WGH_F32X16_3x3_W16, PolF32x16, 64, 64, 2, 2, 3, 3, 16, 13, 247, 2, 0)     \
    X(WGH_F32X16_5x5_W24, PolF32x16, 64, 64, 2, 2, 5, 5, 24, 7, 269, 2, 0)      \
    X(WGH_F64_3x3_W16, PolF64, 64, 64, 2, 2, 3, 3, 16, 7, 147, 2, 0)            \
    X(WGH_F32_3x3_Q12_64x96, PolF32x16, 64, 96, 2, 2, 3, 3, 16, 12, 247, 2, 12)     \
    X(WGH_F32_3x3_Q13, PolF32, 64, 64, 2, 2, 3, 3, 16, 14, 259, 2, 13)                \
    X(WGH_F32X16_5x5_Q20, PolF32x16, 64, 64, 2, 2, 5, 5, 24, 4, 197, 2, 20)          \
    X(WGH_F32X16_5x5_Q27, PolF32x16, 64, 64, 2, 2, 5, 5, 32, 4, 261, 2, 27)          \
    X(WGH_F32X16_5x5_Q20_64x48, PolF32x16, 64, 48, 4, 1, 5, 5, 24, 4, 197, 2, 20)    \
    X(WGH_F32X16_5x5_Q27_64x48, PolF32x16, 64, 48, 4, 1, 5, 5, 40, 4, 333, 2, 27)   \
    X(WGH_F32_3x3_Q13_KS4, PolF32, 64, 64, 2, 2, 3, 3, 16, 14, 259, 4, 13)            \
    X(WGH_F32_3x3_W16_64x96_KS4, PolF32x16, 64, 96, 2, 2, 3, 3, 16, 13, 247, 4, 0)  \
    X(WGH_F32_3x3_Q12_64x96_KS4, PolF32x16, 64, 96, 2, 2, 3, 3, 16, 12, 247, 4, 12)  \
    X(WGH_F32X16_5x5_Q20_64x48_KS4, PolF32x16, 64, 48, 4, 1, 5, 5, 24, 4, 197, 4, 20) \
    X(WGH_F32X16_5x5_Q27_64x48_KS4, PolF32x16, 64, 48, 4, 1, 5, 5, 32, 4, 261, 4, 27)   \
    X(WGH_F32X16_PAIRS_S11_32x32, PolF32x16, 32, 32, 2, 2, 0, 11, 368, 1, 378, 2, 0)      \
    X(WGH_F32X16_PAIRS_S11_32x32_KS4, PolF32x16, 32, 32, 2, 2, 0, 11, 384, 1, 394, 4, 0)  \
    X(WGH_F32X16_PAIRS_S11_32x64, PolF32x16, 32, 64, 2, 2, 0, 11, 368, 1, 378, 2, 0)      \
    X(WGH_F64_3x3_W16_KS4, PolF64, 64, 64, 2, 2, 3, 3, 16, 7, 147, 4, 0)                  \
    X(WGH_F64_3x3_W16_64x96, PolF64, 64, 96, 2, 2, 3, 3, 16, 7, 147, 2, 0)                \
    X(WGH_BF16_3x3_W16, WghBf16<PolF32>, 64, 64, 2, 2, 3, 3, 16, 13, 243, 2, 0)            \
    X(WGH_BF16_3x3_Q13, WghBf16<PolF32>, 64, 64, 2, 2, 3, 3, 16, 14, 259, 2, 13)           \
    X(WGH_BF16_3x3_W16_64x96_KS4, WghBf16<PolF32x16>, 64, 96, 2, 2, 3, 3, 16, 13, 247, 4, 0)

hipError_t launch_bwd_filter_halo(Variant v, const ConvParams& p, int split_k, hipStream_t stream)
{
    switch (v) {
#define X(name, pol, tm, tn, wmm, wnn, r, s, wph, pr, plane, ks, qd) \
    case Variant::name:                                                 \
        return launch_wgh_variant<pol, tm, tn, wmm, wnn, r, s, wph, pr, plane, ks, qd>(p, split_k, stream);
        MICONV_WGH_VARIANTS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace miconv
