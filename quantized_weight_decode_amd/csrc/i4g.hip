// i4g.hip -- grouped-int4 ("fmt=4") GEMV and decode kernels for gfx950.
//
// Format (colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV support",
// sections 1 and 3): row-major u8[O][(I+1)/2], column 2k in the low nibble of
// byte k, column 2k+1 in the high nibble; f32 scales [O][ceil(I/gs)];
// weight = (q - 8) * scale[row][col/gs].  The scale is applied per group,
// before the sum across groups.
//
// Streaming kernel (rows of 16-byte lane chunks, gs % 32 == 0):
//   * each workgroup stages x once in LDS, per 32-column chunk as a
//     shared-exponent fixed point split into signed 4-bit digits;
//   * a wave covers 64/LPR row groups of R rows; LPR lanes sweep a row in
//     16-byte dwordx4 loads (fully coalesced), the R rows of a lane group share
//     the activation digits they read from LDS, and the next chunks' loads are
//     in flight while the current one is multiplied;
//   * per lane chunk c (32 columns, one group): the integer sum of (q - 8) v
//     comes from 24 hardware 8-way 4-bit dot products, and
//     acc += s_g * 2^(E_c - 21) * sum (q - 8) v;
//   * the row sum is a DPP reduction over the LPR lanes;
//   * a workgroup that meets an infinity or NaN in x, or activations whose
//     dynamic range within a chunk the fixed point cannot carry to the
//     precision bound (stage_verdict), computes its rows with per-element f32
//     products instead (infinities and NaNs then propagate as in the plain
//     definition).
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// Tile shape of the streaming kernel for one vector: rows per lane group,
// waves per workgroup, at most QG_I4G_LPR lanes per row and a ring of
// QG_I4G_PF chunk-sweeps, the first issued before the activations are
// converted.  Measured on the 12288 x 6144 workload (mean of six
// interleaved runs of 300 calls): 32 lanes x 3 rows x 8 waves (256
// workgroups of 48 rows, one per CU, six sweeps per row through a ring of
// two) 8.8 us; the same without the early sweep 9.6 us; 64 lanes x 2 rows x
// 12 waves with all three sweeps in one burst 9.4 us; 32 x 2 x 12 with a
// ring of three, two sweeps early, 8.9 us; 32 x 4 x 6 9.1 us; 16 lanes per
// row 9.8-10.0 us.  The early sweep also helps several vectors per call:
// 15.1 -> 14.1 us at S = 2, 23.6 -> 21.9 us at S = 4.
#ifndef QG_I4G_R
#define QG_I4G_R 3
#endif
#ifndef QG_I4G_WPB
#define QG_I4G_WPB 8
#endif
#ifndef QG_I4G_LPR
#define QG_I4G_LPR 32
#endif
#ifndef QG_I4G_PF
#define QG_I4G_PF 2
#endif
// Waves per workgroup for several vectors: the staged activations take S
// times the LDS, so fewer workgroups fit a CU and each must hold more waves.
// With at most 32 lanes per row (as for one vector), measured on 12288 x
// 6144 with two vectors: 12 waves 11.1 us, 14 waves 12.6 us, 10 waves 18.6
// us, 16 lanes per row 16.5 us; the former 64 lanes x 16 waves 14.6 us.
#ifndef QG_I4G_WPB_MULTI
#define QG_I4G_WPB_MULTI 12
#endif
// Lanes per row for several vectors (at most).  Measured at 12288 x 6144:
// 64 lanes x 4 rows x 12 waves 14.1 / 24.0 us at two / four vectors against
// 11.3 / 19.6 us for 32 x 2 x 12; refilling a ring slot before its products
// instead of after them gained nothing (the products are VALU-bound).
#ifndef QG_I4G_LPR_MULTI
#define QG_I4G_LPR_MULTI 32
#endif

// activation items (8 columns each) each thread loads up front
#ifndef QG_I4G_NPRE
#define QG_I4G_NPRE 2
#endif
// Largest S one streaming launch takes; larger S runs in groups.
constexpr int I4G_FAST_MAX_S = 4;

// Rows row0 .. row0 + R - 1 (those below O) of one lane group, with each
// weight decoded to f32 as (q - 8) * s and multiplied by x read from global
// memory: the plain definition's arithmetic, for activations that hold an
// infinity or NaN.
template <int S, int LPR, int R>
__device__ __noinline__ void i4g_rows_plain(const uint8_t *__restrict__ w,
                                            const float *__restrict__ scales,
                                            const float *__restrict__ x, float *__restrict__ y,
                                            int I, int O, int ng, Div20 div_cpg, int row0, int sl)
{
    const int NU = I / 32;
#pragma unroll 1
    for (int r = 0; r < R; r++) {
        const int row = min(row0 + r, O - 1);
        const uint8_t *wr = w + (size_t)row * (I / 2);
        const float *sr = scales + (size_t)row * ng;
        float acc[S];
#pragma unroll
        for (int t = 0; t < S; t++) acc[t] = 0.0f;
        for (int u = sl; u < NU; u += LPR) {
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(wr + (size_t)u * 16);
            const float sg = sr[div_cpg((uint32_t)u)];
#pragma unroll
            for (int dd = 0; dd < 4; dd++) {
                float e[4], o[4];
                nib8(wv[dd], e, o);
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const float we = (e[k] * NIB_XSCALE - 8.0f) * sg;
                    const float wo = (o[k] * NIB_XSCALE - 8.0f) * sg;
                    const int col = 32 * u + 8 * dd + 2 * k;
#pragma unroll
                    for (int t = 0; t < S; t++) {
                        acc[t] = __builtin_fmaf(we, x[(size_t)t * I + col], acc[t]);
                        acc[t] = __builtin_fmaf(wo, x[(size_t)t * I + col + 1], acc[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < S; t++) {
            const float v = sub_reduce<LPR>(acc[t]);
            if (sl == LPR - 1 && row0 + r < O) y[(size_t)t * O + row0 + r] = v;
        }
    }
}

template <int S, int LPR, int R, int PF, int WPB, int EARLY>
__global__ __launch_bounds__(64 * WPB) void i4g_gemv_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ scales,
    const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, int ntiles)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;                       // lane chunks per row
    u32x4 *xq = reinterpret_cast<u32x4 *>(lds_raw);                        // [S][6][NU]
    float *xc = reinterpret_cast<float *>(xq + (size_t)S * 6 * NU);        // [S][NU]
    void *vlds = lds_raw + q8_verdict_offset(S, NU, false);                // stage_verdict

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const int tile = blockIdx.x * WPB + wave;
    const int row0 = tile * ROWS_PER_WAVE + sub * R;
    const size_t rb = (size_t)I / 2;
    const int nit = (NU + LPR - 1) / LPR;
    const int nit_pad = (nit + PF - 1) / PF * PF;

    const uint8_t *wr[R];
    const float *sr[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = min(row0 + r, O - 1);   // rows past O re-read row O-1, never stored
        wr[r] = w + (size_t)row * rb;
        sr[r] = scales + (size_t)row * ng;
    }

    // Every global load below is unconditional (indices clamped into range),
    // so the compiler can wait for exactly the load a value comes from
    // instead of draining all outstanding loads.
    // 1. activations first (L2-resident)
    XStageQ<S, (S > 2 ? 4 : QG_I4G_NPRE), 64 * WPB> xst;
    const int items = S * NU * 4;
    xst.load(x, items);
    // every wave of the workgroup has issued its activation loads before any
    // wave issues weight loads (raw barrier: no drain)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // 2. weight and scale loads of one chunk-sweep into ring slot j.  The
    //    first EARLY sweeps go out right after the activation loads, before
    //    they are converted, the rest of the ring once the activations are
    //    staged.  One early sweep measured best: issuing the whole first round
    //    early (every wave of the chip at once) delays the activation loads
    //    of later workgroups behind the weight traffic.
    u32x4 wb[PF][R];
    float sb[PF][R];
    auto fetch = [&](int c, int j) {
        const int u = min(c * LPR + sl, NU - 1);
        const uint32_t g = div_cpg((uint32_t)u);
#pragma unroll
        for (int r = 0; r < R; r++) {
            wb[j][r] = ld_stream(reinterpret_cast<const u32x4 *>(wr[r] + (uint32_t)u * 16u));
            sb[j][r] = ld_stream(&sr[r][g]);
        }
    };
#pragma unroll
    for (int j = 0; j < EARLY; j++) fetch(j, j);
    __builtin_amdgcn_sched_barrier(0);
    // 3. activations into LDS as fixed-point digits
    const uint32_t bad = xst.store(x, items, NU, reinterpret_cast<uint32_t *>(xq), xc, nullptr);
    // non-finite activations, or a dynamic range the fixed point cannot
    // carry precisely enough: the plain per-element products instead
    const int plain = stage_verdict<WPB, S>(bad, xst.dsum, vlds);
    if (tile >= ntiles) return;
    if (plain) {
        i4g_rows_plain<S, LPR, R>(w, scales, x, y, I, O, ng, div_cpg, row0, sl);
        return;
    }
#pragma unroll
    for (int j = EARLY; j < PF; j++) fetch(j, j);
    __builtin_amdgcn_sched_barrier(0);

    float acc[S][R];
#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[t][r] = 0.0f;
    // running digit sums per vector and row (see q8_dot_run), so no
    // accumulator is cleared per chunk, where the registers allow; otherwise
    // fresh sums per chunk
    constexpr bool RUN = S * R <= 8;
    constexpr int SR = RUN ? S : 1;
    uint32_t P[SR][R][6], V[SR][R];
#pragma unroll
    for (int t = 0; t < SR; t++)
#pragma unroll
        for (int r = 0; r < R; r++) {
            V[t][r] = 0;
#pragma unroll
            for (int k = 0; k < 6; k++) P[t][r][k] = 0;
        }

    // 4. sweep in rounds of PF chunk-sweeps: consume ring slot j, then refill
    //    it with the sweep one round ahead.  All refills are unconditional
    //    (clamped) and pinned in place, so every wait is for exactly the slot
    //    about to be used; the last round issues no refills.  Padding sweeps
    //    past the row end are multiplied by a zero chunk scale.
    auto consume = [&](int c, int j) {
        const int u = c * LPR + sl;
        const bool valid = u < NU;
        const int uu = valid ? u : 0;
        uint32_t wx[R][4];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int d = 0; d < 4; d++) wx[r][d] = wb[j][r][d] ^ Q8_NIB_FLIP;
#pragma unroll
        for (int t = 0; t < S; t++) {
            const u32x4 *xt = xq + (size_t)t * 6 * NU;
            u32x4 L[6];
#pragma unroll
            for (int k = 0; k < 6; k++) L[k] = xt[k * NU + uu];
            const float cs = valid ? xc[(size_t)t * NU + uu] : 0.0f;
#pragma unroll
            for (int r = 0; r < R; r++) {
                int dv;
                if constexpr (RUN) dv = q8_dot_run(wx[r], L, P[t][r], V[t][r]);
                else dv = q8_dot(wx[r], L);
                acc[t][r] = __builtin_fmaf(sb[j][r] * cs, (float)dv, acc[t][r]);
            }
            if constexpr (S > 1) pin_values(acc[t]);   // one vector's digits live at a time
        }
    };
    const int nrounds = nit_pad / PF;
    for (int rd = 0; rd + 1 < nrounds; rd++) {
#pragma unroll
        for (int j = 0; j < PF; j++) {
            const int c = rd * PF + j;
            consume(c, j);
#pragma unroll
            for (int t = 0; t < S; t++) pin_values(acc[t]);
            fetch(c + PF, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < PF; j++) {
        consume((nrounds - 1) * PF + j, j);
#pragma unroll
        for (int t = 0; t < S; t++) pin_values(acc[t]);   // one slot at a time, as in the loop
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float v = sub_reduce<LPR>(acc[t][r]);
            if (sl == LPR - 1 && row0 + r < O) y[(size_t)t * O + row0 + r] = v;
        }
}

// General kernel: any I >= 1, any even gs, S <= QGEMV_MAX_S, any alignment of
// w.  One wave per row; each lane takes bytes lane, lane+64, ...; each weight
// is decoded to f32 as (q - 8) * s (one rounding) and multiplied in f32.
__global__ __launch_bounds__(256) void i4g_gemv_general(
    const uint8_t *__restrict__ w, const float *__restrict__ scales,
    const float *__restrict__ x, float *__restrict__ y, int S, int I, int O, int gs)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= O) return;
    const int rb = (I + 1) / 2;
    const int ng = (I + gs - 1) / gs;
    const uint8_t *wr = w + (size_t)row * rb;
    const float *sr = scales + (size_t)row * ng;
    float acc[QGEMV_MAX_S];
#pragma unroll
    for (int t = 0; t < QGEMV_MAX_S; t++) acc[t] = 0.0f;
    for (int k = lane; k < rb; k += WAVE) {
        float e[4], o[4];
        nib8((uint32_t)wr[k], e, o);
        const int c0 = 2 * k, c1 = 2 * k + 1;
        const float w0 = (e[0] * NIB_XSCALE - 8.0f) * sr[c0 / gs];
        const float w1 = c1 < I ? (o[0] * NIB_XSCALE - 8.0f) * sr[c1 / gs] : 0.0f;
#pragma unroll
        for (int t = 0; t < QGEMV_MAX_S; t++) {
            if (t < S) {
                const float *xt = x + (size_t)t * I;
                acc[t] = __builtin_fmaf(w0, xt[c0], acc[t]);
                if (c1 < I) acc[t] = __builtin_fmaf(w1, xt[c1], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < QGEMV_MAX_S; t++) {
        if (t < S) {
            const float v = sub_reduce<64>(acc[t]);
            if (lane == 63) y[(size_t)t * O + row] = v;
        }
    }
}

// Decode-only: W[o][i] = (q - 8) * s as f32, with the GEMVs' nibble decoder.
__global__ __launch_bounds__(256) void i4g_dequant(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, float *__restrict__ W,
    int I, int O, int gs)
{
    const int rb = (I + 1) / 2;
    const int ng = (I + gs - 1) / gs;
    const size_t n = (size_t)O * rb;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t o = idx / rb;
        const int k = (int)(idx - o * rb);
        float e[4], od[4];
        nib8((uint32_t)w[idx], e, od);
        const int c0 = 2 * k, c1 = 2 * k + 1;
        W[o * I + c0] = (e[0] * NIB_XSCALE - 8.0f) * scales[o * ng + c0 / gs];
        if (c1 < I) W[o * I + c1] = (od[0] * NIB_XSCALE - 8.0f) * scales[o * ng + c1 / gs];
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

// lanes per row: the fullest sweep, at most QG_I4G_LPR (one vector) or
// QG_I4G_LPR_MULTI (several)
// Lanes per row (pick_lpr_wide).  i4g: 3584 x 18944 17.9 -> 11.4 us, 5120 x
// 13824 14.1 -> 11.1 us, 1024 x 4352 8.8 -> 4.0 us; 18944 x 3584 3 % slower;
// 12288 x 6144 and other rows of whole 64-chunk sweeps unchanged.
inline int i4g_lanes_per_row(int I, int S = 1)
{
    const int lpr = pick_lpr_wide(I / 32);
    const int cap = S == 1 ? QG_I4G_LPR : QG_I4G_LPR_MULTI;
    return lpr > cap ? cap : lpr;
}

template <int S, int LPR, int R, int PF>
hipError_t launch_stream_t(const uint8_t *w, const float *s, const float *x, float *y,
                           int I, int O, int gs, hipStream_t st)
{
    const int ng = (I + gs - 1) / gs;
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    const int ntiles = (O + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    constexpr int WPB = S == 1 ? QG_I4G_WPB : QG_I4G_WPB_MULTI;
    const int waves_per_block = WPB;
    const int blocks = (ntiles + waves_per_block - 1) / waves_per_block;
    const size_t lds = i4g_stream_lds_bytes(S, I);
    auto kern = i4g_gemv_stream<S, LPR, R, PF, WPB, 1>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * waves_per_block), lds, st, w, s, x, y,
                       I, O, ng, Div20::make((uint32_t)(gs / 32)), ntiles);
    return hipGetLastError();
}

template <int S, int LPR, int R>
hipError_t launch_stream_pf(const uint8_t *w, const float *s, const float *x, float *y, int I,
                            int O, int gs, hipStream_t st)
{
    // several vectors: 16-wave workgroups leave 128 registers per lane, so
    // two sweeps in flight; one vector: a ring of QG_I4G_PF sweeps
    return launch_stream_t<S, LPR, R, (S > 1 ? 2 : QG_I4G_PF)>(w, s, x, y, I, O, gs, st);
}

template <int S, int R>
hipError_t launch_stream_r(const uint8_t *w, const float *s, const float *x, float *y, int I,
                           int O, int gs, hipStream_t st)
{
    const int lpr = i4g_lanes_per_row(I, S);
    switch (lpr) {
    case 64: return launch_stream_pf<S, 64, R>(w, s, x, y, I, O, gs, st);
    case 32: return launch_stream_pf<S, 32, R>(w, s, x, y, I, O, gs, st);
    case 16: return launch_stream_pf<S, 16, R>(w, s, x, y, I, O, gs, st);
    case 8: return launch_stream_pf<S, 8, R>(w, s, x, y, I, O, gs, st);
    default: return launch_stream_pf<S, 4, R>(w, s, x, y, I, O, gs, st);
    }
}

template <int S>
hipError_t launch_stream_s(const uint8_t *w, const float *s, const float *x, float *y,
                           int I, int O, int gs, hipStream_t st)
{
    // R rows of a lane group share each activation read from LDS
    if constexpr (S == 1) {
        // QG_I4G_R rows per lane group, or two where that puts fewer rows on
        // the busiest CU, or one where that puts fewer still and leaves at
        // most one workgroup per CU.  Measured at 6144 columns: 12288 rows
        // 8.97 (R = 3) against 9.76 us (R = 2); 16384 rows 13.2 against 11.1
        // us; 32768 rows 20.6 against 19.9 us; 65536 rows 39.2 against 36.3
        // us; 4096 rows 5.89 (R = 2) against 5.44 us (R = 1), 1024 rows 5.63
        // against 4.96 us.  Where one-row tiles would put several workgroups
        // on a CU, each staging x, they lose: 28672 x 8192 32.2 us (R = 1)
        // against 25.9 us (R = 2); and on a tie R = 3 wins: 18432 x 7168
        // 15.96 us against 17.52 us (R = 2).
        const long ncu = cu_count();
        // Few rows -- at most one workgroup per CU with 32-lane one-row
        // tiles -- on rows of at least 64 lane chunks: 64 lanes per row (twice
        // the waves) and a ring of four sweeps (twice the bytes in flight per
        // wave), one row per lane group where that leaves at most one
        // workgroup per CU, else two.  2048 x 14336 8.9 -> 6.6 us, 1024 x
        // 28672 15.2 -> 9.8 us, 1536 x 16384 9.8 -> 6.8 us, 4096 x 6144 5.39
        // -> 5.24 us, 4096 x 14336 9.43 -> 9.21 us; and for any row of at
        // least 64 chunks, whatever width the rule above gives it: 2048 x 7168
        // 5.7 -> 4.7 us, 1536 x 7168 5.7 -> 4.6 us, 2048 x 2176 11.5 -> 4.0 us.
        // With more rows the 32-lane tiles stay ahead (12288 x 6144: 10.9 us
        // this way).
        if (I / 32 >= 64 && (O + 2L * QG_I4G_WPB - 1) / (2L * QG_I4G_WPB) <= ncu) {
            if ((O + QG_I4G_WPB - 1) / QG_I4G_WPB <= ncu)
                return launch_stream_t<S, 64, 1, 4>(w, s, x, y, I, O, gs, st);
            return launch_stream_t<S, 64, 2, 4>(w, s, x, y, I, O, gs, st);
        }
        auto rows_wg = [&](int r) { return (long)QG_I4G_WPB * (64 / i4g_lanes_per_row(I)) * r; };
        auto wgs = [&](int r) { return (O + rows_wg(r) - 1) / rows_wg(r); };
        auto busiest = [&](int r) { return (wgs(r) + ncu - 1) / ncu * rows_wg(r); };
        if (QG_I4G_R > 2 && busiest(2) < busiest(QG_I4G_R)) {
            if (wgs(1) <= ncu && busiest(1) < busiest(2))
                return launch_stream_r<S, 1>(w, s, x, y, I, O, gs, st);
            return launch_stream_r<S, 2>(w, s, x, y, I, O, gs, st);
        }
        return launch_stream_r<S, QG_I4G_R>(w, s, x, y, I, O, gs, st);
    } else {
        // several vectors: the staged activations take S times the LDS, so
        // few workgroups fit a CU; R keeps them all resident, ties going to
        // the larger R (fewer workgroups staging the vectors).  12288 rows,
        // two to four vectors: R = 2, 256 workgroups of 48 rows
        static const int cand[] = {3, 2, 1};
        switch (pick_rows_per_group(O, i4g_lanes_per_row(I, S), QG_I4G_WPB_MULTI,
                                    i4g_stream_lds_bytes(S, I), cand, 3)) {
        case 1: return launch_stream_r<S, 1>(w, s, x, y, I, O, gs, st);
        case 2: return launch_stream_r<S, 2>(w, s, x, y, I, O, gs, st);
        default: return launch_stream_r<S, 3>(w, s, x, y, I, O, gs, st);
        }
    }
}

}  // namespace

size_t i4g_stream_lds_bytes(int S, int I)
{
    return q8_verdict_offset(S, I / 32, false) + verdict_bytes(16, S);
}

int i4g_stream_vectors(const void *w, const float *x, int S, int I, int gs)
{
    if (I % 32 != 0 || gs % 32 != 0 || ((uintptr_t)w & 15) != 0 || ((uintptr_t)x & 15) != 0)
        return 0;
    int n = S < I4G_FAST_MAX_S ? S : I4G_FAST_MAX_S;
    while (n > 0 && i4g_stream_lds_bytes(n, I) > LDS_BUDGET) --n;
    return n;
}

hipError_t launch_i4g_gemv(const void *w, const float *scales, const float *x, float *y,
                           int S, int I, int O, int gs, hipStream_t st)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    // vectors per streaming launch; more vectors than one launch takes are
    // done in groups (each group streams the weights once)
    const int nmax = i4g_stream_vectors(w, x, S, I, gs);
    if (nmax > 0) {
        for (int s0 = 0; s0 < S; s0 += nmax) {
            const int n = S - s0 < nmax ? S - s0 : nmax;
            const float *xs = x + (size_t)s0 * I;
            float *ys = y + (size_t)s0 * O;
            hipError_t e;
            switch (n) {
            case 1: e = launch_stream_s<1>(wb, scales, xs, ys, I, O, gs, st); break;
            case 2: e = launch_stream_s<2>(wb, scales, xs, ys, I, O, gs, st); break;
            case 3: e = launch_stream_s<3>(wb, scales, xs, ys, I, O, gs, st); break;
            default: e = launch_stream_s<4>(wb, scales, xs, ys, I, O, gs, st); break;
            }
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int wpb = 4;
    hipLaunchKernelGGL(i4g_gemv_general, dim3((O + wpb - 1) / wpb), dim3(64 * wpb), 0, st, wb,
                       scales, x, y, S, I, O, gs);
    return hipGetLastError();
}

hipError_t launch_i4g_dequant(const void *w, const float *scales, float *W, int I, int O,
                              int gs, hipStream_t st)
{
    const size_t n = (size_t)O * ((I + 1) / 2);
    const int threads = 256;
    const size_t want = (n + threads - 1) / threads;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(i4g_dequant, dim3(blocks), dim3(threads), 0, st,
                       static_cast<const uint8_t *>(w), scales, W, I, O, gs);
    return hipGetLastError();
}

}  // namespace qg
