// i4g.hip -- grouped-int4 ("fmt=4") GEMV and decode kernels for gfx950.
//
// Format (colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV support",
// sections 1 and 3): row-major u8[O][(I+1)/2], column 2k in the low nibble of
// byte k, column 2k+1 in the high nibble; f32 scales [O][ceil(I/gs)];
// weight = (q - 8) * scale[row][col/gs].  The scale is applied per group,
// before the sum across groups.
//
// Streaming kernel (rows of 16-byte lane chunks, gs % 32 == 0):
//   * each workgroup stages x (permuted, with per-chunk sums) in LDS once;
//   * a wave covers 64/LPR row groups of R rows; LPR lanes sweep a row in
//     16-byte dwordx4 loads (fully coalesced), the R rows of a lane group share
//     the activations they read from LDS, and the next chunk's loads are in
//     flight while the current one is decoded;
//   * per lane chunk c (32 columns, one group): P = sum q*x, then
//     acc += s_g * (P - 8 * sum x), which is sum (q - 8) s_g x reassociated;
//   * the row sum is a DPP reduction over the LPR lanes.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// Tile shape of the streaming kernel for S <= 2: rows per lane group and
// waves per workgroup.
#ifndef QG_I4G_R
#define QG_I4G_R 4
#endif
#ifndef QG_I4G_WPB
#define QG_I4G_WPB 4
#endif
// Waves per workgroup for several vectors: the staged activations take S
// times the LDS, so fewer workgroups fit a CU and each must hold more waves.
#ifndef QG_I4G_WPB_MULTI
#define QG_I4G_WPB_MULTI 16
#endif

// chunk-sweeps issued before the activations are staged (at most PF)
#ifndef QG_I4G_PF0
#define QG_I4G_PF0 0
#endif

// Largest S one streaming launch takes; larger S runs in groups.
constexpr int I4G_FAST_MAX_S = 4;

template <int S, int LPR, int R, int PF, int WPB>
__global__ __launch_bounds__(64 * WPB) void i4g_gemv_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ scales,
    const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, int ntiles)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    constexpr int PF0 = QG_I4G_PF0 < PF ? QG_I4G_PF0 : PF;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;                       // lane chunks per row
    f32x4 *xl = reinterpret_cast<f32x4 *>(lds_raw);                  // [S][8][NS]
    float *xs = reinterpret_cast<float *>(xl + (size_t)S * 8 * seg_stride(NU));  // [S][NU]

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
    XStageN<S, 6, 64 * WPB> xst;
    const int total4 = S * NU * 8;
    xst.load(x, total4);
    // every wave of the workgroup has issued its activation loads before any
    // wave issues weight loads (raw barrier: no drain)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // 2. the first PF0 chunk-sweeps of weights and scales.  Only a few: the
    //    memory system serves a flood of streaming weight requests ahead of
    //    the isolated activation reads, so the stream is held back until the
    //    activations have arrived, with just enough weight traffic in flight
    //    to keep HBM busy meanwhile.
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
    for (int j = 0; j < PF0; j++) fetch(j, j);

    // 3. activations into LDS (permuted, chunk sums), then the rest of the
    //    first round of weights
    __builtin_amdgcn_sched_barrier(0);
    xst.store(x, total4, NU, xl, xs);
    __syncthreads();
    if (tile >= ntiles) return;
#pragma unroll
    for (int j = PF0; j < PF; j++) fetch(j, j);
    __builtin_amdgcn_sched_barrier(0);

    float acc[S][R];
#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[t][r] = 0.0f;

    // 4. sweep in rounds of PF chunk-sweeps: consume ring slot j, then refill
    //    it with the sweep one round ahead.  All refills are unconditional
    //    (clamped) and pinned in place, so every wait is for exactly the slot
    //    about to be used; the last round issues no refills.  Padding sweeps
    //    past the row end add zero.
    auto consume = [&](int c, int j) {
        const int u = c * LPR + sl;
        const bool valid = u < NU;
        const int uu = valid ? u : 0;
        if constexpr (S == 1) {
            const float m8xs = -8.0f * xs[uu];
#pragma unroll
            for (int r = 0; r < R; r++) {
                // s * (sum q x - 8 sum x); the chunk dot comes out as 2^-9 sum q x
                const float p = nib_chunk_dot(wb[j][r], xl, NU, uu);
                const float tv = __builtin_fmaf(p, NIB_XSCALE, m8xs);
                acc[0][r] = __builtin_fmaf(valid ? sb[j][r] : 0.0f, tv, acc[0][r]);
            }
        } else {
            // Several vectors: the select form below makes the compiler run
            // each (vector, row) dot under its own lane mask, one after the
            // other.  Written as a multiply by a zeroed scale, every vector's
            // activations and every row's decode get scheduled up front,
            // which takes the whole register file (one wave per SIMD).
#pragma unroll
            for (int t = 0; t < S; t++) {
                const f32x4 *xt = xl + (size_t)t * 8 * seg_stride(NU);
                const float m8xs = -8.0f * xs[(size_t)t * NU + uu];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float p = nib_chunk_dot(wb[j][r], xt, NU, uu);
                    const float tv = __builtin_fmaf(p, NIB_XSCALE, m8xs);
                    acc[t][r] = valid ? __builtin_fmaf(sb[j][r], tv, acc[t][r]) : acc[t][r];
                }
            }
        }
    };
    const int nrounds = nit_pad / PF;
    for (int rd = 0; rd + 1 < nrounds; rd++) {
#pragma unroll
        for (int j = 0; j < PF; j++) {
            const int c = rd * PF + j;
            consume(c, j);
            fetch(c + PF, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < PF; j++) {
        consume((nrounds - 1) * PF + j, j);
        __builtin_amdgcn_sched_barrier(0);   // one slot at a time, as in the loop
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

template <int S, int LPR, int R, int PF>
hipError_t launch_stream_t(const uint8_t *w, const float *s, const float *x, float *y,
                           int I, int O, int gs, hipStream_t st)
{
    const int NU = I / 32;
    const int ng = (I + gs - 1) / gs;
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    const int ntiles = (O + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    constexpr int WPB = S == 1 ? QG_I4G_WPB : QG_I4G_WPB_MULTI;
    const int waves_per_block = WPB;
    const int blocks = (ntiles + waves_per_block - 1) / waves_per_block;
    const size_t lds = i4g_stream_lds_bytes(S, I);
    auto kern = i4g_gemv_stream<S, LPR, R, PF, WPB>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * waves_per_block), lds, st, w, s, x, y,
                       I, O, ng, Div20::make((uint32_t)(gs / 32)), ntiles);
    return hipGetLastError();
}

// chunk sweeps in flight per lane: the depth in {2, 3, 4} that leaves the
// fewest padded sweeps (ties go to the deeper ring)
inline int pick_pf(int nit)
{
    int best = 4, best_pad = 1 << 30;
    for (int pf : {4, 3, 2}) {
        const int pad = (nit + pf - 1) / pf * pf - nit;
        if (pad < best_pad) { best_pad = pad; best = pf; }
    }
    return best;
}

template <int S, int LPR, int R>
hipError_t launch_stream_pf(const uint8_t *w, const float *s, const float *x, float *y, int I,
                            int O, int gs, hipStream_t st)
{
    // several vectors: 16-wave workgroups leave 128 registers per lane, so
    // two sweeps in flight
    if constexpr (S > 1) {
        return launch_stream_t<S, LPR, R, 2>(w, s, x, y, I, O, gs, st);
    } else {
        switch (pick_pf((I / 32 + LPR - 1) / LPR)) {
        case 2: return launch_stream_t<S, LPR, R, 2>(w, s, x, y, I, O, gs, st);
        case 3: return launch_stream_t<S, LPR, R, 3>(w, s, x, y, I, O, gs, st);
        default: return launch_stream_t<S, LPR, R, 4>(w, s, x, y, I, O, gs, st);
        }
    }
}

template <int S, int R>
hipError_t launch_stream_r(const uint8_t *w, const float *s, const float *x, float *y, int I,
                           int O, int gs, hipStream_t st)
{
    switch (pick_lpr(I / 32)) {
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
        return launch_stream_r<S, QG_I4G_R>(w, s, x, y, I, O, gs, st);
    } else {
        // several vectors: the staged activations take S times the LDS, so
        // few workgroups fit a CU; R keeps them all resident (12288 rows,
        // S = 2 or 4: R = 3, 256 workgroups of 48 rows)
        static const int cand[] = {1, 2, 3};
        switch (pick_rows_per_group(O, pick_lpr(I / 32), QG_I4G_WPB_MULTI,
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
    return (size_t)S * ((size_t)8 * seg_stride(I / 32) * sizeof(f32x4) + (I / 32) * sizeof(float));
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
