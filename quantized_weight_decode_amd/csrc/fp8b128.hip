// fp8b128.hip -- fp8-e4m3 GEMV with 128x128 block scales ("fmt=7") for gfx950.
//
// Format ("fmt=7: fp8-e4m3-b128 passthrough weight format", section
// "Design"): row-major u8[O][I] OCP E4M3-FN codes; f32 scale per 128x128
// block in row-major block order; weight = e4m3(code) * scale (a multiply).
//
// Streaming kernel (I % 16 == 0, 16-byte aligned rows):
//   * x is staged once per workgroup in LDS as float4 segments k = 0..3 of
//     each 16-column lane chunk u, stored at float4 index k * NU + u (lanes on
//     consecutive chunks read consecutive LDS words);
//   * a lane group of LPR lanes sweeps R consecutive rows with dwordx4 loads;
//     the R rows share one 128-row band, so one block scale per chunk serves
//     all of them; E4M3 pairs go through the hardware pair converter (exact,
//     OCP semantics: NaN only for 0x7F/0xFF, subnormals, -0);
//   * acc += scale_block * sum_16(w * x); the row sum is a DPP reduction.
#include "qg_device.h"
#include "qg_launch.h"

// Tile shape of the streaming kernel: R rows per lane group, PF sweeps in
// flight, WPB waves per workgroup.  At O = 7168, I = 16384 the 3584 two-row
// waves form 512 workgroups, two per CU (two 64 KB activation copies fit the
// LDS), so every CU gets the same share.
#ifndef QG_FP8_R
#define QG_FP8_R 2
#endif
#ifndef QG_FP8_PF
#define QG_FP8_PF 4
#endif
#ifndef QG_FP8_WPB
#define QG_FP8_WPB 7
#endif
// the alternative one-vector workgroup size (see launch_s), for rows of at
// least QG_FP8_WPB2_MIN_I columns
#ifndef QG_FP8_WPB2
#define QG_FP8_WPB2 8
#endif
#ifndef QG_FP8_WPB2_MIN_I
#define QG_FP8_WPB2_MIN_I 4096
#endif
// waves per workgroup for several vectors (S times the LDS per workgroup)
#ifndef QG_FP8_WPB_MULTI
#define QG_FP8_WPB_MULTI 16
#endif
// sweeps issued before the activations are staged (at most PF).  Unlike the
// nibble formats, the fp8 stream is faster with most of its first round of
// weight loads in flight while the (larger) activation vector is staged.
// Three of a ring of four, against all four (interleaved, three runs, one
// vector): 7168 x 16384 unchanged, 4096 x 7168 -2.3 %, 2048 x 16384 -1.3 %,
// 18432 x 7168 -1.3 %, 12288 x 7168 -1.2 %, 3072 x 7168 -3.1 %, 2048 x 7168
// +1.8 %, 4096 x 16384 +1.1 %; several vectors within 0.5 %.  One or two
// were slower.
#ifndef QG_FP8_PF0
#define QG_FP8_PF0 3
#endif

// activation float4s each thread loads up front (the rest follow one round
// trip later); ten, covering a 16384-column vector with 7 waves in one round
// trip, measured no faster than eight (21.2 against 21.1 us)
#ifndef QG_FP8_NPRE
#define QG_FP8_NPRE 8
#endif

namespace qg {

constexpr int FP8_FAST_MAX_S = 4;

// Stages up to 8 vectors into the fp8 LDS layout with coalesced float4 loads
// (thread f reads float4 number f, from the offset stage_rot picks); the
// first NPRE float4s per thread are loaded unconditionally (indices clamped)
// so later waits count exactly.  The staged columns are the NU chunks from
// float4 off4 of each vector (vectors xs4 float4s apart): a column phase of
// a row too long to stage at once, or the whole row.
template <int NPRE, int NT>
struct XStageF8 {
    f32x4 v[NPRE];
    int rot;

    // global float4 index of the g-th staged float4 (PH: a column phase;
    // otherwise whole rows, where it is g itself)
    template <bool PH>
    __device__ __forceinline__ static uint32_t src(int g, int NU, int xs4, int off4)
    {
        if constexpr (!PH) return (uint32_t)g;
        int t, rem;
        split_f<8>(g, NU * 4, t, rem);
        return (uint32_t)(t * xs4 + off4 + rem);
    }

    template <bool PH>
    __device__ __forceinline__ void load(const float *__restrict__ x, int total, int NU, int xs4,
                                         int off4)
    {
        rot = stage_rot(total);
#pragma unroll
        for (int j = 0; j < NPRE; j++)
            v[j] = ldx4(x, src<PH>(stage_index((int)threadIdx.x + j * NT, total, rot), NU, xs4,
                                   off4));
    }

    // g is the float4 index read for the workgroup's f-th read.  Out-of-range
    // f writes the spare float4 after the staged vectors, so the store (and
    // the load feeding it) is unconditional.
    __device__ __forceinline__ static void put(f32x4 a, int f, int g, int total, int NU,
                                               f32x4 *__restrict__ xl)
    {
        int t, rem;
        split_f<8>(g, NU * 4, t, rem);
        const size_t NS = (size_t)seg_stride(NU);
        const size_t idx = f < total ? (size_t)t * 4 * NS + (size_t)(rem & 3) * NS + (rem >> 2)
                                     : (size_t)(total / (4 * NU)) * 4 * NS;
        xl[idx] = a;
    }

    template <bool PH>
    __device__ __forceinline__ void store(const float *__restrict__ x, int total, int NU,
                                          int xs4, int off4, f32x4 *__restrict__ xl)
    {
#pragma unroll
        for (int j = 0; j < NPRE; j++) {
            const int f = (int)threadIdx.x + j * NT;
            put(v[j], f, stage_index(f, total, rot), total, NU, xl);
        }
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
        for (int f = (int)threadIdx.x + NPRE * NT; f < total; f += NT) {
            const int g = stage_index(f, total, rot);
            put(x4[src<PH>(g, NU, xs4, off4)], f, g, total, NU, xl);
        }
    }
};

// Block scale value: an f32 as stored, or a UE8M0 byte read as 2^(e - 127)
// (e = 0 is the f32 subnormal 2^-127, e = 255 is NaN).
__device__ __forceinline__ float scale_value(float s) { return s; }
__device__ __forceinline__ float scale_value(uint8_t e)
{
    const float v = __builtin_bit_cast(float, (uint32_t)e << 23);
    return e == 0 ? __builtin_bit_cast(float, 0x00400000u) : (e == 255 ? __builtin_nanf("") : v);
}

// sum over the 16 columns of one lane chunk of e4m3(w) * x
__device__ __forceinline__ float fp8_chunk_dot(const u32x4 wv, const f32x4 *__restrict__ xl,
                                               int NU, int u)
{
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        float v[4];
        e4m3x4(wv[d], v);
        const f32x4 xv = xl[(size_t)d * seg_stride(NU) + u];
        p0 = __builtin_fmaf(v[0], xv.x, p0);
        p1 = __builtin_fmaf(v[1], xv.y, p1);
        p0 = __builtin_fmaf(v[2], xv.z, p0);
        p1 = __builtin_fmaf(v[3], xv.w, p1);
    }
    return p0 + p1;
}

template <typename ST, int S, int LPR, int R, int PF, int WPB, bool PH>
__global__ __launch_bounds__(64 * WPB) void fp8_gemv_stream(
    const uint8_t *__restrict__ w, const ST *__restrict__ sc, const float *__restrict__ x,
    float *__restrict__ y, int I, int O, int nbi, int ntiles, int NUP)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    constexpr int PF0 = QG_FP8_PF0 < PF ? QG_FP8_PF0 : PF;
    static_assert(128 % R == 0, "a lane group's rows must share one 128-row band");
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NUA = I / 16;                            // lane chunks per row
    f32x4 *xl = reinterpret_cast<f32x4 *>(lds_raw);   // [S][4][NS] + 1 spare

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const int tile = blockIdx.x * WPB + wave;
    const int row0 = tile * ROWS_PER_WAVE + sub * R;
    const ST *scrow = sc + (size_t)(min(row0, O - 1) / 128) * nbi;
    const uint8_t *wr[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        wr[r] = w + (size_t)min(row0 + r, O - 1) * I;

    float acc[S][R];
#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[t][r] = 0.0f;

    // PH: column phases of NUP chunks, each staging its columns of every
    // vector, then streaming them for the workgroup's rows; the sums run on
    // across phases, so every weight byte is still read once.  Otherwise
    // one phase of whole rows.
    auto phase = [&](int c0, int NU) {
        const int nit = (NU + LPR - 1) / LPR;
        const int nit_pad = (nit + PF - 1) / PF * PF;
        if (PH && c0 > 0) __syncthreads();   // every wave is done with the previous phase

        // activations first; every load unconditional
        XStageF8<QG_FP8_NPRE, 64 * WPB> xst;
        const int total4 = S * NU * 4;
        xst.template load<PH>(x, total4, NU, I / 4, c0 * 4);
        // every wave of the workgroup has issued its activation loads before
        // any wave issues weight loads (raw barrier: no drain)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // only PF0 sweeps go out before the activations are staged: a flood
        // of streaming weight requests is served ahead of the activation reads
        u32x4 wb[PF][R];
        float sb[PF];
        auto fetch = [&](int c, int j) {
            const int u = c0 + min(c * LPR + sl, NU - 1);
#pragma unroll
            for (int r = 0; r < R; r++)
                wb[j][r] = ld_stream(reinterpret_cast<const u32x4 *>(wr[r] + (size_t)u * 16));
            sb[j] = scale_value(ld_stream(&scrow[u >> 3]));
        };
#pragma unroll
        for (int j = 0; j < PF0; j++) fetch(j, j);

        __builtin_amdgcn_sched_barrier(0);
        xst.template store<PH>(x, total4, NU, I / 4, c0 * 4, xl);
        __syncthreads();
        // waves past the last row helped stage; with one phase they are done,
        // with several they run every phase (clamped rows, nothing stored) to
        // reach each phase's barriers
        if (!PH && tile >= ntiles) return false;
#pragma unroll
        for (int j = PF0; j < PF; j++) fetch(j, j);
        __builtin_amdgcn_sched_barrier(0);

        auto consume = [&](int c, int j) {
            const int u = c * LPR + sl;
            const bool valid = u < NU;
            const int uu = valid ? u : 0;
            const float s = valid ? sb[j] : 0.0f;
#pragma unroll
            for (int t = 0; t < S; t++) {
                const f32x4 *xt = xl + (size_t)t * 4 * seg_stride(NU);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float p = fp8_chunk_dot(wb[j][r], xt, NU, uu);
                    // lanes past the row end add nothing (not even a NaN)
                    acc[t][r] = valid ? __builtin_fmaf(s, p, acc[t][r]) : acc[t][r];
                }
            }
        };
        // rounds of PF sweeps; refills unconditional and pinned; last round none
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
        return true;
    };
    if constexpr (PH) {
        for (int c0 = 0; c0 < NUA; c0 += NUP) phase(c0, min(NUP, NUA - c0));
    } else {
        if (!phase(0, NUA)) return;
    }

#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float v = sub_reduce<LPR>(acc[t][r]);
            if (sl == LPR - 1 && row0 + r < O) y[(size_t)t * O + row0 + r] = v;
        }
}

// General kernel: any I >= 1, any alignment, S <= QGEMV_MAX_S.  One wave per
// row; each weight decoded to f32 and multiplied by its block scale (one
// rounding), then multiplied into x in f32.
template <typename ST>
__global__ __launch_bounds__(256) void fp8_gemv_general(
    const uint8_t *__restrict__ w, const ST *__restrict__ sc, const float *__restrict__ x,
    float *__restrict__ y, int S, int I, int O)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= O) return;
    const int nbi = (I + 127) / 128;
    const uint8_t *wr = w + (size_t)row * I;
    const ST *scr = sc + (size_t)(row / 128) * nbi;
    float acc[QGEMV_MAX_S];
#pragma unroll
    for (int t = 0; t < QGEMV_MAX_S; t++) acc[t] = 0.0f;
    for (int i = lane; i < I; i += WAVE) {
        float v[4];
        e4m3x4((uint32_t)wr[i], v);
        const float wv = v[0] * scale_value(scr[i / 128]);
#pragma unroll
        for (int t = 0; t < QGEMV_MAX_S; t++)
            if (t < S) acc[t] = __builtin_fmaf(wv, x[(size_t)t * I + i], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < QGEMV_MAX_S; t++) {
        if (t < S) {
            const float v = sub_reduce<64>(acc[t]);
            if (lane == 63) y[(size_t)t * O + row] = v;
        }
    }
}

// Decode-only: W[o][i] = e4m3(w[o][i]) * scale[o/128][i/128] as f32.
template <typename ST>
__global__ __launch_bounds__(256) void fp8_dequant(const uint8_t *__restrict__ w,
                                                   const ST *__restrict__ sc,
                                                   float *__restrict__ W, int I, int O)
{
    const int nbi = (I + 127) / 128;
    const size_t n = (size_t)O * I;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t o = idx / I;
        const int i = (int)(idx - o * I);
        float v[4];
        e4m3x4((uint32_t)w[idx], v);
        W[idx] = v[0] * scale_value(sc[(o / 128) * nbi + i / 128]);
    }
}

namespace {

// 16 columns per lane chunk = 4 float4 segments, plus one spare float4
size_t fp8_lds_bytes(int S, int I)
{
    return ((size_t)S * 4 * seg_stride(I / 16) + 1) * sizeof(f32x4);
}

// Lane chunks per column phase: the whole row when S vectors of it fit the
// LDS, else the fewest equal phases (multiples of 64 chunks, 1024 columns)
// that do.
int fp8_phase_chunks(int S, int I)
{
    const int NUA = I / 16;
    for (int nph = 1;; nph++) {
        int nup = (NUA + nph - 1) / nph;
        if (nph > 1) nup = (nup + 63) / 64 * 64;
        if (fp8_lds_bytes(S, nup * 16) <= LDS_BUDGET) return nup;
    }
}

template <typename ST, int S, int LPR, int R, int PF, int WPB>
hipError_t launch_t(const uint8_t *w, const ST *sc, const float *x, float *y, int I, int O,
                    hipStream_t st)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    const int ntiles = (O + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    const int blocks = (ntiles + WPB - 1) / WPB;
    const int nup = fp8_phase_chunks(S, I);
    const size_t lds = fp8_lds_bytes(S, nup * 16);
    auto kern = nup < I / 16 ? fp8_gemv_stream<ST, S, LPR, R, PF, WPB, true>
                             : fp8_gemv_stream<ST, S, LPR, R, PF, WPB, false>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WPB), lds, st, w, sc, x, y, I, O,
                       (I + 127) / 128, ntiles, nup);
    return hipGetLastError();
}

// Lanes per row: pick_lpr_wide's width; for one vector
// narrowed (not below 8) until a row takes at least three sweeps, so that
// short rows give each wave more than one or two loads per row to keep in
// flight.  28672 x 1024 13.8 -> 7.9 us, 14336 x 2048 9.8 -> 7.8 us, 7168 x
// 2048 6.0 -> 5.1 us, 28672 x 512 8.0 -> 5.0 us; three-sweep rows stay
// (16384 x 1536: six sweeps 8.85 against 8.60 us).
// The starting width is pick_lpr_wide's (64 or 32 lanes for rows of at
// least 32 chunks): 4096 x 11008 12.7 -> 11.3 us, 1024 x 4352 5.8 -> 5.1 us,
// 2048 x 2176 5.8 -> 4.4 us; other shapes unchanged.  (18944 x 3584 runs
// 9.8 or 13.6 us from one build to another of the same fp8 code, either way.)
inline int fp8_lpr(int I, int S)
{
    int l = pick_lpr_wide(I / 16);
    if (S == 1)
        while (l > 8 && (I / 16) / l < 3) l /= 2;
    return l;
}

template <typename ST, int S, int R, int WPB = S == 1 ? QG_FP8_WPB : QG_FP8_WPB_MULTI>
hipError_t launch_r(const uint8_t *w, const ST *sc, const float *x, float *y, int I, int O,
                    hipStream_t st)
{
    // several vectors: 16-wave workgroups leave 128 registers per lane, so
    // two sweeps in flight
    constexpr int PF = S == 1 ? QG_FP8_PF : 2;
    switch (fp8_lpr(I, S)) {
    case 64: return launch_t<ST, S, 64, R, PF, WPB>(w, sc, x, y, I, O, st);
    case 32: return launch_t<ST, S, 32, R, PF, WPB>(w, sc, x, y, I, O, st);
    case 16: return launch_t<ST, S, 16, R, PF, WPB>(w, sc, x, y, I, O, st);
    case 8: return launch_t<ST, S, 8, R, PF, WPB>(w, sc, x, y, I, O, st);
    default: return launch_t<ST, S, 4, R, PF, WPB>(w, sc, x, y, I, O, st);
    }
}

template <typename ST, int S>
hipError_t launch_s(const uint8_t *w, const ST *sc, const float *x, float *y, int I, int O,
                    hipStream_t st)
{
    if constexpr (S == 1) {
        // Tile: the one that fills whole rounds of the CUs best
        // (pick_fill_tile).  Seven-wave two-row tiles fill two rounds exactly
        // at 7168 rows; eight-wave tiles fill whole rounds at 2048 and 4096
        // rows (measured at 2048 x 7168: 5.8 -> 4.9 us; 4096 x 7168: 8.5 ->
        // 7.2 us; 2048 x 16384: 9.7 -> 8.1 us).  Short rows keep seven waves:
        // at 2048 x 2048 eight-wave one-row tiles took 5.4 us against 4.4 us.
        // One-row tiles only where they leave at most one workgroup per CU:
        // 18432 x 7168 24.6 us (8 x 1, 2304 workgroups) against 23.4 us (8 x 2).
        static const WaveTile cand[] = {{QG_FP8_WPB, QG_FP8_R}, {QG_FP8_WPB2, QG_FP8_R},
                                        {QG_FP8_WPB, 1}, {QG_FP8_WPB2, 1}};
        static const WaveTile cand7[] = {{QG_FP8_WPB, QG_FP8_R}, {QG_FP8_WPB, 1}};
        const long rpg = 64 / fp8_lpr(I, 1);   // lane groups per wave
        int best;
        if (I >= QG_FP8_WPB2_MIN_I) {
            best = pick_fill_tile(O, rpg, cand, 4, cu_count(), true);
        } else {
            best = pick_fill_tile(O, rpg, cand7, 2, cu_count(), true) ? 2 : 0;
        }
        switch (best) {
        case 0: return launch_r<ST, S, QG_FP8_R, QG_FP8_WPB>(w, sc, x, y, I, O, st);
        case 1: return launch_r<ST, S, QG_FP8_R, QG_FP8_WPB2>(w, sc, x, y, I, O, st);
        case 2: return launch_r<ST, S, 1, QG_FP8_WPB>(w, sc, x, y, I, O, st);
        default: return launch_r<ST, S, 1, QG_FP8_WPB2>(w, sc, x, y, I, O, st);
        }
    } else {
        // several vectors: R keeps every workgroup resident at once (the rows
        // of a lane group must share a 128-row band, so R divides 128)
        static const int cand[] = {1, 2};
        switch (pick_rows_per_group(O, pick_lpr_wide(I / 16), QG_FP8_WPB_MULTI,
                                    fp8_lds_bytes(S, fp8_phase_chunks(S, I) * 16), cand, 2)) {
        case 1: return launch_r<ST, S, 1>(w, sc, x, y, I, O, st);
        default: return launch_r<ST, S, 2>(w, sc, x, y, I, O, st);
        }
    }
}

// Vectors one streaming launch takes for this shape (0: not applicable).
// Activations too long for the LDS are staged in column phases.
int fp8_stream_vectors(const void *w, const float *x, int S, int I)
{
    if (I % 16 != 0 || ((uintptr_t)w & 15) != 0 || ((uintptr_t)x & 15) != 0) return 0;
    return S < FP8_FAST_MAX_S ? S : FP8_FAST_MAX_S;
}

template <typename ST>
hipError_t launch_gemv(const void *w, const ST *sc, const float *x, float *y, int S, int I,
                       int O, hipStream_t st)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    // more vectors than one launch takes (S > 4) run in groups, each
    // streaming the weights once
    const int nmax = fp8_stream_vectors(w, x, S, I);
    if (nmax > 0) {
        for (int s0 = 0; s0 < S; s0 += nmax) {
            const int n = S - s0 < nmax ? S - s0 : nmax;
            const float *xs = x + (size_t)s0 * I;
            float *ys = y + (size_t)s0 * O;
            hipError_t e;
            switch (n) {
            case 1: e = launch_s<ST, 1>(wb, sc, xs, ys, I, O, st); break;
            case 2: e = launch_s<ST, 2>(wb, sc, xs, ys, I, O, st); break;
            case 3: e = launch_s<ST, 3>(wb, sc, xs, ys, I, O, st); break;
            default: e = launch_s<ST, 4>(wb, sc, xs, ys, I, O, st); break;
            }
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int wpb = 4;
    hipLaunchKernelGGL(fp8_gemv_general<ST>, dim3((O + wpb - 1) / wpb), dim3(64 * wpb), 0, st,
                       wb, sc, x, y, S, I, O);
    return hipGetLastError();
}

template <typename ST>
hipError_t launch_dequant(const void *w, const ST *sc, float *W, int I, int O, hipStream_t st)
{
    const size_t n = (size_t)O * I;
    const size_t want = (n + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(fp8_dequant<ST>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint8_t *>(w), sc, W, I, O);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8b128_gemv(const void *w, const float *scale_inv, const float *x, float *y,
                               int S, int I, int O, hipStream_t st)
{
    return launch_gemv(w, scale_inv, x, y, S, I, O, st);
}

hipError_t launch_fp8ue8m0_gemv(const void *w, const uint8_t *scale_e8m0, const float *x,
                                float *y, int S, int I, int O, hipStream_t st)
{
    return launch_gemv(w, scale_e8m0, x, y, S, I, O, st);
}

hipError_t launch_fp8b128_dequant(const void *w, const float *scale_inv, float *W, int I, int O,
                                  hipStream_t st)
{
    return launch_dequant(w, scale_inv, W, I, O, st);
}

hipError_t launch_fp8ue8m0_dequant(const void *w, const uint8_t *scale_e8m0, float *W, int I,
                                   int O, hipStream_t st)
{
    return launch_dequant(w, scale_e8m0, W, I, O, st);
}

}  // namespace qg
