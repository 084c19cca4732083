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
//   * a workgroup that meets an infinity or NaN in x computes its rows with
//     per-element f32 products instead, so they propagate as in the plain
//     definition.
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

// activation items (8 columns each) each thread loads up front
#ifndef QG_I4G_NPRE
#define QG_I4G_NPRE 2
#endif
// several vectors on the int8 matrix cores (0: the streaming kernel)
#ifndef QG_I4G_MV
#define QG_I4G_MV 1
#endif
#ifndef QG_I4G_MV_NT
#define QG_I4G_MV_NT 0
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
    int *wflag = reinterpret_cast<int *>(xc + (size_t)S * NU);             // [WPB]

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
    const bool wbad = __ballot(bad != 0) != 0;
    if (lane == 0) wflag[wave] = wbad;
    __syncthreads();
    int anybad = 0;
#pragma unroll
    for (int k = 0; k < WPB; k++) anybad |= wflag[k];
    anybad = __builtin_amdgcn_readfirstlane(anybad);
    if (tile >= ntiles) return;
    if (anybad) {
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
    // one vector: running digit sums per row (see q8_dot_run)
    uint32_t P[R][6], V[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        V[r] = 0;
#pragma unroll
        for (int k = 0; k < 6; k++) P[r][k] = 0;
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
                const int dv = S == 1 ? q8_dot_run(wx[r], L, P[r], V[r]) : q8_dot(wx[r], L);
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

// ---------------------------------------------------------------------------
// Four vectors on the int8 matrix cores.  With several vectors the
// per-vector digit products of the streaming kernel make it VALU-bound (four
// vectors at 12288 x 6144: twice the one-vector time), while the same
// products are a skinny dense contraction: 16 rows x 64 columns of nibbles
// (A, unsigned 0..15 as int8) times 64 columns x 16 (vector, digit) pairs of
// activation digits (B) per v_mfma_i32_16x16x64_i8.
//
// Activations: per 64-column block and vector, E is the smallest integer
// with max|x| < 2^E (E >= -100) and v = RNE(x 2^(22-E)), |v| <= 2^22, split
// into three balanced base-256 digits d0 + 256 d1 + 65536 d2 (each an int8).
// B column j = 4t + d holds digit d of vector t (column 4t + 3 and vectors
// past S hold zeros).  The exact integer sum over a block is
// D = sum q d_j; sum (q - 8) d_j = D - 8 sum d_j, converted to f32 and
// scaled by 2^(E-22) 256^d (exact) and the row's group scale (one rounding),
// then the three digits of a vector are added at the end.
//
// Operand layouts (checked on the device): lane l supplies A[l % 16][16 (l /
// 16) + b] and B[16 (l / 16) + b][l % 16] in byte b of its four dwords; D
// register i of lane l is D[4 (l / 16) + i][l % 16].  A lane's 16 k-slots are
// columns 16 (l / 16) + {0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15} of the
// block: the order a packed dword's low and high nibbles fall in when masked
// apart, which the staging of B follows.
//
// A workgroup owns MV_RB blocks of 16 rows; each is split over MV_KS waves by
// column range, and the partial sums meet in LDS.
// ---------------------------------------------------------------------------
constexpr int MV_RB = 3;     // 16-row blocks per workgroup
constexpr int MV_KS = 4;     // column splits per row block
constexpr int MV_WPB = MV_RB * MV_KS;
constexpr int MV_SS = 4;     // 64-column blocks per wave load step (128 B of each of 16 rows)
#ifndef QG_I4G_MV_PF
#define QG_I4G_MV_PF 2
#endif
constexpr int MV_PF = QG_I4G_MV_PF;     // load steps in flight per wave
constexpr int MV_RS = MV_SS * 32 + 16;   // LDS row stride of a wave's load step (bytes)
constexpr int MV_WL = 16 * MV_RS + MV_SS * 16 * 4;   // a wave's LDS: weights + scales
constexpr int MV_NPRE = 6;   // staging items (8 columns) per thread
typedef int i32x4 __attribute__((ext_vector_type(4)));

size_t i4g_mv_lds_bytes(int I)
{
    const size_t nkb = (size_t)I / 64;
    return nkb * 64 * 16 + nkb * 16 * 8 + (size_t)MV_WPB * 64 * 4 + 16 * 4 +
           (size_t)MV_WPB * MV_WL;
}

template <int S>
__global__ __launch_bounds__(64 * MV_WPB) void i4g_gemv_mv(
    const uint8_t *__restrict__ w, const float *__restrict__ scales,
    const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, Div20 div_bpg)
{
    constexpr int NT = 64 * MV_WPB;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NKB = I / 64;
    u32x4 *bl = reinterpret_cast<u32x4 *>(lds_raw);                      // [NKB][64] B operands
    int2 *ml = reinterpret_cast<int2 *>(bl + (size_t)NKB * 64);          // [NKB][16] (8 sum d, c)
    float *red = reinterpret_cast<float *>(ml + (size_t)NKB * 16);       // [MV_WPB][4][16]
    int *wflag = reinterpret_cast<int *>(red + MV_WPB * 64);             // [16]
    unsigned char *wls = reinterpret_cast<unsigned char *>(wflag + 16);  // [MV_WPB][MV_WL]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rbl = wave / MV_KS, ks = wave - rbl * MV_KS;
    const int row0 = (blockIdx.x * MV_RB + rbl) * 16;
    const int g = lane >> 4, j = lane & 15;

    // 1. activations: item f is 8 columns 64 kb + 8 m of vector t (t = f /
    //    (8 NKB), kb = f / 8 % NKB, m = f % 8): vector-major, so whole waves
    //    of items past S only write zeros
    const int items = NKB * 32;
    const int ipv = NKB * 8;   // items per vector
    auto item_t = [&](int f) { return (f >= ipv) + (f >= 2 * ipv) + (f >= 3 * ipv); };
    f32x4 xa[MV_NPRE], xb[MV_NPRE];
#pragma unroll
    for (int p = 0; p < MV_NPRE; p++) {
        // unconditional loads (clamped index; unused items are zeroed after
        // the loads) so that the waits for them count exactly
        const int f = min((int)threadIdx.x + p * NT, items - 1);
        const int t = min(item_t(f), S - 1), kb = (f - item_t(f) * ipv) >> 3, m = f & 7;
        const float *src = x + (size_t)t * I + kb * 64 + m * 8;
        xa[p] = *reinterpret_cast<const f32x4 *>(src);
        xb[p] = *reinterpret_cast<const f32x4 *>(src + 4);
    }
    // every wave of the workgroup has issued its activation loads before any
    // wave issues weight loads (raw barrier: no drain); without it the last
    // activation loads arrived up to 5 us into the call, behind weight misses
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // 2. this wave's column range of its 16 rows.  A load step is MV_SS
    //    blocks: lane l reads 32 bytes (one block) of row l / 4, so each row's
    //    128 bytes come in one piece, and its group scale; the step goes
    //    through the wave's own LDS (no workgroup barrier: one wave's LDS
    //    accesses execute in order) to the MFMA layout.  MV_PF steps in flight.
    const int per = (NKB + MV_KS - 1) / MV_KS;
    const int kb0 = min(ks * per, NKB);
    const int nk = min(per, NKB - kb0);
    const int lr = lane >> 2, lp = lane & 3;
    const int lrow = min(row0 + lr, O - 1);
    const uint8_t *wrow = w + (size_t)lrow * ((size_t)I / 2);
    const float *srow = scales + (size_t)lrow * ng;
    unsigned char *wl = wls + (size_t)wave * MV_WL;
    float *wsc = reinterpret_cast<float *>(wl + 16 * MV_RS);   // [MV_SS][16]
    u32x4 wq0[MV_PF], wq1[MV_PF];
    float sq[MV_PF];
    auto fetch = [&](int st, int slot) {
        const int kb = max(min(kb0 + st * MV_SS + lp, NKB - 1), 0);
        wq0[slot] = ld_stream(reinterpret_cast<const u32x4 *>(wrow + (size_t)kb * 32));
        wq1[slot] = ld_stream(reinterpret_cast<const u32x4 *>(wrow + (size_t)kb * 32 + 16));
        sq[slot] = ld_stream(&srow[div_bpg((uint32_t)kb)]);
    };
    const int nst = (nk + MV_SS - 1) / MV_SS;
#pragma unroll
    for (int slot = 0; slot < MV_PF; slot++) fetch(slot, slot);   // in flight while x converts
    // the activations count as redefined here: the compiler can neither
    // reload them later (behind the weight loads) nor wait for more than them
#pragma unroll
    for (int p = 0; p < MV_NPRE; p++) asm volatile("" : "+v"(xa[p]), "+v"(xb[p]));

    uint32_t bad = 0;
#pragma unroll
    for (int p = 0; p < MV_NPRE; p++) {
        const int f = (int)threadIdx.x + p * NT;
        if (f >= items) continue;   // whole 8-lane groups (items and NT are multiples of 8)
        const int t = item_t(f), kb = (f - t * ipv) >> 3, m = f & 7;
        // B bytes: digit d of columns 16 (m / 2) + 8 (m % 2) + {0,2,4,6} then
        // {1,3,5,7}, in B slot 16 g + j (g = m / 2, j = 4 t + d) stored at
        // 16 g + (j ^ swz): the slots a wave writes for one (t, d) would all
        // fall on the same LDS banks unswizzled
        const int swz = (kb * 4 + (m >> 1)) & 15;
        uint2 *dst0 = reinterpret_cast<uint2 *>(bl + (size_t)kb * 64 + 16 * (m >> 1)) + (m & 1);
        auto dst = [&](int d) { return dst0 + 2 * ((4 * t + d) ^ swz); };
        int2 *mm = ml + (size_t)kb * 16 + 4 * t;
        if (t >= S) {   // a vector slot past S: zeros
#pragma unroll
            for (int d = 0; d < 4; d++) *dst(d) = uint2{0u, 0u};
            if (m == 0)
#pragma unroll
                for (int d = 0; d < 4; d++) mm[d] = int2{0, 0x3F800000};
            continue;
        }
        const float v[8] = {xa[p].x, xa[p].y, xa[p].z, xa[p].w,
                            xb[p].x, xb[p].y, xb[p].z, xb[p].w};
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) mx = max(mx, __builtin_bit_cast(uint32_t, v[k]) & 0x7FFFFFFFu);
        mx = quad_max_u32(mx);
        mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x141, 0xF, 0xF, false));
        const uint32_t eb = mx >> 23;
        bad |= eb == 255u;
        const uint32_t e = max(eb, 26u);                                  // E = e - 126 >= -100
        const float sin = __builtin_bit_cast(float, (275u - e) << 23);    // 2^(22 - E)
        uint32_t sd[8];   // signed digit bytes of v: (v + 0x808080) ^ 0x808080
#pragma unroll
        for (int k = 0; k < 8; k++)
            sd[k] = (__builtin_bit_cast(uint32_t, __builtin_fmaf(v[k], sin, 12582912.0f)) -
                     0x4ABF7F80u) ^ 0x808080u;
#pragma unroll
        for (int d = 0; d < 3; d++) {
            const uint32_t sel = (uint32_t)d | ((uint32_t)(4 + d) << 8) | 0x0C0C0000u;
            const uint32_t e0 = __builtin_amdgcn_perm(sd[2], sd[0], sel);
            const uint32_t e1 = __builtin_amdgcn_perm(sd[6], sd[4], sel);
            const uint32_t o0 = __builtin_amdgcn_perm(sd[3], sd[1], sel);
            const uint32_t o1 = __builtin_amdgcn_perm(sd[7], sd[5], sel);
            const uint32_t ev = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
            const uint32_t od = __builtin_amdgcn_perm(o1, o0, 0x05040100u);
            *dst(d) = uint2{ev, od};
            // the block's digit sum: four signed bytes per dot, then 8 lanes
            int sum = __builtin_amdgcn_sdot4((int)ev, 0x01010101, 0, false);
            sum = __builtin_amdgcn_sdot4((int)od, 0x01010101, sum, false);
            sum = quad_sum_i32(sum);
            sum += __builtin_amdgcn_update_dpp(0, sum, 0x141, 0xF, 0xF, false);
            if (m == 0)
                // scale 2^(E - 22) 256^d as f32 bits
                mm[d] = int2{8 * sum, (int)((e - 21u + 8u * (uint32_t)d) << 23)};
        }
        *dst(3) = uint2{0u, 0u};   // column 4t + 3
        if (m == 0) mm[3] = int2{0, 0x3F800000};
    }
    const bool wbad = __ballot(bad != 0) != 0;
    if (lane == 0) wflag[wave] = wbad;
    __syncthreads();
    int anybad = 0;
#pragma unroll
    for (int k = 0; k < MV_WPB; k++) anybad |= wflag[k];
    anybad = __builtin_amdgcn_readfirstlane(anybad);
    if (anybad) {
        // the plain definition's arithmetic for the workgroup's rows
        for (int r = wave; r < MV_RB * 16; r += MV_WPB)
            i4g_rows_plain<S, 64, 1>(w, scales, x, y, I, O, ng, div_cpg,
                                     blockIdx.x * MV_RB * 16 + r, lane);
        return;
    }

    // 2. the wave's column range (its first load steps went out above)
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < nst; s0 += MV_PF) {
#pragma unroll
        for (int slot = 0; slot < MV_PF; slot++) {
            const int st = s0 + slot;
            if (st < nst) {
                u32x4 *wd = reinterpret_cast<u32x4 *>(wl + lr * MV_RS + lp * 32);
                wd[0] = wq0[slot];
                wd[1] = wq1[slot];
                wsc[lp * 16 + lr] = sq[slot];
#pragma unroll
                for (int p = 0; p < MV_SS; p++) {
                    const int i = st * MV_SS + p;
                    if (i < nk) {
                        const int kb = kb0 + i;
                        const u32x2 wv = *reinterpret_cast<const u32x2 *>(wl + j * MV_RS + p * 32 +
                                                                          8 * g);
                        const i32x4 a = {(int)(wv.x & 0x0F0F0F0Fu),
                                         (int)((wv.x >> 4) & 0x0F0F0F0Fu),
                                         (int)(wv.y & 0x0F0F0F0Fu),
                                         (int)((wv.y >> 4) & 0x0F0F0F0Fu)};
                        const u32x4 bu = bl[(size_t)kb * 64 + 16 * g + (j ^ ((kb * 4 + g) & 15))];
                        const i32x4 b = {(int)bu.x, (int)bu.y, (int)bu.z, (int)bu.w};
                        const int2 mm = ml[(size_t)kb * 16 + j];
                        const f32x4 sc4 = *reinterpret_cast<const f32x4 *>(wsc + p * 16 + 4 * g);
                        const i32x4 c0 = {0, 0, 0, 0};
                        const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
                        const float cfd = __builtin_bit_cast(float, mm.y);
                        acc[0] = __builtin_fmaf(sc4.x, cfd * (float)(D[0] - mm.x), acc[0]);
                        acc[1] = __builtin_fmaf(sc4.y, cfd * (float)(D[1] - mm.x), acc[1]);
                        acc[2] = __builtin_fmaf(sc4.z, cfd * (float)(D[2] - mm.x), acc[2]);
                        acc[3] = __builtin_fmaf(sc4.w, cfd * (float)(D[3] - mm.x), acc[3]);
                    }
                }
            }
            fetch(st + MV_PF, slot);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // 3. digits of a vector (lanes 4t .. 4t + 3 of each 16), then the column
    //    splits of each row block in order
#pragma unroll
    for (int r = 0; r < 4; r++) {
        float v = acc[r];
        v += dpp<0xB1>(v);
        v += dpp<0x4E>(v);
        if ((lane & 3) == 0) red[(wave * 4 + (j >> 2)) * 16 + 4 * g + r] = v;
    }
    __syncthreads();
    for (int q = (int)threadIdx.x; q < MV_RB * 64; q += NT) {
        const int rb2 = q >> 6, t = (q >> 4) & 3, r16 = q & 15;
        float v = 0.0f;
#pragma unroll
        for (int k2 = 0; k2 < MV_KS; k2++) v += red[((rb2 * MV_KS + k2) * 4 + t) * 16 + r16];
        const int row = (blockIdx.x * MV_RB + rb2) * 16 + r16;
        if (t < S && row < O) y[(size_t)t * O + row] = v;
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

// lanes per row: the fullest sweep, at most QG_I4G_LPR
inline int i4g_lanes_per_row(int I)
{
    const int lpr = pick_lpr(I / 32);
    return lpr > QG_I4G_LPR ? QG_I4G_LPR : lpr;
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
    const int lpr = i4g_lanes_per_row(I);
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
        return launch_stream_r<S, QG_I4G_R>(w, s, x, y, I, O, gs, st);
    } else {
        // several vectors: the staged activations take S times the LDS, so
        // few workgroups fit a CU; R keeps them all resident, ties going to
        // the larger R (fewer workgroups staging the vectors).  12288 rows,
        // two to four vectors: R = 2, 256 workgroups of 48 rows
        static const int cand[] = {3, 2, 1};
        switch (pick_rows_per_group(O, i4g_lanes_per_row(I), QG_I4G_WPB_MULTI,
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
    return q8_stage_bytes(S, I / 32, false) + 16 * sizeof(int);
}

int i4g_stream_vectors(const void *w, const float *x, int S, int I, int gs)
{
    if (I % 32 != 0 || gs % 32 != 0 || ((uintptr_t)w & 15) != 0 || ((uintptr_t)x & 15) != 0)
        return 0;
    int n = S < I4G_FAST_MAX_S ? S : I4G_FAST_MAX_S;
    while (n > 0 && i4g_stream_lds_bytes(n, I) > LDS_BUDGET) --n;
    return n;
}

namespace {

template <int S>
hipError_t launch_mv_s(const uint8_t *w, const float *s, const float *x, float *y, int I,
                       int O, int gs, hipStream_t st)
{
    const size_t lds = i4g_mv_lds_bytes(I);
    auto kern = i4g_gemv_mv<S>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    const int blocks = ((O + 15) / 16 + MV_RB - 1) / MV_RB;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * MV_WPB), lds, st, w, s, x, y, I, O,
                       (I + gs - 1) / gs, Div20::make((uint32_t)(gs / 32)),
                       Div20::make((uint32_t)(gs / 64)));
    return hipGetLastError();
}

// the matrix-core kernel takes four vectors of rows in whole 64-column
// blocks, scale groups of whole blocks, 16-byte aligned weights and
// activations that its staging holds.  Its time barely depends on
// S: at 12288 x 6144 it measured 17.2 us for four vectors and 16.9 us for
// two, against 22.9 and 14.6 us for the streaming kernel, which therefore
// keeps two and three.
bool i4g_mv_fits(const void *w, const float *x, int S, int I, int gs)
{
    return QG_I4G_MV && S == 4 && I % 64 == 0 && gs % 64 == 0 &&
           ((uintptr_t)w & 15) == 0 && ((uintptr_t)x & 15) == 0 &&
           i4g_mv_lds_bytes(I) <= LDS_BUDGET && (I / 64) * 32 <= MV_NPRE * 64 * MV_WPB;
}

}  // namespace

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
            if (i4g_mv_fits(w, xs, n, I, gs)) {
                e = launch_mv_s<4>(wb, scales, xs, ys, I, O, gs, st);
            } else {
                switch (n) {
                case 1: e = launch_stream_s<1>(wb, scales, xs, ys, I, O, gs, st); break;
                case 2: e = launch_stream_s<2>(wb, scales, xs, ys, I, O, gs, st); break;
                case 3: e = launch_stream_s<3>(wb, scales, xs, ys, I, O, gs, st); break;
                default: e = launch_stream_s<4>(wb, scales, xs, ys, I, O, gs, st); break;
                }
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
