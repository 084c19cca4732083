// moe.hip -- routed-expert GEMV over grouped-int4 experts for gfx950.
//
//   y[t][o] = sum_k gates[t][k] * (W_{ids[t][k]} . x[t])[o],  k ascending
//
// (regolith audit "phase 0 + phase 2 m5 air validation", section 2.2: the
// gates are the selection probabilities renormalised over the selected
// experts; colibri PR #457, section 4: routed experts are grouped-int4.)
//
// One launch, no host round trip, no atomics:
//   * workgroup (t, b) owns token t and RT consecutive output rows; the
//     T * NB workgroups (NB row blocks per token) cover about one CU each;
//   * it stages x[t] in LDS as the dense grouped-int4 GEMV does (per-chunk
//     fixed-point digits for the 4-bit integer dot product; one vector:
//     staging every token in every workgroup makes thousands of workgroups
//     fetch the same lines at once, which costs more than it saves); a token
//     whose activations hold an infinity or NaN is multiplied per element in
//     f32 instead, so they propagate as in the plain definition;
//   * one wave reads the token's K ids and hands them over in LDS; every wave
//     derives with ballots the distinct valid experts (first-occurrence
//     order) -- the routing never leaves the device;
//   * work units are (distinct expert, sub-tile of rows); each wave starts
//     on one and takes the next free one from an LDS counter when it is
//     done; a unit streams its rows of that expert (dwordx4, scale gather);
//     a wave's (unit, sweep) steps form one stream with PF sweeps of loads in
//     flight, crossing unit boundaries;
//   * a unit's row sums go to an LDS partial array [K][RT] for every slot k
//     that selected the expert (a duplicated id is streamed once and counted
//     per slot); after a barrier the workgroup forms y[t] = sum_k gates *
//     partial in ascending k (deterministic).
// An expert selected by several tokens is streamed once per selecting token.
// An id outside [0, E) is never dereferenced: its token's row of y is NaN and
// the token's error flag in the workspace is set.
#include "qg_device.h"
#include "qg_launch.h"

#ifndef QG_MOE_R
#define QG_MOE_R 2
#endif
#ifndef QG_MOE_WPB
#define QG_MOE_WPB 8
#endif
// workgroups per launch the row blocking aims at (over all tokens)
#ifndef QG_MOE_WGS
#define QG_MOE_WGS 256
#endif
#ifndef QG_MOE_PF
#define QG_MOE_PF 3
#endif
// activation items (8 columns each) each thread loads up front: two cover a
// 7168-column token with 8 waves, so no second round trip follows the
// conversion (46.4 -> 46.0 us at 256 experts of 2048 x 7168, 4 tokens, top-8)
#ifndef QG_MOE_NPRE
#define QG_MOE_NPRE 2
#endif
// ring slots filled before the activations are converted.  Measured at 256
// experts of 2048 x 7168, 4 tokens, top-8 (mean of five interleaved runs of
// 300 calls): none 45.9 us, one 45.7, two 45.6, three 45.8.
#ifndef QG_MOE_EARLY
#define QG_MOE_EARLY 2
#endif

namespace qg {

constexpr int MOE_MAX_T = 8;
constexpr int MOE_FAST_MAX_K = 64;

// Lane holding the ui-th set bit of a wave-uniform lane mask (-1 if none).
__device__ __forceinline__ int nth_lane(uint64_t m, int ui)
{
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane ? (m & ((1ull << lane) - 1)) : 0ull;
    const uint64_t sel = __ballot(((m >> lane) & 1) && __popcll(below) == ui);
    return __ffsll((long long)sel) - 1;
}

template <int LPR, int R, int PF>
__global__ __launch_bounds__(64 * QG_MOE_WPB) void moe_i4g_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, long long w_stride,
    long long s_stride, int E, const int32_t *__restrict__ ids, const float *__restrict__ gates,
    int T, int K, const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, int RT, int NB, int *__restrict__ err_flag)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    constexpr int MOE_EARLY = QG_MOE_EARLY < PF ? QG_MOE_EARLY : PF;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;
    u32x4 *xq = reinterpret_cast<u32x4 *>(lds_raw);                      // [6][NU]
    float *xc = reinterpret_cast<float *>(xq + 6 * NU);                   // [NU]
    float *part = xc + NU;                                                // [K][RT]
    int *ids_l = reinterpret_cast<int *>(part + (size_t)K * RT);          // [64]
    int *ctr = ids_l + 64;                                                // next unit
    int *wflag = ctr + 1;                                                 // [WPB]

    const int t = blockIdx.x / NB;
    const int o0 = (blockIdx.x - t * NB) * RT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int nwaves = QG_MOE_WPB;
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const size_t rb = (size_t)I / 2;
    const int nit = (NU + LPR - 1) / LPR;
    const int nsub = RT / ROWS_PER_WAVE;

    // the token's ids (one wave; thousands of waves reading one line would
    // queue on one L2 channel) and its activations, before any weight load
    int id = 0;
    if (wave == 0) id = ids[t * K + min(lane, K - 1)];
    const float *xt = x + (size_t)t * I;
    XStageQ<1, QG_MOE_NPRE, 64 * QG_MOE_WPB> xst;
    const int items = NU * 4;
    xst.load(xt, items);
    __builtin_amdgcn_sched_barrier(0);
    if (wave == 0) ids_l[lane] = id;
    if (threadIdx.x == 0) *ctr = nwaves;
    // raw barrier (the activation loads stay in flight); the LDS write must
    // have landed before it
    __builtin_amdgcn_s_waitcnt(QG_WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // distinct valid experts of the token, first-occurrence order
    const int e = lane < K ? ids_l[lane] : -1;
    const bool valid = lane < K && e >= 0 && e < E;
    bool first = valid;
    for (int q = 0; q < K; q++)
        if (q < lane && __builtin_amdgcn_readlane(e, q) == e) first = false;
    const uint64_t firstm = __ballot(first);
    const bool bad = __ballot(lane < K && !valid) != 0;
    if (o0 == 0 && threadIdx.x == 0) {
        err_flag[t] = bad ? 1 : 0;
        if (t == 0)
            for (int u = T; u < MOE_MAX_T; u++) err_flag[u] = 0;
    }

    // Work units are (distinct expert ui, row sub-tile st), numbered
    // i = ui * nsub + st.  Wave w starts on unit w; each later unit goes to
    // whichever wave asks first (an LDS counter), so waves that the SIMDs
    // serve faster take more units and the workgroup finishes together.
    const int nunits = __popcll(firstm) * nsub;

    struct Unit {
        int e, row0;
    };
    auto unit_of = [&](int i) {
        const int ui = i / nsub, st = i - ui * nsub;
        const int ql = nth_lane(firstm, ui);
        Unit u;
        // past the last unit (or none): expert 0, so clamped loads stay valid
        u.e = ql >= 0 && i < nunits ? __builtin_amdgcn_readlane(e, ql) : 0;
        u.row0 = o0 + st * ROWS_PER_WAVE + sub * R;
        return u;
    };
    auto grab = [&]() {
        int v = 0;
        if (lane == 0) v = atomicAdd(ctr, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };

    u32x4 wb[PF][R];
    float sb[PF][R];
    // each ring slot records the unit and sweep its loads belong to
    // (unit >= nunits: nothing, the loads re-read the previous step)
    int slot_u[PF], slot_c[PF];
    // fetch cursor: unit fi, sweep fc
    int fi = wave, fc = 0;
    Unit fu = unit_of(min(fi, nunits > 0 ? nunits - 1 : 0));
    auto fetch = [&](int j) {
        slot_u[j] = fi;
        slot_c[j] = fc;
        const uint8_t *we = w + (size_t)fu.e * (size_t)w_stride;
        const float *se = scales + (size_t)fu.e * (size_t)s_stride;
        const int u = min(fc * LPR + sl, NU - 1);
        const uint32_t g = div_cpg((uint32_t)u);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int row = min(fu.row0 + r, O - 1);
            wb[j][r] = ld_stream(reinterpret_cast<const u32x4 *>(we + (size_t)row * rb +
                                                                 (uint32_t)u * 16u));
            sb[j][r] = ld_stream(se + (size_t)row * ng + g);
        }
        if (fi < nunits) {
            if (fc + 1 < nit) {
                ++fc;
            } else {
                const int nx = grab();
                if (nx < nunits) {
                    fi = nx;
                    fc = 0;
                    fu = unit_of(fi);
                } else {
                    fi = nunits;   // done; keep re-reading the last step
                }
            }
        }
    };

    // the first QG_MOE_EARLY sweeps go out before the activations are
    // converted, the rest of the ring once they are staged
#pragma unroll
    for (int j = 0; j < MOE_EARLY; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t xbad = xst.store(xt, items, NU, reinterpret_cast<uint32_t *>(xq), xc, nullptr);
    const bool wbad = __ballot(xbad != 0) != 0;
    if (lane == 0) wflag[wave] = wbad;
    __syncthreads();
    int xnan = 0;
#pragma unroll
    for (int k = 0; k < QG_MOE_WPB; k++) xnan |= wflag[k];
    xnan = __builtin_amdgcn_readfirstlane(xnan);
#pragma unroll
    for (int j = MOE_EARLY; j < PF; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);

    float acc[R];
    uint32_t P[R][6], V[R];   // running digit sums per row (see q8_dot_run)
#pragma unroll
    for (int r = 0; r < R; r++) {
        acc[r] = 0.0f;
        V[r] = 0;
#pragma unroll
        for (int k = 0; k < 6; k++) P[r][k] = 0;
    }

    auto consume = [&](int j) {
        const int ci = slot_u[j];
        if (ci >= nunits) return;                      // nothing (wave-uniform)
        const int u = slot_c[j] * LPR + sl;
        const bool in_row = u < NU;
        const int uu = in_row ? u : 0;
        if (xnan) {
            if (in_row)
#pragma unroll
                for (int r = 0; r < R; r++)
                    acc[r] += nib_chunk_plain(wb[j][r], sb[j][r], xt + (size_t)uu * 32);
        } else {
            u32x4 L[6];
#pragma unroll
            for (int k = 0; k < 6; k++) L[k] = xq[k * NU + uu];
            const float cs = in_row ? xc[uu] : 0.0f;
#pragma unroll
            for (int r = 0; r < R; r++) {
                uint32_t wx[4];
#pragma unroll
                for (int d = 0; d < 4; d++) wx[d] = wb[j][r][d] ^ Q8_NIB_FLIP;
                const int dv = q8_dot_run(wx, L, P[r], V[r]);
                acc[r] = __builtin_fmaf(sb[j][r] * cs, (float)dv, acc[r]);
            }
        }
        if (slot_c[j] + 1 < nit) return;
        // unit done: row sums -> partials of every slot that chose its expert
        const Unit cu = unit_of(ci);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float v = sub_reduce<LPR>(acc[r]);
            const int lr = cu.row0 + r - o0;
            for (int kk = 0; kk < K; kk++)
                if (__builtin_amdgcn_readlane(e, kk) == cu.e && sl == LPR - 1 && cu.row0 + r < O)
                    part[(size_t)kk * RT + lr] = v;
            acc[r] = 0.0f;
        }
    };

    // rounds of PF slots: consume a slot, then refill it; stop once the
    // oldest slot of a round holds nothing (slots are filled in order)
    while (slot_u[0] < nunits) {
#pragma unroll
        for (int j = 0; j < PF; j++) {
            consume(j);
            pin_values(acc);
            fetch(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();

    // y[t] = sum_k gates * partial, ascending k
    for (int i = threadIdx.x; i < RT; i += 64 * QG_MOE_WPB) {
        const int row = o0 + i;
        if (row >= O) continue;
        float v;
        if (bad) {
            v = __builtin_nanf("");
        } else {
            v = 0.0f;
            for (int kk = 0; kk < K; kk++)
                v = __builtin_fmaf(gates[t * K + kk], part[(size_t)kk * RT + i], v);
        }
        y[(size_t)t * O + row] = v;
    }
}

// General kernel: any shape the streaming kernel does not take (T*K > 64,
// unaligned rows or strides, LDS too small).  One wave per output row; each
// (t, k) dot product is formed from per-weight f32 decodes, combined in
// ascending k.  Also sets the per-token error flags (block 0).
__global__ __launch_bounds__(256) void moe_i4g_general(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, long long w_stride,
    long long s_stride, int E, const int32_t *__restrict__ ids, const float *__restrict__ gates,
    int T, int K, const float *__restrict__ x, float *__restrict__ y, int I, int O, int gs,
    int *__restrict__ err_flag)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x < MOE_MAX_T) {
        const int tt = threadIdx.x;
        int bad = 0;
        if (tt < T)
            for (int kk = 0; kk < K; kk++) bad |= (ids[tt * K + kk] < 0 || ids[tt * K + kk] >= E);
        err_flag[tt] = bad;
    }
    if (row >= O) return;
    const int rb = (I + 1) / 2;
    const int ng = (I + gs - 1) / gs;
    for (int t = 0; t < T; t++) {
        float yt = 0.0f;
        bool bad = false;
        for (int kk = 0; kk < K; kk++) {
            const int e = ids[t * K + kk];
            if (e < 0 || e >= E) { bad = true; continue; }
            const uint8_t *wr = w + (size_t)e * (size_t)w_stride + (size_t)row * rb;
            const float *sr = scales + (size_t)e * (size_t)s_stride + (size_t)row * ng;
            const float *xt = x + (size_t)t * I;
            float acc = 0.0f;
            for (int b = lane; b < rb; b += WAVE) {
                float ev[4], od[4];
                nib8((uint32_t)wr[b], ev, od);
                const int c0 = 2 * b, c1 = 2 * b + 1;
                acc = __builtin_fmaf((ev[0] * NIB_XSCALE - 8.0f) * sr[c0 / gs], xt[c0], acc);
                if (c1 < I)
                    acc = __builtin_fmaf((od[0] * NIB_XSCALE - 8.0f) * sr[c1 / gs], xt[c1], acc);
            }
            const float dot = sub_reduce<64>(acc);
            yt = __builtin_fmaf(gates[t * K + kk], dot, yt);
        }
        if (lane == 63) y[(size_t)t * O + row] = bad ? __builtin_nanf("") : yt;
    }
}

// ---------------------------------------------------------------------------
// Router top-k (regolith audit, sections 2.1 and 2.2): softmax over the valid
// experts (columns 0..E-1 of rows of stride ld), the K most probable picked
// in rank order, gates renormalised over the picked ones.  One wave per
// token; lane l holds the logits of experts l, l + 64, ... (E <= 1024).  Each
// of the K rounds takes the wave-wide largest not-yet-picked logit (the lower
// expert index on a tie) by a butterfly reduction over (value, index) pairs;
// probability order is logit order, so no exponential is needed to pick.
// Lane k keeps pick k; g_k = exp(l_k - m) / sum over picks, m = the largest.
// ---------------------------------------------------------------------------
constexpr int ROUTER_MAX_E = 1024;
constexpr int ROUTER_MAX_K = 64;

__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits, int T,
                                                          int E, int ld, int K,
                                                          int32_t *__restrict__ ids,
                                                          float *__restrict__ gates)
{
    constexpr int PER = ROUTER_MAX_E / WAVE;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                           // whole waves
    const float *l = logits + (size_t)t * ld;
    float v[PER];
    uint32_t taken = 0;                           // bit j: entry j picked or not an expert
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const int e = lane + WAVE * j;
        v[j] = e < E ? l[e] : 0.0f;
        if (e >= E) taken |= 1u << j;
    }
    float pick_l = 0.0f;
    int pick_e = 0;
    for (int k = 0; k < K; k++) {
        float bv = 0.0f;
        int be = 0x7FFFFFFF;                      // none
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const int e = lane + WAVE * j;
            if (!((taken >> j) & 1u) && (be == 0x7FFFFFFF || v[j] > bv)) {
                bv = v[j];
                be = e;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, WAVE);
            const int oe = __shfl_xor(be, m, WAVE);
            const bool better = oe != 0x7FFFFFFF &&
                                (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
            if (better) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == k) {
            pick_l = bv;
            pick_e = be;
        }
    }
    const float m = __shfl(pick_l, 0, WAVE);
    const float ex = lane < K ? expf(pick_l - m) : 0.0f;
    const float sum = __shfl(sub_reduce<64>(ex), 63, WAVE);
    if (lane < K) {
        ids[(size_t)t * K + lane] = pick_e;
        gates[(size_t)t * K + lane] = ex / sum;
    }
}

namespace {

size_t moe_lds_bytes(int K, int I, int RT)
{
    return q8_stage_bytes(1, I / 32, false) + (size_t)K * RT * sizeof(float) +
           (65 + QG_MOE_WPB) * sizeof(int);
}

// Row blocks: about one workgroup per CU over all T tokens, RT rows each (a
// multiple of the wave tile rpw).
void moe_blocks(int T, int O, int rpw, int &RT, int &NB)
{
    const int want = (QG_MOE_WGS + T - 1) / T;
    const int per = (O + want - 1) / want;
    RT = (per + rpw - 1) / rpw * rpw;
    NB = (O + RT - 1) / RT;
}

template <int LPR, int R>
hipError_t launch_t(const uint8_t *w, const float *s, long long ws, long long ss, int E,
                    const int32_t *ids, const float *gates, int T, int K, const float *x,
                    float *y, int I, int O, int gs, int RT, int NB, int *err, hipStream_t st)
{
    const size_t lds = moe_lds_bytes(K, I, RT);
    auto kern = moe_i4g_stream<LPR, R, QG_MOE_PF>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(T * NB), dim3(64 * QG_MOE_WPB), lds, st, w, s, ws, ss, E, ids,
                       gates, T, K, x, y, I, O, (I + gs - 1) / gs,
                       Div20::make((uint32_t)(gs / 32)), RT, NB, err);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_topk(const void *w, const float *scales, long long w_stride,
                           long long s_stride, int E, const int32_t *ids, const float *gates,
                           int T, int K, const float *x, float *y, int I, int O, int gs,
                           int *err_flag, hipStream_t st)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int lpr = pick_lpr(I / 32 > 0 ? I / 32 : 1);
    const int rpw = (WAVE / lpr) * QG_MOE_R;
    int RT, NB;
    moe_blocks(T, O, rpw, RT, NB);
    const bool fast = K <= MOE_FAST_MAX_K && I % 32 == 0 && gs % 32 == 0 &&
                      ((uintptr_t)w & 15) == 0 && (w_stride & 15) == 0 &&
                      ((uintptr_t)x & 15) == 0 && moe_lds_bytes(K, I, RT) <= LDS_BUDGET;
    if (fast) {
        switch (lpr) {
        case 64:
            return launch_t<64, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x,
                                          y, I, O, gs, RT, NB, err_flag, st);
        case 32:
            return launch_t<32, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x,
                                          y, I, O, gs, RT, NB, err_flag, st);
        case 16:
            return launch_t<16, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x,
                                          y, I, O, gs, RT, NB, err_flag, st);
        case 8:
            return launch_t<8, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x,
                                          y, I, O, gs, RT, NB, err_flag, st);
        default:
            return launch_t<4, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y,
                                         I, O, gs, RT, NB, err_flag, st);
        }
    }
    const int wpb = 4;
    hipLaunchKernelGGL(moe_i4g_general, dim3((O + wpb - 1) / wpb), dim3(64 * wpb), 0, st, wb,
                       scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, err_flag);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float *logits, int T, int E, int ld, int K, int32_t *ids,
                              float *gates, hipStream_t st)
{
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, ld,
                       K, ids, gates);
    return hipGetLastError();
}

}  // namespace qg
