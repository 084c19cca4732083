// moe.hip -- routed-expert GEMV over grouped-int4 experts for gfx950.
//
//   y[t][o] = sum_k gates[t][k] * (W_{ids[t][k]} . x[t])[o],  k ascending
//
// (regolith audit "phase 0 + phase 2 m5 air validation", section 2.2: the
// gates are the selection probabilities renormalised over the selected
// experts; colibri PR #457, section 4: routed experts are grouped-int4.)
//
// One launch, no host round trip, no atomics:
//   * a workgroup owns RT consecutive output rows for every token;
//   * each wave reads the T*K ids (T*K <= 64) into its lanes and derives with
//     ballots the distinct valid experts (first-occurrence order) and, for
//     each, the set of tokens that chose it -- the routing never leaves the
//     device;
//   * work units are (distinct expert, sub-tile of rows), dealt round-robin
//     to the waves; a unit streams its rows of that expert once (dwordx4,
//     scale gather) and forms the dot products of every token that chose it,
//     with x of all tokens staged in LDS as for the dense grouped-int4 GEMV;
//     a wave's (unit, sweep) steps form one stream with PF sweeps of loads in
//     flight, crossing unit boundaries;
//   * a unit's row sums go to an LDS partial array [T][K][RT] for every slot
//     (t, k) that selected the expert; after a barrier the workgroup forms
//     y = sum_k gates * partial in ascending k (deterministic).
// An id outside [0, E) is never dereferenced: its token's row of y is NaN and
// the workspace error flag is set.
#include "qg_device.h"
#include "qg_launch.h"

#ifndef QG_MOE_R
#define QG_MOE_R 2
#endif
#ifndef QG_MOE_WPB
#define QG_MOE_WPB 16
#endif
#ifndef QG_MOE_PF
#define QG_MOE_PF 2
#endif
// sweeps issued before the activations are staged (at most PF)
#ifndef QG_MOE_PF0
#define QG_MOE_PF0 0
#endif

namespace qg {

constexpr int MOE_MAX_T = 8;
constexpr int MOE_FAST_MAX_TK = 64;

struct Routing {
    int e;            // this lane's id (lane < T*K), or -1
    uint64_t first;   // lanes holding the first occurrence of a valid id
    uint32_t mask;    // on a first-occurrence lane: tokens that chose the id
    uint32_t bad;     // tokens with an out-of-range id
    int nu;           // distinct valid experts
};

// The id of this lane's (token, slot), loaded unconditionally (clamped) so
// that the load can be issued ahead of others and waited for on its own.
__device__ __forceinline__ int load_id(const int32_t *__restrict__ ids, int T, int K)
{
    const int lane = threadIdx.x & 63;
    return ids[min(lane, T * K - 1)];
}

// Every lane of the wave calls this with its load_id() value (wave-uniform
// results except e / mask).
__device__ __forceinline__ Routing route_ids(int id, int T, int K, int E)
{
    const int lane = threadIdx.x & 63;
    const int TK = T * K;
    Routing rt;
    rt.e = lane < TK ? id : -1;
    const bool in = lane < TK;
    const bool valid = in && rt.e >= 0 && rt.e < E;
    bool first = valid;
    uint32_t mask = 0;
    // slot q belongs to token tq = q / K, tracked incrementally (a division
    // per iteration would run on the scalar unit of every wave)
    for (int q = 0, tq = 0, kq = 0; q < TK; q++) {
        const int eq = __builtin_amdgcn_readlane(rt.e, q);
        if (eq == rt.e) {
            if (q < lane) first = false;
            mask |= 1u << tq;
        }
        if (++kq == K) {
            kq = 0;
            ++tq;
        }
    }
    rt.first = __ballot(first);
    rt.mask = mask;
    const uint64_t badl = __ballot(in && !valid);
    uint32_t bad = 0;
    for (int t = 0; t < T; t++)
        if ((badl >> (t * K)) & ((K == 64) ? ~0ull : ((1ull << K) - 1))) bad |= 1u << t;
    rt.bad = bad;
    rt.nu = __popcll(rt.first);
    return rt;
}

__device__ __forceinline__ Routing route(const int32_t *__restrict__ ids, int T, int K, int E)
{
    return route_ids(load_id(ids, T, K), T, K, E);
}

// Lane holding the ui-th distinct expert.
__device__ __forceinline__ int unique_lane(const Routing &rt, int ui)
{
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane ? (rt.first & ((1ull << lane) - 1)) : 0ull;
    const int idx = __popcll(below);
    const uint64_t sel = __ballot(((rt.first >> lane) & 1) && idx == ui);
    return __ffsll((long long)sel) - 1;
}

template <int LPR, int R, int PF>
__global__ __launch_bounds__(64 * QG_MOE_WPB) void moe_i4g_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, long long w_stride,
    long long s_stride, int E, const int32_t *__restrict__ ids, const float *__restrict__ gates,
    int T, int K, const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, int RT, int *__restrict__ err_flag)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    constexpr int PF0 = QG_MOE_PF0 < PF ? QG_MOE_PF0 : PF;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;
    f32x4 *xl = reinterpret_cast<f32x4 *>(lds_raw);                  // [T][8][NS]
    float *xs = reinterpret_cast<float *>(xl + (size_t)T * 8 * seg_stride(NU));  // [T][NU]
    float *part = xs + (size_t)T * NU;                               // [T][K][RT]
    int *ids_l = reinterpret_cast<int *>(part + (size_t)T * K * RT); // [64]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const int o0 = blockIdx.x * RT;
    const size_t rb = (size_t)I / 2;
    const int nit = (NU + LPR - 1) / LPR;
    const int nsub = RT / ROWS_PER_WAVE;

    // activations of all tokens are requested before any weight; every wave
    // has issued them before any wave issues a weight load
    // one wave per workgroup reads the ids (thousands of waves reading the
    // same line would queue on one L2 channel) and hands them over in LDS
    int id = 0;
    if (wave == 0) id = load_id(ids, T, K);
    const int total4 = T * NU * 8;
    constexpr int NPRE = 8;
    f32x4 xv[NPRE];
    const int rot = stage_rot(total4);
#pragma unroll
    for (int j = 0; j < NPRE; j++)
        xv[j] = ldx4(x, (uint32_t)stage_index((int)(threadIdx.x + j * blockDim.x), total4, rot));
    __builtin_amdgcn_sched_barrier(0);

    if (wave == 0) ids_l[lane] = id;
    // raw barrier (the activation loads stay in flight); the LDS write must
    // have landed before it
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const Routing rt = route_ids(ids_l[lane], T, K, E);
    if (blockIdx.x == 0 && threadIdx.x == 0) err_flag[0] = rt.bad ? 1 : 0;

    // this wave's units: i = wave + k * nwaves (k < my_units); a unit is
    // (distinct expert ui, row sub-tile st); steps s = k * nit + c
    const int nunits = rt.nu * nsub;
    const int my_units = wave < nunits ? (nunits - wave + nwaves - 1) / nwaves : 0;
    const int nsteps = my_units * nit;
    const int nsteps_pad = (nsteps + PF - 1) / PF * PF;

    struct Unit {
        int e, row0;
        uint32_t mask;
    };
    auto unit_of = [&](int k) {
        const int i = wave + k * nwaves;
        const int ui = i / nsub, st = i - ui * nsub;
        const int ql = unique_lane(rt, ui);
        Unit u;
        // a wave without units still issues its (clamped) prefetch: expert 0
        u.e = ql >= 0 ? __builtin_amdgcn_readlane(rt.e, ql) : 0;
        u.mask = ql >= 0 ? (uint32_t)__builtin_amdgcn_readlane((int)rt.mask, ql) : 0u;
        u.row0 = o0 + st * ROWS_PER_WAVE + sub * R;
        return u;
    };

    u32x4 wb[PF][R];
    float sb[PF][R];
    // fetch cursor (unit fk, sweep fc): the step whose loads are issued next.
    // It stops on the wave's last step, so the padded tail of the stream
    // re-issues that step's loads instead of branching around them.
    const Unit u0 = unit_of(0);
    int fk = 0, fc = 0;
    Unit fu = u0;
    auto fetch = [&](int j) {
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
        if (fc + 1 < nit) {
            ++fc;
        } else if (fk + 1 < my_units) {
            fc = 0;
            fu = unit_of(++fk);
        }
    };

    // only PF0 sweeps go out before the activations are staged: a flood of
    // streaming weight requests is served ahead of the activation reads
#pragma unroll
    for (int j = 0; j < PF0; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);

    // stage activations
    const int cpv = NU * 8;
#pragma unroll
    for (int j = 0; j < NPRE; j++) {
        const int f = threadIdx.x + j * blockDim.x;
        int t, rem;
        split_f<MOE_MAX_T>(stage_index(f, total4, rot), cpv, t, rem);
        XStagePut(xv[j], f < total4, t, rem, NU, xl, xs);
    }
    const int nrest = (total4 - NPRE * (int)blockDim.x + (int)blockDim.x - 1) / (int)blockDim.x;
    for (int it = 0; it < nrest; it++) {
        const int f = threadIdx.x + (NPRE + it) * blockDim.x;
        const int g = stage_index(f, total4, rot);
        int t, rem;
        split_f<MOE_MAX_T>(g, cpv, t, rem);
        XStagePut(ldx4(x, (uint32_t)g), f < total4, t, rem, NU, xl, xs);
    }
    __syncthreads();
#pragma unroll
    for (int j = PF0; j < PF; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);

    float acc[MOE_MAX_T][R];
#pragma unroll
    for (int t = 0; t < MOE_MAX_T; t++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[t][r] = 0.0f;

    // consume cursor (unit ck, sweep cc)
    int ck = 0, cc = 0;
    Unit cu = u0;
    auto consume = [&](int s, int j) {
        if (s >= nsteps) return;                       // padding (wave-uniform)
        const int u = cc * LPR + sl;
        const bool valid = u < NU;
        const int uu = valid ? u : 0;
#pragma unroll
        for (int t = 0; t < MOE_MAX_T; t++) {
            if (t < T && ((cu.mask >> t) & 1)) {       // wave-uniform
                const f32x4 *xt = xl + (size_t)t * 8 * seg_stride(NU);
                const float m8xs = -8.0f * xs[(size_t)t * NU + uu];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float p = nib_chunk_dot(wb[j][r], xt, NU, uu);
                    const float tv = __builtin_fmaf(p, NIB_XSCALE, m8xs);
                    acc[t][r] = __builtin_fmaf(valid ? sb[j][r] : 0.0f, tv, acc[t][r]);
                }
            }
        }
        if (cc + 1 < nit) {
            ++cc;
            return;
        }
        // unit done: row sums -> partials of every slot that chose cu.e
#pragma unroll
        for (int t = 0; t < MOE_MAX_T; t++) {
            if (t < T && ((cu.mask >> t) & 1)) {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float v = sub_reduce<LPR>(acc[t][r]);
                    const int lr = cu.row0 + r - o0;
                    for (int kk = 0; kk < K; kk++) {
                        const int ek = __builtin_amdgcn_readlane(rt.e, t * K + kk);
                        if (ek == cu.e && sl == LPR - 1 && cu.row0 + r < O)
                            part[((size_t)t * K + kk) * RT + lr] = v;
                    }
                    acc[t][r] = 0.0f;
                }
            }
        }
        cc = 0;
        if (++ck < my_units) cu = unit_of(ck);
    };

    const int nrounds = nsteps_pad / PF;
    for (int rd = 0; rd + 1 < nrounds; rd++) {
#pragma unroll
        for (int j = 0; j < PF; j++) {
            const int s = rd * PF + j;
            consume(s, j);
            fetch(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (nrounds > 0) {
#pragma unroll
        for (int j = 0; j < PF; j++) consume((nrounds - 1) * PF + j, j);
    }
    __syncthreads();

    // combine in ascending k
    for (int idx = threadIdx.x; idx < T * RT; idx += blockDim.x) {
        const int t = idx / RT, i = idx - t * RT;
        const int row = o0 + i;
        if (row >= O) continue;
        float v;
        if ((rt.bad >> t) & 1) {
            v = __builtin_nanf("");
        } else {
            v = 0.0f;
            for (int kk = 0; kk < K; kk++)
                v = __builtin_fmaf(gates[t * K + kk], part[((size_t)t * K + kk) * RT + i], v);
        }
        y[(size_t)t * O + row] = v;
    }
}

// General kernel: any shape the streaming kernel does not take (T*K > 64,
// unaligned rows or strides, LDS too small).  One wave per output row; each
// (t, k) dot product is formed from per-weight f32 decodes, combined in
// ascending k.  Also sets the error flag (block 0).
__global__ __launch_bounds__(256) void moe_i4g_general(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, long long w_stride,
    long long s_stride, int E, const int32_t *__restrict__ ids, const float *__restrict__ gates,
    int T, int K, const float *__restrict__ x, float *__restrict__ y, int I, int O, int gs,
    int *__restrict__ err_flag)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        int bad = 0;
        for (int p = 0; p < T * K; p++) bad |= (ids[p] < 0 || ids[p] >= E);
        err_flag[0] = bad;
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

namespace {

size_t moe_lds_bytes(int T, int K, int I, int RT)
{
    return (size_t)T * ((size_t)8 * seg_stride(I / 32) * sizeof(f32x4) + (I / 32) * sizeof(float)) +
           (size_t)T * K * RT * sizeof(float) + 64 * sizeof(int);
}

template <int LPR, int R>
hipError_t launch_t(const uint8_t *w, const float *s, long long ws, long long ss, int E,
                    const int32_t *ids, const float *gates, int T, int K, const float *x,
                    float *y, int I, int O, int gs, int RT, int *err, hipStream_t st)
{
    const size_t lds = moe_lds_bytes(T, K, I, RT);
    auto kern = moe_i4g_stream<LPR, R, QG_MOE_PF>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    const int blocks = (O + RT - 1) / RT;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * QG_MOE_WPB), lds, st, w, s, ws, ss, E, ids,
                       gates, T, K, x, y, I, O, (I + gs - 1) / gs,
                       Div20::make((uint32_t)(gs / 32)), RT, err);
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
    const int R = QG_MOE_R;
    const int rpw = (WAVE / lpr) * R;
    // rows per workgroup: a multiple of the wave tile, about one workgroup per CU
    const int per_cu = (O + 255) / 256;
    const int RT = ((per_cu + rpw - 1) / rpw) * rpw;
    const bool fast = T * K <= MOE_FAST_MAX_TK && I % 32 == 0 && gs % 32 == 0 &&
                      ((uintptr_t)w & 15) == 0 && (w_stride & 15) == 0 &&
                      ((uintptr_t)x & 15) == 0 && moe_lds_bytes(T, K, I, RT) <= LDS_BUDGET;
    if (fast) {
        switch (lpr) {
        case 64: return launch_t<64, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, RT, err_flag, st);
        case 32: return launch_t<32, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, RT, err_flag, st);
        case 16: return launch_t<16, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, RT, err_flag, st);
        case 8: return launch_t<8, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, RT, err_flag, st);
        default: return launch_t<4, QG_MOE_R>(wb, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, RT, err_flag, st);
        }
    }
    const int wpb = 4;
    hipLaunchKernelGGL(moe_i4g_general, dim3((O + wpb - 1) / wpb), dim3(64 * wpb), 0, st, wb,
                       scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs, err_flag);
    return hipGetLastError();
}

}  // namespace qg
