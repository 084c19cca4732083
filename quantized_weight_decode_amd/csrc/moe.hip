// moe.hip -- routed-expert GEMV over grouped-int4 experts for gfx950.
//
//   y[t][o] = sum_k gates[t][k] * (W_{ids[t][k]} . x[t])[o],  k ascending
//
// (regolith audit "phase 0 + phase 2 m5 air validation", section 2.2: the
// gates are the selection probabilities renormalised over the selected
// experts; colibri PR #457, section 4: routed experts are grouped-int4.)
//
// One launch, no host round trip, no global atomics, and every distinct
// expert of the call streamed exactly once:
//   * workgroup b owns RT consecutive output rows for every token; the NB
//     workgroups cover about one CU each;
//   * it stages the activations of all tokens in LDS as the dense
//     grouped-int4 GEMV does (per-chunk fixed-point digits for the 4-bit
//     integer dot product); a token whose activations hold an infinity or
//     NaN, or a dynamic range the fixed point cannot carry precisely enough,
//     is multiplied per element in f32 after the stream instead;
//   * one wave reads the T*K ids (lane l holds slot l = t*K + k), finds with
//     ballots the distinct valid experts in first-occurrence order, and hands
//     both over in LDS -- the routing never leaves the device;
//   * work units are (distinct expert, sub-tile of rows); a unit streams its
//     rows of that expert once (dwordx4, scale gather) and multiplies every
//     token that selected the expert with the same weight registers; each
//     wave starts on one unit and takes the next free one from an LDS counter
//     when it is done, and a wave's (unit, sweep) steps form one stream with
//     PF sweeps of loads in flight, crossing unit boundaries;
//   * a unit's row sums go to an LDS partial array [T*K][RT] for every slot
//     that selected the expert (a duplicated id is streamed once and counted
//     per slot); after a barrier the workgroup forms y[t] = sum_k gates *
//     partial in ascending k (deterministic).
// An id outside [0, E) is never dereferenced: its token's row of y is NaN and
// the token's error flag in the workspace is set.  Tokens beyond what the LDS
// stages at once run in groups of launches (an expert shared across groups is
// then read once per group).
#include "qg_device.h"
#include "qg_launch.h"

#ifndef QG_MOE_R
#define QG_MOE_R 2
#endif
#ifndef QG_MOE_WPB
#define QG_MOE_WPB 8
#endif
// workgroups per launch the row blocking aims at
#ifndef QG_MOE_WGS
#define QG_MOE_WGS 256
#endif
#ifndef QG_MOE_PF
#define QG_MOE_PF 3
#endif
// ring slots filled before the activations are converted
#ifndef QG_MOE_EARLY
#define QG_MOE_EARLY 2
#endif

namespace qg {

constexpr int MOE_MAX_T = 8;
constexpr int MOE_FAST_MAX_TK = 64;   // slots t*K + k held by one wave's lanes

// Lane holding the ui-th set bit of a wave-uniform lane mask (-1 if none).
__device__ __forceinline__ int nth_lane(uint64_t m, int ui)
{
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane ? (m & ((1ull << lane) - 1)) : 0ull;
    const uint64_t sel = __ballot(((m >> lane) & 1) && __popcll(below) == ui);
    return __ffsll((long long)sel) - 1;
}

// The workgroup's rows for every (distinct expert, selecting slot) pair of the
// tokens in tokm with per-element f32 products, ((q - 8) * s) * x: the path of
// tokens whose activations hold an infinity or NaN, or too wide a dynamic
// range for the staged fixed point.  Wave w takes units w, w + WPB, ... of
// the (distinct expert ui, lane-group row) units; each writes the partials of
// the slots that chose the expert, as the streaming path does.
template <int LPR, int R>
__device__ __noinline__ void moe_rows_plain(const uint8_t *__restrict__ w,
                                            const float *__restrict__ scales, long long w_stride,
                                            long long s_stride, const float *__restrict__ x,
                                            int I, int O, int ng, Div20 div_cpg, int RT, int o0,
                                            int K, int TK, uint64_t firstm, int e, float *part,
                                            uint32_t tokm)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / LPR, sl = lane % LPR;
    const int NU = I / 32;
    const size_t rb = (size_t)I / 2;
    const int nsub = RT / ROWS_PER_WAVE;
    const int nunits = __popcll(firstm) * nsub;
#pragma unroll 1
    for (int i = wave; i < nunits; i += QG_MOE_WPB) {
        const int ui = i / nsub, st = i - ui * nsub;
        const int ql = nth_lane(firstm, ui);
        const int ue = __builtin_amdgcn_readlane(e, ql);
        const uint64_t slots = __ballot(lane < TK && e == ue);
        const uint8_t *we = w + (size_t)ue * (size_t)w_stride;
        const float *se = scales + (size_t)ue * (size_t)s_stride;
        const int row0 = o0 + st * ROWS_PER_WAVE + sub * R;
#pragma unroll 1
        for (int q = 0; q < TK; q++) {
            if (!((slots >> q) & 1ull)) continue;   // wave-uniform
            const int t = q / K;
            if (!((tokm >> t) & 1u)) continue;
            // the first slot of token t that chose the expert computes; the
            // token's other such slots copy it
            if (q % K > 0 && ((slots >> (t * K)) & ((1ull << (q % K)) - 1))) continue;
#pragma unroll 1
            for (int r = 0; r < R; r++) {
                const int row = min(row0 + r, O - 1);
                float acc = 0.0f;
                for (int u = sl; u < NU; u += LPR)
                    acc += nib_chunk_plain(*reinterpret_cast<const u32x4 *>(we + (size_t)row * rb +
                                                                            (size_t)u * 16),
                                           se[(size_t)row * ng + div_cpg((uint32_t)u)],
                                           x + (size_t)t * I + (size_t)u * 32);
                const float v = sub_reduce<LPR>(acc);
                if (sl == LPR - 1 && row0 + r < O)
                    for (int k = 0; k < K; k++)
                        if ((slots >> (t * K + k)) & 1ull)
                            part[(size_t)(t * K + k) * RT + row0 + r - o0] = v;
            }
        }
    }
}

// TM: the most tokens one launch stages (T <= TM at run time).
template <int TM, int LPR, int R, int PF>
__global__ __launch_bounds__(64 * QG_MOE_WPB) void moe_i4g_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ scales, long long w_stride,
    long long s_stride, int E, const int32_t *__restrict__ ids, const float *__restrict__ gates,
    int T, int K, const float *__restrict__ x, float *__restrict__ y, int I, int O, int ng,
    Div20 div_cpg, int RT, int *__restrict__ err_flag, int nflag)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    constexpr int MOE_EARLY = QG_MOE_EARLY < PF ? QG_MOE_EARLY : PF;
    constexpr int NT = 64 * QG_MOE_WPB;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;
    const int TK = T * K;
    u32x4 *xq = reinterpret_cast<u32x4 *>(lds_raw);                      // [T][6][NU]
    float *xc = reinterpret_cast<float *>(xq + (size_t)T * 6 * NU);       // [T][NU]
    unsigned char *tail = lds_raw + q8_verdict_offset(T, NU, false);
    void *vlds = tail;                                                    // stage_verdict
    float *part = reinterpret_cast<float *>(tail + verdict_bytes(QG_MOE_WPB, TM));  // [TK][RT]
    int *ids_l = reinterpret_cast<int *>(part + (size_t)TK * RT);         // [64]
    uint32_t *meta = reinterpret_cast<uint32_t *>(ids_l + 64);            // slot masks [4]
    int *ctr = reinterpret_cast<int *>(meta + 4);                         // next unit
    float *xacc_base = reinterpret_cast<float *>(ctr + 1);   // [WPB][TM-1][R][64], zeroed

    const int o0 = blockIdx.x * RT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int nwaves = QG_MOE_WPB;
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const size_t rb = (size_t)I / 2;
    const int nit = (NU + LPR - 1) / LPR;
    const int nsub = RT / ROWS_PER_WAVE;

    // the ids (wave 0), then the activations, before any weight load.  One
    // wave reads the ids (thousands of waves reading one line would queue on
    // one L2 channel); lane l holds slot l = t*K + k.  The activation loads
    // behind it are unconditional, so its wait for the ids counts them and
    // lets them stay in flight.
    // two items per token and thread cover 7168 columns (at most eight up front)
    constexpr int NPRE = 2 * TM < 8 ? 2 * TM : 8;
    XStageQ<TM, NPRE, NT> xst;
    const int items = T * NU * 4;
    const int ev = wave == 0 && lane < TK ? ids[min(lane, TK - 1)] : -1;
    __builtin_amdgcn_sched_barrier(0);
    xst.load_all(x, items);
    __builtin_amdgcn_sched_barrier(0);
    if (wave == 0) {
        // the distinct valid experts in first-occurrence order, one pass per
        // distinct expert; ids and slot masks are handed over in LDS
        const bool ok = lane < TK && ev >= 0 && ev < E;
        uint64_t rem = __ballot(ok), fm = 0;
        while (rem) {
            const int q = __builtin_ctzll(rem);
            const int v = __builtin_amdgcn_readlane(ev, q);
            fm |= 1ull << q;
            rem &= ~__ballot(ev == v);
        }
        const uint64_t bm = __ballot(lane < TK && !ok);
        ids_l[lane] = ev;
        if (lane == 0) {
            meta[0] = (uint32_t)fm;
            meta[1] = (uint32_t)(fm >> 32);
            meta[2] = (uint32_t)bm;
            meta[3] = (uint32_t)(bm >> 32);
        }
    }
    if (threadIdx.x == 0) *ctr = nwaves;
#pragma unroll
    for (int m = 0; m < (TM - 1) * R; m++)
        xacc_base[((size_t)wave * (TM - 1) * R + m) * 64 + lane] = 0.0f;
    // raw barrier (the activation loads stay in flight); the LDS write must
    // have landed before it
    __builtin_amdgcn_s_waitcnt(QG_WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // the slots' ids, the first slot of each distinct valid expert, and the
    // slots holding an id outside [0, E)
    // (each half zero-extended; only the TK slot lanes can be set)
    const int e = lane < TK ? ids_l[lane] : -1;
    const uint64_t slotm = TK >= 64 ? ~0ull : (1ull << TK) - 1;
    auto mask64 = [&](int i) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)meta[i]);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)meta[i + 1]);
        return ((uint64_t)hi << 32 | (uint64_t)lo) & slotm;
    };
    const uint64_t firstm = mask64(0);
    const uint64_t badm = mask64(2);
    uint32_t badtok = 0;                                   // tokens with a bad id
    for (int t = 0; t < T; t++)
        if ((badm >> (t * K)) & (K == 64 ? ~0ull : ((1ull << K) - 1))) badtok |= 1u << t;
    // error flags of this launch's tokens, and zeros for the flag slots past
    // the call's last token (nflag slots in all)
    if (blockIdx.x == 0 && (int)threadIdx.x < nflag)
        err_flag[threadIdx.x] = (int)threadIdx.x < T ? (int)((badtok >> threadIdx.x) & 1u) : 0;

    // Work units are (distinct expert ui, row sub-tile st), numbered
    // i = ui * nsub + st.  Wave w starts on unit w; each later unit goes to
    // whichever wave asks first (an LDS counter), so waves that the SIMDs
    // serve faster take more units and the workgroup finishes together.
    const int nunits = __popcll(firstm) * nsub;

    struct Unit {
        int e, row0;
        uint64_t slots;   // slots (lanes) that selected the expert
        uint32_t toks;    // tokens with such a slot
    };
    auto unit_of = [&](int i) {
        const int ui = i / nsub, st = i - ui * nsub;
        const int ql = nth_lane(firstm, ui);
        Unit u;
        // past the last unit (or none): expert 0 and no tokens, so the clamped
        // loads stay valid and nothing is multiplied
        const bool any = ql >= 0 && i < nunits;
        u.e = any ? __builtin_amdgcn_readlane(e, ql) : 0;
        u.row0 = o0 + st * ROWS_PER_WAVE + sub * R;
        u.slots = any ? __ballot(lane < TK && e == u.e) : 0ull;
        u.toks = 0;
#pragma unroll
        for (int t = 0; t < TM; t++)
            if (t < T && ((u.slots >> (t * K)) & (K == 64 ? ~0ull : ((1ull << K) - 1))))
                u.toks |= 1u << t;
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
    // (unit >= nunits: nothing; the loads read the activations)
    int slot_u[PF], slot_c[PF];
    uint32_t slot_t[PF];
    // fetch cursor: unit fi, sweep fc
    int fi = wave, fc = 0;
    Unit fu = unit_of(min(fi, nunits > 0 ? nunits - 1 : 0));
    auto fetch = [&](int j) {
        slot_u[j] = fi;
        slot_c[j] = fc;
        slot_t[j] = fi < nunits ? fu.toks : 0u;
        // past the wave's last unit the refills (unconditional, so that the
        // waits count exactly) read the activations, which the caches hold,
        // instead of streaming weights from memory again
        const bool live = fi < nunits;
        const uint8_t *we = live ? w + (size_t)fu.e * (size_t)w_stride
                                 : reinterpret_cast<const uint8_t *>(x);
        const float *se = live ? scales + (size_t)fu.e * (size_t)s_stride : x;
        const int u = min(fc * LPR + sl, NU - 1);
        const uint32_t g = div_cpg((uint32_t)u);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int row = live ? min(fu.row0 + r, O - 1) : 0;
            wb[j][r] = ld_stream(reinterpret_cast<const u32x4 *>(we + (size_t)row * rb +
                                                                 (uint32_t)u * 16u));
            // the scales as ordinary cached loads: one 128-byte line of them
            // serves several sweeps, and with the streaming hint it was often
            // gone before the next one.  4 tokens x top-8 of 256 experts of
            // 2048 x 7168: 1.037 -> 1.004 of the algorithmic bytes fetched,
            // time within +-2 % (mean of four interleaved runs +0.6 %); one
            // token x top-32: 2-4 % faster
            sb[j][r] = se[(size_t)row * ng + g];
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
                    fi = nunits;   // done
                }
            }
        }
    };

    // the first QG_MOE_EARLY sweeps go out before the activations are
    // converted, the rest of the ring once they are staged
#pragma unroll
    for (int j = 0; j < MOE_EARLY; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t xbad = xst.store(x, items, NU, reinterpret_cast<uint32_t *>(xq), xc, nullptr);
    // tokens whose activations hold an infinity or NaN, or too wide a dynamic
    // range for the fixed point: their products are formed per element after
    // the stream (kept out of the streaming loop)
    const uint32_t plainm = (uint32_t)stage_verdict<QG_MOE_WPB, TM>(xbad, xst.dsum, vlds);

#pragma unroll
    for (int j = MOE_EARLY; j < PF; j++) fetch(j);
    __builtin_amdgcn_sched_barrier(0);

    // The unit's first token accumulates in registers, with running digit
    // sums (q8_dot_run); any further token (an expert several tokens chose)
    // accumulates in this lane's slots of xacc, [wave][extra token][row][lane]
    float acc[R];
    uint32_t P[R][6], V[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        acc[r] = 0.0f;
        V[r] = 0;
#pragma unroll
        for (int k = 0; k < 6; k++) P[r][k] = 0;
    }
    float *xacc = xacc_base + (size_t)wave * (TM - 1) * R * 64 + lane;

    // the row sums of token t (slots km of it chose the expert) -> partials
    auto emit = [&](const Unit &cu, int t, float v, int r) {
        uint64_t km = cu.slots >> (t * K);
        if (K < 64) km &= (1ull << K) - 1;
        const int lr = cu.row0 + r - o0;
        const bool st = sl == LPR - 1 && cu.row0 + r < O;
        for (uint64_t m = km; m; m &= m - 1) {
            const int k = __builtin_ctzll(m);
            if (st) part[(size_t)(t * K + k) * RT + lr] = v;
        }
    };

    auto consume = [&](int j) {
        const int ci = slot_u[j];
        if (ci >= nunits) return;                      // nothing (wave-uniform)
        // tokens on the per-element path are formed after the stream
        const uint32_t toks = slot_t[j] & ~plainm;
        if (!toks) return;
        const int u = slot_c[j] * LPR + sl;
        const bool in_row = u < NU;
        const int uu = in_row ? u : 0;
        const int t0 = __builtin_ctz(toks);
        uint32_t wx[R][4];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int d = 0; d < 4; d++) wx[r][d] = wb[j][r][d] ^ Q8_NIB_FLIP;
        {
            const u32x4 *xt = xq + (size_t)t0 * 6 * NU;
            u32x4 L[6];
#pragma unroll
            for (int k = 0; k < 6; k++) L[k] = xt[k * NU + uu];
            const float cs = in_row ? xc[(size_t)t0 * NU + uu] : 0.0f;
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int dv = q8_dot_run(wx[r], L, P[r], V[r]);
                acc[r] = __builtin_fmaf(sb[j][r] * cs, (float)dv, acc[r]);
            }
        }
        // wave-uniform, usually 0 (never with one token)
        const uint32_t more = TM > 1 ? toks & (toks - 1) : 0u;
        if (more) {
            int m = 0;
#pragma unroll 1
            for (uint32_t b = more; b; b &= b - 1, m++) {
                const int t = __builtin_ctz(b);
                const u32x4 *xt = xq + (size_t)t * 6 * NU;
                u32x4 L[6];
#pragma unroll
                for (int k = 0; k < 6; k++) L[k] = xt[k * NU + uu];
                const float cs = in_row ? xc[(size_t)t * NU + uu] : 0.0f;
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float *a = xacc + (size_t)(m * R + r) * 64;
                    *a = __builtin_fmaf(sb[j][r] * cs, (float)q8_dot(wx[r], L), *a);
                }
            }
        }
        if (slot_c[j] + 1 < nit) return;
        // unit done: row sums -> partials of every slot that chose its expert
        const Unit cu = unit_of(ci);
#pragma unroll
        for (int r = 0; r < R; r++) {
            emit(cu, t0, sub_reduce<LPR>(acc[r]), r);
            acc[r] = 0.0f;
        }
        if (more) {
            int m = 0;
#pragma unroll 1
            for (uint32_t b = more; b; b &= b - 1, m++) {
                const int t = __builtin_ctz(b);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float *a = xacc + (size_t)(m * R + r) * 64;
                    emit(cu, t, sub_reduce<LPR>(*a), r);
                    *a = 0.0f;
                }
            }
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
    if (plainm) {
        // tokens whose activations the fixed point cannot carry: per element
        moe_rows_plain<LPR, R>(w, scales, w_stride, s_stride, x, I, O, ng, div_cpg, RT, o0, K, TK,
                               firstm, e, part, plainm);
        __syncthreads();
    }

    // y[t] = sum_k gates * partial, ascending k
    for (int i = threadIdx.x; i < T * RT; i += NT) {
        const int t = i / RT, r = i - t * RT;
        const int row = o0 + r;
        if (row >= O) continue;
        float v;
        if ((badtok >> t) & 1u) {
            v = __builtin_nanf("");
        } else {
            v = 0.0f;
            for (int kk = 0; kk < K; kk++)
                v = __builtin_fmaf(gates[t * K + kk], part[(size_t)(t * K + kk) * RT + r], v);
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

// LDS of one launch staging T tokens (kernel instance TM >= T)
size_t moe_lds_bytes(int TM, int T, int K, int I, int RT)
{
    return q8_verdict_offset(T, I / 32, false) + verdict_bytes(QG_MOE_WPB, TM) +
           (size_t)T * K * RT * sizeof(float) + 69 * sizeof(int) +
           (size_t)QG_MOE_WPB * (TM - 1) * QG_MOE_R * 64 * sizeof(float);
}

// Row blocks: about QG_MOE_WGS workgroups, RT rows each (a multiple of the
// wave tile rpw).
void moe_blocks(int O, int rpw, int &RT, int &NB)
{
    const int per = (O + QG_MOE_WGS - 1) / QG_MOE_WGS;
    RT = (per + rpw - 1) / rpw * rpw;
    NB = (O + RT - 1) / RT;
}

template <int TM, int LPR>
hipError_t launch_t(const uint8_t *w, const float *s, long long ws, long long ss, int E,
                    const int32_t *ids, const float *gates, int T, int K, const float *x,
                    float *y, int I, int O, int gs, int RT, int NB, int *err, int nflag,
                    hipStream_t st)
{
    const size_t lds = moe_lds_bytes(TM, T, K, I, RT);
    auto kern = moe_i4g_stream<TM, LPR, QG_MOE_R, QG_MOE_PF>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(NB), dim3(64 * QG_MOE_WPB), lds, st, w, s, ws, ss, E, ids, gates,
                       T, K, x, y, I, O, (I + gs - 1) / gs, Div20::make((uint32_t)(gs / 32)), RT,
                       err, nflag);
    return hipGetLastError();
}

template <int TM>
hipError_t launch_tm(int lpr, const uint8_t *w, const float *s, long long ws, long long ss, int E,
                     const int32_t *ids, const float *gates, int T, int K, const float *x,
                     float *y, int I, int O, int gs, int RT, int NB, int *err, int nflag,
                     hipStream_t st)
{
    switch (lpr) {
    case 64: return launch_t<TM, 64>(w, s, ws, ss, E, ids, gates, T, K, x, y, I, O, gs, RT, NB, err, nflag, st);
    case 32: return launch_t<TM, 32>(w, s, ws, ss, E, ids, gates, T, K, x, y, I, O, gs, RT, NB, err, nflag, st);
    case 16: return launch_t<TM, 16>(w, s, ws, ss, E, ids, gates, T, K, x, y, I, O, gs, RT, NB, err, nflag, st);
    case 8: return launch_t<TM, 8>(w, s, ws, ss, E, ids, gates, T, K, x, y, I, O, gs, RT, NB, err, nflag, st);
    default: return launch_t<TM, 4>(w, s, ws, ss, E, ids, gates, T, K, x, y, I, O, gs, RT, NB, err, nflag, st);
    }
}

inline int tm_of(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8)); }

}  // namespace

hipError_t launch_moe_topk(const void *w, const float *scales, long long w_stride,
                           long long s_stride, int E, const int32_t *ids, const float *gates,
                           int T, int K, const float *x, float *y, int I, int O, int gs,
                           int *err_flag, hipStream_t st)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    // Lanes per row: the widest with the fewest idle lanes, narrowed (not
    // below 8) until a unit -- one expert's rows of a wave -- spans at least
    // two sweeps, and from two to four where the workgroups then still cover
    // 7/8 of the CUs.  Each unit pays its own bookkeeping (the next unit from the LDS
    // counter, its expert and tokens, the row sums), so one-sweep units lose:
    // at 7168 x 2048 experts (4 tokens x top-8 of 256) 76.3 us with 64 lanes,
    // 57.2 us with 32, 54.4 us with 16.  At 768 x 2048, 16 lanes would leave
    // 96 workgroups: 19.1 us against 15.4 us with 32 (18.1 us with 64).  At
    // 4096 x 1536 three-sweep units stay: 25.5 us against 26.1 us with six.
    const int NU = I / 32 > 0 ? I / 32 : 1;
    int lpr = pick_lpr_wide(NU);   // 2048 x 1408 experts: 41.5 -> 17.6 us
    while (lpr > 8 && NU / lpr < 2) lpr /= 2;
    if (lpr > 8 && NU / lpr <= 2) {
        int RT2, NB2;
        moe_blocks(O, (WAVE / (lpr / 2)) * QG_MOE_R, RT2, NB2);
        if (8L * NB2 >= 7L * cu_count()) lpr /= 2;
    }
    const int rpw = (WAVE / lpr) * QG_MOE_R;
    int RT, NB;
    moe_blocks(O, rpw, RT, NB);
    // tokens per launch: all of them if the LDS stages them together
    int tg = T;
    while (tg > 1 && moe_lds_bytes(tm_of(tg), tg, K, I, RT) > LDS_BUDGET) --tg;
    const bool fast = tg * K <= MOE_FAST_MAX_TK && I % 32 == 0 && gs % 32 == 0 &&
                      ((uintptr_t)w & 15) == 0 && (w_stride & 15) == 0 &&
                      ((uintptr_t)x & 15) == 0 && moe_lds_bytes(tm_of(tg), tg, K, I, RT) <= LDS_BUDGET;
    if (fast) {
        for (int t0 = 0; t0 < T; t0 += tg) {
            const int n = T - t0 < tg ? T - t0 : tg;
            const int32_t *ids_g = ids + (size_t)t0 * K;
            const float *gates_g = gates + (size_t)t0 * K;
            const float *x_g = x + (size_t)t0 * I;
            float *y_g = y + (size_t)t0 * O;
            int *err_g = err_flag + t0;
            // flag slots this launch writes: its tokens, and for the last one
            // every slot up to MOE_MAX_T
            const int nflag = t0 + n >= T ? MOE_MAX_T - t0 : n;
            hipError_t e;
            switch (tm_of(n)) {
            case 1: e = launch_tm<1>(lpr, wb, scales, w_stride, s_stride, E, ids_g, gates_g, n, K, x_g, y_g, I, O, gs, RT, NB, err_g, nflag, st); break;
            case 2: e = launch_tm<2>(lpr, wb, scales, w_stride, s_stride, E, ids_g, gates_g, n, K, x_g, y_g, I, O, gs, RT, NB, err_g, nflag, st); break;
            case 4: e = launch_tm<4>(lpr, wb, scales, w_stride, s_stride, E, ids_g, gates_g, n, K, x_g, y_g, I, O, gs, RT, NB, err_g, nflag, st); break;
            default: e = launch_tm<8>(lpr, wb, scales, w_stride, s_stride, E, ids_g, gates_g, n, K, x_g, y_g, I, O, gs, RT, NB, err_g, nflag, st); break;
            }
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
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
