// mq4v2.hip -- MQ4-v2 GEMV, decode and the FWHT-256 pre-rotation for gfx950.
//
// Format (hipfire "MQ4 V2", sections 2 and 4): per row, I/256 groups of 136
// bytes, little-endian.  Dword 0 = {fp16 scale, fp16 zero} of weights 0..127,
// dword 1 = the pair of weights 128..255, bytes 8..135 = 128 payload bytes
// with weight j in nibble j (low nibble first).  weight = q * scale + zero,
// the half chosen from the weight's index (j >= 128), never from a lane id.
//
// Streaming kernel: the lane chunk is 16 payload bytes (32 weights), chunk
// u = 8 g + p covers payload bytes 16p..16p+15 of group g, so half = (p >= 4)
// follows from the chunk's own byte offset.  The chunk is fetched with one
// 16-byte load at an 8-byte-aligned address (136 g + 8 + 16 p); the lane's
// header dword (+0 or +4) is a separate 4-byte load that hits the same lines.
// x is staged as for grouped int4 (per-chunk fixed-point digits, chunk scale
// c = 2^(E-21)) plus the chunk sums xsum = c * sum v.  A payload dword XOR
// 0x88888888 read as signed nibbles is q - 8, so the integer dot gives
// P = sum (q - 8) v and
//     sum w x~ = scale * c * P + (8 * scale + zero) * xsum,
// weight = q * scale + zero reassociated.  Activations holding an infinity or
// NaN, or too wide a dynamic range for the fixed point (stage_verdict), are
// multiplied per element in f32 instead (fma(q, scale, zero) * x).
#include "qg_device.h"
#include "qg_launch.h"

// Streaming for one vector: a ring of PF chunk-sweeps per lane, the first
// EARLY sweeps issued before the activations are converted; the tile (waves
// per workgroup, rows per lane group) is chosen per shape at launch.
// Measured on the 8192 x 8192 workload with the fused rotation (mean of six
// interleaved runs of 300 calls): 64 lanes x 2 rows x 16 waves with a ring
// of two and one early sweep 9.2 us; the same with a ring of four 9.4 us,
// and without the early sweep 10.3 us; two early sweeps 9.4 us; 32 lanes
// per row 10.1-10.2 us; 4 rows x 8 waves 10.1 us.
#ifndef QG_MQ4_PF
#define QG_MQ4_PF 2
#endif
// at most this many lanes per row for one vector
#ifndef QG_MQ4_LPR
#define QG_MQ4_LPR 64
#endif
// chunk-sweeps of weights issued before the activations are converted
#ifndef QG_MQ4_EARLY
#define QG_MQ4_EARLY 1
#endif
// waves per workgroup for several vectors (S times the LDS per workgroup)
#ifndef QG_MQ4_WPB_MULTI
#define QG_MQ4_WPB_MULTI 16
#endif
// activation items (8 columns each) each thread loads up front
#ifndef QG_MQ4_NPRE
#define QG_MQ4_NPRE 2
#endif

namespace qg {

constexpr int MQ4_FAST_MAX_S = 4;
constexpr int MQ4_GROUP_BYTES = 136;

// 16 bytes at an 8-byte-aligned address.
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));

// Unlike the other formats, MQ4 weights are read as ordinary cached loads,
// not with the streaming hint: each group's header dword is a second load
// from the lines its payload loads just fetched, and with the payload cached
// that second touch is served close to the CU.  8192 x 8192, interleaved,
// three boxes: 8.89-8.94 -> 8.54-8.57 us pre-rotated, 9.69-9.71 -> 9.55 us
// with the fused rotation; the same bytes fetched.  (Cached headers alone
// gained nothing; cached weights made i4g and fp8 5-8 % slower.)
__device__ __forceinline__ u32x4 load16_a8(const uint8_t *p)
{
    const u32x4_a8 v = *reinterpret_cast<const u32x4_a8 *>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}

// f32 sum over one chunk (x32 = x + 32u) of fma(q, scale, zero) * x: the
// plain definition's arithmetic, for activations holding an infinity or NaN.
__device__ __forceinline__ float mq4_chunk_plain(const u32x4 wv, float scl, float zro,
                                                 const float *__restrict__ x32)
{
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        float e[4], o[4];
        nib8(wv[d], e, o);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float we = __builtin_fmaf(e[k] * NIB_XSCALE, scl, zro);
            const float wo = __builtin_fmaf(o[k] * NIB_XSCALE, scl, zro);
            acc = __builtin_fmaf(we, x32[8 * d + 2 * k], acc);
            acc = __builtin_fmaf(wo, x32[8 * d + 2 * k + 1], acc);
        }
    }
    return acc;
}

// The group header formats that share the 136-byte geometry and the payload
// at bytes 8..135 (hipfire "MQ4 V2", sections 1b, 1e and 2):
//   MQ4_V2  fp16 {scale, zero} pair at +0 for weights 0..127, at +4 for 128..255
//   MQ4_V1  f32 scale at +0, f32 zero at +4, for all 256 weights (qt=13)
//   MQ4_C   one fp16 {scale, zero} pair at +0 for all 256 weights, zero pad at
//           +4 (MQ4C pad, qt=45)
// A fp16 pair holds the scale in its low half and the zero in its high half.
enum : int { MQ4_V2 = 0, MQ4_V1 = 1, MQ4_C = 2 };

template <int HF>
struct Mq4Hdr {
    typedef uint32_t T;
    // header of payload chunk p (16 bytes at +8 + 16p) of group gp
    __device__ __forceinline__ static T load(const uint8_t *gp, int p)
    {
        return *reinterpret_cast<const uint32_t *>(gp + (HF == MQ4_V2 && p >= 4 ? 4 : 0));
    }
    __device__ __forceinline__ static void decode(T h, float &sc, float &zp)
    {
        sc = f16_to_f32(h & 0xFFFFu);
        zp = f16_to_f32(h >> 16);
    }
};
template <>
struct Mq4Hdr<MQ4_V1> {
    typedef u32x2 T;
    __device__ __forceinline__ static T load(const uint8_t *gp, int)
    {
        return *reinterpret_cast<const u32x2 *>(gp);
    }
    __device__ __forceinline__ static void decode(T h, float &sc, float &zp)
    {
        // through scalars: __builtin_bit_cast of a vector element (h.y) is
        // compiled as a cast of element 0 by this compiler
        const uint32_t a = h[0], b = h[1];
        sc = __builtin_bit_cast(float, a);
        zp = __builtin_bit_cast(float, b);
    }
};

// The same header read byte by byte (any alignment), for weight j of the group.
template <int HF>
__device__ __forceinline__ void mq4_hdr_bytes(const uint8_t *gp, int j, float &sc, float &zp)
{
    auto le32 = [&](int off) {
        return (uint32_t)gp[off] | ((uint32_t)gp[off + 1] << 8) | ((uint32_t)gp[off + 2] << 16) |
               ((uint32_t)gp[off + 3] << 24);
    };
    if constexpr (HF == MQ4_V1) {
        sc = __builtin_bit_cast(float, le32(0));
        zp = __builtin_bit_cast(float, le32(4));
    } else {
        const uint32_t hd = le32(HF == MQ4_V2 && j >= 128 ? 4 : 0);
        sc = f16_to_f32(hd & 0xFFFFu);
        zp = f16_to_f32(hd >> 16);
    }
}

// Rows row0 .. row0 + R - 1 (those below O) of one lane group with the plain
// per-element arithmetic (x read from global memory).
template <int HF, int S, int LPR, int R>
__device__ __noinline__ void mq4_rows_plain(const uint8_t *__restrict__ w,
                                            const float *__restrict__ x, float *__restrict__ y,
                                            int I, int O, int row0, int sl)
{
    const int NU = I / 32;
    const size_t rowbytes = (size_t)(I / 256) * MQ4_GROUP_BYTES;
#pragma unroll 1
    for (int r = 0; r < R; r++) {
        const uint8_t *wr = w + (size_t)min(row0 + r, O - 1) * rowbytes;
        float acc[S];
#pragma unroll
        for (int t = 0; t < S; t++) acc[t] = 0.0f;
        for (int u = sl; u < NU; u += LPR) {
            const int g = u >> 3, p = u & 7;
            const uint8_t *gp = wr + (size_t)g * MQ4_GROUP_BYTES;
            const u32x4 wv = load16_a8(gp + 8 + 16 * p);
            float scl, zro;
            Mq4Hdr<HF>::decode(Mq4Hdr<HF>::load(gp, p), scl, zro);
#pragma unroll
            for (int t = 0; t < S; t++)
                acc[t] += mq4_chunk_plain(wv, scl, zro, x + (size_t)t * I + (size_t)u * 32);
        }
#pragma unroll
        for (int t = 0; t < S; t++) {
            const float v = sub_reduce<LPR>(acc[t]);
            if (sl == LPR - 1 && row0 + r < O) y[(size_t)t * O + row0 + r] = v;
        }
    }
}

// ROT: x is unrotated and the workgroup applies the FWHT-256 pre-rotation
// (signs, then H256 / 16 per block) while staging it; the rotated values are
// bit-identical to the stand-alone rotation kernel's.
template <int HF, int S, int LPR, int R, int PF, int WPB, bool ROT, int EARLY>
__global__ __launch_bounds__(64 * WPB) void mq4v2_gemv_stream(
    const uint8_t *__restrict__ w, const float *__restrict__ x, const int8_t *__restrict__ signs,
    float *__restrict__ y, int I, int O, int ntiles)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int NU = I / 32;
    u32x4 *xq = reinterpret_cast<u32x4 *>(lds_raw);                        // [S][6][NU]
    float *xc = reinterpret_cast<float *>(xq + (size_t)S * 6 * NU);        // [S][NU]
    float *xsm = xc + (size_t)S * NU;                                      // [S][NU]
    void *vlds = lds_raw + q8_verdict_offset(S, NU, true);                 // stage_verdict
    // ROT fallback: x_rot as f32 [S][I], over the staging area once it is unused
    float *xf = reinterpret_cast<float *>(lds_raw);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;
    const int sl = lane % LPR;
    const int tile = blockIdx.x * WPB + wave;
    const int row0 = tile * ROWS_PER_WAVE + sub * R;
    const size_t rowbytes = (size_t)(I / 256) * MQ4_GROUP_BYTES;
    const int nit = (NU + LPR - 1) / LPR;
    const int nit_pad = (nit + PF - 1) / PF * PF;

    const uint8_t *wr[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        wr[r] = w + (size_t)min(row0 + r, O - 1) * rowbytes;

    XStageQ<S, (S > 2 ? 4 : QG_MQ4_NPRE), 64 * WPB, true, ROT> xst;
    const int items = S * NU * 4;
    xst.load(x, items, signs, NU * 4);
    if constexpr (ROT) {
        // the early weight sweep waits for the activations: at 8192 x 8192
        // (interleaved, two boxes) 9.78 us against 9.89-9.92 us when the
        // sweep goes out at once and its requests queue ahead of other
        // workgroups' activation reads
        __builtin_amdgcn_s_waitcnt(QG_WAIT_VM0);
    }
    if constexpr (!ROT) {
        // every wave of the workgroup has issued its activation loads before
        // any wave issues weight loads (raw barrier: no drain).  Measured on
        // 8192 x 8192: 11.4 -> 11.0 us per step without the fused rotation,
        // 9.3 -> 9.55 us with it (its longer staging gains nothing from it)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }

    // payload chunk u: group u/8, bytes 8 + 16 (u%8); header dword +0 / +4
    typedef typename Mq4Hdr<HF>::T HdrT;
    u32x4 wb[PF][R];
    HdrT hb[PF][R];
    auto fetch = [&](int u, u32x4 *wv, HdrT *hv) {
        const int g = u >> 3, p = u & 7;
        const size_t goff = (size_t)g * MQ4_GROUP_BYTES;
#pragma unroll
        for (int r = 0; r < R; r++) {
            wv[r] = load16_a8(wr[r] + goff + 8 + 16 * p);
            hv[r] = Mq4Hdr<HF>::load(wr[r] + goff, p);
        }
    };

    // the first EARLY sweeps go out before the activations are converted, the
    // rest once they are staged: a flood of weight requests from every wave
    // at once is served ahead of later workgroups' activation reads
#pragma unroll
    for (int j = 0; j < EARLY; j++) fetch(min(j * LPR + sl, NU - 1), wb[j], hb[j]);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t bad =
        xst.store(x, items, NU, reinterpret_cast<uint32_t *>(xq), xc, xsm, signs);
    // non-finite activations or a dynamic range too wide for the fixed point
    const int plain = stage_verdict<WPB, S>(bad, xst.dsum, vlds);
    if (plain) {
        // the whole workgroup takes this branch; with ROT it first rebuilds
        // x_rot as f32 over the staging area (every wave has read the flags)
        if constexpr (ROT) {
            __syncthreads();
            xst.store_rotated_f32(x, items, NU, signs, xf);
            __syncthreads();
        }
        if (tile < ntiles) mq4_rows_plain<HF, S, LPR, R>(w, ROT ? xf : x, y, I, O, row0, sl);
        return;
    }
    if (tile >= ntiles) return;
#pragma unroll
    for (int j = EARLY; j < PF; j++) fetch(min(j * LPR + sl, NU - 1), wb[j], hb[j]);
    __builtin_amdgcn_sched_barrier(0);

    float acc[S][R];
#pragma unroll
    for (int t = 0; t < S; t++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[t][r] = 0.0f;
    // running digit sums per vector and row (see q8_dot_run) where the
    // registers allow (16-wave workgroups have 128); otherwise fresh sums
    // per chunk
    constexpr bool RUN = S == 1 || (S == 2 && R <= 2);
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

    auto consume = [&](int c, int j) {
        const int u = c * LPR + sl;
        const bool valid = u < NU;
        const int uu = valid ? u : 0;
        float scl[R], zro[R];
#pragma unroll
        for (int r = 0; r < R; r++) Mq4Hdr<HF>::decode(hb[j][r], scl[r], zro[r]);
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
            const float xsum = valid ? xsm[(size_t)t * NU + uu] : 0.0f;
#pragma unroll
            for (int r = 0; r < R; r++) {
                int dv;
                if constexpr (RUN) dv = q8_dot_run(wx[r], L, P[t][r], V[t][r]);
                else dv = q8_dot(wx[r], L);
                const float off = __builtin_fmaf(8.0f, scl[r], zro[r]) * xsum;
                acc[t][r] = __builtin_fmaf(scl[r] * cs, (float)dv, acc[t][r] + off);
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
            fetch(min((c + PF) * LPR + sl, NU - 1), wb[j], hb[j]);
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

// General kernel: any alignment of w, S <= QGEMV_MAX_S.  One wave per row;
// lane takes payload bytes; each weight decoded to f32 as fma(q, scale, zero).
template <int HF>
__global__ __launch_bounds__(256) void mq4v2_gemv_general(const uint8_t *__restrict__ w,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y, int S, int I,
                                                          int O)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= O) return;
    const int G = I / 256;
    const uint8_t *wr = w + (size_t)row * G * MQ4_GROUP_BYTES;
    float acc[QGEMV_MAX_S];
#pragma unroll
    for (int t = 0; t < QGEMV_MAX_S; t++) acc[t] = 0.0f;
    for (int k = lane; k < G * 128; k += WAVE) {     // payload byte k of the row
        const int g = k >> 7, b = k & 127;
        const uint8_t *gp = wr + (size_t)g * MQ4_GROUP_BYTES;
        float scl, zro;
        mq4_hdr_bytes<HF>(gp, 2 * b, scl, zro);
        float e[4], o[4];
        nib8((uint32_t)gp[8 + b], e, o);
        const float w0 = __builtin_fmaf(e[0] * NIB_XSCALE, scl, zro);
        const float w1 = __builtin_fmaf(o[0] * NIB_XSCALE, scl, zro);
        const int c0 = g * 256 + 2 * b;
#pragma unroll
        for (int t = 0; t < QGEMV_MAX_S; t++) {
            if (t < S) {
                const float *xt = x + (size_t)t * I;
                acc[t] = __builtin_fmaf(w1, xt[c0 + 1], __builtin_fmaf(w0, xt[c0], acc[t]));
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

// Decode-only: W[o][i] = fma(q, scale, zero) (one rounding), header format HF.
template <int HF>
__global__ __launch_bounds__(256) void mq4v2_dequant(const uint8_t *__restrict__ w,
                                                     float *__restrict__ W, int I, int O)
{
    const int G = I / 256;
    const size_t n = (size_t)O * G * 128;     // payload bytes
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t og = idx >> 7;             // row * G + g
        const int b = (int)(idx & 127);
        const uint8_t *gp = w + og * MQ4_GROUP_BYTES;
        float scl, zro;
        mq4_hdr_bytes<HF>(gp, 2 * b, scl, zro);
        float e[4], o[4];
        nib8((uint32_t)gp[8 + b], e, o);
        const size_t o_row = og / G;
        const int g = (int)(og - o_row * G);
        float *dst = W + o_row * I + (size_t)g * 256 + 2 * b;
        dst[0] = __builtin_fmaf(e[0] * NIB_XSCALE, scl, zro);
        dst[1] = __builtin_fmaf(o[0] * NIB_XSCALE, scl, zro);
    }
}

// ---------------------------------------------------------------------------
// MQ4-v2 encoder (hipfire "MQ4 V2", section 3) for weights already in the
// rotated space.  One wave per 256-weight group; lane l holds weights
// 4l .. 4l+3, so lanes 0..31 hold half 0 and lanes 32..63 half 1.  Per half:
// lo and hi are the min and max over its 32 lanes; step = (hi - lo) / 15 in
// f32 (correctly rounded); the stored scale and zero are the fp16 (nearest
// even) values of step and lo; every code is chosen against the stored
// values, q = clamp(rint((w - z) / s), 0, 15), so the decoder reproduces the
// encoder's reconstruction.  A stored scale of 0 (a constant half, or a step
// too small for fp16) gives q = 0.  An extreme of -0 counts as +0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mq4v2_encode_kernel(const float *__restrict__ W,
                                                           uint8_t *__restrict__ out, int I,
                                                           int O)
{
    const int lane = threadIdx.x & 63;
    const int G = I / 256;
    const int grp = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (grp >= O * G) return;                    // whole waves
    const int row = grp / G, g = grp - row * G;
    const f32x4 v = *reinterpret_cast<const f32x4 *>(W + (size_t)row * I + (size_t)g * 256 +
                                                      4 * lane);
    float lo = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
    float hi = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {           // within each 32-lane half
        lo = fminf(lo, __shfl_xor(lo, m, WAVE));
        hi = fmaxf(hi, __shfl_xor(hi, m, WAVE));
    }
    lo = lo + 0.0f;                              // a -0 extreme counts as +0
    hi = hi + 0.0f;
    const float step = __fdiv_rn(hi - lo, 15.0f);
    const _Float16 s16 = (_Float16)step, z16 = (_Float16)lo;
    const float st = (float)s16, z = (float)z16;
    const float wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t q = 0;
        if (st != 0.0f) {
            const float qf = __builtin_rintf(__fdiv_rn(wv[k] - z, st));
            q = qf < 0.0f ? 0u : (qf > 15.0f ? 15u : (uint32_t)qf);
        }
        packed |= q << (4 * k);
    }
    uint8_t *gp = out + (size_t)grp * MQ4_GROUP_BYTES;
    *reinterpret_cast<uint16_t *>(gp + 8 + 2 * lane) = (uint16_t)packed;
    if ((lane & 31) == 0) {
        const uint32_t hd = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
        *reinterpret_cast<uint32_t *>(gp + (lane >> 3)) = hd;   // +0 / +4
    }
}

// ---------------------------------------------------------------------------
// FWHT-256 pre-rotation: x_rot = (1/16) H256 (signs . x) per 256-element block,
// H256 the Sylvester Hadamard matrix.  One wave per block; lane l holds
// elements 4l..4l+3.  Radix-2 butterflies (a, b) -> (a + b, a - b) for
// strides 1, 2, 4, ..., 128 in f32: strides 1 and 2 inside a lane, strides
// 4..128 between lanes l and l ^ (stride/4).  The 1/16 is exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_lane(float v, int m)
{
    return __shfl_xor(v, m, WAVE);
}

__global__ __launch_bounds__(256) void fwht256_kernel(const float *__restrict__ x,
                                                      const int8_t *__restrict__ signs,
                                                      float *__restrict__ xr, int I, int nblk)
{
    const int lane = threadIdx.x & 63;
    const int blk = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (blk >= nblk) return;
    const int nb = I / 256;
    const int t = blk / nb, b = blk - t * nb;
    const size_t off = (size_t)t * I + (size_t)b * 256 + 4 * lane;
    const f32x4 xv = *reinterpret_cast<const f32x4 *>(x + off);
    const int8_t *sg = signs + (size_t)b * 256 + 4 * lane;
    float v[4] = {xv.x * (float)sg[0], xv.y * (float)sg[1], xv.z * (float)sg[2],
                  xv.w * (float)sg[3]};
    // stride 1
    float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    // stride 2
    v[0] = a0 + a2; v[2] = a0 - a2; v[1] = a1 + a3; v[3] = a1 - a3;
    // strides 4..128: partner lane l ^ m; the lane whose bit m is clear holds a
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float o = xor_lane(v[k], m);
            v[k] = upper ? o - v[k] : v[k] + o;
        }
    }
    f32x4 out = {v[0] * 0.0625f, v[1] * 0.0625f, v[2] * 0.0625f, v[3] * 0.0625f};
    *reinterpret_cast<f32x4 *>(xr + off) = out;
}

namespace {

// Lanes per row for one vector: pick_lpr_wide (at most QG_MQ4_LPR), narrowed
// (not below 8) until a row takes at least two sweeps.  pick_lpr_wide against
// the fewest idle lanes: 4096 x 11008 8.7 against 19.3 us (fused 10.2 against
// 20.7), 3584 x 18944 13.1 against 18.8, 2048 x 2560 4.1 against 4.6; 18944 x
// 3584 4 % slower (fused 18-21 %).  The narrowing: 28672 x 1024 8.3 -> 5.8
// us, 14336 x 2048 8.4 -> 5.4 us, 7168 x 2048 5.2 -> 4.3 us; four sweeps
// instead of two measured 3-10 % slower.
int mq4_lpr1(int I)
{
    int lpr = pick_lpr_wide(I / 32);
    if (lpr > QG_MQ4_LPR) lpr = QG_MQ4_LPR;
    while (lpr > 8 && (I / 32) / lpr < 2) lpr /= 2;
    return lpr;
}

size_t mq4_lds_bytes(int S, int I, bool rot)
{
    const size_t stage = q8_verdict_offset(S, I / 32, true) + verdict_bytes(16, S);
    const size_t fallback = rot ? (size_t)S * I * sizeof(float) : 0;
    return stage > fallback ? stage : fallback;
}

template <int HF, int S, int LPR, int R, int PF, int WPB, bool ROT>
hipError_t launch_t(const uint8_t *w, const float *x, const int8_t *sg, float *y, int I, int O,
                    hipStream_t st)
{
    constexpr int ROWS_PER_WAVE = (WAVE / LPR) * R;
    const int ntiles = (O + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    const int blocks = (ntiles + WPB - 1) / WPB;
    const size_t lds = mq4_lds_bytes(S, I, ROT);
    constexpr int EARLY = QG_MQ4_EARLY < PF ? QG_MQ4_EARLY : PF;
    auto kern = mq4v2_gemv_stream<HF, S, LPR, R, PF, WPB, ROT, EARLY>;
    hipError_t e = set_max_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WPB), lds, st, w, x, sg, y, I, O, ntiles);
    return hipGetLastError();
}

template <int HF, int S, int R, bool ROT, int WPB = QG_MQ4_WPB_MULTI>
hipError_t launch_r(const uint8_t *w, const float *x, const int8_t *sg, float *y, int I, int O,
                    hipStream_t st)
{
    // several vectors: 16-wave workgroups leave 128 registers per lane, so
    // two sweeps in flight
    constexpr int PF = S == 1 ? QG_MQ4_PF : 2;
    const int lpr = S == 1 ? mq4_lpr1(I) : pick_lpr_wide(I / 32);
    switch (lpr) {
    case 64: return launch_t<HF, S, 64, R, PF, WPB, ROT>(w, x, sg, y, I, O, st);
    case 32: return launch_t<HF, S, 32, R, PF, WPB, ROT>(w, x, sg, y, I, O, st);
    case 16: return launch_t<HF, S, 16, R, PF, WPB, ROT>(w, x, sg, y, I, O, st);
    default: return launch_t<HF, S, 8, R, PF, WPB, ROT>(w, x, sg, y, I, O, st);
    }
}

template <int HF, int S, bool ROT>
hipError_t launch_s(const uint8_t *w, const float *x, const int8_t *sg, float *y, int I, int O,
                    hipStream_t st)
{
    if constexpr (S == 1) {
        // Tile: 16, 14, 12 or 8 waves of two or one rows per lane group,
        // whichever fills whole rounds of the CUs best (pick_fill_tile).  At
        // 8192 x 8192 the 16-wave two-row tile fills one round exactly.
        // Against 16 waves with R by the busiest CU, in us: 2048 x 7168 8.2
        // -> 5.9 (8 waves), 5120 x 5120 7.1 -> 6.2 and 17408 x 5120 17.4 ->
        // 13.8 (12), 7168 x 8192 8.8 -> 8.6 and 14336 x 4096 9.2 -> 8.9 (14).
        // With the fused rotation every workgroup rotates x, so one-row tiles
        // count only where they leave at most one workgroup per CU (18944 x
        // 3584: 12.3 -> 10.9 us; eleven other shapes within 1 %).
        static const WaveTile cand[] = {{16, 2}, {16, 1}, {14, 2}, {14, 1},
                                        {12, 2}, {12, 1}, {8, 2},  {8, 1}};
        switch (pick_fill_tile(O, 64 / mq4_lpr1(I), cand, 8, cu_count(), ROT)) {
        case 0: return launch_r<HF, S, 2, ROT, 16>(w, x, sg, y, I, O, st);
        case 1: return launch_r<HF, S, 1, ROT, 16>(w, x, sg, y, I, O, st);
        case 2: return launch_r<HF, S, 2, ROT, 14>(w, x, sg, y, I, O, st);
        case 3: return launch_r<HF, S, 1, ROT, 14>(w, x, sg, y, I, O, st);
        case 4: return launch_r<HF, S, 2, ROT, 12>(w, x, sg, y, I, O, st);
        case 5: return launch_r<HF, S, 1, ROT, 12>(w, x, sg, y, I, O, st);
        case 6: return launch_r<HF, S, 2, ROT, 8>(w, x, sg, y, I, O, st);
        default: return launch_r<HF, S, 1, ROT, 8>(w, x, sg, y, I, O, st);
        }
    } else {
        // several vectors: R keeps every workgroup resident at once.  Every
        // workgroup converts all S vectors, so ties go to the larger R (fewer
        // workgroups).  Pre-rotated 8192 x 8192, two vectors: 15.0 -> 11.1-11.2
        // us against ties to the smaller R (two workgroups per CU, each
        // converting the vectors); eleven other shapes and counts within 1 %
        static const int cand[] = {3, 2, 1};
        switch (pick_rows_per_group(O, pick_lpr_wide(I / 32), QG_MQ4_WPB_MULTI,
                                    mq4_lds_bytes(S, I, ROT), cand, 3)) {
        case 1: return launch_r<HF, S, 1, ROT>(w, x, sg, y, I, O, st);
        case 2: return launch_r<HF, S, 2, ROT>(w, x, sg, y, I, O, st);
        default: return launch_r<HF, S, 3, ROT>(w, x, sg, y, I, O, st);
        }
    }
}

// Vectors one streaming launch takes for this shape (0: not applicable).
int mq4_stream_vectors(const void *w, const float *x, const int8_t *sg, int S, int I, bool rot)
{
    if (((uintptr_t)w & 7) != 0 || ((uintptr_t)x & 15) != 0) return 0;
    if (rot && ((uintptr_t)sg & 7) != 0) return 0;
    int n = S < MQ4_FAST_MAX_S ? S : MQ4_FAST_MAX_S;
    while (n > 0 && mq4_lds_bytes(n, I, rot) > LDS_BUDGET) --n;
    return n;
}

// Streaming launches in groups of at most nmax vectors.
template <int HF, bool ROT>
hipError_t launch_groups(const uint8_t *w, const float *x, const int8_t *sg, float *y, int S,
                         int I, int O, int nmax, hipStream_t st)
{
    for (int s0 = 0; s0 < S; s0 += nmax) {
        const int n = S - s0 < nmax ? S - s0 : nmax;
        const float *xs = x + (size_t)s0 * I;
        float *ys = y + (size_t)s0 * O;
        hipError_t e;
        switch (n) {
        case 1: e = launch_s<HF, 1, ROT>(w, xs, sg, ys, I, O, st); break;
        case 2: e = launch_s<HF, 2, ROT>(w, xs, sg, ys, I, O, st); break;
        case 3: e = launch_s<HF, 3, ROT>(w, xs, sg, ys, I, O, st); break;
        default: e = launch_s<HF, 4, ROT>(w, xs, sg, ys, I, O, st); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int HF>
hipError_t launch_gemv_hf(const void *w, const float *x, float *y, int S, int I, int O,
                          hipStream_t st)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    // more vectors than one launch takes run in groups, each streaming the
    // weights once
    const int nmax = mq4_stream_vectors(w, x, nullptr, S, I, false);
    if (nmax > 0) return launch_groups<HF, false>(wb, x, nullptr, y, S, I, O, nmax, st);
    const int wpb = 4;
    hipLaunchKernelGGL(mq4v2_gemv_general<HF>, dim3((O + wpb - 1) / wpb), dim3(64 * wpb), 0, st,
                       wb, x, y, S, I, O);
    return hipGetLastError();
}

template <int HF>
hipError_t launch_dequant_hf(const void *w, float *W, int I, int O, hipStream_t st)
{
    const size_t n = (size_t)O * (I / 256) * 128;
    const size_t want = (n + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(mq4v2_dequant<HF>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint8_t *>(w), W, I, O);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mq4v2_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                             hipStream_t st)
{
    return launch_gemv_hf<MQ4_V2>(w, x, y, S, I, O, st);
}

hipError_t launch_mq4v1_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                             hipStream_t st)
{
    return launch_gemv_hf<MQ4_V1>(w, x, y, S, I, O, st);
}

hipError_t launch_mq4c_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                            hipStream_t st)
{
    return launch_gemv_hf<MQ4_C>(w, x, y, S, I, O, st);
}

int mq4v2_rot_check(const void *w, const float *x, const int8_t *signs, int I)
{
    if (((uintptr_t)w & 7) != 0 || ((uintptr_t)x & 15) != 0 || ((uintptr_t)signs & 7) != 0)
        return QGEMV_E_ALIGN;
    if (mq4_lds_bytes(1, I, true) > LDS_BUDGET) return QGEMV_E_DIMS;
    return QGEMV_OK;
}

hipError_t launch_mq4v2_rot_gemv(const void *w, const float *x, const int8_t *signs, float *y,
                                 int S, int I, int O, hipStream_t st)
{
    const int nmax = mq4_stream_vectors(w, x, signs, S, I, true);
    if (nmax <= 0) return hipErrorInvalidValue;   // callers check mq4v2_rot_check first
    return launch_groups<MQ4_V2, true>(static_cast<const uint8_t *>(w), x, signs, y, S, I, O,
                                       nmax, st);
}

hipError_t launch_mq4v2_dequant(const void *w, float *W, int I, int O, hipStream_t st)
{
    return launch_dequant_hf<MQ4_V2>(w, W, I, O, st);
}

hipError_t launch_mq4v1_dequant(const void *w, float *W, int I, int O, hipStream_t st)
{
    return launch_dequant_hf<MQ4_V1>(w, W, I, O, st);
}

hipError_t launch_mq4c_dequant(const void *w, float *W, int I, int O, hipStream_t st)
{
    return launch_dequant_hf<MQ4_C>(w, W, I, O, st);
}

hipError_t launch_mq4v2_encode(const float *W, void *out, int I, int O, hipStream_t st)
{
    const long groups = (long)O * (I / 256);
    hipLaunchKernelGGL(mq4v2_encode_kernel, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, st,
                       W, static_cast<uint8_t *>(out), I, O);
    return hipGetLastError();
}

hipError_t launch_fwht256(const float *x, const int8_t *signs, float *xr, int S, int I,
                          hipStream_t st)
{
    const int nblk = S * (I / 256);
    const int wpb = 4;
    hipLaunchKernelGGL(fwht256_kernel, dim3((nblk + wpb - 1) / wpb), dim3(64 * wpb), 0, st, x,
                       signs, xr, I, nblk);
    return hipGetLastError();
}

}  // namespace qg
