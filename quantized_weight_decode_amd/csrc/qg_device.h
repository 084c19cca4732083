// qg_device.h -- device helpers shared by the gfx950 GEMV kernels.
//
// Wave64 only.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// s_waitcnt operands (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait)
#define QG_WAIT_VM0 0x0F70      /* all vector memory loads returned */
#define QG_WAIT_LGKM0 0xC07F    /* all LDS / scalar memory operations done */

// Weight streams are read with the non-temporal hint: each byte is used once
// per call, and keeping it out of the caches leaves the activations (read by
// every workgroup) resident in L2 across calls.
#ifndef QG_NT
#define QG_NT 1
#endif
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p)
{
#if QG_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

// ---------------------------------------------------------------------------
// Nibble decode.
//
// A byte whose top four bits are clear, read as an OCP E4M3 code, has value
// q * 2^-9 for q = 0..15: q < 8 is the subnormal q * 2^-9, q >= 8 is exponent
// 1 with mantissa q - 8, i.e. (8 + (q-8)) * 2^-9.  So masking the nibbles of a
// packed dword into separate bytes and feeding them to the hardware
// fp8->f32 pair converter decodes two nibbles per instruction, exactly.
// Activations are staged pre-multiplied by 2^9 so products come out as q*x.
// ---------------------------------------------------------------------------
constexpr float NIB_XSCALE = 512.0f;  // 2^9

// fp8 (OCP E4M3) pair conversion of bytes 0-1 / bytes 2-3 of a dword.
__device__ __forceinline__ f32x2 fp8pair_lo(uint32_t w)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
__device__ __forceinline__ f32x2 fp8pair_hi(uint32_t w)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
}

// Decodes the 8 nibbles of one little-endian packed dword.
//   e[0..3] = nibbles of bytes 0..3 low halves  (columns 0, 2, 4, 6)
//   o[0..3] = nibbles of bytes 0..3 high halves (columns 1, 3, 5, 7)
// each as q * 2^-9.
__device__ __forceinline__ void nib8(uint32_t w, float e[4], float o[4])
{
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    const f32x2 a = fp8pair_lo(lo);
    const f32x2 b = fp8pair_hi(lo);
    const f32x2 c = fp8pair_lo(hi);
    const f32x2 d = fp8pair_hi(hi);
    e[0] = a.x; e[1] = a.y; e[2] = b.x; e[3] = b.y;
    o[0] = c.x; o[1] = c.y; o[2] = d.x; o[3] = d.y;
}

// Four E4M3 codes of a dword (byte k = column k) as floats, exactly.
__device__ __forceinline__ void e4m3x4(uint32_t w, float v[4])
{
    const f32x2 a = fp8pair_lo(w);
    const f32x2 b = fp8pair_hi(w);
    v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
}

// IEEE binary16 bits -> f32 (exact).
__device__ __forceinline__ float f16_to_f32(uint32_t h16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// ---------------------------------------------------------------------------
// Activation staging helpers.
// ---------------------------------------------------------------------------
// Segment stride (in float4s) of the fp8 kernel's staged activations: one
// float4 of padding keeps the staging writes of one chunk out of one bank.
__host__ __device__ constexpr int seg_stride(int NU) { return NU + 1; }

// float4 number i of an array (32-bit offset from a wave-uniform base)
__device__ __forceinline__ f32x4 ldx4(const float *__restrict__ base, uint32_t i)
{
    return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const char *>(base) + i * 16u);
}

// vector index t (< TMAX) and in-vector index of float4 number f; cpv = 8 NU
template <int TMAX>
__device__ __forceinline__ void split_f(int f, int cpv, int &t, int &rem)
{
    t = 0;
#pragma unroll
    for (int k = 1; k < TMAX; k++) t += f >= k * cpv;
    rem = f - t * cpv;
}

// Every workgroup reads the same activation vectors.  If all of them walked
// x in the same order, the workgroups sharing an L2 would request the same
// few lines at the same moment and queue on one L2 channel; each workgroup
// therefore starts at its own line-aligned offset (a multiple of 8 float4s,
// so lane chunks stay aligned) and wraps around.  stage_rot() picks the
// offset; stage_index() maps the f-th read of the workgroup to a float4
// index (reads past the end are clamped onto a valid index).
__device__ __forceinline__ int stage_rot(int total)
{
    const unsigned lines = (unsigned)total / 8u;
    return lines ? (int)(((blockIdx.x * 2654435761u) >> 7) % lines) * 8 : 0;
}
__device__ __forceinline__ int stage_index(int f, int total, int rot)
{
    const int g = min(f, total - 1) + rot;
    return g >= total ? g - total : g;
}

// ---------------------------------------------------------------------------
// Integer-dot form of the 4-bit chunk product.
//
// The activations of each 32-column lane chunk are staged in a shared-exponent
// fixed point.  With E the smallest integer such that max|x| < 2^E over the
// chunk (E clamped to at least -100), v = RNE(x * 2^(21 - E)), so |v| <= 2^21
// and x~ = v * 2^(E - 21) is within 2^-21 max|x| of x.  v is written in six
// balanced base-16 digits, v = sum_j d_j 16^j with d_j in [-8, 7], and digit j
// of the eight columns under packed weight dword d forms one dword (column
// 8d + k in nibble k): the operand layout of the 8-way signed 4-bit dot
// product (v_dot8_i32_i4).  A packed weight dword XOR 0x88888888, read as eight
// signed nibbles, is exactly q - 8 per column, so
//     sum over the chunk of (q - 8) v = sum_j 16^j dot8(w ^ 0x88888888, D_j),
// exact in 32-bit integers (|sum| <= 32 * 8 * 2^21 = 2^29).  The fixed-point
// values come from one FMA: x * 2^(21-E) + 1.5 * 2^23 lies in [2^23, 2^24),
// where the float spacing is 1, so the FMA's single rounding is the RNE of
// x * 2^(21-E) and the low bits of the result are 0x400000 + v.
//
// LDS layout of one vector (NU chunks): u32x4 xq[6][NU], component d of
// xq[j][u] = digit j of columns 32u + 8d + 0..7 (biased to the two's-complement
// nibble pattern); float xc[NU] = 2^(E_u - 21); optionally float xsum[NU] =
// 2^(E_u - 21) * sum v over the chunk (for offsets such as MQ4's zero).
// ---------------------------------------------------------------------------
// Orders code: every value in v is computed before this point, and no memory
// operation moves across it.  Used between the consume and refill of a ring
// slot so that the refill can reuse the slot's registers (otherwise the
// compiler may sink a slot's arithmetic below the following loads and keep
// every slot's data live at once).
template <int N>
__device__ __forceinline__ void pin_values(const float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("" ::"v"(v[i]) : "memory");
}

constexpr float Q8_MAGIC = 12582912.0f;        // 1.5 * 2^23
// Precision test of the staged fixed point (see q8_put): the squared bound
// on its estimated relative error on y, (3e-6)^2.
constexpr float Q8_TAU2 = 9.0e-12f;
constexpr uint32_t Q8_UNBIAS = 0x4AB77778u;    // 0x4B400000 - 0x888888
constexpr uint32_t Q8_DIGIT_BIAS = 0x888888u;  // 8 * (16^0 + ... + 16^5)
constexpr uint32_t Q8_NIB_FLIP = 0x88888888u;

// max over the four lanes 4c..4c+3
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t m)
{
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    return m;
}
__device__ __forceinline__ int quad_sum_i32(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    return v;
}

// Converts the eight activations of one weight dword (columns 32u + 8d + 0..7)
// and stores their digit dwords; the stored chunk scale (and sum) is
// multiplied by post, a power of two.  The four lanes 4c..4c+3 hold the
// four dwords d = 0..3 of one chunk and must all call this together (the
// chunk exponent is a max over them).  Lanes with ok == false store nothing.
// Returns nonzero if the chunk holds an infinity or NaN (its staged values
// are then meaningless).
//
// Precision test.  The fixed point represents every element of a chunk to
// within half its quantum 2^(E-21), whatever the element's own size, so
// elements much smaller than the chunk's largest lose relative precision.
// With weights of no particular sign or size, the relative L2 error this
// puts on y is about sqrt(A / B), A the sum of the squared representation
// errors and B the sum of the squared values.  An outlier of the chunk may
// meet a zero weight, so both sums leave out each lane's largest element
// (whose own relative error is at most 2^-21).  dl returns this lane's
// A - TAU^2 B (exact power-of-two rescaling into f64); a vector is staged
// precisely enough when its sum over all lanes is not positive.
template <bool SUM>
__device__ __forceinline__ uint32_t q8_put(const float xv[8], bool ok, uint32_t t, uint32_t u,
                                           uint32_t d, uint32_t NU, uint32_t *__restrict__ xq,
                                           float *__restrict__ xc, float *__restrict__ xsum,
                                           double &dl, float post = 1.0f)
{
    // |x| as ordered integers: every NaN sorts above infinity, above every finite
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) m = max(m, __builtin_bit_cast(uint32_t, xv[k]) & 0x7FFFFFFFu);
    const uint32_t ml = m;                       // this lane's largest |x|
    m = quad_max_u32(m);
    const uint32_t eb = m >> 23;                 // biased exponent of max|x|: E = eb - 126
    const uint32_t e = max(eb, 26u);             // E >= -100
    const float sin = __builtin_bit_cast(float, (274u - e) << 23);   // 2^(21 - E)
    uint32_t n[8];                                // v + 0x888888, in [0x688888, 0xA88888]
    float pa = 0.0f, pb = 0.0f;                   // A and B of the lane, in units of 2^(2E-42)
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const float r = __builtin_fmaf(xv[k], sin, Q8_MAGIC);
        n[k] = __builtin_bit_cast(uint32_t, r) - Q8_UNBIAS;
        const float vf = r - Q8_MAGIC;                            // v, exactly
        const float dv = __builtin_fmaf(xv[k], sin, -vf);         // x 2^(21-E) - v, exactly
        pa = __builtin_fmaf(dv, dv, pa);
        pb = __builtin_fmaf(vf, vf, pb);
    }
    {   // leave out the lane's largest element
        const float xm = __builtin_bit_cast(float, ml);
        const float vm = __builtin_fmaf(xm, sin, Q8_MAGIC) - Q8_MAGIC;
        const float dm = __builtin_fmaf(xm, sin, -vm);
        pa = __builtin_fmaf(-dm, dm, pa);
        pb = __builtin_fmaf(-vm, vm, pb);
    }
    dl = ok ? __builtin_ldexp((double)__builtin_fmaf(-Q8_TAU2, pb, pa), 2 * (int)e - 294) : 0.0;
    // byte b of the even columns (0, 2, 4, 6) and of the odd columns (1, 3, 5, 7)
    const uint32_t te = __builtin_amdgcn_perm(n[2], n[0], 0x05010400u);
    const uint32_t ue = __builtin_amdgcn_perm(n[6], n[4], 0x05010400u);
    const uint32_t te2 = __builtin_amdgcn_perm(n[2], n[0], 0x06020602u);
    const uint32_t ue2 = __builtin_amdgcn_perm(n[6], n[4], 0x06020602u);
    const uint32_t to = __builtin_amdgcn_perm(n[3], n[1], 0x05010400u);
    const uint32_t uo = __builtin_amdgcn_perm(n[7], n[5], 0x05010400u);
    const uint32_t to2 = __builtin_amdgcn_perm(n[3], n[1], 0x06020602u);
    const uint32_t uo2 = __builtin_amdgcn_perm(n[7], n[5], 0x06020602u);
    const uint32_t be[3] = {__builtin_amdgcn_perm(ue, te, 0x05040100u),
                            __builtin_amdgcn_perm(ue, te, 0x07060302u),
                            __builtin_amdgcn_perm(ue2, te2, 0x05040100u)};
    const uint32_t bo[3] = {__builtin_amdgcn_perm(uo, to, 0x05040100u),
                            __builtin_amdgcn_perm(uo, to, 0x07060302u),
                            __builtin_amdgcn_perm(uo2, to2, 0x05040100u)};
    // digit 2b is the low nibble of byte b, digit 2b+1 the high nibble; the
    // even column goes to the low nibble of each output byte
    uint32_t L[6];
#pragma unroll
    for (int b = 0; b < 3; b++) {
        L[2 * b] = ((bo[b] << 4) & 0xF0F0F0F0u) | (be[b] & 0x0F0F0F0Fu);
        L[2 * b + 1] = (bo[b] & 0xF0F0F0F0u) | ((be[b] >> 4) & 0x0F0F0F0Fu);
    }
    int vs = 0;
    if constexpr (SUM) {
#pragma unroll
        for (int k = 0; k < 8; k++) vs += (int)(n[k] - Q8_DIGIT_BIAS);
        vs = quad_sum_i32(vs);
    }
    const float cs = __builtin_bit_cast(float, (e - 20u) << 23) * post;   // 2^(E - 21)
    if (ok) {
        uint32_t *q = xq + (t * 6u * NU + u) * 4u + d;
#pragma unroll
        for (int j = 0; j < 6; j++) q[j * NU * 4u] = L[j] ^ Q8_NIB_FLIP;
        if (d == 0) {
            xc[t * NU + u] = cs;
            if constexpr (SUM) xsum[t * NU + u] = cs * (float)vs;
        }
    }
    return eb == 255u;
}

// Radix-2 Walsh-Hadamard butterflies, (a, b) -> (a + b, a - b), for the
// strides 8, 16, ..., 128 of a 256-element block held as eight consecutive
// values per lane by 32 consecutive lanes (lane bit m <-> stride 8 * 2^m).
// The lane whose stride bit is set holds b and keeps a - b.
template <int M>
__device__ __forceinline__ float lane_xor(float v)
{
    const int iv = __builtin_bit_cast(int, v);
    int r;
    // every source lane of these patterns exists, so bound_ctrl changes no
    // value; it lets the move go without first clearing its destination
    if constexpr (M == 1) r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);
    else if constexpr (M == 2) r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);
    // M == 8: row_ror:8
    else if constexpr (M == 8) r = __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);
    else r = __builtin_amdgcn_ds_swizzle(iv, 0x1F | (M << 10));   // xor M within 32 lanes
    return __builtin_bit_cast(float, r);
}
template <int M>
__device__ __forceinline__ void fwht_lane_stage(float v[8], int lane)
{
    const float sg = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = __builtin_fmaf(sg, v[k], lane_xor<M>(v[k]));
}
// Unnormalised H256 of the block: strides 1, 2, 4 inside the lane, then
// 8 .. 128 across lanes, ascending (the order of the stand-alone kernel).
__device__ __forceinline__ void fwht256_item(float v[8], int lane)
{
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int k = 0; k < 8; k++)
            if (!(k & h)) {
                const float a = v[k], b = v[k + h];
                v[k] = a + b;
                v[k + h] = a - b;
            }
    fwht_lane_stage<1>(v, lane);
    fwht_lane_stage<2>(v, lane);
    fwht_lane_stage<4>(v, lane);
    fwht_lane_stage<8>(v, lane);
    fwht_lane_stage<16>(v, lane);
}

// Stages S activation vectors of I columns (I % 32 == 0) in the fixed-point
// layout above.  Thread f of the workgroup takes item f: the eight columns
// 8f .. 8f + 7 (two float4 loads), so a chunk is four consecutive lanes.
// Each workgroup starts at its own aligned offset and wraps around, as
// stage_rot describes.  load() issues the thread's first NPRE items (those that exist)
// and store() converts them, then any further items one at a time
// (load_all() issues all NPRE, past the end at clamped indices, so that the
// count of loads in flight is the same in every thread and a wait for a load
// issued before them is exact).  Items
// past the end belong to whole lane groups (items is a multiple of 32 with
// ROT, of 4 otherwise; NT a multiple of 64), which skip both.  NT is the
// workgroup size; items may cover fewer than S vectors.  store() returns the
// mask of vectors (bit t) in which this thread met an infinity or NaN.
//
// With ROT the vectors are first rotated as the FWHT-256 pre-rotation
// defines it: x_rot = H256 (signs . x) / 16 per 256-column block (I % 256 ==
// 0; a block is 32 items in 32 consecutive lanes, the rotation offset a
// multiple of a block).  The butterflies run in the stand-alone kernel's
// order, so x_rot is the same to the bit; the 1/16 goes into the chunk
// scales.  store_rotated_f32() writes x_rot itself as f32 (the fallback for
// activations holding an infinity or NaN).
template <int S, int NPRE, int NT, bool SUM = false, bool ROT = false>
struct XStageQ {
    f32x4 a[NPRE], b[NPRE];
    u32x2 sg[ROT ? NPRE : 1];
    int rot;
    double dsum[S];   // per vector: this thread's share of A - TAU^2 B (q8_put)

    __device__ __forceinline__ void load(const float *__restrict__ x, int items,
                                         const int8_t *__restrict__ signs = nullptr, int ipv = 0)
    {
        constexpr unsigned G = ROT ? 32u : 4u;   // rotation granule in items
        const unsigned groups = (unsigned)items / G;
        rot = groups ? (int)(((blockIdx.x * 2654435761u) >> 7) % groups * G) : 0;
#pragma unroll
        for (int j = 0; j < NPRE; j++) {
            const int f = (int)threadIdx.x + j * NT;
            if constexpr (ROT) {
                // unconditional (clamped past the end) and, as a relaxed atomic,
                // kept in place: a sign load behind the branch below ends in a
                // register copy that waits for it before the weight loads
                // behind it are issued
                const uint32_t g = (uint32_t)stage_index(f, items, rot);
                const uint64_t sv = __hip_atomic_load(
                    reinterpret_cast<const uint64_t *>(signs + 8u * sign_item(g, ipv)),
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                sg[j] = u32x2{(uint32_t)sv, (uint32_t)(sv >> 32)};
            }
            if (f < items) {
                const uint32_t g = (uint32_t)stage_index(f, items, rot);
                a[j] = ldx4(x, 2u * g);
                b[j] = ldx4(x, 2u * g + 1u);
            }
        }
    }

    // item g's position within its vector (one vector: g itself)
    __device__ __forceinline__ static uint32_t sign_item(uint32_t g, int ipv)
    {
        return S == 1 ? g : g % (uint32_t)ipv;
    }

    __device__ __forceinline__ void load_all(const float *__restrict__ x, int items)
    {
        static_assert(!ROT, "load_all stages unrotated vectors");
        const unsigned groups = (unsigned)items / 4u;
        rot = groups ? (int)(((blockIdx.x * 2654435761u) >> 7) % groups * 4u) : 0;
#pragma unroll
        for (int j = 0; j < NPRE; j++) {
            const uint32_t g = (uint32_t)stage_index((int)threadIdx.x + j * NT, items, rot);
            a[j] = ldx4(x, 2u * g);
            b[j] = ldx4(x, 2u * g + 1u);
        }
    }

    __device__ __forceinline__ uint32_t put(f32x4 va, f32x4 vb, u32x2 sv, int g, int NU,
                                            uint32_t *__restrict__ xq, float *__restrict__ xc,
                                            float *__restrict__ xsum)
    {
        const int ipv = NU * 4;   // items per vector
        int t, rem;
        split_f<S>(g, ipv, t, rem);
        float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
        float post = 1.0f;
        if constexpr (ROT) {
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const int8_t sk = (int8_t)((k < 4 ? sv.x : sv.y) >> (8 * (k & 3)));
                v[k] *= (float)sk;
            }
            fwht256_item(v, (int)threadIdx.x & 63);
            post = 0.0625f;
        }
        double dl;
        const uint32_t bad = q8_put<SUM>(v, true, (uint32_t)t, (uint32_t)rem >> 2,
                                         (uint32_t)rem & 3u, (uint32_t)NU, xq, xc, xsum, dl, post);
#pragma unroll
        for (int k = 0; k < S; k++) dsum[k] += t == k ? dl : 0.0;
        return bad << t;
    }

    __device__ __forceinline__ uint32_t store(const float *__restrict__ x, int items, int NU,
                                              uint32_t *__restrict__ xq, float *__restrict__ xc,
                                              float *__restrict__ xsum,
                                              const int8_t *__restrict__ signs = nullptr)
    {
        uint32_t bad = 0;
#pragma unroll
        for (int k = 0; k < S; k++) dsum[k] = 0.0;
#pragma unroll
        for (int j = 0; j < NPRE; j++) {
            const int f = (int)threadIdx.x + j * NT;
            if (f < items)
                bad |= put(a[j], b[j], ROT ? sg[j] : u32x2{0, 0}, stage_index(f, items, rot), NU,
                           xq, xc, xsum);
        }
        for (int f = (int)threadIdx.x + NPRE * NT; f < items; f += NT) {
            const int g = stage_index(f, items, rot);
            u32x2 sv = {0, 0};
            if constexpr (ROT)
                sv = *reinterpret_cast<const u32x2 *>(signs + 8u * sign_item((uint32_t)g, NU * 4));
            bad |= put(ldx4(x, 2u * (uint32_t)g), ldx4(x, 2u * (uint32_t)g + 1u), sv, g, NU, xq,
                       xc, xsum);
        }
        return bad;
    }

    // ROT only: writes the rotated vectors as f32, xf[t][I] = x_rot (the
    // stand-alone kernel's values to the bit), for the per-element fallback.
    __device__ __forceinline__ void store_rotated_f32(const float *__restrict__ x, int items,
                                                      int NU, const int8_t *__restrict__ signs,
                                                      float *__restrict__ xf)
    {
        const int ipv = NU * 4;
        for (int f = (int)threadIdx.x; f < items; f += NT) {
            int t, rem;
            split_f<S>(f, ipv, t, rem);
            const f32x4 va = ldx4(x, 2u * (uint32_t)f), vb = ldx4(x, 2u * (uint32_t)f + 1u);
            const u32x2 sv = *reinterpret_cast<const u32x2 *>(signs + 8u * (uint32_t)rem);
            float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int k = 0; k < 8; k++)
                v[k] *= (float)(int8_t)((k < 4 ? sv.x : sv.y) >> (8 * (k & 3)));
            fwht256_item(v, (int)threadIdx.x & 63);
            f32x4 *dst = reinterpret_cast<f32x4 *>(xf + ((size_t)t * ipv * 8 + (size_t)rem * 8));
            dst[0] = f32x4{v[0] * 0.0625f, v[1] * 0.0625f, v[2] * 0.0625f, v[3] * 0.0625f};
            dst[1] = f32x4{v[4] * 0.0625f, v[5] * 0.0625f, v[6] * 0.0625f, v[7] * 0.0625f};
        }
    }
};

// f32 sum over one lane chunk (columns 32u .. 32u + 31, x32 = x + 32u) of
// ((q - 8) * s) * x with each weight decoded as the plain definition does it
// (one rounding) and multiplied by the f32 activation: the fallback for
// activations holding an infinity or NaN, which then propagate as in the
// plain definition.
__device__ __forceinline__ float nib_chunk_plain(const u32x4 wv, float s,
                                                 const float *__restrict__ x32)
{
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        float e[4], o[4];
        nib8(wv[d], e, o);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            acc = __builtin_fmaf((e[k] * NIB_XSCALE - 8.0f) * s, x32[8 * d + 2 * k], acc);
            acc = __builtin_fmaf((o[k] * NIB_XSCALE - 8.0f) * s, x32[8 * d + 2 * k + 1], acc);
        }
    }
    return acc;
}

// LDS bytes of the fixed-point staging of S vectors of NU chunks
__host__ __device__ constexpr size_t q8_stage_bytes(int S, int NU, bool sum)
{
    return (size_t)S * NU * (6 * 16 + 4 + (sum ? 4 : 0));
}
// 8-byte aligned offset just past the fixed-point staging (the verdict area)
__host__ __device__ constexpr size_t q8_verdict_offset(int S, int NU, bool sum)
{
    return (q8_stage_bytes(S, NU, sum) + 7) / 8 * 8;
}

// sum (q - 8) v over one lane chunk of packed weights wx (already XOR-ed with
// 0x88888888) against the chunk's digit dwords L.  P and V carry running
// per-digit sums across calls for the same row (the dot8 accumulates into
// them, so no accumulator is cleared); the chunk's value is the change of
// the combined sum, exact modulo 2^32.
__device__ __forceinline__ int q8_dot_run(const uint32_t wx[4], const u32x4 L[6], uint32_t P[6],
                                          uint32_t &V)
{
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
        for (int j = 0; j < 6; j++)
            P[j] = (uint32_t)__builtin_amdgcn_sdot8((int)wx[d], (int)L[j][d], (int)P[j], false);
    uint32_t v = P[5];
#pragma unroll
    for (int j = 4; j >= 0; j--) v = (v << 4) + P[j];
    const int dv = (int)(v - V);
    V = v;
    return dv;
}

// Same product with fresh accumulators (no carried state).
__device__ __forceinline__ int q8_dot(const uint32_t wx[4], const u32x4 L[6])
{
    int P[6];
#pragma unroll
    for (int j = 0; j < 6; j++) P[j] = __builtin_amdgcn_sdot8((int)wx[0], (int)L[j][0], 0, false);
#pragma unroll
    for (int d = 1; d < 4; d++)
#pragma unroll
        for (int j = 0; j < 6; j++)
            P[j] = __builtin_amdgcn_sdot8((int)wx[d], (int)L[j][d], P[j], false);
    uint32_t v = (uint32_t)P[5];
#pragma unroll
    for (int j = 4; j >= 0; j--) v = (v << 4) + (uint32_t)P[j];
    return (int)v;
}

// ---------------------------------------------------------------------------
// Sub-wave sum over LPR consecutive lanes (LPR in 4..64) with DPP.  The full
// sum lands in the last lane of each LPR-lane group.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

template <int LPR>
__device__ __forceinline__ float sub_reduce(float v)
{
    static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "LPR");
    v += dpp<0xB1>(v);                       // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);                       // quad_perm [2,3,0,1]: lane ^ 2
    if (LPR >= 8) v += dpp<0x141>(v);        // row_half_mirror: 8-lane sums
    if (LPR >= 16) v += dpp<0x140>(v);       // row_mirror: 16-lane sums
    if (LPR >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    if (LPR >= 64) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// Sum of a double over the 64 lanes of a wave (DPP on both halves, the
// order of sub_reduce); the full sum lands in lane 63.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK,
                                                             0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL,
                                                             ROW_MASK, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp64<0xB1>(v);
    v += dpp64<0x4E>(v);
    v += dpp64<0x141>(v);
    v += dpp64<0x140>(v);
    v += dpp64<0x142, 0xA>(v);
    v += dpp64<0x143, 0xC>(v);
    return v;
}

// LDS bytes stage_verdict needs (8-byte aligned start).
__host__ __device__ constexpr size_t verdict_bytes(int WPB, int S)
{
    return (size_t)WPB * (8 * S + 8);
}

// Workgroup verdict on the staged activations, the same in every wave: the
// mask of vectors t (bit t) that must take the per-element path, because a
// thread met an infinity or NaN in it (bit t of bad) or because its summed
// A - TAU^2 B of q8_put is positive (the fixed point is not precise enough
// for it).  The sums run in a fixed order.  Contains the workgroup barrier
// that publishes the staged activations.  lds: an 8-byte aligned area of
// verdict_bytes(WPB, S) bytes.
template <int WPB, int S>
__device__ __forceinline__ int stage_verdict(uint32_t bad, const double (&dsum)[S], void *lds)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    double *dw = reinterpret_cast<double *>(lds);            // [WPB][S]
    int *fw = reinterpret_cast<int *>(dw + WPB * S);           // [WPB]
    uint32_t wbad = 0;
#pragma unroll
    for (int t = 0; t < S; t++) wbad |= (__ballot((bad >> t) & 1u) != 0) ? 1u << t : 0u;
    double r[S];
#pragma unroll
    for (int t = 0; t < S; t++) r[t] = wave_sum_f64(dsum[t]);
    if (lane == 63) {
#pragma unroll
        for (int t = 0; t < S; t++) dw[wave * S + t] = r[t];
        fw[wave] = (int)wbad;
    }
    __syncthreads();
    int v = 0;
#pragma unroll
    for (int t = 0; t < S; t++) {
        double sum = 0.0;
#pragma unroll
        for (int k = 0; k < WPB; k++) sum += dw[k * S + t];
        v |= sum > 0.0 ? 1 << t : 0;
    }
#pragma unroll
    for (int k = 0; k < WPB; k++) v |= fw[k];
    return __builtin_amdgcn_readfirstlane(v);
}

// ---------------------------------------------------------------------------
// floor(u / d) via a 64-bit reciprocal multiply, exact whenever u * d < 2^40
// (here u < 2^20 and d < 2^20): with m = ceil(2^40 / d), u*m / 2^40 exceeds
// u/d by less than u / 2^40 < 1/d, which cannot reach the next integer.
// ---------------------------------------------------------------------------
struct Div20 {
    uint64_t m;
    __host__ __device__ static Div20 make(uint32_t d)
    {
        Div20 r;
        r.m = ((1ull << 40) + d - 1) / d;
        return r;
    }
    __device__ __forceinline__ uint32_t operator()(uint32_t u) const
    {
        return (uint32_t)(((uint64_t)u * m) >> 40);
    }
};

}  // namespace qg
