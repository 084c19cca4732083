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

// 8-lane sum (lanes 8m..8m+7); lane 8m+7 holds it.  Defined before use.
__device__ __forceinline__ float sub_reduce8(float v);

// ---------------------------------------------------------------------------
// Activation staging for the 4-bit formats.
//
// A "lane chunk" is 16 packed bytes = 32 columns.  For chunk u and segment
// k = 0..7 the LDS holds one float4:
//    k = 2d   : x[32u + 8d + {0,2,4,6}]   (matches low nibbles of dword d)
//    k = 2d+1 : x[32u + 8d + {1,3,5,7}]   (matches high nibbles)
// stored at float4 index (k * NS + u), NU = chunks per vector, so that lanes
// reading consecutive chunks touch consecutive 16-byte LDS words (no bank
// conflicts).  The segment stride NS = NU + 1 is padded by one float4: with
// NS a multiple of 16 the staging writes of the eight segments of one chunk
// (made by eight neighbouring lanes) would all land in the same banks.  xs[u] = plain f32 sum of the chunk's 32 activations, used to
// fold per-chunk affine offsets out of the inner loop.  The nibble decoder
// returns q * 2^-9, so a chunk's dot product comes out as 2^-9 sum(q x) and
// the fold multiplies it back by 2^9 (exact).
// ---------------------------------------------------------------------------
// float4 number i of an array (32-bit offset from a wave-uniform base)
__host__ __device__ constexpr int seg_stride(int NU) { return NU + 1; }

__device__ __forceinline__ f32x4 ldx4(const float *__restrict__ base, uint32_t i)
{
    return *reinterpret_cast<const f32x4 *>(reinterpret_cast<const char *>(base) + i * 16u);
}

// Places float4 number f of vector t into the LDS layout and adds its part of
// the chunk sum.  rem = f - t * 8 NU is the float4's index inside its vector.
// Every lane of the wave must call this (the chunk sum is an 8-lane DPP
// reduction over consecutive lanes); lanes with ok == false compute but store
// nothing (their 8-lane group is entirely out of range).
__device__ __forceinline__ void XStagePut(f32x4 a, bool ok, int t, int rem, int NU,
                                          f32x4 *__restrict__ xl, float *__restrict__ xs)
{
    const uint32_t u = (uint32_t)rem >> 3, k = (uint32_t)rem & 7;
    const uint32_t d = k >> 1, h = k & 1;
    const uint32_t NS = (uint32_t)seg_stride(NU);
    float *base = reinterpret_cast<float *>(xl) + (uint32_t)t * 32u * NS;
    const uint32_t oe = ((2 * d) * NS + u) * 4 + 2 * h;
    const uint32_t oo = oe + 4u * NS;
    f32x2 ev = {a.x, a.z};
    f32x2 od = {a.y, a.w};
    const float cs = sub_reduce8((a.x + a.y) + (a.z + a.w));
    if (ok) {
        *reinterpret_cast<f32x2 *>(base + oe) = ev;
        *reinterpret_cast<f32x2 *>(base + oo) = od;
        if (k == 7) xs[(uint32_t)t * (uint32_t)NU + u] = cs;
    }
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

// Stages S (<= 8) activation vectors of I columns into the LDS layout above.
// Loads are coalesced: thread f of the workgroup reads float4 number f of x
// (each load instruction of a wave covers 1 KB of consecutive bytes); the
// eight float4s of one lane chunk sit in eight consecutive lanes, whose sum is
// formed with an 8-lane DPP reduction.  load() issues NPRE float4s per thread
// unconditionally (indices clamped into range) and store() consumes them
// unconditionally, so a caller that issues the weight stream in between
// waits for exactly these loads.  NT is the workgroup size (a multiple of
// 64), a compile-time constant: reading blockDim.x would cost a dependent
// memory load before the first activation load could issue.
template <int S, int NPRE, int NT>
struct XStageN {
    f32x4 v[NPRE];

    int rot;

    __device__ __forceinline__ void load(const float *__restrict__ x, int total)
    {
        rot = stage_rot(total);
#pragma unroll
        for (int j = 0; j < NPRE; j++)
            v[j] = ldx4(x, (uint32_t)stage_index((int)threadIdx.x + j * NT, total, rot));
    }

    __device__ __forceinline__ void store(const float *__restrict__ x, int total, int NU,
                                          f32x4 *__restrict__ xl, float *__restrict__ xs)
    {
        const int cpv = NU * 8;
#pragma unroll
        for (int j = 0; j < NPRE; j++) {
            const int f = (int)threadIdx.x + j * NT;
            int t, rem;
            split_f<S>(stage_index(f, total, rot), cpv, t, rem);
            XStagePut(v[j], f < total, t, rem, NU, xl, xs);
        }
        // remainder (shapes with more than NPRE float4s per thread)
        const int nrest = (total - NPRE * NT + NT - 1) / NT;
        for (int it = 0; it < nrest; it++) {
            const int f = (int)threadIdx.x + (NPRE + it) * NT;
            const int g = stage_index(f, total, rot);
            int t, rem;
            split_f<S>(g, cpv, t, rem);
            XStagePut(ldx4(x, (uint32_t)g), f < total, t, rem, NU, xl, xs);
        }
    }
};

// 2^-9 * sum over the 32 columns of one lane chunk of q*x.
__device__ __forceinline__ float nib_chunk_dot(const u32x4 wv, const f32x4 *__restrict__ xl,
                                               int NU, int u)
{
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        float e[4], o[4];
        nib8(wv[d], e, o);
        const f32x4 xe = xl[(2 * d) * seg_stride(NU) + u];
        const f32x4 xo = xl[(2 * d + 1) * seg_stride(NU) + u];
        p0 = __builtin_fmaf(e[0], xe.x, p0);
        p1 = __builtin_fmaf(o[0], xo.x, p1);
        p0 = __builtin_fmaf(e[1], xe.y, p0);
        p1 = __builtin_fmaf(o[1], xo.y, p1);
        p0 = __builtin_fmaf(e[2], xe.z, p0);
        p1 = __builtin_fmaf(o[2], xo.z, p1);
        p0 = __builtin_fmaf(e[3], xe.w, p0);
        p1 = __builtin_fmaf(o[3], xo.w, p1);
    }
    return p0 + p1;
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

__device__ __forceinline__ float sub_reduce8(float v) { return sub_reduce<8>(v); }

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
