// prefill.hip -- many-token grouped-int4 products on the matrix cores (gfx950).
//
// Y[S][O] = X[S][I] . W^T for S tokens at once (prompt prefill), W grouped
// int4 as the GEMV reads it (colibri PR #457 "metal: grouped-int4 (fmt=4)
// GEMV support", sections 1 and 3: w = (q - 8) * s[row][col / gs]).  With S
// in the tens to thousands this is a real contraction (2*S flops per weight
// byte pair), so it runs on MFMA: v_mfma_f32_16x16x4_f32, f32 operands and
// accumulation, so the result meets the same f32-accumulate bar as the GEMV.
//
// Tiling: a workgroup of 4 waves computes a 64 (tokens) x 64 (rows of W)
// tile; each wave a 32 x 32 quarter as 2 x 2 MFMA blocks.  Per K step of 32
// columns (inside one scale group, gs % 32 == 0) the workgroup stages the
// 64 x 32 activations and the 64 x 32 decoded weights ((q - 8) * s in f32,
// one rounding, as the definition) in LDS, then runs 8 MFMA k-steps; the
// global loads of the next step are in flight meanwhile.  Lane
// layout of the 16x16x4 block (checked on the device): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator register i of lane l
// is D[4 (l / 16) + i][l % 16].
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

namespace {

constexpr int PM = 64;          // tokens per workgroup tile
constexpr int PN = 64;          // weight rows per workgroup tile
constexpr int PK = 32;          // columns per K step
constexpr int PLD = PK + 4;     // LDS row stride in floats (16-byte aligned rows)

typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void i4g_gemm_mfma(const uint8_t *__restrict__ w,
                                                     const float *__restrict__ scales,
                                                     const float *__restrict__ x,
                                                     float *__restrict__ y, int S, int I, int O,
                                                     int ng, int gs)
{
    // The global loads of step k + 1 are in flight while step k multiplies.
    // One LDS buffer: measured against two (one barrier per step, half the
    // resident tiles) at 12288 x 6144, 345 vs 346 us at 256 tokens and 2518
    // vs 2593 us at 2048; without the early loads 361 and 2521 us.
    __shared__ __align__(16) float xs[PM * PLD];
    __shared__ __align__(16) float ws[PN * PLD];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int ntn = (O + PN - 1) / PN;                  // tiles along O
    const int s0 = (int)(blockIdx.x / ntn) * PM, o0 = (int)(blockIdx.x % ntn) * PN;
    const size_t rb = (size_t)I / 2;

    f32x4v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

    // staging assignments: activations, two float4 per thread (row tid / 4,
    // float4 2 (tid % 4) and 2 (tid % 4) + 1); weights, one packed dword per
    // thread (row tid / 4, dword tid % 4 = columns 8 (tid % 4) .. + 7)
    const int xr = tid >> 2, xc = (tid & 3) * 8;
    const int xrow = s0 + xr;
    const bool xok = xrow < S;
    const float *xsrc = x + (size_t)min(xrow, S - 1) * I + xc;
    const int wrr = tid >> 2, wd = tid & 3;
    const int wrow = o0 + wrr;
    const bool wok = wrow < O;
    const uint8_t *wsrc = w + (size_t)min(wrow, O - 1) * rb + wd * 4;
    const float *ssrc = scales + (size_t)min(wrow, O - 1) * ng;

    f32x4v x0, x1;
    uint32_t wv;
    float sg;
    auto load = [&](int k0) {
        x0 = *reinterpret_cast<const f32x4v *>(xsrc + k0);
        x1 = *reinterpret_cast<const f32x4v *>(xsrc + k0 + 4);
        wv = *reinterpret_cast<const uint32_t *>(wsrc + k0 / 2);
        sg = ssrc[k0 / gs];
    };
    auto stage = [&]() {
        const f32x4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
        *reinterpret_cast<f32x4v *>(&xs[xr * PLD + xc]) = xok ? x0 : zero;
        *reinterpret_cast<f32x4v *>(&xs[xr * PLD + xc + 4]) = xok ? x1 : zero;
        float e[4], o[4];
        nib8(wv, e, o);
        f32x4v w0, w1;
        w0.x = (e[0] * NIB_XSCALE - 8.0f) * sg;  w0.y = (o[0] * NIB_XSCALE - 8.0f) * sg;
        w0.z = (e[1] * NIB_XSCALE - 8.0f) * sg;  w0.w = (o[1] * NIB_XSCALE - 8.0f) * sg;
        w1.x = (e[2] * NIB_XSCALE - 8.0f) * sg;  w1.y = (o[2] * NIB_XSCALE - 8.0f) * sg;
        w1.z = (e[3] * NIB_XSCALE - 8.0f) * sg;  w1.w = (o[3] * NIB_XSCALE - 8.0f) * sg;
        *reinterpret_cast<f32x4v *>(&ws[wrr * PLD + wd * 8]) = wok ? w0 : zero;
        *reinterpret_cast<f32x4v *>(&ws[wrr * PLD + wd * 8 + 4]) = wok ? w1 : zero;
    };

    load(0);
    for (int k0 = 0; k0 < I; k0 += PK) {
        if (k0 > 0) __syncthreads();                     // the previous step's reads are done
        stage();
        __syncthreads();
        if (k0 + PK < I) load(k0 + PK);                  // in flight during the products
        const float *xb = xs;
        const float *wb = ws;
#pragma unroll
        for (int kk = 0; kk < PK; kk += 4) {
            float a[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; i++)
                a[i] = xb[(wm * 32 + i * 16 + (lane & 15)) * PLD + kk + (lane >> 4)];
#pragma unroll
            for (int j = 0; j < 2; j++)
                bv[j] = wb[(wn * 32 + j * 16 + (lane & 15)) * PLD + kk + (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bv[j], acc[i][j], 0, 0,
                                                                      0);
        }
    }

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int s = s0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
                const int oo = o0 + wn * 32 + j * 16 + (lane & 15);
                if (s < S && oo < O) y[(size_t)s * O + oo] = acc[i][j][r];
            }
}

}  // namespace

bool i4g_prefill_fast(const void *w, const float *x, int I, int gs)
{
    return I % PK == 0 && gs % PK == 0 && ((uintptr_t)w & 3) == 0 && ((uintptr_t)x & 15) == 0;
}

hipError_t launch_i4g_prefill(const void *w, const float *scales, const float *x, float *y,
                              int S, int I, int O, int gs, hipStream_t st)
{
    if (!i4g_prefill_fast(w, x, I, gs)) {
        // shapes the tiles do not take: the GEMV, QGEMV_MAX_S tokens per call
        for (int s0 = 0; s0 < S; s0 += QGEMV_MAX_S) {
            const int n = S - s0 < QGEMV_MAX_S ? S - s0 : QGEMV_MAX_S;
            hipError_t e = launch_i4g_gemv(w, scales, x + (size_t)s0 * I, y + (size_t)s0 * O, n,
                                           I, O, gs, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const long long tiles = (long long)((S + PM - 1) / PM) * ((O + PN - 1) / PN);
    if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(i4g_gemm_mfma, dim3((unsigned)tiles), dim3(256), 0, st,
                       static_cast<const uint8_t *>(w), scales, x, y, S, I, O,
                       (I + gs - 1) / gs, gs);
    return hipGetLastError();
}

}  // namespace qg
