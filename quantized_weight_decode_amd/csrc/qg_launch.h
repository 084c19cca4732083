// qg_launch.h -- host-side launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

// LDS a workgroup may ask for on gfx950 (160 KiB per CU).
constexpr size_t LDS_BUDGET = 160 * 1024;

// Lanes per row for a row of `nchunks` 16-byte lane chunks: the widest of
// 64/32/16/8/4 lanes whose sweeps leave the fewest lanes idle (the launchers
// use it through pick_lpr_wide, for short rows only).
inline int pick_lpr(int nchunks)
{
    const int opts[] = {64, 32, 16, 8, 4};
    int best = 4;
    double best_eff = -1.0;
    for (int lpr : opts) {
        const int it = (nchunks + lpr - 1) / lpr;
        const double eff = (double)nchunks / ((double)it * lpr);
        if (eff > best_eff + 1e-9) { best_eff = eff; best = lpr; }
    }
    return best;
}

// Lanes per row for the streaming GEMVs (all four formats): for rows of at
// least 32 chunks, 64 or 32, whichever leaves fewer lanes idle (ties to 64);
// shorter rows as pick_lpr.  pick_lpr alone gives rows such as 1408, 2176,
// 4352, 11008 or 18944 columns 4 to 16 lanes, and such short segments per row
// stream far slower (e.g. 4096 x 11008: i4g 18.8 -> 8.8 us, MQ4 19.3 -> 8.7
// us, fp8 12.7 -> 11.3 us; routed experts of 2048 x 1408: 41.5 -> 17.6 us).
// Rows of 48, 80 or 112 chunks, which 16 lanes fit exactly, keep this rule
// too: 16 lanes there gain up to 6 % on some row counts (4-bit 18944 x 3584
// 4-5 %) and lose up to 15 % on others (i4g 37888 x 3584, 12288 x 3584).
inline int pick_lpr_wide(int nchunks)
{
    if (nchunks < 32) return pick_lpr(nchunks);
    const long s64 = (nchunks + 63) / 64, s32 = (nchunks + 31) / 32;
    return s64 * 64 > s32 * 32 ? 32 : 64;
}

// Raises a kernel's dynamic-LDS limit to `bytes` once (cached per kernel).
hipError_t set_max_lds(const void *kernel, size_t bytes);
// Compute units of the current device.
int cu_count();

// Rows per lane group, out of the ncand candidates, for a streaming kernel
// whose workgroups hold wpb waves of 64 / lpr lane groups and lds bytes of
// LDS: the choice keeps every workgroup resident at once (one round) and
// gives the most loaded CU the fewest rows.  Falls back to the largest
// candidate when none fits one round.
int pick_rows_per_group(int O, int lpr, int wpb, size_t lds, const int *cand, int ncand);

// One-vector tile: wpb waves per workgroup, r rows per lane group.
struct WaveTile {
    int wpb, r;
};
// Index of the tile, out of n candidates, for O rows with rpg lane groups per
// wave on ncu CUs.  Workgroups are dealt to the CUs in rounds, so the tile
// whose workgroup count fills its last round best (workgroups / (CUs x
// rounds)) wins; among equals the one with the fewest workgroups, then the
// one with more rows per lane group.  With one_row_single, one-row tiles
// count only where they leave at most one workgroup per CU (the first
// candidate must have more rows).
inline int pick_fill_tile(long O, long rpg, const WaveTile *cand, int n, long ncu,
                          bool one_row_single = false)
{
    int best = 0;
    double best_fill = -1.0;
    long best_wgs = 0;
    for (int i = 0; i < n; i++) {
        const long rows_wg = cand[i].wpb * rpg * cand[i].r;
        const long wgs = (O + rows_wg - 1) / rows_wg;
        if (one_row_single && cand[i].r == 1 && wgs > ncu) continue;
        const double fill = (double)wgs / (double)(((wgs + ncu - 1) / ncu) * ncu);
        const bool better =
            fill > best_fill + 1e-9 ||
            (fill > best_fill - 1e-9 &&
             (wgs < best_wgs || (wgs == best_wgs && cand[i].r > cand[best].r)));
        if (better) {
            best = i;
            best_fill = fill;
            best_wgs = wgs;
        }
    }
    return best;
}

// grouped int4
// Vectors one streaming launch takes for this shape (0: the streaming
// kernel does not apply; larger S runs in groups of this many).
int i4g_stream_vectors(const void *w, const float *x, int S, int I, int gs);
size_t i4g_stream_lds_bytes(int S, int I);
hipError_t launch_i4g_gemv(const void *w, const float *scales, const float *x, float *y,
                           int S, int I, int O, int gs, hipStream_t st);
hipError_t launch_i4g_dequant(const void *w, const float *scales, float *W, int I, int O,
                              int gs, hipStream_t st);

// fp8-e4m3, 128x128 block scales
hipError_t launch_fp8b128_gemv(const void *w, const float *scale_inv, const float *x, float *y,
                               int S, int I, int O, hipStream_t st);
hipError_t launch_fp8b128_dequant(const void *w, const float *scale_inv, float *W, int I, int O,
                                  hipStream_t st);
// fp8-e4m3 with UE8M0 (power-of-two byte) 128x128 block scales
hipError_t launch_fp8ue8m0_gemv(const void *w, const uint8_t *scale_e8m0, const float *x,
                                float *y, int S, int I, int O, hipStream_t st);
hipError_t launch_fp8ue8m0_dequant(const void *w, const uint8_t *scale_e8m0, float *W, int I,
                                   int O, hipStream_t st);

// MQ4-v2 and the FWHT-256 rotation
hipError_t launch_mq4v2_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                             hipStream_t st);
// Fused rotation + GEMV: QGEMV_OK if the fused kernel takes the shape
// (8-byte aligned w and signs, 16-byte aligned x, one vector's staging within
// the LDS), else the refusal code.
int mq4v2_rot_check(const void *w, const float *x, const int8_t *signs, int I);
hipError_t launch_mq4v2_rot_gemv(const void *w, const float *x, const int8_t *signs, float *y,
                                 int S, int I, int O, hipStream_t st);
hipError_t launch_mq4v2_dequant(const void *w, float *W, int I, int O, hipStream_t st);
// MQ4 v1 (f32 header per 256) and MQ4C pad (fp16 pair per 256 + zero pad)
hipError_t launch_mq4v1_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                             hipStream_t st);
hipError_t launch_mq4c_gemv(const void *w, const float *x, float *y, int S, int I, int O,
                            hipStream_t st);
hipError_t launch_mq4v1_dequant(const void *w, float *W, int I, int O, hipStream_t st);
hipError_t launch_mq4c_dequant(const void *w, float *W, int I, int O, hipStream_t st);
// MQ4-v2 encoder: W f32 [O][I] (rotated space, 16-byte aligned) -> 136-byte groups
hipError_t launch_mq4v2_encode(const float *W, void *out, int I, int O, hipStream_t st);
hipError_t launch_fwht256(const float *x, const int8_t *signs, float *xr, int S, int I,
                          hipStream_t st);

// routed experts
constexpr size_t MOE_WORKSPACE_BYTES = 256;
hipError_t launch_moe_topk(const void *w, const float *scales, long long w_stride,
                           long long s_stride, int E, const int32_t *ids, const float *gates,
                           int T, int K, const float *x, float *y, int I, int O, int gs,
                           int *err_flag, hipStream_t st);

// many-token grouped-int4 product on MFMA (any S >= 1)
hipError_t launch_i4g_prefill(const void *w, const float *scales, const float *x, float *y,
                              int S, int I, int O, int gs, hipStream_t st);

// router top-k (E <= 1024, K <= min(E, 64))
hipError_t launch_router_topk(const float *logits, int T, int E, int ld, int K, int32_t *ids,
                              float *gates, hipStream_t st);

}  // namespace qg
