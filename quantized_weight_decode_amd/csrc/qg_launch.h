// qg_launch.h -- host-side launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

// LDS a workgroup may ask for on gfx950 (160 KiB per CU).
constexpr size_t LDS_BUDGET = 160 * 1024;

// Raises a kernel's dynamic-LDS limit to `bytes` once (cached per kernel).
hipError_t set_max_lds(const void *kernel, size_t bytes);

// grouped int4
bool i4g_stream_ok(const void *w, const float *x, int S, int I, int gs);
size_t i4g_stream_lds_bytes(int S, int I);
hipError_t launch_i4g_gemv(const void *w, const float *scales, const float *x, float *y,
                           int S, int I, int O, int gs, hipStream_t st);
hipError_t launch_i4g_dequant(const void *w, const float *scales, float *W, int I, int O,
                              int gs, hipStream_t st);

}  // namespace qg
