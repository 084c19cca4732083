// abi.hip -- the extern "C" entry points: argument validation, then launch.
//
// Validation never touches a pointer's target: it looks at pointer values,
// dimensions and sizes only, so a refused call is safe with any pointers.
#include <mutex>
#include <unordered_map>

#include "qg_launch.h"

namespace qg {

hipError_t set_max_lds(const void *kernel, size_t bytes)
{
    static std::mutex mu;
    static std::unordered_map<const void *, size_t> done;
    if (bytes <= 64 * 1024) return hipSuccess;
    std::lock_guard<std::mutex> lock(mu);
    auto it = done.find(kernel);
    if (it != done.end() && it->second >= bytes) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)bytes);
    if (e == hipSuccess) done[kernel] = bytes;
    return e;
}

int cu_count()
{
    // per device, looked up once (256 on MI355X)
    static std::mutex mu;
    static std::unordered_map<int, int> cus;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus.find(dev);
    if (it != cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    cus[dev] = n;
    return n;
}

int pick_rows_per_group(int O, int lpr, int wpb, size_t lds, const int *cand, int ncand)
{
    const long ncu = cu_count();
    long per_cu = lds ? (long)(LDS_BUDGET / lds) : 32;
    const long by_waves = 32 / wpb;   // waves a CU holds
    per_cu = per_cu < by_waves ? per_cu : by_waves;
    per_cu = per_cu < 1 ? 1 : per_cu;
    int best = cand[ncand - 1];
    long best_rows = -1;
    for (int i = 0; i < ncand; i++) {
        const long rows_wg = (long)wpb * (64 / lpr) * cand[i];
        const long wgs = (O + rows_wg - 1) / rows_wg;
        const long wg_per_cu = (wgs + ncu - 1) / ncu;
        if (wg_per_cu > per_cu) continue;
        const long rows = wg_per_cu * rows_wg;
        if (best_rows < 0 || rows < best_rows) {
            best_rows = rows;
            best = cand[i];
        }
    }
    return best;
}

}  // namespace qg

namespace {

constexpr int MAX_DIM = 1 << 24;

// The calling thread's current device's address of `scratch` (below),
// looked up once per device (with that device current) and kept; no host or
// device memory is allocated.
constexpr int MAX_DEVICES = 64;
hipError_t scratch_address(void **out);

}  // namespace

// Device memory of the allocation-free routed-expert call: its per-token
// error flags (what the workspace of qgemv_moe_topk holds).  Each GPU has its
// own copy at its own address; host code uses that address (scratch_address),
// never this name, which on the host is only a stand-in.
static __device__ __align__(256) int scratch[qg::MOE_WORKSPACE_BYTES / sizeof(int)];

namespace {

hipError_t scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[MAX_DEVICES];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

bool mis4(const void *p) { return ((uintptr_t)p & 3) != 0; }

bool bad_gs(int gs) { return gs < 2 || (gs & 1) || gs > MAX_DIM; }

int launched(hipError_t e) { return e == hipSuccess ? QGEMV_OK : QGEMV_E_HIP; }

int check_gemv_dims(int S, int I, int O)
{
    if (S < 1 || S > QGEMV_MAX_S || I < 1 || O < 1 || I > MAX_DIM || O > MAX_DIM)
        return QGEMV_E_DIMS;
    return QGEMV_OK;
}

}  // namespace

extern "C" {

const char *qgemv_strerror(int status)
{
    switch (status) {
    case QGEMV_OK: return "ok";
    case QGEMV_E_NULL: return "a required pointer is NULL";
    case QGEMV_E_DIMS: return "a dimension is out of range";
    case QGEMV_E_GS: return "group size must be an even number in 2 .. 2^24";
    case QGEMV_E_ALIGN: return "an f32/int32 pointer is not 4-byte aligned";
    case QGEMV_E_K256: return "I must be a multiple of 256 for this format";
    case QGEMV_E_IDS: return "expert strides are smaller than one expert";
    case QGEMV_E_WORKSPACE: return "workspace is NULL or too small";
    case QGEMV_E_HIP: return "the HIP runtime reported an error at launch";
    default: return "unknown status";
    }
}

const char *qgemv_version(void) { return "0.1.0"; }

int qgemv_i4g(const void *w, const float *scales, const float *x, float *y, int S, int I,
              int O, int gs, void *stream)
{
    if (!w || !scales || !x || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (bad_gs(gs)) return QGEMV_E_GS;
    if (mis4(scales) || mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_i4g_gemv(w, scales, x, y, S, I, O, gs, (hipStream_t)stream));
}

int qgemv_i4g_prefill(const void *w, const float *scales, const float *x, float *y, int S,
                      int I, int O, int gs, void *stream)
{
    if (!w || !scales || !x || !y) return QGEMV_E_NULL;
    if (S < 1 || S > MAX_DIM || I < 1 || O < 1 || I > MAX_DIM || O > MAX_DIM) return QGEMV_E_DIMS;
    if ((long long)((S + 63) / 64) * ((O + 63) / 64) > 0x7FFFFFFFLL) return QGEMV_E_DIMS;
    if (bad_gs(gs)) return QGEMV_E_GS;
    if (mis4(scales) || mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_i4g_prefill(w, scales, x, y, S, I, O, gs, (hipStream_t)stream));
}

int qgemv_dequant_i4g(const void *w, const float *scales, float *W, int I, int O, int gs,
                      void *stream)
{
    if (!w || !scales || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (bad_gs(gs)) return QGEMV_E_GS;
    if (mis4(scales) || mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_i4g_dequant(w, scales, W, I, O, gs, (hipStream_t)stream));
}

int qgemv_fp8b128(const void *w, const float *scale_inv, const float *x, float *y, int S,
                  int I, int O, void *stream)
{
    if (!w || !scale_inv || !x || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (mis4(scale_inv) || mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_fp8b128_gemv(w, scale_inv, x, y, S, I, O, (hipStream_t)stream));
}

int qgemv_dequant_fp8b128(const void *w, const float *scale_inv, float *W, int I, int O,
                          void *stream)
{
    if (!w || !scale_inv || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (mis4(scale_inv) || mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_fp8b128_dequant(w, scale_inv, W, I, O, (hipStream_t)stream));
}

int qgemv_fp8b128_ue8m0(const void *w, const uint8_t *scale_e8m0, const float *x, float *y,
                        int S, int I, int O, void *stream)
{
    if (!w || !scale_e8m0 || !x || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_fp8ue8m0_gemv(w, scale_e8m0, x, y, S, I, O, (hipStream_t)stream));
}

int qgemv_dequant_fp8b128_ue8m0(const void *w, const uint8_t *scale_e8m0, float *W, int I, int O,
                                void *stream)
{
    if (!w || !scale_e8m0 || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_fp8ue8m0_dequant(w, scale_e8m0, W, I, O, (hipStream_t)stream));
}

int qgemv_mq4v2(const void *w, const float *x_rot, float *y, int S, int I, int O, void *stream)
{
    if (!w || !x_rot || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(x_rot) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4v2_gemv(w, x_rot, y, S, I, O, (hipStream_t)stream));
}

int qgemv_mq4v2_rot(const void *w, const float *x, const int8_t *signs, float *y, int S, int I,
                    int O, void *stream)
{
    if (!w || !x || !signs || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(y)) return QGEMV_E_ALIGN;
    if (int e = qg::mq4v2_rot_check(w, x, signs, I)) return e;
    return launched(qg::launch_mq4v2_rot_gemv(w, x, signs, y, S, I, O, (hipStream_t)stream));
}

int qgemv_mq4v1(const void *w, const float *x_rot, float *y, int S, int I, int O, void *stream)
{
    if (!w || !x_rot || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(x_rot) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4v1_gemv(w, x_rot, y, S, I, O, (hipStream_t)stream));
}

int qgemv_mq4c(const void *w, const float *x_rot, float *y, int S, int I, int O, void *stream)
{
    if (!w || !x_rot || !y) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(S, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(x_rot) || mis4(y)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4c_gemv(w, x_rot, y, S, I, O, (hipStream_t)stream));
}

int qgemv_dequant_mq4v1(const void *w, float *W, int I, int O, void *stream)
{
    if (!w || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4v1_dequant(w, W, I, O, (hipStream_t)stream));
}

int qgemv_dequant_mq4c(const void *w, float *W, int I, int O, void *stream)
{
    if (!w || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4c_dequant(w, W, I, O, (hipStream_t)stream));
}

int qgemv_mq4v2_encode(const float *W, void *w_out, int I, int O, void *stream)
{
    if (!W || !w_out) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (((uintptr_t)W & 15) || ((uintptr_t)w_out & 7)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4v2_encode(W, w_out, I, O, (hipStream_t)stream));
}

int qgemv_dequant_mq4v2(const void *w, float *W, int I, int O, void *stream)
{
    if (!w || !W) return QGEMV_E_NULL;
    if (int e = check_gemv_dims(1, I, O)) return e;
    if (I % 256) return QGEMV_E_K256;
    if (mis4(W)) return QGEMV_E_ALIGN;
    return launched(qg::launch_mq4v2_dequant(w, W, I, O, (hipStream_t)stream));
}

int qgemv_fwht256(const float *x, const int8_t *signs, float *x_rot, int S, int I, void *stream)
{
    if (!x || !signs || !x_rot) return QGEMV_E_NULL;
    if (S < 1 || S > QGEMV_MAX_S || I < 1 || I > MAX_DIM) return QGEMV_E_DIMS;
    if (I % 256) return QGEMV_E_K256;
    // x and x_rot are read and written as float4
    if (((uintptr_t)x | (uintptr_t)x_rot) & 15) return QGEMV_E_ALIGN;
    return launched(qg::launch_fwht256(x, signs, x_rot, S, I, (hipStream_t)stream));
}

int qgemv_router_topk(const float *logits, int T, int E, int ld, int K, int32_t *ids,
                      float *gates, void *stream)
{
    if (!logits || !ids || !gates) return QGEMV_E_NULL;
    if (T < 1 || T > MAX_DIM || E < 1 || E > 1024 || ld < E || K < 1 || K > 64 || K > E)
        return QGEMV_E_DIMS;
    if (mis4(logits) || mis4(ids) || mis4(gates)) return QGEMV_E_ALIGN;
    return launched(qg::launch_router_topk(logits, T, E, ld, K, ids, gates, (hipStream_t)stream));
}

size_t qgemv_moe_topk_workspace(int T, int K, int O)
{
    (void)T; (void)K; (void)O;
    return qg::MOE_WORKSPACE_BYTES;
}

int qgemv_moe_topk(const void *w, const float *scales, long long w_stride, long long s_stride,
                   int E, const int32_t *ids, const float *gates, int T, int K, const float *x,
                   float *y, int I, int O, int gs, void *workspace, size_t ws_bytes,
                   void *stream)
{
    if (!w || !scales || !ids || !gates || !x || !y) return QGEMV_E_NULL;
    if (T < 1 || T > QGEMV_MAX_S || K < 1 || K > 64 || E < 1 || I < 1 || O < 1 ||
        I > MAX_DIM || O > MAX_DIM)
        return QGEMV_E_DIMS;
    if (bad_gs(gs)) return QGEMV_E_GS;
    if (mis4(scales) || mis4(ids) || mis4(gates) || mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    const long long rb = ((long long)I + 1) / 2, ng = ((long long)I + gs - 1) / gs;
    if (w_stride < (long long)O * rb || s_stride < (long long)O * ng) return QGEMV_E_IDS;
    if (!workspace || ws_bytes < qgemv_moe_topk_workspace(T, K, O) || mis4(workspace))
        return QGEMV_E_WORKSPACE;
    return launched(qg::launch_moe_topk(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y,
                                        I, O, gs, static_cast<int *>(workspace),
                                        (hipStream_t)stream));
}

int qgemv_moe_topk_noalloc(const void *w, const float *scales, long long w_stride,
                           long long s_stride, int E, const int32_t *ids, const float *gates,
                           int T, int K, const float *x, float *y, int I, int O, int gs,
                           void *stream)
{
    if (!w || !scales || !ids || !gates || !x || !y) return QGEMV_E_NULL;
    if (T < 1 || T > QGEMV_MAX_S || K < 1 || K > 64 || E < 1 || I < 1 || O < 1 ||
        I > MAX_DIM || O > MAX_DIM)
        return QGEMV_E_DIMS;
    if (bad_gs(gs)) return QGEMV_E_GS;
    if (mis4(scales) || mis4(ids) || mis4(gates) || mis4(x) || mis4(y)) return QGEMV_E_ALIGN;
    const long long rb = ((long long)I + 1) / 2, ng = ((long long)I + gs - 1) / gs;
    if (w_stride < (long long)O * rb || s_stride < (long long)O * ng) return QGEMV_E_IDS;
    // the flags' room in the device array (the same size as the workspace
    // qgemv_moe_topk asks for)
    if (qgemv_moe_topk_workspace(T, K, O) > sizeof(scratch)) return QGEMV_E_WORKSPACE;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess || !ws) return QGEMV_E_HIP;
    return launched(qg::launch_moe_topk(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y,
                                        I, O, gs, static_cast<int *>(ws), (hipStream_t)stream));
}

int qgemv_moe_topk_error(const void *workspace, int *flag, void *stream)
{
    if (!workspace || !flag) return QGEMV_E_NULL;
    if (mis4(workspace)) return QGEMV_E_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    // one flag per token slot (QGEMV_MAX_S of them)
    int f[QGEMV_MAX_S];
    if (hipMemcpyAsync(f, workspace, sizeof(f), hipMemcpyDeviceToHost, st) != hipSuccess)
        return QGEMV_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return QGEMV_E_HIP;
    int any = 0;
    for (int v : f) any |= v != 0;
    *flag = any;
    return QGEMV_OK;
}

}  // extern "C"
