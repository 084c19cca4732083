// ceiling.hip -- plain streaming reads of device memory (no arithmetic): the
// attainable-bandwidth reference that the GEMV kernels are measured against.
//
// Built into its own library (libqgemv_ceiling.so) for the benchmark only; it
// is not part of the qgemv C ABI.
//
// Two access patterns:
//   * CONTIG: the buffer as consecutive 16-byte chunks, one global_load_dwordx4
//     per lane per chunk (a wave reads 1 KiB per load instruction);
//   * MQ4: the buffer as 136-byte groups (two header dwords, then 128 payload
//     bytes); chunk c is the 16 payload bytes at 136 (c / 8) + 8 + 16 (c % 8),
//     an 8-byte-aligned 16-byte load, plus the header dword at
//     136 (c / 8) + 4 (c % 8 >= 4) -- the reads an MQ4-v2 GEMV makes.
// Each pattern reads with the non-temporal hint or as ordinary cached loads
// (pattern | 2): the faster of the two is the reference.
// Slab mapping: workgroup b reads the b-th contiguous slab of chunks; wave w of it reads
// the 64-chunk pieces w, w + WPB, ... of the slab, U pieces in flight per
// lane (a ring: the oldest is consumed, then refilled U pieces ahead).  The
// XOR of everything a wave read is stored to out[global wave index], so no
// load can be dropped.  Every load is unconditional (indices clamped into the
// slab; a slab's padding re-reads its last chunk and is not XOR-ed in).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));

enum : int { CONTIG = 0, MQ4 = 1, CACHED = 2 };

template <bool NT, typename T>
__device__ __forceinline__ T rd(const T *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int PAT>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t *__restrict__ p, size_t c)
{
    constexpr bool NT = !(PAT & CACHED);
    if constexpr ((PAT & MQ4) == 0) {
        return rd<NT>(reinterpret_cast<const u32x4 *>(p) + c);
    } else {
        const uint8_t *g = p + (c >> 3) * 136;
        const uint32_t q = (uint32_t)c & 7u;
        const u32x4_a8 v = rd<NT>(reinterpret_cast<const u32x4_a8 *>(g + 8 + 16 * q));
        const uint32_t h = rd<NT>(reinterpret_cast<const uint32_t *>(g + (q >= 4 ? 4 : 0)));
        return u32x4{v.x ^ h, v.y, v.z, v.w};
    }
}

template <int PAT, int WPB, int U>
__global__ __launch_bounds__(64 * WPB) void read_stream(const uint8_t *__restrict__ p,
                                                        size_t nchunks, size_t per_wg,
                                                        uint32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const size_t base = (size_t)blockIdx.x * per_wg;
    const size_t end = base + per_wg < nchunks ? base + per_wg : nchunks;
    // piece k of this wave: chunks base + (k * WPB + wave) * 64 + lane
    const size_t npieces = base < end ? (end - base + 63) / 64 : 0;
    const size_t mine = npieces > (size_t)wave ? (npieces - wave + WPB - 1) / WPB : 0;
    if (mine == 0) {
        if (lane == 0) out[(size_t)blockIdx.x * WPB + wave] = 0;
        return;
    }
    auto idx = [&](size_t k) {
        const size_t c = base + (k * WPB + wave) * 64 + lane;
        return c < end ? c : end - 1;
    };
    auto valid = [&](size_t k) { return k < mine && base + (k * WPB + wave) * 64 + lane < end; };
    u32x4 ring[U];
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < U; j++) ring[j] = load_chunk<PAT>(p, idx(j));
    const size_t rounds = (mine + U - 1) / U;
    for (size_t r = 0; r + 1 < rounds; r++) {
#pragma unroll
        for (int j = 0; j < U; j++) {
            const size_t k = r * U + j;
            if (valid(k)) acc ^= ring[j];
            ring[j] = load_chunk<PAT>(p, idx(k + U));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // last round: no refills
#pragma unroll
    for (int j = 0; j < U; j++)
        if (valid((rounds - 1) * U + j)) acc ^= ring[j];
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v ^= __shfl_xor(v, m, 64);
    if (lane == 0) out[(size_t)blockIdx.x * WPB + wave] = v;
}

// One-shot mapping: wave v of the grid reads the U consecutive 64-chunk
// pieces U v .. U v + U - 1 (all loads issued at once) and exits; the grid
// covers the buffer, so the dispatcher keeps the CUs fed with fresh waves.
template <int PAT, int WPB, int U>
__global__ __launch_bounds__(64 * WPB) void read_oneshot(const uint8_t *__restrict__ p,
                                                         size_t nchunks,
                                                         uint32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const size_t v = (size_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    u32x4 r[U];
#pragma unroll
    for (int k = 0; k < U; k++) {
        const size_t c = (v * U + k) * 64 + lane;
        r[k] = load_chunk<PAT>(p, c < nchunks ? c : nchunks - 1);
    }
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < U; k++)
        if ((v * U + k) * 64 + lane < nchunks) acc ^= r[k];
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
    if (lane == 0) out[v] = x;
}

// wgs > 0: slab mapping over wgs workgroups; wgs == 0: one-shot mapping
// (out needs one u32 per wave of the grid)
template <int PAT, int WPB, int U>
hipError_t launch(const void *buf, size_t nchunks, int wgs, uint32_t *out, hipStream_t st)
{
    if (wgs == 0) {
        const size_t waves = (nchunks + 64 * U - 1) / (64 * U);
        const size_t grid = (waves + WPB - 1) / WPB;
        hipLaunchKernelGGL((read_oneshot<PAT, WPB, U>), dim3((unsigned)grid), dim3(64 * WPB), 0,
                           st, static_cast<const uint8_t *>(buf), nchunks, out);
        return hipGetLastError();
    }
    const size_t per_wg = (nchunks + wgs - 1) / wgs;
    hipLaunchKernelGGL((read_stream<PAT, WPB, U>), dim3(wgs), dim3(64 * WPB), 0, st,
                       static_cast<const uint8_t *>(buf), nchunks, per_wg, out);
    return hipGetLastError();
}

template <int PAT, int WPB>
hipError_t launch_u(int u, const void *buf, size_t nchunks, int wgs, uint32_t *out,
                    hipStream_t st)
{
    switch (u) {
    case 1: return launch<PAT, WPB, 1>(buf, nchunks, wgs, out, st);
    case 2: return launch<PAT, WPB, 2>(buf, nchunks, wgs, out, st);
    case 4: return launch<PAT, WPB, 4>(buf, nchunks, wgs, out, st);
    default: return launch<PAT, WPB, 8>(buf, nchunks, wgs, out, st);
    }
}

template <int PAT>
hipError_t launch_wpb(int wpb, int u, const void *buf, size_t nchunks, int wgs, uint32_t *out,
                      hipStream_t st)
{
    switch (wpb) {
    case 4: return launch_u<PAT, 4>(u, buf, nchunks, wgs, out, st);
    case 8: return launch_u<PAT, 8>(u, buf, nchunks, wgs, out, st);
    default: return launch_u<PAT, 16>(u, buf, nchunks, wgs, out, st);
    }
}

}  // namespace

extern "C" {

// Reads `bytes` bytes of device memory at `buf` once.
//   pattern 0: contiguous 16-byte chunks (bytes % 16 == 0, buf 16-byte aligned);
//   pattern 1: MQ4 136-byte groups (bytes % 136 == 0, buf 8-byte aligned);
//   pattern | 2: the same reads as ordinary cached loads instead of with the
//   non-temporal hint.
//   wpb in {4, 8, 16} waves per workgroup, u in {1, 2, 4, 8} loads in flight
//   per lane; wgs >= 1 workgroups of the slab mapping (u >= 2), or 0 for the
//   one-shot mapping.  out: device u32, one per wave of the grid, at most
//   out_len of them.
// Returns 0 if launched, 1 on a refused argument, 2 on a launch error.
int qgemv_ceiling_read(const void *buf, size_t bytes, int pattern, int wpb, int u, int wgs,
                       uint32_t *out, size_t out_len, void *stream)
{
    if (!buf || !out || wgs < 0 || wgs > (1 << 20)) return 1;
    if (wpb != 4 && wpb != 8 && wpb != 16) return 1;
    if (u != 1 && u != 2 && u != 4 && u != 8) return 1;
    if (wgs > 0 && u == 1) return 1;
    if (pattern < 0 || pattern > 3) return 1;
    const bool mq4 = (pattern & MQ4) != 0;
    const size_t nch = mq4 ? bytes / 136 * 8 : bytes / 16;
    const size_t waves = wgs > 0 ? (size_t)wgs * wpb
                                 : ((nch + 64 * (size_t)u - 1) / (64 * u) + wpb - 1) / wpb * wpb;
    if (waves > out_len) return 1;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (!mq4) {
        if (bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15)) return 1;
        e = pattern & CACHED ? launch_wpb<CONTIG | CACHED>(wpb, u, buf, nch, wgs, out, st)
                             : launch_wpb<CONTIG>(wpb, u, buf, nch, wgs, out, st);
    } else {
        if (bytes == 0 || bytes % 136 || ((uintptr_t)buf & 7)) return 1;
        e = pattern & CACHED ? launch_wpb<MQ4 | CACHED>(wpb, u, buf, nch, wgs, out, st)
                             : launch_wpb<MQ4>(wpb, u, buf, nch, wgs, out, st);
    }
    return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
