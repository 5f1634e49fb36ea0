// Internal helpers shared by the HIP sources of the library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/spec.h"

#define SPEC_WAVE 64

namespace spec {

// ---- bf16 <-> f32 -----------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- status word --------------------------------------------------------------

__device__ __forceinline__ void raise_status(int32_t *st, int bits) {
    if (st != nullptr && bits != 0) atomicOr(st, bits);
}

// ---- wave reductions (64 lanes) ---------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workgroups of `kernel` (launched with `threads` threads, no dynamic LDS)
// that the current device holds at once, or 0 when that is unknown (or, with
// need_coop, when the device has no cooperative launch).  Evaluated on every
// call: the library keeps no state between calls.
inline int resident_capacity(const void *kernel, int threads, bool need_coop = false) {
    int dev = 0, cus = 0, per = 0, coop = 1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (need_coop &&
        (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
         coop == 0))
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess)
        return 0;
    return cus * per;
}

// Polls of one exchange or key slot before a wait gives up and raises
// SPEC_ST_SYNC: 2^20 (about a second), or the value of the environment
// variable SPEC_POLL_LIMIT when it holds a decimal number up to 2^30.  Read
// on every call; a small value forces the time-out path from the host.
inline unsigned poll_limit() {
    constexpr unsigned kDefault = 1u << 20;
    const char *s = getenv("SPEC_POLL_LIMIT");
    if (s == nullptr || *s == 0) return kDefault;
    char *end = nullptr;
    const unsigned long v = strtoul(s, &end, 10);
    if (*end != 0 || v > (1ul << 30)) return kDefault;
    return (unsigned)v;
}

// True while `st` records into a graph.  A recorded kernel may run beside
// kernels of other streams, so forms whose workgroups wait on each other are
// not recorded.
inline bool stream_capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

}  // namespace spec
