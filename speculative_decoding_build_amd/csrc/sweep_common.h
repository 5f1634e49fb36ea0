// Helpers shared by the vocabulary sweeps of the accept kernels.
#pragma once

#include <float.h>
#include <limits.h>
#include <math.h>

#include "spec_common.h"

namespace spec {

constexpr int kSweepThreads = 256;
constexpr int kPerThread = 32;                       // elements per thread per row
constexpr int kChunk = kSweepThreads * kPerThread;   // 8192 vocabulary entries per chunk
constexpr int kMaxNodes = 64;

inline int num_chunks(int64_t vocab) { return (int)((vocab + kChunk - 1) / kChunk); }

// ---- loads ----------------------------------------------------------------

// Loads the kPerThread elements thread `tid` owns in [start, end) of `row`
// as floats; missing elements get -inf.  Element e of the thread is at
// start + (e / 8) * kSweepThreads * 8 + tid * 8 + e % 8, so each 8-group is
// one 16-byte load (bf16) and a wave reads 1 KB contiguous.
template <int DT>
__device__ __forceinline__ void load_chunk(const void *base, int64_t start, int64_t end,
                                           bool vec_ok, int tid, float (&x)[kPerThread]) {
#pragma unroll
    for (int g = 0; g < kPerThread / 8; ++g) {
        const int64_t e0 = start + (int64_t)g * kSweepThreads * 8 + tid * 8;
        if (DT == SPEC_BF16) {
            const uint16_t *p = static_cast<const uint16_t *>(base);
            if (vec_ok && e0 + 8 <= end) {
                const uint4 w = *reinterpret_cast<const uint4 *>(p + e0);
                x[g * 8 + 0] = spec::lo_bf16(w.x);
                x[g * 8 + 1] = spec::hi_bf16(w.x);
                x[g * 8 + 2] = spec::lo_bf16(w.y);
                x[g * 8 + 3] = spec::hi_bf16(w.y);
                x[g * 8 + 4] = spec::lo_bf16(w.z);
                x[g * 8 + 5] = spec::hi_bf16(w.z);
                x[g * 8 + 6] = spec::lo_bf16(w.w);
                x[g * 8 + 7] = spec::hi_bf16(w.w);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[g * 8 + j] = (e0 + j < end) ? spec::bf16_to_f32(p[e0 + j]) : -INFINITY;
            }
        } else {
            const float *p = static_cast<const float *>(base);
            if (vec_ok && e0 + 8 <= end) {
                const float4 a = *reinterpret_cast<const float4 *>(p + e0);
                const float4 b = *reinterpret_cast<const float4 *>(p + e0 + 4);
                x[g * 8 + 0] = a.x; x[g * 8 + 1] = a.y; x[g * 8 + 2] = a.z; x[g * 8 + 3] = a.w;
                x[g * 8 + 4] = b.x; x[g * 8 + 5] = b.y; x[g * 8 + 6] = b.z; x[g * 8 + 7] = b.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[g * 8 + j] = (e0 + j < end) ? p[e0 + j] : -INFINITY;
            }
        }
    }
}

__device__ __forceinline__ int64_t elem_index(int64_t start, int tid, int e) {
    return start + (int64_t)(e / 8) * kSweepThreads * 8 + tid * 8 + (e % 8);
}

// exp((x - m) / T) to about one float ulp: x - m as an exact float pair
// (two-sum), 1/T as a float pair, the rounding of the product folded back
// as a first-order correction.  A masked entry (x = -inf) gives 0.
struct Scale {
    float m;
    float ithi;
    float itlo;
};

__device__ __forceinline__ float exp_scaled(float x, const Scale &s) {
    const float d = x - s.m;
    const float bp = d - x;
    const float derr = (x - (d - bp)) + (-s.m - bp);
    const float y = d * s.ithi;
    const float delta = fmaf(d, s.ithi, -y) + fmaf(d, s.itlo, derr * s.ithi);
    const float e = expf(y);
    return x == -INFINITY ? 0.f : fmaf(e, delta, e);   // -inf: the pair above is NaN
}

// exp((x - m) / T) from the hardware base-2 exponential: (x - m) as an
// exact float pair, log2(e) / T as a float pair, so (x - m) log2(e) / T is
// y + delta to about 2^-48 relative; 2^y (v_exp_f32) times (1 + delta ln 2).
// A masked entry (x = -inf) gives 0; results below 2^-126 flush to 0.
struct Scale2 {
    float m;
    float chi;
    float clo;
};

__device__ __forceinline__ Scale2 make_scale2(float m, float temperature) {
    const double c = 1.4426950408889634 / (double)temperature;
    const float hi = (float)c;
    return Scale2{m, hi, (float)(c - (double)hi)};
}

// the same scale at another max
__device__ __forceinline__ Scale2 rebase(const Scale2 &s, float m) {
    return Scale2{m, s.chi, s.clo};
}

__device__ __forceinline__ float exp2_scaled(float x, const Scale2 &s) {
    constexpr float kLn2 = 0.69314718055994531f;
    const float d = x - s.m;
    const float bp = d - x;
    const float derr = (x - (d - bp)) + (-s.m - bp);
    const float y = d * s.chi;
    const float delta = fmaf(d, s.chi, -y) + fmaf(d, s.clo, derr * s.chi);
    const float e = __builtin_amdgcn_exp2f(y);
    return x == -INFINITY ? 0.f : fmaf(e, delta * kLn2, e);
}

// 1/T as a float pair (high part, rounding remainder)
__device__ __forceinline__ Scale make_scale(float m, float temperature) {
    const double it = 1.0 / (double)temperature;
    const float hi = (float)it;
    return Scale{m, hi, (float)(it - (double)hi)};
}

// (v1, i1) beats (v2, i2): larger value, then smaller index; i < 0 = empty
__device__ __forceinline__ bool arg_better(float v1, int i1, float v2, int i2) {
    return i1 >= 0 && (i2 < 0 || v1 > v2 || (v1 == v2 && i1 < i2));
}


}  // namespace spec

// Defined in accept_greedy.hip, used by both accept entry points.
size_t spec_greedy_workspace_bytes(int batch, int n, int64_t vocab);
int spec_check_accept_args(int batch, int n, int s1, int64_t vocab, int dtype);
