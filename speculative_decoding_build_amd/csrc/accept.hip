// Tree accept: greedy (argmax matching) and classic rejection sampling.
//
// Greedy follows "SGLang 源码完全拆解(十一):投机解码" (三条判定路径: argmax per
// verify row, then the tree walk) and "投机解码 Accept:从 Verify 行到最终输出路径"
// (三: accept_index holds verify rows; the last row's target choice is the
// terminal token).  Sampling follows the same walk with the test of
// "Speculative Decoding" (sglang-internals, 接受/拒绝) and the residual of
// "投机解码 Accept" (四, Classic Rejection Sampling).
//
// Both are two launches:
//   1. a vocab sweep over every verify row, split into 8192-element chunks,
//      one 256-thread workgroup per (chunk, row): the chunk is loaded once
//      into registers (16-byte loads) and reduced to a partial (argmax, or
//      max + sum of exponentials for the target and draft rows);
//   2. a walk, one workgroup per request, that merges the chunk partials of
//      its rows and follows first-child / next-sibling links.  The sampled
//      walk runs its residual and inverse-CDF sweeps with the whole 1024-
//      thread workgroup.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "spec_common.h"

namespace {

constexpr int kSweepThreads = 256;
constexpr int kPerThread = 32;                       // elements per thread per row
constexpr int kChunk = kSweepThreads * kPerThread;   // 8192
constexpr int kWalkThreads = 1024;
constexpr int kMaxNodes = 64;

struct ArgPart {
    float v;
    int32_t i;
};

// target / draft row statistics of one chunk: max logit and sum of
// exp((x - max) / T) over the chunk
struct SamplePart {
    float mt, md;
    double st, sd;
};

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

// (v1, i1) beats (v2, i2): larger value, then smaller index; i < 0 = empty
__device__ __forceinline__ bool arg_better(float v1, int i1, float v2, int i2) {
    return i1 >= 0 && (i2 < 0 || v1 > v2 || (v1 == v2 && i1 < i2));
}

// ---- greedy: chunked argmax -----------------------------------------------

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void argmax_partial_kernel(
    const void *__restrict__ logits, int64_t vocab, int nchunks, bool vec_ok,
    ArgPart *__restrict__ part) {
    const int c = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t start = (int64_t)c * kChunk;
    const int64_t end = min(vocab, start + kChunk);
    const char *rowp = static_cast<const char *>(logits) + row * vocab * (DT == SPEC_BF16 ? 2 : 4);
    float x[kPerThread];
    load_chunk<DT>(rowp, start, end, vec_ok, tid, x);
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {       // e increases with element index
        const int64_t idx = elem_index(start, tid, e);
        if (idx < end && (bi < 0 || x[e] > bv)) {
            bv = x[e];
            bi = (int)idx;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, SPEC_WAVE);
        const int oi = __shfl_xor(bi, o, SPEC_WAVE);
        if (arg_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    __shared__ float s_v[kSweepThreads / SPEC_WAVE];
    __shared__ int s_i[kSweepThreads / SPEC_WAVE];
    if ((tid & 63) == 0) { s_v[tid >> 6] = bv; s_i[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kSweepThreads / SPEC_WAVE; ++w)
            if (arg_better(s_v[w], s_i[w], bv, bi)) { bv = s_v[w]; bi = s_i[w]; }
        part[row * nchunks + c] = ArgPart{bv, bi};
    }
}

// One wavefront per request: merge the chunk partials of the request's rows,
// then walk from the root.
__global__ __launch_bounds__(SPEC_WAVE) void greedy_walk_kernel(
    int n, int s1, int total_rows, int nchunks, const ArgPart *__restrict__ part,
    const int32_t *__restrict__ cand, const int32_t *__restrict__ r_index,
    const int32_t *__restrict__ r_next, const int32_t *__restrict__ r_sib,
    int32_t *__restrict__ predict, int32_t *__restrict__ accept_index,
    int32_t *__restrict__ accept_length, int32_t *__restrict__ target_predict,
    int32_t *__restrict__ status) {
    __shared__ int s_tp[kMaxNodes];
    __shared__ int s_row[kMaxNodes];
    __shared__ int s_pred[kMaxNodes];
    __shared__ int s_ai[kMaxNodes + 1];
    __shared__ int s_len;
    const int b = blockIdx.x;
    const int k = threadIdx.x;
    const int base = b * n;
    int err = 0;
    if (k < n) {
        int row = r_index[base + k];
        if (row < base || row >= base + n) { err |= SPEC_ST_RANGE; row = -1; }
        int bi = -1;
        float bv = -INFINITY;
        if (row >= 0)
            for (int c = 0; c < nchunks; ++c) {
                const ArgPart p = part[(int64_t)row * nchunks + c];
                if (arg_better(p.v, p.i, bv, bi)) { bv = p.v; bi = p.i; }
            }
        s_tp[k] = bi;
        s_row[k] = row;
        s_pred[k] = 0;
    }
    __syncthreads();
    if (k == 0) {
        int cur = 0, cnt = 0;
        s_ai[0] = s_row[0];
        for (int guard = 0; guard < n; ++guard) {
            const int want = s_tp[cur];
            int c = r_next[base + cur];
            int hit = -1;
            for (int steps = 0; c != -1 && steps < n; ++steps) {
                if (c < 0 || c >= n) { err |= SPEC_ST_RANGE; break; }
                if (cand[base + c] == want) { hit = c; break; }
                c = r_sib[base + c];
            }
            if (hit < 0) break;
            if (cnt + 1 >= s1) { err |= SPEC_ST_DEPTH; break; }
            s_pred[cur] = cand[base + hit];
            ++cnt;
            s_ai[cnt] = s_row[hit];
            cur = hit;
        }
        s_pred[cur] = s_tp[cur];
        s_len = cnt + 1;
    }
    __syncthreads();
    if (k < n && s_row[k] >= 0) {
        predict[s_row[k]] = s_pred[k];
        if (target_predict != nullptr) target_predict[s_row[k]] = s_tp[k];
    }
    for (int j = k; j < s1; j += SPEC_WAVE)
        accept_index[(int64_t)b * s1 + j] = (j < s_len) ? s_ai[j] : -1;
    if (k == 0) accept_length[b] = s_len;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, SPEC_WAVE);
    if (k == 0) spec::raise_status(status, err);
}

// ---- sampling: per-element probability --------------------------------------

// exp((x - m) / T) evaluated to about one float ulp: x - m as an exact
// float pair (two-sum), times 1/T carried as a float pair, the rounding of
// the scaled argument folded back as a first-order correction.
struct Scale {
    float m;      // row max (raw logit)
    float ithi;   // 1/T rounded to float
    float itlo;   // 1/T - ithi
};

__device__ __forceinline__ float exp_scaled(float x, const Scale &s) {
    const float d = x - s.m;
    const float bp = d - x;
    const float derr = (x - (d - bp)) + (-s.m - bp);     // x - m = d + derr exactly
    const float y = d * s.ithi;
    const float delta = fmaf(d, s.ithi, -y) + fmaf(d, s.itlo, derr * s.ithi);
    const float e = expf(y);
    return fmaf(e, delta, e);
}

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void sample_stats_kernel(
    const void *__restrict__ tlogits, const void *__restrict__ dlogits, int64_t vocab, int n,
    int nchunks, bool vec_ok, const float *__restrict__ temperature,
    SamplePart *__restrict__ part) {
    const int c = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t start = (int64_t)c * kChunk;
    const int64_t end = min(vocab, start + kChunk);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    float xt[kPerThread], xd[kPerThread];
    load_chunk<DT>(static_cast<const char *>(tlogits) + row * vocab * eb, start, end, vec_ok, tid, xt);
    load_chunk<DT>(static_cast<const char *>(dlogits) + row * vocab * eb, start, end, vec_ok, tid, xd);
    float mt = -INFINITY, md = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) { mt = fmaxf(mt, xt[e]); md = fmaxf(md, xd[e]); }
    mt = spec::wave_max(mt);
    md = spec::wave_max(md);
    __shared__ float s_m[2][kSweepThreads / SPEC_WAVE];
    __shared__ double s_s[2][kSweepThreads / SPEC_WAVE];
    if ((tid & 63) == 0) { s_m[0][tid >> 6] = mt; s_m[1][tid >> 6] = md; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) {
        mt = fmaxf(mt, s_m[0][w]);
        md = fmaxf(md, s_m[1][w]);
    }
    const double it = 1.0 / (double)temperature[row / n];
    Scale sct{mt, (float)it, (float)(it - (double)(float)it)};
    Scale scd{md, sct.ithi, sct.itlo};
    float st = 0.f, sd = 0.f;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        if (xt[e] != -INFINITY) st += exp_scaled(xt[e], sct);
        if (xd[e] != -INFINITY) sd += exp_scaled(xd[e], scd);
    }
    double dst = spec::wave_sum_d((double)st);
    double dsd = spec::wave_sum_d((double)sd);
    if ((tid & 63) == 0) { s_s[0][tid >> 6] = dst; s_s[1][tid >> 6] = dsd; }
    __syncthreads();
    if (tid == 0) {
        dst = 0.0;
        dsd = 0.0;
        for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) { dst += s_s[0][w]; dsd += s_s[1][w]; }
        part[row * nchunks + c] = SamplePart{mt, md, dst, dsd};
    }
}

// ---- sampling: the walk -------------------------------------------------------

struct RowDist {
    Scale t, d;          // per-row max and 1/T
    double inv_st, inv_sd;  // 1 / sum exp((x - max) / T)
};

template <int DT>
__device__ __forceinline__ float load_elem(const void *rowp, int64_t v) {
    if (DT == SPEC_BF16) return spec::bf16_to_f32(static_cast<const uint16_t *>(rowp)[v]);
    return static_cast<const float *>(rowp)[v];
}

// Residual after `nres` rejections at one node, at vocabulary entry v:
// R_0 = p, R_{i+1} = max(0, R_i - q) / Z_{i+1} (a level with Z = 0 keeps R).
__device__ __forceinline__ double residual(double p, double q, int nres, const double *inv_z) {
    double r = p;
    for (int i = 0; i < nres; ++i)
        if (inv_z[i] > 0.0) r = fmax(r - q, 0.0) * inv_z[i];
    return r;
}

__device__ double block_sum(double v, double *scratch) {
    v = spec::wave_sum_d(v);
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) scratch[tid >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < kWalkThreads / SPEC_WAVE; ++w) s += scratch[w];
    return s;
}

template <int DT>
__global__ __launch_bounds__(kWalkThreads) void sample_walk_kernel(
    int n, int s1, int64_t vocab, int nchunks, const SamplePart *__restrict__ part,
    const void *__restrict__ tlogits, const void *__restrict__ dlogits,
    const float *__restrict__ temperature, const float *__restrict__ uniforms,
    const float *__restrict__ final_uniforms, const int32_t *__restrict__ cand,
    const int32_t *__restrict__ r_index, const int32_t *__restrict__ r_next,
    const int32_t *__restrict__ r_sib, int32_t *__restrict__ predict,
    int32_t *__restrict__ accept_index, int32_t *__restrict__ accept_length,
    int32_t *__restrict__ status) {
    __shared__ RowDist s_dist[kMaxNodes];
    __shared__ int s_row[kMaxNodes];
    __shared__ int s_pred[kMaxNodes];
    __shared__ int s_ai[kMaxNodes + 1];
    __shared__ double s_inv_z[kMaxNodes];
    __shared__ double s_red[kWalkThreads / SPEC_WAVE];
    __shared__ double s_seg[kWalkThreads];
    __shared__ int s_cur, s_cnt, s_c, s_hit, s_nres, s_err, s_draw;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int base = b * n;
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const double it = 1.0 / (double)temperature[b];
    const float ithi = (float)it;
    const float itlo = (float)(it - (double)ithi);

    if (tid == 0) { s_err = 0; s_cur = 0; s_cnt = 0; }
    if (tid < n) {
        int row = r_index[base + tid];
        if (row < base || row >= base + n) row = -1;
        s_row[tid] = row;
        s_pred[tid] = 0;
        RowDist rd;
        float mt = -INFINITY, md = -INFINITY;
        if (row >= 0)
            for (int c = 0; c < nchunks; ++c) {
                const SamplePart p = part[(int64_t)row * nchunks + c];
                mt = fmaxf(mt, p.mt);
                md = fmaxf(md, p.md);
            }
        double st = 0.0, sd = 0.0;
        if (row >= 0)
            for (int c = 0; c < nchunks; ++c) {
                const SamplePart p = part[(int64_t)row * nchunks + c];
                st += p.st * exp(((double)p.mt - (double)mt) * it);
                sd += p.sd * exp(((double)p.md - (double)md) * it);
            }
        rd.t = Scale{mt, ithi, itlo};
        rd.d = Scale{md, ithi, itlo};
        rd.inv_st = st > 0.0 ? 1.0 / st : 0.0;
        rd.inv_sd = sd > 0.0 ? 1.0 / sd : 0.0;
        s_dist[tid] = rd;
    }
    __syncthreads();
    if (tid == 0) {
        for (int k = 0; k < n; ++k)
            if (s_row[k] < 0) s_err |= SPEC_ST_RANGE;
        s_ai[0] = s_row[0];
    }
    __syncthreads();

    // Node loop.  Every thread runs it; thread 0 takes each decision and
    // publishes it in shared memory; all threads copy it to registers between
    // two barriers before thread 0 may write again, so control flow stays
    // uniform across the workgroup.
    int cur = 0;
    int nres = 0;
    for (int level = 0; level < n; ++level) {
        if (tid == 0) {
            s_nres = 0;
            s_hit = -1;
            s_c = r_next[base + s_cur];
        }
        __syncthreads();
        cur = s_cur;
        nres = 0;
        const int row = s_row[cur];
        __syncthreads();
        if (row < 0) break;
        const void *trow = static_cast<const char *>(tlogits) + (int64_t)row * vocab * eb;
        const void *drow = static_cast<const char *>(dlogits) + (int64_t)row * vocab * eb;
        const RowDist rd = s_dist[cur];
        int hit = -1;
        for (int steps = 0; steps < n; ++steps) {
            if (tid == 0) {
                const int c = s_c;
                if (c < 0 || c >= n) {
                    if (c != -1) s_err |= SPEC_ST_RANGE;
                    s_c = -1;
                } else {
                    const int t = cand[base + c];
                    double ratio = 0.0;
                    if (t >= 0 && t < vocab) {
                        const double p = (double)exp_scaled(load_elem<DT>(trow, t), rd.t) * rd.inv_st;
                        const double q = (double)exp_scaled(load_elem<DT>(drow, t), rd.d) * rd.inv_sd;
                        const double r = residual(p, q, s_nres, s_inv_z);
                        ratio = q > 0.0 ? r / q : (r > 0.0 ? INFINITY : 0.0);
                    } else {
                        s_err |= SPEC_ST_RANGE;
                    }
                    const double u = (double)uniforms[base + c];
                    if (u < fmin(1.0, ratio)) s_hit = c;
                }
            }
            __syncthreads();
            const int c_now = s_c;
            hit = s_hit;
            __syncthreads();
            if (c_now == -1 || hit >= 0) break;
            // rejected: Z = sum_v max(0, R(v) - q(v))
            double z = 0.0;
            for (int64_t v = tid; v < vocab; v += kWalkThreads) {
                const double p = (double)exp_scaled(load_elem<DT>(trow, v), rd.t) * rd.inv_st;
                const double q = (double)exp_scaled(load_elem<DT>(drow, v), rd.d) * rd.inv_sd;
                z += fmax(residual(p, q, nres, s_inv_z) - q, 0.0);
            }
            z = block_sum(z, s_red);
            if (tid == 0) {
                if (z > 0.0) {
                    s_inv_z[nres] = 1.0 / z;
                } else {
                    s_inv_z[nres] = 0.0;
                    s_err |= SPEC_ST_ZERO_RESIDUAL;
                }
                s_nres = nres + 1;
                s_c = r_sib[base + c_now];
            }
            ++nres;
            __syncthreads();
        }
        if (hit < 0) break;
        int moved = 0;
        if (tid == 0) {
            if (s_cnt + 1 >= s1) {
                s_err |= SPEC_ST_DEPTH;
            } else {
                s_pred[cur] = cand[base + hit];
                s_cnt = s_cnt + 1;
                s_ai[s_cnt] = s_row[hit];
                s_cur = hit;
                moved = 1;
            }
            s_hit = moved;
        }
        __syncthreads();
        moved = s_hit;
        __syncthreads();
        if (!moved) break;
    }
    __syncthreads();

    // terminal draw: inverse CDF of the current residual in vocabulary order
    // (cur and nres are the node and residual level the walk stopped at)
    const int row = s_row[cur];
    if (row >= 0) {
        const void *trow = static_cast<const char *>(tlogits) + (int64_t)row * vocab * eb;
        const void *drow = static_cast<const char *>(dlogits) + (int64_t)row * vocab * eb;
        const RowDist rd = s_dist[cur];
        // thread t owns the contiguous segment [t*seg, (t+1)*seg)
        const int64_t seg = (vocab + kWalkThreads - 1) / kWalkThreads;
        const int64_t v0 = min(vocab, (int64_t)tid * seg);
        const int64_t v1 = min(vocab, v0 + seg);
        double mine = 0.0;
        for (int64_t v = v0; v < v1; ++v) {
            const double p = (double)exp_scaled(load_elem<DT>(trow, v), rd.t) * rd.inv_st;
            const double q = (double)exp_scaled(load_elem<DT>(drow, v), rd.d) * rd.inv_sd;
            mine += residual(p, q, nres, s_inv_z);
        }
        s_seg[tid] = mine;
        if (tid == 0) s_draw = INT_MAX;
        __syncthreads();
        // exclusive prefix over segments (sequential in thread order, by wave 0)
        if (tid < SPEC_WAVE) {
            // each lane sums 16 consecutive segments, then a lane scan
            double part16 = 0.0;
            for (int i = 0; i < kWalkThreads / SPEC_WAVE; ++i)
                part16 += s_seg[tid * (kWalkThreads / SPEC_WAVE) + i];
            double incl = part16;
            for (int o = 1; o < SPEC_WAVE; o <<= 1) {
                const double x = __shfl_up(incl, o, SPEC_WAVE);
                if (tid >= o) incl += x;
            }
            double run = incl - part16;
            const double total = __shfl(incl, SPEC_WAVE - 1, SPEC_WAVE);
            for (int i = 0; i < kWalkThreads / SPEC_WAVE; ++i) {
                const int t = tid * (kWalkThreads / SPEC_WAVE) + i;
                const double s = s_seg[t];
                s_seg[t] = run;
                run += s;
            }
            if (tid == 0) s_red[0] = total;
        }
        __syncthreads();
        const double total = s_red[0];
        const double target = (double)final_uniforms[b] * total;
        const double before = s_seg[tid];
        if (v0 < v1 && before <= target && target < before + mine) {
            double run = before;
            int found = -1;
            for (int64_t v = v0; v < v1; ++v) {
                const double p = (double)exp_scaled(load_elem<DT>(trow, v), rd.t) * rd.inv_st;
                const double q = (double)exp_scaled(load_elem<DT>(drow, v), rd.d) * rd.inv_sd;
                run += residual(p, q, nres, s_inv_z);
                if (run > target) { found = (int)v; break; }
            }
            if (found >= 0) atomicMin(&s_draw, found);
        }
        __syncthreads();
        if (tid == 0) {
            const int x = (s_draw == INT_MAX) ? (int)(vocab - 1) : s_draw;
            s_pred[cur] = x;
        }
    }
    __syncthreads();
    if (tid < n && s_row[tid] >= 0) predict[s_row[tid]] = s_pred[tid];
    for (int j = tid; j < s1; j += kWalkThreads)
        accept_index[(int64_t)b * s1 + j] = (j <= s_cnt) ? s_ai[j] : -1;
    if (tid == 0) {
        accept_length[b] = s_cnt + 1;
        spec::raise_status(status, s_err);
    }
}

inline int num_chunks(int64_t vocab) { return (int)((vocab + kChunk - 1) / kChunk); }

}  // namespace

extern "C" size_t spec_accept_workspace_size(int batch, int n, int64_t vocab, int sampled) {
    if (batch <= 0 || n <= 0 || vocab <= 0) return 0;
    const size_t rows = (size_t)batch * n;
    const size_t per = sampled ? sizeof(SamplePart) : sizeof(ArgPart);
    return spec::align_up(rows * num_chunks(vocab) * per, 256);
}

static int check_accept_args(int batch, int n, int s1, int64_t vocab, int dtype) {
    if (batch < 0 || n < 1 || s1 < 1 || vocab < 1) return SPEC_ERR_SHAPE;
    if (n > kMaxNodes || s1 > kMaxNodes + 1) return SPEC_ERR_UNSUPPORTED;
    if (vocab > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    if ((int64_t)batch * n * vocab / vocab != (int64_t)batch * n) return SPEC_ERR_SHAPE;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    return SPEC_OK;
}

extern "C" int spec_accept_greedy(int batch, int n, int s1, int64_t vocab, int dtype,
                                  const void *target_logits, const int32_t *candidates,
                                  const int32_t *retrieve_index,
                                  const int32_t *retrieve_next_token,
                                  const int32_t *retrieve_next_sibling, int32_t *predict,
                                  int32_t *accept_index, int32_t *accept_length,
                                  int32_t *target_predict, void *workspace,
                                  size_t workspace_bytes, int32_t *dev_status,
                                  spec_stream_t stream) {
    int rc = check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (batch == 0) return SPEC_OK;
    if (!target_logits || !candidates || !retrieve_index || !retrieve_next_token ||
        !retrieve_next_sibling || !predict || !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_accept_workspace_size(batch, n, vocab, 0))
        return SPEC_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int nch = num_chunks(vocab);
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0;
    ArgPart *part = static_cast<ArgPart *>(workspace);
    const dim3 grid(nch, batch * n);
    if (dtype == SPEC_BF16)
        hipLaunchKernelGGL(argmax_partial_kernel<SPEC_BF16>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, vocab, nch, vec_ok, part);
    else
        hipLaunchKernelGGL(argmax_partial_kernel<SPEC_F32>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, vocab, nch, vec_ok, part);
    hipLaunchKernelGGL(greedy_walk_kernel, dim3(batch), dim3(SPEC_WAVE), 0, st, n, s1,
                       batch * n, nch, part, candidates, retrieve_index, retrieve_next_token,
                       retrieve_next_sibling, predict, accept_index, accept_length,
                       target_predict, dev_status);
    return spec::launch_status();
}

extern "C" int spec_accept_sample(int batch, int n, int s1, int64_t vocab, int dtype,
                                  const void *target_logits, const void *draft_logits,
                                  const float *temperature, const float *uniforms,
                                  const float *final_uniforms, const int32_t *candidates,
                                  const int32_t *retrieve_index,
                                  const int32_t *retrieve_next_token,
                                  const int32_t *retrieve_next_sibling, int32_t *predict,
                                  int32_t *accept_index, int32_t *accept_length,
                                  void *workspace, size_t workspace_bytes,
                                  int32_t *dev_status, spec_stream_t stream) {
    int rc = check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (batch == 0) return SPEC_OK;
    if (!target_logits || !draft_logits || !temperature || !uniforms || !final_uniforms ||
        !candidates || !retrieve_index || !retrieve_next_token || !retrieve_next_sibling ||
        !predict || !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_accept_workspace_size(batch, n, vocab, 1))
        return SPEC_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int nch = num_chunks(vocab);
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0;
    SamplePart *part = static_cast<SamplePart *>(workspace);
    const dim3 grid(nch, batch * n);
    if (dtype == SPEC_BF16) {
        hipLaunchKernelGGL(sample_stats_kernel<SPEC_BF16>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, draft_logits, vocab, n, nch, vec_ok, temperature, part);
        hipLaunchKernelGGL(sample_walk_kernel<SPEC_BF16>, dim3(batch), dim3(kWalkThreads), 0, st,
                           n, s1, vocab, nch, part, target_logits, draft_logits, temperature,
                           uniforms, final_uniforms, candidates, retrieve_index,
                           retrieve_next_token, retrieve_next_sibling, predict, accept_index,
                           accept_length, dev_status);
    } else {
        hipLaunchKernelGGL(sample_stats_kernel<SPEC_F32>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, draft_logits, vocab, n, nch, vec_ok, temperature, part);
        hipLaunchKernelGGL(sample_walk_kernel<SPEC_F32>, dim3(batch), dim3(kWalkThreads), 0, st,
                           n, s1, vocab, nch, part, target_logits, draft_logits, temperature,
                           uniforms, final_uniforms, candidates, retrieve_index,
                           retrieve_next_token, retrieve_next_sibling, predict, accept_index,
                           accept_length, dev_status);
    }
    return spec::launch_status();
}
