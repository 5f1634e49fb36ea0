// Rejection-sampled tree accept.
//
// The test is the classic one of "Speculative Decoding" (sglang-internals,
// 接受/拒绝) and "投机解码 Accept:从 Verify 行到最终输出路径" (四, Classic Rejection
// Sampling): child c with token t passes iff u < min(1, R(t) / q(t)); each
// rejection replaces the residual R by max(0, R - q) renormalised; without
// an accepted child the terminal token is drawn from R.  The walk over
// first-child / next-sibling links is the greedy one ("把投机采样讲透", 5.6).
//
// Closed form of the residual.  With p, q the target / draft distributions
// of the current node's row and F(c) = sum_v max(0, p_v - c q_v), the
// residual after j rejections (all of them against the same q) is
//     R_j = max(0, p - c_j q) / F(c_j),   c_1 = 1, c_{j+1} = c_j + F(c_j),
// which follows by induction from R_{j+1} = max(0, R_j - q) / Z_{j+1}
// (Z_{j+1} = F(c_{j+1}) / F(c_j)).  Starting from (c, F) = (0, 1) (R_0 = p)
// a rejection is (c, F) <- (c + F, F(c + F)): one reduction over the
// vocabulary, independent of how many rejections came before.  A level with
// F = 0 leaves R unchanged, as the recursive form does.
//
// Launches
//   1. statistics sweep over every verify row (target and draft): max logit
//      and sum of exp((x - max) / T) per 8192-entry chunk, one 256-thread
//      workgroup per (chunk, row), each chunk read once;
//   2. the walk.  Preferred: a cooperative launch with G workgroups per
//      request, each owning a slice of the vocabulary; the F(c) reductions and
//      the inverse-CDF draw are split across the G slices and combined
//      through a per-request barrier in global memory.  Every workgroup of a
//      request replays the same decisions from the same data, so only the
//      slice partial sums travel.  When the grid cannot be co-resident the
//      walk falls back to one 1024-thread workgroup per request.
//
// Per-entry probabilities are float32 exponentials of the exactly formed
// argument (x - max) / T, normalised and accumulated in float64.
#include <algorithm>

#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kSoloThreads = 1024;
constexpr int kCoopThreads = 256;
constexpr unsigned kSpinLimit = 1u << 20;       // about a second of waiting
constexpr int kCoopGridTarget = 512;           // workgroups of a cooperative walk, all requests

struct SamplePart {
    float mt, md;
    double st, sd;
};

// per-request barrier words, one cache line each
struct alignas(64) GroupSync {
    unsigned count;
    unsigned gen;
    unsigned pad[14];
};

// exp((x - m) / T) to about one float ulp: x - m as an exact float pair
// (two-sum), 1/T as a float pair, the rounding of the product folded back
// as a first-order correction.
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
    return fmaf(e, delta, e);
}

struct RowDist {
    Scale t, d;
    double inv_st, inv_sd;
};

template <int DT>
__device__ __forceinline__ float load_elem(const void *rowp, int64_t v) {
    if (DT == SPEC_BF16) return bf16_to_f32(static_cast<const uint16_t *>(rowp)[v]);
    return static_cast<const float *>(rowp)[v];
}

// weight of entry v in the residual state (c, F), without the 1/F factor
__device__ __forceinline__ double resid_weight(float xt, float xd, const RowDist &rd, double c) {
    const double p = (double)exp_scaled(xt, rd.t) * rd.inv_st;
    const double q = (double)exp_scaled(xd, rd.d) * rd.inv_sd;
    return fmax(fma(-c, q, p), 0.0);
}

// Sum of resid_weight over [a, b) in ascending order; 16-byte loads when the
// rows allow them (a is a multiple of 8 then).
template <int DT>
__device__ double range_sum(const void *trow, const void *drow, int64_t a, int64_t b,
                            bool vec_ok, const RowDist &rd, double c) {
    double s = 0.0;
    int64_t v = a;
    if (DT == SPEC_BF16 && vec_ok) {
        for (; v + 8 <= b; v += 8) {
            const uint4 wt = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(trow) + v);
            const uint4 wd = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(drow) + v);
            const uint32_t at[4] = {wt.x, wt.y, wt.z, wt.w};
            const uint32_t ad[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s += resid_weight(lo_bf16(at[j]), lo_bf16(ad[j]), rd, c);
                s += resid_weight(hi_bf16(at[j]), hi_bf16(ad[j]), rd, c);
            }
        }
    }
    for (; v < b; ++v) s += resid_weight(load_elem<DT>(trow, v), load_elem<DT>(drow, v), rd, c);
    return s;
}

// First entry of [a, b) where the running sum, started at `run`, exceeds
// `target`; -1 if none.  Same order of accumulation as range_sum.
template <int DT>
__device__ int64_t range_find(const void *trow, const void *drow, int64_t a, int64_t b,
                              const RowDist &rd, double c, double run, double target) {
    for (int64_t v = a; v < b; ++v) {
        run += resid_weight(load_elem<DT>(trow, v), load_elem<DT>(drow, v), rd, c);
        if (run > target) return v;
    }
    return -1;
}

template <int NT>
__device__ double block_sum(double v, double *scratch) {
    v = wave_sum_d(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += scratch[w];
    return s;
}

// Exclusive prefix of v over threads in thread order; also returns the total.
template <int NT>
__device__ double block_exclusive_scan(double v, double *scratch, double &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    double before = 0.0;
    total = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) before += scratch[w];
        total += scratch[w];
    }
    return before + incl - v;
}

// ---------------------------------------------------------------------------
// 1. statistics sweep
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void sample_stats_kernel(
    const void *__restrict__ tlogits, const void *__restrict__ dlogits, int64_t vocab, int n,
    int batch, int nchunks, bool vec_ok, const float *__restrict__ temperature,
    SamplePart *__restrict__ part, GroupSync *__restrict__ sync) {
    const int c = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    if (sync != nullptr && c == 0 && row == 0)
        for (int r = tid; r < batch; r += kSweepThreads) { sync[r].count = 0; sync[r].gen = 0; }
    const int64_t start = (int64_t)c * kChunk;
    const int64_t end = min(vocab, start + kChunk);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    float xt[kPerThread], xd[kPerThread];
    load_chunk<DT>(static_cast<const char *>(tlogits) + row * vocab * eb, start, end, vec_ok, tid, xt);
    load_chunk<DT>(static_cast<const char *>(dlogits) + row * vocab * eb, start, end, vec_ok, tid, xd);
    float mt = -INFINITY, md = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) { mt = fmaxf(mt, xt[e]); md = fmaxf(md, xd[e]); }
    mt = wave_max(mt);
    md = wave_max(md);
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
    const Scale sct{mt, (float)it, (float)(it - (double)(float)it)};
    const Scale scd{md, sct.ithi, sct.itlo};
    float st = 0.f, sd = 0.f;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        if (xt[e] != -INFINITY) st += exp_scaled(xt[e], sct);
        if (xd[e] != -INFINITY) sd += exp_scaled(xd[e], scd);
    }
    double dst = wave_sum_d((double)st);
    double dsd = wave_sum_d((double)sd);
    if ((tid & 63) == 0) { s_s[0][tid >> 6] = dst; s_s[1][tid >> 6] = dsd; }
    __syncthreads();
    if (tid == 0) {
        dst = 0.0;
        dsd = 0.0;
        for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) { dst += s_s[0][w]; dsd += s_s[1][w]; }
        part[row * nchunks + c] = SamplePart{mt, md, dst, dsd};
    }
}

// ---------------------------------------------------------------------------
// walk state shared by both walk kernels
// ---------------------------------------------------------------------------

struct WalkArgs {
    int n, s1, nchunks;
    int64_t vocab;
    bool vec_ok;
    const SamplePart *part;
    const void *tlogits, *dlogits;
    const float *temperature, *uniforms, *final_uniforms;
    const int32_t *cand, *r_index, *r_next, *r_sib;
    int32_t *predict, *accept_index, *accept_length, *status;
    // cooperative walk only
    int G;              // workgroups per request
    int64_t slice;      // vocabulary entries per workgroup (multiple of 8 * threads)
    GroupSync *sync;    // [batch]
    double *red;        // [batch][2][G]
};

struct WalkShared {
    RowDist dist;
    float cxt[kMaxNodes];      // target / draft logit of each child token of the current node
    float cxd[kMaxNodes];
    int clist[kMaxNodes];      // children of the current node in sibling order
    int nkids;
    int cand[kMaxNodes];
    int next[kMaxNodes];
    int sib[kMaxNodes];
    float unif[kMaxNodes];
    int row[kMaxNodes];
    int pred[kMaxNodes];
    int ai[kMaxNodes + 1];
    double scratch[16];
    double bcast;
    int cur, cnt, err, dec, child, draw, flag;
};

// Thread 0 decides the test of the i-th child of the current node (its
// token's logits were prefetched) and publishes the outcome.
__device__ void decide_child(const WalkShared &Sc, WalkShared &S, int i, int64_t vocab,
                             double c, double F) {
    int dec = 0;
    const int child = Sc.clist[i];
    const int t = Sc.cand[child];
    if (t >= 0 && t < vocab) {
        const RowDist &rd = Sc.dist;
        const double p = (double)exp_scaled(Sc.cxt[i], rd.t) * rd.inv_st;
        const double q = (double)exp_scaled(Sc.cxd[i], rd.d) * rd.inv_sd;
        const double r = fmax(fma(-c, q, p), 0.0) / F;
        const double ratio = q > 0.0 ? r / q : (r > 0.0 ? INFINITY : 0.0);
        dec = (double)Sc.unif[child] < fmin(1.0, ratio);
    } else {
        S.err |= SPEC_ST_RANGE;
    }
    S.dec = dec;
}

// Node entry, all threads: merge the row's chunk statistics (wave 0, one
// lane per chunk), list the children in sibling order and fetch their
// tokens' target / draft logits (one thread per child).
template <int DT>
__device__ void enter_node(const WalkArgs &A, WalkShared &S, int cur, int row, double it,
                           const void *trow, const void *drow) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        float mt = -INFINITY, md = -INFINITY;
        for (int c = tid; c < A.nchunks; c += 64) {
            const SamplePart p = A.part[(int64_t)row * A.nchunks + c];
            mt = fmaxf(mt, p.mt);
            md = fmaxf(md, p.md);
        }
        mt = wave_max(mt);
        md = wave_max(md);
        double st = 0.0, sd = 0.0;
        for (int c = tid; c < A.nchunks; c += 64) {
            const SamplePart p = A.part[(int64_t)row * A.nchunks + c];
            st += p.st * exp(((double)p.mt - (double)mt) * it);
            sd += p.sd * exp(((double)p.md - (double)md) * it);
        }
        st = wave_sum_d(st);
        sd = wave_sum_d(sd);
        if (tid == 0) {
            const float ithi = (float)it;
            const float itlo = (float)(it - (double)ithi);
            S.dist.t = Scale{mt, ithi, itlo};
            S.dist.d = Scale{md, ithi, itlo};
            S.dist.inv_st = st > 0.0 ? 1.0 / st : 0.0;
            S.dist.inv_sd = sd > 0.0 ? 1.0 / sd : 0.0;
            int k = 0;
            int c = S.next[cur];
            for (int steps = 0; steps < A.n && c != -1; ++steps) {
                if (c < 0 || c >= A.n) { S.err |= SPEC_ST_RANGE; break; }
                S.clist[k++] = c;
                c = S.sib[c];
            }
            S.nkids = k;
        }
    }
    __syncthreads();
    if (tid < S.nkids) {
        const int t = S.cand[S.clist[tid]];
        const bool ok = t >= 0 && t < A.vocab;
        S.cxt[tid] = ok ? load_elem<DT>(trow, t) : 0.f;
        S.cxd[tid] = ok ? load_elem<DT>(drow, t) : 0.f;
    }
    __syncthreads();
}

// Per-request barrier among the G workgroups of a cooperative launch.  The
// launch guarantees co-residency; the wait is still bounded, and a timeout
// is reported instead of hanging.  Returns false after a timeout.
__device__ bool group_barrier(GroupSync *gs, unsigned G, unsigned &epoch, WalkShared &S) {
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        __threadfence();
        const unsigned old = __hip_atomic_fetch_add(&gs->count, 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == G - 1) {
            __hip_atomic_store(&gs->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&gs->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // poll with relaxed loads and exponential back-off (polls go to the
            // memory side; hundreds of spinning workgroups would congest it)
            unsigned spins = 0, nap = 1;
            while (__hip_atomic_load(&gs->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
                for (unsigned z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(4);
                nap = nap < 16 ? nap * 2 : 16;
                if (++spins > kSpinLimit) { ok = 0; break; }
            }
        }
        __threadfence();
        epoch += 1;
        S.flag = ok;
    }
    __syncthreads();
    return S.flag != 0;
}

// ---------------------------------------------------------------------------
// 2a. cooperative walk: G workgroups per request
// ---------------------------------------------------------------------------

// Sum over the G slice partials of round `parity` (thread j < G loads entry
// j); the reduction order is fixed, so every workgroup of the request gets
// the bitwise same value.
__device__ double group_total(const double *red, int G, WalkShared &S) {
    double v = 0.0;
    if ((int)threadIdx.x < G)
        v = __hip_atomic_load(&red[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return block_sum<kCoopThreads>(v, S.scratch);
}

template <int DT>
__global__ __launch_bounds__(kCoopThreads) void sample_walk_coop_kernel(WalkArgs A) {
    __shared__ WalkShared S;
    const int G = A.G;
    const int req = blockIdx.x / G;
    const int g = blockIdx.x % G;
    const int tid = threadIdx.x;
    const int n = A.n;
    const int base = req * n;
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const double it = 1.0 / (double)A.temperature[req];
    GroupSync *gs = A.sync + req;
    double *red = A.red + (int64_t)req * 2 * G;
    unsigned epoch = 0;
    int parity = 0;
    bool alive = true;

    // my slice of the vocabulary and, inside it, my contiguous segment
    const int64_t v0 = min(A.vocab, (int64_t)g * A.slice);
    const int64_t v1 = min(A.vocab, v0 + A.slice);
    const int64_t seg = A.slice / kCoopThreads;
    const int64_t sa = min(v1, v0 + tid * seg);
    const int64_t sb = min(v1, sa + seg);

    if (tid < n) {
        int row = A.r_index[base + tid];
        if (row < base || row >= base + n) row = -1;
        S.row[tid] = row;
        S.pred[tid] = 0;
        S.cand[tid] = A.cand[base + tid];
        S.next[tid] = A.r_next[base + tid];
        S.sib[tid] = A.r_sib[base + tid];
        S.unif[tid] = A.uniforms[base + tid];
    }
    if (tid == 0) { S.cur = 0; S.cnt = 0; S.err = 0; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 0; k < n; ++k)
            if (S.row[k] < 0) S.err |= SPEC_ST_RANGE;
        S.ai[0] = S.row[0];
    }
    double c = 0.0, F = 1.0;
    int cur = 0;
    for (int level = 0; level < n && alive; ++level) {
        __syncthreads();
        cur = S.cur;
        const int row = S.row[cur];
        if (row < 0) break;
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)row * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)row * A.vocab * eb;
        enter_node<DT>(A, S, cur, row, it, trow, drow);
        const RowDist rd = S.dist;
        const int nk = S.nkids;
        c = 0.0;
        F = 1.0;
        int hit = -1;
        for (int i = 0; i < nk; ++i) {
            if (tid == 0) decide_child(S, S, i, A.vocab, c, F);
            __syncthreads();
            const int dec = S.dec;
            __syncthreads();
            if (dec) { hit = S.clist[i]; break; }
            // rejected: F(c + F) over the vocabulary, split across the group
            const double cn = c + F;
            const double mine = range_sum<DT>(trow, drow, sa, sb, A.vec_ok, rd, cn);
            const double slice_sum = block_sum<kCoopThreads>(mine, S.scratch);
            if (tid == 0)
                __hip_atomic_store(&red[parity * G + g], slice_sum, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (!group_barrier(gs, G, epoch, S)) { alive = false; break; }
            const double Fn = group_total(red + parity * G, G, S);
            parity ^= 1;
            if (Fn > 0.0) {
                c = cn;
                F = Fn;
            } else if (tid == 0) {
                S.err |= SPEC_ST_ZERO_RESIDUAL;
            }
        }
        if (!alive || hit < 0) break;
        if (tid == 0) {
            if (S.cnt + 1 >= A.s1) {
                S.err |= SPEC_ST_DEPTH;
                S.dec = 0;
            } else {
                S.pred[cur] = S.cand[hit];
                S.cnt = S.cnt + 1;
                S.ai[S.cnt] = S.row[hit];
                S.cur = hit;
                S.dec = 1;
            }
        }
        __syncthreads();
        const int moved = S.dec;
        __syncthreads();
        if (!moved) break;
    }

    // terminal draw: inverse CDF of max(0, p - c q) in vocabulary order
    const int row = S.row[cur];
    if (alive && row >= 0) {
        const RowDist rd = S.dist;
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)row * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)row * A.vocab * eb;
        const double mine = range_sum<DT>(trow, drow, sa, sb, A.vec_ok, rd, c);
        double slice_total;
        const double before = block_exclusive_scan<kCoopThreads>(mine, S.scratch, slice_total);
        if (tid == 0)
            __hip_atomic_store(&red[parity * G + g], slice_total, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (group_barrier(gs, G, epoch, S)) {
            // slice sums in slice order -> owner of the crossing, my slice's offset
            double sj = 0.0;
            if (tid < G)
                sj = __hip_atomic_load(&red[parity * G + tid], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            double total;
            const double pre = block_exclusive_scan<kCoopThreads>(sj, S.scratch, total);
            const double target = (double)A.final_uniforms[req] * total;
            if (tid == 0) { S.dec = G - 1; S.draw = INT_MAX; }
            __syncthreads();
            if (tid < G && sj > 0.0 && pre <= target && target < pre + sj) atomicMin(&S.dec, tid);
            if (tid == g) S.bcast = target - pre;          // target measured from my slice
            __syncthreads();
            if (S.dec == g) {
                const double tgt = S.bcast;
                if (sa < sb && before <= tgt && tgt < before + mine) {
                    const int64_t x = range_find<DT>(trow, drow, sa, sb, rd, c, before, tgt);
                    if (x >= 0) atomicMin(&S.draw, (int)x);
                }
                __syncthreads();
                if (tid == 0) {
                    // no crossing inside the slice (rounding, or a target at the
                    // very end of the mass): its last entry
                    int x = S.draw;
                    if (x == INT_MAX) x = (int)(v1 > v0 ? v1 - 1 : A.vocab - 1);
                    A.predict[row] = x;
                }
            }
        } else {
            alive = false;
        }
    }

    if (!alive && tid == 0) S.err |= SPEC_ST_SYNC;
    __syncthreads();
    if (g == 0) {
        const int terminal = (alive && row >= 0) ? cur : -1;
        if (tid < n && S.row[tid] >= 0 && tid != terminal) A.predict[S.row[tid]] = S.pred[tid];
        for (int j = tid; j < A.s1; j += kCoopThreads)
            A.accept_index[(int64_t)req * A.s1 + j] = (j <= S.cnt) ? S.ai[j] : -1;
        if (tid == 0) A.accept_length[req] = S.cnt + 1;
    }
    if (tid == 0) raise_status(A.status, S.err);
}

// ---------------------------------------------------------------------------
// 2b. one workgroup per request (fallback)
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(kSoloThreads) void sample_walk_solo_kernel(WalkArgs A) {
    __shared__ WalkShared S;
    const int req = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = A.n;
    const int base = req * n;
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const double it = 1.0 / (double)A.temperature[req];
    // contiguous segment per thread, a multiple of 8 entries
    const int64_t seg = ((A.vocab + kSoloThreads - 1) / kSoloThreads + 7) / 8 * 8;
    const int64_t sa = min(A.vocab, (int64_t)tid * seg);
    const int64_t sb = min(A.vocab, sa + seg);

    if (tid < n) {
        int row = A.r_index[base + tid];
        if (row < base || row >= base + n) row = -1;
        S.row[tid] = row;
        S.pred[tid] = 0;
        S.cand[tid] = A.cand[base + tid];
        S.next[tid] = A.r_next[base + tid];
        S.sib[tid] = A.r_sib[base + tid];
        S.unif[tid] = A.uniforms[base + tid];
    }
    if (tid == 0) { S.cur = 0; S.cnt = 0; S.err = 0; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 0; k < n; ++k)
            if (S.row[k] < 0) S.err |= SPEC_ST_RANGE;
        S.ai[0] = S.row[0];
    }
    double c = 0.0, F = 1.0;
    int cur = 0;
    for (int level = 0; level < n; ++level) {
        __syncthreads();
        cur = S.cur;
        const int row = S.row[cur];
        if (row < 0) break;
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)row * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)row * A.vocab * eb;
        enter_node<DT>(A, S, cur, row, it, trow, drow);
        const RowDist rd = S.dist;
        const int nk = S.nkids;
        c = 0.0;
        F = 1.0;
        int hit = -1;
        for (int i = 0; i < nk; ++i) {
            if (tid == 0) decide_child(S, S, i, A.vocab, c, F);
            __syncthreads();
            const int dec = S.dec;
            __syncthreads();
            if (dec) { hit = S.clist[i]; break; }
            const double cn = c + F;
            const double Fn = block_sum<kSoloThreads>(
                range_sum<DT>(trow, drow, sa, sb, A.vec_ok, rd, cn), S.scratch);
            if (Fn > 0.0) {
                c = cn;
                F = Fn;
            } else if (tid == 0) {
                S.err |= SPEC_ST_ZERO_RESIDUAL;
            }
        }
        if (hit < 0) break;
        if (tid == 0) {
            if (S.cnt + 1 >= A.s1) {
                S.err |= SPEC_ST_DEPTH;
                S.dec = 0;
            } else {
                S.pred[cur] = S.cand[hit];
                S.cnt = S.cnt + 1;
                S.ai[S.cnt] = S.row[hit];
                S.cur = hit;
                S.dec = 1;
            }
        }
        __syncthreads();
        const int moved = S.dec;
        __syncthreads();
        if (!moved) break;
    }

    const int row = S.row[cur];
    if (row >= 0) {
        const RowDist rd = S.dist;
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)row * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)row * A.vocab * eb;
        const double mine = range_sum<DT>(trow, drow, sa, sb, A.vec_ok, rd, c);
        double total;
        const double before = block_exclusive_scan<kSoloThreads>(mine, S.scratch, total);
        const double target = (double)A.final_uniforms[req] * total;
        if (tid == 0) S.draw = INT_MAX;
        __syncthreads();
        if (sa < sb && before <= target && target < before + mine) {
            const int64_t x = range_find<DT>(trow, drow, sa, sb, rd, c, before, target);
            if (x >= 0) atomicMin(&S.draw, (int)x);
        }
        __syncthreads();
        if (tid == 0) S.pred[cur] = (S.draw == INT_MAX) ? (int)(A.vocab - 1) : S.draw;
    }
    __syncthreads();
    if (tid < n && S.row[tid] >= 0) A.predict[S.row[tid]] = S.pred[tid];
    for (int j = tid; j < A.s1; j += kSoloThreads)
        A.accept_index[(int64_t)req * A.s1 + j] = (j <= S.cnt) ? S.ai[j] : -1;
    if (tid == 0) {
        A.accept_length[req] = S.cnt + 1;
        raise_status(A.status, S.err);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct CoopPlan {
    int G;
    int64_t slice;
};

// Workgroups per request for the cooperative walk, or G = 0 when the grid
// cannot be co-resident (or cooperative launch is unavailable).
template <int DT>
CoopPlan coop_plan(int batch, int64_t vocab) {
    static int cached_device = -1, cap = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CoopPlan{0, 0};
    if (dev != cached_device) {
        int coop = 0, cus = 0, per = 0;
        bool ok = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess;
        ok = ok && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
        ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &per, reinterpret_cast<const void *>(sample_walk_coop_kernel<DT>),
                       kCoopThreads, 0) == hipSuccess;
        cap = (ok && coop) ? cus * per : 0;
        cached_device = dev;
    }
    const int64_t min_slice = (int64_t)kCoopThreads * 8;
    int64_t G = (vocab + min_slice - 1) / min_slice;
    G = std::min<int64_t>(G, cap / std::max(batch, 1));
    G = std::min<int64_t>(G, std::max(2, kCoopGridTarget / std::max(batch, 1)));
    G = std::min<int64_t>(G, kCoopThreads);      // one partial per thread of a workgroup
    if (G < 2) return CoopPlan{0, 0};
    int64_t slice = (vocab + G - 1) / G;
    slice = (slice + min_slice - 1) / min_slice * min_slice;
    G = (vocab + slice - 1) / slice;
    return CoopPlan{(int)G, slice};
}

size_t sample_workspace_layout(int batch, int n, int64_t vocab, size_t *off_sync, size_t *off_red) {
    const size_t parts = spec::align_up((size_t)batch * n * num_chunks(vocab) * sizeof(SamplePart), 256);
    const size_t syncs = spec::align_up((size_t)batch * sizeof(GroupSync), 256);
    const int64_t gmax = std::min<int64_t>((vocab + kCoopThreads * 8 - 1) / (kCoopThreads * 8),
                                           kCoopThreads);
    const size_t reds = spec::align_up((size_t)batch * 2 * gmax * sizeof(double), 256);
    if (off_sync) *off_sync = parts;
    if (off_red) *off_red = parts + syncs;
    return parts + syncs + reds;
}

template <int DT>
int launch_sample(int batch, int n, int s1, int64_t vocab, const void *tl, const void *dl,
                  const float *temperature, const float *uniforms, const float *final_uniforms,
                  const int32_t *cand, const int32_t *ri, const int32_t *rn, const int32_t *rs,
                  int32_t *predict, int32_t *ai, int32_t *al, void *workspace,
                  int32_t *dev_status, hipStream_t st) {
    size_t off_sync = 0, off_red = 0;
    sample_workspace_layout(batch, n, vocab, &off_sync, &off_red);
    const int nch = num_chunks(vocab);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(tl) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(dl) % 16 == 0;
    SamplePart *part = static_cast<SamplePart *>(workspace);
    GroupSync *sync = reinterpret_cast<GroupSync *>(static_cast<char *>(workspace) + off_sync);
    double *red = reinterpret_cast<double *>(static_cast<char *>(workspace) + off_red);
    hipLaunchKernelGGL(sample_stats_kernel<DT>, dim3(nch, batch * n), dim3(kSweepThreads), 0, st,
                       tl, dl, vocab, n, batch, nch, vec_ok, temperature, part, sync);
    WalkArgs A{};
    A.n = n; A.s1 = s1; A.nchunks = nch; A.vocab = vocab; A.vec_ok = vec_ok; A.part = part;
    A.tlogits = tl; A.dlogits = dl; A.temperature = temperature; A.uniforms = uniforms;
    A.final_uniforms = final_uniforms; A.cand = cand; A.r_index = ri; A.r_next = rn;
    A.r_sib = rs; A.predict = predict; A.accept_index = ai; A.accept_length = al;
    A.status = dev_status; A.sync = sync; A.red = red;
    const CoopPlan pl = coop_plan<DT>(batch, vocab);
    if (pl.G >= 2) {
        A.G = pl.G;
        A.slice = pl.slice;
        void *args[] = {&A};
        const hipError_t e = hipLaunchCooperativeKernel(
            reinterpret_cast<const void *>(sample_walk_coop_kernel<DT>),
            dim3((unsigned)(batch * pl.G)), dim3(kCoopThreads), args, 0, st);
        if (e == hipSuccess) return SPEC_OK;
        (void)hipGetLastError();   // fall back below
    }
    A.G = 1;
    A.slice = vocab;
    hipLaunchKernelGGL(sample_walk_solo_kernel<DT>, dim3(batch), dim3(kSoloThreads), 0, st, A);
    return launch_status();
}

}  // namespace

extern "C" size_t spec_accept_workspace_size(int batch, int n, int64_t vocab, int sampled) {
    if (batch <= 0 || n <= 0 || vocab <= 0) return 0;
    if (!sampled) return spec_greedy_workspace_bytes(batch, n, vocab);
    return sample_workspace_layout(batch, n, vocab, nullptr, nullptr);
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
    int rc = spec_check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (batch == 0) return SPEC_OK;
    if (!target_logits || !draft_logits || !temperature || !uniforms || !final_uniforms ||
        !candidates || !retrieve_index || !retrieve_next_token || !retrieve_next_sibling ||
        !predict || !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_accept_workspace_size(batch, n, vocab, 1))
        return SPEC_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        return launch_sample<SPEC_BF16>(batch, n, s1, vocab, target_logits, draft_logits,
                                        temperature, uniforms, final_uniforms, candidates,
                                        retrieve_index, retrieve_next_token,
                                        retrieve_next_sibling, predict, accept_index,
                                        accept_length, workspace, dev_status, st);
    return launch_sample<SPEC_F32>(batch, n, s1, vocab, target_logits, draft_logits, temperature,
                                   uniforms, final_uniforms, candidates, retrieve_index,
                                   retrieve_next_token, retrieve_next_sibling, predict,
                                   accept_index, accept_length, workspace, dev_status, st);
}
