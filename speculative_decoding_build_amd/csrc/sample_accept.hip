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
//   2. the walk.  A prologue merges the chunk statistics of every row of the
//      request and fetches, for every node, its token's target / draft logit
//      in its parent's row, so accepting a child needs no memory access.
//      Only a rejection (one F(c) reduction) and the terminal draw (an
//      inverse CDF) touch the vocabulary.  Preferred form: G co-resident
//      workgroups per request, each owning a slice of the vocabulary; a
//      reduction is split across the slices and the G slice sums are
//      exchanged through write-once slots (no barrier: every workgroup
//      publishes its sum, then polls the G slots of that exchange).  Every
//      thread of every workgroup of a request evaluates the same decisions
//      from the same data, so decisions need no communication.  When the
//      grid cannot be co-resident the walk runs as one 1024-thread
//      workgroup per request.  The last rejection's sweep at a node is
//      reused by the terminal draw at that node (same residual).
//
// Per-entry probabilities are float32 exponentials of the exactly formed
// argument (x - max) / T, normalised and accumulated in float64.
#include <algorithm>

#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kSoloThreads = 1024;
constexpr int kCoopThreads = 256;
constexpr unsigned kSpinLimit = 1u << 20;      // polls of one slot before giving up
constexpr int kCoopGridTarget = 512;           // workgroups of a cooperative walk, all requests
constexpr int kCacheEntries = 16;              // row entries a walk thread keeps in registers

// Exchange slot contents: kEmpty until written.  kEmpty is a signalling-NaN
// bit pattern that float arithmetic never produces; a written value equal to
// it is replaced by the default quiet NaN.
constexpr uint64_t kEmpty = 0x7FF4DEAD0BADF00Dull;
constexpr uint64_t kQuietNaN = 0x7FF8000000000000ull;

struct SamplePart {
    float mt, md;
    double st, sd;
};

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

// 8 consecutive entries starting at v (a multiple of 8) as floats
template <int DT>
__device__ __forceinline__ void load8(const void *rowp, int64_t v, float (&x)[8]) {
    if (DT == SPEC_BF16) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(rowp) + v);
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = lo_bf16(a[j]);
            x[2 * j + 1] = hi_bf16(a[j]);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(rowp) + v);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(rowp) + v + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// Sum of resid_weight over [a, b) in ascending order; 16-byte loads when the
// rows allow them (a is a multiple of 8 then).
template <int DT>
__device__ double range_sum(const void *trow, const void *drow, int64_t a, int64_t b,
                            bool vec_ok, const RowDist &rd, double c) {
    double s = 0.0;
    int64_t v = a;
    if (vec_ok) {
        for (; v + 8 <= b; v += 8) {
            float xt[8], xd[8];
            load8<DT>(trow, v, xt);
            load8<DT>(drow, v, xd);
#pragma unroll
            for (int j = 0; j < 8; ++j) s += resid_weight(xt[j], xd[j], rd, c);
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

// Exclusive prefix of v over threads in thread order; also returns the total.
// Every workgroup that scans the same values gets the same results.
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

// Also empties the exchange slots of the walk that follows: row r of the
// grid clears slots [r*G, r*G + G) (r = request * n + exchange).
template <int DT>
__global__ __launch_bounds__(kSweepThreads) void sample_stats_kernel(
    const void *__restrict__ tlogits, const void *__restrict__ dlogits, int64_t vocab, int n,
    int nchunks, bool vec_ok, const float *__restrict__ temperature,
    SamplePart *__restrict__ part, uint64_t *__restrict__ xch, int G) {
    const int c = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    if (xch != nullptr && c == 0)
        for (int j = tid; j < G; j += kSweepThreads) xch[row * G + j] = kEmpty;
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
// 2. the walk
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
    int G;              // workgroups per request (1: one workgroup, no exchange)
    int64_t slice;      // vocabulary entries per workgroup, a multiple of 8 * threads
    uint64_t *xch;      // [batch][n][G] exchange slots (G > 1)
};

template <int NT>
struct WalkShared {
    RowDist dist[kMaxNodes];   // by local verify row
    float cxt[kMaxNodes];      // node k's token: target / draft logit in its parent's row
    float cxd[kMaxNodes];
    int cand[kMaxNodes], next[kMaxNodes], sib[kMaxNodes], par[kMaxNodes];
    int row[kMaxNodes];        // local verify row of node k, -1 if invalid
    int pred[kMaxNodes];
    int ai[kMaxNodes + 1];
    float unif[kMaxNodes];
    double scratch[NT / 64];
    double bcast;
    int err, owner, draw;
};

// Running (max, scaled sum) of softmax chunk statistics:
// S = sum_chunks s_k * exp((m_k - M) / T) with M the largest m_k so far.
__device__ __forceinline__ void merge_stat(float &M, double &Sm, float m2, double s2, double it) {
    if (m2 == -INFINITY) return;                  // an empty chunk (its sum is 0)
    if (M == -INFINITY) { M = m2; Sm = s2; return; }
    if (m2 > M) {
        Sm = Sm * exp(((double)M - (double)m2) * it) + s2;
        M = m2;
    } else {
        Sm += s2 * exp(((double)m2 - (double)M) * it);
    }
}

// Poll one exchange slot until it is written (bounded); false on timeout.
__device__ __forceinline__ bool read_slot(uint64_t *slot, double &v) {
    unsigned spins = 0;
    uint64_t bits;
    while ((bits = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == kEmpty) {
        if (++spins > kSpinLimit) { v = 0.0; return false; }
        __builtin_amdgcn_s_sleep(1);
    }
    v = __builtin_bit_cast(double, bits);
    return true;
}

template <int DT, int NT, bool COOP>
__global__ __launch_bounds__(NT) void sample_walk_kernel(WalkArgs A) {
    static_assert(NT % 64 == 0 && 64 % (NT / 64) == 0, "lanes per row must divide a wave");
    __shared__ WalkShared<NT> S;
    const int G = COOP ? A.G : 1;
    const int req = COOP ? blockIdx.x / G : blockIdx.x;
    const int g = COOP ? blockIdx.x % G : 0;
    const int tid = threadIdx.x;
    const int n = A.n;
    const int base = req * n;
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const double it = 1.0 / (double)A.temperature[req];

    // my slice of the vocabulary and, inside it, my contiguous segment
    const int64_t v0 = min(A.vocab, (int64_t)g * A.slice);
    const int64_t v1 = min(A.vocab, v0 + A.slice);
    const int64_t seg = A.slice / NT;
    const int64_t sa = min(v1, v0 + tid * seg);
    const int64_t sb = min(v1, sa + seg);

    // ---- prologue: links, uniforms and the statistics of every row -------
    if (tid < n) {
        int row = A.r_index[base + tid];
        row = (row >= base && row < base + n) ? row - base : -1;
        S.row[tid] = row;
        S.pred[tid] = 0;
        S.par[tid] = -1;
        S.cand[tid] = A.cand[base + tid];
        S.next[tid] = A.r_next[base + tid];
        S.sib[tid] = A.r_sib[base + tid];
        S.unif[tid] = A.uniforms[base + tid];
    }
    if (tid == 0) S.err = 0;
    {
        constexpr int LPR = NT / 64;                  // lanes per row (n <= 64)
        const int k = tid / LPR, sub = tid % LPR;
        float mt = -INFINITY, md = -INFINITY;
        double st = 0.0, sd = 0.0;
        if (k < n) {
            for (int c = sub; c < A.nchunks; c += LPR) {
                const SamplePart p = A.part[(int64_t)(base + k) * A.nchunks + c];
                merge_stat(mt, st, p.mt, p.st, it);
                merge_stat(md, sd, p.md, p.sd, it);
            }
        }
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) {
            const float omt = __shfl_xor(mt, o, 64), omd = __shfl_xor(md, o, 64);
            const double ost = __shfl_xor(st, o, 64), osd = __shfl_xor(sd, o, 64);
            merge_stat(mt, st, omt, ost, it);
            merge_stat(md, sd, omd, osd, it);
        }
        if (k < n && sub == 0) {
            const float ithi = (float)it;
            const float itlo = (float)(it - (double)ithi);
            RowDist rd;
            rd.t = Scale{mt, ithi, itlo};
            rd.d = Scale{md, ithi, itlo};
            rd.inv_st = st > 0.0 ? 1.0 / st : 0.0;
            rd.inv_sd = sd > 0.0 ? 1.0 / sd : 0.0;
            S.dist[k] = rd;
        }
    }
    __syncthreads();
    if (tid < n) {
        if (S.row[tid] < 0) atomicOr(&S.err, SPEC_ST_RANGE);
        int c = S.next[tid];
        for (int steps = 0; steps < n && c != -1; ++steps) {
            if (c < 0 || c >= n) { atomicOr(&S.err, SPEC_ST_RANGE); break; }
            S.par[c] = tid;
            c = S.sib[c];
        }
    }
    __syncthreads();
    if (tid < n) {
        const int p = S.par[tid];
        const int t = S.cand[tid];
        float xt = 0.f, xd = 0.f;
        if (p >= 0 && S.row[p] >= 0 && t >= 0 && t < A.vocab) {
            const int64_t grow = base + S.row[p];
            xt = load_elem<DT>(static_cast<const char *>(A.tlogits) + grow * A.vocab * eb, t);
            xd = load_elem<DT>(static_cast<const char *>(A.dlogits) + grow * A.vocab * eb, t);
        }
        S.cxt[tid] = xt;
        S.cxd[tid] = xd;
    }
    __syncthreads();

    // ---- the walk (every thread takes the same decisions) --------------------
    int e = 0;                         // exchanges used so far (slots of this request)
    bool alive = true;
    double mine = 0.0, before = 0.0;   // my segment's sum and its prefix in my slice
    double sj = 0.0, pre = 0.0;        // thread j < G: slice j's sum and its prefix
    // The current node's row segment, as the exponentials exp_scaled gives
    // (target, draft; 0 past the segment), kept in registers when the segment
    // fits: later rejections at the node and its terminal draw then read no
    // memory.
    const bool use_cache = COOP && seg <= kCacheEntries;   // the solo walk's segments are longer
    float cet[kCacheEntries], ced[kCacheEntries];
    int cached_row = -1;
    auto fill_cache = [&](const void *trow, const void *drow, const RowDist &rd) {
#pragma unroll
        for (int i0 = 0; i0 < kCacheEntries; i0 += 8) {
            float xt[8], xd[8];
            const int64_t v = sa + i0;
            if (A.vec_ok && v + 8 <= sb) {
                load8<DT>(trow, v, xt);
                load8<DT>(drow, v, xd);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool in = v + j < sb;
                    xt[j] = in ? load_elem<DT>(trow, v + j) : -INFINITY;
                    xd[j] = in ? load_elem<DT>(drow, v + j) : -INFINITY;
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                cet[i0 + j] = exp_scaled(xt[j], rd.t);
                ced[i0 + j] = exp_scaled(xd[j], rd.d);
            }
        }
    };
    auto cached_weight = [&](int i, const RowDist &rd, double cc) -> double {
        const double p = (double)cet[i] * rd.inv_st;
        const double q = (double)ced[i] * rd.inv_sd;
        return fmax(fma(-cc, q, p), 0.0);
    };
    // sweep of the current node's row (local row lr) with multiplier cc;
    // returns F(cc)
    auto sweep = [&](const void *trow, const void *drow, const RowDist &rd, int lr,
                     double cc) -> double {
        if (use_cache) {
            if (cached_row != lr) {
                fill_cache(trow, drow, rd);
                cached_row = lr;
            }
            double m = 0.0;
#pragma unroll
            for (int i = 0; i < kCacheEntries; ++i) m += cached_weight(i, rd, cc);
            mine = m;
        } else {
            mine = range_sum<DT>(trow, drow, sa, sb, A.vec_ok, rd, cc);
        }
        double slice_tot;
        before = block_exclusive_scan<NT>(mine, S.scratch, slice_tot);
        if (!COOP) {
            sj = slice_tot;
            pre = 0.0;
            return slice_tot;
        }
        if (e >= n) {                      // more exchanges than a tree of n nodes needs
            if (tid == 0) atomicOr(&S.err, SPEC_ST_RANGE | SPEC_ST_SYNC);
            __syncthreads();
            alive = false;
            return 0.0;
        }
        uint64_t *slots = A.xch + ((int64_t)base + e) * G;
        ++e;
        if (tid == 0) {
            uint64_t bits = __builtin_bit_cast(uint64_t, slice_tot);
            if (bits == kEmpty) bits = kQuietNaN;
            __hip_atomic_store(slots + g, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        sj = 0.0;
        if (tid < G && !read_slot(slots + tid, sj)) atomicOr(&S.err, SPEC_ST_SYNC);
        double tot;
        pre = block_exclusive_scan<NT>(sj, S.scratch, tot);   // also publishes the err bit
        if (S.err & SPEC_ST_SYNC) alive = false;
        return tot;
    };
    // first entry of my segment where the running sum from `before` exceeds tgt
    auto find = [&](const void *trow, const void *drow, const RowDist &rd, double cc,
                    double tgt) -> int64_t {
        if (!use_cache) return range_find<DT>(trow, drow, sa, sb, rd, cc, before, tgt);
        double run = before;
        int64_t x = -1;
#pragma unroll
        for (int i = 0; i < kCacheEntries; ++i) {
            run += cached_weight(i, rd, cc);
            if (x < 0 && run > tgt) x = sa + i;
        }
        return x < sb ? x : -1;
    };

    int cur = 0, cnt = 0;
    if (tid == 0) S.ai[0] = base + max(S.row[0], 0);
    double c = 0.0, F = 1.0;
    bool swept = false;        // the last sweep was of the current node with multiplier c
    for (int level = 0; level < n && alive; ++level) {
        const int lr = S.row[cur];
        if (lr < 0) break;
        const RowDist rd = S.dist[lr];
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)(base + lr) * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)(base + lr) * A.vocab * eb;
        c = 0.0;
        F = 1.0;
        swept = false;
        int hit = -1;
        int k = S.next[cur];
        for (int steps = 0; steps < n && k != -1 && alive; ++steps) {
            if (k < 0 || k >= n) break;                 // reported by the prologue
            const int t = S.cand[k];
            bool dec = false;
            if (t >= 0 && t < A.vocab) {
                const double p = (double)exp_scaled(S.cxt[k], rd.t) * rd.inv_st;
                const double q = (double)exp_scaled(S.cxd[k], rd.d) * rd.inv_sd;
                const double r = fmax(fma(-c, q, p), 0.0) / F;
                const double ratio = q > 0.0 ? r / q : (r > 0.0 ? INFINITY : 0.0);
                dec = (double)S.unif[k] < fmin(1.0, ratio);
            } else if (tid == 0) {
                atomicOr(&S.err, SPEC_ST_RANGE);
            }
            if (dec) { hit = k; break; }
            // rejected: F(c + F)
            const double cn = c + F;
            const double Fn = sweep(trow, drow, rd, lr, cn);
            if (!alive) break;
            if (Fn > 0.0) {
                c = cn;
                F = Fn;
                swept = true;
            } else {
                if (tid == 0) atomicOr(&S.err, SPEC_ST_ZERO_RESIDUAL);
                swept = false;
            }
            k = S.sib[k];
        }
        if (!alive || hit < 0) break;
        if (cnt + 1 >= A.s1) {
            if (tid == 0) atomicOr(&S.err, SPEC_ST_DEPTH);
            break;
        }
        if (tid == 0) {
            S.pred[cur] = S.cand[hit];
            S.ai[cnt + 1] = base + max(S.row[hit], 0);
        }
        ++cnt;
        cur = hit;
    }

    // ---- terminal draw: inverse CDF of max(0, p - c q) in vocabulary order ----
    const int lr = S.row[cur];
    bool terminal_written = false;
    if (alive && lr >= 0) {
        const RowDist rd = S.dist[lr];
        const void *trow = static_cast<const char *>(A.tlogits) + (int64_t)(base + lr) * A.vocab * eb;
        const void *drow = static_cast<const char *>(A.dlogits) + (int64_t)(base + lr) * A.vocab * eb;
        // after a rejection at this node the last sweep's sums are this residual's
        const double tot = swept ? F : sweep(trow, drow, rd, lr, c);
        if (alive) {
            const double target = (double)A.final_uniforms[req] * tot;
            if (tid == 0) { S.owner = INT_MAX; S.draw = INT_MAX; }
            __syncthreads();
            if (COOP) {
                if (tid < G && sj > 0.0 && pre <= target && target < pre + sj) atomicMin(&S.owner, tid);
            } else if (tid == 0 && target < tot) {
                S.owner = 0;
            }
            __syncthreads();
            const int owner = S.owner;
            if (COOP && tid == owner) S.bcast = target - pre;   // target measured from its slice
            __syncthreads();
            if (owner == INT_MAX) {
                // no crossing: the target sits at the very end of the mass
                if (g == 0 && tid == 0) A.predict[base + lr] = (int)(A.vocab - 1);
            } else if (owner == g) {
                const double tgt = COOP ? S.bcast : target;
                if (sa < sb && before <= tgt && tgt < before + mine) {
                    const int64_t x = find(trow, drow, rd, c, tgt);
                    if (x >= 0) atomicMin(&S.draw, (int)x);
                }
                __syncthreads();
                if (tid == 0) {
                    int x = S.draw;
                    if (x == INT_MAX) x = (int)(v1 > v0 ? v1 - 1 : A.vocab - 1);
                    A.predict[base + lr] = x;
                }
            }
            terminal_written = true;
        }
    }
    __syncthreads();
    if (g == 0) {
        const int terminal = terminal_written ? cur : -1;
        if (tid < n && S.row[tid] >= 0 && tid != terminal) A.predict[base + S.row[tid]] = S.pred[tid];
        for (int j = tid; j < A.s1; j += NT)
            A.accept_index[(int64_t)req * A.s1 + j] = (j <= cnt) ? S.ai[j] : -1;
        if (tid == 0) A.accept_length[req] = cnt + 1;
    }
    if (tid == 0) raise_status(A.status, S.err);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr int64_t kMinSlice = (int64_t)kCoopThreads * 8;

int max_groups(int64_t vocab) {
    return (int)std::min<int64_t>((vocab + kMinSlice - 1) / kMinSlice, kCoopThreads);
}

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
                       &per, reinterpret_cast<const void *>(sample_walk_kernel<DT, kCoopThreads, true>),
                       kCoopThreads, 0) == hipSuccess;
        cap = (ok && coop) ? cus * per : 0;
        cached_device = dev;
    }
    int64_t G = max_groups(vocab);
    G = std::min<int64_t>(G, cap / std::max(batch, 1));
    G = std::min<int64_t>(G, std::max(2, kCoopGridTarget / std::max(batch, 1)));
    if (G < 2) return CoopPlan{0, 0};
    int64_t slice = (vocab + G - 1) / G;
    slice = (slice + kMinSlice - 1) / kMinSlice * kMinSlice;
    G = (vocab + slice - 1) / slice;
    if (G < 2) return CoopPlan{0, 0};
    return CoopPlan{(int)G, slice};
}

size_t sample_workspace_layout(int batch, int n, int64_t vocab, size_t *off_xch) {
    const size_t parts = spec::align_up((size_t)batch * n * num_chunks(vocab) * sizeof(SamplePart), 256);
    const size_t xch = spec::align_up((size_t)batch * n * max_groups(vocab) * sizeof(uint64_t), 256);
    if (off_xch) *off_xch = parts;
    return parts + xch;
}

template <int DT>
int launch_sample(int batch, int n, int s1, int64_t vocab, const void *tl, const void *dl,
                  const float *temperature, const float *uniforms, const float *final_uniforms,
                  const int32_t *cand, const int32_t *ri, const int32_t *rn, const int32_t *rs,
                  int32_t *predict, int32_t *ai, int32_t *al, void *workspace,
                  int32_t *dev_status, hipStream_t st) {
    size_t off_xch = 0;
    sample_workspace_layout(batch, n, vocab, &off_xch);
    const int nch = num_chunks(vocab);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(tl) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(dl) % 16 == 0;
    SamplePart *part = static_cast<SamplePart *>(workspace);
    uint64_t *xch = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + off_xch);
    const CoopPlan pl = coop_plan<DT>(batch, vocab);
    hipLaunchKernelGGL(sample_stats_kernel<DT>, dim3(nch, batch * n), dim3(kSweepThreads), 0, st,
                       tl, dl, vocab, n, nch, vec_ok, temperature, part,
                       pl.G >= 2 ? xch : nullptr, pl.G);
    WalkArgs A{};
    A.n = n; A.s1 = s1; A.nchunks = nch; A.vocab = vocab; A.vec_ok = vec_ok; A.part = part;
    A.tlogits = tl; A.dlogits = dl; A.temperature = temperature; A.uniforms = uniforms;
    A.final_uniforms = final_uniforms; A.cand = cand; A.r_index = ri; A.r_next = rn;
    A.r_sib = rs; A.predict = predict; A.accept_index = ai; A.accept_length = al;
    A.status = dev_status; A.xch = xch;
    if (pl.G >= 2) {
        A.G = pl.G;
        A.slice = pl.slice;
        const dim3 grid((unsigned)(batch * pl.G)), block(kCoopThreads);
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive) {
            // recorded into a graph: an ordinary launch of a grid sized to
            // what the device holds at once
            hipLaunchKernelGGL((sample_walk_kernel<DT, kCoopThreads, true>), grid, block, 0, st, A);
            return launch_status();
        }
        void *args[] = {&A};
        const void *fn = reinterpret_cast<const void *>(sample_walk_kernel<DT, kCoopThreads, true>);
        if (hipLaunchCooperativeKernel(fn, grid, block, args, 0, st) == hipSuccess) return SPEC_OK;
        (void)hipGetLastError();   // fall back below; the emptied slots go unused
    }
    A.G = 1;
    A.slice = ((vocab + kSoloThreads - 1) / kSoloThreads + 7) / 8 * 8 * kSoloThreads;
    hipLaunchKernelGGL((sample_walk_kernel<DT, kSoloThreads, false>), dim3(batch),
                       dim3(kSoloThreads), 0, st, A);
    return launch_status();
}

}  // namespace

extern "C" size_t spec_accept_workspace_size(int batch, int n, int64_t vocab, int sampled) {
    if (batch <= 0 || n <= 0 || vocab <= 0) return 0;
    if (!sampled) return spec_greedy_workspace_bytes(batch, n, vocab);
    return sample_workspace_layout(batch, n, vocab, nullptr);
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
