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
// One launch.  Only the rows the walk visits are read: on arrival at a node
// the walk computes that row's softmax statistics (max and sum of
// exp((x - max) / T), target and draft) and fetches its children's token
// logits; a rejection is one F(c) reduction; the terminal token an inverse
// CDF.  Preferred form: G co-resident workgroups per request, each owning a
// slice of the vocabulary, whose entries stay in registers for the whole
// visit.  Slice results are exchanged through write-once slots in the
// workspace (each workgroup publishes, then polls the G slots of that
// exchange); the last workgroup of a request to finish clears the slots it
// used, so the workspace is zero again after every call.  Every thread of
// every workgroup of a request evaluates the same decisions from the same
// data, so decisions need no communication.  When the grid cannot be
// co-resident the walk runs as one 1024-thread workgroup per request, which
// never waits on another workgroup.
//
// Launch forms.  Eager calls launch the co-resident form cooperatively (the
// runtime guarantees co-residency; a wait that still gives up raises
// SPEC_ST_SYNC).  A graph does not record the cooperative guarantee, and a
// recorded kernel may run beside other streams' kernels, so a recorded call
// launches the co-resident form as an ordinary kernel followed by a recovery
// kernel of one workgroup per request: a request whose wait gave up in the
// first kernel is flagged there, and the recovery kernel walks it again
// alone (overwriting whatever the first kernel wrote for it); unflagged
// requests return at once.  Neither kernel waits without bound, and every
// request ends with a complete walk.
//
// Per-entry probabilities are float32 exponentials (the hardware base-2
// exponential) of the argument (x - max) log2(e) / T carried as a float
// pair, normalised and accumulated in float64.
#include <algorithm>

#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kSoloThreads = 1024;
constexpr int kCoopThreads = 256;
constexpr int kCoopGridTarget = 512;           // workgroups of a cooperative walk, all requests
constexpr int kMaxGroups = 64;                 // slices per request (one wave gathers them)
constexpr int kCacheEntries = 16;              // row entries a walk thread keeps in registers
constexpr int kWords = 3;                      // exchange words per workgroup per exchange
constexpr int kSlotWords = 8;                  // one 64-byte slot per workgroup and exchange

// Exchange slot encoding: a slot holds bits(v) ^ kFlip, 0 meaning "not yet
// written" (a zero-filled workspace is empty).  kFlip is a signalling-NaN
// pattern that arithmetic never produces; a value equal to it is stored as
// the default quiet NaN instead.
constexpr uint64_t kFlip = 0x7FF4DEAD0BADF00Dull;
constexpr uint64_t kQuietNaN = 0x7FF8000000000000ull;

__device__ __forceinline__ uint64_t encode_bits(uint64_t b) {
    if (b == kFlip) b = kQuietNaN;
    return b ^ kFlip;
}

struct RowDist {
    Scale2 t, d;
    double inv_st, inv_sd;
};

template <int DT>
__device__ __forceinline__ float load_elem(const void *rowp, int64_t v) {
    if (DT == SPEC_BF16) return bf16_to_f32(static_cast<const uint16_t *>(rowp)[v]);
    return static_cast<const float *>(rowp)[v];
}

// weight of an entry in the residual state (c, F), without the 1/F factor,
// from its two exponentials
__device__ __forceinline__ double resid_from_exp(float et, float ed, const RowDist &rd, double c) {
    const double p = (double)et * rd.inv_st;
    const double q = (double)ed * rd.inv_sd;
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

// Calls f(v, xt, xd, cnt) for consecutive groups of up to 8 entries of
// [a, b) of the two rows (v the group's first entry, cnt its size; entries
// past cnt are -inf), with 16-byte loads when the rows allow them; unrolled
// so that several groups' loads are in flight together.
template <int DT, typename Fn>
__device__ __forceinline__ void for_each8(const void *trow, const void *drow, int64_t a, int64_t b,
                                          bool vec_ok, Fn &&f) {
#pragma unroll 2
    for (int64_t v = a; v < b; v += 8) {
        float xt[8], xd[8];
        const int cnt = (int)min((int64_t)8, b - v);
        if (vec_ok && cnt == 8) {
            load8<DT>(trow, v, xt);
            load8<DT>(drow, v, xd);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = j < cnt;
                xt[j] = in ? load_elem<DT>(trow, v + j) : -INFINITY;
                xd[j] = in ? load_elem<DT>(drow, v + j) : -INFINITY;
            }
        }
        f(v, xt, xd, cnt);
    }
}

// ---- wave and block reductions ---------------------------------------------------
//
// Full-wave reductions (every lane active at the call) kept in registers:
// DPP moves combine lanes inside each 16-lane row (quad xor 1, quad xor 2,
// half-row mirror, row mirror: after each step all lanes of a group hold the
// same value, addition and max being commutative), then the four row results
// are read out as scalars.  Every lane returns the same value, and equal
// inputs give equal results in every workgroup.

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v, double old) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v), o = __builtin_bit_cast(uint64_t, old);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)b, CTRL,
                                                             0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32),
                                                             (int)(uint32_t)(b >> 32), CTRL, 0xF,
                                                             0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

__device__ __forceinline__ double readlane_d(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double full_wave_sum_d(double v) {
    v += dpp_f64<kDppQuadXor1>(v, 0.0);
    v += dpp_f64<kDppQuadXor2>(v, 0.0);
    v += dpp_f64<kDppRowHalfMirror>(v, 0.0);
    v += dpp_f64<kDppRowMirror>(v, 0.0);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

__device__ __forceinline__ float full_wave_max(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadXor1>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppQuadXor2>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v, -INFINITY));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// s * exp((m - M) / T): a partial sum taken at max m, rescaled to max M
// (float exponential of the exactly formed argument; 0 for an empty part)
__device__ __forceinline__ double rescale(float m, double s, float M, float chi, float clo) {
    return m == -INFINITY ? 0.0 : s * (double)exp2_scaled(m, Scale2{M, chi, clo});
}

// Max and sum of exponentials from every thread's partial (m, s), target and
// draft at once; every thread gets the workgroup's values.  No barrier after
// the reads of sm / ss: the walk passes a barrier (the statistics exchange's)
// before it calls this again.
template <int NT>
__device__ void block_stats(float &mt, double &st, float &md, double &sd, float chi, float clo,
                            float *sm, double *ss) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float wt = full_wave_max(mt), wd = full_wave_max(md);
    const double rt = full_wave_sum_d(rescale(mt, st, wt, chi, clo));
    const double rd = full_wave_sum_d(rescale(md, sd, wd, chi, clo));
    if (lane == 0) {
        sm[2 * wave] = wt;
        sm[2 * wave + 1] = wd;
        ss[2 * wave] = rt;
        ss[2 * wave + 1] = rd;
    }
    __syncthreads();
    float Mt = -INFINITY, Md = -INFINITY;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        Mt = fmaxf(Mt, sm[2 * w]);
        Md = fmaxf(Md, sm[2 * w + 1]);
    }
    double St = 0.0, Sd = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        St += rescale(sm[2 * w], ss[2 * w], Mt, chi, clo);
        Sd += rescale(sm[2 * w + 1], ss[2 * w + 1], Md, chi, clo);
    }
    mt = Mt;
    st = St;
    md = Md;
    sd = Sd;
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
    __syncthreads();
    return before + incl - v;
}

// Sum of v over the workgroup.  No barrier after the reads of scratch: the
// caller passes one before the next use of it.
template <int NT>
__device__ double block_sum(double v, double *scratch) {
    v = full_wave_sum_d(v);
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += scratch[w];
    return s;
}

// ---------------------------------------------------------------------------
// the walk
// ---------------------------------------------------------------------------

struct WalkArgs {
    int n, s1;
    int64_t vocab;
    bool vec_ok;
    const void *tlogits, *dlogits;
    const float *temperature, *uniforms, *final_uniforms;
    const int32_t *cand, *r_index, *r_next, *r_sib;
    int32_t *predict, *accept_index, *accept_length, *status;
    int G;              // workgroups per request (1: one workgroup, no exchange)
    int64_t slice;      // vocabulary entries per workgroup, a multiple of 8 * threads
    int E;              // exchanges a request may make
    uint64_t *xch;      // [batch][E][G][kSlotWords] exchange slots (G > 1)
    unsigned *done;     // [batch] workgroups finished (G > 1)
    unsigned *redo;     // [batch] recorded form: requests to walk again; else null
    unsigned poll_limit;  // polls of one slot before giving up
};

template <int NT>
struct WalkShared {
    double cp[kMaxNodes];      // node k's token: target / draft probability in its parent's row
    double cq[kMaxNodes];
    int cand[kMaxNodes], next[kMaxNodes], sib[kMaxNodes], par[kMaxNodes];
    int row[kMaxNodes];        // local verify row of node k, -1 if invalid
    int pred[kMaxNodes];
    int ai[kMaxNodes + 1];
    float unif[kMaxNodes];
    float sm[2 * NT / 64];
    double ss[2 * NT / 64];
    double scratch[NT / 64];
    double bcast[2];           // exchange results, alternating buffers (one barrier each)
    RowDist dist[2];
    double tgt;
    int err, owner, draw, last;
};

template <int W>
__device__ __forceinline__ void load_words(const uint64_t *slot, uint64_t (&w)[W]) {
#pragma unroll
    for (int i = 0; i < W; ++i)
        w[i] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll the W words of one exchange slot until all are written (bounded);
// false on timeout.  The words are read together; one read is in flight at
// a time (more polls in flight only add traffic to the lines every
// workgroup is polling, and arrive later).
template <int W>
__device__ __forceinline__ bool read_slot(const uint64_t *slot, unsigned limit,
                                          uint64_t (&bits)[W]) {
    for (unsigned spins = 0; spins < limit; ++spins) {
        uint64_t w[W];
        load_words<W>(slot, w);
        bool all = true;
#pragma unroll
        for (int i = 0; i < W; ++i) all = all && w[i] != 0;
        if (all) {
#pragma unroll
            for (int i = 0; i < W; ++i) bits[i] = w[i] ^ kFlip;
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int i = 0; i < W; ++i) bits[i] = 0;
    return false;
}

__device__ __forceinline__ void write_word(uint64_t *slot, uint64_t bits) {
    __hip_atomic_store(slot, encode_bits(bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// CACHE: the segments fit in registers (COOP only).  Each launch runs one of
// the two segment paths, so each kernel holds only that one's code (the
// instruction cache is smaller than both together).
template <int DT, int NT, bool COOP, bool CACHE>
__global__ __launch_bounds__(NT) void sample_walk_kernel(WalkArgs A) {
    static_assert(COOP || !CACHE, "the one-workgroup walk does not cache");
    static_assert(NT % 64 == 0, "whole waves");
    __shared__ WalkShared<NT> S;
    const int G = COOP ? A.G : 1;
    const int req = COOP ? blockIdx.x / G : blockIdx.x;
    const int g = COOP ? blockIdx.x % G : 0;
    const int tid = threadIdx.x;
    // the recovery kernel walks only the requests the first kernel flagged
    if (!COOP && A.redo != nullptr && A.redo[req] == 0) return;
    const int n = A.n;
    const int base = req * n;
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    // log2(e) / T as a float pair (the exponentials are base 2)
    const double it = 1.4426950408889634 / (double)A.temperature[req];
    const float chi = (float)it;
    const float clo = (float)(it - (double)chi);

    // my slice of the vocabulary and, inside it, my contiguous segment
    const int64_t v0 = min(A.vocab, (int64_t)g * A.slice);
    const int64_t v1 = min(A.vocab, v0 + A.slice);
    const int64_t seg = A.slice / NT;
    const int64_t sa = min(v1, v0 + tid * seg);
    const int64_t sb = min(v1, sa + seg);
    auto row_ptr = [&](const void *m, int lrow) {
        return static_cast<const char *>(m) + (int64_t)(base + lrow) * A.vocab * eb;
    };

    // The current row's segment in registers when it fits: raw logits on
    // arrival, their exponentials once the row statistics are known.
    constexpr bool use_cache = CACHE;   // the host picks CACHE iff seg <= kCacheEntries
    static_assert(kCacheEntries == 16, "two groups of 8 cached entries");
    float ct[kCacheEntries], cd[kCacheEntries];
    // seg is a multiple of 8: the second group of 8 registers is used only
    // when seg is 16 (a uniform branch around the work on it otherwise)
    const bool wide = seg > 8;
    int cached_row = -1;               // local row whose raw logits ct / cd hold
    // body(i) over the cached entries in order: 0..7, then 8..15 when the
    // segment has 16.  Two loops of fixed length, so both unroll and the
    // register arrays are only ever indexed by constants (a loop with an
    // early exit was left rolled, indexing them through gpr-index mode).
    auto cached_each = [&](auto &&body) {
#pragma unroll
        for (int i = 0; i < 8; ++i) body(i);
        if (wide) {
#pragma unroll
            for (int i = 8; i < kCacheEntries; ++i) body(i);
        }
    };
    auto load_cache = [&](int lrow) {
        const void *trow = row_ptr(A.tlogits, lrow);
        const void *drow = row_ptr(A.dlogits, lrow);
#pragma unroll
        for (int i0 = 0; i0 < kCacheEntries; i0 += 8) {
            if (i0 == 8 && !wide) break;
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
                ct[i0 + j] = xt[j];
                cd[i0 + j] = xd[j];
            }
        }
        cached_row = lrow;
    };

    // ---- prologue: links and uniforms; the root's slice is fetched meanwhile
    // (local row 0, the usual layout; fetched again on arrival if the root
    // names another row) --------------------------------------------------------
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
    if constexpr (use_cache) load_cache(0);
    __syncthreads();
    if (tid < n) {
        if (S.row[tid] < 0) atomicOr(&S.err, SPEC_ST_RANGE);
        int c = S.next[tid];
        for (int steps = 0; steps < n && c != -1; ++steps) {
            if (c < 0 || c >= n) {
                atomicOr(&S.err, SPEC_ST_RANGE);
                break;
            }
            S.par[c] = tid;
            c = S.sib[c];
        }
    }
    __syncthreads();

    // ---- exchanges (uniform across the request's workgroups) -----------------
    int e = 0;                         // exchanges used so far
    int xb = 0;                        // exchange calls so far (result buffer parity)
    bool alive = true;
    auto slot = [&](int ex, int wg) -> uint64_t * {
        return A.xch + (((int64_t)req * A.E + ex) * G + wg) * kSlotWords;
    };
    // row statistics from every workgroup's slice statistics
    auto exchange_stats = [&](float mt, double st, float md, double sd) -> RowDist {
        if (COOP) {
            if (e >= A.E) {
                if (tid == 0) atomicOr(&S.err, SPEC_ST_RANGE | SPEC_ST_SYNC);
            } else {
                if (tid == 0) {
                    const uint64_t mm = (uint64_t)__float_as_uint(mt) |
                                        ((uint64_t)__float_as_uint(md) << 32);
                    write_word(slot(e, g) + 0, mm);
                    write_word(slot(e, g) + 1, __builtin_bit_cast(uint64_t, st));
                    write_word(slot(e, g) + 2, __builtin_bit_cast(uint64_t, sd));
                }
                if (tid < 64) {
                    float jmt = -INFINITY, jmd = -INFINITY;
                    double jst = 0.0, jsd = 0.0;
                    if (tid < G) {
                        uint64_t w[kWords];
                        if (!read_slot<kWords>(slot(e, tid), A.poll_limit, w)) {
                            atomicOr(&S.err, SPEC_ST_SYNC);
                        } else {
                            jmt = __uint_as_float((uint32_t)w[0]);
                            jmd = __uint_as_float((uint32_t)(w[0] >> 32));
                            jst = __builtin_bit_cast(double, w[1]);
                            jsd = __builtin_bit_cast(double, w[2]);
                        }
                    }
                    mt = full_wave_max(jmt);
                    md = full_wave_max(jmd);
                    st = full_wave_sum_d(rescale(jmt, jst, mt, chi, clo));
                    sd = full_wave_sum_d(rescale(jmd, jsd, md, chi, clo));
                }
                ++e;
            }
        }
        if (tid == 0) {
            RowDist r;
            r.t = Scale2{mt, chi, clo};
            r.d = Scale2{md, chi, clo};
            r.inv_st = st > 0.0 ? 1.0 / st : 0.0;
            r.inv_sd = sd > 0.0 ? 1.0 / sd : 0.0;
            S.dist[xb & 1] = r;
        }
        __syncthreads();
        if (S.err & SPEC_ST_SYNC) alive = false;
        // the other buffer is written next; this one not before every thread
        // has passed the next exchange's barrier
        const RowDist r = S.dist[xb & 1];
        ++xb;
        return r;
    };
    double sj = 0.0;                   // wave 0, lane j < G: slice j's sum in the last sweep
    // total over the slices of a per-workgroup sum
    auto exchange_sum = [&](double slice_sum) -> double {
        if (!COOP) {
            __syncthreads();           // every thread has read the block sum's scratch
            sj = slice_sum;
            return slice_sum;
        }
        if (e >= A.E) {
            if (tid == 0) atomicOr(&S.err, SPEC_ST_RANGE | SPEC_ST_SYNC);
            __syncthreads();
            alive = false;
            return 0.0;
        }
        if (tid == 0) write_word(slot(e, g), __builtin_bit_cast(uint64_t, slice_sum));
        if (tid < 64) {
            sj = 0.0;
            uint64_t w[1];
            if (tid < G) {
                if (read_slot<1>(slot(e, tid), A.poll_limit, w)) sj = __builtin_bit_cast(double, w[0]);
                else atomicOr(&S.err, SPEC_ST_SYNC);
            }
            const double tot = full_wave_sum_d(sj);
            if (tid == 0) S.bcast[xb & 1] = tot;
        }
        ++e;
        __syncthreads();
        if (S.err & SPEC_ST_SYNC) alive = false;
        const double tot = S.bcast[xb & 1];
        ++xb;
        return tot;
    };

    // ---- the walk (every thread takes the same decisions) --------------------
    double mine = 0.0;                 // my segment's sum in the last sweep
    int cur = 0, cnt = 0;
    if (tid == 0) S.ai[0] = base + max(S.row[0], 0);
    double c = 0.0, F = 1.0;
    bool swept = false;                // the last sweep was of the current node with multiplier c
    RowDist rd{};
    int lr = -1;
    // sum of my segment's residual weights with multiplier cc
    auto segment_sum = [&](double cc) -> double {
        double m = 0.0;
        if constexpr (use_cache) {
            cached_each([&](int i) { m += resid_from_exp(ct[i], cd[i], rd, cc); });
        } else {
            for_each8<DT>(row_ptr(A.tlogits, lr), row_ptr(A.dlogits, lr), sa, sb, A.vec_ok,
                          [&](int64_t, const float (&xt)[8], const float (&xd)[8], int) {
#pragma unroll
                              for (int j = 0; j < 8; ++j)
                                  m += resid_from_exp(exp2_scaled(xt[j], rd.t),
                                                      exp2_scaled(xd[j], rd.d), rd, cc);
                          });
        }
        return m;
    };
    auto sweep = [&](double cc) -> double {
        mine = segment_sum(cc);
        return exchange_sum(block_sum<NT>(mine, S.scratch));
    };

    for (int level = 0; level < n && alive; ++level) {
        lr = S.row[cur];
        if (lr < 0) break;
        // arrival: the children's token logits (kept in registers until the
        // statistics are exchanged, so their loads overlap that work), this
        // row's slice, its statistics
        const bool is_child = tid < n && S.par[tid] == cur;
        float kid_t = 0.f, kid_d = 0.f;
        if (is_child) {
            const int t = S.cand[tid];
            if (t >= 0 && t < A.vocab) {
                kid_t = load_elem<DT>(row_ptr(A.tlogits, lr), t);
                kid_d = load_elem<DT>(row_ptr(A.dlogits, lr), t);
            }
        }
        float mt = -INFINITY, md = -INFINITY;
        double st = 0.0, sd = 0.0;
        if constexpr (use_cache) {
            if (cached_row != lr) load_cache(lr);
            cached_each([&](int i) {
                mt = fmaxf(mt, ct[i]);
                md = fmaxf(md, cd[i]);
            });
            // the registers now take the exponentials relative to this
            // thread's max; one factor per row moves them to the row's max
            const Scale2 sct{mt, chi, clo}, scd{md, chi, clo};
            float ft = 0.f, fd = 0.f;
            cached_each([&](int i) {
                ct[i] = exp2_scaled(ct[i], sct);
                cd[i] = exp2_scaled(cd[i], scd);
                ft += ct[i];
                fd += cd[i];
            });
            cached_row = -1;
            st = ft;
            sd = fd;
        } else {
            const void *trow = row_ptr(A.tlogits, lr);
            const void *drow = row_ptr(A.dlogits, lr);
            for_each8<DT>(trow, drow, sa, sb, A.vec_ok,
                          [&](int64_t, const float (&xt)[8], const float (&xd)[8], int) {
#pragma unroll
                              for (int j = 0; j < 8; ++j) {
                                  mt = fmaxf(mt, xt[j]);
                                  md = fmaxf(md, xd[j]);
                              }
                          });
            const Scale2 sct{mt, chi, clo}, scd{md, chi, clo};
            float ft = 0.f, fd = 0.f;
            for_each8<DT>(trow, drow, sa, sb, A.vec_ok,
                          [&](int64_t, const float (&xt)[8], const float (&xd)[8], int) {
#pragma unroll
                              for (int j = 0; j < 8; ++j) {
                                  ft += exp2_scaled(xt[j], sct);
                                  fd += exp2_scaled(xd[j], scd);
                              }
                          });
            st = ft;
            sd = fd;
        }
        const float thr_mt = mt, thr_md = md;
        block_stats<NT>(mt, st, md, sd, chi, clo, S.sm, S.ss);
        rd = exchange_stats(mt, st, md, sd);
        if (is_child) {
            S.cp[tid] = (double)exp2_scaled(kid_t, rd.t) * rd.inv_st;
            S.cq[tid] = (double)exp2_scaled(kid_d, rd.d) * rd.inv_sd;
        }
        __syncthreads();
        if (!alive) break;
        if constexpr (use_cache) {
            const float ft = thr_mt == -INFINITY ? 0.f : exp2_scaled(thr_mt, rd.t);
            const float fd = thr_md == -INFINITY ? 0.f : exp2_scaled(thr_md, rd.d);
            cached_each([&](int i) {
                ct[i] *= ft;
                cd[i] *= fd;
            });
        }

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
                // u < min(1, (max(0, p - c q) / F) / q), without the divisions
                const double p = S.cp[k];
                const double q = S.cq[k];
                const double r = fmax(fma(-c, q, p), 0.0);
                const double u = (double)S.unif[k];
                dec = q > 0.0 ? (u < 1.0 && u * q * F < r) : (r > 0.0 ? u < 1.0 : u < 0.0);
            } else if (tid == 0) {
                atomicOr(&S.err, SPEC_ST_RANGE);
            }
            if (dec) {
                hit = k;
                break;
            }
            // rejected: F(c + F)
            const double cn = c + F;
            const double Fn = sweep(cn);
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
    bool terminal_written = false;
    if (alive && lr >= 0 && lr == S.row[cur]) {
        // after a rejection at this node the last sweep's sums are this residual's
        const double tot = swept ? F : sweep(c);
        if (alive) {
            const double target = (double)A.final_uniforms[req] * tot;
            if (tid == 0) {
                S.owner = INT_MAX;
                S.draw = INT_MAX;
            }
            __syncthreads();
            if (COOP) {
                if (tid < 64) {
                    // slice prefix sums in slice order; the owner holds the crossing
                    double incl = sj;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const double x = __shfl_up(incl, o, 64);
                        if (tid >= o) incl += x;
                    }
                    const double pre = incl - sj;
                    const bool here = tid < G && sj > 0.0 && pre <= target && target < pre + sj;
                    const uint64_t bal = __ballot(here);
                    if (bal != 0 && tid == __builtin_ctzll(bal)) {
                        S.owner = tid;
                        S.tgt = target - pre;
                    }
                }
            } else if (tid == 0 && target < tot) {
                S.owner = 0;
                S.tgt = target;
            }
            __syncthreads();
            const int owner = S.owner;
            const double tgt = S.tgt;
            if (owner == INT_MAX) {
                // no crossing: the target sits at the very end of the mass
                if (g == 0 && tid == 0) A.predict[base + lr] = (int)(A.vocab - 1);
            } else if (owner == g) {
                double slice_tot;
                const double before = block_exclusive_scan<NT>(mine, S.scratch, slice_tot);
                if (sa < sb && before <= tgt && tgt < before + mine) {
                    // first entry of my segment where the running sum crosses tgt
                    double run = before;
                    int64_t x = -1;
                    if constexpr (use_cache) {
                        cached_each([&](int i) {
                            run += resid_from_exp(ct[i], cd[i], rd, c);
                            if (x < 0 && run > tgt) x = sa + i;
                        });
                    } else {
                        for_each8<DT>(row_ptr(A.tlogits, lr), row_ptr(A.dlogits, lr), sa, sb,
                                      A.vec_ok,
                                      [&](int64_t v, const float (&xt)[8], const float (&xd)[8],
                                          int cnt) {
                                          if (x >= 0) return;
#pragma unroll
                                          for (int j = 0; j < 8; ++j) {
                                              run += resid_from_exp(exp2_scaled(xt[j], rd.t),
                                                                    exp2_scaled(xd[j], rd.d), rd, c);
                                              if (x < 0 && j < cnt && run > tgt) x = v + j;
                                          }
                                      });
                    }
                    if (x >= 0 && x < sb) atomicMin(&S.draw, (int)x);
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
    if (COOP && A.redo != nullptr && (S.err & SPEC_ST_SYNC)) {
        // a wait gave up: the recovery kernel walks this request again and
        // reports its status
        if (tid == 0)
            __hip_atomic_store(A.redo + req, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (tid == 0) {
        raise_status(A.status, S.err);
    }
    if (!COOP && A.redo != nullptr && tid == 0) A.redo[req] = 0;

    // the last workgroup of the request to get here clears the request's
    // slots: every other one has read all it will read
    if (COOP) {
        if (tid == 0) {
            // relaxed: this workgroup's slot reads have returned their values
            // before the increment is issued, and the clearing needs nothing
            // else from the others (an acquire / release here would write back
            // the L2 on every workgroup)
            const unsigned old = __hip_atomic_fetch_add(A.done + req, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            S.last = old == (unsigned)G - 1;
        }
        __syncthreads();
        if (S.last) {
            const int used = (S.err & SPEC_ST_SYNC) ? A.E : e;
            uint64_t *x = A.xch + (int64_t)req * A.E * G * kSlotWords;
            for (int i = tid; i < used * G * kWords; i += NT)
                __hip_atomic_store(x + (i / kWords) * kSlotWords + i % kWords, (uint64_t)0,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0)
                __hip_atomic_store(A.done + req, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr int64_t kMinSlice = (int64_t)kCoopThreads * 8;

// upper bound of the workgroups per request the plan can pick
int group_cap(int batch, int64_t vocab) {
    int64_t G = std::min<int64_t>((vocab + kMinSlice - 1) / kMinSlice, kMaxGroups);
    G = std::min<int64_t>(G, std::max(2, kCoopGridTarget / std::max(batch, 1)));
    return (int)std::max<int64_t>(G, 1);
}

int exchanges_per_request(int n) { return 2 * n + 2; }

struct CoopPlan {
    int G;
    int64_t slice;
    bool cache;         // segments of at most kCacheEntries entries
};

// Workgroups of one cooperative-walk kernel that fit on the device at once
// (0 if cooperative launch is unavailable).
template <int DT, bool CACHE>
int coop_capacity() {
    return spec::resident_capacity(
        reinterpret_cast<const void *>(sample_walk_kernel<DT, kCoopThreads, true, CACHE>),
        kCoopThreads, true);
}

// Workgroups per request for the cooperative walk, or G = 0 when the grid
// cannot be co-resident (or cooperative launch is unavailable).
template <int DT>
CoopPlan coop_plan(int batch, int64_t vocab) {
    const int cap = std::min(coop_capacity<DT, true>(), coop_capacity<DT, false>());
    int64_t G = group_cap(batch, vocab);
    G = std::min<int64_t>(G, cap / std::max(batch, 1));
    if (G < 2) return CoopPlan{0, 0, false};
    int64_t slice = (vocab + G - 1) / G;
    slice = (slice + kMinSlice - 1) / kMinSlice * kMinSlice;
    G = (vocab + slice - 1) / slice;
    if (G < 2) return CoopPlan{0, 0, false};
    return CoopPlan{(int)G, slice, slice / kCoopThreads <= kCacheEntries};
}

// [exchange slots][done counters][recovery flags], each 256-byte aligned
size_t sample_workspace_layout(int batch, int n, int64_t vocab, size_t *off_done,
                               size_t *off_redo) {
    const size_t xch = spec::align_up((size_t)batch * exchanges_per_request(n) *
                                          group_cap(batch, vocab) * kSlotWords * sizeof(uint64_t),
                                      256);
    const size_t per_req = spec::align_up((size_t)batch * sizeof(unsigned), 256);
    if (off_done) *off_done = xch;
    if (off_redo) *off_redo = xch + per_req;
    return xch + 2 * per_req;
}

template <int DT>
int launch_sample(int batch, int n, int s1, int64_t vocab, const void *tl, const void *dl,
                  const float *temperature, const float *uniforms, const float *final_uniforms,
                  const int32_t *cand, const int32_t *ri, const int32_t *rn, const int32_t *rs,
                  int32_t *predict, int32_t *ai, int32_t *al, void *workspace,
                  int32_t *dev_status, hipStream_t st) {
    size_t off_done = 0, off_redo = 0;
    sample_workspace_layout(batch, n, vocab, &off_done, &off_redo);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    WalkArgs A{};
    A.n = n;
    A.s1 = s1;
    A.vocab = vocab;
    A.vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(tl) % 16 == 0 &&
               reinterpret_cast<uintptr_t>(dl) % 16 == 0;
    A.tlogits = tl;
    A.dlogits = dl;
    A.temperature = temperature;
    A.uniforms = uniforms;
    A.final_uniforms = final_uniforms;
    A.cand = cand;
    A.r_index = ri;
    A.r_next = rn;
    A.r_sib = rs;
    A.predict = predict;
    A.accept_index = ai;
    A.accept_length = al;
    A.status = dev_status;
    A.E = exchanges_per_request(n);
    A.xch = static_cast<uint64_t *>(workspace);
    A.done = reinterpret_cast<unsigned *>(static_cast<char *>(workspace) + off_done);
    A.poll_limit = spec::poll_limit();
    A.redo = nullptr;
    const CoopPlan pl = coop_plan<DT>(batch, vocab);
    const int64_t solo_slice =
        ((vocab + kSoloThreads - 1) / kSoloThreads + 7) / 8 * 8 * kSoloThreads;
    if (pl.G >= 2) {
        A.G = pl.G;
        A.slice = pl.slice;
        const dim3 grid((unsigned)(batch * pl.G)), block(kCoopThreads);
        if (spec::stream_capturing(st)) {
            // recorded: the co-resident form as an ordinary launch, then the
            // recovery kernel for requests whose wait gave up
            A.redo = reinterpret_cast<unsigned *>(static_cast<char *>(workspace) + off_redo);
            if (pl.cache)
                hipLaunchKernelGGL((sample_walk_kernel<DT, kCoopThreads, true, true>), grid, block,
                                   0, st, A);
            else
                hipLaunchKernelGGL((sample_walk_kernel<DT, kCoopThreads, true, false>), grid, block,
                                   0, st, A);
            A.G = 1;
            A.slice = solo_slice;
            hipLaunchKernelGGL((sample_walk_kernel<DT, kSoloThreads, false, false>), dim3(batch),
                               dim3(kSoloThreads), 0, st, A);
            return launch_status();
        }
        const void *fn = pl.cache
            ? reinterpret_cast<const void *>(sample_walk_kernel<DT, kCoopThreads, true, true>)
            : reinterpret_cast<const void *>(sample_walk_kernel<DT, kCoopThreads, true, false>);
        void *args[] = {&A};
        if (hipLaunchCooperativeKernel(fn, grid, block, args, 0, st) == hipSuccess) return SPEC_OK;
        (void)hipGetLastError();   // fall back below
    }
    A.G = 1;
    A.slice = solo_slice;
    hipLaunchKernelGGL((sample_walk_kernel<DT, kSoloThreads, false, false>), dim3(batch),
                       dim3(kSoloThreads), 0, st, A);
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
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return SPEC_ERR_WORKSPACE;
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
