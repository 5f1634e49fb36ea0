// Sampling-parameter pre-pass: top-k / top-p filtering of the target
// distribution before the sampled accepts.
//
// "投机解码 Accept:从 Verify 行到最终输出路径" (四: eagle_sample takes the
// target softmax at the request's temperature, then top-k / top-p filtering
// and renormalisation) and "SGLang 源码完全拆解(十一):投机解码" (三条判定路径).
// Row i belongs to request i / n.  p = softmax(x / T); entries rank by p
// descending (logit descending), lower index first; the entry of rank r is
// kept iff r < top_k (when 1 <= top_k < V) and the mass of the entries
// ranked above it is < top_p (when top_p < 1; a row of -inf logits has no
// distribution and only top_k applies).  Kept logits are copied,
// the others become -inf, so softmax(out / T) is the renormalised
// distribution the accepts read.  A greedy request is top_k = 1.
//
// The kept set is {key >= kappa} for the 64-bit order key (value bits, then
// the complemented index).  Vocabularies above 8192 entries take three
// launches:
//   chunks (row x chunk of <= 8192 entries, 256 threads): the chunk max,
//     sum exp((x - m_c) / T) and the chunk's top K keys in order (K = top_k
//     when 1 <= top_k <= 64, else 64), ranked among the entries at or above
//     tau_c, the least of the four waves' w-th largest thread maxima (4w >=
//     K, so at least K entries of the chunk are >= tau_c);
//   rows (one 1024-thread workgroup): M, Z = sum s_c exp((m_c - M) / T);
//     the chunks' lists merged in pairs give the row's top K; when the
//     kept set ends among them its last key is the cutoff; otherwise the
//     row runs the search below itself;
//   output (row x chunk): kept iff key >= cutoff.
// The search used for the other rows and small vocabularies is a radix
// search on the value bits, one 1024-thread workgroup per row:
//   pass 1: the row max M;
//   pass 2: Z = sum exp((x - M) / T) and a 4096-bin histogram (count,
//     float64 mass) of the top 12 key bits, in LDS (4096 bins spread the
//     atomics of one wave over many addresses);
//   the bin where the kept set ends is the highest bin whose cumulative
//     count reaches top_k or cumulative mass reaches top_p * Z;
//   further passes histogram the next key bits of the entries in that bin
//   (bf16: 4 bits; float: 12, then 8) until the cutoff value v is fixed,
//   with how many entries equal to v are kept (those of lowest index);
//   last pass: entries above v kept, entries equal to v ranked in index
//   order (block scans over tiles of 8192 entries), the output written.
// Exponentials are the float-pair base-2 exponential used by the accept
// sweeps; masses are float64 sums.
#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kRT = 1024;                  // threads per row
constexpr int kRW = kRT / SPEC_WAVE;       // waves per row
constexpr int kTile = kRT * 8;             // entries per pass step (8 per thread)
constexpr int kMaxBins = 4096;

__device__ __forceinline__ uint32_t value_key(float v) {
    uint32_t bits = __float_as_uint(v == 0.f ? 0.f : v);
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

constexpr int kCapK = 64;                  // the largest K: a chunk stores its top K keys
constexpr int kChunkCand = 512;            // candidates a chunk ranks (more: the row is searched whole)
constexpr int kMaxChunks = 64;             // chunks per row of the three-launch path
// calls of at most this many logit bytes re-read the row in the output
// launch (measured faster there than a launch of stores alone)
constexpr int64_t kReadOutBytes = 32ll << 20;

struct ChunkHead {                         // one chunk of one row (16 bytes)
    float m;                               // chunk max
    uint32_t over;                         // 1: too many candidates, the top K not stored
    double s;                              // sum exp((x - m) / T); 0 when top_p is off
};

struct Decision {                          // one row (16 bytes)
    uint64_t cutoff;                       // kept iff key >= cutoff
    uint32_t mode;                         // 0: every entry kept; 1: the row step wrote the row;
                                           // 2: the first nkeep keys of the row's kept list
    uint32_t nkeep;
};

// chunks of a row for the three-launch path (0: one workgroup per row), and
// their size: a multiple of 8 entries, at most kChunk; every chunk but the
// last holds that many, the last more than 3500 (all 256 threads hold entries)
inline int filter_chunks(int64_t rows, int64_t V) {
    if (V <= kChunk) return 0;
    const int64_t nch = (V + kChunk - 1) / kChunk;
    return nch <= kMaxChunks && rows * nch <= INT_MAX ? (int)nch : 0;
}

inline int64_t filter_chunk_size(int64_t V, int nch) {
    return ((V + nch - 1) / nch + 7) / 8 * 8;
}

__device__ __forceinline__ uint64_t order_key(float v, int64_t i) {
    return ((uint64_t)value_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ int64_t key_index(uint64_t key) {
    return (int64_t)(0xFFFFFFFFu - (uint32_t)key);
}

// key(v, i) >= key(cv, ci) as float compares (finite or -inf values; -0
// and +0 are one value); i and ci relative to one chunk start
__device__ __forceinline__ bool at_or_above(float v, int i, float cv, int ci) {
    return v > cv || (v == cv && i <= ci);
}

// the chunk-relative index of a thread's entry e (the layout of load_chunk)
__device__ __forceinline__ int local_index(int tid, int e) {
    return (e >> 3) * kSweepThreads * 8 + tid * 8 + (e & 7);
}

__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t vb = (uint32_t)(key >> 32);
    return __uint_as_float((vb & 0x80000000u) ? (vb & 0x7FFFFFFFu) : ~vb);
}

constexpr int kCand = 1024;                // candidates the fast path ranks
constexpr int kWaveTop = 8;                // tau: the least of the waves' 8th largest thread maxima

struct RowShared {
    union {
        struct {
            uint32_t cnt[kMaxBins];
            double mass[kMaxBins];
        };
        struct {
            uint64_t la[kMaxChunks * kCapK];       // sorted top-K lists being merged
            uint64_t lb[kMaxChunks * kCapK / 2];
        };
        struct {
            uint64_t tk[kRT];              // each thread's largest key
            uint64_t ck[kCand];            // candidates: keys >= tau, their masses
            double cm[kCand];
            uint64_t sk[kCand];            // the candidates by rank
            double sm[kCand];
        };
    };
    uint64_t w8[kRW];
    double hz;
    int over;
    int nc, rmin;
    uint32_t wc[kRW];
    double wm[kRW];
    float wf[kRW];
    int pick;
    uint32_t pick_cnt, pick_n;
    double pick_mass;
};

// 8 entries of the row from index i0 (the caller keeps i0 a multiple of 8)
template <int DT>
__device__ __forceinline__ void load8(const void *row, int64_t i0, int64_t V, bool vec_ok,
                                      float (&x)[8]) {
    if (DT == SPEC_BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(row);
        if (vec_ok && i0 + 8 <= V) {
            const uint4 w = *reinterpret_cast<const uint4 *>(p + i0);
            x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x); x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
            x[4] = lo_bf16(w.z); x[5] = hi_bf16(w.z); x[6] = lo_bf16(w.w); x[7] = hi_bf16(w.w);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = i0 + j < V ? bf16_to_f32(p[i0 + j]) : -INFINITY;
        }
    } else {
        const float *p = static_cast<const float *>(row);
        if (vec_ok && i0 + 8 <= V) {
            const float4 a = *reinterpret_cast<const float4 *>(p + i0);
            const float4 b = *reinterpret_cast<const float4 *>(p + i0 + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = i0 + j < V ? p[i0 + j] : -INFINITY;
        }
    }
}

// Block-wide sums of (count, mass) over the threads above this one
// (thread order = bin order); returns the totals of the threads with a
// higher index.
__device__ __forceinline__ void above_sums(RowShared &S, uint32_t c, double m, uint32_t &ac, double &am) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t ic = c;
    double im = m;
#pragma unroll
    for (int o = 1; o < SPEC_WAVE; o <<= 1) {
        const uint32_t tc = __shfl_down(ic, o, SPEC_WAVE);
        const double tm = __shfl_down(im, o, SPEC_WAVE);
        if (lane + o < SPEC_WAVE) {
            ic += tc;
            im += tm;
        }
    }
    if (lane == 0) {
        S.wc[wave] = ic;
        S.wm[wave] = im;
    }
    __syncthreads();
    ac = ic - c;
    am = im - m;
    for (int w = wave + 1; w < kRW; ++w) {
        ac += S.wc[w];
        am += S.wm[w];
    }
    __syncthreads();
}

// The bin (of nb) where the kept set ends, given the count cb and mass mb
// above all of them; -1 if none (every entry of the current range is kept).
// cut_above_c / cut_above_m: the count and mass above the picked bin,
// cb and mb included.
__device__ __forceinline__ int find_cut(RowShared &S, int nb, int k, double tpz, uint32_t cb, double mb,
                        uint32_t &cut_above_c, double &cut_above_m, uint32_t &cut_n) {
    const int tid = threadIdx.x;
    const int per = nb > kRT ? nb / kRT : 1;
    const int b0 = tid * per;
    uint32_t c = 0;
    double m = 0.0;
    if (b0 < nb)
        for (int i = 0; i < per; ++i) {
            c += S.cnt[b0 + i];
            m += S.mass[b0 + i];
        }
    uint32_t ac;
    double am;
    above_sums(S, c, m, ac, am);
    if (tid == 0) S.pick = -1;
    __syncthreads();
    int mine = -1;
    uint32_t mc = 0, mn = 0;
    double mm = 0.0;
    if (b0 < nb) {
        uint32_t rc = cb + ac;
        double rm = mb + am;
        for (int i = per - 1; i >= 0; --i) {
            const uint32_t bc = S.cnt[b0 + i];
            const double bm = S.mass[b0 + i];
            if (bc > 0 && ((k > 0 && rc + bc >= (uint32_t)k) || rm + bm >= tpz)) {
                mine = b0 + i;
                mc = rc;
                mm = rm;
                mn = bc;
                break;
            }
            rc += bc;
            rm += bm;
        }
    }
    if (mine >= 0) atomicMax(&S.pick, mine);
    __syncthreads();
    const int pick = S.pick;
    if (pick >= 0 && mine == pick) {
        S.pick_cnt = mc;
        S.pick_mass = mm;
        S.pick_n = mn;
    }
    __syncthreads();
    cut_above_c = S.pick_cnt;
    cut_above_m = S.pick_mass;
    cut_n = S.pick_n;
    __syncthreads();
    return pick;
}

// The fast path: the nc (<= kCand) candidates in S.ck / S.cm are the row's
// top nc entries.  Ranks them (keys are unique) and sums their masses in
// rank order; the last kept rank is min(top_k - 1, the first rank whose
// inclusive mass reaches top_p * Z).  Returns whether that rank lies among
// the candidates, with its key in cutoff.  S.rmin must hold INT_MAX.
__device__ __forceinline__ bool cut_among(RowShared &S, int nc, int k, double tpz, uint64_t &cutoff) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int q = tid; q < nc; q += kRT) {
        const uint64_t mine = S.ck[q];
        int r = 0;
        for (int u = 0; u < nc; ++u) r += S.ck[u] > mine;
        S.sk[r] = mine;
        S.sm[r] = S.cm[q];
    }
    __syncthreads();
    // inclusive mass by rank (thread t holds rank t)
    double v = tid < nc ? S.sm[tid] : 0.0;
#pragma unroll
    for (int o = 1; o < SPEC_WAVE; o <<= 1) {
        const double u = __shfl_up(v, o, SPEC_WAVE);
        if (lane >= o) v += u;
    }
    if (lane == 63) S.wm[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += S.wm[w];
    if (tid < nc && ((k > 0 && tid + 1 >= k) || v >= tpz)) atomicMin(&S.rmin, tid);
    __syncthreads();
    const int rstar = S.rmin;
    const bool ok = rstar < nc;
    if (ok) cutoff = S.sk[rstar];
    __syncthreads();
    return ok;
}

// Three-launch path, row step: M = max m_c, Z = sum s_c exp((m_c - M) / T),
// and the row's top K keys, merged from the chunks' sorted top-K lists in
// pairs (an entry's place in a merged pair is its place in its own list
// plus the entries of the other list above it; equal keys are zero padding
// and go to the lower list first).  Returns 0 when the row is decided (the
// kept set ends among the top K, always when 1 <= top_k <= 64, or both
// rules are off): the cutoff goes to dec for the output launch.  Otherwise
// dec says the row is done here and the caller searches the row itself:
// from scratch (1: a chunk had too many candidates) or from the histogram
// on, with M in S.wf[0] and Z in S.hz (2).
__device__ __forceinline__ int merge_chunks(RowShared &S, const ChunkHead *__restrict__ heads,
                                             const uint64_t *__restrict__ keys, int nch,
                                             int64_t row, float T, int k, int K, float tpf,
                                             Decision *__restrict__ dec,
                                             uint64_t *__restrict__ kept) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the chunks' lists, K keys each (stored with a stride of kCapK), loaded
    // together with the chunk heads
    const int total = nch * K;
    constexpr int kPer = kMaxChunks * kCapK / kRT;
    uint64_t lv[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int t = tid + q * kRT, l = t / K;
        lv[q] = t < total ? keys[(row * nch + l) * kCapK + (t - l * K)] : 0;
    }
    ChunkHead hv{-INFINITY, 0u, 0.0};
    if (wave == 0 && lane < nch) hv = heads[row * nch + lane];
#pragma unroll
    for (int q = 0; q < kPer; ++q)
        if (tid + q * kRT < total) S.la[tid + q * kRT] = lv[q];
    if (wave == 0) {
        const float hm = hv.m;
        const double hs = hv.s;
        const uint32_t ho = hv.over;
        const float m = wave_max(hm);
        // a chunk with s_c = 0 adds nothing
        double z = hs > 0.0 ? hs * exp(((double)hm - (double)m) / (double)T) : 0.0;
        z = wave_sum_d(z);
        const bool any_over = __ballot(ho != 0) != 0;
        if (lane == 0) {
            S.wf[0] = m;
            S.hz = z;
            S.over = any_over;
        }
    }
    __syncthreads();
    const float m = S.wf[0];
    const double tpz = tpf < 1.f && S.hz > 0.0 ? (double)tpf * S.hz : INFINITY;
    if (S.over) {
        if (tid == 0) dec[row] = Decision{0, 1u, 0u};
        __syncthreads();
        return 1;
    }
    if (k == 0 && !(tpz < INFINITY)) {             // both rules off: every entry kept
        if (tid == 0) dec[row] = Decision{0, 0u, 0u};
        return 0;
    }
    uint64_t *src = S.la, *dst = S.lb;
    for (int L = nch; L > 1; L = (L + 1) / 2) {
        for (int t = tid; t < L * K; t += kRT) {
            const int l = t / K, j = t - l * K, p = l ^ 1;
            const uint64_t key = src[t];
            int r = j;
            if (p < L) {
                const uint64_t *P = src + p * K;
                int lo = 0, hi = K;                // entries of P above key
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const bool above = l < p ? P[mid] > key : P[mid] >= key;
                    lo = above ? mid + 1 : lo;
                    hi = above ? hi : mid;
                }
                r += lo;
            }
            if (r < K) dst[(l >> 1) * K + r] = key;
        }
        __syncthreads();
        uint64_t *t2 = src;
        src = dst;
        dst = t2;
    }
    // src[0 .. K) is the row's top K, descending; masses and the last kept
    // rank: min(top_k - 1, the first rank whose inclusive mass reaches
    // top_p * Z), in wave 0
    bool ok = false;
    uint64_t cutoff = 0;
    __syncthreads();
    if (wave == 0) {
        const Scale2 scl = make_scale2(m, T);
        const uint64_t key = lane < K ? src[lane] : 0;
        double v = lane < K && m != -INFINITY ? (double)exp2_scaled(key_value(key), scl) : 0.0;
#pragma unroll
        for (int o = 1; o < SPEC_WAVE; o <<= 1) {
            const double u = __shfl_up(v, o, SPEC_WAVE);
            if (lane >= o) v += u;
        }
        const uint64_t hit = __ballot(lane < K && key != 0 && ((k > 0 && lane + 1 >= k) || v >= tpz));
        int rs = -1;
        if (hit != 0) {
            rs = __builtin_ctzll(hit);
            ok = true;
            cutoff = __shfl(key, rs, SPEC_WAVE);
        }
        // the kept entries are the top rs + 1 keys: the output launch writes
        // them from the keys, without reading the row again
        if (lane <= rs) kept[row * kCapK + lane] = key;
        if (lane == 0) {
            dec[row] = ok ? Decision{cutoff, 2u, (uint32_t)(rs + 1)} : Decision{0, 1u, 0u};
            S.over = ok ? 0 : 2;
        }
    }
    __syncthreads();
    ok = S.over == 0;
    __syncthreads();
    return ok ? 0 : 2;
}

template <int DT, int KEYBITS>
__global__ __launch_bounds__(kRT) void filter_row_kernel(
    const void *in, void *out, int64_t V, bool vec_ok, int n,
    const float *__restrict__ temperature, const int32_t *__restrict__ top_k,
    const float *__restrict__ top_p, const ChunkHead *__restrict__ heads,
    const uint64_t *__restrict__ keys, int nch, Decision *__restrict__ dec,
    uint64_t *__restrict__ kept) {
    __shared__ RowShared S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int req = (int)(row / n);
    const float T = temperature[req];
    const int kk = top_k[req];
    const int k = (kk >= 1 && kk < V) ? kk : 0;
    const float tpf = top_p[req];
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const char *rin = static_cast<const char *>(in) + row * V * eb;
    char *rout = static_cast<char *>(out) + row * V * eb;
    float x[8];
    bool known = false;                    // M and Z from the chunks
    float m = -INFINITY;
    double z = 0.0;
    int nc = kCand + 1;                    // no candidates: the fast path is skipped
    if (heads != nullptr) {
        const int K = (k >= 1 && k <= kCapK) ? k : kCapK;
        const int st = merge_chunks(S, heads, keys, nch, row, T, k, K, tpf, dec, kept);
        if (st == 0) return;
        if (st == 2) {
            known = true;
            m = S.wf[0];
            z = S.hz;
        }
        __syncthreads();                   // the search below reuses the shared fields
    }

    if (!known) {
        // pass 1: the row max and each thread's largest 64-bit key (value
        // bits, then the complemented index: unique, larger = ranked higher)
        uint64_t tk = 0;
        for (int64_t t0 = 0; t0 < V; t0 += kTile) {
            const int64_t i0 = t0 + tid * 8;
            load8<DT>(rin, i0, V, vec_ok, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (i0 + j < V) {
                    m = fmaxf(m, x[j]);
                    const uint64_t k64 = ((uint64_t)value_key(x[j]) << 32) |
                                         (uint32_t)(0xFFFFFFFFu - (uint32_t)(i0 + j));
                    tk = k64 > tk ? k64 : tk;
                }
            }
        }
        m = wave_max(m);
        if (lane == 0) S.wf[wave] = m;
        S.tk[tid] = tk;
        if (tid < kRW) S.w8[tid] = 0;
        if (tid == 0) {
            S.nc = 0;
            S.rmin = INT_MAX;
        }
        __syncthreads();
        m = S.wf[0];
        for (int w = 1; w < kRW; ++w) m = fmaxf(m, S.wf[w]);
        const Scale2 scl1 = make_scale2(m, T);
        // tau: the least of the waves' 8th largest thread maxima, so at least
        // 8 x 16 entries are >= tau
        {
            int r = 0;
            const uint64_t *wk = S.tk + wave * SPEC_WAVE;
            for (int u = 0; u < SPEC_WAVE; ++u) r += wk[u] > tk;
            if (tk != 0 && r == kWaveTop - 1) S.w8[wave] = tk;
        }
        __syncthreads();
        uint64_t tau = S.w8[0];
        for (int w = 1; w < kRW; ++w) tau = S.w8[w] < tau ? S.w8[w] : tau;

        // pass 2: Z and the candidates (entries with key >= tau)
        for (int64_t t0 = 0; t0 < V; t0 += kTile) {
            const int64_t i0 = t0 + tid * 8;
            load8<DT>(rin, i0, V, vec_ok, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (i0 + j < V) {
                    const float e = m == -INFINITY ? 0.f : exp2_scaled(x[j], scl1);
                    z += (double)e;
                    const uint64_t k64 = ((uint64_t)value_key(x[j]) << 32) |
                                         (uint32_t)(0xFFFFFFFFu - (uint32_t)(i0 + j));
                    if (k64 >= tau) {
                        const int slot = atomicAdd(&S.nc, 1);
                        if (slot < kCand) {
                            S.ck[slot] = k64;
                            S.cm[slot] = (double)e;
                        }
                    }
                }
            }
        }
        z = wave_sum_d(z);
        if (lane == 0) S.wm[wave] = z;
        __syncthreads();
        z = 0.0;
        for (int w = 0; w < kRW; ++w) z += S.wm[w];
        nc = S.nc;
        __syncthreads();
    }
    const Scale2 scl = make_scale2(m, T);
    // a row of -inf logits (Z = 0) has no distribution: top-p does nothing
    const double tpz = tpf < 1.f && z > 0.0 ? (double)tpf * z : INFINITY;

    // fast path: the candidates are the top nc entries of the row; when the
    // kept set ends among them its last entry's key is the cutoff
    bool fast = false, keep_all = k == 0 && !(tpz < INFINITY);
    uint64_t cutoff = 0;
    if (!keep_all && nc <= kCand) {
        if (cut_among(S, nc, k, tpz, cutoff)) {
            fast = true;
        } else if (nc == V) {
            fast = true;
            keep_all = true;
        }
    }

    if (!fast && !keep_all) {
        // the first level's histogram (top 12 key bits)
        for (int i = tid; i < kMaxBins; i += kRT) {
            S.cnt[i] = 0;
            S.mass[i] = 0.0;
        }
        __syncthreads();
        for (int64_t t0 = 0; t0 < V; t0 += kTile) {
            const int64_t i0 = t0 + tid * 8;
            load8<DT>(rin, i0, V, vec_ok, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (i0 + j < V) {
                    const float e = m == -INFINITY ? 0.f : exp2_scaled(x[j], scl);
                    const uint32_t d = (value_key(x[j]) >> (32 - KEYBITS)) >> (KEYBITS - 12);
                    atomicAdd(&S.cnt[d], 1u);
                    atomicAdd(&S.mass[d], (double)e);
                }
            }
        }
        __syncthreads();
    }
    constexpr int kB1 = 12;

    uint32_t cb = 0;                       // entries above the current range
    double mb = 0.0;                       // their mass
    uint32_t prefix = 0;
    int done_bits = 0;
    uint32_t n_tie = 0;
    int nb = 1 << kB1;
    int bits = kB1;
    while (!fast && !keep_all) {
        uint32_t ac, n_in;
        double am;
        const int pick = find_cut(S, nb, k, tpz, cb, mb, ac, am, n_in);
        if (pick < 0) {
            keep_all = true;
            break;
        }
        cb = ac;                           // find_cut's totals include the earlier levels'
        mb = am;
        prefix = (prefix << bits) | (uint32_t)pick;
        done_bits += bits;
        n_tie = n_in;
        if (done_bits == KEYBITS) break;
        // next level: the following bits of the entries in the picked bin
        bits = KEYBITS - done_bits > 12 ? 12 : KEYBITS - done_bits;
        nb = 1 << bits;
        for (int i = tid; i < nb; i += kRT) {
            S.cnt[i] = 0;
            S.mass[i] = 0.0;
        }
        __syncthreads();
        const int shift = KEYBITS - done_bits - bits;
        for (int64_t t0 = 0; t0 < V; t0 += kTile) {
            const int64_t i0 = t0 + tid * 8;
            load8<DT>(rin, i0, V, vec_ok, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t key = value_key(x[j]) >> (32 - KEYBITS);
                if (i0 + j < V && (key >> (KEYBITS - done_bits)) == prefix) {
                    const uint32_t d = (key >> shift) & (uint32_t)(nb - 1);
                    atomicAdd(&S.cnt[d], 1u);
                    atomicAdd(&S.mass[d], (double)exp2_scaled(x[j], scl));
                }
            }
        }
        __syncthreads();
    }

    // how many entries equal to v are kept: tie i (index order) iff
    // cb + i < top_k and mb + i * e(v) < top_p * Z
    uint32_t keep_tie = n_tie;
    if (!fast && !keep_all) {
        if (k > 0) keep_tie = min(keep_tie, (uint32_t)k - cb);
        if (tpz < INFINITY) {
            const uint32_t vb = prefix << (32 - KEYBITS);
            const uint32_t fb = (vb & 0x80000000u) ? (vb & 0x7FFFFFFFu) : ~vb;
            const float ev = exp2_scaled(__uint_as_float(fb), scl);
            uint32_t cp = n_tie;
            if (ev > 0.f) {
                const double q = (tpz - mb) / (double)ev;
                cp = q <= 0.0 ? 0u : (q >= (double)n_tie ? n_tie : (uint32_t)ceil(q));
                // settle the quotient's rounding on the rule itself
                while (cp > 0 && mb + (double)(cp - 1) * ev >= tpz) --cp;
                while (cp < n_tie && mb + (double)cp * ev < tpz) ++cp;
            }
            keep_tie = min(keep_tie, cp);
        }
    }
    const bool need_rank = !fast && !keep_all && keep_tie < n_tie;

    // last pass: the output, ties ranked in index order
    uint32_t rank0 = 0;
    for (int64_t t0 = 0; t0 < V; t0 += kTile) {
        const int64_t i0 = t0 + tid * 8;
        load8<DT>(rin, i0, V, vec_ok, x);
        bool keep[8], tie[8];
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t key = value_key(x[j]) >> (32 - KEYBITS);
            tie[j] = !fast && !keep_all && key == prefix && i0 + j < V;
            keep[j] = keep_all || (!fast && (key > prefix || (tie[j] && !need_rank)));
            if (fast && !keep_all)
                keep[j] = (((uint64_t)value_key(x[j]) << 32) |
                           (uint32_t)(0xFFFFFFFFu - (uint32_t)(i0 + j))) >= cutoff;
            mine += tie[j];
        }
        if (need_rank) {
            uint32_t incl = mine;
#pragma unroll
            for (int o = 1; o < SPEC_WAVE; o <<= 1) {
                const uint32_t v = __shfl_up(incl, o, SPEC_WAVE);
                if (lane >= o) incl += v;
            }
            if (lane == 63) S.wc[wave] = incl;
            __syncthreads();
            uint32_t r = rank0 + incl - mine, total = 0;
            for (int w = 0; w < kRW; ++w) {
                if (w < wave) r += S.wc[w];
                total += S.wc[w];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (tie[j]) keep[j] = r++ < keep_tie;
            rank0 += total;
        }
        if (DT == SPEC_BF16) {
            uint16_t *o16 = reinterpret_cast<uint16_t *>(rout);
            if (vec_ok && i0 + 8 <= V) {
                uint16_t h[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    h[j] = keep[j] ? (uint16_t)(__float_as_uint(x[j]) >> 16) : (uint16_t)0xFF80u;
                uint4 w;
                w.x = h[0] | ((uint32_t)h[1] << 16);
                w.y = h[2] | ((uint32_t)h[3] << 16);
                w.z = h[4] | ((uint32_t)h[5] << 16);
                w.w = h[6] | ((uint32_t)h[7] << 16);
                *reinterpret_cast<uint4 *>(o16 + i0) = w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i0 + j < V)
                        o16[i0 + j] = keep[j] ? (uint16_t)(__float_as_uint(x[j]) >> 16)
                                              : (uint16_t)0xFF80u;
            }
        } else {
            float *o32 = reinterpret_cast<float *>(rout);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < V) o32[i0 + j] = keep[j] ? x[j] : -INFINITY;
        }
    }
}

// A thread's kPerThread entries of a chunk as stored (bf16: two per word),
// in the layout of load_chunk; missing entries hold -inf.
template <int DT>
struct Packed {
    static constexpr int kWords = DT == SPEC_BF16 ? kPerThread / 2 : kPerThread;
    uint32_t w[kWords];

    __device__ __forceinline__ void load(const void *row, int64_t start, int64_t end, bool vec_ok,
                                         int tid) {
#pragma unroll
        for (int g = 0; g < kPerThread / 8; ++g) {
            const int64_t e0 = start + (int64_t)g * kSweepThreads * 8 + tid * 8;
            if (DT == SPEC_BF16) {
                const uint16_t *p = static_cast<const uint16_t *>(row);
                if (vec_ok && e0 + 8 <= end) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(p + e0);
                    w[g * 4 + 0] = v.x; w[g * 4 + 1] = v.y; w[g * 4 + 2] = v.z; w[g * 4 + 3] = v.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = e0 + 2 * j < end ? p[e0 + 2 * j] : 0xFF80u;
                        const uint32_t hi = e0 + 2 * j + 1 < end ? p[e0 + 2 * j + 1] : 0xFF80u;
                        w[g * 4 + j] = lo | (hi << 16);
                    }
                }
            } else {
                const float *p = static_cast<const float *>(row);
                if (vec_ok && e0 + 8 <= end) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(p + e0);
                    const uint4 b = *reinterpret_cast<const uint4 *>(p + e0 + 4);
                    w[g * 8 + 0] = a.x; w[g * 8 + 1] = a.y; w[g * 8 + 2] = a.z; w[g * 8 + 3] = a.w;
                    w[g * 8 + 4] = b.x; w[g * 8 + 5] = b.y; w[g * 8 + 6] = b.z; w[g * 8 + 7] = b.w;
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        w[g * 8 + j] = e0 + j < end ? __float_as_uint(p[e0 + j]) : 0xFF800000u;
                }
            }
        }
    }

    __device__ __forceinline__ float operator[](int e) const {
        if (DT == SPEC_BF16) return (e & 1) ? hi_bf16(w[e >> 1]) : lo_bf16(w[e >> 1]);
        return __uint_as_float(w[e]);
    }
};

// Three-launch path, chunk step: work item t = (row t / nch, chunk t % nch),
// one 256-thread workgroup, 32 entries per thread in registers.
template <int DT>
__global__ __launch_bounds__(kSweepThreads, 4) void filter_chunk_kernel(
    const void *in, int64_t V, int64_t C, bool vec_ok, int n, int nch,
    const float *__restrict__ temperature, const int32_t *__restrict__ top_k,
    const float *__restrict__ top_p, ChunkHead *__restrict__ heads, uint64_t *__restrict__ keys) {
    constexpr int NW = kSweepThreads / SPEC_WAVE;
    __shared__ uint64_t tks[kSweepThreads];
    __shared__ uint64_t ck[kChunkCand];
    __shared__ uint64_t w8[NW];
    __shared__ float wf[NW];
    __shared__ double wm[NW];
    __shared__ int nc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t item = blockIdx.x;
    const int64_t row = item / nch;
    const int c = (int)(item % nch);
    const int req = (int)(row / n);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const int64_t c0 = (int64_t)c * C, c1 = V < c0 + C ? V : c0 + C;
    Packed<DT> x;
    x.load(static_cast<const char *>(in) + row * V * eb, c0, c1, vec_ok, tid);
    const float T = temperature[req];
    const int kk = top_k[req];
    const int K = (kk >= 1 && kk < V && kk <= kCapK) ? kk : kCapK;
    const int w = (K + NW - 1) / NW;          // NW waves x w entries >= tau
    const bool need_z = top_p[req] < 1.f;

    // each thread's largest key: its max value at its first index (missing
    // entries read as -inf and come after the real ones); the chunk max
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
    const int nl = (int)(c1 - c0);
    int first = nl;
#pragma unroll
    for (int e = kPerThread - 1; e >= 0; --e)
        if (x[e] == m) first = local_index(tid, e);
    const uint64_t tk = first < nl ? order_key(m, c0 + first) : 0;
    m = wave_max(m);
    if (lane == 0) {
        wf[wave] = m;
        w8[wave] = 0;
    }
    if (tid == 0) nc = 0;
    tks[tid] = tk;
    __syncthreads();
    m = wf[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) m = fmaxf(m, wf[v]);
    // the wave's w-th largest thread maximum (keys are unique)
    {
        const uint64_t *wk = tks + wave * SPEC_WAVE;
        int r = 0;
#pragma unroll 8
        for (int u = 0; u < SPEC_WAVE; ++u) r += wk[u] > tk;
        if (tk != 0 && r == w - 1) w8[wave] = tk;
    }
    double s = 0.0;
    if (need_z && m != -INFINITY) {                // missing entries (-inf) add 0
        const Scale2 scl = make_scale2(m, T);
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) s += (double)exp2_scaled(x[e], scl);
        s = wave_sum_d(s);
    }
    if (lane == 0) wm[wave] = s;
    __syncthreads();
    uint64_t tau = w8[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) tau = w8[v] < tau ? w8[v] : tau;
    // the candidates: every entry with key >= tau (only threads whose
    // maximum reaches tau hold one)
    // tau is a real entry's key (every wave has 64 threads holding entries),
    // so a missing entry (-inf, index >= c1) is never >= tau.  Slots: a
    // count per thread, a wave prefix and one shared add per wave.
    {
        const float tv = key_value(tau);
        const int ti = (int)(key_index(tau) - c0);  // tau is an entry of this chunk
        uint32_t mine = 0;
        if (tk >= tau) {
#pragma unroll
            for (int e = 0; e < kPerThread; ++e)
                mine |= (uint32_t)at_or_above(x[e], local_index(tid, e), tv, ti) << e;
        }
        const int cntm = __popc(mine);
        int incl = cntm;
#pragma unroll
        for (int o = 1; o < SPEC_WAVE; o <<= 1) {
            const int u = __shfl_up(incl, o, SPEC_WAVE);
            if (lane >= o) incl += u;
        }
        const int wtot = __shfl(incl, SPEC_WAVE - 1, SPEC_WAVE);
        int base = 0;
        if (lane == SPEC_WAVE - 1 && wtot > 0) base = atomicAdd(&nc, wtot);
        base = __shfl(base, SPEC_WAVE - 1, SPEC_WAVE) + incl - cntm;
        if (mine != 0) {
#pragma unroll
            for (int e = 0; e < kPerThread; ++e)
                if ((mine >> e) & 1u) {
                    if (base < kChunkCand) ck[base] = order_key(x[e], c0 + local_index(tid, e));
                    ++base;
                }
        }
    }
    __syncthreads();
    // the chunk's top K in order (there are at least K candidates)
    const int cnt = nc;
    const bool over = cnt > kChunkCand || tau == 0;
    if (!over) {
        uint64_t *kout = keys + item * kCapK;
        for (int q = tid; q < cnt; q += kSweepThreads) {
            const uint64_t mine = ck[q];
            int r = 0;
#pragma unroll 8
            for (int u = 0; u < cnt; ++u) r += ck[u] > mine;
            if (r < K) kout[r] = mine;
        }
    }
    if (tid == 0) {
        double zs = 0.0;
#pragma unroll
        for (int v = 0; v < NW; ++v) zs += wm[v];
        heads[item] = ChunkHead{m, over ? 1u : 0u, zs};
    }
}

// Eight output entries from e0 (chunk end c1): 16-byte stores when aligned.
template <int DT>
__device__ __forceinline__ void store8(char *rout, int64_t e0, int64_t c1, bool vec_ok,
                                       const float (&v)[8]) {
    if (DT == SPEC_BF16) {
        uint16_t *o16 = reinterpret_cast<uint16_t *>(rout);
        uint16_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (uint16_t)(__float_as_uint(v[j]) >> 16);   // bf16 values
        if (vec_ok && e0 + 8 <= c1) {
            uint4 w;
            w.x = h[0] | ((uint32_t)h[1] << 16);
            w.y = h[2] | ((uint32_t)h[3] << 16);
            w.z = h[4] | ((uint32_t)h[5] << 16);
            w.w = h[6] | ((uint32_t)h[7] << 16);
            *reinterpret_cast<uint4 *>(o16 + e0) = w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (e0 + j < c1) o16[e0 + j] = h[j];
        }
    } else {
        float *o32 = reinterpret_cast<float *>(rout);
        if (vec_ok && e0 + 8 <= c1) {
            *reinterpret_cast<float4 *>(o32 + e0) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(o32 + e0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (e0 + j < c1) o32[e0 + j] = v[j];
        }
    }
}

// Three-launch path, output step: the same work items as the chunk step.
// Rows the row step finished itself are skipped; a row with both rules off
// is copied.  Otherwise, RD: the chunk is read again and an entry kept iff
// its key is >= the cutoff; !RD: the chunk is written as -inf except the
// row's kept entries that fall in it, whose values come from their keys
// (no read: less traffic, but a launch of stores alone was measured slower
// while the whole call is small).  out may be in.
template <int DT, bool RD>
__global__ __launch_bounds__(kSweepThreads) void filter_out_kernel(
    const void *in, void *out, int64_t V, int64_t C, bool vec_ok, int nch,
    const Decision *__restrict__ dec, const uint64_t *__restrict__ kept) {
    __shared__ int kl[kCapK];              // chunk-relative indices of the kept entries here
    __shared__ float kx[kCapK];            // their values
    __shared__ int nk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t item = blockIdx.x;
    const int64_t row = item / nch;
    const int c = (int)(item % nch);
    const size_t eb = DT == SPEC_BF16 ? 2 : 4;
    const int64_t c0 = (int64_t)c * C, c1 = V < c0 + C ? V : c0 + C;
    const Decision d = dec[row];
    // the whole kept list slot, loaded together with the decision (entries
    // past nkeep are ignored)
    uint64_t key = tid < SPEC_WAVE ? kept[row * kCapK + tid] : 0;
    if (d.mode == 1) return;
    char *rout = static_cast<char *>(out) + row * V * eb;
    if (RD || d.mode == 0) {               // mode 0: both rules off, every entry kept
        Packed<DT> x;
        x.load(static_cast<const char *>(in) + row * V * eb, c0, c1, vec_ok, tid);
        const bool all = d.mode == 0;
        const float cv = key_value(d.cutoff);
        const int64_t cd = key_index(d.cutoff) - c0;
        const int ci = cd < 0 ? -1 : (cd > kChunk ? kChunk : (int)cd);
#pragma unroll
        for (int g = 0; g < kPerThread / 8; ++g) {
            const int l0 = local_index(tid, g * 8);
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = all || at_or_above(x[g * 8 + j], l0 + j, cv, ci) ? x[g * 8 + j] : -INFINITY;
            store8<DT>(rout, c0 + l0, c1, vec_ok, v);
        }
        return;
    }
    if (tid < SPEC_WAVE) {
        key = tid < (int)d.nkeep ? key : 0;
        const int64_t i = key_index(key);
        const bool here = key != 0 && i >= c0 && i < c1;
        const uint64_t bal = __ballot(here);
        if (here) {
            const int pos = __popcll(bal & ((1ull << lane) - 1ull));
            kl[pos] = (int)(i - c0);
            float xv = key_value(key);
            // the key holds -0 as +0 (equal logits rank by index alone): a
            // kept zero takes its sign from the input, read before any store
            // of this chunk (the one workgroup that writes it), so in place
            // is safe too
            if (xv == 0.f) {
                const char *src = static_cast<const char *>(in) + (row * V + i) * eb;
                xv = DT == SPEC_BF16
                    ? spec::bf16_to_f32(*reinterpret_cast<const uint16_t *>(src))
                    : *reinterpret_cast<const float *>(src);
            }
            kx[pos] = xv;
        }
        if (tid == 0) nk = __popcll(bal);
    }
    __syncthreads();
    const int n_here = nk;
#pragma unroll
    for (int g = 0; g < kPerThread / 8; ++g) {
        const int l0 = local_index(tid, g * 8);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = -INFINITY;
        for (int t = 0; t < n_here; ++t) {
            const int dl = kl[t] - l0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (dl == j) v[j] = kx[t];
        }
        store8<DT>(rout, c0 + l0, c1, vec_ok, v);
    }
}

struct FilterWs {
    size_t dec, heads, keys, kept, total;
};

FilterWs filter_ws(int64_t rows, int nch) {
    FilterWs w{};
    w.dec = 0;
    w.heads = align_up((size_t)rows * sizeof(Decision), 256);
    w.keys = w.heads + align_up((size_t)rows * nch * sizeof(ChunkHead), 256);
    w.kept = w.keys + align_up((size_t)rows * nch * kCapK * sizeof(uint64_t), 256);
    w.total = w.kept + align_up((size_t)rows * kCapK * sizeof(uint64_t), 256);
    return w;
}

template <int DT, int KEYBITS>
void launch_filter(const void *logits, void *out, int64_t V, bool vec_ok, int n, int64_t rows,
                   const float *temperature, const int32_t *top_k, const float *top_p, int nch,
                   void *workspace, hipStream_t st) {
    if (nch == 0) {
        hipLaunchKernelGGL((filter_row_kernel<DT, KEYBITS>), dim3((unsigned)rows), dim3(kRT), 0, st,
                           logits, out, V, vec_ok, n, temperature, top_k, top_p,
                           (const ChunkHead *)nullptr, (const uint64_t *)nullptr, 0,
                           (Decision *)nullptr, (uint64_t *)nullptr);
        return;
    }
    const FilterWs w = filter_ws(rows, nch);
    char *ws = static_cast<char *>(workspace);
    Decision *dec = reinterpret_cast<Decision *>(ws + w.dec);
    ChunkHead *heads = reinterpret_cast<ChunkHead *>(ws + w.heads);
    uint64_t *keys = reinterpret_cast<uint64_t *>(ws + w.keys);
    uint64_t *kept = reinterpret_cast<uint64_t *>(ws + w.kept);
    const int64_t C = filter_chunk_size(V, nch);
    const unsigned items = (unsigned)(rows * nch);
    hipLaunchKernelGGL((filter_chunk_kernel<DT>), dim3(items), dim3(kSweepThreads), 0, st, logits, V,
                       C, vec_ok, n, nch, temperature, top_k, top_p, heads, keys);
    hipLaunchKernelGGL((filter_row_kernel<DT, KEYBITS>), dim3((unsigned)rows), dim3(kRT), 0, st,
                       logits, out, V, vec_ok, n, temperature, top_k, top_p,
                       (const ChunkHead *)heads, (const uint64_t *)keys, nch, dec, kept);
    if ((int64_t)rows * V * (DT == SPEC_BF16 ? 2 : 4) <= kReadOutBytes)
        hipLaunchKernelGGL((filter_out_kernel<DT, true>), dim3(items), dim3(kSweepThreads), 0, st,
                           logits, out, V, C, vec_ok, nch, (const Decision *)dec,
                           (const uint64_t *)kept);
    else
        hipLaunchKernelGGL((filter_out_kernel<DT, false>), dim3(items), dim3(kSweepThreads), 0, st,
                           logits, out, V, C, vec_ok, nch, (const Decision *)dec,
                           (const uint64_t *)kept);
}

}  // namespace

extern "C" size_t spec_sampling_filter_workspace_size(int batch, int num_draft_tokens,
                                                      int64_t vocab) {
    if (batch <= 0 || num_draft_tokens < 1 || vocab < 1 || vocab > INT_MAX) return 0;
    const int64_t rows = (int64_t)batch * num_draft_tokens;
    const int nch = filter_chunks(rows, vocab);
    return nch == 0 ? 0 : filter_ws(rows, nch).total;
}

extern "C" int spec_sampling_filter(int batch, int num_draft_tokens, int64_t vocab, int dtype,
                                    const void *logits, const float *temperature,
                                    const int32_t *top_k, const float *top_p, void *out,
                                    void *workspace, size_t workspace_bytes,
                                    int32_t *dev_status, spec_stream_t stream) {
    (void)dev_status;
    if (batch < 0 || num_draft_tokens < 1 || vocab < 1) return SPEC_ERR_SHAPE;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if (vocab > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!logits || !temperature || !top_k || !top_p || !out) return SPEC_ERR_NULL;
    const int64_t rows = (int64_t)batch * num_draft_tokens;
    if (rows > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 &&
                        ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(out)) & 15u) == 0;
    const int nch = filter_chunks(rows, vocab);
    if (nch > 0) {
        const size_t need = filter_ws(rows, nch).total;
        if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return SPEC_ERR_WORKSPACE;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        launch_filter<SPEC_BF16, 16>(logits, out, vocab, vec_ok, num_draft_tokens, rows, temperature,
                                     top_k, top_p, nch, workspace, st);
    else
        launch_filter<SPEC_F32, 32>(logits, out, vocab, vec_ok, num_draft_tokens, rows, temperature,
                                    top_k, top_p, nch, workspace, st);
    return spec::launch_status();
}
