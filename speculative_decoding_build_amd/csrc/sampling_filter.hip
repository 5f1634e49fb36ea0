// Sampling-parameter pre-pass: top-k / top-p filtering of the target
// distribution before the sampled accepts.
//
// "投机解码 Accept:从 Verify 行到最终输出路径" (四: eagle_sample takes the
// target softmax at the request's temperature, then top-k / top-p filtering
// and renormalisation) and "SGLang 源码完全拆解(十一):投机解码" (三条判定路径).
// Row i belongs to request i / n.  p = softmax(x / T); entries rank by p
// descending (logit descending), lower index first; the entry of rank r is
// kept iff r < top_k (when 1 <= top_k < V) and the mass of the entries
// ranked above it is < top_p (when top_p < 1).  Kept logits are copied,
// the others become -inf, so softmax(out / T) is the renormalised
// distribution the accepts read.  A greedy request is top_k = 1.
//
// The kept set is {key >= kappa} for the 64-bit order key (value bits, then
// the complemented index), found without sorting by a radix search on the
// value bits, one 1024-thread workgroup per row:
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

constexpr int kCand = 1024;                // candidates the fast path ranks
constexpr int kWaveTop = 8;                // tau: the least of the waves' 8th largest thread maxima

struct RowShared {
    union {
        struct {
            uint32_t cnt[kMaxBins];
            double mass[kMaxBins];
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
__device__ void above_sums(RowShared &S, uint32_t c, double m, uint32_t &ac, double &am) {
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
__device__ int find_cut(RowShared &S, int nb, int k, double tpz, uint32_t cb, double mb,
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

template <int DT, int KEYBITS>
__global__ __launch_bounds__(kRT) void filter_row_kernel(
    const void *in, void *out, int64_t V, bool vec_ok, int n,
    const float *__restrict__ temperature, const int32_t *__restrict__ top_k,
    const float *__restrict__ top_p) {
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

    // pass 1: the row max and each thread's largest 64-bit key (value
    // bits, then the complemented index: unique, larger = ranked higher)
    float m = -INFINITY;
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
    const Scale2 scl = make_scale2(m, T);
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
    double z = 0.0;
    for (int64_t t0 = 0; t0 < V; t0 += kTile) {
        const int64_t i0 = t0 + tid * 8;
        load8<DT>(rin, i0, V, vec_ok, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (i0 + j < V) {
                const float e = m == -INFINITY ? 0.f : exp2_scaled(x[j], scl);
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
    const int nc = S.nc;
    __syncthreads();
    const double tpz = tpf < 1.f ? (double)tpf * z : INFINITY;

    // fast path: the candidates are the top nc entries of the row; when the
    // kept set ends among them its last entry's key is the cutoff
    bool fast = false, keep_all = k == 0 && !(tpz < INFINITY);
    uint64_t cutoff = 0;
    if (!keep_all && nc <= kCand) {
        for (int q = tid; q < nc; q += kRT) {
            const uint64_t mine = S.ck[q];
            int r = 0;
            for (int u = 0; u < nc; ++u) r += S.ck[u] > mine;
            S.sk[r] = mine;
            S.sm[r] = S.cm[q];
        }
        __syncthreads();
        // inclusive mass by rank (thread t holds rank t), then the last kept
        // rank: min(top_k - 1, the first rank whose inclusive mass reaches
        // top_p * Z)
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
        if (rstar < nc) {
            fast = true;
            cutoff = S.sk[rstar];
        } else if (nc == V) {
            fast = true;
            keep_all = true;
        }
        __syncthreads();
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

}  // namespace

extern "C" int spec_sampling_filter(int batch, int num_draft_tokens, int64_t vocab, int dtype,
                                    const void *logits, const float *temperature,
                                    const int32_t *top_k, const float *top_p, void *out,
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
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        hipLaunchKernelGGL((filter_row_kernel<SPEC_BF16, 16>), dim3((unsigned)rows), dim3(kRT), 0, st,
                           logits, out, vocab, vec_ok, num_draft_tokens, temperature, top_k, top_p);
    else
        hipLaunchKernelGGL((filter_row_kernel<SPEC_F32, 32>), dim3((unsigned)rows), dim3(kRT), 0, st,
                           logits, out, vocab, vec_ok, num_draft_tokens, temperature, top_k, top_p);
    return spec::launch_status();
}
