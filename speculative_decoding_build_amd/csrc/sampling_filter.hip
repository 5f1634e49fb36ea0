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
// value bits (16 for bf16, 32 for float), 8 bits per level, over chunks of
// 8192 entries:
//   launch 1: chunk maxima;
//   launch 2: each chunk's sum of exponentials and a 256-bin histogram (count,
//     float64 mass) of the first key byte;
//   launch 3 (and 4, 5 for float): every chunk workgroup merges the row's
//     previous-level histograms in a fixed order (so all of them agree),
//     finds the bin where the kept set ends (the first bin, from the top,
//     where the count reaches top_k or the mass reaches top_p * Z), and
//     histograms the next byte of the entries in that bin;
//   launch 4: the last merge fixes the cutoff value v and how many of the
//     entries equal to v are kept (those of lowest index); each chunk counts
//     its entries equal to v;
//   launch 5: each chunk ranks its entries equal to v in index order after
//     the earlier chunks' and writes the output.
// Exponentials are the float-pair base-2 exponential used by the accept
// sweeps; masses are float64 sums.
#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kBins = 256;
constexpr int kMaxChunks = 64;             // vocab <= 524288
constexpr int kWaves = kSweepThreads / SPEC_WAVE;

// Per row, after each level's merge.
struct State {
    uint32_t prefix;                       // key bits fixed so far
    uint32_t count_before;                 // entries above the current bin
    double mass_before;                    // their mass (unnormalised)
    double tpz;                            // top_p * Z (or +inf when top-p is off)
    float m;                               // row max
    int keep_all;                          // no cutoff: every entry kept
    uint32_t n_tie;                        // entries equal to the cutoff value
    uint32_t keep_tie;                     // of those, kept (lowest indices first)
};

struct FilterArgs {
    const void *in;                        // [rows][vocab]
    void *out;                             // [rows][vocab]
    int64_t vocab;
    bool vec_ok;
    int rows, n, nchunks, levels, key_bits;
    const float *temperature;              // [batch]
    const int32_t *top_k;                  // [batch]
    const float *top_p;                    // [batch]
    float *cmax;                           // [rows][nchunks]
    double *csum;                          // [rows][nchunks]
    uint32_t *hcnt;                        // [2][rows][nchunks][kBins]
    double *hmass;                         // [2][rows][nchunks][kBins]
    uint32_t *ties;                        // [rows][nchunks]
    State *state;                          // [2][rows], alternating between launches
    int32_t *status;
};


__device__ __forceinline__ uint32_t value_key(float v) {
    uint32_t bits = __float_as_uint(v == 0.f ? 0.f : v);
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

// key restricted to the searched bits (bf16: the upper 16)
__device__ __forceinline__ uint32_t search_key(float v, int key_bits) {
    return value_key(v) >> (32 - key_bits);
}

__device__ __forceinline__ int row_topk(const FilterArgs &A, int row) {
    const int k = A.top_k[row / A.n];
    return (k >= 1 && k < A.vocab) ? k : 0;
}

__device__ __forceinline__ double row_topp(const FilterArgs &A, int row) {
    const float p = A.top_p[row / A.n];
    return p < 1.f ? (double)p : 2.0;
}

template <int DT>
__device__ __forceinline__ void load_row_chunk(const FilterArgs &A, int row, int64_t start,
                                               int64_t end, int tid, float (&x)[kPerThread]) {
    load_chunk<DT>(static_cast<const char *>(A.in) + (int64_t)row * A.vocab * (DT == SPEC_BF16 ? 2 : 4),
                   start, end, A.vec_ok, tid, x);
}

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void filter_max_kernel(FilterArgs A) {
    __shared__ float s_f[kWaves];
    const int tid = threadIdx.x;
    const int row = blockIdx.x / A.nchunks, c = blockIdx.x % A.nchunks;
    const int64_t start = (int64_t)c * kChunk, end = min(A.vocab, start + kChunk);
    float x[kPerThread];
    load_row_chunk<DT>(A, row, start, end, tid, x);
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
    m = wave_max(m);
    if ((tid & 63) == 0) s_f[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        float r = s_f[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) r = fmaxf(r, s_f[w]);
        A.cmax[blockIdx.x] = r;
    }
}

struct HistShared {
    uint32_t cnt[kWaves][kBins];
    double mass[kWaves][kBins];
};

// Per-wave histograms of `digit` (only entries with in_bin) into LDS, then
// the chunk's histogram to global level buffer `lvl`.
__device__ void write_histogram(const FilterArgs &A, HistShared &H, int lvl, int64_t item,
                                const uint32_t (&digit)[kPerThread], const bool (&in_bin)[kPerThread],
                                const float (&ev)[kPerThread]) {
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int i = tid; i < kWaves * kBins; i += kSweepThreads) {
        (&H.cnt[0][0])[i] = 0;
        (&H.mass[0][0])[i] = 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        if (in_bin[e]) {
            atomicAdd(&H.cnt[wave][digit[e]], 1u);
            atomicAdd(&H.mass[wave][digit[e]], (double)ev[e]);
        }
    }
    __syncthreads();
    const int64_t base = ((int64_t)lvl * A.rows * A.nchunks + item) * kBins;
    for (int b = tid; b < kBins; b += kSweepThreads) {
        uint32_t cn = 0;
        double ms = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            cn += H.cnt[w][b];
            ms += H.mass[w][b];
        }
        A.hcnt[base + b] = cn;
        A.hmass[base + b] = ms;
    }
}

// The row's max from the chunk maxima (every thread).
__device__ __forceinline__ float row_max(const FilterArgs &A, int row) {
    float m = -INFINITY;
    for (int c = 0; c < A.nchunks; ++c) m = fmaxf(m, A.cmax[(int64_t)row * A.nchunks + c]);
    return m;
}

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void filter_level1_kernel(FilterArgs A) {
    __shared__ HistShared H;
    __shared__ double s_d[kWaves];
    const int tid = threadIdx.x;
    const int row = blockIdx.x / A.nchunks, c = blockIdx.x % A.nchunks;
    const int64_t start = (int64_t)c * kChunk, end = min(A.vocab, start + kChunk);
    float x[kPerThread];
    load_row_chunk<DT>(A, row, start, end, tid, x);
    const float m = row_max(A, row);
    const Scale2 scl = make_scale2(m, A.temperature[row / A.n]);
    float ev[kPerThread];
    uint32_t digit[kPerThread];
    bool in_bin[kPerThread];
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const bool ok = elem_index(start, tid, e) < end;
        ev[e] = (ok && m != -INFINITY) ? exp2_scaled(x[e], scl) : 0.f;
        s += (double)ev[e];
        digit[e] = search_key(x[e], A.key_bits) >> (A.key_bits - 8);
        in_bin[e] = ok;
    }
    s = wave_sum_d(s);
    if ((tid & 63) == 0) s_d[tid >> 6] = s;
    write_histogram(A, H, 0, blockIdx.x, digit, in_bin, ev);
    if (tid == 0) {
        double z = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) z += s_d[w];
        A.csum[blockIdx.x] = z;
    }
}

struct MergeShared {
    uint32_t cnt[kBins];
    double mass[kBins];
    uint32_t sc[kWaves];
    double sm[kWaves];
    int pick;
};

// Merge level `lvl` of the row's chunk histograms (fixed order), find the
// bin where the kept set ends; updates st (every thread holds the same).
// Returns false when no bin ends it (every entry of the current prefix is
// kept).
__device__ bool merge_level(const FilterArgs &A, MergeShared &M, int lvl, int row, State &st) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k = row_topk(A, row);
    // thread b holds bin b (kBins == threads)
    uint32_t cn = 0;
    double ms = 0.0;
    const int64_t base = ((int64_t)lvl * A.rows + row) * A.nchunks * kBins;
    for (int c = 0; c < A.nchunks; ++c) {
        cn += A.hcnt[base + (int64_t)c * kBins + tid];
        ms += A.hmass[base + (int64_t)c * kBins + tid];
    }
    // entries in bins above b: a suffix sum (bins descending), wave scans
    // then the waves above
    uint32_t ic = cn;
    double im = ms;
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
        M.sc[wave] = ic;                  // inclusive suffix of the wave = its total
        M.sm[wave] = im;
    }
    if (tid == 0) M.pick = -1;
    __syncthreads();
    uint32_t above_c = ic - cn;
    double above_m = im - ms;
    for (int w = wave + 1; w < kWaves; ++w) {
        above_c += M.sc[w];
        above_m += M.sm[w];
    }
    const bool hit = (cn > 0) && ((k > 0 && st.count_before + above_c + cn >= (uint32_t)k) ||
                                  (st.mass_before + above_m + ms >= st.tpz));
    // the highest bin that ends the kept set
    if (hit) atomicMax(&M.pick, tid);
    __syncthreads();
    const int pick = M.pick;
    if (pick < 0) return false;
    if (tid == pick) {
        M.cnt[0] = above_c;
        M.mass[0] = above_m;
        M.cnt[1] = cn;
        M.mass[1] = ms;
    }
    __syncthreads();
    st.count_before += M.cnt[0];
    st.mass_before += M.mass[0];
    st.prefix = (st.prefix << 8) | (uint32_t)pick;
    st.n_tie = M.cnt[1];
    __syncthreads();
    return true;
}

// The row state before the first merge (every thread).
__device__ void initial_state(const FilterArgs &A, int row, State &st) {
    st.prefix = 0;
    st.count_before = 0;
    st.mass_before = 0.0;
    double z = 0.0;
    for (int c = 0; c < A.nchunks; ++c) z += A.csum[(int64_t)row * A.nchunks + c];
    const double tp = row_topp(A, row);
    st.tpz = tp < 1.0 ? tp * z : INFINITY;
    st.m = row_max(A, row);
    st.keep_all = 0;
    st.n_tie = 0;
    st.keep_tie = 0;
}

// Level l >= 2: merge level l-1, then histogram the next byte of the
// entries in the picked bin.
template <int DT>
__global__ __launch_bounds__(kSweepThreads) void filter_level_kernel(FilterArgs A, int level) {
    __shared__ HistShared H;
    __shared__ MergeShared M;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / A.nchunks, c = blockIdx.x % A.nchunks;
    // the state record this launch reads is not the one it writes
    State st;
    if (level == 2)
        initial_state(A, row, st);
    else
        st = A.state[(int64_t)(level & 1) * A.rows + row];
    if (!st.keep_all && !merge_level(A, M, (level - 2) & 1, row, st)) st.keep_all = 1;
    if (c == 0 && tid == 0) A.state[(int64_t)((level + 1) & 1) * A.rows + row] = st;
    if (st.keep_all) return;               // uniform over the workgroup
    const int64_t start = (int64_t)c * kChunk, end = min(A.vocab, start + kChunk);
    float x[kPerThread];
    load_row_chunk<DT>(A, row, start, end, tid, x);
    const Scale2 scl = make_scale2(st.m, A.temperature[row / A.n]);
    float ev[kPerThread];
    uint32_t digit[kPerThread];
    bool in_bin[kPerThread];
    const int shift = A.key_bits - 8 * level;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const uint32_t key = search_key(x[e], A.key_bits);
        in_bin[e] = elem_index(start, tid, e) < end && (key >> (shift + 8)) == st.prefix;
        digit[e] = (key >> shift) & 0xFFu;
        ev[e] = in_bin[e] ? exp2_scaled(x[e], scl) : 0.f;
    }
    write_histogram(A, H, (level - 1) & 1, blockIdx.x, digit, in_bin, ev);
}

// Last merge: the cutoff value and how many of its entries are kept; each
// chunk counts its entries equal to it.
template <int DT>
__global__ __launch_bounds__(kSweepThreads) void filter_ties_kernel(FilterArgs A) {
    __shared__ MergeShared M;
    __shared__ uint32_t s_c[kWaves];
    const int tid = threadIdx.x;
    const int row = blockIdx.x / A.nchunks, c = blockIdx.x % A.nchunks;
    State st = A.state[(int64_t)((A.levels + 1) & 1) * A.rows + row];
    if (!st.keep_all) {
        if (!merge_level(A, M, (A.levels - 1) & 1, row, st)) {
            st.keep_all = 1;
        } else {
            // entries equal to v: tie i (index order) is kept iff the count
            // above plus i stays below top_k and the mass above plus i
            // times the entry's mass stays below top_p * Z
            uint32_t keep = st.n_tie;
            const int k = row_topk(A, row);
            if (k > 0) keep = min(keep, (uint32_t)k - st.count_before);
            if (st.tpz < INFINITY) {
                const uint32_t vbits = st.prefix << (32 - A.key_bits);
                const uint32_t fb = (vbits & 0x80000000u) ? (vbits & 0x7FFFFFFFu) : ~vbits;
                const float ev = exp2_scaled(__uint_as_float(fb),
                                             make_scale2(st.m, A.temperature[row / A.n]));
                uint32_t cp = st.n_tie;
                if (ev > 0.f) {
                    const double q = (st.tpz - st.mass_before) / (double)ev;
                    cp = q <= 0.0 ? 0u : (q >= (double)st.n_tie ? st.n_tie : (uint32_t)ceil(q));
                    // settle the rounding of the quotient on the exact rule
                    while (cp > 0 && st.mass_before + (double)(cp - 1) * ev >= st.tpz) --cp;
                    while (cp < st.n_tie && st.mass_before + (double)cp * ev < st.tpz) ++cp;
                }
                keep = min(keep, cp);
            }
            st.keep_tie = keep;
        }
    }
    if (c == 0 && tid == 0) A.state[(int64_t)((A.levels + 2) & 1) * A.rows + row] = st;
    if (st.keep_all) return;
    const int64_t start = (int64_t)c * kChunk, end = min(A.vocab, start + kChunk);
    float x[kPerThread];
    load_row_chunk<DT>(A, row, start, end, tid, x);
    uint32_t t = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
        t += elem_index(start, tid, e) < end && search_key(x[e], A.key_bits) == st.prefix;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, SPEC_WAVE);
    if ((tid & 63) == 0) s_c[tid >> 6] = t;
    __syncthreads();
    if (tid == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) r += s_c[w];
        A.ties[blockIdx.x] = r;
    }
}

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void filter_write_kernel(FilterArgs A) {
    __shared__ uint32_t s_w[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x / A.nchunks, c = blockIdx.x % A.nchunks;
    const State st = A.state[(int64_t)((A.levels + 2) & 1) * A.rows + row];
    const int64_t start = (int64_t)c * kChunk, end = min(A.vocab, start + kChunk);
    float x[kPerThread];
    load_row_chunk<DT>(A, row, start, end, tid, x);
    // ties of the earlier chunks
    uint32_t rank0 = 0;
    if (!st.keep_all)
        for (int cc = 0; cc < c; ++cc) rank0 += A.ties[(int64_t)row * A.nchunks + cc];
    const bool need_rank = !st.keep_all && st.keep_tie < st.n_tie;
    char *orow = static_cast<char *>(A.out) + (int64_t)row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
    // groups of 8 entries per thread (index order: group, thread, entry)
#pragma unroll
    for (int g = 0; g < kPerThread / 8; ++g) {
        bool keep[8];
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = g * 8 + j;
            const uint32_t key = search_key(x[e], A.key_bits);
            const bool tie = !st.keep_all && key == st.prefix && elem_index(start, tid, e) < end;
            keep[j] = st.keep_all || key > st.prefix || (tie && !need_rank);
            mine += tie;
        }
        if (need_rank) {
            // exclusive scan of the ties over (thread) in this group
            uint32_t incl = mine;
#pragma unroll
            for (int o = 1; o < SPEC_WAVE; o <<= 1) {
                const uint32_t v = __shfl_up(incl, o, SPEC_WAVE);
                if (lane >= o) incl += v;
            }
            if (lane == 63) s_w[wave] = incl;
            __syncthreads();
            uint32_t before = rank0 + incl - mine;
            uint32_t total = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                if (w < wave) before += s_w[w];
                total += s_w[w];
            }
            __syncthreads();
            uint32_t r = before;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int e = g * 8 + j;
                const bool tie = search_key(x[e], A.key_bits) == st.prefix &&
                                 elem_index(start, tid, e) < end;
                if (tie) {
                    keep[j] = r < st.keep_tie;
                    ++r;
                }
            }
            rank0 += total;
        }
        const int64_t e0 = elem_index(start, tid, g * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (e0 + j < end) {
                if (DT == SPEC_BF16) {
                    const uint16_t bits = keep[j] ? (uint16_t)(__float_as_uint(x[g * 8 + j]) >> 16)
                                                  : (uint16_t)0xFF80u;
                    reinterpret_cast<uint16_t *>(orow)[e0 + j] = bits;
                } else {
                    reinterpret_cast<float *>(orow)[e0 + j] = keep[j] ? x[g * 8 + j] : -INFINITY;
                }
            }
        }
    }
}

size_t align8k(size_t x) { return spec::align_up(x, 256); }

struct Layout {
    size_t cmax, csum, hcnt, hmass, ties, state, total;
};

Layout layout(int rows, int nch) {
    Layout L;
    size_t off = 0;
    L.cmax = off;  off += align8k((size_t)rows * nch * 4);
    L.csum = off;  off += align8k((size_t)rows * nch * 8);
    L.hcnt = off;  off += align8k((size_t)2 * rows * nch * kBins * 4);
    L.hmass = off; off += align8k((size_t)2 * rows * nch * kBins * 8);
    L.ties = off;  off += align8k((size_t)rows * nch * 4);
    L.state = off; off += align8k((size_t)2 * rows * sizeof(State));
    L.total = off;
    return L;
}

template <int DT>
void launch_all(const FilterArgs &A, hipStream_t st) {
    const dim3 g((unsigned)(A.rows * A.nchunks)), b(kSweepThreads);
    hipLaunchKernelGGL(filter_max_kernel<DT>, g, b, 0, st, A);
    hipLaunchKernelGGL(filter_level1_kernel<DT>, g, b, 0, st, A);
    for (int level = 2; level <= A.levels; ++level)
        hipLaunchKernelGGL(filter_level_kernel<DT>, g, b, 0, st, A, level);
    hipLaunchKernelGGL(filter_ties_kernel<DT>, g, b, 0, st, A);
    hipLaunchKernelGGL(filter_write_kernel<DT>, g, b, 0, st, A);
}

}  // namespace

extern "C" size_t spec_sampling_filter_workspace_size(int batch, int num_draft_tokens,
                                                      int64_t vocab) {
    if (batch <= 0 || num_draft_tokens <= 0 || vocab <= 0) return 0;
    return layout(batch * num_draft_tokens, num_chunks(vocab)).total;
}

extern "C" int spec_sampling_filter(int batch, int num_draft_tokens, int64_t vocab, int dtype,
                                    const void *logits, const float *temperature,
                                    const int32_t *top_k, const float *top_p, void *out,
                                    void *workspace, size_t workspace_bytes, int32_t *dev_status,
                                    spec_stream_t stream) {
    if (batch < 0 || num_draft_tokens < 1 || vocab < 1) return SPEC_ERR_SHAPE;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    const int nch = num_chunks(vocab);
    if (nch > kMaxChunks) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!logits || !temperature || !top_k || !top_p || !out) return SPEC_ERR_NULL;
    const int64_t rows = (int64_t)batch * num_draft_tokens;
    if (rows * nch > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    const Layout L = layout((int)rows, nch);
    if (!workspace || workspace_bytes < L.total || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return SPEC_ERR_WORKSPACE;
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    char *ws = static_cast<char *>(workspace);
    FilterArgs A{};
    A.in = logits;
    A.out = out;
    A.vocab = vocab;
    A.vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
    A.rows = (int)rows;
    A.n = num_draft_tokens;
    A.nchunks = nch;
    A.key_bits = dtype == SPEC_BF16 ? 16 : 32;
    A.levels = A.key_bits / 8;
    A.temperature = temperature;
    A.top_k = top_k;
    A.top_p = top_p;
    A.cmax = reinterpret_cast<float *>(ws + L.cmax);
    A.csum = reinterpret_cast<double *>(ws + L.csum);
    A.hcnt = reinterpret_cast<uint32_t *>(ws + L.hcnt);
    A.hmass = reinterpret_cast<double *>(ws + L.hmass);
    A.ties = reinterpret_cast<uint32_t *>(ws + L.ties);
    A.state = reinterpret_cast<State *>(ws + L.state);
    A.status = dev_status;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        launch_all<SPEC_BF16>(A, st);
    else
        launch_all<SPEC_F32>(A, st);
    return spec::launch_status();
}
