// Draft step: one call of select_top_k_tokens for a batch.
//
// Follows "SGLang 源码完全拆解(十一):投机解码" (organize_draft_results and the
// select_top_k_tokens it reads): every live branch has a draft distribution
// p = softmax(logits); the step takes its top-k (tokens and float32
// probabilities).  Step 0 (the root's single branch) records scores = those
// probabilities, tokens = those ids and the parent block arange(-1, topk).
// A later step multiplies each branch's path score by its top-k
// probabilities (float32 products, topk x topk of them), records all
// products and ids, keeps the top-k products and records their flat indices
// plus topk*topk*(step-1) + topk as the parent block; the kept products and
// ids are the next step's branch scores and input tokens.  Blocks go to the
// offsets organize_draft_results expects (scores / tokens: 0, then
// topk + (step-1) topk^2; parents: 0, then topk + 1 + (step-1) topk; the
// last step's parent block is not part of the list).  Ties rank the lower
// index first.
//
// Two launches.  In the first, each workgroup takes one (branch row,
// chunk) item, a chunk being 2048 or 8192 vocabulary entries (the smaller
// when the grid would otherwise leave most of the device idle), and writes
// the chunk's max, its float64 sum of exponentials (float32 base-2
// exponentials of the argument carried as a float pair) and its top-k
// entries as 64-bit order keys (the logit's order-preserving bits, then the
// complemented index: a larger key is a larger logit, or the lower index of
// equal logits; logit order is probability order).  The top-k needs no
// per-element sort: with tau the k-th largest of the threads' maxima, only
// the k threads whose maximum reaches tau can hold entries >= tau, and
// every top-k entry is >= tau, so the at most k x (entries per thread)
// candidates >= tau are ranked among themselves.  In the second launch one
// workgroup per request merges the request's chunks the same way (per row,
// tau = the k-th largest chunk best: at most k x k candidates), forms each
// row's max and normaliser, the probabilities of the kept entries (float64
// exponential, rounded to float32), then the step's products and selection.
#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / SPEC_WAVE;
constexpr int kMaxK = 8;                   // topk at most
constexpr int kItemWords = 2 + kMaxK;      // per chunk item: max, sum, keys (descending)
constexpr int kMergePer = 8;               // chunk items per merge thread, separate launch
constexpr int kMergeChunks = kMergePer * kThreads;   // rows x chunks of one request
constexpr int kSmallE = 8;                 // entries per thread of a 2048-entry chunk
constexpr int kLargeE = 32;                // ... of an 8192-entry chunk
constexpr int64_t kSmallGrid = 2048;       // largest grid of 2048-entry chunks

__device__ __forceinline__ uint64_t order_key(float v, int64_t i) {
    uint32_t bits = __float_as_uint(v == 0.f ? 0.f : v);
    bits = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    return ((uint64_t)bits << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ float key_value(uint64_t k) {
    uint32_t bits = (uint32_t)(k >> 32);
    bits = (bits & 0x80000000u) ? (bits & 0x7FFFFFFFu) : ~bits;
    return __uint_as_float(bits);
}

__device__ __forceinline__ int key_index(uint64_t k) {
    return (int)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ void put(uint64_t *p, uint64_t v) { *p = v; }

struct DraftArgs {
    const void *logits;                    // [batch][rows][vocab]
    int64_t vocab;
    bool vec_ok;
    int batch, topk, num_steps, step, rows, nchunks, ncand, npar;
    const float *branch_scores;            // [batch][topk] (step >= 1)
    float *scores;                         // [batch][ncand]
    int32_t *tokens;                       // [batch][ncand]
    int32_t *parents;                      // [batch][npar]
    float *next_scores;                    // [batch][topk]
    int32_t *next_tokens;                  // [batch][topk]
    uint64_t *items;                       // [batch][rows][nchunks][kItemWords]
    int32_t *status;
};

// Element e of thread tid sits at start + (e / 8) * 2048 + tid * 8 + e % 8:
// each 8-group is one 16-byte load (bf16), a wave reads 1 KB contiguous.
__device__ __forceinline__ int64_t elem_at(int64_t start, int tid, int e) {
    return start + (int64_t)(e / 8) * kThreads * 8 + tid * 8 + (e % 8);
}

template <int DT, int E>
__device__ __forceinline__ void load_elems(const void *base, int64_t start, int64_t end,
                                           bool vec_ok, int tid, float (&x)[E]) {
#pragma unroll
    for (int g = 0; g < E / 8; ++g) {
        const int64_t e0 = elem_at(start, tid, g * 8);
        if (DT == SPEC_BF16) {
            const uint16_t *p = static_cast<const uint16_t *>(base);
            if (vec_ok && e0 + 8 <= end) {
                const uint4 w = *reinterpret_cast<const uint4 *>(p + e0);
                x[g * 8 + 0] = lo_bf16(w.x);
                x[g * 8 + 1] = hi_bf16(w.x);
                x[g * 8 + 2] = lo_bf16(w.y);
                x[g * 8 + 3] = hi_bf16(w.y);
                x[g * 8 + 4] = lo_bf16(w.z);
                x[g * 8 + 5] = hi_bf16(w.z);
                x[g * 8 + 6] = lo_bf16(w.w);
                x[g * 8 + 7] = hi_bf16(w.w);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[g * 8 + j] = (e0 + j < end) ? bf16_to_f32(p[e0 + j]) : -INFINITY;
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

constexpr int kRegPer = 2;                 // register path: up to kRegPer x 256 chunk items a request
constexpr int kRegChunks = kRegPer * kThreads;
constexpr int kMT = 512;                   // threads of a merge workgroup (one item each in registers)
constexpr int kMW = kMT / SPEC_WAVE;

struct ChunkShared {
    uint64_t tkey[kThreads];               // thread maxima
    uint64_t cand[kThreads];               // candidates (at most k x E <= 256)
    uint64_t wtop[kWaves][kMaxK];          // each wave's top-k thread maxima
    double dred[kWaves];
    uint64_t tau, best;
    int nc;
};

template <int CAP>
struct MergeShared {
    uint64_t bk[CAP];                      // chunk bests (their values: the chunk maxima)
    double cs[CAP];                        // chunk sums
    uint64_t rc[kMaxK][kMaxK * kMaxK];     // each row's candidates
    uint64_t sel[kMaxK][kMaxK];            // each row's top-k keys by rank
    uint64_t rtau[kMaxK];
    double Z[kMaxK];                       // each row's normaliser
    float M[kMaxK];                        // each row's max
    float ex[SPEC_WAVE];                   // the step's products
    float bs[SPEC_WAVE];                   // their branch scores
    int rn[kMaxK];
};

// Number of entries of u[0, n) greater than `mine` (LDS, 8 reads in flight).
__device__ __forceinline__ int count_greater(const uint64_t *u, int n, uint64_t mine) {
    int c = 0, i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = u[i + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) c += v[k] > mine;
    }
    for (; i < n; ++i) c += u[i] > mine;
    return c;
}

// One (branch row, chunk) item: max, sum and top-k keys into its slot.
template <int DT, int E>
__device__ void chunk_item(const DraftArgs &A, ChunkShared &S, int64_t t) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = A.topk;
    const int64_t row = t / A.nchunks;     // request * rows + branch
    const int64_t start = (t % A.nchunks) * (int64_t)(kThreads * E);
    const int64_t end = min(A.vocab, start + kThreads * E);
    float x[E];
    load_elems<DT, E>(static_cast<const char *>(A.logits) + row * A.vocab * (DT == SPEC_BF16 ? 2 : 4),
                      start, end, A.vec_ok, tid, x);
    // this thread's largest key: its max value at its lowest index (0: no entry)
    float vm = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) vm = fmaxf(vm, x[e]);
    int first = -1;
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
        if (elem_at(start, tid, e) < end && x[e] == vm) first = e;
    const uint64_t mk = first >= 0 ? order_key(vm, elem_at(start, tid, first)) : 0;
    S.tkey[tid] = mk;
    if (tid < kWaves * kMaxK) S.wtop[tid / kMaxK][tid % kMaxK] = 0;
    if (tid == 0) {
        S.nc = 0;
        S.tau = 1;                         // every entry, until a k-th thread maximum exists
    }
    __syncthreads();
    // the wave's top-k thread maxima, then the block's among those
    const int wr = count_greater(S.tkey + wave * SPEC_WAVE, SPEC_WAVE, mk);
    const bool wtop = mk != 0 && wr < K;
    if (wtop) S.wtop[wave][wr] = mk;
    __syncthreads();
    if (wtop) {
        const int br = count_greater(&S.wtop[0][0], kWaves * kMaxK, mk);
        if (br == 0) S.best = mk;
        if (br == K - 1) S.tau = mk;
    }
    __syncthreads();
    const uint64_t tau = S.tau;
    const float m = key_value(S.best);
    if (mk >= tau) {
        // only the k threads whose maximum reaches tau hold candidates
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t idx = elem_at(start, tid, e);
            const uint64_t k = idx < end ? order_key(x[e], idx) : 0;
            if (k >= tau) S.cand[atomicAdd(&S.nc, 1)] = k;
        }
    }
    double s = 0.0;
    if (m != -INFINITY) {
        const Scale2 scl = make_scale2(m, 1.0f);
#pragma unroll
        for (int e = 0; e < E; ++e) s += (double)exp2_scaled(x[e], scl);
    }
    s = wave_sum_d(s);
    if (lane == 0) S.dred[wave] = s;
    __syncthreads();
    const int nc = S.nc;
    uint64_t *it = A.items + t * kItemWords;
    if (tid < nc) {
        const uint64_t mine = S.cand[tid];
        const int rank = count_greater(S.cand, nc, mine);
        if (rank < K) put(it + 2 + rank, mine);
    }
    if (tid >= nc && tid < K) put(it + 2 + tid, 0);      // a chunk with fewer than k entries
    if (tid == 0) {
        double sum = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += S.dred[w];
        put(it, (uint64_t)__float_as_uint(m));
        put(it + 1, __builtin_bit_cast(uint64_t, sum));
    }
}

// The step's outputs for request r from S.M, S.Z, S.sel (wave 0).
template <int CAP>
__device__ void finish_request(const DraftArgs &A, MergeShared<CAP> &S, int r, int err, float bsv) {
    const int lane = threadIdx.x & 63;
    const int K = A.topk, R = A.rows;
    // probabilities of the selected entries (lane = row * K + rank)
    float p = 0.f;
    int tok = -1;
    if (lane < R * K) {
        const int j = lane / K, k = lane % K;
        const uint64_t key = S.sel[j][k];
        tok = key_index(key);
        if (tok < 0 || tok >= A.vocab) {
            err |= SPEC_ST_RANGE;
            tok = 0;
        }
        const double z = S.Z[j];
        const double e = exp((double)key_value(key) - (double)S.M[j]);
        p = z > 0.0 ? (float)(e / z) : 0.f;
    }
    const int K2 = K * K;
    float *sc = A.scores + (int64_t)r * A.ncand;
    int32_t *tk = A.tokens + (int64_t)r * A.ncand;
    int32_t *pa = A.parents != nullptr ? A.parents + (int64_t)r * A.npar : nullptr;
    if (A.step == 0) {
        if (lane < K) {
            sc[lane] = p;
            tk[lane] = tok;
            A.next_scores[(int64_t)r * K + lane] = p;
            A.next_tokens[(int64_t)r * K + lane] = tok;
        }
        if (pa != nullptr && A.num_steps > 1 && lane <= K) pa[lane] = lane - 1;
    } else {
        // path products (float32), all of them recorded; then the top-k of
        // the products by rank (value descending, lower flat index first)
        const int off = K + (A.step - 1) * K2;
        float ex = 0.f;
        if (lane < K2) {
            ex = bsv * p;
            sc[off + lane] = ex;
            tk[off + lane] = tok;
        }
        int rank = 0;
        for (int u = 0; u < K2; ++u) {
            const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), u));
            rank += (o > ex) || (o == ex && u < lane);
        }
        if (lane < K2 && rank < K) {
            A.next_scores[(int64_t)r * K + rank] = ex;
            A.next_tokens[(int64_t)r * K + rank] = tok;
            if (pa != nullptr && A.step < A.num_steps - 1)
                pa[K + 1 + (A.step - 1) * K + rank] = lane + K2 * (A.step - 1) + K;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, SPEC_WAVE);
    if (lane == 0) raise_status(A.status, err);
}

// Request r's chunk items (rows x chunks, at most CAP of them) -> each
// row's max, normaliser and top-k keys; then the step's outputs.  REG: at
// most kRegChunks items, one per thread, whose keys stay in registers;
// otherwise the candidate chunks' keys are read again.
template <int CAP, bool REG>
__device__ void merge_request(const DraftArgs &A, MergeShared<CAP> &S, int r) {
    constexpr int P = kRegChunks / kMT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = A.topk, R = A.rows, nch = A.nchunks, nq = R * nch, nw = 2 + K;
    const uint64_t *items = A.items + (int64_t)r * nq * kItemWords;
    float bsv = 0.f;
    if (wave == 0 && A.step > 0 && lane < K * K) bsv = A.branch_scores[(int64_t)r * K + lane / K];
    uint64_t w[P][kItemWords];
    for (int q0 = 0; q0 < nq; q0 += P * kMT) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int q = q0 + tid + i * kMT;
#pragma unroll
            for (int u = 0; u < kItemWords; ++u)
                w[i][u] = (q < nq && u < nw) ? items[(int64_t)q * kItemWords + u] : 0;
        }
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int q = q0 + tid + i * kMT;
            if (q < nq) {
                S.cs[q] = __builtin_bit_cast(double, w[i][1]);
                S.bk[q] = w[i][2];
            }
        }
        if (REG) break;
    }
    if (tid < R) {
        S.rn[tid] = 0;
        S.rtau[tid] = 1;                   // every nonzero key, until a k-th chunk best exists
    }
    if (wave == 0) S.bs[lane] = bsv;
    __syncthreads();
    // each row's max (its largest chunk best) and tau (its k-th largest)
    for (int q = tid; q < nq; q += kMT) {
        const int j = q / nch;
        const uint64_t mine = S.bk[q];
        const int rank = count_greater(S.bk + j * nch, nch, mine);
        if (rank == 0) S.M[j] = key_value(mine);
        if (rank == K - 1) S.rtau[j] = mine;
    }
    __syncthreads();
    // each row's normaliser (a wave per row)
    for (int j = wave; j < R; j += kMW) {
        const Scale2 scl = make_scale2(S.M[j], 1.0f);
        double z = 0.0;
        for (int c = lane; c < nch; c += SPEC_WAVE) {
            const float mc = key_value(S.bk[j * nch + c]);
            if (mc != -INFINITY) z += S.cs[j * nch + c] * (double)exp2_scaled(mc, scl);
        }
        z = wave_sum_d(z);
        if (lane == 0) S.Z[j] = z;
    }
    // candidates: the keys >= tau of the chunks whose best reaches tau (at
    // most k chunks of a row, k keys each)
    if (REG) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int q = tid + i * kMT;
            if (q < nq) {
                const int j = q / nch;
                const uint64_t tau = S.rtau[j];
                if (w[i][2] >= tau) {
#pragma unroll
                    for (int u = 2; u < kItemWords; ++u)
                        if (u < nw && w[i][u] != 0 && w[i][u] >= tau)
                            S.rc[j][atomicAdd(&S.rn[j], 1)] = w[i][u];
                }
            }
        }
    } else {
        for (int q = tid; q < nq; q += kMT) {
            const int j = q / nch;
            const uint64_t tau = S.rtau[j];
            const uint64_t *it = items + (int64_t)q * kItemWords;
            if (S.bk[q] >= tau) {
                for (int u = 2; u < nw; ++u) {
                    const uint64_t key = it[u];
                    if (key != 0 && key >= tau) S.rc[j][atomicAdd(&S.rn[j], 1)] = key;
                }
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < R * kMaxK * kMaxK; q += kMT) {
        const int j = q / (kMaxK * kMaxK), c = q % (kMaxK * kMaxK);
        const int n = S.rn[j];
        if (c < n) {
            const uint64_t mine = S.rc[j][c];
            const int rank = count_greater(S.rc[j], n, mine);
            if (rank < K) S.sel[j][rank] = mine;
        }
    }
    __syncthreads();
    if (wave == 0) finish_request<CAP>(A, S, r, 0, S.bs[lane]);
}

template <int DT, int E>
__global__ __launch_bounds__(kThreads) void draft_chunk_kernel(DraftArgs A) {
    __shared__ ChunkShared S;
    chunk_item<DT, E>(A, S, blockIdx.x);
}

template <int CAP, bool REG>
__global__ __launch_bounds__(kMT) void draft_merge_kernel(DraftArgs A) {
    __shared__ MergeShared<CAP> S;
    merge_request<CAP, REG>(A, S, blockIdx.x);
}

int64_t small_chunks(int64_t vocab) { return (vocab + kThreads * kSmallE - 1) / (kThreads * kSmallE); }

int chunk_entries(int batch, int rows, int64_t vocab) {
    const int64_t small = small_chunks(vocab);
    if ((int64_t)batch * rows * small <= kSmallGrid && rows * small <= kRegChunks)
        return kThreads * kSmallE;
    return kThreads * kLargeE;
}

size_t items_bytes(int batch, int topk, int64_t vocab) {
    return spec::align_up((size_t)batch * topk * small_chunks(vocab) * kItemWords * 8, 256);
}

template <int DT>
void launch(const DraftArgs &A, int64_t items, int chunk, hipStream_t st) {
    const dim3 b(kThreads);
    if (chunk == kThreads * kSmallE)
        hipLaunchKernelGGL((draft_chunk_kernel<DT, kSmallE>), dim3((unsigned)items), b, 0, st, A);
    else
        hipLaunchKernelGGL((draft_chunk_kernel<DT, kLargeE>), dim3((unsigned)items), b, 0, st, A);
    if (A.rows * A.nchunks <= kRegChunks)
        hipLaunchKernelGGL((draft_merge_kernel<kRegChunks, true>), dim3((unsigned)A.batch), dim3(kMT), 0,
                           st, A);
    else
        hipLaunchKernelGGL((draft_merge_kernel<kMergeChunks, false>), dim3((unsigned)A.batch), dim3(kMT),
                           0, st, A);
}

}  // namespace

extern "C" size_t spec_draft_step_workspace_size(int batch, int topk, int64_t vocab) {
    if (batch <= 0 || topk <= 0 || vocab <= 0) return 0;
    return items_bytes(batch, topk, vocab);
}

extern "C" int spec_draft_step(int batch, int topk, int num_steps, int step, int64_t vocab,
                               int dtype, const void *draft_logits, const float *branch_scores,
                               float *scores, int32_t *tokens, int32_t *parents,
                               float *next_scores, int32_t *next_tokens, void *workspace,
                               size_t workspace_bytes, int32_t *dev_status,
                               spec_stream_t stream) {
    if (batch < 0 || topk < 1 || num_steps < 1 || step < 0 || step >= num_steps || vocab < 1)
        return SPEC_ERR_SHAPE;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if (vocab < topk) return SPEC_ERR_SHAPE;
    const int rows = step == 0 ? 1 : topk;
    if (topk > kMaxK || vocab > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    const int chunk = chunk_entries(batch < 1 ? 1 : batch, rows, vocab);
    const int64_t nch = (vocab + chunk - 1) / chunk;
    if (rows * nch > kMergeChunks) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!draft_logits || !scores || !tokens || !next_scores || !next_tokens) return SPEC_ERR_NULL;
    if (step > 0 && !branch_scores) return SPEC_ERR_NULL;
    if (num_steps > 1 && step < num_steps - 1 && !parents) return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < items_bytes(batch, topk, vocab) ||
        reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return SPEC_ERR_WORKSPACE;
    const int64_t items = (int64_t)batch * rows * nch;
    if (items > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    DraftArgs A{};
    A.logits = draft_logits;
    A.vocab = vocab;
    A.vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0;
    A.batch = batch;
    A.topk = topk;
    A.num_steps = num_steps;
    A.step = step;
    A.rows = rows;
    A.nchunks = (int)nch;
    A.ncand = topk + (num_steps - 1) * topk * topk;
    A.npar = 1 + (num_steps - 1) * topk;
    A.branch_scores = branch_scores;
    A.scores = scores;
    A.tokens = tokens;
    A.parents = parents;
    A.next_scores = next_scores;
    A.next_tokens = next_tokens;
    A.items = static_cast<uint64_t *>(workspace);
    A.status = dev_status;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        launch<SPEC_BF16>(A, items, chunk, st);
    else
        launch<SPEC_F32>(A, items, chunk, st);
    return spec::launch_status();
}
