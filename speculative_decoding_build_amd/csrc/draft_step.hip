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
// Launch 1, one workgroup per (branch row, 8192-entry chunk): the chunk's
// max, its float64 sum of exponentials (float32 base-2 exponentials of the
// argument carried as a float pair) and its top-k entries as 64-bit order
// keys (the logit's order-preserving bits, then the complemented index: a
// larger key is a larger logit, or the lower index of equal logits; logit
// order is probability order).  Launch 2, one workgroup per request: each
// row's max and normaliser from its chunks, its top-k by rank among the
// chunks' keys, the probabilities of those entries (float64 exponential,
// rounded to float32), then the step's products and selection.
#include "sweep_common.h"

using namespace spec;

namespace {

constexpr int kMaxK = 8;                   // topk at most
constexpr int kItemWords = 2 + kMaxK;      // per chunk item: max, sum, keys
constexpr int kMaxKeys = 4096;             // rows x chunks x topk a request merges in LDS

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

struct DraftArgs {
    const void *logits;                    // [batch][rows][vocab]
    int64_t vocab;
    bool vec_ok;
    int batch, topk, num_steps, step, rows, nchunks;
    const float *branch_scores;            // [batch][topk] (step >= 1)
    float *scores;                         // [batch][ncand]
    int32_t *tokens;                       // [batch][ncand]
    int32_t *parents;                      // [batch][npar]
    float *next_scores;                    // [batch][topk]
    int32_t *next_tokens;                  // [batch][topk]
    int ncand, npar;
    uint64_t *items;                       // [batch * rows * nchunks][kItemWords]
    int32_t *status;
};

// insert key k into the descending list t (largest first), keeping K entries
template <int K>
__device__ __forceinline__ void insert_desc(uint64_t (&t)[K], uint64_t k) {
    if (k <= t[K - 1]) return;
    t[K - 1] = k;
#pragma unroll
    for (int j = K - 1; j > 0; --j) {
        if (t[j] > t[j - 1]) {
            const uint64_t x = t[j];
            t[j] = t[j - 1];
            t[j - 1] = x;
        }
    }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t w = __shfl_xor(v, o, SPEC_WAVE);
        v = w > v ? w : v;
    }
    return v;
}

// KT >= topk: the per-thread and per-wave lists hold KT keys
template <int DT, int KT>
__global__ __launch_bounds__(kSweepThreads) void draft_chunk_kernel(DraftArgs A) {
    __shared__ float s_f[kSweepThreads / SPEC_WAVE];
    __shared__ double s_d[kSweepThreads / SPEC_WAVE];
    __shared__ uint64_t s_k[kSweepThreads / SPEC_WAVE][KT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    const int64_t row = t / A.nchunks;     // (request, branch) row
    const int64_t start = (t % A.nchunks) * kChunk;
    const int64_t end = min(A.vocab, start + kChunk);
    const char *rowp = static_cast<const char *>(A.logits) + row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
    float x[kPerThread];
    load_chunk<DT>(rowp, start, end, A.vec_ok, tid, x);
    // max
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, SPEC_WAVE));
    if (lane == 0) s_f[wave] = m;
    __syncthreads();
    m = s_f[0];
#pragma unroll
    for (int w = 1; w < kSweepThreads / SPEC_WAVE; ++w) m = fmaxf(m, s_f[w]);
    // sum of exponentials, and this thread's top-k keys
    const Scale2 sc = make_scale2(m, 1.0f);
    double s = 0.0;
    uint64_t top[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) top[j] = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const int64_t idx = elem_index(start, tid, e);
        if (idx < end) {
            if (m != -INFINITY) s += (double)exp2_scaled(x[e], sc);
            insert_desc<KT>(top, order_key(x[e], idx));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, SPEC_WAVE);
    if (lane == 0) s_d[wave] = s;
    // the wave's top-k: k rounds of a wave max over the lists' heads
#pragma unroll
    for (int r = 0; r < KT; ++r) {
        const uint64_t best = wave_max_u64(top[0]);
        if (best != 0 && top[0] == best) {
#pragma unroll
            for (int j = 0; j < KT - 1; ++j) top[j] = top[j + 1];
            top[KT - 1] = 0;
        }
        if (lane == 0) s_k[wave][r] = best;
    }
    __syncthreads();
    if (wave == 0) {
        // rank of each of the block's 4 x KT keys among them; the chunk
        // keeps the first topk
        constexpr int NK = (kSweepThreads / SPEC_WAVE) * KT;
        const uint64_t mine = lane < NK ? s_k[lane / KT][lane % KT] : 0;
        int rank = 0;
        for (int q = 0; q < NK; ++q) rank += s_k[q / KT][q % KT] > mine;
        uint64_t *it = A.items + t * kItemWords;
        if (lane == 0) {
            double sum = 0.0;
#pragma unroll
            for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) sum += s_d[w];
            it[0] = (uint64_t)__float_as_uint(m);
            it[1] = __builtin_bit_cast(uint64_t, sum);
        }
        if (lane < NK && mine != 0 && rank < A.topk) it[2 + rank] = mine;
        // empty entries (a chunk with fewer than topk entries) read as 0
        if (lane < A.topk) {
            int filled = 0;
            for (int q = 0; q < NK; ++q) filled += s_k[q / KT][q % KT] != 0;
            if (lane >= filled) it[2 + lane] = 0;
        }
    }
}

__global__ __launch_bounds__(kSweepThreads) void draft_select_kernel(DraftArgs A) {
    __shared__ uint64_t s_keys[kMaxKeys];
    __shared__ float s_M[kMaxK];
    __shared__ double s_Z[kMaxK];
    __shared__ uint64_t s_sel[kMaxK][kMaxK];   // [row][rank]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;
    const int K = A.topk, rows = A.rows, nch = A.nchunks;
    const int per_row = nch * K;               // keys of one row
    // every row's chunk keys into LDS (chunk c's keys c*K .. c*K+K-1)
    const uint64_t *items = A.items + (int64_t)r * rows * nch * kItemWords;
    for (int q = tid; q < rows * per_row; q += blockDim.x) {
        const int j = q / per_row, rest = q % per_row;
        s_keys[q] = items[((int64_t)j * nch + rest / K) * kItemWords + 2 + rest % K];
    }
    // each row's max and normaliser: a wave per row
    for (int j = wave; j < rows; j += kSweepThreads / SPEC_WAVE) {
        float m = -INFINITY;
        for (int c = lane; c < nch; c += SPEC_WAVE)
            m = fmaxf(m, __uint_as_float((uint32_t)items[((int64_t)j * nch + c) * kItemWords]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, SPEC_WAVE));
        const Scale2 sc = make_scale2(m, 1.0f);
        double z = 0.0;
        for (int c = lane; c < nch; c += SPEC_WAVE) {
            const uint64_t *it = items + ((int64_t)j * nch + c) * kItemWords;
            const float mc = __uint_as_float((uint32_t)it[0]);
            if (mc != -INFINITY) z += __builtin_bit_cast(double, it[1]) * (double)exp2_scaled(mc, sc);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, SPEC_WAVE);
        if (lane == 0) {
            s_M[j] = m;
            s_Z[j] = z;
        }
    }
    __syncthreads();
    // each row's top-k: rank of every key among its row's keys
    for (int q = tid; q < rows * per_row; q += blockDim.x) {
        const uint64_t mine = s_keys[q];
        if (mine == 0) continue;
        const int j = q / per_row;
        const uint64_t *rk = s_keys + j * per_row;
        int rank = 0;
        for (int u = 0; u < per_row; ++u) rank += rk[u] > mine;
        if (rank < K) s_sel[j][rank] = mine;
    }
    __syncthreads();
    if (wave != 0) return;
    // probabilities of the selected entries (lane = row * K + rank)
    const int nsel = rows * K;
    int err = 0;
    float p = 0.f;
    int tok = -1;
    if (lane < nsel) {
        const int j = lane / K, k = lane % K;
        const uint64_t key = s_sel[j][k];
        tok = key_index(key);
        if (tok < 0 || tok >= A.vocab) {
            err |= SPEC_ST_RANGE;
            tok = 0;
        }
        const double z = s_Z[j];
        const double e = exp((double)key_value(key) - (double)s_M[j]);
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
            ex = A.branch_scores[(int64_t)r * K + lane / K] * p;
            sc[off + lane] = ex;
            tk[off + lane] = tok;
        }
        __builtin_amdgcn_wave_barrier();
        int rank = 0;
        for (int u = 0; u < K2; ++u) {
            const float o = __shfl(ex, u, SPEC_WAVE);
            rank += (o > ex) || (o == ex && u < lane);
        }
        if (lane < K2 && rank < K) {
            A.next_scores[(int64_t)r * K + rank] = ex;
            A.next_tokens[(int64_t)r * K + rank] = tok;
            if (pa != nullptr && A.step < A.num_steps - 1)
                pa[K + 1 + (A.step - 1) * K + rank] = lane + K2 * (A.step - 1) + K;
        }
    }
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, SPEC_WAVE);
    if (lane == 0) raise_status(A.status, err);
}

template <int DT>
void launch_chunks(const DraftArgs &A, int64_t items, hipStream_t st) {
    const dim3 g((unsigned)items), b(kSweepThreads);
    if (A.topk == 1)
        hipLaunchKernelGGL((draft_chunk_kernel<DT, 1>), g, b, 0, st, A);
    else if (A.topk == 2)
        hipLaunchKernelGGL((draft_chunk_kernel<DT, 2>), g, b, 0, st, A);
    else if (A.topk <= 4)
        hipLaunchKernelGGL((draft_chunk_kernel<DT, 4>), g, b, 0, st, A);
    else
        hipLaunchKernelGGL((draft_chunk_kernel<DT, kMaxK>), g, b, 0, st, A);
}

}  // namespace

extern "C" size_t spec_draft_step_workspace_size(int batch, int topk, int64_t vocab) {
    if (batch <= 0 || topk <= 0 || vocab <= 0) return 0;
    return spec::align_up((size_t)batch * topk * num_chunks(vocab) * kItemWords * sizeof(uint64_t), 256);
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
    const int nch = num_chunks(vocab);
    if (topk > kMaxK || vocab > INT_MAX || (int64_t)rows * nch * topk > kMaxKeys)
        return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!draft_logits || !scores || !tokens || !next_scores || !next_tokens) return SPEC_ERR_NULL;
    if (step > 0 && !branch_scores) return SPEC_ERR_NULL;
    if (num_steps > 1 && step < num_steps - 1 && !parents) return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_draft_step_workspace_size(batch, topk, vocab) ||
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
    A.nchunks = nch;
    A.branch_scores = branch_scores;
    A.scores = scores;
    A.tokens = tokens;
    A.parents = parents;
    A.next_scores = next_scores;
    A.next_tokens = next_tokens;
    A.ncand = topk + (num_steps - 1) * topk * topk;
    A.npar = 1 + (num_steps - 1) * topk;
    A.items = static_cast<uint64_t *>(workspace);
    A.status = dev_status;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16)
        launch_chunks<SPEC_BF16>(A, items, st);
    else
        launch_chunks<SPEC_F32>(A, items, st);
    hipLaunchKernelGGL(draft_select_kernel, dim3(batch), dim3(kSweepThreads), 0, st, A);
    return spec::launch_status();
}
