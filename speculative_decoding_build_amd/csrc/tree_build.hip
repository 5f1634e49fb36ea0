// Tree build: draft score/token/parent lists -> pruned tree, mask, positions
// and first-child / next-sibling lists.
//
// Follows "SGLang 源码完全拆解(十一):投机解码" (organize_draft_results; 从树到
// mask:build_tree_kernel_efficient; 邻接表:retrieve_* 三兄弟) and
// "把投机采样讲透:以 SGLang 中的 EAGLE-2 为例" (4.3 tree mask, positions).
//
// One 1024-thread workgroup per request.  Every input of the request
// (scores, tokens, parent list, bonus token, sequence length) is read into
// LDS in one round of loads at the start, so the rest of the kernel waits
// on memory once.  Selection needs no sort: a
// candidate is kept iff fewer than n-1 candidates beat it under
// (score desc, flat index asc), and its node index is one plus the number of
// kept candidates with a smaller flat index (a block prefix count), which is
// exactly "take the top n-1, then sort their indices ascending"; the
// comparisons of each candidate are shared among all threads of the
// workgroup.  Structure work (depth, ancestor bits, child/sibling links)
// runs on one wavefront with a lane per node.  When every candidate is kept
// (the chain of a topk-1 draft, n = num_steps + 1, the case the pages give a
// dedicated chain builder), the ranking is skipped and no score is read.
#include "spec_common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxCand = 4096;
constexpr int kMaxNodes = 64;

// Order key of a candidate: larger score first, then smaller flat index.
// The float maps monotonically onto uint32 (+0 and -0 made equal), the
// index goes in the low word complemented, so "beats" is one unsigned
// 64-bit comparison.
__device__ __forceinline__ uint64_t order_key(float s, int f) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)f);
}

__global__ __launch_bounds__(kThreads) void build_tree_kernel(
    int topk, int n, int ncand, int npar, int mask_mode, int word_bytes,
    const float *__restrict__ scores, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ parents, const int32_t *__restrict__ bonus,
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ draft_tokens,
    int32_t *__restrict__ positions, uint8_t *__restrict__ tree_mask,
    int32_t *__restrict__ r_index, int32_t *__restrict__ r_next, int32_t *__restrict__ r_sib,
    int32_t *__restrict__ selected, int32_t *__restrict__ status) {
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kMaxCand];
    __shared__ int32_t s_tok[kMaxCand];        // candidate tokens
    __shared__ int32_t s_plist[kMaxCand];      // parent list (npar <= ncand entries)
    __shared__ int16_t s_node[kMaxCand];       // flat index -> node (0 = not kept)
    __shared__ int32_t s_flat[kMaxNodes];      // node -> flat index
    __shared__ int32_t s_parent[kMaxNodes];
    __shared__ uint64_t s_kids[kMaxNodes];     // children of each node as a bit set
    __shared__ int32_t s_wave_cnt[kThreads / SPEC_WAVE];
    __shared__ int32_t s_beats[kThreads];      // per-candidate beat counts (one round)
    __shared__ int32_t s_bonus, s_len;

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (SPEC_WAVE - 1);
    const int wave = tid / SPEC_WAVE;
    const int keep = n - 1;
    const float *sc = scores + (size_t)r * ncand;
    // every candidate kept (a chain: topk 1, n = num_steps + 1, or any tree
    // with n - 1 = ncand): the selection is the identity and no score is read
    const bool all_kept = keep == ncand;

    for (int f = tid; f < ncand; f += kThreads) {
        if (!all_kept) s_key[f] = order_key(sc[f], f);
        s_tok[f] = tokens[(size_t)r * ncand + f];
    }
    if (parents != nullptr)
        for (int i = tid; i < npar; i += kThreads) s_plist[i] = parents[(size_t)r * npar + i];
    if (tid == 0) {
        s_bonus = bonus[r];
        s_len = seq_lens[r];
    }
    if (tid < kMaxNodes) s_flat[tid] = 0;
    __syncthreads();

    // ---- kept iff fewer than n-1 candidates beat it; node index = 1 + number
    // of kept candidates with a smaller flat index.  A round ranks up to
    // `per` candidates in flat order (round i: f = i*per + c); each
    // candidate's count is split into `parts` ranges of the keys, one per
    // thread, so all waves share the comparisons.
    const int per = ncand < kThreads ? (ncand + SPEC_WAVE - 1) / SPEC_WAVE * SPEC_WAVE : kThreads;
    const int parts = kThreads / per;                  // 1 .. 16
    const int span = ((ncand + parts - 1) / parts + 1) & ~1;   // keys per part, even
    int before_rounds = 0;
    if (all_kept) {
        for (int f = tid; f < ncand; f += kThreads) {
            s_node[f] = static_cast<int16_t>(f + 1);
            s_flat[f + 1] = f;
        }
        __syncthreads();
    }
    for (int f0 = 0; f0 < (all_kept ? 0 : ncand); f0 += per) {
        {
            const int c = tid % per, part = tid / per;
            const int f = f0 + c;
            int beats = 0;
            if (part < parts && f < ncand && keep > 0) {
                const uint64_t mine = s_key[f];
                const int g_lo = part * span;
                const int g_hi = min(ncand, g_lo + span);
                const int g_hi2 = g_lo + ((g_hi - g_lo) & ~1);
                // two independent counts, so several LDS reads are in flight
                int b0 = 0, b1 = 0;
                int g = g_lo;
                for (; g + 4 <= g_hi2; g += 4) {
                    const uint4 w0 = *reinterpret_cast<const uint4 *>(&s_key[g]);
                    const uint4 w1 = *reinterpret_cast<const uint4 *>(&s_key[g + 2]);
                    b0 += (((uint64_t)w0.y << 32 | w0.x) > mine) + (((uint64_t)w0.w << 32 | w0.z) > mine);
                    b1 += (((uint64_t)w1.y << 32 | w1.x) > mine) + (((uint64_t)w1.w << 32 | w1.z) > mine);
                }
                for (; g < g_hi2; g += 2) {
                    const uint4 w = *reinterpret_cast<const uint4 *>(&s_key[g]);
                    b0 += (((uint64_t)w.y << 32 | w.x) > mine) + (((uint64_t)w.w << 32 | w.z) > mine);
                }
                if (g_hi2 < g_hi) b0 += s_key[g_hi2] > mine;
                beats = b0 + b1;
            }
            if (part == 0) s_beats[c] = beats;
            __syncthreads();
            if (part > 0 && part < parts && f < ncand) atomicAdd(&s_beats[c], beats);
            __syncthreads();
        }
        const int f = f0 + tid;
        const bool kept = tid < per && f < ncand && keep > 0 && s_beats[tid] < keep;
        // block prefix count of kept flags in thread order
        const uint64_t ball = __ballot(kept);
        const int in_wave = __popcll(ball & ((1ull << lane) - 1ull));
        if (lane == 0) s_wave_cnt[wave] = __popcll(ball);
        __syncthreads();
        int before = before_rounds + in_wave;
        int round_total = 0;
        for (int w = 0; w < kThreads / SPEC_WAVE; ++w) {
            if (w < wave) before += s_wave_cnt[w];
            round_total += s_wave_cnt[w];
        }
        if (tid < per && f < ncand) {
            int node = 0;
            if (kept && before < keep) {
                node = before + 1;               // node index 1 .. n-1
                s_flat[node] = f;
            }
            s_node[f] = static_cast<int16_t>(node);
        }
        before_rounds += round_total;
        __syncthreads();
    }

    // ---- per-node structure, one lane of wave 0 per node ------------------
    const int k = lane;
    int err = 0;
    int par = -1;
    if (wave == 0 && k >= 1 && k < n) {
        const int f = s_flat[k];
        if (f < topk) {
            par = 0;
        } else {
            const int g = s_plist[f / topk];
            if (g < 0 || g >= ncand) {
                err |= SPEC_ST_RANGE;
                par = 0;
            } else {
                const int pn = s_node[g];
                if (pn == 0 || pn >= k) {
                    err |= SPEC_ST_NOT_CLOSED;
                    par = 0;
                } else {
                    par = pn;
                }
            }
        }
    }
    if (wave == 0 && k < n) {
        s_parent[k] = par;
        s_kids[k] = 0;
    }
    __syncthreads();
    if (wave != 0) return;

    // children of every node as a bit set: first child = lowest set bit,
    // next sibling = lowest bit of the parent's set above k
    if (k >= 1 && k < n) atomicOr(reinterpret_cast<unsigned long long *>(&s_kids[par]), 1ull << k);
    // only wave 0 is left, and one wave's LDS accesses complete in order
    __builtin_amdgcn_wave_barrier();
    const uint64_t kids = k < n ? s_kids[k] : 0;
    if (k < n) {
        uint64_t bits = 1ull << k;
        int depth = 0;
        int j = k;
        while (j != 0) {
            j = s_parent[j];
            bits |= 1ull << j;
            ++depth;
        }
        const int first = kids ? __builtin_ctzll(kids) : -1;
        int sib = -1;
        if (k >= 1) {
            const uint64_t later = s_kids[par] & ~((2ull << k) - 1ull);   // siblings above k
            sib = later ? __builtin_ctzll(later) : -1;
        }
        const size_t row = (size_t)r * n + k;
        draft_tokens[row] = (k == 0) ? s_bonus : s_tok[s_flat[k]];
        positions[row] = s_len + depth;
        r_index[row] = static_cast<int32_t>(row);
        r_next[row] = first;
        r_sib[row] = sib;
        if (selected != nullptr && k >= 1) selected[(size_t)r * keep + (k - 1)] = s_flat[k];
        if (mask_mode == SPEC_MASK_QLEN_U8) {
            uint8_t *m = tree_mask + row * n;
            for (int jj = 0; jj < n; ++jj) m[jj] = (bits >> jj) & 1u;
        } else {
            uint8_t *m = tree_mask + row * word_bytes;
            switch (word_bytes) {
                case 1: *m = static_cast<uint8_t>(bits); break;
                case 2: *reinterpret_cast<uint16_t *>(m) = static_cast<uint16_t>(bits); break;
                case 4: *reinterpret_cast<uint32_t *>(m) = static_cast<uint32_t>(bits); break;
                default: *reinterpret_cast<uint64_t *>(m) = bits; break;
            }
        }
    }
    // one status write per wave
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, SPEC_WAVE);
    if (lane == 0) spec::raise_status(status, err);
}

}  // namespace

extern "C" int spec_mask_word_bytes(int n) {
    if (n < 1 || n > 64) return 0;
    const int groups = (n + 7) / 8;            // 1..8
    int idx = 0;
    while ((1 << idx) < groups) ++idx;         // ceil(log2(groups))
    return 1 << idx;
}

extern "C" int spec_build_tree(int batch, int topk, int num_steps, int n, int mask_mode,
                               const float *scores, const int32_t *tokens,
                               const int32_t *parents, const int32_t *bonus,
                               const int32_t *seq_lens, int32_t *draft_tokens,
                               int32_t *positions, void *tree_mask, int32_t *retrieve_index,
                               int32_t *retrieve_next_token, int32_t *retrieve_next_sibling,
                               int32_t *selected, int32_t *dev_status, spec_stream_t stream) {
    if (batch < 0 || topk < 1 || num_steps < 1 || n < 1) return SPEC_ERR_SHAPE;
    if (n > kMaxNodes) return SPEC_ERR_UNSUPPORTED;
    if (mask_mode != SPEC_MASK_QLEN_U8 && mask_mode != SPEC_MASK_QLEN_BITS)
        return SPEC_ERR_SHAPE;
    const int64_t ncand = (int64_t)topk + (int64_t)(num_steps - 1) * topk * topk;
    const int64_t npar = 1 + (int64_t)(num_steps - 1) * topk;
    if (ncand > kMaxCand) return SPEC_ERR_UNSUPPORTED;
    if (n - 1 > ncand) return SPEC_ERR_SHAPE;
    if (batch == 0) return SPEC_OK;
    if (!scores || !tokens || !bonus || !seq_lens || !draft_tokens || !positions ||
        !tree_mask || !retrieve_index || !retrieve_next_token || !retrieve_next_sibling)
        return SPEC_ERR_NULL;
    if (num_steps > 1 && !parents) return SPEC_ERR_NULL;
    if (mask_mode == SPEC_MASK_QLEN_BITS &&
        reinterpret_cast<uintptr_t>(tree_mask) % spec_mask_word_bytes(n) != 0)
        return SPEC_ERR_SHAPE;
    hipLaunchKernelGGL(build_tree_kernel, dim3(batch), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), topk, n, (int)ncand, (int)npar,
                       mask_mode, spec_mask_word_bytes(n), scores, tokens, parents, bonus,
                       seq_lens, draft_tokens, positions, static_cast<uint8_t *>(tree_mask),
                       retrieve_index, retrieve_next_token, retrieve_next_sibling, selected,
                       dev_status);
    return spec::launch_status();
}
