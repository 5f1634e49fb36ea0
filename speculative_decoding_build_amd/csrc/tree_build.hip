// Tree build: draft score/token/parent lists -> pruned tree, mask, positions
// and first-child / next-sibling lists.
//
// Follows "SGLang 源码完全拆解(十一):投机解码" (organize_draft_results; 从树到
// mask:build_tree_kernel_efficient; 邻接表:retrieve_* 三兄弟) and
// "把投机采样讲透:以 SGLang 中的 EAGLE-2 为例" (4.3 tree mask, positions).
//
// One 256-thread workgroup per request.  Selection needs no sort: a
// candidate is kept iff fewer than n-1 candidates beat it under
// (score desc, flat index asc), and its node index is one plus the number of
// kept candidates with a smaller flat index (a block prefix count), which is
// exactly "take the top n-1, then sort their indices ascending".  Structure
// work (depth, ancestor bits, child/sibling links) runs on one wavefront with
// a lane per node.
#include "spec_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxCand = 4096;
constexpr int kMaxNodes = 64;

__global__ __launch_bounds__(kThreads) void build_tree_kernel(
    int topk, int n, int ncand, int npar, int mask_mode, int word_bytes,
    const float *__restrict__ scores, const int32_t *__restrict__ tokens,
    const int32_t *__restrict__ parents, const int32_t *__restrict__ bonus,
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ draft_tokens,
    int32_t *__restrict__ positions, uint8_t *__restrict__ tree_mask,
    int32_t *__restrict__ r_index, int32_t *__restrict__ r_next, int32_t *__restrict__ r_sib,
    int32_t *__restrict__ selected, int32_t *__restrict__ status) {
    __shared__ float s_score[kMaxCand];
    __shared__ int16_t s_node[kMaxCand];       // flat index -> node (0 = not kept)
    __shared__ int32_t s_flat[kMaxNodes];      // node -> flat index
    __shared__ int32_t s_parent[kMaxNodes];
    __shared__ int32_t s_wave_cnt[kThreads / SPEC_WAVE + 1];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (SPEC_WAVE - 1);
    const int wave = tid / SPEC_WAVE;
    const int keep = n - 1;
    const float *sc = scores + (size_t)r * ncand;

    for (int f = tid; f < ncand; f += kThreads) s_score[f] = sc[f];
    if (tid < kMaxNodes) s_flat[tid] = 0;
    __syncthreads();

    // ---- rank each candidate; kept iff rank < n-1 -------------------------
    // Threads own flat indices in contiguous runs so the prefix count below
    // follows flat order: thread t owns [t*per, (t+1)*per).
    const int per = (ncand + kThreads - 1) / kThreads;   // <= 16
    uint32_t kept_bits = 0;                                // bit i: f = t*per + i kept
    for (int i = 0; i < per; ++i) {
        const int f = tid * per + i;
        if (f >= ncand || keep == 0) break;
        const float v = s_score[f];
        int beats = 0;
        for (int g = 0; g < ncand && beats < keep; ++g) {
            const float w = s_score[g];
            beats += (w > v) || (w == v && g < f);
        }
        if (beats < keep) kept_bits |= 1u << i;
    }
    // ---- prefix count of kept candidates in flat order --------------------
    const int my_cnt = __popc(kept_bits);
    int incl = my_cnt;
#pragma unroll
    for (int o = 1; o < SPEC_WAVE; o <<= 1) {
        int x = __shfl_up(incl, o, SPEC_WAVE);
        if (lane >= o) incl += x;
    }
    if (lane == SPEC_WAVE - 1) s_wave_cnt[wave] = incl;
    __syncthreads();
    int before = incl - my_cnt;
    for (int w = 0; w < wave; ++w) before += s_wave_cnt[w];
    for (int i = 0; i < per; ++i) {
        const int f = tid * per + i;
        if (f >= ncand) break;
        int node = 0;
        if ((kept_bits & (1u << i)) && before < keep) {
            node = ++before;                 // node index 1 .. n-1
            s_flat[node] = f;
        }
        s_node[f] = static_cast<int16_t>(node);
    }
    __syncthreads();

    // ---- per-node structure, one lane of wave 0 per node ------------------
    const int k = lane;
    int err = 0;
    int par = -1;
    if (wave == 0 && k >= 1 && k < n) {
        const int f = s_flat[k];
        if (f < topk) {
            par = 0;
        } else {
            const int g = parents[(size_t)r * npar + f / topk];
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
    if (wave == 0 && k < n) s_parent[k] = par;
    __syncthreads();
    if (wave != 0) return;

    if (k < n) {
        // depth and ancestor-or-self bits by walking up the parent chain
        uint64_t bits = 1ull << k;
        int depth = 0;
        int j = k;
        while (j != 0) {
            j = s_parent[j];
            bits |= 1ull << j;
            ++depth;
        }
        // first child: smallest c with parent c == k; next sibling: smallest
        // c > k sharing k's parent
        int first = -1, sib = -1;
        for (int c = n - 1; c >= 1; --c) {
            const int pc = s_parent[c];
            if (pc == k) first = c;
            if (k >= 1 && c > k && pc == par) sib = c;
        }
        const size_t row = (size_t)r * n + k;
        draft_tokens[row] = (k == 0) ? bonus[r] : tokens[(size_t)r * ncand + s_flat[k]];
        positions[row] = seq_lens[r] + depth;
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
