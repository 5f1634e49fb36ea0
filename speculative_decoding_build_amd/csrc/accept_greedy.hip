// Greedy tree accept: per-row argmax over the vocabulary, then the tree walk.
//
// Follows "SGLang 源码完全拆解(十一):投机解码" (三条判定路径: argmax per verify
// row, then the first-child / next-sibling walk) and "投机解码 Accept:从 Verify
// 行到最终输出路径" (三: accept_index holds verify rows; the last row's target
// choice is the terminal token).
//
// Two launches: a chunked argmax sweep over every verify row (one 256-thread
// workgroup per (8192-entry chunk, row), the chunk loaded once with 16-byte
// loads), then one wavefront per request that merges its rows' chunk
// partials and walks the tree.
#include "sweep_common.h"

using namespace spec;

namespace {

struct ArgPart {
    float v;
    int32_t i;
};

// ---- greedy: chunked argmax -----------------------------------------------

template <int DT>
__global__ __launch_bounds__(kSweepThreads) void argmax_partial_kernel(
    const void *__restrict__ logits, int64_t vocab, int nchunks, bool vec_ok,
    ArgPart *__restrict__ part) {
    const int c = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t start = (int64_t)c * kChunk;
    const int64_t end = min(vocab, start + kChunk);
    const char *rowp = static_cast<const char *>(logits) + row * vocab * (DT == SPEC_BF16 ? 2 : 4);
    float x[kPerThread];
    load_chunk<DT>(rowp, start, end, vec_ok, tid, x);
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {       // e increases with element index
        const int64_t idx = elem_index(start, tid, e);
        if (idx < end && (bi < 0 || x[e] > bv)) {
            bv = x[e];
            bi = (int)idx;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, SPEC_WAVE);
        const int oi = __shfl_xor(bi, o, SPEC_WAVE);
        if (arg_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    __shared__ float s_v[kSweepThreads / SPEC_WAVE];
    __shared__ int s_i[kSweepThreads / SPEC_WAVE];
    if ((tid & 63) == 0) { s_v[tid >> 6] = bv; s_i[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kSweepThreads / SPEC_WAVE; ++w)
            if (arg_better(s_v[w], s_i[w], bv, bi)) { bv = s_v[w]; bi = s_i[w]; }
        part[row * nchunks + c] = ArgPart{bv, bi};
    }
}

// One wavefront per request: merge the chunk partials of the request's rows,
// then walk from the root.
__global__ __launch_bounds__(SPEC_WAVE) void greedy_walk_kernel(
    int n, int s1, int total_rows, int nchunks, const ArgPart *__restrict__ part,
    const int32_t *__restrict__ cand, const int32_t *__restrict__ r_index,
    const int32_t *__restrict__ r_next, const int32_t *__restrict__ r_sib,
    int32_t *__restrict__ predict, int32_t *__restrict__ accept_index,
    int32_t *__restrict__ accept_length, int32_t *__restrict__ target_predict,
    int32_t *__restrict__ status) {
    __shared__ int s_tp[kMaxNodes];
    __shared__ int s_row[kMaxNodes];
    __shared__ int s_pred[kMaxNodes];
    __shared__ int s_cand[kMaxNodes];
    __shared__ int s_next[kMaxNodes];
    __shared__ int s_sib[kMaxNodes];
    __shared__ int s_ai[kMaxNodes + 1];
    __shared__ int s_len;
    const int b = blockIdx.x;
    const int k = threadIdx.x;
    const int base = b * n;
    int err = 0;
    if (k < n) {
        // every lane loads its node's links and reduces its row's chunk partials
        int row = r_index[base + k];
        s_cand[k] = cand[base + k];
        s_next[k] = r_next[base + k];
        s_sib[k] = r_sib[base + k];
        if (row < base || row >= base + n) { err |= SPEC_ST_RANGE; row = -1; }
        int bi = -1;
        float bv = -INFINITY;
        if (row >= 0)
            for (int c = 0; c < nchunks; ++c) {
                const ArgPart p = part[(int64_t)row * nchunks + c];
                if (arg_better(p.v, p.i, bv, bi)) { bv = p.v; bi = p.i; }
            }
        s_tp[k] = bi;
        s_row[k] = row;
        s_pred[k] = 0;
    }
    __syncthreads();
    if (k == 0) {
        int cur = 0, cnt = 0;
        s_ai[0] = s_row[0];
        for (int guard = 0; guard < n; ++guard) {
            const int want = s_tp[cur];
            int c = s_next[cur];
            int hit = -1;
            for (int steps = 0; c != -1 && steps < n; ++steps) {
                if (c < 0 || c >= n) { err |= SPEC_ST_RANGE; break; }
                if (s_cand[c] == want) { hit = c; break; }
                c = s_sib[c];
            }
            if (hit < 0) break;
            if (cnt + 1 >= s1) { err |= SPEC_ST_DEPTH; break; }
            s_pred[cur] = s_cand[hit];
            ++cnt;
            s_ai[cnt] = s_row[hit];
            cur = hit;
        }
        s_pred[cur] = s_tp[cur];
        s_len = cnt + 1;
    }
    __syncthreads();
    if (k < n && s_row[k] >= 0) {
        predict[s_row[k]] = s_pred[k];
        if (target_predict != nullptr) target_predict[s_row[k]] = s_tp[k];
    }
    for (int j = k; j < s1; j += SPEC_WAVE)
        accept_index[(int64_t)b * s1 + j] = (j < s_len) ? s_ai[j] : -1;
    if (k == 0) accept_length[b] = s_len;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, SPEC_WAVE);
    if (k == 0) raise_status(status, err);
}

}  // namespace

size_t spec_greedy_workspace_bytes(int batch, int n, int64_t vocab) {
    return spec::align_up((size_t)batch * n * num_chunks(vocab) * sizeof(ArgPart), 256);
}

int spec_check_accept_args(int batch, int n, int s1, int64_t vocab, int dtype) {
    if (batch < 0 || n < 1 || s1 < 1 || vocab < 1) return SPEC_ERR_SHAPE;
    if (n > kMaxNodes || s1 > kMaxNodes + 1) return SPEC_ERR_UNSUPPORTED;
    if (vocab > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    return SPEC_OK;
}

extern "C" int spec_accept_greedy(int batch, int n, int s1, int64_t vocab, int dtype,
                                  const void *target_logits, const int32_t *candidates,
                                  const int32_t *retrieve_index,
                                  const int32_t *retrieve_next_token,
                                  const int32_t *retrieve_next_sibling, int32_t *predict,
                                  int32_t *accept_index, int32_t *accept_length,
                                  int32_t *target_predict, void *workspace,
                                  size_t workspace_bytes, int32_t *dev_status,
                                  spec_stream_t stream) {
    int rc = spec_check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (batch == 0) return SPEC_OK;
    if (!target_logits || !candidates || !retrieve_index || !retrieve_next_token ||
        !retrieve_next_sibling || !predict || !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_greedy_workspace_bytes(batch, n, vocab))
        return SPEC_ERR_WORKSPACE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int nch = num_chunks(vocab);
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    const bool vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0;
    ArgPart *part = static_cast<ArgPart *>(workspace);
    const dim3 grid(nch, batch * n);
    if (dtype == SPEC_BF16)
        hipLaunchKernelGGL(argmax_partial_kernel<SPEC_BF16>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, vocab, nch, vec_ok, part);
    else
        hipLaunchKernelGGL(argmax_partial_kernel<SPEC_F32>, grid, dim3(kSweepThreads), 0, st,
                           target_logits, vocab, nch, vec_ok, part);
    hipLaunchKernelGGL(greedy_walk_kernel, dim3(batch), dim3(SPEC_WAVE), 0, st, n, s1,
                       batch * n, nch, part, candidates, retrieve_index, retrieve_next_token,
                       retrieve_next_sibling, predict, accept_index, accept_length,
                       target_predict, dev_status);
    return spec::launch_status();
}

