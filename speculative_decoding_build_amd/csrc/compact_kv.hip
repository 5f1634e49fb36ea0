// Accepted-KV compaction.
//
// "SGLang 源码完全拆解(十一):投机解码" (KV 回写: target slots for positions
// [seq_len, seq_len + accepted), the accepted verify slots gathered through
// accept_index, then the KV rows moved) and "投机解码 Accept" (六: the rows
// committed are the root and the accepted drafts, the terminal token has no
// KV yet; new_seq_lens = prefix + committed).
//
// One workgroup per (request, layer).  The request's moves are staged
// through LDS one column range at a time: every source row's bytes in the
// range are read before any target row's bytes in that range are written,
// and different ranges never overlap, so overlapping source / target slots
// (verify rows written in place) move correctly.  The free list (verify
// slots that did not become a target slot) is built by the layer-0
// workgroup.
#include "spec_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 65;
constexpr int kStageUnits = 3072;          // 16-byte units staged per pass (48 KB)

__global__ __launch_bounds__(kThreads) void compact_kv_kernel(
    int n, int s1, int total_rows, int row16, int page_size, int max_pages, int64_t num_slots,
    int64_t layer_stride16, uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ out_cache_loc, const int32_t *__restrict__ accept_index,
    const int32_t *__restrict__ accept_length, int32_t *__restrict__ new_seq_lens,
    int32_t *__restrict__ free_slots, int32_t *__restrict__ num_free, int32_t *__restrict__ status) {
    __shared__ int64_t s_src[kMaxRows], s_tgt[kMaxRows];
    __shared__ int64_t s_jsrc[kMaxRows], s_jtgt[kMaxRows];
    __shared__ int s_m, s_err, s_keep[kMaxRows + 1];
    __shared__ uint4 s_stage[kStageUnits];
    const int b = blockIdx.x;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    // the accepted row of move tid is read without waiting for the length,
    // so both loads (and the sequence length) are in flight together
    const int row_j = tid < s1 ? accept_index[(int64_t)b * s1 + tid] : -1;
    const int L = seq_lens[b];
    int acc = accept_length[b];
    int err = 0;
    if (acc < 0) { acc = 0; err |= SPEC_ST_RANGE; }
    if (acc > s1) { acc = s1; err |= SPEC_ST_RANGE; }
    if (tid == 0) s_err = 0;
    __syncthreads();
    // thread j resolves move j: source = verify slot of accepted row j,
    // target = slot of sequence position L + j (-1 when skipped)
    if (tid < s1) {
        int64_t src = -1, tgt = -1;
        const int j = tid;
        if (j < acc) {
            const int row = row_j;
            if (row >= 0) {
                if (row >= total_rows) {
                    err |= SPEC_ST_RANGE;
                } else {
                    const int64_t pos = (int64_t)L + j;
                    const int64_t pidx = pos / page_size;
                    if (L < 0 || pidx >= max_pages) {
                        err |= SPEC_ST_RANGE;
                    } else {
                        const int page = page_table[(int64_t)b * max_pages + pidx];
                        const int64_t s = out_cache_loc[row];
                        const int64_t t = (int64_t)page * page_size + pos % page_size;
                        if (s < 0 || s >= num_slots || page < 0 || t < 0 || t >= num_slots)
                            err |= SPEC_ST_RANGE;
                        else { src = s; tgt = t; }
                    }
                }
            }
        }
        s_jsrc[j] = src;
        s_jtgt[j] = tgt;
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0) {
        int cnt = 0;
        for (int j = 0; j < acc; ++j)
            if (s_jsrc[j] >= 0) { s_src[cnt] = s_jsrc[j]; s_tgt[cnt] = s_jtgt[j]; ++cnt; }
        s_m = cnt;
    }
    __syncthreads();
    if (layer == 0) {
        // free list: verify slots of the request that did not become a target
        const int cnt = s_m;
        int kept = 1;
        int slot = -1;
        if (tid < n) {
            slot = out_cache_loc[(int64_t)b * n + tid];
            kept = 0;
            for (int j = 0; j < cnt; ++j) kept |= (s_tgt[j] == slot);
            s_keep[tid] = kept;
        }
        __syncthreads();
        if (tid < n) {
            int before = 0;
            for (int k = 0; k < tid; ++k) before += 1 - s_keep[k];
            if (!kept) free_slots[(int64_t)b * n + before] = slot;
            int total_free = before + (1 - kept);
            for (int k = tid + 1; k < n; ++k) total_free += 1 - s_keep[k];
            if (tid >= total_free) free_slots[(int64_t)b * n + tid] = -1;
            if (tid == 0) num_free[b] = total_free;
        }
        if (tid == 0) {
            new_seq_lens[b] = L + acc;
            spec::raise_status(status, s_err);
        }
    }
    const int m = s_m;
    if (m == 0) return;
    const int chunk = max(1, min(row16, kStageUnits / m));   // 16-byte units per row per pass
    for (int pool = 0; pool < 2; ++pool) {
        uint4 *base = (pool == 0 ? k_pool : v_pool) + (int64_t)layer * layer_stride16;
        for (int c0 = 0; c0 < row16; c0 += chunk) {
            const int w = min(chunk, row16 - c0);
            const int items = m * w;
            for (int it = tid; it < items; it += kThreads) {
                const int j = it / w, u = it % w;
                s_stage[j * w + u] = base[s_src[j] * row16 + c0 + u];
            }
            __syncthreads();
            for (int it = tid; it < items; it += kThreads) {
                const int j = it / w, u = it % w;
                base[s_tgt[j] * row16 + c0 + u] = s_stage[j * w + u];
            }
            __syncthreads();
        }
    }
}

}  // namespace

extern "C" int spec_compact_kv(int batch, int n, int s1, int num_layers, int hkv, int d,
                               int page_size, int dtype, void *k_pool, void *v_pool,
                               int64_t num_slots, const int32_t *page_table, int max_pages,
                               const int32_t *seq_lens, const int32_t *out_cache_loc,
                               const int32_t *accept_index, const int32_t *accept_length,
                               int32_t *new_seq_lens, int32_t *free_slots, int32_t *num_free,
                               int32_t *dev_status, spec_stream_t stream) {
    if (batch < 0 || n < 1 || s1 < 1 || num_layers < 1 || hkv < 1 || d < 1 || page_size < 1 ||
        max_pages < 0 || num_slots < 0)
        return SPEC_ERR_SHAPE;
    if (s1 > kMaxRows) return SPEC_ERR_UNSUPPORTED;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    const int64_t row_bytes = (int64_t)hkv * d * (dtype == SPEC_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!k_pool || !v_pool || !page_table || !seq_lens || !out_cache_loc || !accept_index ||
        !accept_length || !new_seq_lens || !free_slots || !num_free)
        return SPEC_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15u)
        return SPEC_ERR_SHAPE;
    const int row16 = (int)(row_bytes / 16);
    hipLaunchKernelGGL(compact_kv_kernel, dim3(batch, num_layers), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), n, s1, batch * n, row16, page_size,
                       max_pages, num_slots, num_slots * row16, static_cast<uint4 *>(k_pool),
                       static_cast<uint4 *>(v_pool), page_table, seq_lens, out_cache_loc,
                       accept_index, accept_length, new_seq_lens, free_slots, num_free,
                       dev_status);
    return spec::launch_status();
}
