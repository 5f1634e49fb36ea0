// Accepted-KV compaction.
//
// "SGLang 源码完全拆解(十一):投机解码" (KV 回写: target slots for positions
// [seq_len, seq_len + accepted), the accepted verify slots gathered through
// accept_index, then the KV rows moved) and "投机解码 Accept" (六: the rows
// committed are the root and the accepted drafts, the terminal token has no
// KV yet; new_seq_lens = prefix + committed).
//
// One workgroup per (request, layer).  All loads that depend only on the
// request go out together; the moves' slots follow in one round.  The moves
// are staged through LDS one column range at a time, K and V in the same
// pass: every source row's bytes in the range are read before any target
// row's bytes in that range are written, and different ranges never
// overlap, so overlapping source / target slots (verify rows written in
// place) move correctly.  The free list (verify slots that did not become a
// target slot) is built by the layer-0 workgroup.
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
    __shared__ int s_err;
    __shared__ uint4 s_stage[kStageUnits];
    const int b = blockIdx.x;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    // first load round: the accepted row of move tid, the length, the sequence length
    // and (for the free list) verify slot tid, all in flight together
    const int row_j = tid < s1 ? accept_index[(int64_t)b * s1 + tid] : -1;
    const int own_slot = (layer == 0 && tid < n) ? out_cache_loc[(int64_t)b * n + tid] : -1;
    const int L = seq_lens[b];
    int acc = accept_length[b];
    int err = 0;
    if (acc < 0) { acc = 0; err |= SPEC_ST_RANGE; }
    if (acc > s1) { acc = s1; err |= SPEC_ST_RANGE; }
    if (tid == 0) s_err = 0;
    // second load round: thread j resolves move j: source = verify slot of accepted row
    // j, target = slot of sequence position L + j (-1 when skipped)
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
                        const int64_t sl = out_cache_loc[row];
                        const int64_t t = (int64_t)page * page_size + pos % page_size;
                        if (sl < 0 || sl >= num_slots || page < 0 || t < 0 || t >= num_slots)
                            err |= SPEC_ST_RANGE;
                        else { src = sl; tgt = t; }
                    }
                }
            }
        }
        s_src[j] = src;
        s_tgt[j] = tgt;
    }
    __syncthreads();                       // s_err zeroed, moves resolved
    if (err) atomicOr(&s_err, err);
    if (layer == 0) {
        // free list: verify slots of the request that did not become a
        // target, in node order (n <= 64: one lane of wave 0 per slot)
        if (tid < SPEC_WAVE) {
            bool is_free = false;
            if (tid < n) {
                bool kept = false;
                for (int j = 0; j < acc; ++j) kept |= (s_tgt[j] == own_slot);
                is_free = !kept;
            }
            const uint64_t freed = __ballot(is_free);
            const int before = __popcll(freed & ((1ull << tid) - 1ull));
            const int total_free = __popcll(freed);
            if (is_free) free_slots[(int64_t)b * n + before] = own_slot;
            if (tid < n && tid >= total_free) free_slots[(int64_t)b * n + tid] = -1;
            if (tid == 0) num_free[b] = total_free;
        }
        __syncthreads();                   // every status bit is in s_err
        if (tid == 0) {
            new_seq_lens[b] = L + acc;
            spec::raise_status(status, s_err);
        }
    }
    if (acc == 0) return;
    // moves j < acc with a source (the others are skipped); K and V together
    const int chunk = max(1, min(row16, kStageUnits / (2 * acc)));   // units per row per pass
    uint4 *kbase = k_pool + (int64_t)layer * layer_stride16;
    uint4 *vbase = v_pool + (int64_t)layer * layer_stride16;
    for (int c0 = 0; c0 < row16; c0 += chunk) {
        const int w = min(chunk, row16 - c0);
        const int items = 2 * acc * w;
        for (int it = tid; it < items; it += kThreads) {
            const int pool = it / (acc * w), rem = it % (acc * w);
            const int j = rem / w, u = rem % w;
            const int64_t src = s_src[j];
            if (src >= 0) s_stage[it] = (pool == 0 ? kbase : vbase)[src * row16 + c0 + u];
        }
        __syncthreads();
        for (int it = tid; it < items; it += kThreads) {
            const int pool = it / (acc * w), rem = it % (acc * w);
            const int j = rem / w, u = rem % w;
            const int64_t tgt = s_tgt[j];
            if (s_src[j] >= 0) (pool == 0 ? kbase : vbase)[tgt * row16 + c0 + u] = s_stage[it];
        }
        __syncthreads();
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
    if (s1 > kMaxRows || n > SPEC_WAVE) return SPEC_ERR_UNSUPPORTED;
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
