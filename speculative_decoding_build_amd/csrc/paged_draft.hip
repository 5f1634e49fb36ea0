// Memory-side neighbours of the tree build and the compaction.
//
// FULL mask ("SGLang 源码完全拆解(十一):投机解码", 三种 mask 形态 and the
// fill_prefix_mask switch): every verify row sees the whole committed prefix
// and, among the tree nodes, its QLEN_ONLY row.  Request b's block starts at
// n * sum_{b' < b} (L_b' + n) bytes and holds n rows of L_b + n bytes: L_b
// prefix bytes of 1, then the tree row expanded from its bit-packed word.
// Without the prefix fill only the tree bytes are written.  One workgroup
// per (row, 32 KB range of the row), aligned 16-byte streaming stores inside the row
// and byte stores at its two ends; the request offset is a block sum of the
// earlier requests' lengths.
//
// Paged draft-branch planning (same page, prepare_for_draft and
// duplicate_prefix_tail_to_draft_branches): with page_size > 1 and topk > 1
// each branch owns a page-aligned region whose first tail = L mod page_size
// slots stand for the prefix tail; the prefix tail's KV is copied into them
// (every layer, K and V) so that whole-page reads of a branch see its
// tokens, and draft step s of branch j writes region slot tail + s.  With
// topk 1 the single branch continues the prefix in place (the contiguous
// case): step s writes the slot of position L + s through the page table.
// One workgroup per (request, layer, 1024 16-byte units of the copies, each
// thread's four loads in flight together); the first workgroup of layer 0
// writes the draft slots.
#include <algorithm>

#include "spec_common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPer = 4;                    // 16-byte units per thread, in flight together
constexpr int kMaskPer = 8;                // 16-byte mask units per thread
constexpr int kRowSpan = kThreads * 16 * kMaskPer;   // bytes of a mask row per workgroup

__device__ __forceinline__ uint64_t mask_word(const uint8_t *p, int wb) {
    switch (wb) {
        case 1: return *p;
        case 2: return *reinterpret_cast<const uint16_t *>(p);
        case 4: return *reinterpret_cast<const uint32_t *>(p);
        default: return *reinterpret_cast<const uint64_t *>(p);
    }
}

// sum of seq_lens[0, r) over the block (int64)
__device__ int64_t lengths_before(const int32_t *seq_lens, int r, int64_t *s_part) {
    const int tid = threadIdx.x;
    int64_t s = 0;
    for (int i = tid; i < r; i += kThreads) s += max(seq_lens[i], 0);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, SPEC_WAVE);
    if ((tid & 63) == 0) s_part[tid >> 6] = s;
    __syncthreads();
    int64_t t = 0;
#pragma unroll
    for (int w = 0; w < kThreads / SPEC_WAVE; ++w) t += s_part[w];
    return t;
}

__global__ __launch_bounds__(kThreads) void full_mask_kernel(
    int n, int word_bytes, int max_seq_len, int blocks_per_row, int fill_prefix,
    const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ tree_bits,
    uint8_t *__restrict__ out, int64_t out_bytes, int32_t *__restrict__ status) {
    __shared__ int64_t s_part[kThreads / SPEC_WAVE];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x / blocks_per_row;     // request * n + node
    const int part = (int)(blockIdx.x % blocks_per_row);
    const int r = (int)(row / n), k = (int)(row % n);
    const int64_t before = lengths_before(seq_lens, r, s_part);
    int L = seq_lens[r];
    int err = 0;
    if (L < 0 || L > max_seq_len) {
        err |= SPEC_ST_RANGE;
        L = max(L, 0);
    }
    const int64_t w = (int64_t)L + n;
    const int64_t a0 = (int64_t)n * (before + (int64_t)r * n) + (int64_t)k * w;   // row start
    const uint64_t bits = mask_word(tree_bits + row * word_bytes, word_bytes);
    if (a0 + w > out_bytes) err |= SPEC_ST_RANGE;
    const int64_t end = min(a0 + w, out_bytes);
    if (!fill_prefix) {
        // the tree bytes only
        if (part == 0 && tid < n && a0 + L + tid < end) out[a0 + L + tid] = (bits >> tid) & 1u;
    } else {
#pragma unroll
      for (int h = 0; h < kMaskPer; ++h) {
        const int64_t A = (a0 & ~(int64_t)15) + (int64_t)part * kRowSpan + (h * kThreads + tid) * 16;
        if (A >= a0 && A + 16 <= a0 + L && A + 16 <= end) {
            // inside the prefix: sixteen ones, no per-byte work
            u32x4 u;
            u.x = u.y = u.z = u.w = 0x01010101u;
            __builtin_nontemporal_store(u, reinterpret_cast<u32x4 *>(out + A));
        } else if (A < end && A + 16 > a0) {
            uint8_t v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t col = A + i - a0;
                v[i] = (col < 0 || col >= w) ? 0
                       : col < L ? 1 : (uint8_t)((bits >> (int)(col - L)) & 1u);
            }
            if (A >= a0 && A + 16 <= end) {
                u32x4 u;
                u.x = v[0] | (v[1] << 8) | (v[2] << 16) | ((uint32_t)v[3] << 24);
                u.y = v[4] | (v[5] << 8) | (v[6] << 16) | ((uint32_t)v[7] << 24);
                u.z = v[8] | (v[9] << 8) | (v[10] << 16) | ((uint32_t)v[11] << 24);
                u.w = v[12] | (v[13] << 8) | (v[14] << 16) | ((uint32_t)v[15] << 24);
                __builtin_nontemporal_store(u, reinterpret_cast<u32x4 *>(out + A));
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (A + i >= a0 && A + i < end) out[A + i] = v[i];
            }
        }
      }
    }
    if (tid == 0 && part == 0) spec::raise_status(status, err);
}

__global__ __launch_bounds__(kThreads) void plan_branches_kernel(
    int topk, int num_steps, int page_size, int max_pages, int pages_per_branch, int row16,
    int64_t num_pages, int64_t layer_stride16, uint4 *__restrict__ k_pool,
    uint4 *__restrict__ v_pool, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ branch_pages,
    int32_t *__restrict__ out_cache_loc, int32_t *__restrict__ status) {
    __shared__ int s_err;
    const int b = blockIdx.x, layer = blockIdx.y, part = blockIdx.z, tid = threadIdx.x;
    if (tid == 0) s_err = 0;
    __syncthreads();
    int err = 0;
    int L = seq_lens[b];
    if (L < 0) {
        err |= SPEC_ST_RANGE;
        L = 0;
    }
    const int tail = L % page_size;
    const int32_t *pt = page_table + (int64_t)b * max_pages;
    const int32_t *bp = branch_pages + (int64_t)b * topk * pages_per_branch;
    // the draft write slots
    if (layer == 0 && part == 0) {
        for (int q = tid; q < topk * num_steps; q += kThreads) {
            const int j = q / num_steps, s = q % num_steps;
            int64_t page = -1;
            int off = 0;
            if (topk == 1) {
                const int64_t pos = (int64_t)L + s;
                if (pos / page_size < max_pages) page = pt[pos / page_size];
                off = (int)(pos % page_size);
            } else {
                const int t = tail + s;           // < pages_per_branch * page_size (host check)
                page = bp[(int64_t)j * pages_per_branch + t / page_size];
                off = t % page_size;
            }
            int32_t slot = -1;
            if (page < 0 || page >= num_pages)
                err |= SPEC_ST_RANGE;
            else
                slot = (int32_t)(page * page_size + off);
            out_cache_loc[((int64_t)b * topk + j) * num_steps + s] = slot;
        }
    }
    // the prefix tail's KV into every branch region's first slots
    if (topk > 1 && tail > 0) {
        const int64_t src_page = L / page_size < max_pages ? pt[L / page_size] : -1;
        if (src_page < 0 || src_page >= num_pages) {
            err |= SPEC_ST_RANGE;
        } else {
            // this workgroup's kThreads * kPer units of the topk * tail rows
            const int64_t units = (int64_t)topk * tail * row16;
            uint4 *kl = k_pool + layer * layer_stride16;
            uint4 *vl = v_pool + layer * layer_stride16;
            int64_t dst[kPer];
            uint4 kv[kPer], vv[kPer];
#pragma unroll
            for (int h = 0; h < kPer; ++h) {
                const int64_t q = ((int64_t)part * kPer + h) * kThreads + tid;
                dst[h] = -1;
                kv[h] = make_uint4(0, 0, 0, 0);
                vv[h] = kv[h];
                if (q < units) {
                    const int u = (int)(q % row16);
                    const int t = (int)((q / row16) % tail);
                    const int j = (int)(q / ((int64_t)row16 * tail));
                    const int64_t dst_page = bp[(int64_t)j * pages_per_branch];   // t < page_size
                    if (dst_page < 0 || dst_page >= num_pages) {
                        err |= SPEC_ST_RANGE;
                    } else {
                        const int64_t src = (src_page * page_size + t) * row16 + u;
                        dst[h] = (dst_page * page_size + t) * row16 + u;
                        kv[h] = kl[src];
                        vv[h] = vl[src];
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < kPer; ++h) {
                if (dst[h] >= 0) {
                    kl[dst[h]] = kv[h];
                    vl[dst[h]] = vv[h];
                }
            }
        }
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0) spec::raise_status(status, s_err);
}

}  // namespace

extern "C" int spec_full_mask(int batch, int num_draft_tokens, const int32_t *seq_lens,
                              int max_seq_len, const void *tree_mask_bits, int fill_prefix,
                              void *full_mask, int64_t full_mask_bytes, int32_t *dev_status,
                              spec_stream_t stream) {
    const int n = num_draft_tokens;
    if (batch < 0 || n < 1 || max_seq_len < 0 || full_mask_bytes < 0) return SPEC_ERR_SHAPE;
    const int wb = spec_mask_word_bytes(n);
    if (wb == 0) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!seq_lens || !tree_mask_bits || !full_mask) return SPEC_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(tree_mask_bits) % wb != 0 ||
        reinterpret_cast<uintptr_t>(full_mask) % 16 != 0)
        return SPEC_ERR_SHAPE;
    const int64_t wmax = (int64_t)max_seq_len + n;
    const int64_t per_row = fill_prefix ? ((wmax / 16 + 2) * 16 + kRowSpan - 1) / kRowSpan : 1;
    const int64_t grid = (int64_t)batch * n * per_row;
    if (grid > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(full_mask_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), n, wb, max_seq_len, (int)per_row,
                       fill_prefix ? 1 : 0, seq_lens, static_cast<const uint8_t *>(tree_mask_bits),
                       static_cast<uint8_t *>(full_mask), full_mask_bytes, dev_status);
    return spec::launch_status();
}

extern "C" int spec_plan_draft_branches(int batch, int topk, int num_steps, int page_size,
                                        int num_layers, int num_kv_heads, int head_dim,
                                        int dtype, void *k_pool, void *v_pool,
                                        int64_t num_slots, const int32_t *seq_lens,
                                        const int32_t *page_table, int max_pages,
                                        const int32_t *branch_pages, int pages_per_branch,
                                        int32_t *out_cache_loc, int32_t *dev_status,
                                        spec_stream_t stream) {
    if (batch < 0 || topk < 1 || num_steps < 1 || page_size < 1 || num_layers < 1 ||
        num_kv_heads < 1 || head_dim < 1 || num_slots < 0 || max_pages < 1 ||
        pages_per_branch < 0)
        return SPEC_ERR_SHAPE;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    // a branch region must hold the longest tail and every draft step
    if (topk > 1 && (int64_t)pages_per_branch * page_size < (int64_t)page_size - 1 + num_steps)
        return SPEC_ERR_SHAPE;
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * (dtype == SPEC_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0) return SPEC_ERR_UNSUPPORTED;
    if (num_slots > INT_MAX) return SPEC_ERR_UNSUPPORTED;    // slots are written as int32
    if (batch == 0) return SPEC_OK;
    if (!k_pool || !v_pool || !seq_lens || !page_table || !out_cache_loc ||
        (topk > 1 && !branch_pages))
        return SPEC_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15u)
        return SPEC_ERR_SHAPE;
    const int row16 = (int)(row_bytes / 16);
    // copy units of a (request, layer): at most topk * (page_size - 1) rows
    const int64_t max_units = topk > 1 ? (int64_t)topk * (page_size - 1) * row16 : 0;
    const int64_t parts = std::max<int64_t>(1, (max_units + kThreads * kPer - 1) / (kThreads * kPer));
    if (parts > 65535) return SPEC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(plan_branches_kernel, dim3(batch, num_layers, (unsigned)parts), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), topk, num_steps, page_size,
                       max_pages, pages_per_branch, row16, num_slots / page_size,
                       num_slots * row16, static_cast<uint4 *>(k_pool),
                       static_cast<uint4 *>(v_pool), seq_lens, page_table, branch_pages,
                       out_cache_loc, dev_status);
    return spec::launch_status();
}
