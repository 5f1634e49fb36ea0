// Greedy tree accept: per-row argmax over the vocabulary, then the tree walk.
//
// Follows "SGLang 源码完全拆解(十一):投机解码" (三条判定路径: argmax per verify
// row, then the first-child / next-sibling walk) and "投机解码 Accept:从 Verify
// 行到最终输出路径" (三: accept_index holds verify rows; the last row's target
// choice is the terminal token).
//
// Two launches, neither of which waits for another workgroup:
// * the sweep: workgroup t loads 8192-entry chunk t % nchunks of verify row
//   t / nchunks once (16-byte loads), finds its best entry and folds it, as
//   one 64-bit key, into the row's key with an atomic max (no return, so the
//   workgroup ends at once);
// * the walk: one workgroup per request reads its rows' keys (every atomic
//   of the sweep is complete at the kernel boundary), clears them for the
//   next call (the workspace is zero after every call), finds every node's
//   matching child in parallel and follows them from the root.
// Nothing depends on which workgroups are resident, so the same two
// launches run eagerly and recorded into a graph.
#include <algorithm>
#include <mutex>

#include "sweep_common.h"

using namespace spec;

namespace {

// A row's best entry as one 64-bit key: the value's order-preserving bits
// above, 0xFFFFFFFF - index below, so a larger key is a larger value or,
// for equal values, a smaller index (the first index of the row maximum).
// 0 is no entry; -0 is keyed as +0, the two comparing equal.
__device__ __forceinline__ uint64_t arg_key(float v, int i) {
    if (i < 0) return 0;
    uint32_t bits = __float_as_uint(v == 0.f ? 0.f : v);
    bits = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    return ((uint64_t)bits << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ int arg_key_index(uint64_t key) {
    return key == 0 ? -1 : (int)(0xFFFFFFFFu - (uint32_t)key);
}

struct GreedyArgs {
    const void *logits;
    int64_t vocab;
    bool vec_ok;
    int batch, n, s1, nchunks;
    const int32_t *cand, *r_index, *r_next, *r_sib;
    int32_t *predict, *accept_index, *accept_length, *target_predict, *status;
    uint64_t *keys;      // [batch * n] row keys: 0 on entry, the row's best after the sweep
};

// Sweep: the best entry of chunk t % nchunks of verify row t / nchunks,
// folded into the row's key.
template <int DT>
__global__ __launch_bounds__(kSweepThreads) void greedy_sweep_kernel(GreedyArgs A) {
    __shared__ uint64_t s_wave[kSweepThreads / SPEC_WAVE];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t row = t / A.nchunks;
    const int64_t start = (t % A.nchunks) * kChunk;
    const int64_t end = min(A.vocab, start + kChunk);
    const char *rowp = static_cast<const char *>(A.logits) + row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
    float x[kPerThread];
    load_chunk<DT>(rowp, start, end, A.vec_ok, tid, x);
    float bv = -INFINITY;
    int bi = -1;
    if (end - start == kChunk) {
        // a whole chunk: the thread's maximum, then the first of its entries
        // (they ascend in index with e) equal to it
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) bv = fmaxf(bv, x[e]);
        int be = 0;
#pragma unroll
        for (int e = kPerThread - 1; e >= 0; --e) be = x[e] == bv ? e : be;
        bi = (int)elem_index(start, tid, be);
    } else {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {   // e increases with element index
            const int64_t idx = elem_index(start, tid, e);
            if (idx < end && (bi < 0 || x[e] > bv)) {
                bv = x[e];
                bi = (int)idx;
            }
        }
    }
    uint64_t key = arg_key(bv, bi);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t other = __shfl_xor(key, o, SPEC_WAVE);
        key = other > key ? other : key;
    }
    if ((tid & 63) == 0) s_wave[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int w = 1; w < kSweepThreads / SPEC_WAVE; ++w) key = s_wave[w] > key ? s_wave[w] : key;
        __hip_atomic_fetch_max(A.keys + row, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Walk: request blockIdx.x.  Its tree and its rows' keys are loaded
// together; the keys are cleared; every node's thread scans its own child
// list for the child holding its row's choice; one thread then follows those
// children from the root and the outputs are written.
__global__ __launch_bounds__(kSweepThreads) void greedy_walk_kernel(GreedyArgs A) {
    __shared__ int s_tp[kMaxNodes], s_row[kMaxNodes], s_pred[kMaxNodes];
    __shared__ int s_cand[kMaxNodes], s_sib[kMaxNodes], s_hit[kMaxNodes], s_bad[kMaxNodes];
    __shared__ int s_ai[kMaxNodes + 1];
    __shared__ int s_len, s_err;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = A.n;
    const int base = b * n;
    if (tid == 0) s_err = 0;
    int err = 0;
    if (tid < n) {
        int row = A.r_index[base + tid];
        const int next = A.r_next[base + tid];
        s_cand[tid] = A.cand[base + tid];
        s_sib[tid] = A.r_sib[base + tid];
        const uint64_t key = A.keys[base + tid];      // row base + tid's key
        A.keys[base + tid] = 0;
        s_tp[tid] = arg_key_index(key);               // indexed by row here
        if (row < base || row >= base + n) { err |= SPEC_ST_RANGE; row = -1; }
        s_row[tid] = row;
        s_pred[tid] = 0;
        s_hit[tid] = next;                            // the first child, for now
    }
    __syncthreads();
    // node tid's choice (its row's key) and first child in sibling order
    // holding it
    int want = -1, hit = -1, bad = 0;
    if (tid < n) {
        want = s_row[tid] >= 0 ? s_tp[s_row[tid] - base] : -1;
        int c = s_hit[tid];
        for (int steps = 0; c != -1 && steps < n; ++steps) {
            if (c < 0 || c >= n) { bad = SPEC_ST_RANGE; break; }
            if (s_cand[c] == want) { hit = c; break; }
            c = s_sib[c];
        }
    }
    __syncthreads();
    if (tid < n) {
        s_tp[tid] = want;                             // indexed by node from here on
        s_hit[tid] = hit;
        s_bad[tid] = bad;
    }
    __syncthreads();
    if (tid == 0) {
        int cur = 0, cnt = 0, werr = 0;
        s_ai[0] = s_row[0];
        for (int guard = 0; guard < n; ++guard) {
            werr |= s_bad[cur];
            const int h = s_hit[cur];
            if (h < 0) break;
            if (cnt + 1 >= A.s1) { werr |= SPEC_ST_DEPTH; break; }
            s_pred[cur] = s_cand[h];
            ++cnt;
            s_ai[cnt] = s_row[h];
            cur = h;
        }
        s_pred[cur] = s_tp[cur];
        s_len = cnt + 1;
        err |= werr;
    }
    __syncthreads();
    if (tid < n && s_row[tid] >= 0) {
        A.predict[s_row[tid]] = s_pred[tid];
        if (A.target_predict != nullptr) A.target_predict[s_row[tid]] = s_tp[tid];
    }
    for (int j = tid; j < A.s1; j += blockDim.x)
        A.accept_index[(int64_t)b * A.s1 + j] = (j < s_len) ? s_ai[j] : -1;
    if (tid == 0) A.accept_length[b] = s_len;
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (tid == 0) raise_status(A.status, s_err);
}

}  // namespace

size_t spec_greedy_workspace_bytes(int batch, int n, int64_t vocab) {
    (void)vocab;
    return spec::align_up((size_t)batch * n * sizeof(uint64_t), 256);
}

int spec_check_accept_args(int batch, int n, int s1, int64_t vocab, int dtype) {
    if (batch < 0 || n < 1 || s1 < 1 || vocab < 1) return SPEC_ERR_SHAPE;
    if (n > kMaxNodes || s1 > kMaxNodes + 1) return SPEC_ERR_UNSUPPORTED;
    if (vocab > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    return SPEC_OK;
}

namespace {

// Validated launch of the greedy accept over the row keys `keys` (zero on
// entry; left zero).
int launch_greedy(int batch, int n, int s1, int64_t vocab, int dtype, const void *target_logits,
                  const int32_t *candidates, const int32_t *retrieve_index,
                  const int32_t *retrieve_next_token, const int32_t *retrieve_next_sibling,
                  int32_t *predict, int32_t *accept_index, int32_t *accept_length,
                  int32_t *target_predict, uint64_t *keys, int32_t *dev_status, hipStream_t st) {
    const int nch = num_chunks(vocab);
    const int64_t items = (int64_t)batch * n * nch;
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    GreedyArgs A{};
    A.logits = target_logits;
    A.vocab = vocab;
    A.vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0;
    A.batch = batch;
    A.n = n;
    A.s1 = s1;
    A.nchunks = nch;
    A.cand = candidates;
    A.r_index = retrieve_index;
    A.r_next = retrieve_next_token;
    A.r_sib = retrieve_next_sibling;
    A.predict = predict;
    A.accept_index = accept_index;
    A.accept_length = accept_length;
    A.target_predict = target_predict;
    A.status = dev_status;
    A.keys = keys;
    const dim3 grid((unsigned)items);
    if (dtype == SPEC_BF16)
        hipLaunchKernelGGL((greedy_sweep_kernel<SPEC_BF16>), grid, dim3(kSweepThreads), 0, st, A);
    else
        hipLaunchKernelGGL((greedy_sweep_kernel<SPEC_F32>), grid, dim3(kSweepThreads), 0, st, A);
    hipLaunchKernelGGL(greedy_walk_kernel, dim3(batch), dim3(kSweepThreads), 0, st, A);
    return spec::launch_status();
}

// Host checks shared by both entry points: SPEC_OK, a SPEC_ERR_* code, or 1
// for a valid empty call.
int check_greedy(int batch, int n, int s1, int64_t vocab, int dtype, const void *target_logits,
                 const int32_t *candidates, const int32_t *retrieve_index,
                 const int32_t *retrieve_next_token, const int32_t *retrieve_next_sibling,
                 const int32_t *predict, const int32_t *accept_index,
                 const int32_t *accept_length) {
    int rc = spec_check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (batch == 0) return 1;
    if (!target_logits || !candidates || !retrieve_index || !retrieve_next_token ||
        !retrieve_next_sibling || !predict || !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if ((int64_t)batch * n * num_chunks(vocab) > INT_MAX) return SPEC_ERR_UNSUPPORTED;
    return SPEC_OK;
}

}  // namespace

extern "C" int spec_accept_greedy(int batch, int n, int s1, int64_t vocab, int dtype,
                                  const void *target_logits, const int32_t *candidates,
                                  const int32_t *retrieve_index,
                                  const int32_t *retrieve_next_token,
                                  const int32_t *retrieve_next_sibling, int32_t *predict,
                                  int32_t *accept_index, int32_t *accept_length,
                                  int32_t *target_predict, void *workspace,
                                  size_t workspace_bytes, int32_t *dev_status,
                                  spec_stream_t stream) {
    const int rc = check_greedy(batch, n, s1, vocab, dtype, target_logits, candidates,
                                retrieve_index, retrieve_next_token, retrieve_next_sibling,
                                predict, accept_index, accept_length);
    if (rc != SPEC_OK) return rc == 1 ? SPEC_OK : rc;
    if (!workspace || workspace_bytes < spec_greedy_workspace_bytes(batch, n, vocab) ||
        reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return SPEC_ERR_WORKSPACE;
    return launch_greedy(batch, n, s1, vocab, dtype, target_logits, candidates, retrieve_index,
                         retrieve_next_token, retrieve_next_sibling, predict, accept_index,
                         accept_length, target_predict, static_cast<uint64_t *>(workspace),
                         dev_status, reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: the row keys live in a fixed
// array of the library, one copy per device.
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kNoAllocKeys = 32768;     // 256 KiB of 64-bit row keys
static __device__ __align__(256) uint64_t scratch[kNoAllocKeys];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
uint64_t *scratch_ptr[kMaxDevices];         // written once per device, under scratch_once

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with it current), or null if the lookup failed.  The
// array's host-side name is not a device address and is never passed on.
uint64_t *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(scratch_once[dev], [dev] {
        void *p = nullptr;
        scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess
                               ? static_cast<uint64_t *>(p) : nullptr;
    });
    return scratch_ptr[dev];
}

__global__ __launch_bounds__(256) void clear_keys_kernel(uint64_t *keys, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * 256)
        keys[i] = 0;
}

}  // namespace

extern "C" int spec_accept_greedy_noalloc(int batch, int n, int s1, int64_t vocab, int dtype,
                                          const void *target_logits, const int32_t *candidates,
                                          const int32_t *retrieve_index,
                                          const int32_t *retrieve_next_token,
                                          const int32_t *retrieve_next_sibling,
                                          int32_t *predict, int32_t *accept_index,
                                          int32_t *accept_length, int32_t *target_predict,
                                          int32_t *dev_status, spec_stream_t stream) {
    const int rc = check_greedy(batch, n, s1, vocab, dtype, target_logits, candidates,
                                retrieve_index, retrieve_next_token, retrieve_next_sibling,
                                predict, accept_index, accept_length);
    if (rc != SPEC_OK) return rc == 1 ? SPEC_OK : rc;
    const int64_t used = (int64_t)batch * n;
    if (used > kNoAllocKeys) return SPEC_ERR_WORKSPACE;
    uint64_t *keys = scratch_address();
    if (keys == nullptr) return SPEC_ERR_HIP;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // every call leaves the keys it used zero, but the array is shared by
    // every call on the device (one on another stream may overlap): the
    // keys this call uses start at zero
    const unsigned blocks = (unsigned)std::min<int64_t>((used + 255) / 256, 512);
    hipLaunchKernelGGL(clear_keys_kernel, dim3(blocks), dim3(256), 0, st, keys, used);
    if (hipPeekAtLastError() != hipSuccess) return spec::launch_status();
    return launch_greedy(batch, n, s1, vocab, dtype, target_logits, candidates, retrieve_index,
                         retrieve_next_token, retrieve_next_sibling, predict, accept_index,
                         accept_length, target_predict, keys, dev_status, st);
}
