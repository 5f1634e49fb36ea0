// Target-only tree accept: per-chunk softmax statistics of every verify row,
// then the tree walk with the sibling-mass rule.
//
// Follows "投机解码 Accept:从 Verify 行到最终输出路径" (四, Target-only Tree
// Sampling) with the two thresholds of "SGLang 源码完全拆解(十一)" (三条判定
// 路径): at node cur, p = softmax(target_logits[row(cur)] / T); the children
// are tried in sibling order, each adding p(token) to a running mass, and a
// child is accepted iff p(token) > 0 and (coin < mass / threshold_acc or
// p(token) >= threshold_single), the coin of cur's children being
// uniforms[b][cur].  A rejected child's p(token) goes into the row's work
// buffer, so the terminal token is drawn (inverse CDF in vocabulary order,
// final_uniforms[b]) from relu(p - buffer): p with the rejected children's
// tokens removed.  No draft distribution is read.
//
// Work item t (verify row t / nchunks, 8192-entry chunk t % nchunks) is
// workgroup t of the grid: it reads the chunk once and writes the chunk's
// max m and sum s = sum exp((x - m) / T) (float32 exponentials, float64 sum)
// to write-once slot t, both words XOR-coded so that 0 means unwritten (the
// exponentials come from the hardware base-2 exponential with the argument
// carried as a float pair).
// The last `batch` workgroups then walk a request each: a visited row's
// statistics come from its slots, the children's probabilities from their
// logits alone; the terminal draw finds the chunk holding the crossing from
// the chunk masses and scans only that chunk.  Every slot of the request is
// polled and cleared before the walker ends (the workspace is zero after
// every call).  Walkers wait only for chunk work, which never waits; with
// fewer walkers than the device holds at once, one launch suffices,
// otherwise (and whenever the call is recorded into a graph, where other
// streams' kernels may hold the device) a second launch walks.
#include "sweep_common.h"

using namespace spec;

namespace {

constexpr uint64_t kCode = 0x7FF4DEAD0BADF00Dull;   // XOR code: a NaN pattern no
                                                    // max or sum takes
constexpr int kScanPer = kChunk / kSweepThreads;   // entries per thread, terminal scan
constexpr int kChunksPerThread = 4;                 // a walker thread's chunk statistics,
                                                    // kept in registers
constexpr int64_t kMaxVocab = (int64_t)kChunksPerThread * kSweepThreads * kChunk;

__device__ __forceinline__ uint64_t encode(uint64_t bits) {
    return bits ^ kCode;
}

struct TargetArgs {
    const void *logits;
    int64_t vocab;
    bool vec_ok;
    int batch, n, s1, nchunks;
    const float *temperature, *uniforms, *final_uniforms;
    double ts, ta;                      // threshold_single, threshold_acc
    const int32_t *cand, *r_index, *r_next, *r_sib;
    int32_t *predict, *accept_index, *accept_length, *status;
    uint64_t *slots;                    // [batch * n][nchunks][2] (max bits, sum bits), coded
    unsigned poll_limit;                // polls of one slot before giving up
};

template <int DT>
__device__ __forceinline__ float logit_at(const TargetArgs &A, int64_t row, int64_t v) {
    const char *p = static_cast<const char *>(A.logits) + row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
    if (DT == SPEC_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[v]);
    return reinterpret_cast<const float *>(p)[v];
}

__device__ __forceinline__ float block_max(float v, float *s_f) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, SPEC_WAVE));
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) s_f[tid >> 6] = v;
    __syncthreads();
    float r = s_f[0];
#pragma unroll
    for (int w = 1; w < kSweepThreads / SPEC_WAVE; ++w) r = fmaxf(r, s_f[w]);
    return r;
}

__device__ __forceinline__ double block_sum_d(double v, double *s_d) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, SPEC_WAVE);
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) s_d[tid >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) r += s_d[w];
    return r;
}

// exclusive prefix of v over the threads in thread order; total in `total`
__device__ __forceinline__ double block_exclusive_d(double v, double *s_d, double &total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, SPEC_WAVE);
        if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) s_d[wave] = incl;
    __syncthreads();
    double before = 0.0;
    total = 0.0;
#pragma unroll
    for (int w = 0; w < kSweepThreads / SPEC_WAVE; ++w) {
        if (w < wave) before += s_d[w];
        total += s_d[w];
    }
    return before + incl - v;
}

// Max and sum of exponentials of chunk t % nchunks of verify row t / nchunks
// into slot t.
template <int DT>
__device__ __forceinline__ void chunk_item(const TargetArgs &A, int64_t t, float *s_f, double *s_d) {
    const int tid = threadIdx.x;
    const int64_t row = t / A.nchunks;
    const int64_t start = (t % A.nchunks) * kChunk;
    const int64_t end = min(A.vocab, start + kChunk);
    const char *rowp = static_cast<const char *>(A.logits) + row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
    float x[kPerThread];
    load_chunk<DT>(rowp, start, end, A.vec_ok, tid, x);
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
    m = block_max(m, s_f);
    const Scale2 sc = make_scale2(m, A.temperature[row / A.n]);
    double s = 0.0;
    if (m != -INFINITY) {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) s += (double)exp2_scaled(x[e], sc);
    }
    s = block_sum_d(s, s_d);
    if (tid == 0) {
        uint64_t *slot = A.slots + 2 * t;
        __hip_atomic_store(slot, encode(__float_as_uint(m)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, encode(__builtin_bit_cast(uint64_t, s)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Both words of a slot, polled until written (bounded); false on timeout.
__device__ __forceinline__ bool read_slot(const uint64_t *slot, unsigned limit, float &m,
                                          double &s) {
    uint64_t w0 = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t w1 = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned spins = 0; w0 == 0 || w1 == 0; ++spins) {
        if (spins >= limit) {
            m = -INFINITY;
            s = 0.0;
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
        w0 = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w1 = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    m = __uint_as_float((uint32_t)encode(w0));
    s = __builtin_bit_cast(double, encode(w1));
    return true;
}

struct WalkShared {
    int cand[kMaxNodes], next[kMaxNodes], sib[kMaxNodes], row[kMaxNodes], pred[kMaxNodes];
    int ai[kMaxNodes + 1];
    int kid[kMaxNodes];        // children of the current node, sibling order
    float xk[kMaxNodes];       // their logits in the current row
    int rejtok[kMaxNodes];     // rejected children's tokens at the current node
    float rejx[kMaxNodes];     // and their logits
    float cmax[kChunksPerThread * kSweepThreads];   // the current row's chunk maxima
    float coin[kMaxNodes];     // uniforms[b][k]: the coin of node k's children
    float ufinal;
    float f[kSweepThreads / SPEC_WAVE];
    double d[kSweepThreads / SPEC_WAVE];
    double tgt;
    int nk, nrej, hit, err, owner, draw;
};

// Request b: walk from the root with the target-only rule, draw the
// terminal token, write the outputs, then clear the request's slots.
template <int DT>
__device__ void walk_request(const TargetArgs &A, int b) {
    __shared__ WalkShared S;
    const int tid = threadIdx.x;
    const int n = A.n;
    const int64_t base = (int64_t)b * n;
    const int nch = A.nchunks;
    const Scale2 tsc = make_scale2(0.f, A.temperature[b]);   // 1/T pair, rebased per max
    if (tid == 0) {
        S.err = 0;
        S.ufinal = A.final_uniforms[b];
    }
    __syncthreads();
    if (tid < n) {
        S.coin[tid] = A.uniforms[base + tid];
        int row = A.r_index[base + tid];
        int err = 0;
        if (row < base || row >= base + n) {
            err |= SPEC_ST_RANGE;
            row = -1;
        }
        S.row[tid] = row;
        S.cand[tid] = A.cand[base + tid];
        S.next[tid] = A.r_next[base + tid];
        S.sib[tid] = A.r_sib[base + tid];
        S.pred[tid] = 0;
        if (err) atomicOr(&S.err, err);
    }
    __syncthreads();
    if (tid == 0) S.ai[0] = S.row[0];
    // chunks of this thread: a contiguous run (thread order is chunk order),
    // their (max, sum) kept in registers for the current row
    const int j0 = min(nch, tid * kChunksPerThread);
    float cm[kChunksPerThread];
    double cs[kChunksPerThread];
    int cur = 0, cnt = 0;
    float M = -INFINITY;
    double Z = 0.0;
    int64_t row = -1;
    bool sync_ok = true;
    for (int guard = 0; guard <= n; ++guard) {
        row = S.row[cur];
        if (row < 0) break;
        // children of cur in sibling order
        if (tid == 0) {
            int c = S.next[cur], k = 0, err = 0;
            for (int steps = 0; c != -1 && steps < n; ++steps) {
                if (c < 0 || c >= n) {
                    err |= SPEC_ST_RANGE;
                    break;
                }
                S.kid[k++] = c;
                c = S.sib[c];
            }
            S.nk = k;
            S.nrej = 0;
            S.hit = -1;
            if (err) S.err |= err;
        }
        __syncthreads();
        const int nk = S.nk;
        // the row's chunk statistics and the children's logits, loaded together
        float xk = -INFINITY;
        if (tid < nk) {
            const int tok = S.cand[S.kid[tid]];
            if (tok >= 0 && tok < A.vocab) xk = logit_at<DT>(A, row, tok);
            else atomicOr(&S.err, SPEC_ST_RANGE);
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int k = 0; k < kChunksPerThread; ++k) {
            cm[k] = -INFINITY;
            cs[k] = 0.0;
            if (j0 + k < nch) {
                sync_ok &= read_slot(A.slots + 2 * (row * nch + j0 + k), A.poll_limit, cm[k], cs[k]);
                S.cmax[j0 + k] = cm[k];
            }
            mloc = fmaxf(mloc, cm[k]);
        }
        M = block_max(mloc, S.f);
        const Scale2 gsc = rebase(tsc, M);
        double zloc = 0.0;
#pragma unroll
        for (int k = 0; k < kChunksPerThread; ++k)
            if (cm[k] != -INFINITY) zloc += cs[k] * (double)exp2_scaled(cm[k], gsc);
        Z = block_sum_d(zloc, S.d);
        if (tid < nk) S.xk[tid] = xk;
        __syncthreads();
        // the sibling-mass test, in sibling order
        if (tid == 0) {
            const double coin = (double)S.coin[cur];
            const double rz = Z > 0.0 ? 1.0 / Z : 0.0;
            double mass = 0.0;
            for (int i = 0; i < nk; ++i) {
                const double p = (double)exp2_scaled(S.xk[i], gsc) * rz;
                mass += p;
                if (p > 0.0 && (coin < mass / A.ta || p >= A.ts)) {
                    S.hit = S.kid[i];
                    break;
                }
                S.rejtok[S.nrej] = S.cand[S.kid[i]];
                S.rejx[S.nrej] = S.xk[i];
                ++S.nrej;
            }
            if (S.hit >= 0) {
                if (cnt + 1 >= A.s1) {
                    S.err |= SPEC_ST_DEPTH;
                    S.hit = -2;                 // stop here, the draw is at cur
                } else {
                    S.pred[cur] = S.cand[S.hit];
                    S.ai[cnt + 1] = S.row[S.hit];
                }
            }
        }
        __syncthreads();
        const int hit = S.hit;
        if (hit < 0) break;
        ++cnt;
        cur = hit;
    }

    // ---- terminal draw: inverse CDF of p without the rejected tokens ------
    int x = -1;
    if (row >= 0) {
        const Scale2 gsc = rebase(tsc, M);
        const int nrej = S.nrej;
        // my chunks' masses in the row's scale, each chunk's rejected entries
        // (same float exponentials as the chunk's sum) taken out
        double cmass[kChunksPerThread];
        double mine = 0.0;
#pragma unroll
        for (int k = 0; k < kChunksPerThread; ++k) {
            cmass[k] = 0.0;
            if (cm[k] == -INFINITY) continue;
            const Scale2 csc = rebase(tsc, cm[k]);
            double sk = cs[k];
            for (int i = 0; i < nrej; ++i) {
                const int tok = S.rejtok[i];
                if (tok >= 0 && tok < A.vocab && tok / kChunk == j0 + k)
                    sk -= (double)exp2_scaled(S.rejx[i], csc);
            }
            cmass[k] = fmax(sk, 0.0) * (double)exp2_scaled(cm[k], gsc);
            mine += cmass[k];
        }
        double total;
        const double before = block_exclusive_d(mine, S.d, total);
        const double target = (double)S.ufinal * total;
        if (tid == 0) {
            S.owner = -1;
            S.draw = INT_MAX;
            if (!(total > 0.0)) S.err |= SPEC_ST_ZERO_RESIDUAL;
        }
        __syncthreads();
        // the thread whose chunks hold the crossing names the chunk
        if (mine > 0.0 && before <= target && target < before + mine) {
            double run = before, last_run = before;
            int own = -1, last = -1;
#pragma unroll
            for (int k = 0; k < kChunksPerThread; ++k) {
                if (own < 0 && cmass[k] > 0.0) {
                    if (target < run + cmass[k]) {
                        own = j0 + k;
                        S.tgt = target - run;
                    }
                    last = j0 + k;
                    last_run = run;
                }
                if (own < 0) run += cmass[k];
            }
            if (own < 0) {               // summed in another order, the run fell an ulp short
                own = last;
                S.tgt = target - last_run;
            }
            S.owner = own;
        }
        __syncthreads();
        const int j = S.owner;
        if (j >= 0) {
            // scan chunk j in vocabulary order: thread tid owns kScanPer
            // consecutive entries, loaded 16 bytes at a time when aligned
            const float m = S.cmax[j];
            const Scale2 csc = rebase(tsc, m);
            const double scale = (double)exp2_scaled(m, gsc);
            const int64_t v0 = (int64_t)j * kChunk + (int64_t)tid * kScanPer;
            const int64_t vend = min(A.vocab, (int64_t)(j + 1) * kChunk);
            const char *rowp = static_cast<const char *>(A.logits) +
                               row * A.vocab * (DT == SPEC_BF16 ? 2 : 4);
            float xs[kScanPer];
#pragma unroll
            for (int g = 0; g < kScanPer / 8; ++g) {
                const int64_t e0 = v0 + 8 * g;
                if (DT == SPEC_BF16) {
                    const uint16_t *p = reinterpret_cast<const uint16_t *>(rowp);
                    if (A.vec_ok && e0 + 8 <= vend) {
                        const uint4 w = *reinterpret_cast<const uint4 *>(p + e0);
                        xs[8 * g + 0] = lo_bf16(w.x); xs[8 * g + 1] = hi_bf16(w.x);
                        xs[8 * g + 2] = lo_bf16(w.y); xs[8 * g + 3] = hi_bf16(w.y);
                        xs[8 * g + 4] = lo_bf16(w.z); xs[8 * g + 5] = hi_bf16(w.z);
                        xs[8 * g + 6] = lo_bf16(w.w); xs[8 * g + 7] = hi_bf16(w.w);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            xs[8 * g + i] = e0 + i < vend ? bf16_to_f32(p[e0 + i]) : -INFINITY;
                    }
                } else {
                    const float *p = reinterpret_cast<const float *>(rowp);
                    if (A.vec_ok && e0 + 8 <= vend) {
                        const float4 u = *reinterpret_cast<const float4 *>(p + e0);
                        const float4 w = *reinterpret_cast<const float4 *>(p + e0 + 4);
                        xs[8 * g + 0] = u.x; xs[8 * g + 1] = u.y; xs[8 * g + 2] = u.z; xs[8 * g + 3] = u.w;
                        xs[8 * g + 4] = w.x; xs[8 * g + 5] = w.y; xs[8 * g + 6] = w.z; xs[8 * g + 7] = w.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) xs[8 * g + i] = e0 + i < vend ? p[e0 + i] : -INFINITY;
                    }
                }
            }
            // rejected tokens in my range read as -inf (weight 0)
            for (int i = 0; i < nrej; ++i) {
                const int64_t off = (int64_t)S.rejtok[i] - v0;
#pragma unroll
                for (int q = 0; q < kScanPer; ++q)
                    if (off == q) xs[q] = -INFINITY;
            }
            double e[kScanPer];
            double mine2 = 0.0;
#pragma unroll
            for (int i = 0; i < kScanPer; ++i) {
                e[i] = (double)exp2_scaled(xs[i], csc) * scale;
                mine2 += e[i];
            }
            double tot2;
            const double before2 = block_exclusive_d(mine2, S.d, tot2);
            const double tgt = S.tgt;
            if (mine2 > 0.0 && before2 <= tgt && tgt < before2 + mine2) {
                double run = before2;
                int found = -1;
#pragma unroll
                for (int i = 0; i < kScanPer; ++i) {
                    run += e[i];
                    if (found < 0 && e[i] > 0.0 && run > tgt) found = i;
                }
                if (found >= 0) atomicMin(&S.draw, (int)(v0 + found));
            }
            __syncthreads();
            // rounding can leave the crossing just past the scanned total:
            // the chunk's last entry
            x = S.draw != INT_MAX ? S.draw : (int)(vend - 1);
        } else {
            x = (int)(A.vocab - 1);    // no crossing: the target sits at the end of the mass
        }
    }
    if (!sync_ok) atomicOr(&S.err, SPEC_ST_SYNC);
    __syncthreads();
    if (tid < n && S.row[tid] >= 0) {
        int v = S.pred[tid];
        if (tid == cur && row >= 0) v = x;
        A.predict[S.row[tid]] = v;
    }
    for (int k = tid; k < A.s1; k += blockDim.x)
        A.accept_index[(int64_t)b * A.s1 + k] = k <= cnt ? S.ai[k] : -1;
    if (tid == 0) A.accept_length[b] = cnt + 1;

    // every slot of the request, visited or not, is read once written and
    // cleared for the next call
    const int nslots = n * nch;
    uint64_t *rs = A.slots + 2 * base * nch;
    bool ok = true;
    for (int q = tid; q < nslots; q += blockDim.x) {
        float m;
        double sv;
        ok &= read_slot(rs + 2 * q, A.poll_limit, m, sv);
        __hip_atomic_store(rs + 2 * q, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(rs + 2 * q + 1, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!ok) atomicOr(&S.err, SPEC_ST_SYNC);
    __syncthreads();
    if (tid == 0) raise_status(A.status, S.err);
}

// Chunk work for every (row, chunk); with WALK the last `batch` workgroups
// then walk a request each.
template <int DT, bool WALK>
__global__ __launch_bounds__(kSweepThreads) void target_only_kernel(TargetArgs A) {
    __shared__ float s_f[kSweepThreads / SPEC_WAVE];
    __shared__ double s_d[kSweepThreads / SPEC_WAVE];
    const int64_t t = blockIdx.x;
    chunk_item<DT>(A, t, s_f, s_d);
    if constexpr (WALK) {
        const int64_t first_walker = (int64_t)gridDim.x - A.batch;
        if (t >= first_walker) walk_request<DT>(A, (int)(t - first_walker));
    }
}

// Second launch when the walkers cannot all be resident with the chunk work.
template <int DT>
__global__ __launch_bounds__(kSweepThreads) void target_only_walk_kernel(TargetArgs A) {
    walk_request<DT>(A, blockIdx.x);
}

// Workgroups of the fused kernel the device holds at once (0 if unknown).
template <int DT>
int fused_capacity() {
    return spec::resident_capacity(
        reinterpret_cast<const void *>(target_only_kernel<DT, true>), kSweepThreads);
}

template <int DT>
void launch(const TargetArgs &A, int64_t items, hipStream_t st) {
    const bool fused = !spec::stream_capturing(st) && A.batch < fused_capacity<DT>();
    const dim3 grid((unsigned)items);
    if (fused) {
        hipLaunchKernelGGL((target_only_kernel<DT, true>), grid, dim3(kSweepThreads), 0, st, A);
    } else {
        hipLaunchKernelGGL((target_only_kernel<DT, false>), grid, dim3(kSweepThreads), 0, st, A);
        hipLaunchKernelGGL((target_only_walk_kernel<DT>), dim3(A.batch), dim3(kSweepThreads), 0, st, A);
    }
}

}  // namespace

extern "C" size_t spec_accept_target_only_workspace_size(int batch, int n, int64_t vocab) {
    if (batch <= 0 || n <= 0 || vocab <= 0) return 0;
    return spec::align_up((size_t)batch * n * num_chunks(vocab) * 2 * sizeof(uint64_t), 256);
}

extern "C" int spec_accept_target_only(int batch, int n, int s1, int64_t vocab, int dtype,
                                       const void *target_logits, const float *temperature,
                                       float threshold_single, float threshold_acc,
                                       const float *uniforms, const float *final_uniforms,
                                       const int32_t *candidates, const int32_t *retrieve_index,
                                       const int32_t *retrieve_next_token,
                                       const int32_t *retrieve_next_sibling, int32_t *predict,
                                       int32_t *accept_index, int32_t *accept_length,
                                       void *workspace, size_t workspace_bytes,
                                       int32_t *dev_status, spec_stream_t stream) {
    int rc = spec_check_accept_args(batch, n, s1, vocab, dtype);
    if (rc != SPEC_OK) return rc;
    if (!(threshold_acc > 0.f) || !(threshold_single == threshold_single)) return SPEC_ERR_SHAPE;
    if (batch == 0) return SPEC_OK;
    if (!target_logits || !temperature || !uniforms || !final_uniforms || !candidates ||
        !retrieve_index || !retrieve_next_token || !retrieve_next_sibling || !predict ||
        !accept_index || !accept_length)
        return SPEC_ERR_NULL;
    if (!workspace || workspace_bytes < spec_accept_target_only_workspace_size(batch, n, vocab) ||
        reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return SPEC_ERR_WORKSPACE;
    const int nch = num_chunks(vocab);
    const int64_t items = (int64_t)batch * n * nch;
    if (items > INT_MAX || vocab > kMaxVocab) return SPEC_ERR_UNSUPPORTED;
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    TargetArgs A{};
    A.logits = target_logits;
    A.vocab = vocab;
    A.vec_ok = (vocab * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0;
    A.batch = batch;
    A.n = n;
    A.s1 = s1;
    A.nchunks = nch;
    A.temperature = temperature;
    A.uniforms = uniforms;
    A.final_uniforms = final_uniforms;
    A.ts = (double)threshold_single;
    A.ta = (double)threshold_acc;
    A.cand = candidates;
    A.r_index = retrieve_index;
    A.r_next = retrieve_next_token;
    A.r_sib = retrieve_next_sibling;
    A.predict = predict;
    A.accept_index = accept_index;
    A.accept_length = accept_length;
    A.status = dev_status;
    A.slots = static_cast<uint64_t *>(workspace);
    A.poll_limit = spec::poll_limit();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SPEC_BF16) launch<SPEC_BF16>(A, items, st);
    else launch<SPEC_F32>(A, items, st);
    return spec::launch_status();
}
