// Tree-masked verify attention.
//
// "把投机采样讲透:以 SGLang 中的 EAGLE-2 为例" (4.2 query / KV, 4.3 tree mask):
// every flattened tree node is a query; it attends to the request's whole
// cached history and to the tree nodes on its own root path (its mask row),
// whose K/V were written at out_cache_loc ("SGLang 源码完全拆解(十一)",
// 验证前向的组装).  The history is read from HBM once per KV head and reused
// by all n tree queries of the request and all G query heads of the group.
//
// Layout of the work
//   * key space of request b: positions 0 .. L_b-1 are history (paged),
//     L_b .. L_b+n-1 are the tree nodes; the key space is cut into splits
//     of split_len keys, one workgroup per (split, KV head, request);
//   * the workgroup's query rows are rho = node * G + g (n*G of them);
//   * bf16: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16.
//     With keys on the M side each lane owns one query column, so the
//     running max, the rescale of its O^T column and the probabilities stay
//     in the lane (one cross-half exchange for the max).  P^T feeds the PV
//     product straight from the score registers: the 16 keys of one MFMA
//     k-step are taken in the order the score layout already holds them, and
//     V^T is read in that same key order.  K tiles sit row-major in LDS; V
//     tiles are transposed on their way into LDS so the V^T operand is two
//     8-byte reads.  64-key tiles are double-buffered, the next tile's global
//     loads in flight during the current tile's math.
//   * f32: the same splits on the vector ALUs (one wavefront per query row,
//     lanes across head_dim).
//   * splits > 1: each writes (max, sum, unnormalised O) partials in fp32; a
//     merge kernel combines them by log-sum-exp.  One split writes O directly.
#include <math.h>

#include "spec_common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileKeys = 64;

struct AttnParams {
    int batch, n, hq, hkv, group, rows;   // rows = n * group
    int page_size, max_pages, max_seq_len;
    int split_len, nsplit, rowgroups, rows_per_group;
    int word_bytes;
    float scale_log2;                      // sm_scale * log2(e)
    int64_t num_slots;
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *out_cache_loc;
    const uint8_t *mask;
    void *out;
    float *part_o;                         // [b][hkv][nsplit][rows][D]
    float2 *part_ml;                       // [b][hkv][nsplit][rows] (max log2, sum)
    int32_t *status;
};

__device__ __forceinline__ uint64_t load_mask_word(const uint8_t *m, int word_bytes) {
    switch (word_bytes) {
        case 1: return *m;
        case 2: return *reinterpret_cast<const uint16_t *>(m);
        case 4: return *reinterpret_cast<const uint32_t *>(m);
        default: return *reinterpret_cast<const uint64_t *>(m);
    }
}

// Physical slot of key position p of request b, or -1 when out of range.
__device__ __forceinline__ int64_t key_slot(const AttnParams &P, int b, int L, int p, int &err) {
    int64_t slot;
    if (p < L) {
        const int page = P.page_table[(int64_t)b * P.max_pages + p / P.page_size];
        slot = (int64_t)page * P.page_size + p % P.page_size;
        if (page < 0) slot = -1;
    } else {
        slot = P.out_cache_loc[(int64_t)b * P.n + (p - L)];
    }
    if (slot < 0 || slot >= P.num_slots) {
        err |= SPEC_ST_RANGE;
        return -1;
    }
    return slot;
}

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel
// ---------------------------------------------------------------------------

template <int D, int NW, int QT>
__global__ __launch_bounds__(NW * 64) void attn_split_mfma_kernel(AttnParams P) {
    static_assert(D == 64 || D == 128, "head_dim");
    constexpr int KS = D + 8;              // K row stride (bf16), 16-byte pad
    constexpr int VS = kTileKeys + 8;      // V^T row stride (bf16)
    constexpr int NT = NW * 64;
    constexpr int KUNITS = kTileKeys * (D / 8);        // 16-byte K pieces per tile
    constexpr int VUNITS = (kTileKeys / 4) * (D / 8);  // 4 keys x 8 dims per V piece
    constexpr int KPER = (KUNITS + NT - 1) / NT;
    constexpr int VPER = (VUNITS + NT - 1) / NT;
    constexpr int DK = D / 16;             // MFMA k-steps over head_dim
    constexpr int DT = D / 32;             // 32-row d tiles of O^T

    __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kTileKeys * KS];
    __shared__ __attribute__((aligned(16))) __bf16 vt_lds[2][D * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;            // 0 / 1
    const int col = lane & 31;

    const int split = blockIdx.x / P.rowgroups;
    const int rg = blockIdx.x % P.rowgroups;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int L = P.seq_lens[b];
    int err = 0;
    if (L < 0 || L > P.max_seq_len) {
        if (tid == 0 && split == 0 && rg == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        return;
    }
    const int total_keys = L + P.n;
    const int kb = split * P.split_len;
    const int ke = min(total_keys, kb + P.split_len);
    if (kb >= ke) return;

    // ---- query fragments (B operand of S^T = K Q^T) -----------------------
    bf16x8 qf[QT][DK];
    uint64_t mword[QT];
    int qrho[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int rho = rg * P.rows_per_group + (wave * QT + t) * 32 + col;
        qrho[t] = rho;
        if (rho < P.rows) {
            const int node = rho / P.group;
            const int h = kvh * P.group + rho % P.group;
            const __bf16 *qp = static_cast<const __bf16 *>(P.q) +
                               (((int64_t)b * P.n + node) * P.hq + h) * D + 8 * half;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                qf[t][kk] = *reinterpret_cast<const bf16x8 *>(qp + kk * 16);
            mword[t] = load_mask_word(P.mask + ((int64_t)b * P.n + node) * P.word_bytes, P.word_bytes);
        } else {
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) qf[t][kk] = bf16x8{};
            mword[t] = 0;
        }
    }

    floatx16 oacc[QT][DT];
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[t][dt] = floatx16{};
    }

    // ---- global -> register staging of one 64-key tile --------------------
    uint4 kreg[KPER];
    uint4 vreg[VPER][4];
    const __bf16 *kpool = static_cast<const __bf16 *>(P.k_pool);
    const __bf16 *vpool = static_cast<const __bf16 *>(P.v_pool);

    auto fetch = [&](int tile_base) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int u = tid + i * NT;
            kreg[i] = make_uint4(0, 0, 0, 0);
            if (u < KUNITS) {
                const int key = u / (D / 8), d8 = u % (D / 8);
                const int p = tile_base + key;
                if (p < ke) {
                    const int64_t slot = key_slot(P, b, L, p, err);
                    if (slot >= 0)
                        kreg[i] = *reinterpret_cast<const uint4 *>(
                            kpool + (slot * P.hkv + kvh) * D + d8 * 8);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int u = tid + i * NT;
#pragma unroll
            for (int j = 0; j < 4; ++j) vreg[i][j] = make_uint4(0, 0, 0, 0);
            if (u < VUNITS) {
                const int kq = u % (kTileKeys / 4), d8 = u / (kTileKeys / 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int p = tile_base + kq * 4 + j;
                    if (p < ke) {
                        const int64_t slot = key_slot(P, b, L, p, err);
                        if (slot >= 0)
                            vreg[i][j] = *reinterpret_cast<const uint4 *>(
                                vpool + (slot * P.hkv + kvh) * D + d8 * 8);
                    }
                }
            }
        }
    };

    auto stash = [&](int stage) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int u = tid + i * NT;
            if (u < KUNITS) {
                const int key = u / (D / 8), d8 = u % (D / 8);
                *reinterpret_cast<uint4 *>(&k_lds[stage][key * KS + d8 * 8]) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int u = tid + i * NT;
            if (u < VUNITS) {
                const int kq = u % (kTileKeys / 4), d8 = u / (kTileKeys / 4);
                // vreg[i][j] holds dims d8*8 .. d8*8+7 of key kq*4+j; write, for
                // each dim, the 4 keys as one 8-byte run of V^T.
                const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vreg[i][0]);
                const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vreg[i][1]);
                const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&vreg[i][2]);
                const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&vreg[i][3]);
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {       // dim pair (2*pr, 2*pr+1)
                    const uint32_t a = w0[pr], bb = w1[pr], c = w2[pr], d = w3[pr];
                    uint2 lo, hi;
                    lo.x = __builtin_amdgcn_perm(bb, a, 0x05040100u);   // keys 0,1 of dim 2pr
                    lo.y = __builtin_amdgcn_perm(d, c, 0x05040100u);    // keys 2,3
                    hi.x = __builtin_amdgcn_perm(bb, a, 0x07060302u);   // keys 0,1 of dim 2pr+1
                    hi.y = __builtin_amdgcn_perm(d, c, 0x07060302u);
                    const int dim = d8 * 8 + 2 * pr;
                    *reinterpret_cast<uint2 *>(&vt_lds[stage][dim * VS + kq * 4]) = lo;
                    *reinterpret_cast<uint2 *>(&vt_lds[stage][(dim + 1) * VS + kq * 4]) = hi;
                }
            }
        }
    };

    const int ntiles = (ke - kb + kTileKeys - 1) / kTileKeys;
    fetch(kb);
    for (int it = 0; it < ntiles; ++it) {
        const int stage = it & 1;
        const int tile_base = kb + it * kTileKeys;
        stash(stage);
        __syncthreads();
        if (it + 1 < ntiles) fetch(tile_base + kTileKeys);

        const __bf16 *kt = k_lds[stage];
        const __bf16 *vt = vt_lds[stage];
#pragma unroll
        for (int sub = 0; sub < kTileKeys / 32; ++sub) {
            // K operand rows: key sub*32 + col, dims 8*half .. of each k-step
            bf16x8 kf[DK];
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                kf[kk] = *reinterpret_cast<const bf16x8 *>(&kt[(sub * 32 + col) * KS + kk * 16 + 8 * half]);
            // V^T operand: dim dt*32 + col; keys 16s + 4*half + {0..3} and +8
            bf16x8 vf[DT][2];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const __bf16 *vp = &vt[(dt * 32 + col) * VS + sub * 32 + 16 * s + 4 * half];
                    const uint2 x0 = *reinterpret_cast<const uint2 *>(vp);
                    const uint2 x1 = *reinterpret_cast<const uint2 *>(vp + 8);
                    uint4 w = make_uint4(x0.x, x0.y, x1.x, x1.y);
                    vf[dt][s] = *reinterpret_cast<const bf16x8 *>(&w);
                }
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                if (wave * QT * 32 + t * 32 + rg * P.rows_per_group >= P.rows) continue;
                floatx16 sacc = floatx16{};
#pragma unroll
                for (int kk = 0; kk < DK; ++kk)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[t][kk], sacc, 0, 0, 0);
                // scores of keys sub*32 + 8*(i/4) + 4*half + i%4 for query col
                float s[16];
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = tile_base + sub * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    float v = sacc[i] * P.scale_log2;
                    if (p >= ke) v = -INFINITY;
                    else if (p >= L && !((mword[t] >> (p - L)) & 1ull)) v = -INFINITY;
                    s[i] = v;
                    mx = fmaxf(mx, v);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[t], mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = exp2f(m_run[t] - m_use);
                m_run[t] = m_new;
                float lsum = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] = exp2f(s[i] - m_use);
                    lsum += s[i];
                }
                l_run[t] = l_run[t] * alpha + lsum;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[t][dt] *= alpha;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    bf16x8 pf;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(s[8 * st + e]);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        oacc[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][st], pf, oacc[t][dt], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue -----------------------------------------------------------
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int rho = qrho[t];
        const float l_tot = l_run[t] + __shfl_xor(l_run[t], 32, 64);
        if (rho >= P.rows) continue;
        const int node = rho / P.group;
        const int h = kvh * P.group + rho % P.group;
        if (P.nsplit == 1) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            __bf16 *op = static_cast<__bf16 *>(P.out) + (((int64_t)b * P.n + node) * P.hq + h) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int d0 = dt * 32 + 8 * j4 + 4 * half;
                    uint2 w;
                    __bf16 v4[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) v4[j] = static_cast<__bf16>(oacc[t][dt][4 * j4 + j] * inv);
                    w = *reinterpret_cast<uint2 *>(v4);
                    *reinterpret_cast<uint2 *>(op + d0) = w;
                }
        } else {
            const int64_t pidx = (((int64_t)b * P.hkv + kvh) * P.nsplit + split) * P.rows + rho;
            float *po = P.part_o + pidx * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int d0 = dt * 32 + 8 * j4 + 4 * half;
                    *reinterpret_cast<float4 *>(po + d0) =
                        make_float4(oacc[t][dt][4 * j4 + 0], oacc[t][dt][4 * j4 + 1],
                                    oacc[t][dt][4 * j4 + 2], oacc[t][dt][4 * j4 + 3]);
                }
            if (half == 0) P.part_ml[pidx] = make_float2(m_run[t], l_tot);
        }
    }
    // status: one atomic per wave at most
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, 64);
    if (lane == 0) spec::raise_status(P.status, err);
}

// ---------------------------------------------------------------------------
// f32 split kernel (vector ALUs): one wavefront per query row at a time
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void attn_split_f32_kernel(AttnParams P) {
    constexpr int PER = D / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int split = blockIdx.x / P.rowgroups;
    const int rg = blockIdx.x % P.rowgroups;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int L = P.seq_lens[b];
    int err = 0;
    if (L < 0 || L > P.max_seq_len) {
        if (tid == 0 && split == 0 && rg == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        return;
    }
    const int kb = split * P.split_len;
    const int ke = min(L + P.n, kb + P.split_len);
    if (kb >= ke) return;
    const float *kpool = static_cast<const float *>(P.k_pool);
    const float *vpool = static_cast<const float *>(P.v_pool);
    const int r0 = rg * P.rows_per_group;
    const int r1 = min(P.rows, r0 + P.rows_per_group);
    for (int rho = r0 + wave; rho < r1; rho += 4) {
        const int node = rho / P.group;
        const int h = kvh * P.group + rho % P.group;
        const float *qp = static_cast<const float *>(P.q) + (((int64_t)b * P.n + node) * P.hq + h) * D;
        const uint64_t mw = load_mask_word(P.mask + ((int64_t)b * P.n + node) * P.word_bytes, P.word_bytes);
        float qv[PER], o[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) { qv[j] = qp[lane + 64 * j]; o[j] = 0.f; }
        float m = -INFINITY, l = 0.f;
        for (int p = kb; p < ke; ++p) {
            if (p >= L && !((mw >> (p - L)) & 1ull)) continue;
            const int64_t slot = key_slot(P, b, L, p, err);
            float kv[PER], vv[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                kv[j] = slot >= 0 ? kpool[(slot * P.hkv + kvh) * D + lane + 64 * j] : 0.f;
                vv[j] = slot >= 0 ? vpool[(slot * P.hkv + kvh) * D + lane + 64 * j] : 0.f;
            }
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < PER; ++j) dot = fmaf(qv[j], kv[j], dot);
            const float s = spec::wave_sum(dot) * P.scale_log2;
            const float m_new = fmaxf(m, s);
            const float alpha = exp2f(m - m_new);
            const float pw = exp2f(s - m_new);
            l = l * alpha + pw;
#pragma unroll
            for (int j = 0; j < PER; ++j) o[j] = fmaf(pw, vv[j], o[j] * alpha);
            m = m_new;
        }
        if (P.nsplit == 1) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            float *op = static_cast<float *>(P.out) + (((int64_t)b * P.n + node) * P.hq + h) * D;
#pragma unroll
            for (int j = 0; j < PER; ++j) op[lane + 64 * j] = o[j] * inv;
        } else {
            const int64_t pidx = (((int64_t)b * P.hkv + kvh) * P.nsplit + split) * P.rows + rho;
#pragma unroll
            for (int j = 0; j < PER; ++j) P.part_o[pidx * D + lane + 64 * j] = o[j];
            if (lane == 0) P.part_ml[pidx] = make_float2(m, l);
        }
    }
    for (int o2 = 32; o2 > 0; o2 >>= 1) err |= __shfl_xor(err, o2, 64);
    if (lane == 0) spec::raise_status(P.status, err);
}

// ---------------------------------------------------------------------------
// merge of split partials: one wavefront per (row, head) output vector
// ---------------------------------------------------------------------------

template <int D, int DTYPE>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams P) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t vec = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b*n + node)*hq + h
    const int64_t nvec = (int64_t)P.batch * P.n * P.hq;
    if (vec >= nvec) return;
    const int h = vec % P.hq;
    const int64_t row = vec / P.hq;
    const int node = row % P.n;
    const int b = row / P.n;
    const int L = P.seq_lens[b];
    if (L < 0 || L > P.max_seq_len) return;
    const int kvh = h / P.group;
    const int rho = node * P.group + h % P.group;
    const int ns = min(P.nsplit, (L + P.n + P.split_len - 1) / P.split_len);
    const int64_t base = ((int64_t)b * P.hkv + kvh) * P.nsplit;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, P.part_ml[(base + s) * P.rows + rho].x);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float acc[PER] = {};
    float lsum = 0.f;
    for (int s = 0; s < ns; ++s) {
        const int64_t pidx = (base + s) * P.rows + rho;
        const float2 ml = P.part_ml[pidx];
        const float w = exp2f(ml.x - Mu);
        lsum = fmaf(w, ml.y, lsum);
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, P.part_o[pidx * D + lane + 64 * j], acc[j]);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (DTYPE == SPEC_BF16) {
        __bf16 *op = static_cast<__bf16 *>(P.out) + vec * D;
#pragma unroll
        for (int j = 0; j < PER; ++j) op[lane + 64 * j] = static_cast<__bf16>(acc[j] * inv);
    } else {
        float *op = static_cast<float *>(P.out) + vec * D;
#pragma unroll
        for (int j = 0; j < PER; ++j) op[lane + 64 * j] = acc[j] * inv;
    }
}

// ---------------------------------------------------------------------------
// host-side planning
// ---------------------------------------------------------------------------

struct Plan {
    int nw, qt;           // waves per workgroup, 32-query tiles per wave (bf16)
    int rows_per_group, rowgroups;
    int split_len, nsplit;
};

Plan make_plan(int batch, int n, int hq, int hkv, int max_seq_len, int dtype) {
    Plan pl{};
    const int rows = n * (hq / hkv);
    if (dtype == SPEC_BF16) {
        if (rows <= 64) { pl.nw = 2; pl.qt = 1; }
        else if (rows <= 128) { pl.nw = 4; pl.qt = 1; }
        else { pl.nw = 4; pl.qt = 2; }      // 256 rows per workgroup
        pl.rows_per_group = pl.nw * pl.qt * 32;
    } else {
        pl.nw = 4;
        pl.qt = 1;
        pl.rows_per_group = rows;
    }
    pl.rowgroups = (rows + pl.rows_per_group - 1) / pl.rows_per_group;
    const int keys = max_seq_len + n;
    const int tiles = (keys + kTileKeys - 1) / kTileKeys;
    const int base = batch * hkv * pl.rowgroups;
    const int target = 1024;                       // workgroups to aim for
    int ns = (target + base - 1) / base;
    ns = min(ns, max(1, tiles / 2));               // at least two tiles per split
    ns = max(ns, 1);
    const int tiles_per = (tiles + ns - 1) / ns;
    pl.split_len = tiles_per * kTileKeys;
    pl.nsplit = (keys + pl.split_len - 1) / pl.split_len;
    return pl;
}

size_t workspace_bytes_for(const Plan &pl, int batch, int n, int hq, int hkv, int d) {
    if (pl.nsplit <= 1) return 0;
    const size_t rows = (size_t)n * (hq / hkv);
    const size_t parts = (size_t)batch * hkv * pl.nsplit * rows;
    return spec::align_up(parts * d * sizeof(float), 256) + spec::align_up(parts * sizeof(float2), 256);
}

template <int D>
void launch_mfma(const Plan &pl, const AttnParams &P, dim3 grid, hipStream_t st) {
    if (pl.nw == 2)
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 2, 1>), grid, dim3(128), 0, st, P);
    else if (pl.nw == 4 && pl.qt == 1)
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 4, 1>), grid, dim3(256), 0, st, P);
    else
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 4, 2>), grid, dim3(256), 0, st, P);
}

}  // namespace

extern "C" size_t spec_verify_attention_workspace_size(int batch, int n, int hq, int hkv, int d,
                                                       int max_seq_len, int dtype) {
    if (batch <= 0 || n <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_seq_len < 0) return 0;
    const Plan pl = make_plan(batch, n, hq, hkv, max_seq_len, dtype);
    return workspace_bytes_for(pl, batch, n, hq, hkv, d);
}

extern "C" int spec_verify_attention(int batch, int n, int hq, int hkv, int d, int page_size,
                                     int dtype, float sm_scale, const void *q, const void *k_pool,
                                     const void *v_pool, int64_t num_slots,
                                     const int32_t *page_table, int max_pages,
                                     const int32_t *seq_lens, int max_seq_len,
                                     const int32_t *out_cache_loc, const void *tree_mask,
                                     void *out, void *workspace, size_t workspace_bytes,
                                     int32_t *dev_status, spec_stream_t stream) {
    if (batch < 0 || n < 1 || hq < 1 || hkv < 1 || page_size < 1 || max_pages < 0 ||
        max_seq_len < 0 || num_slots < 0)
        return SPEC_ERR_SHAPE;
    if (hq % hkv != 0) return SPEC_ERR_SHAPE;
    if (n > 64 || (d != 64 && d != 128)) return SPEC_ERR_UNSUPPORTED;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if ((int64_t)max_pages * page_size < (int64_t)max_seq_len && max_seq_len > 0) return SPEC_ERR_SHAPE;
    if (batch == 0) return SPEC_OK;
    if (!q || !k_pool || !v_pool || !seq_lens || !out_cache_loc || !tree_mask || !out)
        return SPEC_ERR_NULL;
    if (max_seq_len > 0 && !page_table) return SPEC_ERR_NULL;
    const int wb = spec_mask_word_bytes(n);
    const uintptr_t align_bad = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
                                 reinterpret_cast<uintptr_t>(v_pool) | reinterpret_cast<uintptr_t>(out)) & 15u;
    if (align_bad || reinterpret_cast<uintptr_t>(tree_mask) % wb) return SPEC_ERR_SHAPE;

    const Plan pl = make_plan(batch, n, hq, hkv, max_seq_len, dtype);
    const size_t need = workspace_bytes_for(pl, batch, n, hq, hkv, d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SPEC_ERR_WORKSPACE;

    AttnParams P{};
    P.batch = batch; P.n = n; P.hq = hq; P.hkv = hkv; P.group = hq / hkv; P.rows = n * P.group;
    P.page_size = page_size; P.max_pages = max_pages; P.max_seq_len = max_seq_len;
    P.split_len = pl.split_len; P.nsplit = pl.nsplit; P.rowgroups = pl.rowgroups;
    P.rows_per_group = pl.rows_per_group; P.word_bytes = wb;
    const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)d);
    P.scale_log2 = scale * kLog2e;
    P.num_slots = num_slots;
    P.q = q; P.k_pool = k_pool; P.v_pool = v_pool; P.page_table = page_table;
    P.seq_lens = seq_lens; P.out_cache_loc = out_cache_loc;
    P.mask = static_cast<const uint8_t *>(tree_mask); P.out = out;
    if (need > 0) {
        const size_t rows = (size_t)P.rows;
        const size_t parts = (size_t)batch * hkv * pl.nsplit * rows;
        P.part_o = static_cast<float *>(workspace);
        P.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(workspace) +
                                               spec::align_up(parts * d * sizeof(float), 256));
    }
    P.status = dev_status;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid(pl.nsplit * pl.rowgroups, hkv, batch);
    if (dtype == SPEC_BF16) {
        if (d == 128) launch_mfma<128>(pl, P, grid, st);
        else launch_mfma<64>(pl, P, grid, st);
    } else {
        if (d == 128) hipLaunchKernelGGL(attn_split_f32_kernel<128>, grid, dim3(256), 0, st, P);
        else hipLaunchKernelGGL(attn_split_f32_kernel<64>, grid, dim3(256), 0, st, P);
    }
    if (pl.nsplit > 1) {
        const int64_t nvec = (int64_t)batch * n * hq;
        const dim3 mgrid((unsigned)((nvec + 3) / 4));
        if (dtype == SPEC_BF16) {
            if (d == 128) hipLaunchKernelGGL((attn_merge_kernel<128, SPEC_BF16>), mgrid, dim3(256), 0, st, P);
            else hipLaunchKernelGGL((attn_merge_kernel<64, SPEC_BF16>), mgrid, dim3(256), 0, st, P);
        } else {
            if (d == 128) hipLaunchKernelGGL((attn_merge_kernel<128, SPEC_F32>), mgrid, dim3(256), 0, st, P);
            else hipLaunchKernelGGL((attn_merge_kernel<64, SPEC_F32>), mgrid, dim3(256), 0, st, P);
        }
    }
    return spec::launch_status();
}
