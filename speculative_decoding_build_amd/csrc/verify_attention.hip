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
//     V^T is stored in that same key order.  K tiles sit row-major in LDS; V
//     tiles are transposed on their way into LDS so the V^T operand is one
//     16-byte read.  64-key tiles are double-buffered, the next tile's global
//     loads in flight during the current tile's math.
//   * f32: the same splits on the vector ALUs (one wavefront per query row,
//     lanes across head_dim).
//   * splits > 1: each writes its (max, sum) in fp32 and its O partial (bf16
//     O / sum, or unnormalised f32 O on the f32 path); a merge kernel
//     combines them by log-sum-exp.  One split writes O directly.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "spec_common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileKeys = 64;
constexpr int kTargetGroups = 512;      // workgroups a launch aims for (one co-resident round)
constexpr int kMinTiles = 4;            // 64-key tiles per split at least
constexpr int kChunkTiles = 8;          // tiles per chunk of the slot ring
constexpr int kChunkKeys = kChunkTiles * kTileKeys;
constexpr int kMaxTreeNodes = 64;
constexpr int kSmallGrid = 512;         // fewer 8-wave workgroups than this: use 4-wave ones
constexpr int kOneRound = 256;          // workgroups that fit one per CU
constexpr int kPlanBatch = 1024;        // most requests a length-balanced plan covers
constexpr int kMergeVec = 1;            // output vectors per merge wave (bf16)

struct AttnParams {
    int batch, n, hq, hkv, group, rows;   // rows = n * group
    int page_size, max_pages, max_seq_len;
    int split_len, nsplit, rowgroups, rows_per_group;
    int dyn;                               // 1: splits follow the actual lengths (see plan_split)
    int slots;                             // split slots per (KV head, row group) when dyn
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
    // partials of split slot j: O [j][hkv][rows][D] and (max log2, sum)
    // [j][hkv][rows].  O is bf16 and already divided by the split's sum on
    // the bf16 path, unnormalised f32 on the f32 path.  Static plan: request
    // b's splits are slots b*nsplit + s; length-balanced plan: slots
    // plan[b].x .. plan[b].x + plan[b].y - 1.
    void *part_o;
    float2 *part_ml;
    int2 *plan;                            // [batch] (first slot, splits), dyn only
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

// A split with no keys (past the sequence, or a sequence length out of
// range) still writes (max, sum) = (-inf, 0) for its rows, so the merge can
// take every split's partial without reading the sequence length.
__device__ __forceinline__ void mark_empty_split(const AttnParams &P, int b, int kvh, int split,
                                                 int rg) {
    if (P.nsplit == 1 || P.dyn) return;
    const int r0 = rg * P.rows_per_group;
    const int r1 = min(P.rows, r0 + P.rows_per_group);
    const int64_t base = (((int64_t)b * P.nsplit + split) * P.hkv + kvh) * P.rows;
    for (int rho = r0 + (int)threadIdx.x; rho < r1; rho += blockDim.x)
        P.part_ml[base + rho] = make_float2(-INFINITY, 0.f);
}

// ---------------------------------------------------------------------------
// work decomposition shared by the split kernels
// ---------------------------------------------------------------------------

struct Work {
    int b, kvh, split, rg;
};

// Workgroup w of the 1-D grid -> (request, KV head, split, row group).  The
// row groups of one split read the same K/V, so they are made neighbours in
// the dispatch order of one XCD (workgroups go to the 8 XCDs round-robin by
// id): XCD x takes the contiguous run of work items x*total/8 .. .
__device__ __forceinline__ Work decode_work(const AttnParams &P, int w, bool xcd_remap) {
    const int total = P.nsplit * P.rowgroups * P.hkv * P.batch;
    int j = w;
    if (xcd_remap) j = (w % 8) * (total / 8) + w / 8;
    Work k;
    k.rg = j % P.rowgroups;
    j /= P.rowgroups;
    k.split = j % P.nsplit;
    j /= P.nsplit;
    k.kvh = j % P.hkv;
    k.b = j / P.hkv;
    return k;
}

// Length-balanced plan (batch > 1): request b has t_b = ceil((L_b + n) / 64)
// tiles (L_b read as 0 when out of range) and gets
//     s_b = max(1, min(t_b / kMinTiles, kMaxSplits, 1 + (S - batch) t_b / T))
// of the S split slots, T = sum of t_b, so sum s_b <= S and long requests get
// proportionally more splits; split k covers tiles [k t_b / s_b, (k+1) t_b / s_b).
// Slots are handed out in request order.  Wave 0 of every workgroup
// evaluates it from the sequence lengths (a deterministic computation,
// identical in every workgroup; lane l holds requests l, 64 + l, ...) and
// finds the request and split of its slot j; workgroup 0 also stores
// (first slot, s_b) per request for the merge.  Returns in out[0..3]
// (b, k, s_b, t_b), b = -1 when slot j is unused.
constexpr int kMaxSplits = 64;

__device__ void plan_split(const AttnParams &P, int j, bool store, int *out) {
    constexpr int E = kPlanBatch / 64;
    const int lane = threadIdx.x & 63;
    const int ne = (P.batch + 63) / 64;    // entries in use; request e*64 + lane
    int tb[E];
    long long tsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        tb[e] = 0;
        if (e < ne) {
            const int r = e * 64 + lane;
            if (r < P.batch) {
                int L = P.seq_lens[r];
                if (L < 0 || L > P.max_seq_len) L = 0;
                tb[e] = (L + P.n + kTileKeys - 1) / kTileKeys;
            }
            tsum += tb[e];
        }
    }
    for (int o = 32; o > 0; o >>= 1) tsum += __shfl_xor(tsum, o, 64);
    // exact floor((S - batch) t_b / T): a double estimate (off by at most
    // one) corrected with integer products
    const long long spare = (long long)P.slots - P.batch;
    const double rden = 1.0 / (double)tsum;
    int off = 0;                           // slots of all requests before entry e
    bool found = false;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e >= ne) continue;
        const int r = e * 64 + lane;
        int sb = 0;
        if (tb[e] > 0) {
            const long long num = spare * tb[e];
            long long q = (long long)((double)num * rden);
            if (q * tsum > num) --q;
            if ((q + 1) * tsum <= num) ++q;
            sb = max(1, min(1 + (int)q, min(tb[e] / kMinTiles, kMaxSplits)));
        }
        // slots of the lanes before this one, then of the whole entry
        int incl = sb;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const int first = off + incl - sb;
        if (r < P.batch) {
            if (j >= first && j < first + sb) {
                out[0] = r;
                out[1] = j - first;
                out[2] = sb;
                out[3] = tb[e];
                found = true;
            }
            if (store) P.plan[r] = make_int2(first, sb);
        }
        off += __shfl(incl, 63, 64);
    }
    if (__ballot(found) == 0 && lane == 0) out[0] = -1;
}

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel
// ---------------------------------------------------------------------------
//
// One workgroup: NW waves, each owning 32 query rows (one 32x32 MFMA column
// block).  Per 64-key tile the pipeline is
//     compute tile t (S^T = K Q^T, softmax, O^T += V^T P^T)
//     write tile t+1 (registers -> LDS, V transposed)
//     issue the global loads of tile t+3 (slots read from the LDS slot ring)
//     barrier
// so two tiles of K/V are in flight while one is computed, and the wait for
// tile t+1's loads comes after tile t's math.  A tile wholly inside the
// split loads without per-key conditions.  The slot ring holds two chunks
// of 8 tiles; a chunk's page-table entries are loaded 7 tiles before the
// first load that needs them, so no tile waits on the page table.
//
// Softmax runs in the log2 domain on raw scores: p = exp2(s*C - m) with
// C = scale*log2(e).  A column's running max m is set by its first
// sub-block with a visible key; later sub-blocks take no max: a score far
// above m shows as a probability of 2^64 or more (or an infinite one), and
// only then is m raised to that sub-block's max and O, l rescaled.  The
// softmax is exact at any common offset, so probabilities up to 2^64 are
// kept as they are.

// KH = 2: the waves come in pairs that own the same 32 query rows and take
// the two 32-key halves of every tile; the pair merges its (max, sum, O)
// through LDS at the end.  NW / KH row blocks per workgroup.
template <int D, int NW, int KH>
__global__ __launch_bounds__(NW * 64, 2) void attn_split_mfma_kernel(AttnParams P, int xcd_remap) {
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(KH == 1 || KH == 2, "key halves");
    constexpr int KS = D + 8;              // K row stride (bf16), 16-byte pad
    constexpr int VS = kTileKeys + 8;      // V^T row stride (bf16): 36 dwords, so the
                                           // 16-byte reads of 16 rows hit distinct banks
    constexpr int NT = NW * 64;
    constexpr int KUNITS = kTileKeys * (D / 8);        // 16-byte K pieces per tile
    constexpr int VUNITS = (kTileKeys / 4) * (D / 8);  // 4 keys x 8 dims per V piece
    static_assert(kChunkKeys % NT == 0, "chunk keys per thread");
    // a tile's loads are issued LEAD tiles before it is computed (two
    // register sets in flight)
    constexpr int LEAD = 3;
    constexpr int KPER = (KUNITS + NT - 1) / NT;
    constexpr int VPER = (VUNITS + NT - 1) / NT;
    constexpr int DK = D / 16;             // MFMA k-steps over head_dim
    constexpr int DT = D / 32;             // 32-row d tiles of O^T

    // K and V^T tile stages; after the loop the same bytes hold the key-half
    // partners' (max, sum, O) for the merge
    constexpr int KBYTES = 2 * kTileKeys * KS * 2, VBYTES = 2 * D * VS * 2;
    constexpr int MSTRIDE = DT * 16 + 2;   // floats per lane: O^T, max, sum
    constexpr int MBYTES = KH == 2 ? (NW / 2) * 64 * MSTRIDE * 4 : 0;
    static_assert(MBYTES <= KBYTES + VBYTES, "merge buffer");
    __shared__ __attribute__((aligned(16))) char lds_tiles[KBYTES + VBYTES];
    auto k_lds = reinterpret_cast<__bf16 (*)[kTileKeys * KS]>(lds_tiles);
    auto vt_lds = reinterpret_cast<__bf16 (*)[D * VS]>(lds_tiles + KBYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;

    int b, kvh, split, rg, nsp, kb, span;
    int64_t slot_j;                        // split slot of the partials
    if (P.dyn) {
        // length-balanced plan: this workgroup is split slot j of (KV head,
        // row group); rows groups of one slot are neighbours as below
        const int total = P.slots * P.rowgroups * P.hkv;
        int w = blockIdx.x;
        if (xcd_remap) w = (w % 8) * (total / 8) + w / 8;
        rg = w % P.rowgroups;
        w /= P.rowgroups;
        const int j = w % P.slots;
        kvh = w / P.slots;
        __shared__ int s_plan[4];
        if (wave == 0) plan_split(P, j, blockIdx.x == 0, s_plan);
        __syncthreads();
        b = s_plan[0];
        if (b < 0) return;                 // unused slot: no keys, no partials
        split = s_plan[1];
        nsp = s_plan[2];
        const int t = s_plan[3];
        const int tlo = (int)((int64_t)split * t / nsp), thi = (int)((int64_t)(split + 1) * t / nsp);
        kb = tlo * kTileKeys;
        span = (thi - tlo) * kTileKeys;
        slot_j = j;
    } else {
        const Work wk = decode_work(P, blockIdx.x, xcd_remap != 0);
        b = wk.b; kvh = wk.kvh; split = wk.split; rg = wk.rg;
        nsp = P.nsplit;
        kb = split * P.split_len;
        span = P.split_len;
        slot_j = (int64_t)b * P.nsplit + split;
    }
    // Loads that do not depend on the sequence length go out with it: the
    // page-table entries of the split's first two slot chunks and the
    // request's tree slots.
    constexpr int KPT = kChunkKeys / NT;   // chunk keys per thread
    int pg[2 * KPT];
#pragma unroll
    for (int j = 0; j < 2 * KPT; ++j) {
        const int p = kb + tid + j * NT;
        pg[j] = -1;
        if (P.page_table != nullptr && p < P.max_pages * P.page_size)
            pg[j] = P.page_table[(int64_t)b * P.max_pages + p / P.page_size];
    }
    int pre_tree = -1;
    if (tid < P.n) pre_tree = P.out_cache_loc[(int64_t)b * P.n + tid];
    const int L = P.seq_lens[b];
    int err = 0;
    if (L < 0 || L > P.max_seq_len) {
        if (tid == 0 && split == 0 && rg == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    const int ke = min(L + P.n, kb + span);
    if (kb >= ke) {
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    const int ntiles = (ke - kb + kTileKeys - 1) / kTileKeys;
    // Slot ring: the physical slots of two chunks of kChunkKeys keys (-1 past
    // the split or invalid).  Chunk c lives in half c & 1; its page entries
    // are loaded seven tiles before its first tile's K/V loads need them.
    __shared__ int32_t s_ring[2][kChunkKeys];
    __shared__ int32_t s_tree[kMaxTreeNodes];
    if (tid < P.n) s_tree[tid] = pre_tree;

    // ---- query fragments (B operand of S^T = K Q^T) -----------------------
    const int rblk = wave % (NW / KH);     // row block of this wave
    const int khalf = wave / (NW / KH);    // key half of this wave (KH = 2)
    const int rho = rg * P.rows_per_group + rblk * 32 + col;
    const bool wave_active = rg * P.rows_per_group + rblk * 32 < P.rows;
    bf16x8 qf[DK];
    uint64_t mword = 0;
    if (rho < P.rows) {
        const int node = rho / P.group;
        const int h = kvh * P.group + rho % P.group;
        const __bf16 *qp = static_cast<const __bf16 *>(P.q) +
                           (((int64_t)b * P.n + node) * P.hq + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8 *>(qp + kk * 16);
        mword = load_mask_word(P.mask + ((int64_t)b * P.n + node) * P.word_bytes, P.word_bytes);
    } else {
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qf[kk] = bf16x8{};
    }

    floatx16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx16{};
    float m_run = -INFINITY;   // running max, log2 domain (already times C)
    float l_run = 0.f;         // this lane-half's share of the softmax sum
    const float C = P.scale_log2;

    const __bf16 *kpool = static_cast<const __bf16 *>(P.k_pool);
    const __bf16 *vpool = static_cast<const __bf16 *>(P.v_pool);

    // slot of key position p of this request from its page entry (history)
    // or the tree slots; -1 past the split or when out of range
    auto slot_of = [&](int p, int page) -> int32_t {
        if (p >= ke) return -1;
        int64_t slot;
        if (p < L)
            slot = page < 0 ? -1 : (int64_t)page * P.page_size + p % P.page_size;
        else
            slot = s_tree[p - L];
        if (slot < 0 || slot >= P.num_slots) {
            err |= SPEC_ST_RANGE;
            return -1;
        }
        return (int32_t)slot;
    };

    // ---- register staging: two tiles in flight, in two statically named sets
    uint4 kreg0[KPER], kreg1[KPER];
    uint4 vreg0[VPER][4], vreg1[VPER][4];
    auto issue = [&](uint4 (&kr)[KPER], uint4 (&vr)[VPER][4], int t) {
        const int32_t *sl = &s_ring[(t / kChunkTiles) & 1][(t % kChunkTiles) * kTileKeys];
        if (kb + (t + 1) * kTileKeys <= ke) {
            // every key of the tile is in the split: unconditional loads (a
            // slot the ring marks invalid, -1 after a range error, reads slot
            // 0, which exists: the host refuses an empty pool; the call has
            // then raised SPEC_ST_RANGE and its output is unspecified)
#pragma unroll
            for (int i = 0; i < KPER; ++i) {
                const int u = tid + i * NT;
                if (KUNITS % NT == 0 || u < KUNITS) {
                    const int32_t slot = max(sl[u / (D / 8)], 0);
                    kr[i] = *reinterpret_cast<const uint4 *>(
                        kpool + ((int64_t)slot * P.hkv + kvh) * D + (u % (D / 8)) * 8);
                }
            }
#pragma unroll
            for (int i = 0; i < VPER; ++i) {
                const int u = tid + i * NT;
                if (VUNITS % NT == 0 || u < VUNITS) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int32_t slot = max(sl[(u % (kTileKeys / 4)) * 4 + j], 0);
                        vr[i][j] = *reinterpret_cast<const uint4 *>(
                            vpool + ((int64_t)slot * P.hkv + kvh) * D + (u / (kTileKeys / 4)) * 8);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int u = tid + i * NT;
            kr[i] = make_uint4(0, 0, 0, 0);
            if (u < KUNITS) {
                const int32_t slot = sl[u / (D / 8)];
                if (slot >= 0)
                    kr[i] = *reinterpret_cast<const uint4 *>(
                        kpool + ((int64_t)slot * P.hkv + kvh) * D + (u % (D / 8)) * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int u = tid + i * NT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vr[i][j] = make_uint4(0, 0, 0, 0);
                if (u < VUNITS) {
                    const int32_t slot = sl[(u % (kTileKeys / 4)) * 4 + j];
                    if (slot >= 0)
                        vr[i][j] = *reinterpret_cast<const uint4 *>(
                            vpool + ((int64_t)slot * P.hkv + kvh) * D + (u / (kTileKeys / 4)) * 8);
                }
            }
        }
    };
    auto word = [](const uint4 &v, int k) -> uint32_t {
        return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
    };
    auto stash = [&](const uint4 (&kr)[KPER], const uint4 (&vr)[VPER][4], int stage) {
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int u = tid + i * NT;
            if (u < KUNITS)
                *reinterpret_cast<uint4 *>(&k_lds[stage][(u / (D / 8)) * KS + (u % (D / 8)) * 8]) =
                    kr[i];
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int u = tid + i * NT;
            if (u < VUNITS) {
                const int kq = u % (kTileKeys / 4), d8 = u / (kTileKeys / 4);
                // vr[i][j] holds dims d8*8 .. +7 of key kq*4+j; write, per dim,
                // its 4 keys as one 8-byte run of V^T.  Within each run of 4
                // groups of 4 keys the middle two swap places, so the 8 keys
                // one lane feeds an MFMA k-step (groups g and g+2) sit together.
                const int kp = (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t a = word(vr[i][0], pr), bb = word(vr[i][1], pr);
                    const uint32_t c = word(vr[i][2], pr), d = word(vr[i][3], pr);
                    uint2 lo, hi;
                    lo.x = __builtin_amdgcn_perm(bb, a, 0x05040100u);
                    lo.y = __builtin_amdgcn_perm(d, c, 0x05040100u);
                    hi.x = __builtin_amdgcn_perm(bb, a, 0x07060302u);
                    hi.y = __builtin_amdgcn_perm(d, c, 0x07060302u);
                    const int dim = d8 * 8 + 2 * pr;
                    *reinterpret_cast<uint2 *>(&vt_lds[stage][dim * VS + kp * 4]) = lo;
                    *reinterpret_cast<uint2 *>(&vt_lds[stage][(dim + 1) * VS + kp * 4]) = hi;
                }
            }
        }
    };

    // ---- prologue: slots of chunks 0 and 1 into the ring, tile 0 in LDS,
    // tiles 1 and 2 loading ---------------------------------------------------
    __syncthreads();                       // s_tree
#pragma unroll
    for (int j = 0; j < 2 * KPT; ++j) {
        const int e = tid + j * NT;
        s_ring[e / kChunkKeys][e % kChunkKeys] = slot_of(kb + e, pg[j]);
    }
    __syncthreads();
    issue(kreg0, vreg0, 0);
    if (ntiles > 1) issue(kreg1, vreg1, 1);
    stash(kreg0, vreg0, 0);
    __syncthreads();
    if (ntiles > 2) issue(kreg0, vreg0, 2);

    // one pipeline step; tile it+1 and then tile it+LEAD live in the register
    // set (kr, vr).  Chunk c's ring half is last read when tile 8c+7 is issued
    // (step 8c+7-LEAD); chunk c+2's page entries are loaded in the next step
    // and turned into slots at the end of step 8c+15-LEAD, one step before
    // tile 8c+16 is issued.
    int cpg[KPT];
    auto step = [&](int it, uint4 (&kr)[KPER], uint4 (&vr)[VPER][4]) {
        const int tile_base = kb + it * kTileKeys;
        // write tile it+1 (registers -> LDS stage (it+1)&1), then reuse its
        // registers for tile it+LEAD
        if (it % kChunkTiles == kChunkTiles - LEAD) {
            const int cbase = kb + ((it + kChunkTiles + LEAD) / kChunkTiles) * kChunkKeys;
            if (cbase < ke) {
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    const int p = cbase + tid + j * NT;
                    cpg[j] = p < L ? P.page_table[(int64_t)b * P.max_pages + p / P.page_size] : -1;
                }
            }
        }

        if (wave_active) {
            const __bf16 *kt = k_lds[it & 1];
            const __bf16 *vt = vt_lds[it & 1];
            const bool edge = (tile_base + kTileKeys > ke) || (tile_base + kTileKeys > L);
#pragma unroll
            for (int si = 0; si < kTileKeys / 32 / KH; ++si) {
                const int sub = KH == 2 ? khalf : si;
                floatx16 sacc = floatx16{};
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                        &kt[(sub * 32 + col) * KS + kk * 16 + 8 * half]);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc, 0, 0, 0);
                }
                // lane holds keys sub*32 + 8*(i/4) + 4*half + i%4 of query col;
                // masking is a branch-free select on a plain float copy
                float sv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
                if (edge) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int p = tile_base + sub * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        const int rel = p - L;
                        const uint32_t sh = (uint32_t)max(rel, 0) & 63u;
                        const bool bit = ((mword >> sh) & 1ull) != 0;
                        const bool vis = (p < ke) & ((rel < 0) | bit);
                        sv[i] = vis ? sv[i] : -INFINITY;
                    }
                }
                // probabilities at the running max (set here by a column's
                // first sub-block with a visible key; raised only when some
                // probability reaches 2^64)
                auto colmax = [&]() {
                    float mx = sv[0];
#pragma unroll
                    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
                    return fmaxf(mx, __shfl_xor(mx, 32, 64)) * C;
                };
                if (__ballot(m_run == -INFINITY)) {
                    const float mx = colmax();
                    if (m_run == -INFINITY) m_run = mx;
                }
                bf16x8 pf[2];
                auto probs = [&](float mneg) {
                    float s = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[i], C, mneg));
                        const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[8 + i], C, mneg));
                        s += e0 + e1;
                        pf[0][i] = static_cast<__bf16>(e0);
                        pf[1][i] = static_cast<__bf16>(e1);
                    }
                    return s;
                };
                float lsum = probs(m_run == -INFINITY ? 0.f : -m_run);
                if (__ballot(!(lsum < 0x1p64f))) {
                    const float mx = colmax();
                    const float m_new = fmaxf(m_run, mx);
                    const float alpha = (m_new == m_run || m_run == -INFINITY)
                                            ? 1.f : exp2f(m_run - m_new);
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
                    m_run = m_new;
                    lsum = probs(m_run == -INFINITY ? 0.f : -m_run);
                }
                l_run += lsum;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        // keys sub*32 + 16*st + 4*half + {0..3, 8..11}: groups
                        // g and g+2, stored side by side
                        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(
                            &vt[(dt * 32 + col) * VS + sub * 32 + 16 * st + 8 * half]);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], oacc[dt],
                                                                           0, 0, 0);
                    }
                }
            }
        }
        // after the tile's math: the next tile into LDS (its loads have had
        // two steps), then this register set's next loads
        if (it + 1 < ntiles) stash(kr, vr, (it + 1) & 1);
        if (it + LEAD < ntiles) issue(kr, vr, it + LEAD);
        if (it % kChunkTiles == kChunkTiles - 1 - LEAD && it >= 2 * kChunkTiles - 1 - LEAD) {
            const int c = (it + LEAD + 1) / kChunkTiles;
            const int cbase = kb + c * kChunkKeys;
            if (cbase < ke) {
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    const int e = tid + j * NT;
                    s_ring[c & 1][e] = slot_of(cbase + e, cpg[j]);
                }
            }
        }
        __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
        step(it, kreg1, vreg1);                  // even step: tiles it+1, it+3 use set 1
        if (it + 1 < ntiles) step(it + 1, kreg0, vreg0);
    }

    // ---- key-half merge: the second wave of a pair hands over its state ----
    if constexpr (KH == 2) {
        float *mb = reinterpret_cast<float *>(lds_tiles) + (rblk * 64 + lane) * MSTRIDE;
        __syncthreads();                   // every wave is done with the tiles
        if (khalf == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mb[dt * 16 + i] = oacc[dt][i];
            mb[DT * 16] = m_run;
            mb[DT * 16 + 1] = l_run;
        }
        __syncthreads();
        if (khalf == 1) {
            for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, 64);
            if (lane == 0) spec::raise_status(P.status, err);
            return;
        }
        const float m2 = mb[DT * 16], l2 = mb[DT * 16 + 1];
        const float mm = fmaxf(m_run, m2);
        const float a1 = m_run == -INFINITY ? 0.f : exp2f(m_run - mm);
        const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mm);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] = oacc[dt][i] * a1 + mb[dt * 16 + i] * a2;
        l_run = l_run * a1 + l2 * a2;
        m_run = mm;
    }

    // ---- epilogue -------------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (rho < P.rows) {
        const int node = rho / P.group;
        const int h = kvh * P.group + rho % P.group;
        // O / sum in bf16: the output itself for a request with one split,
        // else this split's partial (the merge weights it by its sum)
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        __bf16 *op;
        if (nsp == 1) {
            op = static_cast<__bf16 *>(P.out) + (((int64_t)b * P.n + node) * P.hq + h) * D;
        } else {
            const int64_t pidx = (slot_j * P.hkv + kvh) * P.rows + rho;
            op = static_cast<__bf16 *>(P.part_o) + pidx * D;
            if (half == 0) P.part_ml[pidx] = make_float2(m_run, l_tot);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                uint32_t hv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hv[j] = __builtin_bit_cast(uint16_t,
                                               static_cast<__bf16>(oacc[dt][4 * j4 + j] * inv));
                *reinterpret_cast<uint2 *>(op + dt * 32 + 8 * j4 + 4 * half) =
                    make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
            }
    }
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, 64);
    if (lane == 0) spec::raise_status(P.status, err);
}

// ---------------------------------------------------------------------------
// bf16 MFMA split kernel with K/V loaded straight into LDS (head dim 128,
// 8 waves, power-of-two page sizes up to 64)
// ---------------------------------------------------------------------------
//
// The 8-wave form above without its register staging: each 64-key tile
// travels from HBM into LDS by buffer loads whose destination is the LDS
// (no registers, no ALU work, no LDS writes of the workgroup's own), with
// four tiles in flight.  A tile buffer holds 64 rows of 256 bytes (K, and V
// as it is stored); the 16-byte piece c of key k sits at piece c ^ swz(k),
// so the 32 keys one K fragment read touches and the 4 keys x 32 bytes one
// transposing V read touches fall on distinct banks.  V^T fragments come
// from ds_read_b64_tr_b16, four keys of one dimension per lane and read.
// Each wave loads 8 keys of a tile (two 1 KB runs of K, two of V) with
// indexed loads (record = one slot's row of all KV heads, so no 64-bit
// address per lane; a bad slot is an index past the records, which reads
// zeros).  The split's page ids are copied into LDS before the loop, which
// then loads nothing but tiles; with pages of 8 slots or more a wave's 8 keys
// lie in one page (one id per wave), with smaller pages every lane looks its
// key's page up.  Tile t sits in buffer t % 4, a static buffer per unrolled
// step, so the compiler can tell one buffer's loads from another's reads;
// the wait for tile t is explicit (this wave's vector-memory count, then a
// barrier).  Scores, softmax and the PV product are the 8-wave form's; with
// KH = 2 the waves pair up as in that form (each pair owns 32 rows, its two
// waves take the two 32-key halves of every tile) and merge through LDS.

constexpr int kDmaTile = kTileKeys * 128 * 2;          // 16 KB: K (or V) of one tile
constexpr int kDmaMaxPages = 2048;                     // page ids of a split held in LDS
constexpr uint32_t kRsrcWord3 = 0x00020000u;           // raw buffer access, gfx9 format

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// four tile buffers, each a K tile and a V tile (distinct arrays)
__shared__ __attribute__((aligned(1024))) char dma_k0[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_k1[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_k2[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_k3[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_v0[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_v1[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_v2[kDmaTile];
__shared__ __attribute__((aligned(1024))) char dma_v3[kDmaTile];

template <int S>
__device__ __forceinline__ char *dma_kbuf() {
    if constexpr (S == 0) return dma_k0;
    else if constexpr (S == 1) return dma_k1;
    else if constexpr (S == 2) return dma_k2;
    else return dma_k3;
}

template <int S>
__device__ __forceinline__ char *dma_vbuf() {
    if constexpr (S == 0) return dma_v0;
    else if constexpr (S == 1) return dma_v1;
    else if constexpr (S == 2) return dma_v2;
    else return dma_v3;
}

// tile buffer i of the eight (K buffers 0..3, then V buffers 0..3)
__device__ __forceinline__ char *dma_wave_buf(int i) {
    switch (i) {
        case 0: return dma_k0;
        case 1: return dma_k1;
        case 2: return dma_k2;
        case 3: return dma_k3;
        case 4: return dma_v0;
        case 5: return dma_v1;
        case 6: return dma_v2;
        default: return dma_v3;
    }
}

// position of 16-byte piece c of key k in its row is c ^ piece_swz(k)
__device__ __forceinline__ int piece_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }

// wait until at most n (8, 4 or 0) vector-memory operations of this wave are
// in flight, then a workgroup barrier; memory accesses are not moved across
// either
__device__ __forceinline__ void wait_tiles_barrier(int n) {
    if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
}

template <int V> using ic = std::integral_constant<int, V>;

template <int KH>
__global__ __launch_bounds__(512, 1) void attn_dma_kernel(AttnParams P, int xcd_remap) {
    static_assert(KH == 1 || KH == 2, "key halves");
    constexpr int D = 128, NT = 512, DK = D / 16, DT = D / 32;
    constexpr int kOpsPerTile = 4;        // loads per wave and tile: two K runs, two V runs
    constexpr int NRB = 8 / KH;           // row blocks per workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int rblk = wave_u % NRB;        // row block of this wave
    const int khalf = wave_u / NRB;       // key half of this wave (KH = 2)
    const int ps = P.page_size;           // a power of two, at most 64
    const int psh = __builtin_ctz((unsigned)ps);

    int b, kvh, split, rg, nsp, kb, span;
    int64_t slot_j;                        // split slot of the partials
    if (P.dyn) {
        const int total = P.slots * P.rowgroups * P.hkv;
        int w = blockIdx.x;
        if (xcd_remap) w = (w % 8) * (total / 8) + w / 8;
        rg = w % P.rowgroups;
        w /= P.rowgroups;
        const int j = w % P.slots;
        kvh = w / P.slots;
        __shared__ int s_plan[4];
        if (wave == 0) plan_split(P, j, blockIdx.x == 0, s_plan);
        __syncthreads();
        b = s_plan[0];
        if (b < 0) return;                 // unused slot: no keys, no partials
        split = s_plan[1];
        nsp = s_plan[2];
        const int t = s_plan[3];
        const int tlo = (int)((int64_t)split * t / nsp), thi = (int)((int64_t)(split + 1) * t / nsp);
        kb = tlo * kTileKeys;
        span = (thi - tlo) * kTileKeys;
        slot_j = j;
    } else {
        const Work wk = decode_work(P, blockIdx.x, xcd_remap != 0);
        b = wk.b; kvh = wk.kvh; split = wk.split; rg = wk.rg;
        nsp = P.nsplit;
        kb = split * P.split_len;
        span = P.split_len;
        slot_j = (int64_t)b * P.nsplit + split;
    }
    // all of these are the workgroup's: kept in scalar registers, so the
    // page-id loads below are scalar loads
    b = __builtin_amdgcn_readfirstlane(b);
    kvh = __builtin_amdgcn_readfirstlane(kvh);
    split = __builtin_amdgcn_readfirstlane(split);
    rg = __builtin_amdgcn_readfirstlane(rg);
    nsp = __builtin_amdgcn_readfirstlane(nsp);
    kb = __builtin_amdgcn_readfirstlane(kb);
    span = __builtin_amdgcn_readfirstlane(span);
    __shared__ int32_t s_tree[kMaxTreeNodes];
    __shared__ int32_t s_pages[kDmaMaxPages];
    // Loads that do not depend on the sequence length go out with it: the
    // request's tree slots, the page-table entries of the whole split (kb is
    // a multiple of 64, so of the page size; entries past the request's
    // pages are loaded but never used), the query fragments and mask word.
    constexpr int kPagesPerThread = kDmaMaxPages / NT;
    int pre_tree = -1;
    if (tid < P.n) pre_tree = P.out_cache_loc[(int64_t)b * P.n + tid];
    const int span_pages = (span + ps - 1) >> psh;
    const int page0 = kb >> psh;
    int pgv[kPagesPerThread];
#pragma unroll
    for (int j = 0; j < kPagesPerThread; ++j) {
        const int i = tid + j * NT;
        pgv[j] = (i < span_pages && page0 + i < P.max_pages)
                     ? P.page_table[(int64_t)b * P.max_pages + page0 + i] : -1;
    }
    const int rho = rg * P.rows_per_group + rblk * 32 + col;
    const bool wave_active = rg * P.rows_per_group + rblk * 32 < P.rows;
    bf16x8 qf[DK];
    uint64_t mword = 0;
    if (rho < P.rows) {
        const int node = rho / P.group;
        const int h = kvh * P.group + rho % P.group;
        const __bf16 *qp = static_cast<const __bf16 *>(P.q) +
                           (((int64_t)b * P.n + node) * P.hq + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8 *>(qp + kk * 16);
        mword = load_mask_word(P.mask + ((int64_t)b * P.n + node) * P.word_bytes, P.word_bytes);
    } else {
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qf[kk] = bf16x8{};
    }
    const int L = P.seq_lens[b];
    int err = 0;
    if (span_pages > kDmaMaxPages) {       // the host plans splits of at most kDmaMaxPages pages
        if (tid == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    if (L < 0 || L > P.max_seq_len) {
        if (tid == 0 && split == 0 && rg == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    const int ke = min(L + P.n, kb + span);
    if (kb >= ke) {
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    const int ntiles = (ke - kb + kTileKeys - 1) / kTileKeys;
    if (tid < P.n) s_tree[tid] = pre_tree;
    // the split's page-table entries into LDS, so the loop makes no other
    // memory loads than the tiles'
#pragma unroll
    for (int j = 0; j < kPagesPerThread; ++j)
        if (tid + j * NT < span_pages) s_pages[tid + j * NT] = pgv[j];

    // ---- loads: this lane's two keys of a tile are kl0 and kl0 + 4 ----------
    const int kl0 = 8 * wave + (lane >> 4);
    uint32_t voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int piece = (lane & 15) ^ piece_swz(kl0 + 4 * j);
        voff[j] = (uint32_t)((kvh * D + piece * 8) * 2);
    }
    const int stride = P.hkv * D * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(P.k_pool), (short)stride, (int)P.num_slots, (int)kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(P.v_pool), (short)stride, (int)P.num_slots, (int)kRsrcWord3);
    // page id of this wave's 8 keys of tile t (-1 when its first key is not
    // a history key, or pages are smaller than 8 slots), from the LDS copy of
    // the split's page-table entries
    auto wave_page = [&](int t) -> int {
        const int p = kb + t * kTileKeys + 8 * wave_u;
        if (t >= ntiles || p >= L || ps < 8) return -1;
        return s_pages[(p - kb) >> psh];
    };
    // slot of history key p of the split (-1 for a negative page id)
    auto hist_slot = [&](int p) -> int64_t {
        const int page = s_pages[(p - kb) >> psh];
        return page < 0 ? -1 : ((int64_t)page << psh) + (p & (ps - 1));
    };
    auto dma_tile = [&](char *kdst, char *vdst, int t, int page) {
        uint32_t idx[2];
        const int tb = kb + t * kTileKeys;
        if (tb + kTileKeys <= min(L, ke) && ps >= 8) {
            // a tile of history keys only, the wave's 8 keys in one page:
            // the wave's page (uniform), then the lane's slot within it
            page = __builtin_amdgcn_readfirstlane(page);
            const bool ok = page >= 0 && ((int64_t)page << psh) + ps <= P.num_slots;
            if (!ok) err |= SPEC_ST_RANGE;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                idx[j] = ok ? ((uint32_t)page << psh) + (uint32_t)((kl0 + 4 * j) & (ps - 1))
                            : 0xFFFFFFFFu;
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int p = tb + kl0 + 4 * j;
                int64_t slot = -1;
                if (p < L) slot = hist_slot(p);
                else if (p < ke) slot = s_tree[p - L];
                const bool ok = slot >= 0 && slot < P.num_slots;
                if (!ok && p < ke) err |= SPEC_ST_RANGE;
                idx[j] = ok ? (uint32_t)slot : 0xFFFFFFFFu;
            }
        }
        char *kd = kdst + wave * 2048;
        char *vd = vdst + wave * 2048;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void_t *)(kd + j * 1024), 16,
                                                        idx[j], voff[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_struct_ptr_buffer_load_lds(rv, (lds_void_t *)(vd + j * 1024), 16,
                                                        idx[j], voff[j], 0, 0, 0);
    };

    // ---- LDS read addresses (bytes from a tile buffer) ---------------------
    uint32_t kaddr[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        kaddr[kk] = (uint32_t)(col * 256 + (((2 * kk + half) ^ piece_swz(col)) * 16));
    uint32_t vaddr[DT][2];
    {
        const int g = lane >> 4, r = lane & 15, m = r >> 2, i = r & 3;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = 4 * (g >> 1) + 8 * e + m;
                const int pc = (4 * dt + 2 * (g & 1) + (i >> 1)) ^ piece_swz(key);
                vaddr[dt][e] = (uint32_t)(key * 256 + pc * 16 + (i & 1) * 8);
            }
    }

    floatx16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx16{};
    float m_run = -INFINITY;   // running max, log2 domain (already times C)
    float l_run = 0.f;         // this lane-half's share of the softmax sum
    const float C = P.scale_log2;

    // ---- prologue: tiles 0..2 loading ---------------------------------------
    __syncthreads();                       // s_tree
    if (0 < ntiles) dma_tile(dma_k0, dma_v0, 0, wave_page(0));
    if (1 < ntiles) dma_tile(dma_k1, dma_v1, 1, wave_page(1));
    if (2 < ntiles) dma_tile(dma_k2, dma_v2, 2, wave_page(2));

    auto step = [&](auto stage, int it) {
        constexpr int S = decltype(stage)::value;
        constexpr int SN = (S + 3) & 3;    // buffer of tile it + 3 (tile it - 1's)
        // tile it has landed once at most the loads of tiles it+1, it+2 are
        // in flight; the barrier also ends every wave's use of tile it-1
        wait_tiles_barrier(kOpsPerTile * min(2, ntiles - 1 - it));
        if (it + 3 < ntiles) dma_tile(dma_kbuf<SN>(), dma_vbuf<SN>(), it + 3, wave_page(it + 3));
        if (!wave_active) return;
        const char *kt = dma_kbuf<S>();
        const char *vt = dma_vbuf<S>();
        const int tile_base = kb + it * kTileKeys;
        const bool edge = (tile_base + kTileKeys > ke) || (tile_base + kTileKeys > L);
#pragma unroll
        for (int si = 0; si < 2 / KH; ++si) {
            const int sub = KH == 2 ? khalf : si;
            // the sub-block's K fragments, then its score products; its V^T
            // fragments (which do not depend on the scores) go out before
            // the softmax, so their LDS latency passes under it
            floatx16 sacc = floatx16{};
            bf16x8 kfa[DK];
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                kfa[kk] = *reinterpret_cast<const bf16x8 *>(kt + sub * 8192 + kaddr[kk]);
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfa[kk], qf[kk], sacc, 0, 0, 0);
            bf16x8 vfa[2][DT];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    // V^T rows dt*32 .. +31, keys sub*32 + 16*st + 4*half +
                    // {0..3, 8..11}: two transposing reads
                    const char *vb = vt + sub * 8192 + st * 4096;
                    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_short4v *)(vb + vaddr[dt][0]));
                    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_short4v *)(vb + vaddr[dt][1]));
                    const short4v v8[2] = {lo, hi};
                    vfa[st][dt] = __builtin_bit_cast(bf16x8, v8);
                }
            __builtin_amdgcn_sched_barrier(0);
            // lane holds keys sub*32 + 8*(i/4) + 4*half + i%4 of query col
            float sv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
            if (edge) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = tile_base + sub * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    const int rel = p - L;
                    const uint32_t sh = (uint32_t)max(rel, 0) & 63u;
                    const bool bit = ((mword >> sh) & 1ull) != 0;
                    const bool vis = (p < ke) & ((rel < 0) | bit);
                    sv[i] = vis ? sv[i] : -INFINITY;
                }
            }
            // probabilities at the running max (set here by a column's
            // first sub-block with a visible key; raised only when some
            // probability reaches 2^64)
            auto colmax = [&]() {
                float mx = sv[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
                return fmaxf(mx, __shfl_xor(mx, 32, 64)) * C;
            };
            if (__ballot(m_run == -INFINITY)) {
                const float mx = colmax();
                if (m_run == -INFINITY) m_run = mx;
            }
            bf16x8 pf[2];
            auto probs = [&](float mneg) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[i], C, mneg));
                    const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[8 + i], C, mneg));
                    s += e0 + e1;
                    pf[0][i] = static_cast<__bf16>(e0);
                    pf[1][i] = static_cast<__bf16>(e1);
                }
                return s;
            };
            float lsum = probs(m_run == -INFINITY ? 0.f : -m_run);
            if (__ballot(!(lsum < 0x1p64f))) {
                const float mx = colmax();
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_new == m_run || m_run == -INFINITY)
                                        ? 1.f : exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
                m_run = m_new;
                lsum = probs(m_run == -INFINITY ? 0.f : -m_run);
            }
            l_run += lsum;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfa[st][dt], pf[st],
                                                                       oacc[dt], 0, 0, 0);
        }
    };
    for (int it = 0; it < ntiles; it += 4) {
        step(ic<0>{}, it);
        if (it + 1 < ntiles) step(ic<1>{}, it + 1);
        if (it + 2 < ntiles) step(ic<2>{}, it + 2);
        if (it + 3 < ntiles) step(ic<3>{}, it + 3);
    }

    // ---- key-half merge: the second wave of a pair hands over its state ----
    // (the last step waited for every tile load, and the barrier below ends
    // every wave's reads: K buffer rblk takes the pair's O^T, lane-minor, V
    // buffer 0 the (max, sum) of every pair)
    if constexpr (KH == 2) {
        float *mo = reinterpret_cast<float *>(dma_wave_buf(rblk));
        float *mml = reinterpret_cast<float *>(dma_v0) + rblk * 128;
        __syncthreads();
        if (khalf == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mo[(dt * 16 + i) * 64 + lane] = oacc[dt][i];
            mml[lane] = m_run;
            mml[64 + lane] = l_run;
        }
        __syncthreads();
        if (khalf == 1) {
            for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, 64);
            if (lane == 0) spec::raise_status(P.status, err);
            return;
        }
        const float m2 = mml[lane], l2 = mml[64 + lane];
        const float mm = fmaxf(m_run, m2);
        const float a1 = m_run == -INFINITY ? 0.f : exp2f(m_run - mm);
        const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mm);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                oacc[dt][i] = oacc[dt][i] * a1 + mo[(dt * 16 + i) * 64 + lane] * a2;
        l_run = l_run * a1 + l2 * a2;
        m_run = mm;
    }

    // ---- epilogue: O / sum in bf16 (the output itself for a request with
    // one split, else this split's partial, which the merge weights by its
    // sum).  A lane's O^T fragment holds 4-dim runs of its row, so the
    // wave's 32 x 128 block goes through LDS (rows 272 bytes apart) and
    // leaves as whole 16-byte pieces of each row.
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (rho < P.rows && nsp != 1 && half == 0)
        P.part_ml[(slot_j * P.hkv + kvh) * P.rows + rho] = make_float2(m_run, l_tot);
    constexpr int kStageRow = D * 2 + 16;
    if constexpr (KH == 1) __syncthreads();    // every wave is done with the tiles
    // a buffer of this wave's own: with KH = 2 the one its pair merged in
    char *stage = dma_wave_buf(KH == 2 ? rblk : wave_u);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            uint32_t hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                hv[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(oacc[dt][4 * j4 + j] * inv));
            *reinterpret_cast<uint2 *>(stage + col * kStageRow + (dt * 32 + 8 * j4 + 4 * half) * 2) =
                make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int row0 = rg * P.rows_per_group + rblk * 32;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int c = lane + 64 * r;
        const int row = c >> 4, piece = c & 15;
        const uint4 v = *reinterpret_cast<const uint4 *>(stage + row * kStageRow + piece * 16);
        const int rr = row0 + row;
        if (rr < P.rows) {
            __bf16 *op;
            if (nsp == 1) {
                const int node = rr / P.group;
                const int h = kvh * P.group + rr % P.group;
                op = static_cast<__bf16 *>(P.out) + (((int64_t)b * P.n + node) * P.hq + h) * D;
            } else {
                op = static_cast<__bf16 *>(P.part_o) + ((slot_j * P.hkv + kvh) * P.rows + rr) * D;
            }
            *reinterpret_cast<uint4 *>(op + piece * 8) = v;
        }
    }
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
    const Work wk = decode_work(P, blockIdx.x, false);
    const int split = wk.split, rg = wk.rg, kvh = wk.kvh, b = wk.b;
    const int L = P.seq_lens[b];
    int err = 0;
    if (L < 0 || L > P.max_seq_len) {
        if (tid == 0 && split == 0 && rg == 0) spec::raise_status(P.status, SPEC_ST_RANGE);
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
    const int kb = split * P.split_len;
    const int ke = min(L + P.n, kb + P.split_len);
    if (kb >= ke) {
        mark_empty_split(P, b, kvh, split, rg);
        return;
    }
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
            const int64_t pidx = (((int64_t)b * P.nsplit + split) * P.hkv + kvh) * P.rows + rho;
#pragma unroll
            for (int j = 0; j < PER; ++j) static_cast<float *>(P.part_o)[pidx * D + lane + 64 * j] = o[j];
            if (lane == 0) P.part_ml[pidx] = make_float2(m, l);
        }
    }
    for (int o2 = 32; o2 > 0; o2 >>= 1) err |= __shfl_xor(err, o2, 64);
    if (lane == 0) spec::raise_status(P.status, err);
}

// ---------------------------------------------------------------------------
// merge of split partials: one wavefront per (row, head) output vector
// ---------------------------------------------------------------------------
//
// A wave merges VPW output vectors (consecutive (row, head) indices), so the
// loads of all of them go out together: first their plan entries, then every
// split's (max, sum) and partial.  Lane s holds split s's (max, sum) (at most
// 64 splits); the weights go to every lane by readlane and the partials are
// accumulated 16 splits at a time.  Lanes own D/64 consecutive dims.

template <int D, int DTYPE, int VPW>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams P) {
    constexpr int PER = D / 64;
    constexpr int kBatch = 16;
    // bf16 partials are O / sum (weight exp2(m - M) * sum), kept packed as
    // loaded (PER values in one word) until used; f32 ones are unnormalised
    // O (weight exp2(m - M))
    constexpr bool kBf = DTYPE == SPEC_BF16;
    typedef typename std::conditional<kBf, typename std::conditional<PER == 2, uint32_t, uint16_t>::type,
                                      float>::type WT;      // one lane's word of a partial
    constexpr int NW_ = kBf ? 1 : PER;                      // words per lane and split
    auto val = [](const WT (&w)[NW_], int j) -> float {
        if constexpr (kBf) return spec::bf16_to_f32((uint16_t)(w[0] >> (16 * j)));
        else return w[j];
    };
    const int lane = threadIdx.x & 63;
    const int64_t vec0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW;
    const int64_t nvec = (int64_t)P.batch * P.n * P.hq;
    const int64_t vstride = (int64_t)P.hkv * P.rows;   // between split slots
    const int64_t sstride = vstride * D / (kBf ? PER : 1);   // in words

    int64_t base[VPW];
    int ns[VPW];
    // (1) plan entries
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        const int64_t vec = vec0 + i;
        ns[i] = 0;
        base[i] = 0;
        if (vec >= nvec) continue;
        const int h = vec % P.hq;
        const int64_t row = vec / P.hq;
        const int node = row % P.n;
        const int b = row / P.n;
        int64_t first = (int64_t)b * P.nsplit;
        int cnt = P.nsplit;
        if (P.dyn) {
            const int2 pl = P.plan[b];
            first = pl.x;
            cnt = pl.y > 1 ? pl.y : 0;     // one split wrote O itself
        }
        ns[i] = cnt;
        base[i] = first * vstride + (int64_t)(h / P.group) * P.rows + node * P.group + h % P.group;
    }
    // (2) every split's (max, sum) and the first kBatch partials of all VPW
    // vectors.  An empty split (static plan) wrote (-inf, 0), so its O is
    // never read into the sum (weight 0; its memory was not written).
    auto words = [&](int i) -> const WT * {
        return reinterpret_cast<const WT *>(static_cast<const char *>(P.part_o) +
                                            (base[i] * D + lane * PER) * (kBf ? 2 : 4));
    };
    float2 ml[VPW];
    WT x[VPW][kBatch][NW_];
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        ml[i] = lane < ns[i] ? P.part_ml[base[i] + lane * vstride] : make_float2(-INFINITY, 0.f);
        const WT *po = words(i);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
#pragma unroll
            for (int j = 0; j < NW_; ++j) x[i][u][j] = u < ns[i] ? po[u * sstride + j] : WT(0);
        }
    }
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        if (ns[i] == 0) continue;
        const WT *po = words(i);
        const float M = spec::wave_max(ml[i].x);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        const float ex = (lane < ns[i] && ml[i].x != -INFINITY) ? exp2f(ml[i].x - Mu) : 0.f;
        const float lsum = spec::wave_sum(ex * ml[i].y);
        const float w = kBf ? ex * ml[i].y : ex;
        float acc[PER] = {};
        for (int s0 = 0; s0 < ns[i]; s0 += kBatch) {
            if (s0 > 0) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
#pragma unroll
                    for (int j = 0; j < NW_; ++j)
                        x[i][u][j] = s0 + u < ns[i] ? po[(s0 + u) * sstride + j] : WT(0);
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const float ws = s0 + u < ns[i]
                    ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u)) : 0.f;
                if (ws > 0.f) {
#pragma unroll
                    for (int j = 0; j < PER; ++j) acc[j] = fmaf(ws, val(x[i][u], j), acc[j]);
                }
            }
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const int64_t vec = vec0 + i;
        if (kBf) {
            uint16_t *op = static_cast<uint16_t *>(P.out) + vec * D + lane * PER;
            uint32_t hb[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j)
                hb[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j] * inv));
            if (PER == 2)
                *reinterpret_cast<uint32_t *>(op) = hb[0] | (hb[PER - 1] << 16);
            else
                op[0] = (uint16_t)hb[0];
        } else {
            float *op = static_cast<float *>(P.out) + vec * D + lane * PER;
#pragma unroll
            for (int j = 0; j < PER; ++j) op[j] = acc[j] * inv;
        }
    }
}

// ---------------------------------------------------------------------------
// host-side planning
// ---------------------------------------------------------------------------

struct Plan {
    int nw;               // waves per workgroup
    int kh;               // bf16: waves per 32-row query block (2: key halves)
    int rows_per_group, rowgroups;
    int split_len, nsplit;  // static plan: every request cut at max_seq_len's splits
    int dyn, slots;         // length-balanced plan over `slots` split slots (bf16, batch > 1)
    int max_span_tiles;     // an upper bound of any split's tiles
};

Plan make_plan(int batch, int n, int hq, int hkv, int max_seq_len, int dtype) {
    Plan pl{};
    const int rows = n * (hq / hkv);
    if (dtype == SPEC_BF16) {
        // 8-wave workgroups of one wave per 32-row block (row groups of up to
        // 256 rows) unless that leaves the device short of workgroups; then
        // row groups of up to 128 rows, which read the same K/V (from L2) in
        // parallel, each block served by two waves (key halves)
        pl.nw = rows <= 128 ? 4 : 8;
        if (pl.nw == 8) {
            const int tiles8 = (max_seq_len + n + kTileKeys - 1) / kTileKeys;
            const int groups8 = batch * hkv * ((rows + 255) / 256) *
                                std::max(1, std::min(tiles8 / kMinTiles, kMaxSplits));
            if (groups8 < kSmallGrid) pl.nw = 4;
        }
        pl.kh = 1;
        pl.rows_per_group = pl.nw * 32;
    } else {
        pl.nw = 4;
        pl.kh = 1;
        pl.rows_per_group = rows;
    }
    pl.rowgroups = (rows + pl.rows_per_group - 1) / pl.rows_per_group;
    // split the key range so the grid has about kTargetGroups workgroups,
    // with at least kMinTiles tiles per split
    const int keys = max_seq_len + n;
    const int tiles = (keys + kTileKeys - 1) / kTileKeys;
    // No split when the (request, KV head, row group) items alone fill the
    // device: splitting would only add partials and the merge.
    const int base = batch * hkv * pl.rowgroups;
    int ns = (kTargetGroups + base - 1) / base;
    ns = std::max(1, std::min({ns, tiles / kMinTiles, kMaxSplits}));
    if (base >= kOneRound) ns = 1;
    const int tiles_per = (tiles + ns - 1) / ns;
    pl.split_len = tiles_per * kTileKeys;
    pl.nsplit = (keys + pl.split_len - 1) / pl.split_len;
    // Several requests: split by the actual lengths instead, so a batch of
    // mixed lengths gives every workgroup about the same number of tiles.
    // No more slots than requests at max_seq_len could use.
    if (dtype == SPEC_BF16 && batch > 1 && batch <= kPlanBatch && base < kOneRound) {
        const int per_head = hkv * pl.rowgroups;
        int S = (kTargetGroups + per_head - 1) / per_head;
        S = std::min(S, batch * std::max(1, std::min(tiles / kMinTiles, kMaxSplits)));
        if (S > batch) {
            pl.dyn = 1;
            pl.slots = S;
        }
    }
    // Longest split: the static plan's split_len; for the length-balanced
    // plan, request b's s_b is t_b / 4 (splits of at most 7 tiles), 64
    // (t_b / 64 tiles) or 1 + floor((S - batch) t_b / T) >= (S - batch) t_b
    // / T (at most T / (S - batch) <= batch t_max / (S - batch) tiles, plus
    // one for rounding).
    pl.max_span_tiles = tiles_per;
    if (pl.dyn)
        pl.max_span_tiles = std::max({7, (tiles + kMaxSplits - 1) / kMaxSplits,
                                      (int)(((int64_t)batch * tiles + (pl.slots - batch) - 1) /
                                            (pl.slots - batch)) + 1});
    // A grid of 4-wave workgroups that fits one workgroup per CU leaves
    // every SIMD one wave: give each 32-row block two waves instead, each
    // taking one 32-key half of every tile.
    const int groups = pl.dyn ? pl.slots * pl.rowgroups * hkv : pl.nsplit * pl.rowgroups * hkv * batch;
    if (dtype == SPEC_BF16 && pl.nw == 4 && groups <= kOneRound) {
        pl.nw = 8;
        pl.kh = 2;
    }
    return pl;
}

// Workspace: partial O [slots][hkv][rows][D] (bf16 or f32, the dtype), then
// (max, sum) [slots][hkv][rows], then the per-request plan (dyn only).
size_t workspace_bytes_for(const Plan &pl, int batch, int n, int hq, int hkv, int d, int dtype,
                           size_t *off_ml = nullptr, size_t *off_plan = nullptr) {
    if (!pl.dyn && pl.nsplit <= 1) return 0;
    const size_t rows = (size_t)n * (hq / hkv);
    const size_t slots = pl.dyn ? (size_t)pl.slots : (size_t)batch * pl.nsplit;
    const size_t parts = slots * hkv * rows;
    const size_t o_ml = spec::align_up(parts * d * (dtype == SPEC_BF16 ? 2 : 4), 256);
    const size_t o_plan = o_ml + spec::align_up(parts * sizeof(float2), 256);
    if (off_ml) *off_ml = o_ml;
    if (off_plan) *off_plan = o_plan;
    return o_plan + (pl.dyn ? spec::align_up((size_t)batch * sizeof(int2), 256) : 0);
}

// The LDS-load form serves 8-wave workgroups (one or two waves per 32-row
// block) at head dim 128 and power-of-two page sizes up to 64, when a slot's
// row of all KV heads fits a buffer record (stride below 2^14 bytes), the
// pool fits 32-bit buffer offsets and no split spans more pages than the
// kernel holds in LDS.
bool dma_form(const Plan &pl, const AttnParams &P, int d) {
    const int64_t stride = (int64_t)P.hkv * d * 2;
    const int ps = P.page_size;
    return d == 128 && pl.nw == 8 && ps >= 1 && ps <= kTileKeys && (ps & (ps - 1)) == 0 &&
           stride < (1 << 14) && P.num_slots * stride < (int64_t(1) << 32) &&
           (int64_t)pl.max_span_tiles * kTileKeys / ps <= kDmaMaxPages;
}

template <int D>
void launch_mfma(const Plan &pl, const AttnParams &P, unsigned groups, hipStream_t st) {
    const int remap = groups % 8 == 0 ? 1 : 0;
    // Up to two rounds of workgroups (the length-balanced plan's usual 512),
    // 4-wave register-staged workgroups two per CU give way to the LDS-load
    // form's 8-wave key-half workgroups one per CU where that form applies
    // (16 x 1024..8192 keys, 32 rows per KV head: 98 -> 87 us per call).
    // The key halves change no row group, so neither the workspace nor the
    // split plan changes.
    if (D == 128 && pl.nw == 4 && groups <= 2 * kOneRound) {
        Plan kh2 = pl;
        kh2.nw = 8;
        kh2.kh = 2;
        if (dma_form(kh2, P, D)) {
            hipLaunchKernelGGL(attn_dma_kernel<2>, dim3(groups), dim3(512), 0, st, P, remap);
            return;
        }
    }
    if (D == 128 && dma_form(pl, P, D) && pl.kh == 2)
        hipLaunchKernelGGL(attn_dma_kernel<2>, dim3(groups), dim3(512), 0, st, P, remap);
    else if (D == 128 && dma_form(pl, P, D))
        hipLaunchKernelGGL(attn_dma_kernel<1>, dim3(groups), dim3(512), 0, st, P, remap);
    else if (pl.kh == 2)
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 8, 2>), dim3(groups), dim3(512), 0, st, P, remap);
    else if (pl.nw == 4)
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 4, 1>), dim3(groups), dim3(256), 0, st, P, remap);
    else
        hipLaunchKernelGGL((attn_split_mfma_kernel<D, 8, 1>), dim3(groups), dim3(512), 0, st, P, remap);
}

}  // namespace

extern "C" size_t spec_verify_attention_workspace_size(int batch, int n, int hq, int hkv, int d,
                                                       int max_seq_len, int dtype) {
    if (batch <= 0 || n <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_seq_len < 0) return 0;
    const Plan pl = make_plan(batch, n, hq, hkv, max_seq_len, dtype);
    return workspace_bytes_for(pl, batch, n, hq, hkv, d, dtype);
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
    if (n > 64 || (d != 64 && d != 128) || num_slots > INT32_MAX) return SPEC_ERR_UNSUPPORTED;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if ((int64_t)max_pages * page_size < (int64_t)max_seq_len && max_seq_len > 0) return SPEC_ERR_SHAPE;
    if (batch == 0) return SPEC_OK;
    if (num_slots == 0) return SPEC_ERR_SHAPE;   // the tree keys alone need slots
    if (!q || !k_pool || !v_pool || !seq_lens || !out_cache_loc || !tree_mask || !out)
        return SPEC_ERR_NULL;
    if (max_seq_len > 0 && !page_table) return SPEC_ERR_NULL;
    const int wb = spec_mask_word_bytes(n);
    const uintptr_t align_bad = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
                                 reinterpret_cast<uintptr_t>(v_pool) | reinterpret_cast<uintptr_t>(out)) & 15u;
    if (align_bad || reinterpret_cast<uintptr_t>(tree_mask) % wb) return SPEC_ERR_SHAPE;

    const Plan pl = make_plan(batch, n, hq, hkv, max_seq_len, dtype);
    size_t off_ml = 0, off_plan = 0;
    const size_t need = workspace_bytes_for(pl, batch, n, hq, hkv, d, dtype, &off_ml, &off_plan);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SPEC_ERR_WORKSPACE;

    AttnParams P{};
    P.batch = batch; P.n = n; P.hq = hq; P.hkv = hkv; P.group = hq / hkv; P.rows = n * P.group;
    P.page_size = page_size; P.max_pages = max_pages; P.max_seq_len = max_seq_len;
    P.split_len = pl.split_len; P.nsplit = pl.nsplit; P.rowgroups = pl.rowgroups;
    P.rows_per_group = pl.rows_per_group; P.word_bytes = wb;
    P.dyn = pl.dyn; P.slots = pl.slots;
    const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)d);
    P.scale_log2 = scale * kLog2e;
    P.num_slots = num_slots;
    P.q = q; P.k_pool = k_pool; P.v_pool = v_pool; P.page_table = page_table;
    P.seq_lens = seq_lens; P.out_cache_loc = out_cache_loc;
    P.mask = static_cast<const uint8_t *>(tree_mask); P.out = out;
    if (need > 0) {
        P.part_o = workspace;
        P.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(workspace) + off_ml);
        if (pl.dyn) P.plan = reinterpret_cast<int2 *>(static_cast<char *>(workspace) + off_plan);
    }
    P.status = dev_status;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const unsigned groups = pl.dyn ? (unsigned)(pl.slots * pl.rowgroups * hkv)
                                   : (unsigned)(pl.nsplit * pl.rowgroups * hkv * batch);
    if (dtype == SPEC_BF16) {
        if (d == 128) launch_mfma<128>(pl, P, groups, st);
        else launch_mfma<64>(pl, P, groups, st);
    } else {
        if (d == 128) hipLaunchKernelGGL(attn_split_f32_kernel<128>, dim3(groups), dim3(256), 0, st, P);
        else hipLaunchKernelGGL(attn_split_f32_kernel<64>, dim3(groups), dim3(256), 0, st, P);
    }
    if (pl.dyn || pl.nsplit > 1) {
        const int64_t nvec = (int64_t)batch * n * hq;
        if (dtype == SPEC_BF16) {
            const dim3 mgrid((unsigned)((nvec + 4 * kMergeVec - 1) / (4 * kMergeVec)));
            if (d == 128)
                hipLaunchKernelGGL((attn_merge_kernel<128, SPEC_BF16, kMergeVec>), mgrid, dim3(256), 0, st, P);
            else
                hipLaunchKernelGGL((attn_merge_kernel<64, SPEC_BF16, kMergeVec>), mgrid, dim3(256), 0, st, P);
        } else {
            const dim3 mgrid((unsigned)((nvec + 3) / 4));
            if (d == 128) hipLaunchKernelGGL((attn_merge_kernel<128, SPEC_F32, 1>), mgrid, dim3(256), 0, st, P);
            else hipLaunchKernelGGL((attn_merge_kernel<64, SPEC_F32, 1>), mgrid, dim3(256), 0, st, P);
        }
    }
    return spec::launch_status();
}
