// Per-level router: score candidate nodes for every query head of a KV group,
// keep each head's minimal top-p set, and compact the union of kept nodes into
// the next level's parent list, all on the device.
//
// Method (page "Zyphra 分层注意力（ZHA）…", section 机制拆解; page "ZHA
// 用树形稀疏注意力改造现有大模型", section 稀疏注意力为什么还会被索引拖慢; page
// geek-terminal "階層型疎Attention「ZHA」…", section 技術的ディープダイブ):
//   sigma_n(q) = max_r (tau q.s_{n,r} + b_{n,r}), pi = softmax(sigma) over the
//   level's candidates, keep the shortest prefix in descending-pi order whose
//   cumulative probability reaches p (ties by ascending node index), expand
//   only the kept nodes' children.
//
// Scoring is a [G x d] x [d x (candidates*R)] product per group: one MFMA
// 16x16x4 fp32 tile holds 16 heads (G real) against 16 planes, and the planes
// stream from HBM once per group whatever the number of heads that see them.
//
// Selection keeps, per query head, the shortest prefix of candidates in
// descending-probability order whose mass reaches p.  Probabilities are handled
// as 2^40-scaled integers e_i = exp(sigma_i - max) so that every sum is exact and
// order-free (bitwise-reproducible).  Candidates are ranked by delta_i = max -
// sigma_i quantised to 2^-27 (monotone in sigma) and the cut is found by a
// mass-weighted radix select; candidates whose quantised delta equals the cut's
// are taken in ascending position (= node) order until the cumulative mass
// reaches ceil(p * sum e).  Small frontiers (<= 1024 candidates per group) are
// selected by one workgroup, one wave per head, with 8-bit digits; larger ones
// by one 1024-thread workgroup per head with 11/11/10-bit digits, whose kept
// flags go to per-head bitmaps over the candidate positions.  A merge kernel, or
// the next level's score kernel, turns the bitmaps into the group's kept list.
//
// The candidates of a level are never written out: they are the children of the
// level above's kept nodes (kept list and head masks, ascending) followed by the
// level's orphans, so a candidate's node id and head mask come from one read of
// its parent's kept-list entry (or, below an unmerged level, from that level's
// bitmaps staged in LDS).
#include <algorithm>

#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kScoreThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr float kFix = 1099511627776.0f;   // 2^40: fixed-point scale of e_i in [0, 1]
constexpr float kKeyScale = 134217728.0f;  // 2^27: delta quantum
constexpr float kDeltaMax = 32.0f;         // e^-32 * 2^40 < 1: heavier deltas carry no mass

// threadIdx.x as a value that the compiler cannot hoist out of a loop: per-lane
// addresses are recomputed where they are used instead of held in registers
__device__ __forceinline__ int lane_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ uint32_t all_heads(int G) { return G >= 32 ? 0xFFFFFFFFu : ((1u << G) - 1u); }

// Kept parents of group g (0 at the first routed level, whose parent pointer is
// readable memory with an unused value), read after every read the caller issued
// before it so that all of them share one round trip: left alone, the compiler
// waits for a load whose value it needs in a scalar register right where it
// issues it, ahead of everything else, and sinks reads used only past an early
// return below that wait.
__device__ __forceinline__ int parent_count(const ZhaLevelArgs& a, int g) {
    int raw = a.pnkept[g];
    asm volatile("" : "+v"(raw)::"memory");
    return a.top ? 0 : __builtin_amdgcn_readfirstlane(raw);
}

// Bit `lane` of a 64-bit word, and the number of set bits below it.
__device__ __forceinline__ uint32_t lane_bit(uint64_t w, int lane) {
    const uint32_t h = lane < 32 ? (uint32_t)w : (uint32_t)(w >> 32);
    return (h >> (lane & 31)) & 1u;
}
__device__ __forceinline__ uint32_t bits_below_lane(uint64_t w) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(w >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)w, 0u));
}

// A level whose merge is left to the level below it: the score workgroups of the
// level below stage its per-head kept bitmaps (position-indexed, [G][wc] words),
// their union and its popcount prefix, and the kept list of the level above it
// (its parents), then read any entry of its kept list from LDS.
constexpr int kDeferW = ZHA_DEFER_WORDS / kScoreThreads;    // head words per thread
constexpr int kDeferP = ZHA_DEFER_PARENTS / kScoreThreads;  // parent entries per thread
static_assert(kDeferW * kScoreThreads == ZHA_DEFER_WORDS && kDeferP * kScoreThreads == ZHA_DEFER_PARENTS,
              "deferred merge staging");

struct DeferView {
    const uint64_t* hw;    // [G][wc] head words
    const uint64_t* u;     // [wc] union of the head words (zero from word nw on)
    const uint32_t* pre;   // [wc] kept nodes in the words below
    const int32_t* gk;     // the level's parents (kept list of the level above it)
    int wc, nw, gn;        // words per head, words holding candidates, parents kept
};

// Node id and head mask of the level's candidate at position qp.
__device__ __forceinline__ void defer_node(const ZhaLevelArgs& pa, const DeferView& v, int G, int c, int qp,
                                           int32_t& node, uint32_t& mask) {
    const int w = qp >> 6, b = qp & 63;
    if (pa.top) node = qp;
    else if (qp < v.gn * c) {
        const int gi = (int)zha_div((uint32_t)qp, pa.dc);
        node = v.gk[gi] * c + (qp - gi * c);
    } else node = (int32_t)pa.orph_lo + (qp - v.gn * c);
    uint32_t m = 0;
    for (int hh = 0; hh < G; ++hh) m |= (uint32_t)((v.hw[hh * v.wc + w] >> b) & 1ull) << hh;
    mask = m;
}

// Entry r (< the kept count) of the level's kept list: the word holding it (the
// last whose prefix is <= r), then its bit by halving popcounts.
__device__ __forceinline__ void defer_entry(const ZhaLevelArgs& pa, const DeferView& v, int G, int c, uint32_t r,
                                            int32_t& node, uint32_t& mask) {
    int lo = 0, hi = v.nw - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (v.pre[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    uint64_t x = v.u[lo];
    uint32_t k = r - v.pre[lo];
    int b = 0;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
        const uint32_t cnt = (uint32_t)__popcll(x & ((1ull << sh) - 1ull));
        if (k >= cnt) {
            k -= cnt;
            x >>= sh;
            b += sh;
        }
    }
    defer_node(pa, v, G, c, lo * 64 + b, node, mask);
}

// Scores one level's candidates for every head of group g, as workgroup blk of
// nblk (256 threads).  Each wave scores items of U = 16/R candidates (R <= 16)
// or one candidate over R/16 column blocks (R > 16).  ALL: every node of the
// level is a candidate of every head (positions are node ids), whatever the
// level above kept.  hm gets the largest score of the lane's heads 4 kq + i.
// DEF: the level above (pa) was selected but not merged; its kept list is
// derived here from its bitmaps (dynamic LDS), and this workgroup writes its
// share of it (all of it together with the other workgroups).
// Candidate positions and node ids fit in 32 bits (capacity < 2^31).
template <bool BF16, bool ALL, bool DEF = false>
__device__ __forceinline__ void score_level(const void* __restrict__ q, const ZhaLevelArgs& a, int G, int c, int R,
                                            float tau, int g, int blk, int nblk, float (&hm)[4],
                                            const ZhaLevelArgs* pa = nullptr) {
    // every argument the kernel uses, fetched in one batch before any of them is
    // needed (otherwise the loads come in dependent rounds behind uniform branches)
    asm volatile("" ::"s"(q), "s"(a.S), "s"(a.B), "s"(a.cap), "s"(a.top), "s"(a.n_top), "s"(a.pklist),
                 "s"(a.pkmask), "s"(a.pnkept), "s"(a.pcap), "s"(a.orph_lo), "s"(a.orph_hi), "s"(a.dc.m),
                 "s"(a.dc.s1), "s"(a.dc.s2), "s"(a.ncand), "s"(a.sig), "s"(a.hblk), "s"(G), "s"(c), "s"(R),
                 "s"(tau));
    const bool top = ALL || a.top;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kq = lane >> 4;
    const int U = R <= 16 ? 16 / R : 1;
    const int CB = R <= 16 ? 1 : R / 16;
    const int span = R <= 16 ? R : 16;
    const int cl = R <= 16 ? j / R : 0;
    const uint32_t allg = all_heads(G);
    const size_t lrow = (size_t)g * a.cap;
    const size_t prow = (size_t)g * a.pcap;
    const int stride = nblk * 4;
    const int pcap = (int)a.pcap;

    // One round trip before any work: the parent count, the first item's parent
    // entry (its index clamped to the parent level's capacity, not bounded by the
    // count) and the query rows are all in flight together.  At the first routed
    // level the parent arrays point at readable memory whose values go unused.
    int it = blk * 4 + wave;
    int32_t pk = 0;
    uint32_t pm = 0;
    int pn_raw = 0;
    uint64_t dw[DEF ? kDeferW : 1];
    int32_t dg[DEF ? kDeferP : 1];
    if (DEF) {
        // the level above's head words, its parents' node ids and their count
        const int nall = G * (int)pa->wcap;
        const uint64_t* kb = pa->kbm + (size_t)g * G * pa->wcap;
#pragma unroll
        for (int k = 0; k < kDeferW; ++k) {
            dw[k] = 0ull;
            if (k * kScoreThreads < nall) {           // uniform: slots wholly past the end skipped
                const int i = (int)threadIdx.x + k * kScoreThreads;
                if (i < nall) dw[k] = kb[i];
            }
        }
        const int gcap = pa->top ? 0 : (int)pa->pcap;
#pragma unroll
        for (int k = 0; k < kDeferP; ++k) {
            dg[k] = 0;
            if (k * kScoreThreads < gcap) {
                const int i = (int)threadIdx.x + k * kScoreThreads;
                if (i < gcap) dg[k] = pa->pklist[(size_t)g * pa->pcap + i];
            }
        }
        pn_raw = pa->pnkept[g];
    } else {
        const int pi0 = min((int)zha_div((uint32_t)(it * U + cl), a.dc), pcap - 1);
        pk = a.pklist[prow + pi0];
        pm = a.pkmask[prow + pi0];
        pn_raw = a.pnkept[g];
    }
    // A operand: row = query head j of the group (zero beyond G), contraction index
    // d = 16m + 4kq + e.
    float qa[32];
    const int jq = j < G ? j : 0;
    if (BF16) {
        const uint16_t* qr = static_cast<const uint16_t*>(q) + ((size_t)g * G + jq) * ZHA_D + 4 * kq;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint2 v = *reinterpret_cast<const uint2*>(qr + 16 * m);
            qa[4 * m + 0] = zha_bf16_to_f32(v.x & 0xFFFFu);
            qa[4 * m + 1] = zha_bf16_to_f32(v.x >> 16);
            qa[4 * m + 2] = zha_bf16_to_f32(v.y & 0xFFFFu);
            qa[4 * m + 3] = zha_bf16_to_f32(v.y >> 16);
        }
    } else {
        const float* qr = static_cast<const float*>(q) + ((size_t)g * G + jq) * ZHA_D + 4 * kq;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 v = *reinterpret_cast<const float4*>(qr + 16 * m);
            qa[4 * m + 0] = v.x; qa[4 * m + 1] = v.y; qa[4 * m + 2] = v.z; qa[4 * m + 3] = v.w;
        }
    }
    asm volatile("" ::"v"(pk), "v"(pm), "s"(pn_raw), "v"(qa[0]), "v"(qa[31]));
#pragma unroll
    for (int k = 0; k < 32; ++k) qa[k] = j < G ? qa[k] : 0.f;
    DeferView dv{};
    if constexpr (DEF) {
        extern __shared__ __align__(16) uint64_t zha_defer_lds[];
        __shared__ uint32_t s_wsum[kScoreThreads / 64];
        const int tid = threadIdx.x;
        const int wc = (int)pa->wcap, nall = G * wc;
        const int gcap = pa->top ? 0 : (int)pa->pcap;
        uint64_t* hw = zha_defer_lds;
        uint64_t* uu = hw + nall;
        uint32_t* pre = reinterpret_cast<uint32_t*>(uu + wc);
        int32_t* gk = reinterpret_cast<int32_t*>(pre + wc);
        const int gn = pa->top ? 0 : pn_raw;
        const int nl = pa->top ? (int)pa->n_top : gn * c + (int)(pa->orph_hi - pa->orph_lo);
        const int nwl = (nl + 63) >> 6;
#pragma unroll
        for (int k = 0; k < kDeferW; ++k) {
            const int i = tid + k * kScoreThreads;
            if (i < nall) hw[i] = dw[k];
        }
#pragma unroll
        for (int k = 0; k < kDeferP; ++k) {
            const int i = tid + k * kScoreThreads;
            if (i < gcap) gk[i] = dg[k];
        }
        __syncthreads();
        // union of words [tid P, tid P + P) (words from nwl on hold no candidate),
        // then the workgroup's exclusive popcount prefix
        const int P = (wc + kScoreThreads - 1) / kScoreThreads;
        uint32_t cnt = 0;
#pragma unroll 1
        for (int k = 0; k < P; ++k) {
            const int w = tid * P + k;
            uint64_t x = 0;
            if (w < nwl)
                for (int hh = 0; hh < G; ++hh) x |= hw[hh * wc + w];
            if (w < wc) uu[w] = x;
            cnt += (uint32_t)__popcll(x);
        }
        const uint32_t inc = (uint32_t)zha_wave_incl_scan_u64(cnt);
        if (lane == 63) s_wsum[wave] = inc;
        __syncthreads();
        uint32_t run = inc - cnt, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kScoreThreads / 64; ++w2) {
            const uint32_t x = s_wsum[w2];
            run += w2 < wave ? x : 0u;
            tot += x;
        }
#pragma unroll 1
        for (int k = 0; k < P; ++k) {
            const int w = tid * P + k;
            if (w < wc) {
                pre[w] = run;
                run += (uint32_t)__popcll(uu[w]);
            }
        }
        __syncthreads();
        dv = DeferView{hw, uu, pre, gk, wc, nwl, gn};
        pn_raw = (int)tot;
    }
    if (top) {
        pk = 0;
        pm = allg;
    }
    const int pn = top ? 0 : pn_raw;
    const int n_cand = top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);

    const int items = (n_cand + U - 1) / U;
#pragma unroll
    for (int i = 0; i < 4; ++i) hm[i] = zha_neg_inf();   // largest score per head
    for (; it < items; it += stride) {
        const int pos = it * U + cl;
        const bool valid = pos < n_cand;
        int32_t node = 0;
        uint32_t cm = 0;
        if (valid) {
            if (top) {
                node = pos;
                cm = allg;
            } else if (pos < pn * c) {
                // child pos % c of the kept parent at index pos / c
                const int pi = (int)zha_div((uint32_t)pos, a.dc);
                if (DEF) defer_entry(*pa, dv, G, c, (uint32_t)pi, pk, pm);
                node = pk * c + (pos - pi * c);
                cm = pm;
            } else {
                node = (int32_t)a.orph_lo + (pos - pn * c);
                cm = allg;
            }
        }
        if (!DEF && !top) {
            // parent entry of this wave's next item, in flight with this item's planes
            const int npi = (int)zha_div((uint32_t)((it + stride) * U + cl), a.dc);
            if (it + stride < items && npi < pn) {
                pk = a.pklist[prow + npi];
                pm = a.pkmask[prow + npi];
            }
        }
        float best[4] = {zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf()};
        for (int cb = 0; cb < CB; ++cb) {
            const int r = R <= 16 ? (j % R) : (cb * 16 + j);
            const size_t prw = (lrow + (size_t)node) * R + r;
            float4 sv[8];
            if (valid) {
                const float4* plane = reinterpret_cast<const float4*>(a.S + prw * ZHA_D);
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = plane[4 * m + kq];
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            const float bv = valid ? a.B[prw] : zha_neg_inf();
            zha_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * m + 0], sv[m].x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * m + 1], sv[m].y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * m + 2], sv[m].z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * m + 3], sv[m].w, acc, 0, 0, 0);
            }
            // lane holds heads 4kq+i against plane j
#pragma unroll
            for (int i = 0; i < 4; ++i) best[i] = fmaxf(best[i], fmaf(tau, acc[i], bv));
        }
        // max over the planes of one candidate (adjacent columns)
        if (span == 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) best[i] = zha_row16_max(best[i]);
        } else {
            for (int o = span >> 1; o > 0; o >>= 1)
#pragma unroll
                for (int i = 0; i < 4; ++i) best[i] = fmaxf(best[i], __shfl_xor(best[i], o, 16));
        }
        if (valid && (j % span) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * kq + i;
                if (h < G) a.sig[((size_t)g * G + h) * a.cap + (size_t)pos] = ((cm >> h) & 1u) ? best[i] : zha_neg_inf();
            }
        }
        if (valid) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((cm >> (4 * kq + i)) & 1u) hm[i] = fmaxf(hm[i], best[i]);
        }
    }
    // Stores issued before the loop would hold up its first loads (the memory
    // counter waits are in order), so the counts and the derived kept list go last.
    if (blk == 0 && threadIdx.x == 0) a.ncand[g] = n_cand;
    if constexpr (DEF) {
        // this workgroup's share of the level above's kept list: words 4 blk + wave
        // + 4 nblk k, one position per lane
        int32_t* kl = pa->klist + (size_t)g * pa->cap;
        uint32_t* km = pa->kmask + (size_t)g * pa->cap;
#pragma unroll 1
        for (int w = blk * 4 + wave; w < dv.nw; w += 4 * nblk) {
            const uint64_t x = dv.u[w];
            if (lane_bit(x, lane)) {
                int32_t node;
                uint32_t msk;
                defer_node(*pa, dv, G, c, w * 64 + lane, node, msk);
                const uint32_t rank = dv.pre[w] + bits_below_lane(x);
                kl[rank] = node;
                km[rank] = msk;
            }
        }
        if (blk == 0 && threadIdx.x == 0) pa->nkept[g] = pn;
    }
}

// Sliced levels: the largest score of each head over this workgroup.
__device__ __forceinline__ void block_head_max(const ZhaLevelArgs& a, int g, int G, const float (&hm)[4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kq = lane >> 4;
    __shared__ float s_hm[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x = zha_row16_max(hm[i]);
        if (j == 0) s_hm[wave][4 * kq + i] = x;
    }
    __syncthreads();
    if ((int)threadIdx.x < G) {
        const int h = threadIdx.x;
        const float x = fmaxf(fmaxf(s_hm[0][h], s_hm[1][h]), fmaxf(s_hm[2][h], s_hm[3][h]));
        a.hblk[(size_t)(g * G + h) * ZHA_SCORE_MAXB + blockIdx.x] = x;
    }
}

// grid (blocks, H_kv), 256 threads: one level's candidate scores.
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_kernel(const void* __restrict__ q,
                                                                        ZhaLevelArgs a, int G, int c, int R,
                                                                        float tau) {
    const int g = blockIdx.y;
    float hm[4];
    score_level<BF16, false>(q, a, G, c, R, tau, g, blockIdx.x, gridDim.x, hm);
    if (a.hblk) block_head_max(a, g, G, hm);
}

// As zha_route_score_kernel, for a level whose parent level (pa) was selected but
// not merged: the workgroups derive and write that level's kept list themselves
// (dynamic LDS: zha_defer_lds_bytes).
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_defer_kernel(const void* __restrict__ q,
                                                                              ZhaLevelArgs a, ZhaLevelArgs pa,
                                                                              int G, int c, int R, float tau) {
    ZHA_LEVEL_ARGS_READY(pa, "s"(G));
    const int g = blockIdx.y;
    float hm[4];
    score_level<BF16, false, true>(q, a, G, c, R, tau, g, blockIdx.x, gridDim.x, hm, &pa);
    if (a.hblk) block_head_max(a, g, G, hm);
}

// grid (max blocks, H_kv, levels), 256 threads: every node of each of the first
// routed levels scored for every head of the group, positions = node ids (the
// levels' selection then gathers its candidates' scores from these).
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_all_kernel(const void* __restrict__ q,
                                                                            ZhaChainArgs m, int G, int c, int R,
                                                                            float tau) {
    const int z = blockIdx.z;
    if ((int)blockIdx.x >= m.blocks[z]) return;
    float hm[4];
    score_level<BF16, true>(q, m.lv[z], G, c, R, tau, blockIdx.y, blockIdx.x, m.blocks[z], hm);
}

// ---- selection helpers

// Exclusive prefix sum across one wave (all lanes active); *total gets the wave sum.
__device__ __forceinline__ uint64_t wave_excl_scan_u64(uint64_t v, uint64_t* total) {
    const uint64_t x = zha_wave_incl_scan_u64(v);
    *total = zha_readlane_u64(x, 63);
    return x - v;
}

// Selection keys: the quantised delta of a candidate that carries mass, or one
// of two sentinels.  A candidate's fixed-point mass is a function of its key
// alone, so every pass sees exactly the same masses.
constexpr uint32_t kNotCand = 0xFFFFFFFFu;    // not this head's candidate
constexpr uint32_t kNoMass = 0xFFFFFFFEu;     // candidate with delta >= kDeltaMax (mass 0)
constexpr float kDeltaBelowMax = 31.999998092651367f;   // largest float below kDeltaMax

__device__ __forceinline__ uint32_t key_of(float s, float m) {
    const float dl = m - s;                   // NaN or +inf only for s = -inf
    const uint32_t k = (uint32_t)(fminf(dl, kDeltaBelowMax) * kKeyScale);
    return s == zha_neg_inf() ? kNotCand : (dl < kDeltaMax ? k : kNoMass);
}

__device__ __forceinline__ uint64_t mass_of(uint32_t key) {
    // e^{-delta} with delta = key * 2^-27, as 2^40-scaled fixed point truncated to
    // an integer.  x <= 2^40 has 24 significant bits, so x = hi * 2^32 + lo with
    // both parts exact.  The exponent lies in [-46.2, 0] for every 32-bit key,
    // where the hardware exp2 is what exp2f returns (exp2f only rescales
    // arguments below -126).
    const float x = __builtin_amdgcn_exp2f(-(float)key * (1.4426950408889634f / kKeyScale)) * kFix;
    const float hi = floorf(x * 0x1p-32f);
    const float lo = fmaf(hi, -0x1p32f, x);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Large frontiers: 2048-bin histograms of key digits 31..21, 20..10 and 9..0.
// Bin b sits at b + b / 32 so that one lane's 32 consecutive bins are read
// without LDS bank conflicts.
constexpr int kHistBins = 2048;
constexpr int kHistPadded = kHistBins + kHistBins / 32;
__device__ __forceinline__ int hpad(uint32_t b) { return (int)(b + (b >> 5)); }

// Run by one whole wave: the bin b with before(b) < need <= before(b) + hist[b]
// (before(b) = mass of the bins below b) goes to *out_bin / *out_before.  When
// `need` is 0 it is first set to ceil(p * total) (clamped to [1, total]).  Two
// scans: over the 64 lanes' 32-bin sums, then over the 32 bins of the lane
// whose range holds the crossing.
__device__ void wave_find_cross(const uint64_t* hist, uint64_t need, float top_p, int* out_bin,
                                uint64_t* out_before, uint64_t* out_need) {
    const int lane = threadIdx.x & 63;
    const uint64_t* row = hist + lane * 33;
    uint64_t mine = 0;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) mine += row[i];
    uint64_t total;
    const uint64_t before = wave_excl_scan_u64(mine, &total);
    if (need == 0) {
        uint64_t T = (uint64_t)ceil((double)top_p * (double)total);
        if (T < 1) T = 1;
        if (T > total) T = total;
        need = T;
    }
    const uint64_t hit = __ballot(before < need && before + mine >= need);
    const int L = hit ? __ffsll((long long)hit) - 1 : 63;
    const uint64_t base = zha_readlane_u64(before, L);
    const uint64_t x = lane < 32 ? hist[L * 33 + lane] : 0ull;
    uint64_t t2;
    const uint64_t ex = wave_excl_scan_u64(x, &t2);
    const uint64_t hit2 = __ballot(lane < 32 && base + ex < need && base + ex + x >= need);
    const int jb = hit2 ? __ffsll((long long)hit2) - 1 : 31;
    const uint64_t ex_j = zha_readlane_u64(ex, jb);
    if (lane == 0) {
        *out_bin = L * 32 + jb;
        *out_before = base + ex_j;
        *out_need = need;
    }
}

constexpr int kLdsKeys = ZHA_LDS_KEYS;        // heads with at most this many candidates keep their keys in LDS
constexpr int kSlots = kLdsKeys / kSelThreads;   // positions tid + 1024 k held in registers while staging
constexpr int kMergeW = kLdsKeys / 64;        // bitmap words merged per step
constexpr int kBatch = 8;                     // LDS keys read together in a pass
constexpr int kGlobBatch = 16;                // scores re-read together from global memory
constexpr int kMergeBlocks = 64;              // merge workgroups per group
constexpr int kRankMax = 128;                 // crossing-bin keys ranked directly instead of histogrammed
static_assert((kSlots & (kSlots - 1)) == 0 && kSlots % kBatch == 0, "slot batches");
constexpr int kSmallN = 1024;                 // groups with at most this many candidates select in one workgroup
static_assert(kSmallN == ZHA_SMALL_SLOTS, "small levels");
constexpr int kSmallK = kSmallN / 64;
static_assert(kSelThreads == kSmallN, "small path: one position per thread");
static_assert(2 * ZHA_MAX_GROUP * kMergeW + kMergeW * 32 <= kLdsKeys,
              "merge: head words and parent ids must fit the key buffer");
static_assert(kMergeW + kMergeW / 2 <= kHistPadded, "merge: union words and prefixes must fit the histogram");
static_assert(kMergeW <= kSelThreads, "merge: one thread per word of a step");
static_assert(ZHA_MAX_GROUP * (kSmallN + 2 * 256) + kSmallN <= kLdsKeys, "small path inside the key buffer");
static_assert(ZHA_MAX_GROUP * kSmallK <= kHistPadded, "small-path kept words inside the histogram");

// The cut inside a crossing bin that holds few keys.  Ordered by (key,
// position), the bin's keys are taken while the mass before them is below
// `need` (what the bin must still supply); the cut is the key, and the position,
// whose own mass reaches it.  Entry e = {key, position, mass lo, mass hi}: the mass
// before entry j is the sum over the entries that precede it in that order.
__device__ __forceinline__ bool rank_precedes(const uint4& f, const uint4& e) {
    return f.x < e.x || (f.x == e.x && f.y < e.y);
}
__device__ __forceinline__ uint64_t entry_mass(const uint4& e) { return ((uint64_t)e.w << 32) | e.z; }

// Small-path histogram bins pack a key count above a mass sum: at most kSmallN
// keys of mass <= 2^40 sum below 2^52, so the fields never carry into each other
// and one 64-bit LDS atomic per key updates both.
constexpr int kCntShift = 52;
constexpr uint64_t kMassMask = (1ull << kCntShift) - 1ull;

// One wave selects for one query head among n <= 64 K candidates whose scores
// are in LDS (sg); position lane + 64k sits in register slot k.  8-bit digits,
// a wave-local packed histogram (hist: 256 u64), no workgroup barrier.
// The kept bitmap words go to kw[16 k], k < nk.
template <int K>
__device__ void select_head_wave(const float* sg, int n, float top_p, uint64_t* hist, uint64_t* kw,
                                 uint32_t* n_cand_out, uint32_t* n_kept_out) {
    const int lane = lane_tid() & 63;
    const int nk = (n + 63) >> 6;
    float sv[K];
    float m = zha_neg_inf();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int pos = lane + 64 * k;
        sv[k] = pos < n ? sg[pos] : zha_neg_inf();
        m = fmaxf(m, sv[k]);
    }
    m = zha_wave_max(m);
    uint32_t key[K];
#pragma unroll
    for (int k = 0; k < K; ++k) key[k] = key_of(sv[k], m);
    const bool none = m == zha_neg_inf();
    const bool keep_all = !none && top_p >= 1.0f;
    uint32_t ustar = 0, ties = 0;
    uint64_t need = 0;
    if (!none && !keep_all) {
        uint32_t prefix = 0;
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            reinterpret_cast<uint4*>(hist)[2 * lane] = make_uint4(0u, 0u, 0u, 0u);
            reinterpret_cast<uint4*>(hist)[2 * lane + 1] = make_uint4(0u, 0u, 0u, 0u);
            zha_wave_lds_sync();
            // keys whose digits above this pass's match the prefix found so far
            const uint32_t hs = pass == 0 ? 31u : (uint32_t)(shift + 8);
            const uint32_t want = pass == 0 ? 0u : prefix;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t kk = key[k];
                const uint32_t top = pass == 0 ? 0u : (kk >> hs);
                if (kk < kNoMass && top == want)
                    atomicAdd((unsigned long long*)&hist[(kk >> shift) & 255u],
                              (unsigned long long)(mass_of(kk) | (1ull << kCntShift)));
            }
            zha_wave_lds_sync();
            const uint4 h01 = reinterpret_cast<const uint4*>(hist)[2 * lane];
            const uint4 h23 = reinterpret_cast<const uint4*>(hist)[2 * lane + 1];
            const uint64_t hb[4] = {((uint64_t)h01.y << 32) | h01.x, ((uint64_t)h01.w << 32) | h01.z,
                                    ((uint64_t)h23.y << 32) | h23.x, ((uint64_t)h23.w << 32) | h23.z};
            const uint64_t mine = hb[0] + hb[1] + hb[2] + hb[3];
            uint64_t total;
            uint64_t before = wave_excl_scan_u64(mine, &total) & kMassMask;
            if (pass == 0) {
                const uint64_t tm = total & kMassMask;
                const uint64_t T = (uint64_t)ceil((double)top_p * (double)tm);
                need = T < 1 ? 1 : (T > tm ? tm : T);
            }
            int my_bin = -1;
            uint64_t my_before = 0, my_val = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t hm = hb[i] & kMassMask;
                const bool cross = before < need && before + hm >= need && my_bin < 0;
                my_bin = cross ? lane * 4 + i : my_bin;
                my_before = cross ? before : my_before;
                my_val = cross ? hb[i] : my_val;
                before += hm;
            }
            const uint64_t found = __ballot(my_bin >= 0);
            const int src = found ? __ffsll((long long)found) - 1 : 0;
            const uint32_t bin = (uint32_t)__builtin_amdgcn_readlane(my_bin, src);
            need -= zha_readlane_u64(my_before, src);
            prefix = (prefix << 8) | bin;
            const uint32_t cnt = (uint32_t)(zha_readlane_u64(my_val, src) >> kCntShift);
            zha_wave_lds_sync();
            if (cnt == 1 || pass == 3) {
                // the crossing bin holds one key (or the keys equal to the cut): the cut
                // is the largest key with this prefix
                ustar = (prefix << shift) | ((1u << shift) - 1u);
                ties = cnt;
                break;
            }
        }
    }
    uint32_t n_cand = 0, n_kept = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool cand = k < nk && key[k] != kNotCand;
        const bool kept = !none && (keep_all ? cand : (cand && key[k] < kNoMass && (key[k] < ustar || (key[k] == ustar && ties == 1))));
        const uint64_t wk = __ballot(kept);
        n_cand += __popcll(__ballot(cand));
        n_kept += __popcll(wk);
        if (lane == 0 && k < nk) kw[16 * k] = wk;
    }
    zha_wave_lds_sync();
    if (!none && !keep_all && ties > 1) {
        // several candidates share the cut key: take them in ascending position order
        uint64_t run = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint64_t w = (k < nk && key[k] == ustar) ? mass_of(key[k]) : 0ull;
            uint64_t tot;
            const uint64_t ex = wave_excl_scan_u64(w, &tot);
            const uint64_t extra = __ballot(w > 0 && run + ex < need);
            n_kept += __popcll(extra);
            if (lane == 0 && k < nk) kw[16 * k] |= extra;
            run += tot;
        }
        zha_wave_lds_sync();
    }
    *n_cand_out = n_cand;
    *n_kept_out = n_kept;
}

// Scores of all G heads at position tid (< cap) into LDS, and the node id of
// that position; every global read, the parent count among them, is issued
// before any result is used.  Returns the parent count.
__device__ __forceinline__ int stage_small(const ZhaLevelArgs& a, int g, int G, int c, int tid,
                                           float* s_sig, int32_t* s_nid) {
    const bool in = tid < a.cap;
    float v[ZHA_MAX_GROUP];
#pragma unroll
    for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) {
        v[hh] = zha_neg_inf();
        if (hh < G && in) v[hh] = a.sig[((size_t)g * G + hh) * a.cap + tid];   // hh < G: uniform
    }
    const int pi = (int)zha_div((uint32_t)tid, a.dc);
    const int32_t pk = pi < a.pcap ? a.pklist[(size_t)g * a.pcap + pi] : 0;   // unused at the first level
    const int pn = parent_count(a, g);
#pragma unroll
    for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh)
        if (hh < G) s_sig[hh * kSmallN + tid] = v[hh];
    int32_t node = tid;
    if (!a.top) node = tid < pn * c ? pk * c + (tid - pi * c) : (int32_t)a.orph_lo + (tid - pn * c);
    s_nid[tid] = node;
    return pn;
}

// Small frontiers (n <= kSmallN candidates): one workgroup selects for all G
// heads of group g (one wave each) from the scores staged in LDS (s_sig
// [G][kSmallN], s_nid node ids) and writes the kept list.  LDS scratch: s_hist
// [G][256] (u64), s_kw [kSmallK][16] (u64, word-major: a word's
// 16 head words are adjacent; heads >= G hold zero).
__device__ __forceinline__ void select_small_group(const ZhaLevelArgs& a, int g, int G, float top_p, int n,
                                                   const float* s_sig, const int32_t* s_nid, uint64_t* s_hist,
                                                   uint64_t* s_kw, int32_t* o_pk = nullptr,
                                                   uint32_t* o_pm = nullptr, int* o_pn = nullptr) {
    const int tid = lane_tid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t lrow = (size_t)g * a.cap;
    const int nk = (n + 63) >> 6;
    if (wave < G) {
        uint32_t nc_h, nk_h;
        const float* sg = s_sig + wave * kSmallN;
        uint64_t* hh_ = s_hist + wave * 256;
        uint64_t* kk_ = s_kw + wave;
        if (nk <= 1) select_head_wave<1>(sg, n, top_p, hh_, kk_, &nc_h, &nk_h);
        else if (nk <= 2) select_head_wave<2>(sg, n, top_p, hh_, kk_, &nc_h, &nk_h);
        else if (nk <= 4) select_head_wave<4>(sg, n, top_p, hh_, kk_, &nc_h, &nk_h);
        else if (nk <= 8) select_head_wave<8>(sg, n, top_p, hh_, kk_, &nc_h, &nk_h);
        else select_head_wave<16>(sg, n, top_p, hh_, kk_, &nc_h, &nk_h);
        if (lane == 0) {
            a.stats[2 * (g * G + wave) + 0] = (int32_t)nc_h;
            a.stats[2 * (g * G + wave) + 1] = (int32_t)nk_h;
        }
        if (lane < nk) a.kbm[((size_t)g * G + wave) * a.wcap + lane] = kk_[16 * lane];
    } else if (wave < ZHA_MAX_GROUP && lane < nk) {
        s_kw[16 * lane + wave] = 0ull;
    }
    __syncthreads();
    // union of the heads' kept words -> kept list (ascending node) and head masks:
    // wave w < nk handles word w; its rank offset is the popcount of the words below
    // (with o_pk, the kept list, its masks and its length also go to LDS)
    if (nk == 0) {
        if (tid == 0) {
            a.nkept[g] = 0;
            if (o_pn) *o_pn = 0;
        }
    } else if (wave < nk) {
        // word `wave` of the 16 heads (128 contiguous bytes, read by every lane at
        // once) and, for the lanes below `wave`, word `lane`: all reads in flight
        const uint4* wq = reinterpret_cast<const uint4*>(s_kw + 16 * wave);
        const uint4* lq = reinterpret_cast<const uint4*>(s_kw + 16 * (lane < wave ? lane : 0));
        uint4 hq[ZHA_MAX_GROUP / 2], lw[ZHA_MAX_GROUP / 2];
#pragma unroll
        for (int t = 0; t < ZHA_MAX_GROUP / 2; ++t) {
            hq[t] = wq[t];
            lw[t] = lq[t];
        }
        uint32_t ulo = 0, uhi = 0, llo = 0, lhi = 0;
#pragma unroll
        for (int t = 0; t < ZHA_MAX_GROUP / 2; ++t) {
            ulo |= hq[t].x | hq[t].z;
            uhi |= hq[t].y | hq[t].w;
            llo |= lw[t].x | lw[t].z;
            lhi |= lw[t].y | lw[t].w;
        }
        const uint64_t u = ((uint64_t)uhi << 32) | ulo;
        uint32_t below = lane < wave ? (uint32_t)(__popc(llo) + __popc(lhi)) : 0u;
        for (int o = 32; o > 0; o >>= 1) below += __shfl_xor(below, o, 64);
        if (lane_bit(u, lane)) {
            const uint32_t rank = below + bits_below_lane(u);
            // lane's bit of each head word: low dword for lanes < 32, high dword above
            const int sh = lane & 31;
            const bool hi = lane >= 32;
            uint32_t msk = 0;
#pragma unroll
            for (int t = 0; t < ZHA_MAX_GROUP / 2; ++t) {
                const uint32_t w0 = hi ? hq[t].y : hq[t].x;
                const uint32_t w1 = hi ? hq[t].w : hq[t].z;
                msk |= ((w0 >> sh) & 1u) << (2 * t);
                msk |= ((w1 >> sh) & 1u) << (2 * t + 1);
            }
            const int32_t node = s_nid[lane + 64 * wave];
            a.klist[lrow + rank] = node;
            a.kmask[lrow + rank] = msk;
            if (o_pk) {
                o_pk[rank] = node;
                o_pm[rank] = msk;
            }
        }
        if (wave == nk - 1 && lane == 0) {
            const uint32_t tot = below + (uint32_t)__popcll(u);
            a.nkept[g] = (int32_t)tot;
            if (o_pn) *o_pn = (int)tot;
        }
    }
}

// grid (H_kv), 1024 threads: levels with at most kSmallN node slots.  The
// group's workgroup stages every head's scores with one round trip and selects.
__global__ __launch_bounds__(kSelThreads) void zha_select_small_kernel(ZhaLevelArgs a, int G, int c,
                                                                       float top_p) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p));
    __shared__ __align__(16) float s_sig[ZHA_MAX_GROUP * kSmallN];
    __shared__ __align__(16) uint64_t s_hist[ZHA_MAX_GROUP * 256];
    __shared__ int32_t s_nid[kSmallN];
    __shared__ __align__(16) uint64_t s_kw[ZHA_MAX_GROUP * kSmallK];

    const int g = blockIdx.x;
    const int n_orph = a.top ? 0 : (int)(a.orph_hi - a.orph_lo);
    const int pn = stage_small(a, g, G, c, threadIdx.x, s_sig, s_nid);
    const int n = a.top ? (int)a.n_top : pn * c + n_orph;
    __syncthreads();
    select_small_group(a, g, G, top_p, n, s_sig, s_nid, s_hist, s_kw);
}

// grid (H_kv), 1024 threads: the first routed levels, all small, selected one
// after the other by one workgroup per group with the kept lists in LDS.  Every
// node of these levels was scored beforehand (positions = node ids); each level
// gathers its candidates' scores, writes them back in candidate order, and
// selects.
__global__ __launch_bounds__(kSelThreads) void zha_select_chain_kernel(ZhaChainArgs m, int G, int c, float top_p) {
    __shared__ __align__(16) float s_sig[ZHA_MAX_GROUP * kSmallN];
    __shared__ __align__(16) uint64_t s_hist[ZHA_MAX_GROUP * 256];
    __shared__ int32_t s_nid[kSmallN];
    __shared__ __align__(16) uint64_t s_kw[ZHA_MAX_GROUP * kSmallK];
    __shared__ int32_t s_pk[kSmallN];
    __shared__ uint32_t s_pm[kSmallN];
    __shared__ int s_pn;

    const int g = blockIdx.x;
    const uint32_t allg = all_heads(G);
#pragma unroll 1
    for (int li = 0; li < m.n; ++li) {
        const ZhaLevelArgs& a = m.lv[li];
        const int p = lane_tid();                      // candidate position (n <= kSmallN)
        const int pn = li == 0 ? 0 : s_pn;
        const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
        int32_t node = 0;
        uint32_t msk = 0;
        if (p < n) {
            if (a.top) {
                node = p;
                msk = allg;
            } else if (p < pn * c) {
                const int pi = (int)zha_div((uint32_t)p, a.dc);
                node = s_pk[pi] * c + (p - pi * c);
                msk = s_pm[pi];
            } else {
                node = (int32_t)a.orph_lo + (p - pn * c);
                msk = allg;
            }
        }
        float v[ZHA_MAX_GROUP];
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) {
            v[hh] = zha_neg_inf();
            if (hh < G && p < n && ((msk >> hh) & 1u)) v[hh] = a.sig[((size_t)g * G + hh) * a.cap + node];
        }
        __syncthreads();                               // every gather done before the write-back below
        // all gathered values in registers at once (otherwise the compiler waits for
        // each write-back store before the next LDS write)
        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
                     "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh)
            if (hh < G) s_sig[hh * kSmallN + p] = v[hh];
        s_nid[p] = node;
        float* sgw = a.sig + (size_t)g * G * a.cap + p;
        if (p < n) {
#pragma unroll
            for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh)
                if (hh < G) sgw[(size_t)hh * a.cap] = v[hh];
        }
        if (p == 0) a.ncand[g] = n;
        __syncthreads();
        select_small_group(a, g, G, top_p, n, s_sig, s_nid, s_hist, s_kw, s_pk, s_pm, &s_pn);
        __syncthreads();
    }
}

// grid (H_q), 1024 threads: levels with more than kSmallN node slots, one query
// head per workgroup.  Up to kLdsKeys candidates the keys stay in LDS (position
// tid + 1024 k in slot k); larger frontiers recompute them from the scores on
// every pass.  Each head writes its kept bitmap; the kept list is formed later.
// A frontier of at most kSmallN candidates is instead selected for every head,
// and its kept list written, by the group's first workgroup (the small path).
__global__ __launch_bounds__(kSelThreads) void zha_select_large_kernel(ZhaLevelArgs a, int G, int c,
                                                                       float top_p, int small_only) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p), "s"(small_only));
    // keys: the keys (for the ordered tie pass); merge: head words [kMergeW][16]
    // (u64), then the step's parent node ids
    __shared__ __align__(16) uint32_t keys[kLdsKeys];
    __shared__ __align__(16) uint64_t hist[kHistPadded];   // merge: union words, then popcount prefixes
    __shared__ uint32_t cntb[kHistBins];
    __shared__ uint64_t s_wt[kSelWaves];
    __shared__ float swf[kSelWaves];
    __shared__ int s_bin;
    __shared__ uint64_t s_before, s_need, s_run;
    __shared__ uint32_t s_cnt[2];
    // the keys of the previous pass's crossing bin {key, position, mass lo, mass hi}
    // while there are at most kRankMax, their partial ranks, their count, the cut
    __shared__ __align__(16) uint4 s_ent[kRankMax];
    __shared__ uint64_t s_rank[kRankMax];
    __shared__ uint32_t s_nent, s_cut[2];

    const int h = blockIdx.x, g = h / G, hl = h - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (small_only) {
        // a sliced level: only a frontier of at most kSmallN candidates is selected
        // here (by the group's first workgroup); the slice kernels take larger ones
        const int pn0 = a.top ? 0 : a.pnkept[g];
        const int n0 = a.top ? (int)a.n_top : pn0 * c + (int)(a.orph_hi - a.orph_lo);
        if (n0 > kSmallN || hl != 0) return;
        float* s_sig = reinterpret_cast<float*>(keys);                                   // [G][kSmallN]
        uint64_t* s_hist = reinterpret_cast<uint64_t*>(keys + ZHA_MAX_GROUP * kSmallN);  // [G][256]
        int32_t* s_nid = reinterpret_cast<int32_t*>(keys + ZHA_MAX_GROUP * kSmallN + 2 * ZHA_MAX_GROUP * 256);
        stage_small(a, g, G, c, tid, s_sig, s_nid);
        __syncthreads();
        select_small_group(a, g, G, top_p, n0, s_sig, s_nid, s_hist, hist);
        return;
    }
    const int n_orph = a.top ? 0 : (int)(a.orph_hi - a.orph_lo);
    const float* sg = a.sig + ((size_t)g * G + hl) * a.cap;

    // The count and the scores of the first half of the LDS positions are read
    // together (one round trip, bounded by the capacity); the second half's reads,
    // bounded by the count, follow as soon as it arrives.  Positions >= n are
    // ignored afterwards.
    // (slots that lie wholly past the bound are skipped by a uniform branch: no
    // per-lane work for them)
    uint32_t kr[kSlots];
    const int lim = (int)min(a.cap, (int64_t)kLdsKeys);
#pragma unroll
    for (int k = 0; k < kSlots / 2; ++k) {
        kr[k] = __float_as_uint(zha_neg_inf());
        if (k * kSelThreads < lim) {
            const int pos = tid + k * kSelThreads;
            if (pos < lim) kr[k] = __float_as_uint(sg[pos]);
        }
    }
    const int pn = parent_count(a, g);
    const int n = a.top ? (int)a.n_top : pn * c + n_orph;
    {
        const int lim2 = min(lim, n);
#pragma unroll
        for (int k = kSlots / 2; k < kSlots; ++k) {
            kr[k] = __float_as_uint(zha_neg_inf());
            if (k * kSelThreads < lim2) {
                const int pos = tid + k * kSelThreads;
                if (pos < lim2) kr[k] = __float_as_uint(sg[pos]);
            }
        }
    }
    if (n <= kSmallN) {
        // a small frontier at a large level: the group's first workgroup selects for
        // all heads, with the key buffer as its LDS
        if (hl != 0) return;
        float* s_sig = reinterpret_cast<float*>(keys);                                   // [G][kSmallN]
        uint64_t* s_hist = reinterpret_cast<uint64_t*>(keys + ZHA_MAX_GROUP * kSmallN);  // [G][256]
        int32_t* s_nid = reinterpret_cast<int32_t*>(keys + ZHA_MAX_GROUP * kSmallN + 2 * ZHA_MAX_GROUP * 256);
        uint64_t* s_kw = hist;                                                           // [kSmallK][16]
        stage_small(a, g, G, c, tid, s_sig, s_nid);
        __syncthreads();
        select_small_group(a, g, G, top_p, n, s_sig, s_nid, s_hist, s_kw);
        return;
    }
    const int nwords = (n + 63) >> 6;
    const int nslot = (n + kSelThreads - 1) / kSelThreads;   // positions per thread
    const bool staged = n <= kLdsKeys;

    if (tid < 2) s_cnt[tid] = 0;
    float m = zha_neg_inf();
    if (staged) {
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            if (k < nslot) {
                if (tid + k * kSelThreads >= n) kr[k] = __float_as_uint(zha_neg_inf());
                m = fmaxf(m, __uint_as_float(kr[k]));
            }
        }
    } else {
        // frontiers beyond the LDS keys: the scores are re-read (from L2) kGlobBatch
        // positions per thread at a time, all reads of a batch in flight together
#pragma unroll 1
        for (int k0 = 0; k0 < nslot; k0 += kGlobBatch) {
            float xs[kGlobBatch];
#pragma unroll
            for (int j = 0; j < kGlobBatch; ++j) {
                const int pos = tid + (k0 + j) * kSelThreads;
                xs[j] = pos < n ? sg[pos] : zha_neg_inf();
            }
#pragma unroll
            for (int j = 0; j < kGlobBatch; ++j) m = fmaxf(m, xs[j]);
        }
    }
    // the first pass's histogram, cleared before the barrier below
    for (int i = tid; i < kHistPadded; i += kSelThreads) hist[i] = 0;
    for (int i = tid; i < kHistBins; i += kSelThreads) cntb[i] = 0;
    m = zha_wave_max(m);
    if (lane == 0) swf[wave] = m;
    __syncthreads();
    m = swf[0];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, swf[w]);

    // Kept rule: keep_all, or key < ustar, or key == ustar when that key is unique
    // (a ranked cut: key == ustar at a position <= plim).
    const bool none = m == zha_neg_inf();        // this head has no candidate at this level
    const bool keep_all = !none && top_p >= 1.0f;
    const bool cut = !none && !keep_all;
    if (staged) {
        // keys to LDS and, when there is a cut to find, the first digit pass in the
        // same loop: every key's mass into its top-digit bin, a key without mass
        // adding zero to its lane's unused padding entry (33 lane + 32, never read)
        const int dummy = 33 * lane + 32;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            if (k < nslot) {
                const uint32_t key = key_of(__uint_as_float(kr[k]), m);
                keys[tid + k * kSelThreads] = key;
                if (cut) {
                    const bool has = key < kNoMass;
                    const int at = has ? hpad((key >> 21) & 2047u) : dummy;
                    const uint64_t ms = has ? mass_of(key) : 0ull;
                    atomicAdd((unsigned long long*)&hist[at], (unsigned long long)ms);
                }
            }
        }
    }
    uint32_t ustar = 0, ties = 0, plim = 0xFFFFFFFFu;
    uint64_t need = 0;
    if (cut) {
        uint32_t mshift = 31, mval = 0, bshift = 21, bmask = 2047;
        bool rec = false;                        // this pass records the previous crossing bin's keys
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            // pass 0 adds the mass of every key that carries mass; later passes count
            // and add only the keys whose higher digits equal the bins found so far
            const bool all = pass == 0;
            if (staged) {
                // pass 0 went with the staging; later passes read the keys from LDS
                // kBatch slots at a time (all reads in flight together), test a batch
                // first and touch the histogram only for the few keys that match
#pragma unroll 1
                for (int k0 = 0; k0 < (all ? 0 : nslot); k0 += kBatch) {
                    uint32_t kk[kBatch];
#pragma unroll
                    for (int j = 0; j < kBatch; ++j) kk[j] = keys[tid + ((k0 + j) & (kSlots - 1)) * kSelThreads];
                    {
                        uint32_t hit = 0;
#pragma unroll
                        for (int j = 0; j < kBatch; ++j) {
                            const uint32_t key = kk[j];
                            const bool mt = k0 + j < nslot && key < kNoMass && (key >> mshift) == mval;
                            hit |= (uint32_t)mt << j;
                        }
                        if (hit) {
#pragma unroll
                            for (int j = 0; j < kBatch; ++j) {
                                if ((hit >> j) & 1u) {
                                    const uint32_t key = kk[j];
                                    const uint32_t b = (key >> bshift) & bmask;
                                    const uint64_t ms = mass_of(key);
                                    atomicAdd((unsigned long long*)&hist[hpad(b)], (unsigned long long)ms);
                                    atomicAdd(&cntb[b], 1u);
                                    if (rec) {
                                        const uint32_t e = atomicAdd(&s_nent, 1u);
                                        if (e < kRankMax)
                                            s_ent[e] = make_uint4(key, (uint32_t)(tid + (k0 + j) * kSelThreads),
                                                                  (uint32_t)ms, (uint32_t)(ms >> 32));
                                    }
                                }
                            }
                        }
                    }
                }
            } else {
#pragma unroll 1
                for (int k0 = 0; k0 < nslot; k0 += kGlobBatch) {
                    float xs[kGlobBatch];
#pragma unroll
                    for (int j = 0; j < kGlobBatch; ++j) {
                        const int pos = tid + (k0 + j) * kSelThreads;
                        xs[j] = pos < n ? sg[pos] : zha_neg_inf();
                    }
#pragma unroll
                    for (int j = 0; j < kGlobBatch; ++j) {
                        const uint32_t key = key_of(xs[j], m);
                        if (key < kNoMass && (all || (key >> mshift) == mval)) {
                            const uint32_t b = (key >> bshift) & bmask;
                            const uint64_t ms = mass_of(key);
                            atomicAdd((unsigned long long*)&hist[hpad(b)], (unsigned long long)ms);
                            if (!all) {
                                atomicAdd(&cntb[b], 1u);
                                if (rec) {
                                    const uint32_t e = atomicAdd(&s_nent, 1u);
                                    if (e < kRankMax)
                                        s_ent[e] = make_uint4(key, (uint32_t)(tid + (k0 + j) * kSelThreads),
                                                              (uint32_t)ms, (uint32_t)(ms >> 32));
                                }
                            }
                        }
                    }
                }
            }
            __syncthreads();
            const int nent = rec ? (int)s_nent : 0;
            if (nent > 0 && nent <= kRankMax) {
                // the previous crossing bin holds few keys: rank them directly.  Entry j's
                // mass before it is summed in C chunks of the entries (one chunk per
                // thread, a wave's threads sharing theirs: broadcast reads), then the entry
                // whose own mass reaches what the bin must supply is the cut.
                const int np = (nent + 63) & ~63;
                const int C = kSelThreads / np;
                const int j = tid % np, ck = tid / np;
                const int chunk = (nent + C - 1) / C;
                if (j < nent && ck < C) {
                    const uint4 e = s_ent[j];
                    const int i0 = ck * chunk, i1 = min(nent, i0 + chunk);
                    uint64_t acc = 0;
#pragma unroll 4
                    for (int i = i0; i < i1; ++i) {
                        const uint4 f = s_ent[i];
                        acc += rank_precedes(f, e) ? entry_mass(f) : 0ull;
                    }
                    if (i1 > i0) atomicAdd((unsigned long long*)&s_rank[j], (unsigned long long)acc);
                }
                __syncthreads();
                if (tid < nent) {
                    const uint4 e = s_ent[tid];
                    const uint64_t before = s_rank[tid];
                    if (before < need && before + entry_mass(e) >= need) {
                        s_cut[0] = e.x;
                        s_cut[1] = e.y;
                    }
                }
                __syncthreads();
                ustar = s_cut[0];
                plim = s_cut[1];
                ties = 1;
                break;
            }
            if (wave == 0) wave_find_cross(hist, need, top_p, &s_bin, &s_before, &s_need);
            __syncthreads();
            const uint32_t bin = (uint32_t)s_bin;
            need = s_need - s_before;            // mass still needed inside this bin
            // pass 0 counts no keys (its bins hold many at these sizes): it never ends
            // the search
            const uint32_t cnt = pass == 0 ? 0u : cntb[bin];
            const uint32_t pref = pass == 0 ? bin : (mval << (pass == 1 ? 11 : 10)) | bin;
            if (cnt == 1 || pass == 2) {
                // the crossing bin holds one key (or the keys equal to the cut): the cut
                // is the largest key with this prefix
                ustar = (pref << bshift) | ((1u << bshift) - 1u);
                ties = cnt;
                break;
            }
            {
                // every key of the crossing bin has at least the mass of its largest key,
                // so the bin's mass over that bounds how many keys the next pass meets
                const uint64_t mmin = mass_of((pref << bshift) | ((1u << bshift) - 1u));
                rec = mmin > 0 && hist[hpad(bin)] <= (uint64_t)kRankMax * mmin;
            }
            if (pass == 0) { mshift = 21; mval = pref; bshift = 10; bmask = 2047; }
            else { mshift = 10; mval = pref; bshift = 0; bmask = 1023; }
            __syncthreads();                     // every thread has read this pass's result
            for (int i = tid; i < kHistPadded; i += kSelThreads) hist[i] = 0;
            for (int i = tid; i < kHistBins; i += kSelThreads) cntb[i] = 0;
            for (int i = tid; i < kRankMax; i += kSelThreads) s_rank[i] = 0;
            if (tid == 0) {
                s_nent = 0;
                s_cut[0] = 0;
                s_cut[1] = 0;
            }
            __syncthreads();
        }
    }
    const uint64_t need_tie = need;

    // kept flags -> this head's bitmap: slot k of wave w is word 16 k + w
    uint64_t* bm = a.kbm + ((size_t)g * G + hl) * a.wcap;
    uint32_t my_cand = 0, my_kept = 0;
    if (staged) {
#pragma unroll 1
        for (int k = 0; k < nslot; ++k) {
            {
                const uint32_t key = keys[tid + k * kSelThreads];
                const bool cand = key != kNotCand;
                const bool kept = !none && (keep_all ? cand
                                                     : (key < kNoMass &&
                                                        (key < ustar || (key == ustar && ties == 1 &&
                                                                         (uint32_t)(tid + k * kSelThreads) <= plim))));
                const uint64_t word = __ballot(kept);
                const int wi = k * kSelWaves + wave;
                if (lane == 0 && wi < nwords) bm[wi] = word;
                my_cand += cand;
                my_kept += kept;
            }
        }
    } else {
#pragma unroll 1
        for (int k0 = 0; k0 < nslot; k0 += kGlobBatch) {
            float xs[kGlobBatch];
#pragma unroll
            for (int j = 0; j < kGlobBatch; ++j) {
                const int pos = tid + (k0 + j) * kSelThreads;
                xs[j] = pos < n ? sg[pos] : zha_neg_inf();
            }
#pragma unroll
            for (int j = 0; j < kGlobBatch; ++j) {
                const int k = k0 + j;
                if (k < nslot) {
                    const uint32_t key = key_of(xs[j], m);
                    const bool cand = key != kNotCand;
                    const bool kept = !none && (keep_all ? cand
                                                         : (key < kNoMass &&
                                                            (key < ustar || (key == ustar && ties == 1 &&
                                                                             (uint32_t)(tid + k * kSelThreads) <= plim))));
                    const uint64_t word = __ballot(kept);
                    const int wi = k * kSelWaves + wave;
                    if (lane == 0 && wi < nwords) bm[wi] = word;
                    my_cand += cand;
                    my_kept += kept;
                }
            }
        }
    }
    if (!none && !keep_all && ties > 1) {
        // several candidates share the cut key: take them in ascending position order
        __syncthreads();
        __threadfence();
        if (tid == 0) s_run = 0;
#pragma unroll 1
        for (int base = 0; base < n; base += kSelThreads) {
            const int pos = base + tid;
            const uint32_t key = pos < n ? (staged ? keys[pos] : key_of(sg[pos], m)) : kNotCand;
            const uint64_t w = key == ustar ? mass_of(key) : 0ull;
            uint64_t wt;
            const uint64_t ex = wave_excl_scan_u64(w, &wt);
            __syncthreads();
            if (lane == 0) s_wt[wave] = wt;
            __syncthreads();
            uint64_t before = s_run;
            for (int ww = 0; ww < wave; ++ww) before += s_wt[ww];
            uint64_t tot = 0;
            for (int ww = 0; ww < kSelWaves; ++ww) tot += s_wt[ww];
            if (w > 0 && before + ex < need_tie) {
                atomicOr((unsigned long long*)&bm[pos >> 6], 1ull << (pos & 63));
                ++my_kept;
            }
            __syncthreads();
            if (tid == 0) s_run = s_run + tot;
            __syncthreads();
            if (s_run >= need_tie) break;
        }
    }
    {
        const uint64_t both = zha_readlane_u64(zha_wave_incl_scan_u64(((uint64_t)my_kept << 32) | my_cand), 63);
        if (lane == 0) {
            atomicAdd(&s_cnt[0], (uint32_t)both);
            atomicAdd(&s_cnt[1], (uint32_t)(both >> 32));
        }
    }

    __syncthreads();
    if (tid == 0) {
        a.stats[2 * h + 0] = (int32_t)s_cnt[0];
        a.stats[2 * h + 1] = (int32_t)s_cnt[1];
    }
}

// grid (blocks, H_kv), 1024 threads: the kept list of a level whose heads were
// selected by zha_select_large_kernel.  Block b owns bitmap words [b share,
// (b + 1) share) of its group (share <= kMergeW, a multiple of 16): it ORs the G
// heads' words, writes the kept list entries of its positions (ascending
// position = ascending node) with the mask of heads that kept each node, and
// offsets their ranks by the kept nodes in the words before its share.  The
// count, the share's words, its parents' node ids and the words before it are
// all read before the count is known (bounded by the capacities), so they cost
// one memory round trip together.
__global__ __launch_bounds__(kSelThreads) void zha_route_merge_kernel(ZhaLevelArgs a, int G, int c, int share) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(share));
    // [word][16 heads (+1 padding)], heads >= G zero: a row of 17 words, so that the
    // threads of a wave (consecutive rows) reach distinct LDS banks
    constexpr int kRow = ZHA_MAX_GROUP + 1;
    __shared__ __align__(16) uint64_t hw[kMergeW * kRow];
    __shared__ int32_t s_par[kMergeW * 32];                            // parents' node ids
    __shared__ uint64_t s_union[kMergeW];
    __shared__ uint32_t s_wpre[kMergeW];
    __shared__ uint32_t s_part[kSelWaves];
    __shared__ uint32_t s_tot;
    const int g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wcap = (int)a.wcap;
    const int w0 = blockIdx.x * share;
    const int wend_s = min(w0 + share, wcap);                 // words this block may own
    const uint64_t* gbm = a.kbm + (size_t)g * G * a.wcap;
    const int32_t* par = a.top ? nullptr : a.pklist + (size_t)g * a.pcap;
    const int p0 = w0 * 64;
    const int pb0 = (int)zha_div((uint32_t)p0, a.dc);
    const int pb_s = a.top ? pb0 : min((int)a.pcap, (int)zha_div((uint32_t)(wend_s * 64 + c - 1), a.dc));
    const int npar_s = max(0, pb_s - pb0);

    constexpr int kPerW = ZHA_MAX_GROUP * kMergeW / kSelThreads;
    constexpr int kPerP = kMergeW * 32 / kSelThreads;
    uint64_t hv[kPerW];
    int32_t pv[kPerP];
    uint64_t pw[ZHA_MAX_GROUP];
    // (slots whose heads or parents all lie past their bound are skipped by a
    // uniform branch)
    constexpr int kHeadsPerSlot = kSelThreads / kMergeW;
#pragma unroll
    for (int t = 0; t < kPerW; ++t) {
        hv[t] = 0ull;
        if (t * kHeadsPerSlot < G) {
            const uint32_t i = (uint32_t)(tid + t * kSelThreads);
            const uint32_t hh = i / kMergeW, wi = i % kMergeW;
            if (hh < (uint32_t)G && w0 + (int)wi < wend_s) hv[t] = gbm[(size_t)hh * a.wcap + w0 + wi];
        }
    }
#pragma unroll
    for (int t = 0; t < kPerP; ++t) {
        pv[t] = 0;
        if (t * kSelThreads < npar_s) {
            const int i = tid + t * kSelThreads;
            if (i < npar_s) pv[t] = par[pb0 + i];
        }
    }
    const bool chunked = a.chunk_cnt != nullptr;   // sliced level: kept counts per 512-word chunk
    const int nch = (wcap + kMergeW - 1) / kMergeW;
    // (one straight-line block of reads: a branch here makes the compiler wait for
    // every read before the two paths join; a sliced level reads its chunk counts
    // after the early return)
#pragma unroll
    for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) {
        pw[hh] = 0ull;
        if (!chunked && hh < G && tid < w0) pw[hh] = gbm[(size_t)hh * a.wcap + tid];
    }
    const int pn = parent_count(a, g);

    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kSmallN) return;                    // selected and merged by the select kernel
    const int nwords = (n + 63) >> 6;
    if (w0 >= nwords) {
        if (blockIdx.x == 0 && nwords == 0 && tid == 0) a.nkept[g] = 0;
        return;
    }
    const int w1 = min(wend_s, nwords);
    const int nw = w1 - w0;
    const int pnc = pn * c;

    // rank offset: kept nodes in words [0, w0)
    uint32_t cnt = 0;
    if (chunked) {
#pragma unroll 1
        for (int i = tid; i < w0 / kMergeW; i += kSelThreads) cnt += a.chunk_cnt[(size_t)g * nch + i];
    } else {
        uint64_t u = 0;
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) u |= pw[hh];
        cnt = (uint32_t)__popcll(u);
#pragma unroll 1
        for (int w = tid + kSelThreads; w < w0; w += kSelThreads) {
            uint64_t v = 0;
            for (int hh = 0; hh < G; ++hh) v |= gbm[(size_t)hh * a.wcap + w];
            cnt += (uint32_t)__popcll(v);
        }
    }
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if (lane == 0) s_part[wave] = cnt;
#pragma unroll
    for (int t = 0; t < kPerW; ++t) {
        const uint32_t i = (uint32_t)(tid + t * kSelThreads);
        hw[(i % kMergeW) * kRow + i / kMergeW] = (int)(i % kMergeW) < nw ? hv[t] : 0ull;
    }
#pragma unroll
    for (int t = 0; t < kPerP; ++t) {
        const int i = tid + t * kSelThreads;
        if (i < npar_s) s_par[i] = pv[t];
    }
    __syncthreads();
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) run += s_part[w];
    if (tid < nw) {
        uint64_t u = 0;
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) u |= hw[tid * kRow + hh];
        s_union[tid] = u;
    }
    __syncthreads();
    if (wave == 0) {
        // exclusive popcount prefix of the union words (kMergeW / 64 words per lane)
        constexpr int per = kMergeW / 64;
        uint32_t c2 = 0;
#pragma unroll
        for (int q = 0; q < per; ++q) {
            const int wi = lane * per + q;
            c2 += wi < nw ? (uint32_t)__popcll(s_union[wi]) : 0u;
        }
        uint64_t tot;
        uint32_t pre = (uint32_t)wave_excl_scan_u64(c2, &tot);
#pragma unroll
        for (int q = 0; q < per; ++q) {
            const int wi = lane * per + q;
            s_wpre[wi] = pre;
            pre += wi < nw ? (uint32_t)__popcll(s_union[wi]) : 0u;
        }
        if (lane == 0) s_tot = (uint32_t)tot;
    }
    __syncthreads();
    int32_t* kl = a.klist + (size_t)g * a.cap;
    uint32_t* km = a.kmask + (size_t)g * a.cap;
    // word wi = 16 k + wave, bit = lane
#pragma unroll 1
    for (int wi = wave; wi < nw; wi += kSelWaves) {
        const uint64_t u = s_union[wi];
        const uint32_t pre = s_wpre[wi];
        uint64_t hr[ZHA_MAX_GROUP];                   // the row's head words (one address per read)
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) hr[hh] = hw[wi * kRow + hh];
        const int pos = p0 + wi * 64 + lane;
        const bool child = par && pos < pnc;
        const int pi = (int)zha_div((uint32_t)pos, a.dc);
        const int32_t pnode = child ? s_par[pi - pb0] : 0;
        if (!lane_bit(u, lane)) continue;
        // lane's bit of each head word
        uint32_t msk = 0;
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) msk |= (uint32_t)((hr[hh] >> lane) & 1ull) << hh;
        const uint32_t rank = run + pre + bits_below_lane(u);
        int32_t node;
        if (!par) node = pos;
        else if (child) node = pnode * c + (pos - pi * c);
        else node = (int32_t)a.orph_lo + (pos - pnc);
        kl[rank] = node;
        km[rank] = msk;
    }
    if (w1 == nwords && tid == 0) a.nkept[g] = (int32_t)(run + s_tot);
}


// ---- levels with more than kLdsKeys node slots: the candidates of each head are
// cut into slices of ZHA_SLICE positions, one 256-thread workgroup per (slice,
// head), so a pass over the keys uses the whole GPU.  Digit histograms are summed
// per head in global memory with integer atomics (exact and order-free); each
// pass kernel first replays the crossings of the passes before it from those
// histograms, so every workgroup reaches the same cut.

constexpr int kHugeThreads = 1024;
constexpr int kHugeWaves = kHugeThreads / 64;
constexpr int kHugePer = ZHA_SLICE / kHugeThreads;   // positions per thread
static_assert(ZHA_SLICE % 64 == 0 && kHugePer * kHugeThreads == ZHA_SLICE, "slice layout");
static_assert(ZHA_SLICE % (kHugeWaves * 64) == 0, "a slice holds whole words of every wave");
static_assert(kHugeWaves * 64 == kHugeThreads, "slot k of wave w is bitmap word (p0 >> 6) + w + kHugeWaves k");

// grid (H_q), kHugeThreads (1024) threads: clears the level's histograms and counts.
__global__ __launch_bounds__(kHugeThreads) void zha_huge_init_kernel(ZhaLevelArgs a, int Hq) {
    ZHA_LEVEL_ARGS_READY(a, "s"(Hq));
    const int h = blockIdx.x;
    for (int i = threadIdx.x; i < 3 * kHistBins; i += kHugeThreads) {
        const int pass = i / kHistBins, b = i - pass * kHistBins;
        a.hmass[((size_t)pass * Hq + h) * kHistBins + b] = 0ull;
        a.hcnt[((size_t)pass * Hq + h) * kHistBins + b] = 0u;
    }
    if (threadIdx.x < 3) a.hdone[threadIdx.x * Hq + h] = 0u;
    if (threadIdx.x == 0) {
        a.stats[2 * h + 0] = 0;
        a.stats[2 * h + 1] = 0;
    }
}

// The candidate count of the level and the head's largest score (from the score
// kernel's per-block maxima); called by the whole workgroup.
struct SliceView {
    int n, p0;
    float m;
};
// Candidates of head h at this level (a uniform scalar read: idle slices leave on it).
__device__ __forceinline__ int head_n(const ZhaLevelArgs& a, int G, int c, int h) {
    const int pn = a.top ? 0 : a.pnkept[h / G];
    return a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
}
__device__ __forceinline__ SliceView slice_view(const ZhaLevelArgs& a, int G, int c, int h, int s, float* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = h / G;
    SliceView v;
    v.p0 = s * ZHA_SLICE;
    const int pn = a.top ? 0 : a.pnkept[g];
    float x = tid < a.score_blocks ? a.hblk[(size_t)h * ZHA_SCORE_MAXB + tid] : zha_neg_inf();
    x = zha_wave_max(x);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    v.m = red[0];
#pragma unroll
    for (int w = 1; w < kHugeWaves; ++w) v.m = fmaxf(v.m, red[w]);
    v.n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    __syncthreads();
    return v;
}

// The slice's keys in registers: position p0 + tid + kHugeThreads k (= 1024 k) in slot k,
// so wave w's lanes of slot k cover bitmap word (p0 >> 6) + w + kHugeWaves k.
__device__ __forceinline__ void slice_keys(const ZhaLevelArgs& a, int h, const SliceView& v,
                                           uint32_t (&key)[kHugePer]) {
    const int tid = threadIdx.x;
    const float* sg = a.sig + (size_t)h * a.cap;
    const int lim = min(v.n, v.p0 + ZHA_SLICE);
    float x[kHugePer];
#pragma unroll
    for (int k = 0; k < kHugePer; ++k) {
        const int pos = v.p0 + tid + k * kHugeThreads;
        x[k] = pos < lim ? sg[pos] : zha_neg_inf();
    }
#pragma unroll
    for (int k = 0; k < kHugePer; ++k) {
        const int pos = v.p0 + tid + k * kHugeThreads;
        key[k] = pos < v.n ? key_of(x[k], v.m) : kNotCand;
    }
}


// Run by the whole workgroup that finished pass PASS of head h last: read that
// pass's complete histogram, find the bin where the cumulative mass crosses, and
// record the head's cut state for the following kernels.
__device__ void advance_cut(const ZhaLevelArgs& a, int Hq, int h, int pass, float top_p, const HugeCut& prev,
                            uint64_t* lhist, uint32_t* lcnt, int* s_bin, uint64_t* s_before, uint64_t* s_need) {
    const int tid = threadIdx.x;
    const uint64_t* gm = a.hmass + ((size_t)pass * Hq + h) * kHistBins;
    const uint32_t* gc = a.hcnt + ((size_t)pass * Hq + h) * kHistBins;
    for (int b = tid; b < kHistBins; b += kHugeThreads) {
        // the other workgroups' sums, read past this device's caches
        lhist[hpad((uint32_t)b)] = __hip_atomic_load(gm + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lcnt[b] = __hip_atomic_load(gc + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid < 64) wave_find_cross(lhist, pass == 0 ? 0ull : prev.need, top_p, s_bin, s_before, s_need);
    __syncthreads();
    if (tid == 0) {
        const uint32_t bin = (uint32_t)*s_bin;
        const uint32_t cnt = lcnt[bin];
        const uint32_t pref = pass == 0 ? bin : (prev.mval << (pass == 1 ? 11 : 10)) | bin;
        const uint32_t bshift = pass == 0 ? 21u : pass == 1 ? 10u : 0u;
        HugeCut nx;
        nx.need = *s_need - *s_before;
        nx.pad = 0;
        if (cnt == 1 || pass == 2) {
            // the crossing bin holds one key (or the keys equal to the cut): the cut is
            // the largest key with this prefix
            nx.done = 1;
            nx.ustar = (pref << bshift) | ((1u << bshift) - 1u);
            nx.ties = cnt;
            nx.mshift = nx.mval = nx.bshift = nx.bmask = 0;
        } else {
            nx.done = 0;
            nx.ustar = nx.ties = 0;
            nx.mshift = pass == 0 ? 21u : 10u;
            nx.mval = pref;
            nx.bshift = pass == 0 ? 10u : 0u;
            nx.bmask = pass == 0 ? 2047u : 1023u;
        }
        a.hstate[h] = nx;
    }
}

// grid (slices, H_q): digit histogram of pass PASS over one slice, added into the
// head's global histogram; the last slice to finish records the head's cut state.
template <int PASS>
__global__ __launch_bounds__(kHugeThreads) void zha_huge_pass_kernel(ZhaLevelArgs a, int G, int c, float top_p, int Hq) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p), "s"(Hq));
    __shared__ __align__(16) uint64_t lhist[kHistPadded];
    __shared__ uint32_t lcnt[kHistBins];
    __shared__ int s_bin, s_last;
    __shared__ uint64_t s_before, s_need;
    __shared__ float red[kHugeWaves];
    const int h = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    HugeCut st;
    if (PASS > 0) {
        st = a.hstate[h];
        if (st.done) return;                   // an earlier pass already found the cut
    }
    const int nh = head_n(a, G, c, h);
    if (nh <= kSmallN || s * ZHA_SLICE >= nh) return;   // small frontiers: selected whole elsewhere
    const SliceView v = slice_view(a, G, c, h, s, red);
    if (v.p0 >= v.n || v.m == zha_neg_inf() || top_p >= 1.0f) return;
    const uint32_t mshift = PASS > 0 ? st.mshift : 31u, mval = PASS > 0 ? st.mval : 0u;
    const uint32_t bshift = PASS > 0 ? st.bshift : 21u, bmask = PASS > 0 ? st.bmask : 2047u;
    uint32_t key[kHugePer];
    slice_keys(a, h, v, key);
    for (int i = tid; i < kHistPadded; i += kHugeThreads) lhist[i] = 0ull;
    for (int i = tid; i < kHistBins; i += kHugeThreads) lcnt[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kHugePer; ++k) {
        const uint32_t kk = key[k];
        if (kk < kNoMass && (PASS == 0 || (kk >> mshift) == mval)) {
            const uint32_t b = (kk >> bshift) & bmask;
            atomicAdd((unsigned long long*)&lhist[hpad(b)], (unsigned long long)mass_of(kk));
            atomicAdd(&lcnt[b], 1u);
        }
    }
    __syncthreads();
    uint64_t* gm = a.hmass + ((size_t)PASS * Hq + h) * kHistBins;
    uint32_t* gc = a.hcnt + ((size_t)PASS * Hq + h) * kHistBins;
    for (int b = tid; b < kHistBins; b += kHugeThreads) {
        const uint32_t cnt = lcnt[b];
        if (cnt) {
            atomicAdd((unsigned long long*)&gm[b], (unsigned long long)lhist[hpad((uint32_t)b)]);
            atomicAdd(&gc[b], cnt);
        }
    }
    // the last of the head's active slices to get here resolves this pass: every
    // wave's histogram atomics complete, then one release fence and the counter
    zha_wave_mem_wait();
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int active = (v.n + ZHA_SLICE - 1) / ZHA_SLICE;
        s_last = atomicAdd(&a.hdone[PASS * Hq + h], 1u) == (uint32_t)(active - 1);
        if (s_last) __threadfence();
    }
    __syncthreads();
    if (!s_last) return;
    advance_cut(a, Hq, h, PASS, top_p, st, lhist, lcnt, &s_bin, &s_before, &s_need);
}

// Block-wide sums over kHugeThreads threads (all threads receive the result).
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t t;
    wave_excl_scan_u64(v, &t);
    __syncthreads();
    if (lane == 0) red[wave] = t;
    __syncthreads();
    uint64_t sum = 0;
#pragma unroll
    for (int w = 0; w < kHugeWaves; ++w) sum += red[w];
    return sum;
}

// grid (slices, H_q), kHugeThreads (1024) threads: kept flags of one slice into the head's bitmap
// (words of 64 positions, each written by one lane), candidate and kept counts,
// and the slice's mass of keys equal to the cut when the cut key is shared.
__global__ __launch_bounds__(kHugeThreads) void zha_huge_bitmap_kernel(ZhaLevelArgs a, int G, int c, float top_p,
                                                                      int Hq) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p), "s"(Hq));
    __shared__ uint64_t red[kHugeWaves];
    __shared__ float redf[kHugeWaves];
    const int h = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nh = head_n(a, G, c, h);
    if (nh <= kSmallN || s * ZHA_SLICE >= nh) return;   // small frontiers: selected whole elsewhere
    const HugeCut cut = a.hstate[h];
    const SliceView v = slice_view(a, G, c, h, s, redf);
    if (v.p0 >= v.n) return;
    uint32_t key[kHugePer];
    slice_keys(a, h, v, key);
    const bool none = v.m == zha_neg_inf();
    const bool keep_all = !none && top_p >= 1.0f;
    uint32_t ustar = 0, ties = 0;
    if (!none && !keep_all) {
        ustar = cut.ustar;
        ties = cut.ties;
    }
    uint64_t* bm = a.kbm + (size_t)h * a.wcap;
    const int nwords = (v.n + 63) >> 6;
    uint32_t my_cand = 0, my_kept = 0;
    uint64_t my_tie = 0;
#pragma unroll
    for (int k = 0; k < kHugePer; ++k) {
        const uint32_t kk = key[k];
        const bool cand = kk != kNotCand;
        const bool kept = !none && (keep_all ? cand : (kk < kNoMass && (kk < ustar || (kk == ustar && ties == 1))));
        const uint64_t word = __ballot(kept);
        const int wi = (v.p0 >> 6) + wave + kHugeWaves * k;
        if (lane == 0 && wi < nwords) bm[wi] = word;
        my_cand += cand;
        my_kept += kept;
        if (ties > 1 && kk == ustar) my_tie += mass_of(kk);
    }
    const uint64_t both = block_sum_u64(((uint64_t)my_kept << 32) | my_cand, red);
    if (tid == 0) {
        atomicAdd(&a.stats[2 * h + 0], (int32_t)(uint32_t)both);
        atomicAdd(&a.stats[2 * h + 1], (int32_t)(both >> 32));
    }
    if (ties > 1) {
        const uint64_t t = block_sum_u64(my_tie, red);
        if (tid == 0) a.tiem[(size_t)h * a.slices + s] = t;
    }
}

// grid (slices, H_q): when several keys equal the cut key, take them in ascending
// position order (slice by slice, then within the slice) until the mass still
// needed at the cut is reached.  A slice whose equal keys all come before that
// point takes them all, one that starts after it takes none; only the slice where
// it falls walks its positions in order.
__global__ __launch_bounds__(kHugeThreads) void zha_huge_ties_kernel(ZhaLevelArgs a, int G, int c, float top_p,
                                                                    int Hq) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p), "s"(Hq));
    __shared__ uint64_t red[kHugeWaves];
    __shared__ float redf[kHugeWaves];
    __shared__ uint64_t wsum[kHugeWaves][kHugePer];   // equal-key mass per (wave, slot)
    const int h = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const HugeCut st = a.hstate[h];
    if (st.ties <= 1u) return;                 // the cut key is unique
    const int nh = head_n(a, G, c, h);
    if (nh <= kSmallN || s * ZHA_SLICE >= nh) return;   // small frontiers: selected whole elsewhere
    const SliceView v = slice_view(a, G, c, h, s, redf);
    if (v.p0 >= v.n || v.m == zha_neg_inf() || top_p >= 1.0f) return;
    // equal-key mass of the slices before this one, and of this one
    uint64_t prev = 0;
    for (int i = tid; i < s; i += kHugeThreads) prev += a.tiem[(size_t)h * a.slices + i];
    const uint64_t before_slice = block_sum_u64(prev, red);
    const uint64_t mine = a.tiem[(size_t)h * a.slices + s];
    const uint64_t need = st.need;
    if (before_slice >= need) return;          // the cut was reached in an earlier slice
    uint32_t key[kHugePer];
    slice_keys(a, h, v, key);
    uint64_t* bm = a.kbm + (size_t)h * a.wcap;
    const int nwords = (v.n + 63) >> 6;
    uint32_t my_extra = 0;
    if (before_slice + mine <= need) {
        // every equal key of this slice precedes the point where the cut is reached
#pragma unroll
        for (int k = 0; k < kHugePer; ++k) {
            const bool take = key[k] == st.ustar;
            const uint64_t extra = __ballot(take);
            const int wi = (v.p0 >> 6) + wave + kHugeWaves * k;
            if (lane == 0 && extra && wi < nwords) atomicOr((unsigned long long*)&bm[wi], (unsigned long long)extra);
            my_extra += take;
        }
    } else {
        // positions run k-major (slot k covers p0 + 1024 k .. p0 + 1024 k + 1023): the mass
        // before (slot k, wave w) is every slot < k plus the waves < w of slot k
#pragma unroll
        for (int k = 0; k < kHugePer; ++k) {
            const uint64_t wk = key[k] == st.ustar ? mass_of(key[k]) : 0ull;
            uint64_t t;
            wave_excl_scan_u64(wk, &t);
            if (lane == 0) wsum[wave][k] = t;
        }
        __syncthreads();
        uint64_t run = before_slice;
#pragma unroll 1
        for (int k = 0; k < kHugePer; ++k) {
            uint64_t bw = 0, tot = 0;
            for (int ww = 0; ww < kHugeWaves; ++ww) {
                const uint64_t x = wsum[ww][k];
                bw += ww < wave ? x : 0ull;
                tot += x;
            }
            uint32_t kk = 0;                       // slot k's key, selected without indexing registers
#pragma unroll
            for (int q = 0; q < kHugePer; ++q) kk = q == k ? key[q] : kk;
            const uint64_t wk = kk == st.ustar ? mass_of(kk) : 0ull;
            uint64_t t;
            const uint64_t ex = wave_excl_scan_u64(wk, &t);
            const bool take = wk > 0 && run + bw + ex < need;
            const uint64_t extra = __ballot(take);
            const int wi = (v.p0 >> 6) + wave + kHugeWaves * k;
            if (lane == 0 && extra && wi < nwords) atomicOr((unsigned long long*)&bm[wi], (unsigned long long)extra);
            my_extra += take;
            run += tot;
            if (run >= need) break;                // uniform: every thread holds the same run
        }
    }
    const uint64_t tot = block_sum_u64(my_extra, red);
    if (tid == 0 && tot) atomicAdd(&a.stats[2 * h + 1], (int32_t)tot);
}

// grid (chunks, H_kv), 512 threads: kept nodes (union over the group's heads) in
// each chunk of kMergeW bitmap words, for the merge's rank offsets.
__global__ __launch_bounds__(kMergeW) void zha_chunk_count_kernel(ZhaLevelArgs a, int G, int c) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c));
    __shared__ uint32_t part[kMergeW / 64];
    const int g = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int nch = (int)((a.wcap + kMergeW - 1) / kMergeW);
    const int w = ch * kMergeW + tid;
    uint64_t hv[ZHA_MAX_GROUP];
#pragma unroll
    for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh)
        hv[hh] = (hh < G && w < a.wcap) ? a.kbm[((size_t)g * G + hh) * a.wcap + w] : 0ull;
    const int pn = a.top ? 0 : a.pnkept[g];
    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kSmallN) return;                  // selected and merged by the select kernel
    const int nwords = (n + 63) >> 6;
    uint64_t u = 0;
#pragma unroll
    for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) u |= hv[hh];
    uint32_t cnt = w < nwords ? (uint32_t)__popcll(u) : 0u;
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
    if ((tid & 63) == 0) part[tid >> 6] = cnt;
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int i = 0; i < kMergeW / 64; ++i) t += part[i];
        a.chunk_cnt[(size_t)g * nch + ch] = t;
    }
}

}  // namespace

int zha_score_blocks(int64_t max_cand, int R) {
    const int64_t U = R <= 16 ? 16 / R : 1;
    const int64_t items = (max_cand + U - 1) / U;
    int64_t blocks = (items + 3) / 4;        // one item per wave
    if (blocks < 1) blocks = 1;
    if (blocks > ZHA_SCORE_MAXB) blocks = ZHA_SCORE_MAXB;
    return (int)blocks;
}

bool zha_defer_fits(int G, int64_t wcap, int64_t pcap) {
    return (int64_t)G * wcap <= ZHA_DEFER_WORDS && pcap <= ZHA_DEFER_PARENTS;
}

size_t zha_defer_lds_bytes(int G, int64_t wcap, int64_t pcap) {
    return sizeof(uint64_t) * (size_t)(G + 1) * (size_t)wcap + sizeof(uint32_t) * (size_t)wcap +
           sizeof(int32_t) * (size_t)pcap;
}

hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream, const ZhaLevelArgs* defer) {
    if (a.hblk) {
        hipLaunchKernelGGL(zha_huge_init_kernel, dim3((unsigned)(H_kv * G)), dim3(kHugeThreads), 0, stream, a, H_kv * G);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)blocks, (unsigned)H_kv);
    if (defer) {
        const int64_t pcap = defer->top ? 0 : defer->pcap;
        if (a.top || defer->hblk || !zha_defer_fits(G, defer->wcap, pcap)) return hipErrorInvalidValue;
        const size_t lds = zha_defer_lds_bytes(G, defer->wcap, pcap);
        if (kv_dtype == 0)
            hipLaunchKernelGGL(zha_route_score_defer_kernel<true>, grid, dim3(kScoreThreads), lds, stream, q, a, *defer,
                               G, c, R, tau);
        else
            hipLaunchKernelGGL(zha_route_score_defer_kernel<false>, grid, dim3(kScoreThreads), lds, stream, q, a,
                               *defer, G, c, R, tau);
        return hipGetLastError();
    }
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_route_score_kernel<true>, grid, dim3(kScoreThreads), 0, stream, q, a, G, c, R, tau);
    else
        hipLaunchKernelGGL(zha_route_score_kernel<false>, grid, dim3(kScoreThreads), 0, stream, q, a, G, c, R, tau);
    return hipGetLastError();
}

hipError_t zha_launch_route_chain(int kv_dtype, const void* q, const ZhaChainArgs& m, int H_kv, int G, int c, int R,
                                  float tau, float top_p, hipStream_t stream) {
    int bmax = 1;
    for (int i = 0; i < m.n; ++i) {
        if (m.lv[i].cap > kSmallN) return hipErrorInvalidValue;
        bmax = std::max(bmax, m.blocks[i]);
    }
    const dim3 grid((unsigned)bmax, (unsigned)H_kv, (unsigned)m.n);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_route_score_all_kernel<true>, grid, dim3(kScoreThreads), 0, stream, q, m, G, c, R, tau);
    else
        hipLaunchKernelGGL(zha_route_score_all_kernel<false>, grid, dim3(kScoreThreads), 0, stream, q, m, G, c, R,
                           tau);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zha_select_chain_kernel, dim3((unsigned)H_kv), dim3(kSelThreads), 0, stream, m, G, c, top_p);
    return hipGetLastError();
}

hipError_t zha_launch_route_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream,
                                   bool merge) {
    if (a.cap <= kSmallN) {
        hipLaunchKernelGGL(zha_select_small_kernel, dim3((unsigned)H_kv), dim3(kSelThreads), 0, stream, a, G, c,
                           top_p);
        return hipGetLastError();
    }
    if (a.hblk) {
        // sliced level: a frontier of at most kSmallN candidates is selected and merged
        // by one workgroup per group; larger ones take three digit passes over slices,
        // the bitmap, the ordered ties, chunk counts and the merge (each of which
        // leaves at once for a small frontier)
        const int Hq = H_kv * G;
        hipLaunchKernelGGL(zha_select_large_kernel, dim3((unsigned)Hq), dim3(kSelThreads), 0, stream, a, G, c, top_p,
                           1);
        const dim3 sg((unsigned)a.slices, (unsigned)Hq);
        hipLaunchKernelGGL(zha_huge_pass_kernel<0>, sg, dim3(kHugeThreads), 0, stream, a, G, c, top_p, Hq);
        hipLaunchKernelGGL(zha_huge_pass_kernel<1>, sg, dim3(kHugeThreads), 0, stream, a, G, c, top_p, Hq);
        hipLaunchKernelGGL(zha_huge_pass_kernel<2>, sg, dim3(kHugeThreads), 0, stream, a, G, c, top_p, Hq);
        hipLaunchKernelGGL(zha_huge_bitmap_kernel, sg, dim3(kHugeThreads), 0, stream, a, G, c, top_p, Hq);
        hipLaunchKernelGGL(zha_huge_ties_kernel, sg, dim3(kHugeThreads), 0, stream, a, G, c, top_p, Hq);
        const int64_t nch = (a.wcap + kMergeW - 1) / kMergeW;
        hipLaunchKernelGGL(zha_chunk_count_kernel, dim3((unsigned)nch, (unsigned)H_kv), dim3(kMergeW), 0, stream, a,
                           G, c);
        hipLaunchKernelGGL(zha_route_merge_kernel, dim3((unsigned)nch, (unsigned)H_kv), dim3(kSelThreads), 0, stream,
                           a, G, c, kMergeW);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(zha_select_large_kernel, dim3((unsigned)(H_kv * G)), dim3(kSelThreads), 0, stream, a, G,
                       c, top_p, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !merge) return e;   // without merge: the next level's score kernel derives the list
    // bitmap words per merge block: a multiple of 16, at most kMergeW, over at
    // least kMergeBlocks blocks when the level is large enough
    const int64_t wcap = a.wcap;
    int64_t share = (wcap + kMergeBlocks - 1) / kMergeBlocks;
    share = std::min<int64_t>(kMergeW, (share + kSelWaves - 1) / kSelWaves * kSelWaves);
    const int64_t blocks = (wcap + share - 1) / share;
    hipLaunchKernelGGL(zha_route_merge_kernel, dim3((unsigned)blocks, (unsigned)H_kv), dim3(kSelThreads), 0, stream,
                       a, G, c, (int)share);
    return hipGetLastError();
}
