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
// mass-weighted radix select over 11/11/10-bit digits; candidates whose quantised
// delta equals the cut's are taken in ascending position (= node) order until the
// cumulative mass reaches ceil(p * sum e).
//
// Levels, top-down:
//   * the chain: the first levels of at most ZHA_CHAIN_SLOTS node slots are scored
//     whole by one launch (every node, every head), then one workgroup per query
//     head selects them one after the other with its own kept set in LDS, and
//     writes per-head kept bitmaps over node ids;
//   * every level below: a score launch over the group's candidates (the children
//     of the group's kept nodes of the level above, then the level's orphans),
//     then a selection launch: a group whose frontier has at most 1024
//     candidates is selected, and its kept list written, by one workgroup; larger
//     frontiers are histogrammed over slices by up to eight workgroups per head
//     and the head's last workgroup finishes its cut (at levels that can hold
//     frontiers past the keys one workgroup stages, a cross launch lists the
//     crossing bin's keys over the whole GPU and a resolve launch cuts them);
//     then an apply launch forms every candidate's mask of the heads that keep
//     it and writes the group's kept list in order (decoupled look-back).  Below
//     the chain, the first score kernel derives the chain's last level's group
//     kept list from the per-head bitmaps.  When that first level's planes are
//     small enough, the chain launch carries more workgroups, dispatched after
//     the selecting ones onto the compute units they leave idle, which score
//     every node of it while the chain selects; its score kernel then only
//     copies its candidates' scores (the same values: the same products over the
//     same operands).
//
// The candidates of a level are never written out: they are the children of the
// level above's kept nodes (kept list and head masks, ascending) followed by the
// level's orphans, so a candidate's node id and head mask come from one read of
// its parent's kept-list entry (or, below an unmerged level, from that level's
// bitmaps staged in LDS).
#include <algorithm>
#include <type_traits>

#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kScoreThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr float kFix = 1099511627776.0f;   // 2^40: fixed-point scale of e_i in [0, 1]
constexpr float kKeyScale = 134217728.0f;  // 2^27: delta quantum
constexpr float kDeltaMax = 32.0f;         // e^-32 * 2^40 < 1: heavier deltas carry no mass
constexpr int kHistBins = ZHA_HIST_BINS;    // bins of a selection digit histogram

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

// The chain's last level, whose group kept list is derived by the score
// workgroups of the level below it: they stage its per-head kept bitmaps over node
// ids ([G][wc] words, wc = ceil(n / 64) for its n complete nodes), their union and
// its popcount prefix, then read any entry of its kept list from LDS.
constexpr int kDeferW = ZHA_DEFER_WORDS / kScoreThreads;    // head words per thread
static_assert(kDeferW * kScoreThreads == ZHA_DEFER_WORDS, "deferred merge staging");
static_assert(ZHA_MAX_GROUP * (ZHA_CHAIN_SLOTS / 64) <= ZHA_DEFER_WORDS, "a chained level's head words fit");

struct DeferView {
    const uint64_t* hw;    // [G][wc] head words
    const uint64_t* u;     // [wc] union of the head words
    const uint32_t* pre;   // [wc] kept nodes in the words below
    int wc;                // words per head
};

// Head mask of the level's node qp.
__device__ __forceinline__ uint32_t defer_mask(const DeferView& v, int G, int qp) {
    const int w = qp >> 6, b = qp & 63;
    uint32_t m = 0;
    for (int hh = 0; hh < G; ++hh) m |= (uint32_t)((v.hw[hh * v.wc + w] >> b) & 1ull) << hh;
    return m;
}

// Entry r (< the kept count) of the level's kept list: the word holding it (the
// last whose prefix is <= r), then its bit by halving popcounts.
__device__ __forceinline__ void defer_entry(const DeferView& v, int G, uint32_t r, int32_t& node, uint32_t& mask) {
    int lo = 0, hi = v.wc - 1;
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
    node = lo * 64 + b;
    mask = defer_mask(v, G, node);
}

// Four FP8 E4M3 codes (bytes of w, low first: sign, 4 exponent bits of bias 7, 3
// mantissa bits, subnormals m 2^-9) as the float32 values they stand for, exactly:
// gfx950's packed conversion decodes this (OCP) layout.
typedef float zha_f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 e4m3x4_to_f32(uint32_t w) {
    const zha_f32x2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const zha_f32x2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_float4(lo.x, lo.y, hi.x, hi.y);
}

// Scores one level's candidates for every head of group g, as workgroup blk of
// nblk (256 threads).  Each wave scores items of U = 16/R candidates (R <= 16)
// or one candidate over R/16 column blocks (R > 16).  ALL: every node of the
// level is a candidate of every head (positions are node ids), whatever the
// level above kept.  hm gets the largest score of the lane's heads 4 kq + i.
// DEF: the level above (pa) was selected but not merged; its kept list is
// derived here from its bitmaps (dynamic LDS), and this workgroup writes its
// share of it (all of it together with the other workgroups).  NW: waves per
// workgroup.  NODE: the level's every node was scored already (a.sigN, node
// indexed, by this same arithmetic), and the candidates' scores are copied from
// there instead of computed.
// Candidate positions and node ids fit in 32 bits (capacity < 2^31).
template <bool BF16, bool ALL, bool DEF = false, int PF = 0, int NW = 4, bool NODE = false>
__device__ __forceinline__ void score_level(const void* __restrict__ q, const ZhaLevelArgs& a, int G, int c, int R,
                                            float tau, int g, int blk, int nblk, float (&hm)[4],
                                            const ZhaLevelArgs* pa = nullptr) {
    // every argument the kernel uses, fetched in one batch before any of them is
    // needed (otherwise the loads come in dependent rounds behind uniform branches)
    asm volatile("" ::"s"(q), "s"(a.S), "s"(a.B), "s"(a.cap), "s"(a.top), "s"(a.n_top), "s"(a.pklist),
                 "s"(a.pkmask), "s"(a.pnkept), "s"(a.pcap), "s"(a.orph_lo), "s"(a.orph_hi), "s"(a.dc.m),
                 "s"(a.dc.s1), "s"(a.dc.s2), "s"(a.ncand), "s"(a.sig), "s"(a.hblk), "s"(G), "s"(c), "s"(R),
                 "s"(tau));
    static_assert(!DEF || NW == 4, "the deferred merge stages its words over four waves");
    const bool top = ALL || a.top;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kq = lane >> 4;
    const int U = R <= 16 ? 16 / R : 1;
    const int CB = R <= 16 ? 1 : R / 16;
    const int span = R <= 16 ? R : 16;
    const int cl = R <= 16 ? j / R : 0;
    const uint32_t allg = all_heads(G);
    const size_t lrow = (size_t)(g % a.hkv) * a.cap;   // the tree's group (a batch routes virtual groups)
    const size_t prow = (size_t)g * a.pcap;
    const int stride = nblk * NW;
    const int pcap = (int)a.pcap;

    // One round trip before any work: the parent count, the first item's parent
    // entry (its index clamped to the parent level's capacity, not bounded by the
    // count) and the query rows are all in flight together.  At the first routed
    // level the parent arrays point at readable memory whose values go unused.
    int it = blk * NW + wave;
    int32_t pk = 0;
    uint32_t pm = 0;
    int pn_raw = 0;
    uint64_t dw[DEF ? kDeferW : 1];
    if (DEF) {
        // the chain's last level's head words over its complete nodes
        const int wcd = (int)((pa->n_top + 63) >> 6), nall = G * wcd;
        const uint64_t* kb = pa->kbm + (size_t)g * G * pa->wcap;
#pragma unroll
        for (int k = 0; k < kDeferW; ++k) {
            dw[k] = 0ull;
            if (k * kScoreThreads < nall) {           // uniform: slots wholly past the end skipped
                const int i = (int)threadIdx.x + k * kScoreThreads;
                const int hh = i / wcd, w = i - hh * wcd;
                if (i < nall) dw[k] = kb[(size_t)hh * pa->wcap + w];
            }
        }
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
    if (NODE) {
#pragma unroll
        for (int k = 0; k < 32; ++k) qa[k] = 0.f;
    } else if (BF16) {
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
        const int wc = (int)((pa->n_top + 63) >> 6), nall = G * wc;
        uint64_t* hw = zha_defer_lds;
        uint64_t* uu = hw + nall;
        uint32_t* pre = reinterpret_cast<uint32_t*>(uu + wc);
#pragma unroll
        for (int k = 0; k < kDeferW; ++k) {
            const int i = tid + k * kScoreThreads;
            if (i < nall) hw[i] = dw[k];
        }
        __syncthreads();
        // union word tid (wc <= 64 words), then the workgroup's exclusive popcount prefix
        uint64_t x = 0;
        if (tid < wc)
            for (int hh = 0; hh < G; ++hh) x |= hw[hh * wc + tid];
        if (tid < wc) uu[tid] = x;
        const uint32_t cnt = (uint32_t)__popcll(x);
        const uint32_t inc = (uint32_t)zha_wave_incl_scan_u64(cnt);
        if (lane == 63) s_wsum[wave] = inc;
        __syncthreads();
        uint32_t run = inc - cnt, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kScoreThreads / 64; ++w2) {
            const uint32_t y = s_wsum[w2];
            run += w2 < wave ? y : 0u;
            tot += y;
        }
        if (tid < wc) pre[tid] = run;
        __syncthreads();
        dv = DeferView{hw, uu, pre, wc};
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
                if (DEF) defer_entry(dv, G, (uint32_t)pi, pk, pm);
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
        if (NODE) {
            // the candidate's scores for the lane's heads 4 kq + i, already maxed over its planes
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * kq + i;
                if (valid && h < G) best[i] = a.sigN[((size_t)g * G + h) * (size_t)a.nstride + (size_t)node];
            }
        }
        for (int cb = 0; cb < (NODE ? 0 : CB); ++cb) {
            const int r = R <= 16 ? (j % R) : (cb * 16 + j);
            const size_t prw = (lrow + (size_t)node) * R + r;
            float4 sv[8];
            if (valid && PF == 2) {
                // the router's 8-bit copy: the same four elements per lane (one 4-byte
                // load each), decoded exactly; the plane's scale multiplies the product
                const uint32_t* plane = reinterpret_cast<const uint32_t*>(a.S8 + prw * ZHA_D);
                uint32_t u[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) u[m] = plane[4 * m + kq];
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = e4m3x4_to_f32(u[m]);
            } else if (valid && PF == 1) {
                // the router's bfloat16 copy: the same four elements per lane, widened exactly
                const uint2* plane = reinterpret_cast<const uint2*>(a.S16 + prw * ZHA_D);
                uint2 u[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) u[m] = plane[4 * m + kq];
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    sv[m] = make_float4(__uint_as_float(u[m].x << 16), __uint_as_float(u[m].x & 0xFFFF0000u),
                                        __uint_as_float(u[m].y << 16), __uint_as_float(u[m].y & 0xFFFF0000u));
            } else if (valid) {
                const float4* plane = reinterpret_cast<const float4*>(a.S + prw * ZHA_D);
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = plane[4 * m + kq];
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            const float bv = valid ? a.B[prw] : zha_neg_inf();
            const float ts = PF == 2 && valid ? tau * a.SC[prw] : tau;    // the scale is a power of two
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
            for (int i = 0; i < 4; ++i) best[i] = fmaxf(best[i], fmaf(ts, acc[i], bv));
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
                if (h < G) a.sig[((size_t)g * G + h) * a.sstride + (size_t)pos] = ((cm >> h) & 1u) ? best[i] : zha_neg_inf();
            }
        }
        if (valid) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((cm >> (4 * kq + i)) & 1u) hm[i] = fmaxf(hm[i], best[i]);
        }
    }
    // Stores issued before the loop would hold up its first loads (the memory
    // counter waits are in order), so the counts, the cleared selection state and
    // the derived kept list go last.
    if (blk == 0 && threadIdx.x == 0) a.ncand[g] = n_cand;
    if (!ALL && a.desc) {
        // this level's selection histograms and counters, apply tickets and look-back
        // descriptors, for the select and apply kernels' atomics
        if (blk == 0 && (int)threadIdx.x == 0) a.tick[g] = 0u;
        if (blk == 0 && (int)threadIdx.x < G) a.hdone[g * G + threadIdx.x] = 0u;
        uint32_t* desc = a.desc + (size_t)g * a.ndesc;
        for (int i = blk * NW * 64 + (int)threadIdx.x; i < a.ndesc; i += nblk * NW * 64) desc[i] = 0u;
        uint64_t* gm = a.ghist + (size_t)g * G * kHistBins;
        for (int i = blk * NW * 64 + (int)threadIdx.x; i < G * kHistBins; i += nblk * NW * 64) gm[i] = 0ull;
    }
    if constexpr (DEF) {
        // this workgroup's share of the chain's last level's kept list: words 4 blk +
        // wave + 4 nblk k, one node per lane
        int32_t* kl = pa->klist + (size_t)g * pa->cap;
        uint32_t* km = pa->kmask + (size_t)g * pa->cap;
#pragma unroll 1
        for (int w = blk * NW + wave; w < dv.wc; w += NW * nblk) {
            const uint64_t x = dv.u[w];
            if (lane_bit(x, lane)) {
                const int node = w * 64 + lane;
                const uint32_t rank = dv.pre[w] + bits_below_lane(x);
                kl[rank] = node;
                km[rank] = defer_mask(dv, G, node);
            }
        }
        if (blk == 0 && threadIdx.x == 0) pa->nkept[g] = pn;
    }
}

// The largest score of each head over this workgroup (for the selection's maximum).
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
template <bool BF16, int PF>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_kernel(const void* __restrict__ q,
                                                                        ZhaLevelArgs a, int G, int c, int R,
                                                                        float tau) {
    const int g = blockIdx.y;
    float hm[4];
    score_level<BF16, false, false, PF>(q, a, G, c, R, tau, g, blockIdx.x, gridDim.x, hm);
    if (a.hblk) block_head_max(a, g, G, hm);
}

// As zha_route_score_kernel, for a level whose parent level (pa) was selected but
// not merged: the workgroups derive and write that level's kept list themselves
// (dynamic LDS: zha_defer_lds_bytes).
template <bool BF16, int PF, bool NODE = false>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_defer_kernel(const void* __restrict__ q,
                                                                              ZhaLevelArgs a, ZhaLevelArgs pa,
                                                                              int G, int c, int R, float tau) {
    ZHA_LEVEL_ARGS_READY(pa, "s"(G));
    const int g = blockIdx.y;
    float hm[4];
    score_level<BF16, false, true, PF, 4, NODE>(q, a, G, c, R, tau, g, blockIdx.x, gridDim.x, hm, &pa);
    if (a.hblk) block_head_max(a, g, G, hm);
}

// grid (max blocks, H_kv, levels), 256 threads: every node of each of the first
// routed levels scored for every head of the group, positions = node ids (the
// levels' selection then gathers its candidates' scores from these).
template <bool BF16, int PF>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_all_kernel(const void* __restrict__ q,
                                                                            ZhaChainArgs m, int G, int c, int R,
                                                                            float tau) {
    const int z = blockIdx.z;
    if ((int)blockIdx.x >= m.blocks[z]) return;
    float hm[4];
    score_level<BF16, true, false, PF>(q, m.lv[z], G, c, R, tau, blockIdx.y, blockIdx.x, m.blocks[z], hm);
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

// Selection histograms: 2048 bins of key digits 31..21, 20..10 and 9..0.
constexpr int kBT = 1024;                     // threads of a selecting workgroup
constexpr int kBW = kBT / 64;
constexpr int kLdsKeys = ZHA_LDS_KEYS;        // a head's keys staged in LDS by the workgroup that cuts it
constexpr int kGList = ZHA_GLIST;             // a large frontier's crossing-bin keys listed per head
constexpr uint32_t kNotLarge = 0xFFFFFFFFu;   // published for a head the select kernel cut itself
constexpr int kSmallN = 1024;                 // groups with at most this many candidates select in one workgroup
static_assert(kSmallN == kSelThreads && kBT == kSelThreads, "small path: one position per thread");
constexpr int kSmallK = kSmallN / 64;
static_assert(ZHA_MAX_GROUP * (kSmallN + 2 * 256) + kSmallN <= kLdsKeys, "small path inside the key buffer");
static_assert(ZHA_MAX_GROUP * kSmallK <= kHistBins, "small-path kept words inside the histogram");
constexpr int kKeyRegs = kLdsKeys / kBT;       // positions per thread of a staged head
constexpr int kSlice = 4 * kBT;                 // positions a slice workgroup histograms (four per thread)
constexpr int kSliceW = 8;                      // slice workgroups per head
constexpr int kChainSlots = ZHA_CHAIN_SLOTS;
constexpr int kChainStage = 8192;               // chained scores of one head staged in LDS (floats)
constexpr int kChainPer = kChainSlots / kBT;  // candidate positions per thread in the chain
static_assert(kChainPer * kBT == kChainSlots && kChainPer * kBW <= 128, "chain rows: at most two scan entries per lane");
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
        if (hh < G && in) v[hh] = a.sig[((size_t)g * G + hh) * a.sstride + tid];   // hh < G: uniform
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


// ---- block-wide selection: the minimal top-p cut of one head over n keys, by one
// 1024-thread workgroup.  Position p's key comes from a functor; positions are
// walked p = tid + 1024 k.  A 2048-bin LDS histogram of the fixed-point mass of
// the first key digit (bits 31..21) locates the bin where the cumulative mass
// reaches ceil(p * total); the crossing bin's keys are then gathered, and if there
// are at most kRankMax of them the cut is found by ranking them directly, else by
// the next digit (bits 20..10, then 9..0).  Keys equal to the cut key all carry
// the same mass m, so the first t = ceil(need / m) of them in position order are
// kept (ties by ascending node index).

struct LdsKeys {
    const uint32_t* k;
    __device__ uint32_t operator()(int p) const { return k[p]; }
};
struct GlobKeys {        // frontiers beyond the LDS keys: formed again from the scores
    const float* sg;
    float m;
    __device__ uint32_t operator()(int p) const { return key_of(sg[p], m); }
};

constexpr int kRankMax = 64;   // crossing-bin keys ranked directly (one per lane of a wave)
constexpr int kGather = kBT;   // crossing-bin keys listed for the later passes (one per thread)
static_assert(kRankMax == 64 && kBT % 64 == 0, "rank: entry = lane, j split over the waves");

struct CutShared {
    uint64_t ws[kBW];          // per-wave sums
    uint32_t wc[kBW];          // per-wave counts
    int bin;
    uint32_t nent, plim, ustar;
    uint64_t before, need;
    uint4 ent[kRankMax];       // the crossing bin's keys: {key, position, mass lo, mass hi}
    uint64_t rank[kRankMax];   // mass of the entries before each
};

// The bin b of hist where before(b) < need <= before(b) + hist[b] (before(b): the
// mass of the bins below b).  need0 = 0: need = ceil(p * total), clamped to
// [1, total].  Found by the first kFindW waves, kFindPer consecutive bins per
// thread (the other waves wait at the barriers: every instruction here would
// otherwise run on all the workgroup's waves).  Results in st.
constexpr int kFindW = 4;
constexpr int kFindPer = kHistBins / (kFindW * 64);
static_assert(kFindPer % 2 == 0 && kFindW <= kBW, "find split");
__device__ __forceinline__ void block_find(const uint64_t* hist, uint64_t need0, float top_p, CutShared* st) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t h[kFindPer];
    uint64_t sum = 0, inc = 0;
    if (wave < kFindW) {
        const ulonglong2* hv = reinterpret_cast<const ulonglong2*>(hist) + tid * (kFindPer / 2);
#pragma unroll
        for (int k = 0; k < kFindPer / 2; ++k) {
            const ulonglong2 v = hv[k];
            h[2 * k] = v.x;
            h[2 * k + 1] = v.y;
        }
#pragma unroll
        for (int k = 0; k < kFindPer; ++k) sum += h[k];
        inc = zha_wave_incl_scan_u64(sum);
        if (lane == 63) st->ws[wave] = inc;
    }
    __syncthreads();
    if (wave < kFindW) {
        uint64_t wb = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kFindW; ++w) {
            const uint64_t x = st->ws[w];
            wb += w < wave ? x : 0ull;
            total += x;
        }
        uint64_t need = need0;
        if (need == 0) {
            need = (uint64_t)ceil((double)top_p * (double)total);
            if (need < 1) need = 1;
            if (need > total) need = total;
        }
        uint64_t bt = wb + inc - sum;          // mass below this thread's first bin
        if (bt < need && bt + sum >= need) {   // the one thread whose bins cross
#pragma unroll
            for (int k = 0; k < kFindPer; ++k) {
                if (bt < need && bt + h[k] >= need) {
                    st->bin = tid * kFindPer + k;
                    st->before = bt;
                    st->need = need;
                }
                bt += h[k];
            }
        }
    }
    __syncthreads();
}

// The cut among ne <= kRankMax keys listed in st->ent (st->rank cleared): entry
// i = lane's mass before it in (key, position) order is summed by every wave over
// its own kRankMax / kBW entries j (the same j for the whole wave: broadcast
// reads); the entry whose own mass reaches `need` is the cut.
__device__ __forceinline__ void rank_entries(CutShared* st, int ne, uint64_t need, uint32_t& ustar, uint32_t& plim) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kPerW = kRankMax / kBW;
    {
        const uint4 me = st->ent[lane < ne ? lane : 0];
        const uint64_t mk = ((uint64_t)me.x << 32) | me.y;      // (key, position) order
        uint64_t acc = 0;
#pragma unroll
        for (int jj = 0; jj < kPerW; ++jj) {
            const int j = wave * kPerW + jj;
            if (j < ne) {
                const uint4 f = st->ent[j];
                acc += (((uint64_t)f.x << 32) | f.y) < mk ? (((uint64_t)f.w << 32) | f.z) : 0ull;
            }
        }
        if (lane < ne && acc) atomicAdd((unsigned long long*)&st->rank[lane], (unsigned long long)acc);
    }
    __syncthreads();
    if (tid < ne) {
        const uint4 me = st->ent[tid];
        const uint64_t before = st->rank[tid], own = ((uint64_t)me.w << 32) | me.z;
        if (before < need && before + own >= need) {
            st->ustar = me.x;
            st->plim = me.y;
        }
    }
    __syncthreads();
    ustar = st->ustar;
    plim = st->plim;
}

// Visits every position p = tid + kBT i < n with its key, in batches of
// kSweepB per thread whose keys are all read before any is used: the visitors'
// LDS atomics and stores would otherwise order each later key read after them.
constexpr int kSweepB = 8;
template <class KF, class F, int NB = kSweepB>
__device__ __forceinline__ void sweep_keys(const KF& key_at, int n, F&& f) {
#pragma unroll 1
    for (int base = threadIdx.x; base < n; base += NB * kBT) {
        uint32_t kk[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int p = base + j * kBT;
            kk[j] = kNotCand;
            if (p < n) kk[j] = key_at(p);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) f(kk[j], base + j * kBT);
    }
}

// Calls f with the batch size of a sweep over n positions: one key per thread
// up to kBT positions, four up to 4 kBT, else kSweepB (no batch slot that lies
// past n for every thread).
template <class F>
__device__ __forceinline__ void with_batch(int n, F&& f) {
    if (n <= kBT) f(std::integral_constant<int, 1>{});
    else if (n <= 4 * kBT) f(std::integral_constant<int, 4>{});
    else f(std::integral_constant<int, kSweepB>{});
}

// The cut of one head: kept iff key < ustar, or key == ustar and p <= plim.  With
// `pre0`, hist already holds the first digit's histogram over all keys.  Called by
// the whole workgroup when the head has candidates and p < 1.  Each pass finds the
// crossing bin of its digit, then counts the bin's keys (building the next digit's
// histogram over them) and writes them out at their block-wide ranks: to the rank
// table when there are at most kRankMax of them (the cut is then found by ranking
// them), and, the first time there are at most kGather of them, to the list gl
// [kGather] that later passes sweep instead of all n keys.
// Entry i of a key set is the candidate at position pos_at(i) (the identity for a
// head's whole frontier).  need0 > 0: the cut must supply exactly that mass (keys
// gathered from one crossing bin); 0: ceil(p * total).  Returns false, leaving
// the cut unset, only when more than kRankMax keys equal the cut key and
// `ties_in_order` is false (their entries are then not in position order).
struct IdPos {
    __device__ uint32_t operator()(int i) const { return (uint32_t)i; }
};
template <class KF, class PF>
__device__ bool block_cut(const KF& key_at, const PF& pos_at, int n, float top_p, uint64_t need0, bool pre0,
                          bool ties_in_order, uint64_t* hist, uint2* gl, CutShared* st, uint32_t& ustar,
                          uint32_t& plim) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t pref = 0;
    uint64_t need = need0;
    ustar = 0;
    plim = 0xFFFFFFFFu;
    if (n <= kRankMax) {
        // every key ranked directly: massless keys and non-candidates enter with
        // mass 0, which never reaches the cut
        if (tid < kRankMax) {
            const uint32_t k = tid < n ? key_at(tid) : kNotCand;
            const uint32_t pos = tid < n ? pos_at(tid) : 0xFFFFFFFFu;
            const uint64_t ms = k < kNoMass ? mass_of(k) : 0ull;
            st->ent[tid] = make_uint4(k, pos, (uint32_t)ms, (uint32_t)(ms >> 32));
            st->rank[tid] = 0ull;
        }
        __syncthreads();
        if (need == 0) {
            // the total over the entries (one per lane), formed by every wave
            const uint4 e0 = st->ent[lane];
            const uint64_t total = zha_readlane_u64(zha_wave_incl_scan_u64(((uint64_t)e0.w << 32) | e0.z), 63);
            need = (uint64_t)ceil((double)top_p * (double)total);
            if (need < 1) need = 1;
            if (need > total) need = total;
        }
        rank_entries(st, n, need, ustar, plim);
        return true;
    }
    if (!pre0) {
        hist[2 * tid] = 0ull;
        hist[2 * tid + 1] = 0ull;
        __syncthreads();
        const auto add = [&](uint32_t k, int) {
            if (k < kNoMass) atomicAdd((unsigned long long*)&hist[k >> 21], (unsigned long long)mass_of(k));
        };
        with_batch(n, [&](auto nbc) { sweep_keys<KF, decltype(add) const&, decltype(nbc)::value>(key_at, n, add); });
        __syncthreads();
    }
    int nl = -1;                               // >= 0: the crossing keys of an earlier pass are gl[0, nl)
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const uint32_t shift = pass == 0 ? 21u : pass == 1 ? 10u : 0u;
        block_find(hist, need, top_p, st);     // (ends with a barrier: hist free again)
        const uint32_t bin = (uint32_t)st->bin;
        need = st->need - st->before;          // mass still needed inside the crossing bin
        pref = pass == 0 ? bin : ((pref << (pass == 1 ? 11 : 10)) | bin);
        // the next digit (bits 20..10, then 9..0) of the crossing bin's keys
        const uint32_t nshift = pass == 0 ? 10u : 0u;
        const uint32_t nmask = pass == 0 ? 2047u : 1023u;
        if (pass < 2) {
            hist[2 * tid] = 0ull;
            hist[2 * tid + 1] = 0ull;
        }
        if (tid < kRankMax) st->rank[tid] = 0ull;
        if (tid == 0) st->nent = 0u;
        __syncthreads();
        // the crossing bin's keys, appended a wave and a batch at a time (one LDS
        // atomic per wave and batch reserves their slots): the first kRankMax to the
        // rank table, the first kGather to the list while none is kept yet; each adds
        // its mass to the next digit's histogram
        const bool listing = nl < 0;
        const auto append = [&](const uint32_t* kk, const int* pp, auto nbc) {
            constexpr int NB = decltype(nbc)::value;
            bool in[NB];
            uint64_t bal[NB];
            uint32_t tot = 0;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                in[j] = (kk[j] < kNoMass) & ((kk[j] >> shift) == pref);
                bal[j] = __ballot(in[j]);
                tot += (uint32_t)__popcll(bal[j]);
            }
            if (tot == 0u) return;             // uniform over the wave
            uint32_t e0 = 0;
            if (lane == 0) e0 = atomicAdd(&st->nent, tot);
            e0 = (uint32_t)__shfl((int)e0, 0);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (in[j]) {
                    const uint32_t k = kk[j];
                    const uint32_t e = e0 + bits_below_lane(bal[j]);
                    const uint64_t ms = mass_of(k);
                    if (e < (uint32_t)kRankMax) st->ent[e] = make_uint4(k, (uint32_t)pp[j], (uint32_t)ms, (uint32_t)(ms >> 32));
                    if (listing && e < (uint32_t)kGather) gl[e] = make_uint2(k, (uint32_t)pp[j]);
                    if (pass < 2) atomicAdd((unsigned long long*)&hist[(k >> nshift) & nmask], (unsigned long long)ms);
                }
                e0 += (uint32_t)__popcll(bal[j]);
            }
        };
        if (!listing) {
            uint32_t kk[1];
            int pp[1];
            const uint2 le = tid < nl ? gl[tid] : make_uint2(kNotCand, 0u);
            kk[0] = le.x;
            pp[0] = (int)le.y;
            append(kk, pp, std::integral_constant<int, 1>{});
        } else {
            with_batch(n, [&](auto nbc) {
                constexpr int NB = decltype(nbc)::value;
#pragma unroll 1
                for (int base = tid; base - tid < n; base += NB * kBT) {   // uniform
                    uint32_t kk[NB];
                    int pp[NB];
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int i = base + j * kBT;
                        kk[j] = kNotCand;
                        pp[j] = 0;
                        if (i < n) {
                            kk[j] = key_at(i);
                            pp[j] = (int)pos_at(i);
                        }
                    }
                    append(kk, pp, nbc);
                }
            });
        }
        __syncthreads();
        const uint32_t ne = st->nent;
        const bool to_rank = ne <= (uint32_t)kRankMax;
        const bool to_list = listing && ne <= (uint32_t)kGather;
        if (to_list) nl = (int)ne;
        if (to_rank) {
            rank_entries(st, (int)ne, need, ustar, plim);
            return true;
        }
        if (pass == 2) {
            if (!ties_in_order) return false;
            // more than kRankMax keys equal to the cut key: the first t of them in
            // position order
            ustar = pref;
            const uint64_t ms = mass_of(ustar);
            const uint64_t t = (need + ms - 1) / ms;
            if (tid == 0) st->plim = 0xFFFFFFFFu;
            __syncthreads();
            uint32_t run = 0;
#pragma unroll 1
            for (int base = 0; base < n; base += kBT) {
                const int p = base + tid;
                const bool tie = p < n && key_at(p) == ustar;
                const uint64_t bal = __ballot(tie);
                if (lane == 0) st->wc[wave] = (uint32_t)__popcll(bal);
                __syncthreads();
                uint32_t before = run, tot = 0;
#pragma unroll
                for (int w2 = 0; w2 < kBW; ++w2) {
                    const uint32_t x = st->wc[w2];
                    before += w2 < wave ? x : 0u;
                    tot += x;
                }
                if (tie && before + bits_below_lane(bal) + 1 == (uint32_t)t) st->plim = (uint32_t)p;
                __syncthreads();
                run += tot;
                if (run >= (uint32_t)t) break;   // uniform
            }
            plim = st->plim;
            return true;
        }
    }
    return true;                               // (not reached: the third pass always returns)
}

// Kept iff (key, position) <= the head's limit in lexicographic order: the cut's
// (key, position) (a cut key always carries mass, so it lies below kNoMass); with
// keep_all every candidate key, massless ones included; with none nothing (a head
// with no candidate has only kNotCand keys, which pass no limit).  One 64-bit
// comparison per key, its mask usable as a ballot: no per-key mask arithmetic on
// the scalar unit, which every wave of a workgroup shares.
__device__ __forceinline__ uint64_t kept_limit(bool none, bool keep_all, uint32_t ustar, uint32_t plim) {
    return none ? 0ull : keep_all ? (((uint64_t)kNoMass << 32) | 0xFFFFFFFFull) : (((uint64_t)ustar << 32) | plim);
}
__device__ __forceinline__ bool kept_by(uint32_t key, uint32_t p, bool none, bool keep_all, uint32_t ustar,
                                        uint32_t plim) {
    return ((((uint64_t)key) << 32) | p) <= kept_limit(none, keep_all, ustar, plim);
}

// Maximum over the workgroup (every thread receives it).
__device__ __forceinline__ float block_max(float x, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x = zha_wave_max(x);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kBW; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

// Exclusive prefix sums of s[0, kRows) in place by one wave, kRows <= 128 (entries
// lane * kPer .. lane * kPer + kPer - 1 per lane, so the order is kept); returns the
// total.
template <int kRows>
__device__ __forceinline__ uint32_t wave_scan_rows(uint32_t* s) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = (kRows + 63) / 64;
    uint32_t v[kPer];
    uint32_t loc = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = lane * kPer + j;
        v[j] = i < kRows ? s[i] : 0u;
        loc += v[j];
    }
    uint64_t tot;
    uint32_t ex = (uint32_t)wave_excl_scan_u64(loc, &tot);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = lane * kPer + j;
        if (i < kRows) s[i] = ex;
        ex += v[j];
    }
    return (uint32_t)tot;
}

// ---- the chain: the first routed levels, each at most kChainSlots complete nodes,
// every node of them scored beforehand (node-indexed scores).  One workgroup per
// query head walks them top-down with its own kept set in LDS: its candidates at a
// level are the children of its kept nodes of the level above, in ascending node
// order, then the level's orphans.  Per level it writes its kept bitmap over node
// ids and its candidate and kept counts.
template <bool BF16, int PF>
__global__ __launch_bounds__(kBT) void zha_chain_kernel(ZhaChainSel m, int G, int c, float top_p) {
    __shared__ __align__(16) uint32_t s_keys[kChainSlots];
    __shared__ int32_t s_kept[kChainSlots];
    __shared__ int32_t s_node[kChainSlots];
    __shared__ __align__(16) uint64_t s_hist[kHistBins];
    __shared__ uint2 s_gl[kGather];
    __shared__ uint64_t s_bm[kChainSlots / 64];
    __shared__ uint32_t s_pre[kChainPer * kBW];
    __shared__ uint32_t s_tot[2];
    __shared__ float s_red[kBW];
    __shared__ CutShared st;
    __shared__ __align__(16) float s_sig[kChainStage];
    if ((int)blockIdx.x >= m.nsel) {
        // dispatched after the selecting workgroups: score every node of the level
        // below the chain for every head (node-indexed), by the score kernels' own
        // arithmetic, while the selection runs (groups interleaved)
        const int sb = (int)blockIdx.x - m.nsel, ng = m.nsel / G;
        float hm[4];
        score_level<BF16, true, false, PF, kBT / 64>(m.q, m.spec, G, c, m.R, m.tau, sb % ng, sb / ng, m.spec_blocks,
                                                     hm);
        return;
    }
    const int h = blockIdx.x, g = h / G, hl = h - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the head's scores of every chained level, staged in LDS together (one round
    // trip) when they fit: level li's complete nodes at soff[li] (rows read as
    // whole 16-byte vectors, which never pass a row's padded end)
    int soff[ZHA_MAX_CHAIN + 1];
    soff[0] = 0;
#pragma unroll
    for (int li = 0; li < ZHA_MAX_CHAIN; ++li)
        soff[li + 1] = soff[li] + (li < m.n ? (m.lv[li].n_nodes + 3) / 4 * 4 : 0);
    const bool staged = soff[ZHA_MAX_CHAIN] <= kChainStage;
    if (staged) {
        constexpr int kStageV = kChainStage / 4 / kBT;     // 16-byte vectors per thread
        float4 t[kStageV];
#pragma unroll
        for (int k = 0; k < kStageV; ++k) {
            const int o = 4 * (tid + k * kBT);               // staged float index
            const float* row = m.lv[0].sig + ((size_t)g * G + hl) * (size_t)m.lv[0].sstride;
            int base = 0;
#pragma unroll
            for (int j = 1; j < ZHA_MAX_CHAIN; ++j) {
                if (j < m.n && o >= soff[j]) {
                    row = m.lv[j].sig + ((size_t)g * G + hl) * (size_t)m.lv[j].sstride;
                    base = soff[j];
                }
            }
            t[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (o < soff[ZHA_MAX_CHAIN]) t[k] = *reinterpret_cast<const float4*>(row + (o - base));
        }
#pragma unroll
        for (int k = 0; k < kStageV; ++k) {
            const int o = 4 * (tid + k * kBT);
            if (o < soff[ZHA_MAX_CHAIN]) *reinterpret_cast<float4*>(s_sig + o) = t[k];
        }
        __syncthreads();
    }
    int nk = 0;
    int so = 0;                                // soff[li], kept as a running sum
#pragma unroll 1
    for (int li = 0; li < m.n; ++li) {
        const ZhaChainLevel& L = m.lv[li];
        const int n = li == 0 ? L.n_nodes : nk * c + (L.orph_hi - L.orph_lo);
        const float* sg = L.sig + ((size_t)g * G + hl) * (size_t)L.sstride;
        const float* ss = s_sig + so;
        so += (L.n_nodes + 3) / 4 * 4;
        // (rows of 1024 positions wholly past n are skipped: a uniform branch)
        float x[kChainPer];
#pragma unroll
        for (int k = 0; k < kChainPer; ++k) {
            x[k] = zha_neg_inf();
            if (k * kBT < n) {
                const int p = tid + k * kBT;
                int32_t nd = p;
                if (li > 0) {
                    const int pc = p < nk * c ? p : 0;
                    const int pi = pc / c;
                    nd = p < nk * c ? s_kept[pi] * c + (pc - pi * c) : L.orph_lo + (p - nk * c);
                }
                nd = p < n ? nd : 0;
                s_node[p] = nd;
                if (p < n) x[k] = staged ? ss[nd] : sg[nd];
            }
        }
        float mx = zha_neg_inf();
#pragma unroll
        for (int k = 0; k < kChainPer; ++k) mx = fmaxf(mx, x[k]);
        const float M = block_max(mx, s_red);   // (its barriers also end every read of s_kept)
#pragma unroll
        for (int k = 0; k < kChainPer; ++k) {
            const int p = tid + k * kBT;
            if (k * kBT < n) s_keys[p] = p < n ? key_of(x[k], M) : kNotCand;
        }
        for (int i = tid; i < kChainSlots / 64; i += kBT) s_bm[i] = 0ull;
        __syncthreads();
        const bool none = M == zha_neg_inf();
        const bool keep_all = !none && top_p >= 1.0f;
        uint32_t ustar = 0, plim = 0xFFFFFFFFu;
        if (!none && !keep_all) block_cut(LdsKeys{s_keys}, IdPos{}, n, top_p, 0, false, true, s_hist, s_gl, &st, ustar, plim);
        // kept flags and their ranks in position order (rows of 1024 positions);
        // keys and node ids read back from LDS (not held across the cut)
        bool kept[kChainPer];
        uint64_t bal[kChainPer];
        uint32_t ncand = 0;
#pragma unroll
        for (int k = 0; k < kChainPer; ++k) {
            kept[k] = false;
            bal[k] = 0ull;
            if (k * kBT < n) {
                const uint32_t p = (uint32_t)(tid + k * kBT);
                const uint32_t key = s_keys[p];
                kept[k] = kept_by(key, p, none, keep_all, ustar, plim);
                bal[k] = __ballot(kept[k]);
                ncand += (uint32_t)__popcll(__ballot(key != kNotCand));
            }
            if (lane == 0) s_pre[k * kBW + wave] = (uint32_t)__popcll(bal[k]);
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t tot = wave_scan_rows<kChainPer * kBW>(s_pre);
            if (lane == 0) s_tot[0] = tot;
        }
        if (tid == 0) s_tot[1] = 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kChainPer; ++k) {
            if (kept[k]) {
                const int32_t nd = s_node[tid + k * kBT];
                const uint32_t r = s_pre[k * kBW + wave] + bits_below_lane(bal[k]);
                s_kept[r] = nd;
                atomicOr((unsigned long long*)&s_bm[nd >> 6], 1ull << (nd & 63));
            }
        }
        // candidates counted per wave above are the whole wave's: lane 0 of every wave
        // adds them once
        if (lane == 0) atomicAdd(&s_tot[1], ncand);
        __syncthreads();
        nk = (int)s_tot[0];
        // the words holding the level's complete nodes (at most kChainSlots / 64)
        uint64_t* bm = L.kbm + ((size_t)g * G + hl) * (size_t)L.wcap;
        for (int i = tid; i < (L.n_nodes + 63) / 64; i += kBT) bm[i] = s_bm[i];
        if (tid == 0) {
            L.stats[2 * h + 0] = (int32_t)s_tot[1];
            L.stats[2 * h + 1] = nk;
        }
        __syncthreads();                        // LDS reused by the next level
    }
}

// ---- the kept list of a group from its per-head kept bitmaps over node ids (a
// chained level 1): each position's mask of heads, the ascending ranks of the
// union's positions, and the list.  One 1024-thread workgroup per group.
__global__ __launch_bounds__(kBT) void zha_merge_ids_kernel(ZhaLevelArgs a, int G, int c) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c));
    __shared__ uint32_t s_wc[kChainPer * kBW];
    __shared__ uint32_t s_tot;
    const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)a.n_top;                    // <= kChainSlots
    const uint64_t* gbm = a.kbm + (size_t)g * G * a.wcap;
    uint32_t msk[kChainPer];
    uint64_t bal[kChainPer];
#pragma unroll
    for (int k = 0; k < kChainPer; ++k) {
        const int p = tid + k * kBT;
        uint64_t hw[ZHA_MAX_GROUP];
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh)
            hw[hh] = (hh < G && p < n) ? gbm[(size_t)hh * a.wcap + (p >> 6)] : 0ull;
        uint32_t m = 0;
#pragma unroll
        for (int hh = 0; hh < ZHA_MAX_GROUP; ++hh) m |= (uint32_t)((hw[hh] >> lane) & 1ull) << hh;
        msk[k] = m;
        bal[k] = __ballot(m != 0u);
        if (lane == 0) s_wc[k * kBW + wave] = (uint32_t)__popcll(bal[k]);
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t tot = wave_scan_rows<kChainPer * kBW>(s_wc);
        if (lane == 0) s_tot = tot;
    }
    __syncthreads();
    int32_t* kl = a.klist + (size_t)g * a.cap;
    uint32_t* km = a.kmask + (size_t)g * a.cap;
#pragma unroll
    for (int k = 0; k < kChainPer; ++k) {
        if (msk[k]) {
            const uint32_t r = s_wc[k * kBW + wave] + bits_below_lane(bal[k]);
            kl[r] = tid + k * kBT;
            km[r] = msk[k];
        }
    }
    if (tid == 0) a.nkept[g] = (int32_t)s_tot;
}

// A head's kept flags over positions [0, n) as bitmap words (one per 64 positions,
// to `bits`), wave w taking words w, w + kBW, ... in batches whose keys are all read
// before any is used.  Returns the wave's kept count (high word) and candidate
// count (low word), the same in every lane.
template <class KF>
__device__ __forceinline__ uint64_t head_words(const KF& key_at, int n, bool none, bool keep_all, uint32_t ustar,
                                               uint32_t plim, uint64_t* bits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = (n + 63) >> 6;
    uint32_t w_kept = 0, w_cand = 0;
#pragma unroll 1
    for (int w0 = wave; w0 < nw; w0 += kBW * kSweepB) {   // uniform per wave
        uint32_t kk[kSweepB];
#pragma unroll
        for (int j = 0; j < kSweepB; ++j) {
            const int p = (w0 + j * kBW) * 64 + lane;
            kk[j] = kNotCand;
            if (p < n) kk[j] = key_at(p);
        }
#pragma unroll
        for (int j = 0; j < kSweepB; ++j) {
            const int wd = w0 + j * kBW;
            const uint64_t b = __ballot(kept_by(kk[j], (uint32_t)(wd * 64 + lane), none, keep_all, ustar, plim));
            w_cand += (uint32_t)__popcll(__ballot(kk[j] != kNotCand));
            w_kept += (uint32_t)__popcll(b);
            if (lane == 0 && wd < nw) bits[wd] = b;
        }
    }
    return ((uint64_t)w_kept << 32) | w_cand;
}

// ---- levels below the chain: two launches after the score kernel.
//
// zha_select_kernel, grid (kSliceW, H_q), 1024 threads: a frontier of at most
// kSmallN candidates per group is selected for every head, and its kept list
// written, by the group's first workgroup (small path).  Otherwise workgroup w of
// head h adds the first-digit mass histogram of slices w, w + kSliceW, ... of the
// head's candidates (kSlice positions each) into the head's global histogram with
// integer atomics; the head's last workgroup to finish (a counter; every wave first
// waits for its own atomics, and the histogram is read back with device-scope
// loads, which bypass this device's non-coherent caches) stages the head's keys in
// LDS, finishes the cut, and writes it as the head's cut descriptor with its
// candidate and kept counts.  The histograms and counters were cleared by this
// level's score kernel.
//
// zha_apply_kernel, grid (chunks, H_kv), 256 or 1024 threads: each workgroup takes
// the next kApplyChunk candidate positions of its group (a ticket, so chunks run in
// order of start), forms every position's mask of the heads that keep it from the
// heads' scores and cuts, and writes the kept positions' entries of the group's
// kept list at ranks found by a decoupled look-back: each chunk publishes its kept
// count, then adds its predecessors' published counts (or a predecessor's
// published inclusive prefix) to find where its entries start.  A chunk waits only
// on chunks that started before it, so the waits always end.  Published values are
// device-scope atomics read with device-scope loads.
// Apply workgroups take four positions per thread: 256 threads at levels of at most
// kApplyWideCap slots, else 1024 (fewer chunks, fewer tickets drawn on one word).
#ifndef ZHA_APPLY_WIDE_CAP
#define ZHA_APPLY_WIDE_CAP 131072
#endif
constexpr int kApplyWideCap = ZHA_APPLY_WIDE_CAP;
constexpr int kApplyEarly = 64;                   // apply workgroups per group drawing their ticket at once
__host__ __device__ constexpr int apply_threads(int64_t cap) { return cap > kApplyWideCap ? 1024 : 256; }
constexpr uint32_t kDescAgg = 1u << 30;           // descriptor: the chunk's kept count is published
constexpr uint32_t kDescInc = 2u << 30;           // descriptor: its inclusive prefix is published
constexpr uint32_t kDescVal = kDescAgg - 1u;
constexpr uint32_t kSpinMax = 1u << 22;           // bound on a look-back wait (a safety net)

struct HeadCut {                                  // written by zha_select_kernel per head
    float m;                                      // largest score of the head's candidates
    uint32_t ustar, plim;                         // kept: key < ustar, or key == ustar and position <= plim
    uint32_t mode;                                // 0 cut, 1 keep all, 2 no candidate
};

__global__ __launch_bounds__(kBT) void zha_select_kernel(ZhaLevelArgs a, int G, int c, float top_p) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p));
    __shared__ __align__(16) uint32_t s_keys[kLdsKeys];
    __shared__ __align__(16) uint64_t s_hist[kHistBins];
    __shared__ uint2 s_gl[kGather];
    __shared__ float s_red[kBW];
    __shared__ uint64_t s_wred[kBW];
    __shared__ CutShared st;
    __shared__ int s_last;
    const int h = blockIdx.y, g = h / G, hl = h - g * G, w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* sg = a.sig + ((size_t)g * G + hl) * (size_t)a.sstride;
    const float4* sg4 = reinterpret_cast<const float4*>(sg);

    // one round trip: the head's per-block maxima, this workgroup's slice of
    // kSlice positions as one 16-byte load per thread (rows are 16-byte aligned and
    // padded to whole vectors), with one workgroup per head every position of the
    // level's capacity (at most kLdsKeys), and, last, the parent count
    const bool single = gridDim.x == 1;        // the level's capacity is one slice: one workgroup per head
    const float hb = tid < a.score_blocks ? a.hblk[(size_t)h * ZHA_SCORE_MAXB + tid] : zha_neg_inf();
    const int nv_cap = (int)(a.sstride / 4);
    constexpr int kVec = kKeyRegs / 4;         // float4 loads per thread of a staged head
    float4 y[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) y[k] = make_float4(zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf());
    {
        const int v = w * (kSlice / 4) + tid;
        if (v < nv_cap) y[0] = sg4[v];
    }
    if (single) {
#pragma unroll
        for (int k = 1; k < kVec; ++k) {
            if (k * kBT < nv_cap) {            // uniform: rows wholly past the capacity skipped
                const int v = tid + k * kBT;
                if (v < nv_cap) y[k] = sg4[v];
            }
        }
    }
    float4 x = y[0];
    const int pn = parent_count(a, g);
    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kSmallN) {
        if (w != 0 || hl != 0) return;
        float* s_sig = reinterpret_cast<float*>(s_keys);                                   // [G][kSmallN]
        uint64_t* s_hs = reinterpret_cast<uint64_t*>(s_keys + ZHA_MAX_GROUP * kSmallN);    // [G][256]
        int32_t* s_nid = reinterpret_cast<int32_t*>(s_keys + ZHA_MAX_GROUP * kSmallN + 2 * ZHA_MAX_GROUP * 256);
        stage_small(a, g, G, c, tid, s_sig, s_nid);
        __syncthreads();
        select_small_group(a, g, G, top_p, n, s_sig, s_nid, s_hs, s_hist);
        return;
    }
    const int nsl = (n + kSlice - 1) / kSlice;
    const int active = min(kSliceW, nsl);
    if (w >= active) return;
    const float M = block_max(hb, s_red);
    const bool none = M == zha_neg_inf();
    const bool keep_all = !none && top_p >= 1.0f;
    const bool cut = !none && !keep_all;
    uint64_t* gm = a.ghist + (size_t)h * kHistBins;
    if (cut && !single) {
        // the first digit's mass histogram of slices w, w + kSliceW, ..., added into
        // the head's global histogram (integer atomics: exact and order-free)
        s_hist[2 * tid] = 0ull;
        s_hist[2 * tid + 1] = 0ull;
        __syncthreads();
#pragma unroll 1
        for (int sl = w; sl < nsl; sl += kSliceW) {
            if (sl != w) {
                const int v = sl * (kSlice / 4) + tid;
                x = v < nv_cap ? sg4[v] : make_float4(zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf());
            }
            const float v4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = sl * kSlice + 4 * tid + j;
                const uint32_t key = p < n ? key_of(v4[j], M) : kNotCand;
                if (key < kNoMass) atomicAdd((unsigned long long*)&s_hist[key >> 21], (unsigned long long)mass_of(key));
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint64_t v = s_hist[2 * tid + i];
            if (v) atomicAdd((unsigned long long*)&gm[2 * tid + i], (unsigned long long)v);
        }
        zha_wave_mem_wait();                   // this wave's histogram adds have completed
    }
    if (!single) {
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(&a.hdone[h], 1u) == (uint32_t)(active - 1);
        __syncthreads();
        if (!s_last) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }

    // ---- the head's last workgroup: the complete histogram (read past this
    // device's caches) and the head's keys (LDS, 16-byte loads), then the cut
    const bool staged = n <= kLdsKeys;        // (always, with one workgroup per head)
    const bool large = !staged && cut && a.glist != nullptr;
    if (large) {
        // a frontier beyond the LDS keys: publish the first digit's crossing bin and
        // the mass still needed inside it; the cross and resolve kernels finish
#pragma unroll
        for (int i = 0; i < 2; ++i)
            s_hist[2 * tid + i] = __hip_atomic_load(gm + 2 * tid + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        block_find(s_hist, 0, top_p, &st);
        if (tid == 0) {
            const uint64_t need = st.need - st.before;
            a.pub[h] = make_uint4((uint32_t)st.bin, (uint32_t)need, (uint32_t)(need >> 32), __float_as_uint(M));
            a.gcnt[h] = make_uint4(0u, 0u, 0u, 0u);
        }
        return;
    }
    {
        uint64_t hm2[2] = {0ull, 0ull};
        if (cut && !single) {
#pragma unroll
            for (int i = 0; i < 2; ++i) hm2[i] = __hip_atomic_load(gm + 2 * tid + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const int nvn = (n + 3) / 4;
        if (!single) {
            // the head's keys, read again by its last slice workgroup
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                y[k] = make_float4(zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf());
                if (staged && k * kBT < nvn) {     // uniform: rows wholly past n skipped
                    const int v = tid + k * kBT;
                    if (v < nvn) y[k] = sg4[v];
                }
            }
        }
        s_hist[2 * tid] = hm2[0];
        s_hist[2 * tid + 1] = hm2[1];
        if (staged) {
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const int p = 4 * (tid + k * kBT);
                if (p < n) {
                    const float v[4] = {y[k].x, y[k].y, y[k].z, y[k].w};
                    uint32_t kk[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) kk[j] = p + j < n ? key_of(v[j], M) : kNotCand;
                    *reinterpret_cast<uint4*>(s_keys + p) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
                }
            }
        }
    }
    __syncthreads();
    uint32_t ustar = 0, plim = 0xFFFFFFFFu;
    if (cut) {
        // (one workgroup per head: block_cut builds the first digit's histogram itself)
        if (staged) block_cut(LdsKeys{s_keys}, IdPos{}, n, top_p, 0, !single, true, s_hist, s_gl, &st, ustar, plim);
        else block_cut(GlobKeys{sg, M}, IdPos{}, n, top_p, 0, true, true, s_hist, s_gl, &st, ustar, plim);
    }
    // the head's kept flags as a bitmap over positions, one word per 64 (read by the
    // apply), and its kept and candidate counts
    {
        uint64_t* hbits = a.kbm + ((size_t)g * G + hl) * (size_t)a.wcap;
        const uint64_t kc = staged ? head_words(LdsKeys{s_keys}, n, none, keep_all, ustar, plim, hbits)
                                   : head_words(GlobKeys{sg, M}, n, none, keep_all, ustar, plim, hbits);
        if (lane == 0) s_wred[wave] = kc;
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t t = 0;
#pragma unroll
        for (int w2 = 0; w2 < kBW; ++w2) t += s_wred[w2];
        a.stats[2 * h + 0] = (int32_t)(uint32_t)t;
        a.stats[2 * h + 1] = (int32_t)(t >> 32);
        HeadCut hc;
        hc.m = M;
        hc.ustar = ustar;
        hc.plim = plim;
        hc.mode = none ? 2u : keep_all ? 1u : 0u;
        reinterpret_cast<HeadCut*>(a.hcut)[h] = hc;
        if (a.glist) a.pub[h] = make_uint4(kNotLarge, 0u, 0u, 0u);   // the cross and resolve kernels skip it
    }
}

// ---- frontiers beyond the LDS keys (n > kLdsKeys candidates per head, at a
// level whose capacity allows it): the select kernel's last workgroup of a head
// published the first digit's crossing bin b0 and the mass still needed in it.
//
// zha_cross_kernel, grid (workgroups per head, H_q), 256 threads: workgroup w
// takes slices w, w + gridDim.x, ... of kCrossSlice positions (four per thread,
// 16-byte loads), counts the head's candidates and its keys below b0 (all of
// them kept), and lists b0's keys {key, position} in LDS; then it reserves
// room in the head's global list with one atomic and copies them there.  A
// list that would pass ZHA_GLIST entries (or a workgroup's LDS) sets the
// overflow word, and the resolve kernel falls back to every key.
constexpr int kCrossThreads = 256;
constexpr int kCrossWaves = kCrossThreads / 64;
constexpr int kCrossSlice = 4 * kCrossThreads;
static_assert(kCrossSlice == 1024, "zha_cross_blocks counts slices of 1024 positions");
constexpr int kCrossLocal = 4096;                 // listed keys a workgroup holds
constexpr int kCrossMaxW = ZHA_CROSS_MAXW;        // workgroups per head (each writes its counts to its own slot)

__global__ __launch_bounds__(kCrossThreads) void zha_cross_kernel(ZhaLevelArgs a, int G, int c) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c));
    __shared__ uint2 s_list[kCrossLocal];
    __shared__ uint32_t s_n, s_base;
    __shared__ uint32_t s_cnt[2][kCrossWaves];
    const int h = blockIdx.y, g = h / G, hl = h - g * G, w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint4 pub = a.pub[h];
    const int pn = parent_count(a, g);
    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kLdsKeys || pub.x == kNotLarge) return;   // (uniform) cut by the select kernel
    const uint32_t b0 = pub.x;
    const float M = __uint_as_float(pub.w);
    const float4* sg4 = reinterpret_cast<const float4*>(a.sig + ((size_t)g * G + hl) * (size_t)a.sstride);
    const int nv_cap = (int)(a.sstride / 4);
    const int nsl = (n + kCrossSlice - 1) / kCrossSlice;
    if (tid == 0) s_n = 0u;
    __syncthreads();
    uint32_t cand = 0, below = 0;
#pragma unroll 1
    for (int sl0 = w; sl0 < nsl; sl0 += 4 * (int)gridDim.x) {
        // up to four slices' scores in flight together
        float4 x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int v = (sl0 + r * (int)gridDim.x) * (kCrossSlice / 4) + tid;
            x[r] = make_float4(zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf());
            if (sl0 + r * (int)gridDim.x < nsl && v < nv_cap) x[r] = sg4[v];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v4[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
            const int p0 = (sl0 + r * (int)gridDim.x) * kCrossSlice + 4 * tid;
            bool in[4];
            uint64_t bal[4];
            uint32_t tot = 0;
            uint32_t k[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                k[j] = p0 + j < n ? key_of(v4[j], M) : kNotCand;
                cand += k[j] != kNotCand;
                below += (k[j] < kNoMass) & ((k[j] >> 21) < b0);
                in[j] = (k[j] < kNoMass) & ((k[j] >> 21) == b0);
                bal[j] = __ballot(in[j]);
                tot += (uint32_t)__popcll(bal[j]);
            }
            if (tot) {                         // uniform over the wave
                uint32_t e0 = 0;
                if (lane == 0) e0 = atomicAdd(&s_n, tot);
                e0 = (uint32_t)__shfl((int)e0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t e = e0 + bits_below_lane(bal[j]);
                    if (in[j] && e < (uint32_t)kCrossLocal) s_list[e] = make_uint2(k[j], (uint32_t)(p0 + j));
                    e0 += (uint32_t)__popcll(bal[j]);
                }
            }
        }
    }
    // the workgroup's counts to its own slot (no atomics on one word from every
    // workgroup), then its room in the head's list (one atomic, when it has keys)
    const uint64_t both = zha_readlane_u64(zha_wave_incl_scan_u64(((uint64_t)below << 32) | cand), 63);
    if (lane == 0) {
        s_cnt[0][wave] = (uint32_t)both;
        s_cnt[1][wave] = (uint32_t)(both >> 32);
    }
    __syncthreads();
    const uint32_t nl = s_n;
    if (tid == 0) {
        uint32_t tc = 0, tb = 0;
#pragma unroll
        for (int i = 0; i < kCrossWaves; ++i) {
            tc += s_cnt[0][i];
            tb += s_cnt[1][i];
        }
        uint4* gc = a.gcnt + h;
        const uint32_t base = nl ? atomicAdd(&gc->x, nl) : 0u;
        if (nl > (uint32_t)kCrossLocal || base + nl > (uint32_t)kGList) atomicOr(&gc->w, 1u);
        a.gpart[(size_t)h * kCrossMaxW + w] = make_uint2(tb, tc);
        s_base = base;
    }
    __syncthreads();
    const uint32_t base = s_base;
    uint2* gl = a.glist + (size_t)h * kGList;
    const uint32_t m = nl < (uint32_t)kCrossLocal ? nl : (uint32_t)kCrossLocal;
    for (uint32_t i = tid; i < m; i += kCrossThreads)
        if (base + i < (uint32_t)kGList) gl[base + i] = s_list[i];
}

// zha_resolve_kernel, grid (H_q), 1024 threads: a large frontier's cut from its
// listed crossing-bin keys (LDS), kept = keys below the bin + listed keys kept;
// after an overflow, or more than kRankMax keys equal to the cut key (the list is
// not in position order), the cut is taken again over every key from the first
// digit's complete histogram.  Writes the head's counts and cut descriptor.
struct PairKey {
    const uint2* e;
    __device__ uint32_t operator()(int i) const { return e[i].x; }
};
struct PairPos {
    const uint2* e;
    __device__ uint32_t operator()(int i) const { return e[i].y; }
};

__global__ __launch_bounds__(kBT) void zha_resolve_kernel(ZhaLevelArgs a, int G, int c, float top_p) {
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c), "s"(top_p));
    __shared__ __align__(16) uint2 s_pairs[kGList];
    __shared__ __align__(16) uint64_t s_hist[kHistBins];
    __shared__ uint2 s_gl[kGather];
    __shared__ uint32_t s_wred[kBW];
    __shared__ CutShared st;
    const int h = blockIdx.x, g = h / G, hl = h - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint4 pub = a.pub[h];
    const uint4 cnt = a.gcnt[h];
    const int pn = parent_count(a, g);
    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kLdsKeys || pub.x == kNotLarge) return;   // (uniform)
    const float M = __uint_as_float(pub.w);
    const uint64_t need = ((uint64_t)pub.z << 32) | pub.y;
    const float* sg = a.sig + ((size_t)g * G + hl) * (size_t)a.sstride;
    // the cross kernel's per-workgroup counts: keys below the crossing bin, candidates
    __shared__ uint32_t s_below, s_cand;
    if (wave == 0) {
        const int nw = zha_cross_blocks(a.cap);
        uint2 v = make_uint2(0u, 0u);
        for (int i = lane; i < nw; i += 64) {
            const uint2 t2 = a.gpart[(size_t)h * kCrossMaxW + i];
            v.x += t2.x;
            v.y += t2.y;
        }
        const uint64_t s2 = zha_readlane_u64(zha_wave_incl_scan_u64(((uint64_t)v.x << 32) | v.y), 63);
        if (lane == 0) {
            s_below = (uint32_t)(s2 >> 32);
            s_cand = (uint32_t)s2;
        }
    }
    __syncthreads();
    const uint32_t below = s_below, ncand = s_cand;
    uint32_t ustar = 0, plim = 0xFFFFFFFFu, kept = 0;
    bool ok = false;
    if (cnt.w == 0u && cnt.x <= (uint32_t)kGList) {
        const int ne = (int)cnt.x;
        const uint2* gl = a.glist + (size_t)h * kGList;
        constexpr int kPer = kGList / kBT;
        uint2 t[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + k * kBT;
            t[k] = make_uint2(kNotCand, 0u);
            if (i < ne) t[k] = gl[i];
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) s_pairs[tid + k * kBT] = t[k];
        __syncthreads();
        ok = block_cut(PairKey{s_pairs}, PairPos{s_pairs}, ne, top_p, need, false, false, s_hist, s_gl, &st, ustar,
                       plim);
        if (ok) {
            uint32_t mine = 0;
#pragma unroll
            for (int k = 0; k < kPer; ++k) mine += kept_by(t[k].x, t[k].y, false, false, ustar, plim);
            mine = (uint32_t)zha_readlane_u64(zha_wave_incl_scan_u64(mine), 63);
            if (lane == 0) s_wred[wave] = mine;
            __syncthreads();
#pragma unroll
            for (int w2 = 0; w2 < kBW; ++w2) kept += s_wred[w2];
            kept += below;
        }
    }
    if (!ok) {
        // every key again, from the first digit's complete histogram
        const uint64_t* gm = a.ghist + (size_t)h * kHistBins;
        s_hist[2 * tid] = gm[2 * tid];
        s_hist[2 * tid + 1] = gm[2 * tid + 1];
        __syncthreads();
        block_cut(GlobKeys{sg, M}, IdPos{}, n, top_p, 0, true, true, s_hist, s_gl, &st, ustar, plim);
        uint32_t mine = 0;
        sweep_keys(GlobKeys{sg, M}, n, [&](uint32_t k, int p) { mine += kept_by(k, (uint32_t)p, false, false, ustar, plim); });
        mine = (uint32_t)zha_readlane_u64(zha_wave_incl_scan_u64(mine), 63);
        __syncthreads();
        if (lane == 0) s_wred[wave] = mine;
        __syncthreads();
        kept = 0;
#pragma unroll
        for (int w2 = 0; w2 < kBW; ++w2) kept += s_wred[w2];
    }
    if (tid == 0) {
        a.stats[2 * h + 0] = (int32_t)ncand;
        a.stats[2 * h + 1] = (int32_t)kept;
        HeadCut hc;
        hc.m = M;
        hc.ustar = ustar;
        hc.plim = plim;
        hc.mode = 0u;
        reinterpret_cast<HeadCut*>(a.hcut)[h] = hc;
    }
}

// MG: the largest group the launch serves (8 or ZHA_MAX_GROUP): the per-head
// registers of a 1024-thread workgroup stay within its register budget at G <= 8.
template <int kApplyThreads, bool BITS, int MG = ZHA_MAX_GROUP>
__global__ __launch_bounds__(kApplyThreads) void zha_apply_kernel(ZhaLevelArgs a, int G, int c) {
    constexpr int kApplyWaves = kApplyThreads / 64;
    constexpr int kApplyChunk = 4 * kApplyThreads;    // positions per apply workgroup (four per thread)
    ZHA_LEVEL_ARGS_READY(a, "s"(G), "s"(c));
    __shared__ uint32_t s_wc[kApplyWaves];
    __shared__ uint32_t s_ticket, s_prefix;
    __shared__ HeadCut s_hc[ZHA_MAX_GROUP];
    const int g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the first kApplyEarly workgroups of a group draw their ticket in the parent
    // count's round trip (one that then finds nothing to do leaves with it: later
    // tickets only run past the chunks); the others first learn the chunk count and
    // draw one only when a chunk is left for them, so a wide level's idle workgroups
    // add no atomics on the group's ticket word.  Every ticket drawn below the chunk
    // count belongs to a running workgroup, so the look-back waits always end.
    const bool early = blockIdx.x < kApplyEarly;
    if (early && tid == 0) s_ticket = atomicAdd(&a.tick[g], 1u);
    const int pn = parent_count(a, g);
    const int n = a.top ? (int)a.n_top : pn * c + (int)(a.orph_hi - a.orph_lo);
    if (n <= kSmallN) return;                  // the select kernel wrote the kept list
    const int nch = (n + kApplyChunk - 1) / kApplyChunk;
    if (!early) {
        if ((int)blockIdx.x >= nch) return;
        if (tid == 0) s_ticket = atomicAdd(&a.tick[g], 1u);
    }
    __syncthreads();
    const int ci = (int)s_ticket;
    if (ci >= nch) return;
    const int p0 = ci * kApplyChunk + 4 * tid;
    const int pnc = a.top ? 0 : pn * c;
    int32_t pk[4];
    uint32_t msk[4] = {0u, 0u, 0u, 0u};
    if constexpr (BITS) {
        // the heads' kept bitmaps over positions (written by the select kernel): bits
        // p0 .. p0 + 3 of word p0 / 64 of every head, with the parents' kept entries
        // of the thread's positions, in one round trip
        const int wd = (p0 < n ? p0 : 0) >> 6;
        uint64_t hw[MG];
#pragma unroll
        for (int hh = 0; hh < MG; ++hh) {
            hw[hh] = 0ull;
            if (hh < G) hw[hh] = a.kbm[((size_t)g * G + hh) * (size_t)a.wcap + wd];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = p0 + j;
            pk[j] = 0;
            if (p < pnc) pk[j] = a.pklist[(size_t)g * a.pcap + zha_div((uint32_t)p, a.dc)];
        }
#pragma unroll
        for (int hh = 0; hh < MG; ++hh)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                msk[j] |= (uint32_t)(p0 + j < n ? (hw[hh] >> ((p0 + j) & 63)) & 1ull : 0ull) << hh;
    } else {
        // the heads' cuts (to LDS, one thread each) and the chunk's scores, positions
        // p0 .. p0 + 3 of this thread for every head as one 16-byte load each (rows are
        // 16-byte aligned; the vector holding position n - 1 may run past n, never past
        // the row), all in flight together; scores of heads beyond G come from a valid
        // row and are masked afterwards
        const HeadCut mine = reinterpret_cast<const HeadCut*>(a.hcut)[(size_t)g * G + (tid < G ? tid : 0)];
        const int pv = p0 < n ? p0 : 0;
        float4 x[MG];
#pragma unroll
        for (int hh = 0; hh < MG; ++hh)
            x[hh] = *reinterpret_cast<const float4*>(a.sig + ((size_t)g * G + (hh < G ? hh : 0)) * a.sstride + pv);
        // the parents' kept entries of the thread's positions, in the same round trip
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = p0 + j;
            pk[j] = 0;
            if (p < pnc) pk[j] = a.pklist[(size_t)g * a.pcap + zha_div((uint32_t)p, a.dc)];
        }
        if (tid < G) s_hc[tid] = mine;
        __syncthreads();
        // every head's cut read from LDS at once, then the masks without branches
        HeadCut hcs[MG];
#pragma unroll
        for (int hh = 0; hh < MG; ++hh) hcs[hh] = s_hc[hh < G ? hh : 0];
#pragma unroll
        for (int hh = 0; hh < MG; ++hh) {
            const HeadCut& hc = hcs[hh];
            const float v[4] = {x[hh].x, x[hh].y, x[hh].z, x[hh].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = p0 + j < n ? key_of(v[j], hc.m) : kNotCand;
                const bool k = (hh < G) & kept_by(key, (uint32_t)(p0 + j), hc.mode == 2u, hc.mode == 1u, hc.ustar, hc.plim);
                msk[j] |= (uint32_t)k << hh;
            }
        }
    }
    // the chunk's kept positions in order (4 per thread, thread-major): this
    // thread's count, the wave's inclusive scan, the waves' counts
    const uint32_t mine_cnt = (msk[0] != 0u) + (msk[1] != 0u) + (msk[2] != 0u) + (msk[3] != 0u);
    const uint32_t inc = (uint32_t)zha_wave_incl_scan_u64(mine_cnt);
    if (lane == 63) s_wc[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        // the chunk's count (wave prefixes into s_wc), published; then the
        // predecessors' descriptors, read by wave 0's lanes together (lane j reads
        // chunk ci - 1 - j, 64 at a time, again while any of them has not
        // published): the sum up to the nearest published inclusive prefix
        uint32_t wcnt = lane < kApplyWaves ? s_wc[lane] : 0u;
        uint64_t ctot;
        const uint32_t wex = (uint32_t)wave_excl_scan_u64(wcnt, &ctot);
        if (lane < kApplyWaves) s_wc[lane] = wex;
        const uint32_t cnt = (uint32_t)ctot;
        uint32_t* desc = a.desc + (size_t)g * a.ndesc;
        if (lane == 0)
            __hip_atomic_store(desc + ci, (ci == 0 ? kDescInc : kDescAgg) | cnt, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        uint32_t prefix = 0;
        int top = ci - 1;                      // nearest predecessor not yet summed
        uint32_t spins = 0;
        while (top >= 0) {                     // uniform
            const int j = top - lane;
            uint32_t d = j >= 0 ? __hip_atomic_load(desc + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kDescInc;
            // lanes up to the first inclusive prefix (or the first unpublished chunk)
            const uint64_t inc_b = __ballot((d & kDescInc) != 0u);
            const uint64_t none_b = __ballot((d & (kDescInc | kDescAgg)) == 0u);
            const int first_inc = inc_b ? __ffsll((long long)inc_b) - 1 : 64;
            const int first_none = none_b ? __ffsll((long long)none_b) - 1 : 64;
            const int upto = min(first_inc, first_none);       // lanes [0, upto) are aggregates
            uint32_t v = lane < upto ? (d & kDescVal) : 0u;
            if (first_inc < first_none && lane == first_inc) v = d & kDescVal;
            uint64_t vt;
            wave_excl_scan_u64(v, &vt);
            prefix += (uint32_t)vt;
            if (first_inc < first_none) break;                 // reached an inclusive prefix (or chunk 0)
            top -= upto;                                       // continue below the summed aggregates
            if (first_none < 64) {
                if (++spins > kSpinMax) break;                 // not reached: those chunks started before this one
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            if (ci > 0)
                __hip_atomic_store(desc + ci, kDescInc | (prefix + cnt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_prefix = prefix;
            if (ci == nch - 1) a.nkept[g] = (int32_t)(prefix + cnt);
        }
    }
    __syncthreads();
    uint32_t r = s_prefix + s_wc[wave] + inc - mine_cnt;
    int32_t* kl = a.klist + (size_t)g * a.cap;
    uint32_t* km = a.kmask + (size_t)g * a.cap;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (msk[j]) {
            const int p = p0 + j;
            int32_t node;
            if (a.top) node = p;
            else if (p < pnc) node = pk[j] * c + (p - (int)zha_div((uint32_t)p, a.dc) * c);
            else node = (int32_t)a.orph_lo + (p - pnc);
            kl[r] = node;
            km[r] = msk[j];
            ++r;
        }
    }
}

}  // namespace

#ifndef ZHA_SCORE_CAP
#define ZHA_SCORE_CAP 192
#endif
int zha_score_blocks(int64_t max_cand, int R) {
    const int64_t U = R <= 16 ? 16 / R : 1;
    const int64_t items = (max_cand + U - 1) / U;
    int64_t blocks = (items + 3) / 4;        // one item per wave
    if (blocks < 1) blocks = 1;
    if (blocks > ZHA_SCORE_CAP) blocks = ZHA_SCORE_CAP;
    return (int)blocks;
}

// LDS of a score kernel that derives the chain's last level's kept list (n nodes).
size_t zha_defer_lds_bytes(int G, int64_t n) {
    const size_t wc = (size_t)((n + 63) / 64);
    return sizeof(uint64_t) * (size_t)(G + 1) * wc + sizeof(uint32_t) * wc;
}

// A launch of kernel template K<bf16 q, plane format> picked by the cache and plane formats.
#define ZHA_SCORE_LAUNCH_PF(K, BQ, grid, lds, stream, pf, ...)                                              \
    do {                                                                                                     \
        if (pf == 2)                                                                                         \
            hipLaunchKernelGGL((K<BQ, 2>), grid, dim3(kScoreThreads), lds, stream, __VA_ARGS__);             \
        else if (pf == 1)                                                                                    \
            hipLaunchKernelGGL((K<BQ, 1>), grid, dim3(kScoreThreads), lds, stream, __VA_ARGS__);             \
        else                                                                                                 \
            hipLaunchKernelGGL((K<BQ, 0>), grid, dim3(kScoreThreads), lds, stream, __VA_ARGS__);             \
    } while (0)
#define ZHA_SCORE_LAUNCH(K, grid, lds, stream, pf, ...)                                                    \
    do {                                                                                                     \
        if (kv_dtype == 0)                                                                                   \
            ZHA_SCORE_LAUNCH_PF(K, true, grid, lds, stream, pf, __VA_ARGS__);                                \
        else                                                                                                 \
            ZHA_SCORE_LAUNCH_PF(K, false, grid, lds, stream, pf, __VA_ARGS__);                               \
    } while (0)

// The plane format a level's arguments ask for: 2 with an 8-bit copy, 1 with a
// bfloat16 copy, else 0 (the float32 planes).
static int plane_format_of(const ZhaLevelArgs& a) { return a.S8 ? 2 : a.S16 ? 1 : 0; }

hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream, const ZhaLevelArgs* defer) {
    dim3 grid((unsigned)blocks, (unsigned)H_kv);
    const int pf = plane_format_of(a);
    if (defer) {
        if (a.top || !defer->top || defer->n_top > ZHA_CHAIN_SLOTS) return hipErrorInvalidValue;
        const size_t lds = zha_defer_lds_bytes(G, defer->n_top);
        if (a.sigN) {
            // the candidates' scores copied from the node-indexed ones (planes unread)
            if (kv_dtype == 0)
                hipLaunchKernelGGL((zha_route_score_defer_kernel<true, 0, true>), grid, dim3(kScoreThreads), lds,
                                   stream, q, a, *defer, G, c, R, tau);
            else
                hipLaunchKernelGGL((zha_route_score_defer_kernel<false, 0, true>), grid, dim3(kScoreThreads), lds,
                                   stream, q, a, *defer, G, c, R, tau);
            return hipGetLastError();
        }
        ZHA_SCORE_LAUNCH(zha_route_score_defer_kernel, grid, lds, stream, pf, q, a, *defer, G, c, R, tau);
        return hipGetLastError();
    }
    ZHA_SCORE_LAUNCH(zha_route_score_kernel, grid, 0, stream, pf, q, a, G, c, R, tau);
    return hipGetLastError();
}

hipError_t zha_launch_score_all(int kv_dtype, const void* q, const ZhaChainArgs& m, int H_kv, int G, int c, int R,
                                float tau, hipStream_t stream) {
    int bmax = 1;
    for (int i = 0; i < m.n; ++i) bmax = std::max(bmax, m.blocks[i]);
    const dim3 grid((unsigned)bmax, (unsigned)H_kv, (unsigned)m.n);
    const int pf = plane_format_of(m.lv[0]);
    ZHA_SCORE_LAUNCH(zha_route_score_all_kernel, grid, 0, stream, pf, q, m, G, c, R, tau);
    return hipGetLastError();
}

hipError_t zha_launch_chain(int kv_dtype, const ZhaChainSel& m, int H_kv, int G, int c, float top_p,
                            hipStream_t stream) {
    for (int i = 0; i < m.n; ++i)
        if (m.lv[i].n_nodes > kChainSlots) return hipErrorInvalidValue;
    if (m.nsel != H_kv * G || m.spec_blocks < 0 || (m.spec_blocks > 0 && (!m.spec.sig || !m.q))) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(H_kv * G + H_kv * m.spec_blocks));
    const int pf = m.spec_blocks > 0 ? plane_format_of(m.spec) : 0;
#define ZHA_CHAIN_LAUNCH(BQ)                                                                                  \
    do {                                                                                                     \
        if (pf == 2) hipLaunchKernelGGL((zha_chain_kernel<BQ, 2>), grid, dim3(kBT), 0, stream, m, G, c, top_p); \
        else if (pf == 1) hipLaunchKernelGGL((zha_chain_kernel<BQ, 1>), grid, dim3(kBT), 0, stream, m, G, c, top_p); \
        else hipLaunchKernelGGL((zha_chain_kernel<BQ, 0>), grid, dim3(kBT), 0, stream, m, G, c, top_p);      \
    } while (0)
    if (kv_dtype == 0) ZHA_CHAIN_LAUNCH(true);
    else ZHA_CHAIN_LAUNCH(false);
#undef ZHA_CHAIN_LAUNCH
    return hipGetLastError();
}

hipError_t zha_launch_merge_ids(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream) {
    if (a.n_top > kChainSlots) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zha_merge_ids_kernel, dim3((unsigned)H_kv), dim3(kBT), 0, stream, a, G, c);
    return hipGetLastError();
}

hipError_t zha_launch_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream) {
    if (!a.hblk || !a.hcut || !a.tick || !a.desc || !a.ghist || !a.hdone) return hipErrorInvalidValue;
    // slices of kSlice positions, at most kSliceW per head (one slice: one workgroup
    // per head selects alone; a frontier of several slices is histogrammed by them
    // first, measured faster than one workgroup building the histogram itself)
    int64_t w = (a.cap + kSlice - 1) / kSlice;
    if (w > kSliceW) w = kSliceW;
    if (w < 1) w = 1;
    hipLaunchKernelGGL(zha_select_kernel, dim3((unsigned)w, (unsigned)(H_kv * G)), dim3(kBT), 0, stream, a, G, c,
                       top_p);
    return hipGetLastError();
}

hipError_t zha_launch_apply(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream) {
    if (!a.hcut || !a.tick || !a.desc) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.ndesc, (unsigned)H_kv);
    // without the cross launch every head's kept bitmap was written by the select kernel
    const bool bits = a.glist == nullptr;
    if (apply_threads(a.cap) == 1024) {
        if (bits) hipLaunchKernelGGL((zha_apply_kernel<1024, true>), grid, dim3(1024), 0, stream, a, G, c);
        else if (G <= 8) hipLaunchKernelGGL((zha_apply_kernel<1024, false, 8>), grid, dim3(1024), 0, stream, a, G, c);
        else hipLaunchKernelGGL((zha_apply_kernel<1024, false>), grid, dim3(1024), 0, stream, a, G, c);
    } else {
        if (bits) hipLaunchKernelGGL((zha_apply_kernel<256, true>), grid, dim3(256), 0, stream, a, G, c);
        else hipLaunchKernelGGL((zha_apply_kernel<256, false>), grid, dim3(256), 0, stream, a, G, c);
    }
    return hipGetLastError();
}

hipError_t zha_launch_cross(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream) {
    if (!a.pub || !a.gcnt || !a.glist || !a.gpart) return hipErrorInvalidValue;
    const int w = zha_cross_blocks(a.cap);
    hipLaunchKernelGGL(zha_cross_kernel, dim3((unsigned)w, (unsigned)(H_kv * G)), dim3(kCrossThreads), 0, stream, a,
                       G, c);
    return hipGetLastError();
}

hipError_t zha_launch_resolve(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream) {
    if (!a.pub || !a.gcnt || !a.glist || !a.gpart || !a.hcut || !a.ghist) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zha_resolve_kernel, dim3((unsigned)(H_kv * G)), dim3(kBT), 0, stream, a, G, c, top_p);
    return hipGetLastError();
}

int zha_apply_chunks(int64_t cap) {
    const int64_t chunk = 4 * apply_threads(cap);
    return (int)((cap + chunk - 1) / chunk);
}
