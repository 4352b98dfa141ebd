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
// Selection runs one 1024-thread workgroup per query head.  Probabilities are
// handled as 2^40-scaled integers e_i = exp(sigma_i - max) so that every sum
// is exact and order-free (bitwise-reproducible).  Candidates are ranked by
// delta_i = max - sigma_i quantised to 2^-27 (monotone in sigma), located by a
// three-pass mass-weighted radix select (11 + 11 + 10 bits); candidates whose
// quantised delta equals the cut's are taken in ascending position (= node)
// order until the cumulative mass reaches ceil(p * sum e).  Each head writes
// its kept flags as a bitmap (one wave ballot per 64 positions, no atomics);
// the last head of the group to finish ORs the group's bitmaps into the kept
// list and writes the next level's candidates (children of kept nodes, then
// that level's orphans), so the next score kernel reaches its planes in one
// dependent load.
#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kScoreThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr float kFix = 1099511627776.0f;   // 2^40: fixed-point scale of e_i in [0, 1]
constexpr float kKeyScale = 134217728.0f;  // 2^27: delta quantum
constexpr float kDeltaMax = 32.0f;         // e^-32 * 2^40 < 1: heavier deltas carry no mass

__device__ __forceinline__ uint32_t all_heads(int G) { return G >= 32 ? 0xFFFFFFFFu : ((1u << G) - 1u); }

// grid (blocks, H_kv), 256 threads.  Each wave scores items of U = 16/R
// candidates (R <= 16) or one candidate over R/16 column blocks (R > 16).
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void zha_route_score_kernel(const void* __restrict__ q,
                                                                        ZhaLevelArgs a, int G, int c, int R,
                                                                        float tau) {
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kq = lane >> 4;
    const int U = R <= 16 ? 16 / R : 1;
    const int CB = R <= 16 ? 1 : R / 16;
    const int span = R <= 16 ? R : 16;
    const int cl = R <= 16 ? j / R : 0;
    const uint32_t allg = all_heads(G);
    const size_t lrow = (size_t)g * a.cap;

    // first item's candidate fetched together with the candidate count
    int64_t it = (int64_t)blockIdx.x * 4 + wave;
    int32_t node0 = 0;
    uint32_t mask0 = allg;
    if (!a.top) {
        const int64_t p0 = it * U + cl;
        if (p0 < a.cap) {
            node0 = a.cand_node[lrow + p0];
            mask0 = a.cand_mask[lrow + p0];
        }
    }
    const int64_t n_cand = a.top ? a.n_top : (int64_t)a.ncand[g];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (a.top) a.ncand[g] = (int32_t)n_cand;
        a.done[g] = 0;
    }
    // A operand: row = query head j of the group, contraction index d = 16m + 4kq + e.
    float qa[32];
    if (j < G) {
        if (BF16) {
            const uint16_t* qr = static_cast<const uint16_t*>(q) + ((size_t)g * G + j) * ZHA_D + 4 * kq;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint2 v = *reinterpret_cast<const uint2*>(qr + 16 * m);
                qa[4 * m + 0] = zha_bf16_to_f32(v.x & 0xFFFFu);
                qa[4 * m + 1] = zha_bf16_to_f32(v.x >> 16);
                qa[4 * m + 2] = zha_bf16_to_f32(v.y & 0xFFFFu);
                qa[4 * m + 3] = zha_bf16_to_f32(v.y >> 16);
            }
        } else {
            const float* qr = static_cast<const float*>(q) + ((size_t)g * G + j) * ZHA_D + 4 * kq;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float4 v = *reinterpret_cast<const float4*>(qr + 16 * m);
                qa[4 * m + 0] = v.x; qa[4 * m + 1] = v.y; qa[4 * m + 2] = v.z; qa[4 * m + 3] = v.w;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) qa[k] = 0.f;
    }

    const int64_t items = (n_cand + U - 1) / U;
    bool first = true;
    for (; it < items; it += (int64_t)gridDim.x * 4) {
        const int64_t pos = it * U + cl;
        const bool valid = pos < n_cand;
        int64_t node = 0;
        uint32_t cm = 0;
        if (valid) {
            if (a.top) {
                node = pos;
                cm = allg;
            } else if (first) {
                node = node0;
                cm = mask0;
            } else {
                node = a.cand_node[lrow + pos];
                cm = a.cand_mask[lrow + pos];
            }
        }
        first = false;
        float best[4] = {zha_neg_inf(), zha_neg_inf(), zha_neg_inf(), zha_neg_inf()};
        for (int cb = 0; cb < CB; ++cb) {
            const int r = R <= 16 ? (j % R) : (cb * 16 + j);
            const size_t prow = (lrow + (size_t)node) * R + r;
            float4 sv[8];
            if (valid) {
                const float4* plane = reinterpret_cast<const float4*>(a.S + prow * ZHA_D);
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = plane[4 * m + kq];
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) sv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            const float bv = valid ? a.B[prow] : zha_neg_inf();
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
    }
}

// ---- selection helpers (kSelThreads threads, one wave does the scans)

// Exclusive prefix sum across one wave (all lanes active); *total gets the wave sum.
__device__ __forceinline__ uint64_t wave_excl_scan_u64(uint64_t v, uint64_t* total) {
    const uint64_t x = zha_wave_incl_scan_u64(v);
    *total = zha_readlane_u64(x, 63);
    return x - v;
}

// Run by one whole wave: the bin b with before(b) < need <= before(b) + hist[b]
// (before(b) = sum of bins < b) goes to *out_bin / *out_before.  When `need`
// is 0 it is first set to ceil(p * total) (clamped to [1, total]).
template <int NBINS>
__device__ void wave_find_cross(const uint64_t* hist, uint64_t need, float top_p, int* out_bin,
                                uint64_t* out_before, uint64_t* out_need) {
    constexpr int per = NBINS / 64;
    const int lane = threadIdx.x & 63;
    const int b0 = lane * per;
    uint64_t mine = 0;
#pragma unroll 8
    for (int i = 0; i < per; ++i) mine += hist[b0 + i];
    uint64_t total;
    uint64_t before = wave_excl_scan_u64(mine, &total);
    if (need == 0) {
        uint64_t T = (uint64_t)ceil((double)top_p * (double)total);
        if (T < 1) T = 1;
        if (T > total) T = total;
        need = T;
    }
    if (before < need && before + mine >= need) {          // the crossing bin is one of this lane's
#pragma unroll 1
        for (int i = 0; i < per; ++i) {
            const uint64_t hb = hist[b0 + i];
            if (before + hb >= need) {
                *out_bin = b0 + i;
                *out_before = before;
                *out_need = need;
                break;
            }
            before += hb;
        }
    }
}

__device__ __forceinline__ uint64_t fixed_mass(float delta) { return (uint64_t)(__expf(-delta) * kFix); }
__device__ __forceinline__ uint32_t delta_key(float delta) { return (uint32_t)(delta * kKeyScale); }

// Selection keys: the quantised delta of a candidate that carries mass, or one
// of two sentinels.  A candidate's fixed-point mass is a function of its key
// alone, so every pass sees exactly the same masses.
constexpr uint32_t kNotCand = 0xFFFFFFFFu;    // not this head's candidate
constexpr uint32_t kNoMass = 0xFFFFFFFEu;     // candidate with delta >= kDeltaMax (mass 0)
constexpr int kLdsKeys = 16384;               // heads with at most this many candidates stage keys in LDS

__device__ __forceinline__ uint32_t key_of(float s, float m) {
    if (s == zha_neg_inf()) return kNotCand;
    const float dl = m - s;
    return dl < kDeltaMax ? delta_key(dl) : kNoMass;
}

__device__ __forceinline__ uint64_t mass_of(uint32_t key) {
    // e^{-delta} with delta = key * 2^-27, as 2^40-scaled fixed point
    return (uint64_t)(exp2f(-(float)key * (1.4426950408889634f / kKeyScale)) * kFix);
}

constexpr int kSmallN = 1024;   // groups with at most this many candidates select in one workgroup
constexpr int kSmallK = kSmallN / 64;
static_assert(ZHA_MAX_GROUP * kSmallN <= 16384, "small-path scores must fit the key buffer");
static_assert(ZHA_MAX_GROUP * 256 <= 2 * 2048, "small-path histograms must fit the histogram buffers");

// One wave selects for query head (g, hl) among n <= kSmallN candidates whose
// scores are in LDS (sg); position lane + 64k sits in register slot k.  8-bit
// digits, wave-local histograms (hist: 256 u64, cntb: 256 u32), no workgroup
// barrier.  The kept bitmap words go to kw[0 .. nk).
__device__ void select_head_wave(const float* sg, int64_t n, float top_p, uint64_t* hist, uint32_t* cntb,
                                 uint64_t* kw, uint32_t* n_cand_out, uint32_t* n_kept_out) {
    constexpr int K = kSmallK;
    const int lane = threadIdx.x & 63;
    const int nk = (int)((n + 63) / 64);
    float sv[K];
    float m = zha_neg_inf();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t pos = lane + 64 * k;
        sv[k] = (pos < n) ? sg[pos] : zha_neg_inf();
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
#pragma unroll
            for (int i = 0; i < 4; ++i) { hist[lane * 4 + i] = 0; cntb[lane * 4 + i] = 0; }
            zha_wave_lds_sync();
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (k < nk && key[k] < kNoMass && (pass == 0 || (key[k] >> (shift + 8)) == prefix)) {
                    const uint32_t b = (key[k] >> shift) & 255u;
                    atomicAdd((unsigned long long*)&hist[b], (unsigned long long)mass_of(key[k]));
                    atomicAdd(&cntb[b], 1u);
                }
            }
            zha_wave_lds_sync();
            uint64_t hb[4], mine = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { hb[i] = hist[lane * 4 + i]; mine += hb[i]; }
            uint64_t total;
            uint64_t before = wave_excl_scan_u64(mine, &total);
            if (pass == 0) {
                uint64_t T = (uint64_t)ceil((double)top_p * (double)total);
                need = T < 1 ? 1 : (T > total ? total : T);
            }
            int my_bin = -1;
            uint64_t my_before = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (before < need && before + hb[i] >= need && my_bin < 0) { my_bin = lane * 4 + i; my_before = before; }
                before += hb[i];
            }
            const uint64_t found = __ballot(my_bin >= 0);
            const int src = __ffsll((long long)found) - 1;
            const uint32_t bin = (uint32_t)__shfl(my_bin, src, 64);
            need -= zha_readlane_u64(my_before, src);
            prefix = (prefix << 8) | bin;
            if (pass == 3) { ustar = prefix; ties = cntb[bin]; }
            zha_wave_lds_sync();
        }
    }
    uint32_t n_cand = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool cand = k < nk && key[k] != kNotCand;
        const bool kept = !none && (keep_all ? cand : (cand && key[k] < kNoMass && (key[k] < ustar || (key[k] == ustar && ties == 1))));
        const uint64_t wk = __ballot(kept);
        n_cand += __popcll(__ballot(cand));
        if (lane == 0 && k < nk) kw[k] = wk;
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
            if (lane == 0 && k < nk) kw[k] |= extra;
            run += tot;
        }
        zha_wave_lds_sync();
    }
    uint32_t n_kept = 0;
#pragma unroll 1
    for (int k = 0; k < nk; ++k) n_kept += __popcll(kw[k]);
    *n_cand_out = n_cand;
    *n_kept_out = n_kept;
}

// grid (H_q), 1024 threads: one query head per workgroup; the last head of a
// group to finish writes the group's kept list and the next level's candidates.
// Keys sit in LDS (kLdsKeys candidates) or are recomputed from the scores on
// every pass for larger frontiers; all passes are rolled loops.
__global__ __launch_bounds__(kSelThreads) void zha_route_select_kernel(ZhaLevelArgs a, int G, int c,
                                                                       float top_p) {
    __shared__ uint32_t keys[kLdsKeys];                 // also: small-path scores [G][kSmallN]
    __shared__ uint64_t histbuf[2][2048];               // also: small-path histograms [G][256]
    __shared__ uint32_t cntbuf[2][2048];                // also: small-path counts [G][256]
    __shared__ int32_t s_nid[kSmallN];
    __shared__ uint64_t s_kw[ZHA_MAX_GROUP * kSmallK];
    __shared__ float swf[kSelWaves];
    __shared__ int s_bin;
    __shared__ uint64_t s_before, s_need, s_run;
    __shared__ uint32_t s_cnt[2];
    __shared__ int s_last;

    const int h = blockIdx.x, g = h / G, hl = h - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t lrow = (size_t)g * a.cap;
    // Small frontiers: the group's first workgroup selects for all G heads (one wave
    // each) and merges from LDS.  Scores and node ids of the first kSmallN positions
    // are fetched together with the candidate count.
    float* s_sig = reinterpret_cast<float*>(keys);                        // [G][kSmallN]
    int64_t n;
    if (a.top) {
        n = a.n_top;
    } else {
        const int32_t nc = a.ncand[g];
        const int32_t nd = tid < a.cap ? a.cand_node[lrow + tid] : 0;
        n = nc;
        if (n <= kSmallN && hl == 0) s_nid[tid] = nd;
    }
    if (n <= kSmallN) {
        if (hl != 0) return;                       // the same decision for every head of the group
        for (int i = tid; i < G * kSmallN; i += kSelThreads) {
            const int hh = i / kSmallN, pos = i - hh * kSmallN;
            s_sig[i] = pos < n ? a.sig[((size_t)g * G + hh) * a.cap + pos] : zha_neg_inf();
        }
        __syncthreads();
        uint64_t* kw = s_kw;                                              // [G][kSmallK]
        if (wave < G) {
            uint32_t nc_h, nk_h;
            select_head_wave(s_sig + wave * kSmallN, n, top_p, &histbuf[0][0] + wave * 256,
                             &cntbuf[0][0] + wave * 256, kw + wave * kSmallK, &nc_h, &nk_h);
            if (lane == 0) {
                a.stats[2 * (g * G + wave) + 0] = (int32_t)nc_h;
                a.stats[2 * (g * G + wave) + 1] = (int32_t)nk_h;
            }
            for (int k = lane; k < (int)((n + 63) / 64); k += 64)
                a.kbm[((size_t)g * G + wave) * a.wcap + k] = kw[wave * kSmallK + k];
        }
        __syncthreads();
        if (wave != 0) return;
        // merge the heads' kept words: kept list and the next level's candidates
        const int nk = (int)((n + 63) / 64);
        const size_t nrow = (size_t)g * a.next_cap;
        const uint64_t lt = (1ull << lane) - 1ull;
        uint64_t run = 0;
#pragma unroll 1
        for (int k = 0; k < nk; ++k) {
            uint64_t u = 0;
#pragma unroll 1
            for (int hh = 0; hh < G; ++hh) u |= kw[hh * kSmallK + k];
            if ((u >> lane) & 1ull) {
                const uint64_t rank = run + __popcll(u & lt);
                uint32_t msk = 0;
#pragma unroll 1
                for (int hh = 0; hh < G; ++hh) msk |= (uint32_t)((kw[hh * kSmallK + k] >> lane) & 1ull) << hh;
                const int64_t pos = lane + 64 * k;
                const int32_t node = a.top ? (int32_t)pos : s_nid[pos];
                a.klist[lrow + rank] = node;
                a.kmask[lrow + rank] = msk;
                if (a.next_node) {
#pragma unroll 1
                    for (int i = 0; i < c; ++i) {
                        a.next_node[nrow + rank * c + i] = node * c + i;
                        a.next_mask[nrow + rank * c + i] = msk;
                    }
                }
            }
            run += __popcll(u);
        }
        if (a.next_node) {
            const uint32_t allg = all_heads(G);
            const int64_t n_orph = a.orph_hi - a.orph_lo;
            for (int64_t o = lane; o < n_orph; o += 64) {
                a.next_node[nrow + run * c + o] = (int32_t)(a.orph_lo + o);
                a.next_mask[nrow + run * c + o] = allg;
            }
            if (lane == 0) a.next_ncand[g] = (int32_t)(run * c + n_orph);
        }
        if (lane == 0) a.nkept[g] = (int32_t)run;
        return;
    }
    const float* sg = a.sig + ((size_t)g * G + hl) * a.cap;
    uint64_t* bm = a.kbm + ((size_t)g * G + hl) * a.wcap;
    const int64_t nwords = (n + 63) / 64;
    const bool staged = n <= kLdsKeys;

    if (tid < 2) s_cnt[tid] = 0;
    float m = zha_neg_inf();
#pragma unroll 4
    for (int64_t pos = tid; pos < n; pos += kSelThreads) {
        const float s = sg[pos];
        m = fmaxf(m, s);
        if (staged) keys[pos] = __float_as_uint(s);        // raw score until the max is known
    }
    m = zha_wave_max(m);
    if (lane == 0) swf[wave] = m;
    __syncthreads();
    m = swf[0];
    for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, swf[w]);
    if (staged) {
#pragma unroll 2
        for (int64_t pos = tid; pos < n; pos += kSelThreads) keys[pos] = key_of(__uint_as_float(keys[pos]), m);
    }

    // Kept rule: keep_all, or key < ustar, or key == ustar when that key is unique.
    const bool none = m == zha_neg_inf();        // this head has no candidate at this level
    const bool keep_all = !none && top_p >= 1.0f;
    uint32_t ustar = 0, ties = 0;
    uint64_t need = 0;
    if (!none && !keep_all) {
        // digits of the key: bits 31..21, 20..10, 9..0; pass p counts into buffer p & 1
        // while the other buffer is cleared for pass p + 1
        uint32_t mshift = 32, mval = 0, bshift = 21, bmask = 2047;
        for (int i = tid; i < 2048; i += kSelThreads) { histbuf[0][i] = 0; cntbuf[0][i] = 0; }
        __syncthreads();
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            uint64_t* hist = histbuf[pass & 1];
            uint32_t* cntb = cntbuf[pass & 1];
            for (int i = tid; i < 2048; i += kSelThreads) { histbuf[(pass + 1) & 1][i] = 0; cntbuf[(pass + 1) & 1][i] = 0; }
#pragma unroll 2
            for (int64_t pos = tid; pos < n; pos += kSelThreads) {
                const uint32_t key = staged ? keys[pos] : key_of(sg[pos], m);
                if (key < kNoMass && (uint32_t)((uint64_t)key >> mshift) == mval) {
                    const uint32_t b = (key >> bshift) & bmask;
                    atomicAdd((unsigned long long*)&hist[b], (unsigned long long)mass_of(key));
                    atomicAdd(&cntb[b], 1u);
                }
            }
            __syncthreads();
            if (wave == 0) wave_find_cross<2048>(hist, need, top_p, &s_bin, &s_before, &s_need);
            __syncthreads();
            const uint32_t bin = (uint32_t)s_bin;
            need = s_need - s_before;            // mass still needed inside this bin
            if (pass == 0) { mshift = 21; mval = bin; bshift = 10; bmask = 2047; }
            else if (pass == 1) { mshift = 10; mval = (mval << 11) | bin; bshift = 0; bmask = 1023; }
            else { ustar = (mval << 10) | bin; ties = cntb[bin]; }
        }
    }
    const uint64_t need_tie = need;

    // kept flags -> this head's bitmap, one ballot per 64 positions
    uint32_t my_cand = 0, my_kept = 0;
#pragma unroll 2
    for (int64_t base = 0; base < n; base += kSelThreads) {
        const int64_t pos = base + tid;
        const uint32_t key = pos < n ? (staged ? keys[pos] : key_of(sg[pos], m)) : kNotCand;
        const bool cand = key != kNotCand;
        const bool kept = !none && (keep_all ? cand : (key < kNoMass && (key < ustar || (key == ustar && ties == 1))));
        const uint64_t word = __ballot(kept);
        const int64_t wi = base / 64 + wave;
        if (lane == 0 && wi < nwords) bm[wi] = word;
        my_cand += cand;
        my_kept += kept;
    }
    if (!none && !keep_all && ties > 1) {
        // several candidates share the cut key: take them in ascending position order
        __syncthreads();
        __threadfence();
        if (tid == 0) s_run = 0;
#pragma unroll 1
        for (int64_t base = 0; base < n; base += kSelThreads) {
            const int64_t pos = base + tid;
            const uint32_t key = pos < n ? (staged ? keys[pos] : key_of(sg[pos], m)) : kNotCand;
            const uint64_t w = key == ustar ? mass_of(key) : 0ull;
            uint64_t wt;
            const uint64_t ex = wave_excl_scan_u64(w, &wt);
            __syncthreads();
            if (lane == 0) histbuf[1][wave] = wt;
            __syncthreads();
            uint64_t before = s_run;
            for (int ww = 0; ww < wave; ++ww) before += histbuf[1][ww];
            uint64_t tot = 0;
            for (int ww = 0; ww < kSelWaves; ++ww) tot += histbuf[1][ww];
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

    // ---- the last head of the group to finish merges the group's bitmaps
    __syncthreads();
    if (tid == 0) {
        a.stats[2 * h + 0] = (int32_t)s_cnt[0];
        a.stats[2 * h + 1] = (int32_t)s_cnt[1];
        __threadfence();
        const int prev = atomicAdd(&a.done[g], 1);
        s_last = (prev == G - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const uint64_t* gbm = a.kbm + (size_t)g * G * a.wcap;
    const size_t nrow = (size_t)g * a.next_cap;
    // Merge in steps of mw bitmap words (16384 positions).  LDS is reused: node ids
    // of the step's positions in `keys`, the G head words in histbuf, the union in
    // cntbuf[0] (as 64-bit words) and its exclusive popcount prefix in cntbuf[1].
    constexpr int mw = kLdsKeys / 64;                       // 256 words
    int32_t* nid = reinterpret_cast<int32_t*>(keys);        // [mw * 64]
    uint64_t* hw = &histbuf[0][0];                          // [G][mw], G * mw <= 4096
    uint64_t* s_union = reinterpret_cast<uint64_t*>(cntbuf[0]);
    uint32_t* s_wpre = cntbuf[1];
    if (tid == 0) s_run = 0;
#pragma unroll 1
    for (int64_t wb = 0; wb < nwords; wb += mw) {
        const int nw = (int)min((int64_t)mw, nwords - wb);
        const int64_t npos = min((int64_t)nw * 64, n - wb * 64);
        for (int i = tid; i < G * nw; i += kSelThreads) {
            const int hh = i / nw, wi = i - hh * nw;
            hw[hh * mw + wi] = __hip_atomic_load(gbm + (size_t)hh * a.wcap + wb + wi, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        }
        if (!a.top) {
#pragma unroll 4
            for (int64_t p = tid; p < npos; p += kSelThreads) nid[p] = a.cand_node[lrow + wb * 64 + p];
        }
        __syncthreads();
        if (wave == 0) {
            // union words and their exclusive popcount prefix (4 words per lane)
            uint32_t cnt = 0;
            for (int q = 0; q < mw / 64; ++q) {
                const int wi = lane * (mw / 64) + q;
                uint64_t u = 0;
                if (wi < nw)
                    for (int hh = 0; hh < G; ++hh) u |= hw[hh * mw + wi];
                s_union[wi] = u;
                cnt += __popcll(u);
            }
            uint64_t tot;
            uint32_t pre = (uint32_t)wave_excl_scan_u64(cnt, &tot);
            for (int q = 0; q < mw / 64; ++q) {
                const int wi = lane * (mw / 64) + q;
                s_wpre[wi] = pre;
                pre += __popcll(s_union[wi]);
            }
            if (lane == 0) s_before = tot;
        }
        __syncthreads();
        const uint64_t run = s_run;
#pragma unroll 1
        for (int64_t p = tid; p < npos; p += kSelThreads) {
            const int wi = (int)(p >> 6), b = (int)(p & 63);
            const uint64_t u = s_union[wi];
            if (!((u >> b) & 1ull)) continue;
            const uint64_t rank = run + s_wpre[wi] + __popcll(u & ((1ull << b) - 1ull));
            uint32_t msk = 0;
            for (int hh = 0; hh < G; ++hh) msk |= (uint32_t)((hw[hh * mw + wi] >> b) & 1ull) << hh;
            const int32_t node = a.top ? (int32_t)(wb * 64 + p) : nid[p];
            a.klist[lrow + rank] = node;
            a.kmask[lrow + rank] = msk;
            if (a.next_node) {
                for (int i = 0; i < c; ++i) {
                    a.next_node[nrow + rank * c + i] = node * c + i;
                    a.next_mask[nrow + rank * c + i] = msk;
                }
            }
        }
        __syncthreads();
        if (tid == 0) s_run = run + s_before;
        __syncthreads();
    }
    const uint64_t total = s_run;
    if (a.next_node) {
        const uint32_t allg = all_heads(G);
        const int64_t n_orph = a.orph_hi - a.orph_lo;
        for (int64_t o = tid; o < n_orph; o += kSelThreads) {
            a.next_node[nrow + total * c + o] = (int32_t)(a.orph_lo + o);
            a.next_mask[nrow + total * c + o] = allg;
        }
        if (tid == 0) a.next_ncand[g] = (int32_t)(total * c + n_orph);
    }
    if (tid == 0) a.nkept[g] = (int32_t)total;
}


}  // namespace

int zha_score_blocks(int64_t max_cand, int R) {
    const int64_t U = R <= 16 ? 16 / R : 1;
    const int64_t items = (max_cand + U - 1) / U;
    int64_t blocks = (items + 7) / 8;        // about two items per wave
    if (blocks < 1) blocks = 1;
    if (blocks > ZHA_SCORE_MAXB) blocks = ZHA_SCORE_MAXB;
    return (int)blocks;
}

hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream) {
    dim3 grid((unsigned)blocks, (unsigned)H_kv);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_route_score_kernel<true>, grid, dim3(kScoreThreads), 0, stream, q, a, G, c, R, tau);
    else
        hipLaunchKernelGGL(zha_route_score_kernel<false>, grid, dim3(kScoreThreads), 0, stream, q, a, G, c, R, tau);
    return hipGetLastError();
}

hipError_t zha_launch_route_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream) {
    hipLaunchKernelGGL(zha_route_select_kernel, dim3((unsigned)(H_kv * G)), dim3(kSelThreads), 0, stream, a, G,
                       c, top_p);
    return hipGetLastError();
}
