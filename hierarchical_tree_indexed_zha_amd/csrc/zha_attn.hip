// Exact attention over the tokens a decode step selected (sparse mode) or over
// every cached token (dense mode), as a split-K flash decode with an online
// softmax in fp32, followed by a combine of the split partials.
//
// Sparse mode attends, for each query head, over the raw keys of the level-1
// chunks it kept, token 0 (the attention sink) and the raw tail [c*n_1, N)
// (page rit.work "zha-tree-indexer-long-context", section "Дерево сокращает
// сам поиск нужных ключей": exact attention over the raw keys of the reached
// leaves; page "ZHA 用树形稀疏注意力改造现有大模型", section
// 稀疏注意力为什么还会被索引拖慢: the first token is always kept).  The KV
// bytes of a chunk are read once per KV group: a per-chunk bit mask says
// which of the group's query heads selected it.
//
// Slot space of a group (32-slot tiles):
//   [0]                 token 0 for every head (when chunk 0 is complete)
//   [sink, lead)        the tail tokens, every head
//   [lead, total)       kept chunks in ascending order; token 0 is masked here
// The lead (sink and tail) depends on N alone, so a slot's token is known before
// the kept count arrives.  Wave w of block b takes tiles 4b + w, then every
// 4 nact-th tile after it: its first tile's kept-list entries are read together
// with the count (one memory round trip), and only the later tiles wait for it.
//
// bf16 path: QK^T and PV run on v_mfma_f32_16x16x32_bf16 with the group's
// heads as the 16 MFMA rows.  V stays in its row-major layout: a lane loads 16
// bytes of one token row and the contraction index of the PV product is
// permuted so that each lane's eight B-operand values come from eight such
// loads.  P is split into bf16 hi + lo parts (two MFMAs), so the PV product
// keeps 16 significant bits of P.  fp32 path: the same tiling on v_mfma_f32_16x16x4_f32.
#include <hip/hip_ext.h>

#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileSlots = 32;
#ifndef ZHA_ATTN_MIN_TILES
#define ZHA_ATTN_MIN_TILES 4
#endif
constexpr int kMinTilesPerBlock = ZHA_ATTN_MIN_TILES;   // fewest 32-slot tiles a split block takes
constexpr float kLog2e = 1.4426950408889634f;

// Byte permute: bytes of (hi_src:lo_src) picked by `sel` (v_perm_b32).
__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}
constexpr uint32_t kLowHalves = 0x05040100u;    // (lo half of lo_src) | (lo half of hi_src) << 16
constexpr uint32_t kHighHalves = 0x07060302u;   // (hi half of lo_src) | (hi half of hi_src) << 16

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct Slots {
    int64_t lead, total, tail_start;   // total: known once the kept count is
    int sink;
};

// The slot space's lead (from N alone); total is set from the kept count later.
template <bool DENSE>
__device__ __forceinline__ Slots slot_lead(const ZhaAttnArgs& a, int c) {
    Slots s;
    if (DENSE) {
        s.sink = 0;
        s.tail_start = 0;
        s.lead = 0;
        s.total = a.n_tokens;
    } else {
        const int64_t n1 = a.n_tokens / c;
        s.tail_start = (int64_t)c * n1;
        s.sink = n1 > 0 ? 1 : 0;
        s.lead = s.sink + (a.n_tokens - s.tail_start);
        s.total = s.lead;
    }
    return s;
}

// Token and head mask of a slot, whatever the kept count (a slot at or beyond
// the total is masked by the caller).  Branch-free, with both kept-list reads
// issued together: a kept-chunk slot outside the list's capacity (cap1 = 0 when
// no level is routed) reads the group's first entry and is masked.
// In two halves, so that a caller can issue the reads and use them later:
// slot_fetch reads the kept-list entry, slot_finish forms the token and mask.
struct SlotRaw {
    int32_t kn;
    uint32_t km;
};
template <bool DENSE>
__device__ __forceinline__ SlotRaw slot_fetch(const ZhaAttnArgs& a, const Slots& s, int g, int c, int64_t slot) {
    SlotRaw r{0, 0u};
    if (!DENSE) {
        const bool chunk = slot >= s.lead;
        const int64_t e = chunk ? (slot - s.lead) / c : 0;
        const size_t idx = (size_t)g * a.cap1 + (size_t)((chunk && e < a.cap1) ? e : 0);
        r.kn = a.klist[idx];
        r.km = a.kmask[idx];
    }
    return r;
}
template <bool DENSE>
__device__ __forceinline__ void slot_finish(const ZhaAttnArgs& a, const Slots& s, int c, uint32_t allg, int64_t slot,
                                            const SlotRaw& r, int32_t* tok, uint32_t* msk) {
    if (DENSE) {
        *tok = (int32_t)slot;
        *msk = allg;
        return;
    }
    const bool chunk = slot >= s.lead;
    const int64_t e = chunk ? (slot - s.lead) / c : 0;
    const bool ok = chunk && e < a.cap1;
    const int64_t t = (int64_t)r.kn * c + (slot - s.lead - e * c);
    const int32_t tail_tok = (s.sink && slot == 0) ? 0 : (int32_t)(s.tail_start + slot - s.sink);
    *tok = chunk ? (ok ? (int32_t)t : 0) : tail_tok;
    *msk = chunk ? ((ok && t != 0) ? r.km : 0u) : allg;
}
template <bool DENSE>
__device__ __forceinline__ void slot_to_token(const ZhaAttnArgs& a, const Slots& s, int g, int c, uint32_t allg,
                                              int64_t slot, int32_t* tok, uint32_t* msk) {
    slot_finish<DENSE>(a, s, c, allg, slot, slot_fetch<DENSE>(a, s, g, c, slot), tok, msk);
}

__device__ __forceinline__ int active_blocks(int64_t tiles, int Bg) {
    int64_t n = (tiles + kMinTilesPerBlock - 1) / kMinTilesPerBlock;
    if (n < 1) n = 1;
    if (n > Bg) n = Bg;
    return (int)n;
}

// The K and V rows of one 32-slot tile (bf16), token ids in LDS: K as the B
// operand of QK^T (lane j, q4: slot 16 bb + j, columns 32 s + 8 q4), V in row
// order (lane j, q4: slot 4 i + q4, columns 8 j .. 8 j + 7).
__device__ __forceinline__ void load_kv_bf16(const uint16_t* K, const uint16_t* V, size_t head_row0,
                                             const int32_t* tok, int j, int q4, uint4 (&kr)[2][4],
                                             uint4 (&vr)[8]) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const uint16_t* row = K + (head_row0 + (size_t)tok[16 * bb + j]) * ZHA_D + 8 * q4;
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[bb][s] = *reinterpret_cast<const uint4*>(row + 32 * s);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        vr[i] = *reinterpret_cast<const uint4*>(V + (head_row0 + (size_t)tok[4 * i + q4]) * ZHA_D + 8 * j);
}

// Masked, scaled logits of one tile folded into the running softmax of the
// lane's heads 4 q4 + i; the tile's probabilities go to s_p [16 heads][33].
__device__ __forceinline__ void softmax_tile(const zha_f32x4 (&S)[2], uint32_t mk0, uint32_t mk1, float scale,
                                             int j, int q4, float (&m_run)[4], float (&l_run)[4],
                                             zha_f32x4 (&O)[8], float* s_p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        const float x0 = ((mk0 >> h) & 1u) ? S[0][i] * scale : zha_neg_inf();
        const float x1 = ((mk1 >> h) & 1u) ? S[1][i] * scale : zha_neg_inf();
        const float mx = zha_row16_max(fmaxf(x0, x1));
        const float mn = fmaxf(m_run[i], mx);
        float alpha, p0, p1;
        if (mn == zha_neg_inf()) {
            alpha = 1.f; p0 = 0.f; p1 = 0.f;
        } else {
            alpha = exp2f(m_run[i] - mn);
            p0 = exp2f(x0 - mn);
            p1 = exp2f(x1 - mn);
        }
        const float rs = zha_row16_sum(p0 + p1);
        l_run[i] = l_run[i] * alpha + rs;
        m_run[i] = mn;
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) O[c8][i] *= alpha;
        s_p[h * 33 + j] = p0;
        s_p[h * 33 + 16 + j] = p1;
    }
}

// O += P V for one bf16 tile: P (from s_p) as bf16 hi + lo parts, V rows vr.
__device__ __forceinline__ void pv_tile_bf16(const float* s_p, const uint4 (&vr)[8], int j, int q4,
                                             zha_f32x4 (&O)[8]) {
    // A operand: row head j, contraction slots 4e + q4, e = 0..7, as bf16 hi + lo
    // parts: hi = P truncated to bf16, lo = the residual truncated to bf16, so
    // hi + lo keeps 16 significant bits of P.
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        const float pa = s_p[j * 33 + 4 * (2 * e2) + q4];
        const float pb = s_p[j * 33 + 4 * (2 * e2 + 1) + q4];
        const uint32_t ua = __float_as_uint(pa), ub = __float_as_uint(pb);
        hi[e2] = perm(ub, ua, kHighHalves);
        const float ra = pa - __uint_as_float(ua & 0xFFFF0000u);
        const float rb = pb - __uint_as_float(ub & 0xFFFF0000u);
        lo[e2] = perm(__float_as_uint(rb), __float_as_uint(ra), kHighHalves);
    }
    const zha_bf16x8 Ahi = zha_as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
    const zha_bf16x8 Alo = zha_as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
        const int w = c8 >> 1;
        const uint32_t sel = (c8 & 1) ? kHighHalves : kLowHalves;
        uint32_t bw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) bw[e2] = perm(comp(vr[2 * e2 + 1], w), comp(vr[2 * e2], w), sel);
        const zha_bf16x8 Bv = zha_as_bf16x8(make_uint4(bw[0], bw[1], bw[2], bw[3]));
        O[c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, Bv, O[c8], 0, 0, 0);
        O[c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, Bv, O[c8], 0, 0, 0);
    }
}

// grid (Bg, H_kv), 256 threads.
template <bool BF16, bool DENSE>
__global__ __launch_bounds__(kThreads, BF16 ? ZHA_ATTN_BLOCKS_BF16 : ZHA_ATTN_BLOCKS_F32) void zha_attn_kernel(ZhaAttnArgs a, int G, int c, float tau, int Bg) {
    ZHA_ATTN_ARGS_READY(a, "s"(G), "s"(c), "s"(tau), "s"(Bg));
    __shared__ int32_t s_tok[kWaves][kTileSlots];
    __shared__ uint32_t s_msk[kWaves][kTileSlots];
    __shared__ float s_buf[kWaves * 16 * ZHA_D];          // P tiles during the loop, partial O after it
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];

    const int g = blockIdx.y, b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, q4 = lane >> 4;
    const uint32_t allg = (G >= 32) ? 0xFFFFFFFFu : ((1u << G) - 1u);
    Slots sp = slot_lead<DENSE>(a, c);
    // this wave's first tile (4 b + wave, whatever the count): its slots' tokens
    // are requested before the kept count is
    const int64_t tw0 = (int64_t)b * kWaves + wave;
    const int64_t slot0 = tw0 * kTileSlots + (lane & (kTileSlots - 1));
    SlotRaw raw0 = slot_fetch<DENSE>(a, sp, g, c, slot0);
    const float scale = tau * kLog2e;                     // logits in log2 units
    float* s_p = s_buf + wave * 16 * 33;                  // [16 heads][33]

    const size_t head_row0 = (size_t)(g % a.hkv) * (size_t)a.cap_tok;   // (a batch routes virtual groups)

    // Q as the A operand: row = head j (zero beyond G)
    uint4 qa16[4];
    float qa32[32];
    if (BF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (j < G)
                qa16[s] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                          ((size_t)g * G + j) * ZHA_D + 32 * s + 8 * q4);
            else
                qa16[s] = make_uint4(0u, 0u, 0u, 0u);
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                qa32[4 * m + e] = (j < G) ? static_cast<const float*>(a.q)[((size_t)g * G + j) * ZHA_D + 16 * m + 4 * q4 + e] : 0.f;
    }

    // the kept count, read after every read above (one round trip for all of them)
    // (the first tile's entries are used only after this point)
    if (!DENSE) {
        int nk_raw = a.nkept[g];
        asm volatile("" : "+v"(nk_raw), "+v"(raw0.kn), "+v"(raw0.km)::"memory");
        const int nk = a.cap1 > 0 ? __builtin_amdgcn_readfirstlane(nk_raw) : 0;
        sp.total = sp.lead + (int64_t)nk * c;
    }
    const int64_t tiles = (sp.total + kTileSlots - 1) / kTileSlots;
    const int nact = active_blocks(tiles, Bg);
    if (b == 0 && threadIdx.x == 0) a.nact[g] = nact;
    if (b >= nact) return;
    const int64_t tstep = (int64_t)nact * kWaves;         // tiles of one round over the active waves
    int32_t nx_tok = 0;
    uint32_t nx_msk = 0;
    slot_finish<DENSE>(a, sp, c, allg, slot0, raw0, &nx_tok, &nx_msk);
    if (slot0 >= sp.total) {
        nx_tok = 0;
        nx_msk = 0u;
    }

    float m_run[4], l_run[4];
    zha_f32x4 O[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = zha_neg_inf(); l_run[i] = 0.f; }
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) O[c8] = zha_f32x4{0.f, 0.f, 0.f, 0.f};

    // the slot -> token map of the next tile is fetched while this tile computes
    for (int64_t t = tw0; t < tiles; t += tstep) {
        if (lane < kTileSlots) {
            s_tok[wave][lane] = nx_tok;
            s_msk[wave][lane] = nx_msk;
            const int64_t ns = (t + tstep) * kTileSlots + lane;
            if (t + tstep < tiles) {
                slot_to_token<DENSE>(a, sp, g, c, allg, ns, &nx_tok, &nx_msk);
                if (ns >= sp.total) {
                    nx_tok = 0;
                    nx_msk = 0u;
                }
            }
        }
        zha_wave_lds_sync();

        zha_f32x4 S[2];
        if constexpr (BF16) {
            uint4 kr[2][4], vr[8];
            load_kv_bf16(static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.V), head_row0,
                         s_tok[wave], j, q4, kr, vr);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                zha_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zha_as_bf16x8(qa16[s]), zha_as_bf16x8(kr[bb][s]), acc, 0, 0, 0);
                S[bb] = acc;
            }
            // S[bb][i]: head 4*q4+i against slot 16*bb+j.  Mask, scale, online softmax.
            softmax_tile(S, s_msk[wave][j], s_msk[wave][16 + j], scale, j, q4, m_run, l_run, O, s_p);
            zha_wave_lds_sync();
            pv_tile_bf16(s_p, vr, j, q4, O);
        } else {
            const float* K = static_cast<const float*>(a.K);
            const float* V = static_cast<const float*>(a.V);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const float4* row = reinterpret_cast<const float4*>(K + (head_row0 + (size_t)s_tok[wave][16 * bb + j]) * ZHA_D);
                zha_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float4 kf = row[4 * m + q4];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa32[4 * m + 0], kf.x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa32[4 * m + 1], kf.y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa32[4 * m + 2], kf.z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa32[4 * m + 3], kf.w, acc, 0, 0, 0);
                }
                S[bb] = acc;
            }
            float4 vf[8][2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4* row = reinterpret_cast<const float4*>(V + (head_row0 + (size_t)s_tok[wave][4 * i + q4]) * ZHA_D + 8 * j);
                vf[i][0] = row[0];
                vf[i][1] = row[1];
            }
            softmax_tile(S, s_msk[wave][j], s_msk[wave][16 + j], scale, j, q4, m_run, l_run, O, s_p);
            zha_wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pa = s_p[j * 33 + 4 * i + q4];
                const float v8[8] = {vf[i][0].x, vf[i][0].y, vf[i][0].z, vf[i][0].w,
                                     vf[i][1].x, vf[i][1].y, vf[i][1].z, vf[i][1].w};
#pragma unroll
                for (int c8 = 0; c8 < 8; ++c8) O[c8] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, v8[c8], O[c8], 0, 0, 0);
            }
        }
        zha_wave_lds_sync();
    }

    // ---- combine the block's waves; O[c8][i] is head 4*q4+i, column d = 8*j + c8
    __syncthreads();
    if (j == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s_m[wave][4 * q4 + i] = m_run[i];
            s_l[wave][4 * q4 + i] = l_run[i];
        }
    float* so = s_buf + wave * 16 * ZHA_D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) so[(4 * q4 + i) * ZHA_D + 8 * j + c8] = O[c8][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * ZHA_D; idx += kThreads) {
        const int h = idx >> 7, d = idx & (ZHA_D - 1);
        float M = zha_neg_inf();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, acc = 0.f;
        if (M != zha_neg_inf()) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = exp2f(s_m[w][h] - M);
                L = fmaf(s_l[w][h], f, L);
                acc = fmaf(s_buf[(w * 16 + h) * ZHA_D + d], f, acc);
            }
        }
        const size_t ph = ((size_t)g * Bg + b) * G + h;
        if (d == 0) {
            a.pm[ph] = M;
            a.pl[ph] = L;
        }
        a.po[ph * ZHA_D + d] = acc;
    }
}

// grid (H_q, 128 / 32), NT threads = NT / 32 partial lanes x 32 columns, NT >= Bg
// (256, or ZHA_ATTN_MAXB for wider splits):
// out[h][d] = sum_b O_b[d] 2^(m_b - M) / sum_b l_b 2^(m_b - M).
// Every read (the partial count, and each partial's m, l and columns, bounded by
// the launch's Bg and masked by the count afterwards) goes out in one batch: one
// memory round trip.  Partials at or beyond the count are never combined
// arithmetically (their memory may hold anything), only selected away.
template <int NT>
__global__ __launch_bounds__(NT) void zha_combine_kernel(ZhaAttnArgs a, int G, int Bg, float* __restrict__ out) {
    constexpr int kWv = NT / 64;
    constexpr int kLanes = NT / 32;        // partial lanes of the column pass
    constexpr int kPerO = NT / kLanes;     // columns (partials) per thread: 32
    static_assert(NT <= ZHA_ATTN_MAXB && kPerO * kLanes == NT, "combine split");
    ZHA_ATTN_ARGS_READY(a, "s"(G), "s"(Bg), "s"(out));
    __shared__ float f[NT];
    __shared__ float red[NT];
    __shared__ float wred[2][kWv];
    const int h = blockIdx.x, g = h / G, hl = h - g * G, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int dd = tid & 31, bl = tid >> 5;
    const int d = blockIdx.y * 32 + dd;
    const size_t base = (size_t)g * Bg * G + hl;          // partial b of head h at base + b*G
    // partial tid's m and l; columns d of partials bl + kLanes j
    const float mb = tid < Bg ? a.pm[base + (size_t)tid * G] : zha_neg_inf();
    const float lb = tid < Bg ? a.pl[base + (size_t)tid * G] : 0.f;
    float ov[kPerO];
#pragma unroll
    for (int j = 0; j < kPerO; ++j) {
        const int b = bl + j * kLanes;
        ov[j] = b < Bg ? a.po[(base + (size_t)b * G) * ZHA_D + d] : 0.f;
    }
    int nraw = a.nact[g];
    asm volatile("" : "+v"(nraw)::"memory");
    const int n = __builtin_amdgcn_readfirstlane(nraw);

    const bool live = tid < n && mb != zha_neg_inf();
    float m = zha_wave_max(live ? mb : zha_neg_inf());
    if (lane == 0) wred[0][wave] = m;
    __syncthreads();
    float M = wred[0][0];
#pragma unroll
    for (int w = 1; w < kWv; ++w) M = fmaxf(M, wred[0][w]);
    const float fb = live ? exp2f(mb - M) : 0.f;
    f[tid] = fb;
    const float l = zha_wave_sum(live ? lb * fb : 0.f);
    if (lane == 0) wred[1][wave] = l;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWv; ++w) L += wred[1][w];
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kPerO; ++j) {
        const int b = bl + j * kLanes;
        acc = b < n ? fmaf(ov[j], f[b], acc) : acc;
    }
    red[tid] = acc;
    __syncthreads();
    if (bl == 0) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < kLanes; ++k) t += red[k * 32 + dd];
        out[(size_t)h * ZHA_D + d] = t / L;
    }
}

}  // namespace

hipError_t zha_launch_attention(int kv_dtype, bool dense, const ZhaAttnArgs& a, int H_kv, int G, int c, float tau,
                                int Bg, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const dim3 grid((unsigned)Bg, (unsigned)H_kv);
    // start / stop (may be null) are recorded by the dispatch itself: they time
    // the kernel alone
    if (kv_dtype == 0) {
        if (dense)
            hipExtLaunchKernelGGL((zha_attn_kernel<true, true>), grid, dim3(kThreads), 0, stream, start, stop, 0, a, G,
                                  c, tau, Bg);
        else
            hipExtLaunchKernelGGL((zha_attn_kernel<true, false>), grid, dim3(kThreads), 0, stream, start, stop, 0, a,
                                  G, c, tau, Bg);
    } else {
        if (dense)
            hipExtLaunchKernelGGL((zha_attn_kernel<false, true>), grid, dim3(kThreads), 0, stream, start, stop, 0, a,
                                  G, c, tau, Bg);
        else
            hipExtLaunchKernelGGL((zha_attn_kernel<false, false>), grid, dim3(kThreads), 0, stream, start, stop, 0, a,
                                  G, c, tau, Bg);
    }
    return hipGetLastError();
}

hipError_t zha_launch_combine(const ZhaAttnArgs& a, int H_kv, int G, int Bg, float* out, hipStream_t stream) {
    if (Bg < 1 || Bg > ZHA_ATTN_MAXB) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(H_kv * G), ZHA_D / 32);
    if (Bg <= 256)
        hipLaunchKernelGGL(zha_combine_kernel<256>, grid, dim3(256), 0, stream, a, G, Bg, out);
    else
        hipLaunchKernelGGL(zha_combine_kernel<ZHA_ATTN_MAXB>, grid, dim3(ZHA_ATTN_MAXB), 0, stream, a, G, Bg, out);
    return hipGetLastError();
}
