// Summary-tree kernels: leaf summaries from raw keys, exact merges up the tree,
// and the KV row write of an append.
//
// A node's summary holds, for every reference query q_r of its KV head, the
// tangent plane of the node's log attention mass at q_r (page "ZHA
// 用树形稀疏注意力改造现有大模型", section 稀疏注意力为什么还会被索引拖慢; page
// "Zyphra 分层注意力（ZHA）…", section 机制拆解):
//   z_t = tau q_r.k_t,  LSE_r = log sum_t e^{z_t},  w_t = e^{z_t - LSE_r},
//   s_r = sum_t w_t k_t,  b_r = LSE_r - tau q_r.s_r = LSE_r - sum_t w_t z_t.
// The last form (the entropy of w) needs no second dot product.  Parents are
// built from their c children with the exact identity (the pages summarise
// summaries recursively; with reference queries shared across levels this
// equals summarising the raw keys):
//   LSE_P = log sum_j e^{LSE_j},  a_j = e^{LSE_j - LSE_P},
//   s_P = sum_j a_j s_j,  b_P = sum_j a_j (b_j - log a_j).
#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kTile = 64;          // raw tokens staged per step
constexpr int kKStride = ZHA_D + 4; // padded LDS row (floats)

template <bool BF16>
__device__ __forceinline__ void load_key_tile(const void* __restrict__ Kv, int64_t row0, int ntok,
                                              float* __restrict__ Ks) {
    // rows row0 .. row0+ntok of one KV head are contiguous: ntok*128 elements
    if (BF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Kv) + row0 * ZHA_D);
        for (int i = threadIdx.x; i < ntok * (ZHA_D / 8); i += blockDim.x) {
            uint4 v = src[i];
            int t = i / (ZHA_D / 8), d = (i % (ZHA_D / 8)) * 8;
            float* dst = Ks + t * kKStride + d;
            dst[0] = zha_bf16_to_f32(v.x & 0xFFFFu); dst[1] = zha_bf16_to_f32(v.x >> 16);
            dst[2] = zha_bf16_to_f32(v.y & 0xFFFFu); dst[3] = zha_bf16_to_f32(v.y >> 16);
            dst[4] = zha_bf16_to_f32(v.z & 0xFFFFu); dst[5] = zha_bf16_to_f32(v.z >> 16);
            dst[6] = zha_bf16_to_f32(v.w & 0xFFFFu); dst[7] = zha_bf16_to_f32(v.w >> 16);
        }
    } else {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(Kv) + row0 * ZHA_D);
        for (int i = threadIdx.x; i < ntok * (ZHA_D / 4); i += blockDim.x) {
            float4 v = src[i];
            int t = i / (ZHA_D / 4), d = (i % (ZHA_D / 4)) * 4;
            *reinterpret_cast<float4*>(Ks + t * kKStride + d) = v;
        }
    }
}

__device__ __forceinline__ float dot128(const float* __restrict__ a, const float* __restrict__ b) {
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < ZHA_D; i += 4) {
        float4 x = *reinterpret_cast<const float4*>(a + i);
        float4 y = *reinterpret_cast<const float4*>(b + i);
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
    }
    return acc;
}

// grid (ceil(n_leaves / leaves_per_block), H_kv), 256 threads.
// Leaves [first_leaf, first_leaf + n_leaves) of every KV head.
template <bool BF16>
__global__ __launch_bounds__(256) void zha_leaf_summary_kernel(
    const void* __restrict__ Kv, const float* __restrict__ Qref,
    float* __restrict__ S, float* __restrict__ B, float* __restrict__ LSE,
    int64_t cap_tok, int64_t cap1, int c, int R, int64_t first_leaf, int64_t n_leaves, float tau) {
    extern __shared__ float smem[];
    float* Qs = smem;                       // [R][128]
    float* Ks = Qs + R * ZHA_D;             // [64][132]
    float* Z = Ks + kTile * kKStride;       // [R][64]
    float* aux = Z + R * kTile;             // [4][R]
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t head_row0 = (size_t)g * cap_tok;

    if (c <= kTile) {
        const int lpb = kTile / c;
        const int64_t leaf0 = first_leaf + (int64_t)blockIdx.x * lpb;
        const int64_t end = first_leaf + n_leaves;
        if (leaf0 >= end) return;
        const int nl = (int)min((int64_t)lpb, end - leaf0);
        const int ntok = nl * c;
        for (int i = tid; i < R * ZHA_D; i += blockDim.x) Qs[i] = Qref[(size_t)g * R * ZHA_D + i];
        const void* kbase = BF16 ? (const void*)(static_cast<const uint16_t*>(Kv)) : Kv;
        load_key_tile<BF16>(kbase, (int64_t)head_row0 + leaf0 * c, ntok, Ks);
        __syncthreads();
        for (int pr = tid; pr < R * ntok; pr += blockDim.x) {
            int r = pr / ntok, t = pr - r * ntok;
            Z[r * kTile + t] = tau * dot128(Qs + r * ZHA_D, Ks + t * kKStride);
        }
        __syncthreads();
        for (int pr = tid; pr < nl * R; pr += blockDim.x) {
            int lf = pr / R, r = pr - lf * R;
            float* z = Z + r * kTile + lf * c;
            float m = zha_neg_inf();
            for (int t = 0; t < c; ++t) m = fmaxf(m, z[t]);
            float l = 0.f;
            for (int t = 0; t < c; ++t) l += expf(z[t] - m);
            float lse = m + logf(l);
            float ez = 0.f;
            for (int t = 0; t < c; ++t) {
                float w = expf(z[t] - lse);
                ez = fmaf(w, z[t], ez);
                z[t] = w;
            }
            size_t o = ((size_t)g * cap1 + (size_t)(leaf0 + lf)) * R + r;
            LSE[o] = lse;
            B[o] = lse - ez;
        }
        __syncthreads();
        for (int o = tid; o < nl * R * ZHA_D; o += blockDim.x) {
            int d = o & (ZHA_D - 1);
            int rl = o >> 7;
            int r = rl % R, lf = rl / R;
            const float* w = Z + r * kTile + lf * c;
            const float* k = Ks + lf * c * kKStride + d;
            float acc = 0.f;
            for (int t = 0; t < c; ++t) acc = fmaf(w[t], k[t * kKStride], acc);
            S[(((size_t)g * cap1 + (size_t)(leaf0 + lf)) * R + r) * ZHA_D + d] = acc;
        }
        return;
    }

    // c > 64: one leaf per block, 64-token steps with an online softmax.
    const int64_t leaf = first_leaf + blockIdx.x;
    if (leaf >= first_leaf + n_leaves) return;
    float* mrun = aux;
    float* lrun = aux + R;
    float* ezrun = aux + 2 * R;
    float* alpha = aux + 3 * R;
    for (int i = tid; i < R * ZHA_D; i += blockDim.x) Qs[i] = Qref[(size_t)g * R * ZHA_D + i];
    if (tid < R) { mrun[tid] = zha_neg_inf(); lrun[tid] = 0.f; ezrun[tid] = 0.f; }
    constexpr int kMaxAcc = 32 * ZHA_D / 256;      // R <= 32
    float acc[kMaxAcc];
#pragma unroll
    for (int k = 0; k < kMaxAcc; ++k) acc[k] = 0.f;
    const int nacc = R * ZHA_D / 256 > 0 ? R * ZHA_D / 256 : 1;
    for (int sub = 0; sub < c; sub += kTile) {
        const int nt = min(kTile, c - sub);
        __syncthreads();
        load_key_tile<BF16>(Kv, (int64_t)head_row0 + leaf * c + sub, nt, Ks);
        __syncthreads();
        for (int pr = tid; pr < R * nt; pr += blockDim.x) {
            int r = pr / nt, t = pr - r * nt;
            Z[r * kTile + t] = tau * dot128(Qs + r * ZHA_D, Ks + t * kKStride);
        }
        __syncthreads();
        if (tid < R) {
            float* z = Z + tid * kTile;
            float mt = zha_neg_inf();
            for (int t = 0; t < nt; ++t) mt = fmaxf(mt, z[t]);
            float mn = fmaxf(mrun[tid], mt);
            float a = expf(mrun[tid] - mn);           // 0 on the first step
            float l = a * lrun[tid], ez = a * ezrun[tid];
            for (int t = 0; t < nt; ++t) {
                float pz = expf(z[t] - mn);
                l += pz;
                ez = fmaf(pz, z[t], ez);
                z[t] = pz;
            }
            mrun[tid] = mn; lrun[tid] = l; ezrun[tid] = ez; alpha[tid] = a;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxAcc; ++k) {
            if (k < nacc) {
                int o = tid + k * 256;
                if (o < R * ZHA_D) {
                    int r = o >> 7, d = o & (ZHA_D - 1);
                    const float* w = Z + r * kTile;
                    float s = alpha[r] * acc[k];
                    for (int t = 0; t < nt; ++t) s = fmaf(w[t], Ks[t * kKStride + d], s);
                    acc[k] = s;
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxAcc; ++k) {
        if (k < nacc) {
            int o = tid + k * 256;
            if (o < R * ZHA_D) {
                int r = o >> 7, d = o & (ZHA_D - 1);
                S[(((size_t)g * cap1 + (size_t)leaf) * R + r) * ZHA_D + d] = acc[k] / lrun[r];
            }
        }
    }
    if (tid < R) {
        size_t o = ((size_t)g * cap1 + (size_t)leaf) * R + tid;
        float lse = mrun[tid] + logf(lrun[tid]);
        LSE[o] = lse;
        B[o] = lse - ezrun[tid] / lrun[tid];
    }
}

// ---- leaf summaries on the matrix cores (R <= 16, c a power of two).
//
// One wave takes a unit of 16 consecutive tokens (16 / c leaves for c <= 16) or one
// whole leaf (c >= 32, its c / 16 tiles of 16 tokens in turn, the next tile's keys
// requested before the current one is computed; a leaf dealt to the four waves of a
// workgroup and combined measured slower).  Per tile:
//   Z = tau Q K^T      16 refs x 16 tokens, 32 v_mfma_f32_16x16x4_f32 (refs past R zero);
//                      lane (j, q4) brings K[t0 + j][32 q4 .. 32 q4 + 31] (the
//                      contraction index d = 32 q4 + m of step m), Q likewise;
//   softmax per (r, leaf) over the tile's lanes j (segmented shuffles), or online
//                      across the tiles of one leaf (running max, sum, sum of w z);
//   S += W K           per 16-column slice, the tile's tokens in groups of four:
//                      W from LDS as the A operand (row r, token 4 kk + q4), K from
//                      LDS as the B operand (token 4 kk + q4, column 16 s + j).
// Outputs as the scalar kernel's: S[leaf][r][d], B, LSE (rows r < R).  With `fuse`
// (c in {2, 4}: a unit holds 16 / c^2 whole level-2 nodes; first_leaf a multiple of
// c) the unit's level-2 nodes are written too, merged as the merge kernel does: per
// ref, the node's LSE is the log-sum-exp of its leaves' (one lane per leaf segment
// over the node's c^2 lanes), a = exp(LSE_leaf - LSE_node), b = sum a (b_leaf - log a),
// and s = sum over the node's tokens of (a w) k, one more pass of the products with
// each token's weight scaled by its leaf's a (which the token's own lane holds).
constexpr int kLmMinR = 4;         // fewer reference queries leave most MFMA rows empty:
                                   // the scalar kernel is faster there (measured at R = 1)
constexpr int kLmStride = 144;     // LDS row of a staged key tile (floats): the B reads of
                                   // a half-wave (rows q4 and q4 + 1) fall 16 banks apart

// Butterfly steps within a row of 16 lanes as DPP moves (no LDS traffic): lane
// pairs at distance 1 and 2 (quad permutations), then 4 and 8 (mirrors within 8
// and 16 lanes, which pair the already uniform quads and halves).  Every lane of a
// segment ends with the same value, bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __uint_as_float(zha_dpp<CTRL, 0xF>(__float_as_uint(v), __float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
__device__ __forceinline__ float seg_max(float x, int c) {
    x = fmaxf(x, dpp_row<kDppXor1>(x));
    if (c > 2) x = fmaxf(x, dpp_row<kDppXor2>(x));
    if (c > 4) x = fmaxf(x, dpp_row<kDppHalfMirror>(x));
    if (c > 8) x = fmaxf(x, dpp_row<kDppMirror>(x));
    return x;
}
__device__ __forceinline__ float seg_sum(float x, int c) {
    x += dpp_row<kDppXor1>(x);
    if (c > 2) x += dpp_row<kDppXor2>(x);
    if (c > 4) x += dpp_row<kDppHalfMirror>(x);
    if (c > 8) x += dpp_row<kDppMirror>(x);
    return x;
}

template <bool BF16>
__global__ __launch_bounds__(256) void zha_leaf_mfma_kernel(
    const void* __restrict__ Kv, const float* __restrict__ Qref,
    float* __restrict__ S, float* __restrict__ B, float* __restrict__ LSE,
    int64_t cap_tok, int64_t cap1, int c, int R, int64_t first_leaf, int64_t n_leaves, float tau,
    float* __restrict__ Sp, float* __restrict__ Bp, float* __restrict__ Lp, int64_t cap2, int fuse) {
    __shared__ __align__(16) float s_k[4][16 * kLmStride];
    __shared__ float s_w[4][16 * 17];
    __shared__ __align__(16) float s_q[16 * kLmStride];
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, q4 = lane >> 4;
    float* sk = s_k[wave];
    float* sw = s_w[wave];

    // the reference queries, the A operand of Z (row j, zero past R; d = 32 q4 + m),
    // staged in LDS once and read per product: held in registers they cost the
    // second resident wave per SIMD
    for (int i = threadIdx.x; i < 16 * (ZHA_D / 4); i += 256) {
        const int r = i / (ZHA_D / 4), v = i - r * (ZHA_D / 4);
        const float4 x = r < R ? reinterpret_cast<const float4*>(Qref + ((size_t)g * R + r) * ZHA_D)[v]
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(s_q + r * kLmStride + 4 * v) = x;
    }
    __syncthreads();
    const float* qrow = s_q + j * kLmStride + 32 * q4;
    const bool big = c > 16;                            // a leaf spans several tiles
    const int lpu = big ? 1 : 16 / c;                   // leaves per unit
    const int tpu = big ? c / 16 : 1;                   // tiles per unit
    const int64_t n_units = (n_leaves + lpu - 1) / lpu;
    const size_t head_row0 = (size_t)g * cap_tok;

    for (int64_t u = (int64_t)blockIdx.x * 4 + wave; u < n_units; u += (int64_t)gridDim.x * 4) {
        const int64_t leaf0 = first_leaf + u * lpu;
        const int nl = (int)min((int64_t)lpu, first_leaf + n_leaves - leaf0);
        const int ntok = big ? 16 : nl * c;              // valid tokens of each tile
        float m_run[4], l_run[4], ez_run[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { m_run[i] = zha_neg_inf(); l_run[i] = 0.f; ez_run[i] = 0.f; }
        zha_f32x4 acc[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) acc[sl] = zha_f32x4{0.f, 0.f, 0.f, 0.f};

        // K row j of a tile, columns 32 q4 .. 32 q4 + 31, as raw 16-byte vectors: the
        // next tile's are requested before the current one is computed
        uint4 raw[BF16 ? 4 : 8];
        auto fetch = [&](int tt) {
#pragma unroll
            for (int v = 0; v < (BF16 ? 4 : 8); ++v) raw[v] = make_uint4(0u, 0u, 0u, 0u);
            if (tt < tpu && j < ntok) {
                const size_t row = head_row0 + (size_t)(leaf0 * c + 16 * tt + j);
                const uint4* src = BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Kv) + row * ZHA_D + 32 * q4)
                                        : reinterpret_cast<const uint4*>(static_cast<const float*>(Kv) + row * ZHA_D + 32 * q4);
#pragma unroll
                for (int v = 0; v < (BF16 ? 4 : 8); ++v) raw[v] = src[v];
            }
        };
        fetch(0);
        for (int tt = 0; tt < tpu; ++tt) {
            // widened exactly (bf16 bits, or float32), then staged in LDS
            float kb[32];
            if (BF16) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t w4[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kb[8 * v + 2 * e] = __uint_as_float(w4[e] << 16);
                        kb[8 * v + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    kb[4 * v] = __uint_as_float(raw[v].x);
                    kb[4 * v + 1] = __uint_as_float(raw[v].y);
                    kb[4 * v + 2] = __uint_as_float(raw[v].z);
                    kb[4 * v + 3] = __uint_as_float(raw[v].w);
                }
            }
            fetch(tt + 1);
#pragma unroll
            for (int v = 0; v < 8; ++v)
                *reinterpret_cast<float4*>(sk + j * kLmStride + 32 * q4 + 4 * v) =
                    make_float4(kb[4 * v], kb[4 * v + 1], kb[4 * v + 2], kb[4 * v + 3]);
            // Z: lane holds refs 4 q4 + i against token j; four independent chains of
            // eight products (a single chain of 32 waits on every product in turn)
            zha_f32x4 zc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) zc[e] = zha_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 32; ++m) zc[m & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[m], kb[m], zc[m & 3], 0, 0, 0);
            zha_f32x4 z4;
#pragma unroll
            for (int i = 0; i < 4; ++i) z4[i] = (zc[0][i] + zc[1][i]) + (zc[2][i] + zc[3][i]);
            const bool tv = j < ntok;
            float w[4];
            float ap[4];                                // this token's leaf's weight in its level-2 node
            if (c <= 16) {
                // one leaf per c lanes: its log-sum-exp, weights and offset
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float z = tv ? tau * z4[i] : zha_neg_inf();
                    const float mx = seg_max(z, c);
                    const float e = (tv && mx != zha_neg_inf()) ? expf(z - mx) : 0.f;
                    const float sum = seg_sum(e, c);
                    const float lse = mx + logf(sum);
                    const float wi = tv ? e / sum : 0.f;
                    const float wz = seg_sum(tv ? wi * z : 0.f, c);
                    w[i] = wi;
                    const int r = 4 * q4 + i;
                    if (tv && (j & (c - 1)) == 0 && r < R) {
                        const size_t o = ((size_t)g * cap1 + (size_t)(leaf0 + j / c)) * R + r;
                        LSE[o] = lse;
                        B[o] = lse - wz;
                    }
                    ap[i] = 0.f;
                    if (fuse) {
                        // the node of c leaves over lanes j / c^2: one lane per leaf segment
                        const int cc = c * c;
                        const bool head = (j & (c - 1)) == 0;
                        const float mp = seg_max(lse, cc);
                        const float sp = seg_sum(head ? expf(lse - mp) : 0.f, cc);
                        const float lp = mp + logf(sp);
                        const float la = lse - lp;              // log a of this lane's leaf
                        const float a = expf(la);
                        const float bp = seg_sum(head ? a * ((lse - wz) - la) : 0.f, cc);
                        ap[i] = a;
                        const int np = j / cc;                  // the node within the unit
                        if ((j & (cc - 1)) == 0 && (np + 1) * cc <= ntok && r < R) {
                            const size_t o = ((size_t)g * cap2 + (size_t)((leaf0 + np * c) / c)) * R + r;
                            Lp[o] = lp;
                            Bp[o] = bp;
                        }
                    }
                }
            } else {
                // online across the leaf's tiles
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float z = tau * z4[i];
                    const float mt = seg_max(z, 16);
                    const float mn = fmaxf(m_run[i], mt);
                    const float alpha = expf(m_run[i] - mn);   // 0 on the first tile
                    const float e = expf(z - mn);
                    const float es = seg_sum(e, 16), ezs = seg_sum(e * z, 16);
                    l_run[i] = l_run[i] * alpha + es;
                    ez_run[i] = ez_run[i] * alpha + ezs;
                    m_run[i] = mn;
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) acc[sl][i] *= alpha;
                    w[i] = e;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sw[(4 * q4 + i) * 17 + j] = w[i];
            zha_wave_lds_sync();
            // S: the tile's tokens in groups of four (kk), each slice of 16 columns
            if (c > 16) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = sw[j * 17 + 4 * kk + q4];
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl)
                        acc[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sk[(4 * kk + q4) * kLmStride + 16 * sl + j],
                                                                       acc[sl], 0, 0, 0);
                }
            } else {
                for (int f = 0; f < nl; ++f) {
                    zha_f32x4 o[8];
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) o[sl] = zha_f32x4{0.f, 0.f, 0.f, 0.f};
                    const int kk0 = (f * c) >> 2, kk1 = ((f + 1) * c - 1) >> 2;
                    for (int kk = kk0; kk <= kk1; ++kk) {
                        const int tok = 4 * kk + q4;
                        const float a = (tok >= f * c && tok < (f + 1) * c) ? sw[j * 17 + tok] : 0.f;
#pragma unroll
                        for (int sl = 0; sl < 8; ++sl)
                            o[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sk[tok * kLmStride + 16 * sl + j], o[sl],
                                                                         0, 0, 0);
                    }
                    float* so = S + ((size_t)g * cap1 + (size_t)(leaf0 + f)) * R * ZHA_D;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * q4 + i;
                        if (r < R)
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl) so[r * ZHA_D + 16 * sl + j] = o[sl][i];
                    }
                }
                if (fuse) {
                    // the unit's whole level-2 nodes: tokens weighted by a w
                    const int cc = c * c;
                    zha_wave_lds_sync();                // every read of sw above is done
#pragma unroll
                    for (int i = 0; i < 4; ++i) sw[(4 * q4 + i) * 17 + j] = w[i] * ap[i];
                    zha_wave_lds_sync();
                    // (acc, the running sums of leaves longer than a tile, is free here)
                    for (int np = 0; (np + 1) * cc <= ntok; ++np) {
#pragma unroll
                        for (int sl = 0; sl < 8; ++sl) acc[sl] = zha_f32x4{0.f, 0.f, 0.f, 0.f};
                        for (int kk = (np * cc) >> 2; kk <= ((np + 1) * cc - 1) >> 2; ++kk) {
                            const int tok = 4 * kk + q4;
                            const float a = (tok >= np * cc && tok < (np + 1) * cc) ? sw[j * 17 + tok] : 0.f;
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl)
                                acc[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sk[tok * kLmStride + 16 * sl + j],
                                                                               acc[sl], 0, 0, 0);
                        }
                        float* po = Sp + ((size_t)g * cap2 + (size_t)((leaf0 + np * c) / c)) * R * ZHA_D;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 4 * q4 + i;
                            if (r < R)
#pragma unroll
                                for (int sl = 0; sl < 8; ++sl) po[r * ZHA_D + 16 * sl + j] = acc[sl][i];
                        }
                    }
                }
            }
            zha_wave_lds_sync();                        // the next tile overwrites sk, sw
        }
        if (big) {
            float* so = S + ((size_t)g * cap1 + (size_t)leaf0) * R * ZHA_D;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q4 + i;
                if (r < R) {
                    const float inv = 1.f / l_run[i];
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) so[r * ZHA_D + 16 * sl + j] = acc[sl][i] * inv;
                    if (j == 0) {
                        const size_t o = ((size_t)g * cap1 + (size_t)leaf0) * R + r;
                        const float lse = m_run[i] + logf(l_run[i]);
                        LSE[o] = lse;
                        B[o] = lse - ez_run[i] * inv;
                    }
                }
            }
        }

    }
}

// ---- one reference query, short leaves (R = 1, c <= 16, bfloat16 keys): a streaming
// kernel.  Lane l of a wave takes leaf l / 8 of the wave's eight and dims 16 (l % 8) ..
// 16 (l % 8) + 15: it loads those 16 dims of each of the leaf's c key rows (the eight
// lanes of a leaf read each row's 256 bytes together), forms its part of every logit,
// and the leaf's eight lanes add the parts with a DPP butterfly (the same sum in each
// lane); each lane then forms the softmax of the c logits and the weighted mean of
// its own 16 dims.  No LDS staging and no barrier: the kernel streams the keys once.
constexpr int kR1MaxC = 16;
template <int CMAX>
__global__ __launch_bounds__(256) void zha_leaf_r1_kernel(
    const uint16_t* __restrict__ K, const float* __restrict__ Qref,
    float* __restrict__ S, float* __restrict__ B, float* __restrict__ LSE,
    int64_t cap_tok, int64_t cap1, int c, int64_t first_leaf, int64_t n_leaves, float tau) {
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sl = lane & 7;                             // dims 16 sl .. 16 sl + 15
    float qv[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 x = reinterpret_cast<const float4*>(Qref + (size_t)g * ZHA_D + 16 * sl)[v];
        qv[4 * v] = x.x; qv[4 * v + 1] = x.y; qv[4 * v + 2] = x.z; qv[4 * v + 3] = x.w;
    }
    for (int64_t lb = ((int64_t)blockIdx.x * 4 + wave) * 8; lb < n_leaves; lb += (int64_t)gridDim.x * 32) {
        const int64_t lf = lb + (lane >> 3);
        const bool ok = lf < n_leaves;
        const int64_t leaf = first_leaf + (ok ? lf : n_leaves - 1);
        const uint16_t* row = K + ((size_t)g * cap_tok + (size_t)leaf * c) * ZHA_D + 16 * sl;
        uint4 kr[CMAX][2];
#pragma unroll
        for (int t = 0; t < CMAX; ++t) {
            if (t < c) {
                kr[t][0] = reinterpret_cast<const uint4*>(row + (size_t)t * ZHA_D)[0];
                kr[t][1] = reinterpret_cast<const uint4*>(row + (size_t)t * ZHA_D)[1];
            }
        }
        // logits: this lane's 16-dim parts, then the leaf's eight lanes summed
        float z[CMAX];
        float m = zha_neg_inf();
#pragma unroll
        for (int t = 0; t < CMAX; ++t) {
            if (t < c) {
                float acc = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t w4[4] = {kr[t][h].x, kr[t][h].y, kr[t][h].z, kr[t][h].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(qv[8 * h + 2 * e], __uint_as_float(w4[e] << 16), acc);
                        acc = fmaf(qv[8 * h + 2 * e + 1], __uint_as_float(w4[e] & 0xFFFF0000u), acc);
                    }
                }
                z[t] = tau * seg_sum(acc, 8);
                m = fmaxf(m, z[t]);
            }
        }
        float l = 0.f;
#pragma unroll
        for (int t = 0; t < CMAX; ++t)
            if (t < c) l += expf(z[t] - m);
        const float lse = m + logf(l);
        // the keys are decoded again below rather than held as floats across the softmax
#pragma unroll
        for (int t = 0; t < CMAX; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                asm volatile("" : "+v"(kr[t][h].x), "+v"(kr[t][h].y), "+v"(kr[t][h].z), "+v"(kr[t][h].w));
        float ez = 0.f;
        float sv[16];
#pragma unroll
        for (int d = 0; d < 16; ++d) sv[d] = 0.f;
#pragma unroll
        for (int t = 0; t < CMAX; ++t) {
            if (t < c) {
                const float w = expf(z[t] - lse);
                ez = fmaf(w, z[t], ez);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t w4[4] = {kr[t][h].x, kr[t][h].y, kr[t][h].z, kr[t][h].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sv[8 * h + 2 * e] = fmaf(w, __uint_as_float(w4[e] << 16), sv[8 * h + 2 * e]);
                        sv[8 * h + 2 * e + 1] = fmaf(w, __uint_as_float(w4[e] & 0xFFFF0000u), sv[8 * h + 2 * e + 1]);
                    }
                }
            }
        }
        if (ok) {
            float4* so = reinterpret_cast<float4*>(S + ((size_t)g * cap1 + (size_t)leaf) * ZHA_D + 16 * sl);
#pragma unroll
            for (int v = 0; v < 4; ++v) so[v] = make_float4(sv[4 * v], sv[4 * v + 1], sv[4 * v + 2], sv[4 * v + 3]);
            if (sl == 0) {
                const size_t o = (size_t)g * cap1 + (size_t)leaf;
                LSE[o] = lse;
                B[o] = lse - ez;
            }
        }
    }
}

// ---- long leaves (c a multiple of 32, R <= 16, bfloat16 keys) on bfloat16 products.
//
// The reference queries and the softmax weights enter as three bfloat16 parts each
// (hi + mid + lo is a float32 value exactly: each part is the remainder cut to its
// leading 8 significant bits, each remainder is exact (the part and what it is cut
// from share sign and exponent, so their difference is exact by Sterbenz's lemma),
// and what is left after two parts has at most 8 significant bits), the keys as they
// are; the float32 sums of the parts' products are those of the float32 products,
// at an eighth of the matrix work.  One wave per leaf, tiles of 32 tokens.  Per tile:
//   Z = tau Q K^T    per 16-token half h and 32-dim block kb, one
//                    v_mfma_f32_16x16x32_bf16 per query part (A: Q part row j, dims
//                    32 kb + 8 q .. + 7, from LDS; B: key row 16 h + j, the same dims,
//                    straight from the lane's 16-byte loads);
//   online softmax of the lane's refs 4 q + i over the tile's 32 tokens;
//   S += W K         the contraction over the tile's tokens is permuted (index 8 q + e
//                    is token 4 e + q) so that each lane's B operand comes from its own
//                    16-byte loads of rows 4 e + q, dims 8 j .. 8 j + 7, and output
//                    column j of block c8 is dim 8 j + c8 (as in the gather's PV).
// Outputs as the other leaf kernels: S[leaf][r][d], B, LSE (rows r < R).
typedef unsigned int zha_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kB3QRow = 68;        // LDS row of a query part (u32, two bf16 each): 16-byte aligned

// x = h + m + l exactly, as float32 bit patterns whose low 16 bits are zero (the
// bfloat16 values in their high halves).
__device__ __forceinline__ void split3_bf16(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
    h = __float_as_uint(x) & 0xFFFF0000u;
    const float r1 = x - __uint_as_float(h);
    m = __float_as_uint(r1) & 0xFFFF0000u;
    l = __float_as_uint(r1 - __uint_as_float(m));
}
// The bfloat16 pair {a, b} (a in the low half) from two such patterns.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ uint32_t b3_word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__global__ __launch_bounds__(256) void zha_leaf_b3_kernel(
    const uint16_t* __restrict__ K, const float* __restrict__ Qref,
    float* __restrict__ S, float* __restrict__ B, float* __restrict__ LSE,
    int64_t cap_tok, int64_t cap1, int c, int R, int64_t first_leaf, int64_t n_leaves, float tau) {
    __shared__ __align__(16) uint32_t s_q[3][16 * kB3QRow];
    __shared__ float s_w[4][16 * 33];
    __shared__ __align__(16) uint32_t s_k[4][32 * kB3QRow];   // a wave's key tile: 32 rows of 64 words (+4)
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, q = lane >> 4;
    float* sw = s_w[wave];
    uint32_t* sk = s_k[wave];
    // the reference queries' three parts, rows past R zero
    for (int i = threadIdx.x; i < 16 * (ZHA_D / 2); i += 256) {
        const int r = i / (ZHA_D / 2), dp = i - r * (ZHA_D / 2);
        float2 v = make_float2(0.f, 0.f);
        if (r < R) v = reinterpret_cast<const float2*>(Qref + ((size_t)g * R + r) * ZHA_D)[dp];
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(v.x, h0, m0, l0);
        split3_bf16(v.y, h1, m1, l1);
        s_q[0][r * kB3QRow + dp] = bf16_pair(h0, h1);
        s_q[1][r * kB3QRow + dp] = bf16_pair(m0, m1);
        s_q[2][r * kB3QRow + dp] = bf16_pair(l0, l1);
    }
    __syncthreads();
    const int tpl = c / 32;
    for (int64_t lf = (int64_t)blockIdx.x * 4 + wave; lf < n_leaves; lf += (int64_t)gridDim.x * 4) {
        const int64_t leaf = first_leaf + lf;
        const size_t row0 = (size_t)g * cap_tok + (size_t)leaf * c;
        float m_run[4], l_run[4], ez_run[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { m_run[i] = zha_neg_inf(); l_run[i] = 0.f; ez_run[i] = 0.f; }
        zha_f32x4 acc[8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) acc[c8] = zha_f32x4{0.f, 0.f, 0.f, 0.f};
        // a tile's 32 key rows, loaded once and whole (lane l: 16-byte pieces l + 64 m,
        // rows 4 m + l / 16), staged in the wave's LDS tile and read back in the two
        // operand layouts; the next tile's pieces are requested before the current one
        // is computed
        // (the last tile requests itself again: every load stays in the leaf)
        const uint16_t* kt = K + (row0 + (size_t)(lane >> 4)) * ZHA_D + 8 * (lane & 15);
        zha_u32x4 raw[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) raw[m] = *reinterpret_cast<const zha_u32x4*>(kt + (size_t)(4 * m) * ZHA_D);
        for (int tt = 0; tt < tpl; ++tt) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
                *reinterpret_cast<zha_u32x4*>(sk + (4 * m + (lane >> 4)) * kB3QRow + 4 * (lane & 15)) = raw[m];
            zha_wave_lds_sync();
            const int tn = tt + 1 < tpl ? tt + 1 : tt;
#pragma unroll
            for (int m = 0; m < 8; ++m)
                raw[m] = *reinterpret_cast<const zha_u32x4*>(kt + (size_t)(32 * tn + 4 * m) * ZHA_D);
            // key rows 16 h + j, dims 32 kb + 8 q .. + 7 (the B operand of Q K^T)
            uint4 kz[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    kz[h][kb] = *reinterpret_cast<const uint4*>(sk + (16 * h + j) * kB3QRow + 4 * (4 * kb + q));
            // Z: four independent accumulator chains (half h, parts alternating)
            zha_f32x4 zz[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2) zz[h][a2] = zha_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int pt = 0; pt < 3; ++pt) {
                    const zha_bf16x8 qa = zha_as_bf16x8(*reinterpret_cast<const uint4*>(&s_q[pt][j * kB3QRow + 16 * kb + 4 * q]));
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        zz[h][(kb * 3 + pt) & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, zha_as_bf16x8(kz[h][kb]),
                                                                                           zz[h][(kb * 3 + pt) & 1], 0, 0, 0);
                }
            }
            // online softmax of refs 4 q + i over tokens j and 16 + j; the sums are
            // rescaled only on tiles that raise some lane's running maximum
            float alph[4];
            bool grew = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z0 = tau * (zz[0][0][i] + zz[0][1][i]);
                const float z1 = tau * (zz[1][0][i] + zz[1][1][i]);
                const float mt = seg_max(fmaxf(z0, z1), 16);
                const float mn = fmaxf(m_run[i], mt);
                const float alpha = expf(m_run[i] - mn);   // 0 on the first tile
                const float e0 = expf(z0 - mn), e1 = expf(z1 - mn);
                const float es = seg_sum(e0 + e1, 16), ezs = seg_sum(e0 * z0 + e1 * z1, 16);
                l_run[i] = l_run[i] * alpha + es;
                ez_run[i] = ez_run[i] * alpha + ezs;
                m_run[i] = mn;
                alph[i] = alpha;
                grew |= alpha != 1.0f;
                sw[(4 * q + i) * 33 + j] = e0;
                sw[(4 * q + i) * 33 + 16 + j] = e1;
            }
            if (__ballot(grew) != 0ull) {
#pragma unroll
                for (int c8 = 0; c8 < 8; ++c8)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[c8][i] *= alph[i];
            }
            zha_wave_lds_sync();
            // rows 4 e + q of the tile, dims 8 j .. 8 j + 7 (the B operand of W K)
            uint4 kv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[e] = *reinterpret_cast<const uint4*>(sk + (4 * e + q) * kB3QRow + 4 * j);
            // W (row j, tokens 4 e + q) in three parts; B from the tile's rows
            uint32_t wp[3][4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                uint32_t ha, ma, la, hb, mb, lb;
                split3_bf16(sw[j * 33 + 4 * (2 * e2) + q], ha, ma, la);
                split3_bf16(sw[j * 33 + 4 * (2 * e2 + 1) + q], hb, mb, lb);
                wp[0][e2] = bf16_pair(ha, hb);
                wp[1][e2] = bf16_pair(ma, mb);
                wp[2][e2] = bf16_pair(la, lb);
            }
            const zha_bf16x8 wa0 = zha_as_bf16x8(make_uint4(wp[0][0], wp[0][1], wp[0][2], wp[0][3]));
            const zha_bf16x8 wa1 = zha_as_bf16x8(make_uint4(wp[1][0], wp[1][1], wp[1][2], wp[1][3]));
            const zha_bf16x8 wa2 = zha_as_bf16x8(make_uint4(wp[2][0], wp[2][1], wp[2][2], wp[2][3]));
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) {
                const int wsel = c8 >> 1;
                const uint32_t sel = (c8 & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
                uint32_t bw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    bw[e2] = __builtin_amdgcn_perm(b3_word(kv[2 * e2 + 1], wsel), b3_word(kv[2 * e2], wsel), sel);
                const zha_bf16x8 bv = zha_as_bf16x8(make_uint4(bw[0], bw[1], bw[2], bw[3]));
                acc[c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa0, bv, acc[c8], 0, 0, 0);
                acc[c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa1, bv, acc[c8], 0, 0, 0);
                acc[c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa2, bv, acc[c8], 0, 0, 0);
            }
            zha_wave_lds_sync();                        // the next tile rewrites sw and sk
        }
        // S[leaf][r][8 j .. 8 j + 7] = acc / l; B and LSE from the running sums
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * q + i;
            if (r < R) {
                const float inv = 1.f / l_run[i];
                float4* so = reinterpret_cast<float4*>(S + (((size_t)g * cap1 + (size_t)leaf) * R + r) * ZHA_D + 8 * j);
                so[0] = make_float4(acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv);
                so[1] = make_float4(acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv, acc[7][i] * inv);
                if (j == 0) {
                    const size_t o = ((size_t)g * cap1 + (size_t)leaf) * R + r;
                    const float lse = m_run[i] + logf(l_run[i]);
                    LSE[o] = lse;
                    B[o] = lse - ez_run[i] * inv;
                }
            }
        }
    }
}

// Merges np parents (local index pl) from their c children each, as the whole
// workgroup: per (parent, plane) its LSE and b, with the children's weights a_j
// kept in a_s [np][R][c], then its weighted mean s.  A child's (L, B) comes from
// cl(pl, r, j) and its s from cs(pl, r, j, d4) (float4 d4 of the plane); results go
// to wl(pl, r, L, B) and ws(pl, r, d4, s).  CMAX > 0: c <= CMAX, and each thread
// loads all of its c children before it combines them (the loads overlap); CMAX ==
// 0: any c, one child at a time.  The arithmetic and its order are the same in
// both forms and for every caller.  Ends with a barrier.
template <int CMAX, class CL, class CS, class WL, class WS>
__device__ __forceinline__ void merge_block(int np, int c, int R, float* a_s, CL&& cl, CS&& cs, WL&& wl, WS&& ws) {
    const int tid = threadIdx.x;
    const int per_parent = R * (ZHA_D / 4);              // float4 outputs per parent
    for (int pr = tid; pr < np * R; pr += blockDim.x) {
        const int pl = pr / R, r = pr - pl * R;
        float m = zha_neg_inf(), sum = 0.f, bp = 0.f;
        float* a = a_s + (pl * R + r) * c;
        if constexpr (CMAX > 0) {
            float lv[CMAX], bv[CMAX];
#pragma unroll
            for (int j = 0; j < CMAX; ++j)
                if (j < c) {
                    const float2 t = cl(pl, r, j);
                    lv[j] = t.x;
                    bv[j] = t.y;
                }
#pragma unroll
            for (int j = 0; j < CMAX; ++j)
                if (j < c) m = fmaxf(m, lv[j]);
#pragma unroll
            for (int j = 0; j < CMAX; ++j)
                if (j < c) sum += expf(lv[j] - m);
            const float lse = m + logf(sum);
#pragma unroll
            for (int j = 0; j < CMAX; ++j) {
                if (j < c) {
                    const float la = lv[j] - lse;                // log a_j
                    const float aj = expf(la);
                    a[j] = aj;
                    bp = fmaf(aj, bv[j] - la, bp);
                }
            }
            m = lse;
        } else {
            for (int j = 0; j < c; ++j) m = fmaxf(m, cl(pl, r, j).x);
            for (int j = 0; j < c; ++j) sum += expf(cl(pl, r, j).x - m);
            const float lse = m + logf(sum);
            for (int j = 0; j < c; ++j) {
                const float2 t = cl(pl, r, j);
                const float la = t.x - lse;                      // log a_j
                const float aj = expf(la);
                a[j] = aj;
                bp = fmaf(aj, t.y - la, bp);
            }
            m = lse;
        }
        wl(pl, r, m, bp);
    }
    __syncthreads();
    for (int o = tid; o < np * per_parent; o += blockDim.x) {
        const int pl = o / per_parent, rem = o - pl * per_parent;
        const int r = rem / (ZHA_D / 4), d4 = rem - r * (ZHA_D / 4);
        const float* a = a_s + (pl * R + r) * c;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (CMAX > 0) {
            float4 sv[CMAX];
#pragma unroll
            for (int j = 0; j < CMAX; ++j)
                if (j < c) sv[j] = cs(pl, r, j, d4);
#pragma unroll
            for (int j = 0; j < CMAX; ++j) {
                if (j < c) {
                    acc.x = fmaf(a[j], sv[j].x, acc.x);
                    acc.y = fmaf(a[j], sv[j].y, acc.y);
                    acc.z = fmaf(a[j], sv[j].z, acc.z);
                    acc.w = fmaf(a[j], sv[j].w, acc.w);
                }
            }
        } else {
            for (int j = 0; j < c; ++j) {
                const float4 t = cs(pl, r, j, d4);
                acc.x = fmaf(a[j], t.x, acc.x);
                acc.y = fmaf(a[j], t.y, acc.y);
                acc.z = fmaf(a[j], t.z, acc.z);
                acc.w = fmaf(a[j], t.w, acc.w);
            }
        }
        ws(pl, r, d4, acc);
    }
    __syncthreads();
}

// grid (ceil(n_parents / parents_per_block), H_kv), 256 threads: parents
// first_parent .. + n_parents of one level from their children one level down.
template <int CMAX>
__global__ __launch_bounds__(256) void zha_merge_kernel(
    const float* __restrict__ Sc, const float* __restrict__ Bc, const float* __restrict__ Lc,
    float* __restrict__ Sp, float* __restrict__ Bp, float* __restrict__ Lp,
    int64_t cap_c, int64_t cap_p, int c, int R, int64_t first_parent, int64_t n_parents) {
    extern __shared__ float a_s[];                       // [ppb][R][c]
    const int g = blockIdx.y;
    const int per_parent = R * (ZHA_D / 4);
    const int ppb = per_parent >= 256 ? 1 : 256 / per_parent;
    const int64_t p0 = first_parent + (int64_t)blockIdx.x * ppb;
    const int64_t end = first_parent + n_parents;
    if (p0 >= end) return;
    const int np = (int)min((int64_t)ppb, end - p0);
    const size_t step = (size_t)R * (ZHA_D / 4);         // float4s from one child to the next
    merge_block<CMAX>(
        np, c, R, a_s,
        [&](int pl, int r, int j) {
            const size_t o = ((size_t)g * cap_c + (size_t)((p0 + pl) * c)) * R + r + (size_t)j * R;
            return make_float2(Lc[o], Bc[o]);
        },
        [&](int pl, int r, int j, int d4) {
            const float4* sc = reinterpret_cast<const float4*>(
                Sc + (((size_t)g * cap_c + (size_t)((p0 + pl) * c)) * R + r) * ZHA_D) + d4;
            return sc[(size_t)j * step];
        },
        [&](int pl, int r, float lse, float b) {
            const size_t op = ((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r;
            Lp[op] = lse;
            Bp[op] = b;
        },
        [&](int pl, int r, int d4, float4 v) {
            reinterpret_cast<float4*>(Sp + (((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r) * ZHA_D)[d4] = v;
        });
}

// grid (n_grand, H_kv), 256 threads: two levels at once.  Workgroup k merges the
// c children of grandparent first_grand + k (level l, written out and kept in
// LDS) from their own children (level l - 1), then the grandparent (level l + 1)
// from those: the same merge, so the same values as two merge launches, in one.
// LDS: [c][R] L and B, [c][R][128] s of the middle level, and the weights.
template <int CMAX>
__global__ __launch_bounds__(256) void zha_merge2_kernel(
    const float* __restrict__ Sc, const float* __restrict__ Bc, const float* __restrict__ Lc,
    float* __restrict__ Sp, float* __restrict__ Bp, float* __restrict__ Lp,
    float* __restrict__ Sg, float* __restrict__ Bg, float* __restrict__ Lg,
    int64_t cap_c, int64_t cap_p, int64_t cap_g, int c, int R, int64_t first_grand) {
    extern __shared__ float m_s[];
    float* sL = m_s;                                     // [c][R]
    float* sB = sL + c * R;                              // [c][R]
    float4* sS = reinterpret_cast<float4*>(sB + c * R + ((4 - (2 * c * R) % 4) % 4));   // [c][R][32]
    float* a_s = reinterpret_cast<float*>(sS + (size_t)c * R * (ZHA_D / 4));            // [c][R][c]
    const int g = blockIdx.y;
    const int64_t gp = first_grand + blockIdx.x;
    const int64_t p0 = gp * c;                           // its first child (middle level)
    const size_t step = (size_t)R * (ZHA_D / 4);
    merge_block<CMAX>(
        c, c, R, a_s,
        [&](int pl, int r, int j) {
            const size_t o = ((size_t)g * cap_c + (size_t)((p0 + pl) * c)) * R + r + (size_t)j * R;
            return make_float2(Lc[o], Bc[o]);
        },
        [&](int pl, int r, int j, int d4) {
            const float4* sc = reinterpret_cast<const float4*>(
                Sc + (((size_t)g * cap_c + (size_t)((p0 + pl) * c)) * R + r) * ZHA_D) + d4;
            return sc[(size_t)j * step];
        },
        [&](int pl, int r, float lse, float b) {
            const size_t op = ((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r;
            Lp[op] = lse;
            Bp[op] = b;
            sL[pl * R + r] = lse;
            sB[pl * R + r] = b;
        },
        [&](int pl, int r, int d4, float4 v) {
            reinterpret_cast<float4*>(Sp + (((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r) * ZHA_D)[d4] = v;
            sS[((size_t)pl * R + r) * (ZHA_D / 4) + d4] = v;
        });
    merge_block<CMAX>(
        1, c, R, a_s,
        [&](int, int r, int j) { return make_float2(sL[j * R + r], sB[j * R + r]); },
        [&](int, int r, int j, int d4) { return sS[((size_t)j * R + r) * (ZHA_D / 4) + d4]; },
        [&](int, int r, float lse, float b) {
            const size_t og = ((size_t)g * cap_g + (size_t)gp) * R + r;
            Lg[og] = lse;
            Bg[og] = b;
        },
        [&](int, int r, int d4, float4 v) {
            reinterpret_cast<float4*>(Sg + (((size_t)g * cap_g + (size_t)gp) * R + r) * ZHA_D)[d4] = v;
        });
}

// grid (blocks, H_kv), 256 threads: S16 <- bfloat16(S), round to nearest, ties to
// even, over one KV head's contiguous planes of nodes [first, first + n), four
// elements per thread step.  Planes are finite, so no NaN case arises.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__global__ __launch_bounds__(256) void zha_planes16_kernel(const float* __restrict__ S, uint16_t* __restrict__ S16,
                                                          int64_t cap, int R, int64_t first, int64_t n) {
    const int g = blockIdx.y;
    const size_t row = (size_t)R * ZHA_D;               // elements per node
    const size_t base = ((size_t)g * cap + (size_t)first) * row;
    const size_t count4 = (size_t)n * row / 4;
    const float4* src = reinterpret_cast<const float4*>(S + base);
    uint2* dst = reinterpret_cast<uint2*>(S16 + base);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < count4; i += (size_t)gridDim.x * 256) {
        const float4 v = src[i];
        dst[i] = make_uint2(f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16),
                            f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16));
    }
}

// grid (blocks, H_kv), 256 threads: the router's 8-bit copy of the planes s of
// nodes [first, first + n), one wave per plane (R per node), two elements per lane.
// Per plane: k, the exponent of the smallest power of two with max_d |s_d| <= 448
// 2^k (k >= -126; 0 for an all-zero plane), SC <- 2^k, and S8 <- the FP8 E4M3
// codes (sign, 4 exponent bits of bias 7, 3 mantissa bits, subnormals below 2^-6,
// largest 448) of s_d / 2^k, rounded to nearest, ties to even.
__device__ __forceinline__ int fp8_scale_exp(float m) {
    if (m == 0.f) return 0;
    const uint32_t u = __float_as_uint(m);
    const int e = (int)((u >> 23) & 0xFFu) - 127;              // m = 1.f 2^e
    const int k = (u & 0x7FFFFFu) <= 0x600000u ? e - 8 : e - 7;  // 1.f <= 1.75: 448 2^(e-8) >= m
    return k < -126 ? -126 : k;
}
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float x) {     // |x| <= 448
    const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);          // spacing 2^-9; 8 is the smallest normal
    } else {
        const uint32_t u = __float_as_uint(a);
        const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);    // three mantissa bits, ties to even
        code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    }
    return sgn | code;
}
__global__ __launch_bounds__(256) void zha_planes8_kernel(const float* __restrict__ S, uint8_t* __restrict__ S8,
                                                         float* __restrict__ SC, int64_t cap, int R, int64_t first,
                                                         int64_t n) {
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const size_t p0 = ((size_t)g * (size_t)cap + (size_t)first) * (size_t)R;
    const size_t np = (size_t)n * (size_t)R;
    for (size_t i = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < np; i += (size_t)gridDim.x * 4) {
        const size_t p = p0 + i;
        const float2 v = reinterpret_cast<const float2*>(S + p * ZHA_D)[lane];
        float m = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const int k = fp8_scale_exp(m);
        const uint32_t lo = f32_to_e4m3_rne(ldexpf(v.x, -k)), hi = f32_to_e4m3_rne(ldexpf(v.y, -k));
        reinterpret_cast<uint16_t*>(S8 + p * ZHA_D)[lane] = (uint16_t)(lo | (hi << 8));
        if (lane == 0) SC[p] = ldexpf(1.0f, k);
    }
}

// grid (H_kv), 128 threads: row `row` of K and V <- k_new, v_new.
template <typename T>
__global__ void zha_kv_write_kernel(T* __restrict__ K, T* __restrict__ V, const T* __restrict__ kn,
                                    const T* __restrict__ vn, int64_t cap_tok, int64_t row) {
    const int g = blockIdx.x;
    for (int d = threadIdx.x; d < ZHA_D; d += blockDim.x) {
        K[((size_t)g * cap_tok + (size_t)row) * ZHA_D + d] = kn[g * ZHA_D + d];
        V[((size_t)g * cap_tok + (size_t)row) * ZHA_D + d] = vn[g * ZHA_D + d];
    }
}

}  // namespace

size_t zha_leaf_summary_lds_bytes(int R) {
    return sizeof(float) * ((size_t)R * ZHA_D + (size_t)kTile * kKStride + (size_t)R * kTile + 4 * (size_t)R);
}

hipError_t zha_launch_leaf_summary(int kv_dtype, const void* K, const float* Qref, float* S, float* B,
                                   float* LSE, int H_kv, int64_t cap_tok, int64_t cap1, int c, int R,
                                   int64_t first_leaf, int64_t n_leaves, float tau, float* Sp, float* Bp, float* Lp,
                                   int64_t cap2, int* fused, hipStream_t stream) {
    if (fused) *fused = 0;
    if (n_leaves <= 0) return hipSuccess;
    const bool aligned = Sp != nullptr && fused != nullptr && first_leaf % c == 0;
    if (kv_dtype == 0 && R == 1 && c <= kR1MaxC) {
        // one reference query, short leaves: the streaming kernel, 32 leaves per workgroup
        int64_t blocks = (n_leaves + 31) / 32;
        if (blocks > 4096) blocks = 4096;
        const dim3 grid((unsigned)blocks, (unsigned)H_kv);
        const uint16_t* K16 = static_cast<const uint16_t*>(K);
        if (c <= 8)
            hipLaunchKernelGGL(zha_leaf_r1_kernel<8>, grid, dim3(256), 0, stream, K16, Qref, S, B, LSE, cap_tok, cap1,
                               c, first_leaf, n_leaves, tau);
        else
            hipLaunchKernelGGL(zha_leaf_r1_kernel<16>, grid, dim3(256), 0, stream, K16, Qref, S, B, LSE, cap_tok, cap1,
                               c, first_leaf, n_leaves, tau);
        return hipGetLastError();
    }
    if (kv_dtype == 0 && R >= kLmMinR && R <= 16 && c % 32 == 0) {
        // long leaves, bfloat16 keys: bfloat16 products in three parts, four leaves
        // per workgroup
        int64_t blocks = (n_leaves + 3) / 4;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(zha_leaf_b3_kernel, dim3((unsigned)blocks, (unsigned)H_kv), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(K), Qref, S, B, LSE, cap_tok, cap1, c, R, first_leaf, n_leaves,
                           tau);
        return hipGetLastError();
    }
    if (R >= kLmMinR && R <= 16 && (c & (c - 1)) == 0) {
        // matrix-core kernel: units of 16 tokens (c <= 16) or whole leaves, four per workgroup
        const int64_t lpu = c <= 16 ? 16 / c : 1;
        const int64_t units = (n_leaves + lpu - 1) / lpu;
        int64_t blocks = (units + 3) / 4;
        if (blocks > 2048) blocks = 2048;
        dim3 grid((unsigned)blocks, (unsigned)H_kv);
        const int fuse = aligned && (c == 2 || c == 4) ? 1 : 0;
        if (kv_dtype == 0)
            hipLaunchKernelGGL(zha_leaf_mfma_kernel<true>, grid, dim3(256), 0, stream, K, Qref, S, B, LSE, cap_tok,
                               cap1, c, R, first_leaf, n_leaves, tau, Sp, Bp, Lp, cap2, fuse);
        else
            hipLaunchKernelGGL(zha_leaf_mfma_kernel<false>, grid, dim3(256), 0, stream, K, Qref, S, B, LSE, cap_tok,
                               cap1, c, R, first_leaf, n_leaves, tau, Sp, Bp, Lp, cap2, fuse);
        if (fuse) *fused = 1;
        return hipGetLastError();
    }
    const int64_t lpb = c <= kTile ? kTile / c : 1;
    dim3 grid((unsigned)((n_leaves + lpb - 1) / lpb), (unsigned)H_kv);
    size_t lds = zha_leaf_summary_lds_bytes(R);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_leaf_summary_kernel<true>, grid, dim3(256), lds, stream, K, Qref, S, B, LSE,
                           cap_tok, cap1, c, R, first_leaf, n_leaves, tau);
    else
        hipLaunchKernelGGL(zha_leaf_summary_kernel<false>, grid, dim3(256), lds, stream, K, Qref, S, B, LSE,
                           cap_tok, cap1, c, R, first_leaf, n_leaves, tau);
    return hipGetLastError();
}

size_t zha_merge_lds_bytes(int c, int R) {
    const int per_parent = R * (ZHA_D / 4);
    const int ppb = per_parent >= 256 ? 1 : 256 / per_parent;
    return sizeof(float) * (size_t)ppb * R * c;
}

hipError_t zha_launch_merge(const float* Sc, const float* Bc, const float* Lc, float* Sp, float* Bp, float* Lp,
                            int H_kv, int64_t cap_c, int64_t cap_p, int c, int R, int64_t first_parent,
                            int64_t n_parents, hipStream_t stream) {
    if (n_parents <= 0) return hipSuccess;
    const int per_parent = R * (ZHA_D / 4);
    const int64_t ppb = per_parent >= 256 ? 1 : 256 / per_parent;
    dim3 grid((unsigned)((n_parents + ppb - 1) / ppb), (unsigned)H_kv);
    const size_t lds = zha_merge_lds_bytes(c, R);
    if (c <= 8)
        hipLaunchKernelGGL(zha_merge_kernel<8>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, cap_c, cap_p,
                           c, R, first_parent, n_parents);
    else if (c <= 16)
        hipLaunchKernelGGL(zha_merge_kernel<16>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, cap_c, cap_p,
                           c, R, first_parent, n_parents);
    else
        hipLaunchKernelGGL(zha_merge_kernel<0>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, cap_c, cap_p,
                           c, R, first_parent, n_parents);
    return hipGetLastError();
}

size_t zha_merge2_lds_bytes(int c, int R) {
    return sizeof(float) * (size_t)(2 * c * R + 4 + c * R * ZHA_D + c * R * c);
}

hipError_t zha_launch_merge2(const float* Sc, const float* Bc, const float* Lc, float* Sp, float* Bp, float* Lp,
                             float* Sg, float* Bg, float* Lg, int H_kv, int64_t cap_c, int64_t cap_p, int64_t cap_g,
                             int c, int R, int64_t first_grand, int64_t n_grand, hipStream_t stream) {
    if (n_grand <= 0) return hipSuccess;
    const size_t lds = zha_merge2_lds_bytes(c, R);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    dim3 grid((unsigned)n_grand, (unsigned)H_kv);
    if (c <= 8)
        hipLaunchKernelGGL(zha_merge2_kernel<8>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, Sg, Bg, Lg,
                           cap_c, cap_p, cap_g, c, R, first_grand);
    else if (c <= 16)
        hipLaunchKernelGGL(zha_merge2_kernel<16>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, Sg, Bg, Lg,
                           cap_c, cap_p, cap_g, c, R, first_grand);
    else
        hipLaunchKernelGGL(zha_merge2_kernel<0>, grid, dim3(256), lds, stream, Sc, Bc, Lc, Sp, Bp, Lp, Sg, Bg, Lg,
                           cap_c, cap_p, cap_g, c, R, first_grand);
    return hipGetLastError();
}

hipError_t zha_launch_planes16(const float* S, uint16_t* S16, int H_kv, int64_t cap, int R, int64_t first, int64_t n,
                               hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t count4 = n * R * ZHA_D / 4;
    int64_t blocks = (count4 + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zha_planes16_kernel, dim3((unsigned)blocks, (unsigned)H_kv), dim3(256), 0, stream, S, S16, cap,
                       R, first, n);
    return hipGetLastError();
}

hipError_t zha_launch_planes8(const float* S, uint8_t* S8, float* SC, int H_kv, int64_t cap, int R, int64_t first,
                              int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n * R + 3) / 4;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zha_planes8_kernel, dim3((unsigned)blocks, (unsigned)H_kv), dim3(256), 0, stream, S, S8, SC,
                       cap, R, first, n);
    return hipGetLastError();
}

hipError_t zha_launch_kv_write(int kv_dtype, void* K, void* V, const void* kn, const void* vn, int H_kv,
                               int64_t cap_tok, int64_t row, hipStream_t stream) {
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_kv_write_kernel<uint16_t>, dim3(H_kv), dim3(128), 0, stream,
                           static_cast<uint16_t*>(K), static_cast<uint16_t*>(V),
                           static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn), cap_tok, row);
    else
        hipLaunchKernelGGL(zha_kv_write_kernel<float>, dim3(H_kv), dim3(128), 0, stream, static_cast<float*>(K),
                           static_cast<float*>(V), static_cast<const float*>(kn), static_cast<const float*>(vn),
                           cap_tok, row);
    return hipGetLastError();
}
