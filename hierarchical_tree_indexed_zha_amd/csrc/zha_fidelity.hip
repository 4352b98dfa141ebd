// Router fidelity of a decode step (a diagnostic beside the hot path).
//
// For query head h with exact attention probabilities p_t = e^{z_t - LSE(q)},
// z_t = tau q.k_t over every cached token (page "ZHA 用树形稀疏注意力改造现有大模型",
// section 256K 的质量结果: the router is judged by how much of the true attention
// it keeps), level l's mass recall is the probability mass of the tokens whose
// level-l node the head kept, that is the sum over kept nodes n of
// e^{LSE_n(q) - LSE(q)} with LSE_n the log-sum-exp over n's raw keys; tokens under
// no complete level-l node are never dropped at that level and count as kept.  The
// step's captured mass is the probability mass of the token set it attended (kept
// level-1 chunks, token 0 and the raw tail).
//
// Three passes over the cache, one query head per workgroup row, kTok tokens per
// workgroup: (1) each workgroup's max logit and sum of e^{z - max}; (2) per head,
// LSE(q) from those partials; (3) each workgroup's recall sums per level and its
// captured sum, then (4) per head, their totals.  The kept sets come as per-head
// bitmaps over node ids, written for every level below the chain from its group
// kept list first (the chain's levels have them already).
#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kFidThreads = 256;
constexpr int kFidPer = 8;                         // tokens per thread
constexpr int kTok = kFidThreads * kFidPer;        // tokens per workgroup

template <bool BF16>
__device__ __forceinline__ float logit(const void* K, size_t row, const float* qs, float tau) {
    float acc = 0.f;
    if (BF16) {
        const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(K) + row * ZHA_D);
#pragma unroll
        for (int i = 0; i < ZHA_D / 8; ++i) {
            const uint4 v = kr[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = fmaf(qs[8 * i + 2 * j], zha_bf16_to_f32(w[j] & 0xFFFFu), acc);
                acc = fmaf(qs[8 * i + 2 * j + 1], zha_bf16_to_f32(w[j] >> 16), acc);
            }
        }
    } else {
        const float4* kr = reinterpret_cast<const float4*>(static_cast<const float*>(K) + row * ZHA_D);
#pragma unroll
        for (int i = 0; i < ZHA_D / 4; ++i) {
            const float4 v = kr[i];
            acc = fmaf(qs[4 * i], v.x, acc);
            acc = fmaf(qs[4 * i + 1], v.y, acc);
            acc = fmaf(qs[4 * i + 2], v.z, acc);
            acc = fmaf(qs[4 * i + 3], v.w, acc);
        }
    }
    return tau * acc;
}

template <bool BF16>
__device__ __forceinline__ void load_query(const void* q, int h, float* qs) {
    for (int d = threadIdx.x; d < ZHA_D; d += blockDim.x)
        qs[d] = BF16 ? zha_bf16_to_f32(static_cast<const uint16_t*>(q)[(size_t)h * ZHA_D + d])
                     : static_cast<const float*>(q)[(size_t)h * ZHA_D + d];
    __syncthreads();
}

// Sum over the workgroup (thread 0 receives it).
__device__ __forceinline__ float block_sum(float x, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0)
        for (int w = 0; w < kFidThreads / 64; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float block_max(float x, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float t = zha_neg_inf();
    for (int w = 0; w < kFidThreads / 64; ++w) t = fmaxf(t, red[w]);
    __syncthreads();
    return t;
}

// grid (blocks, H_q): partial[h][b] = {max z, sum e^{z - max}} over the workgroup's tokens.
template <bool BF16>
__global__ __launch_bounds__(kFidThreads) void zha_fid_lse_kernel(const void* K, const void* q, int64_t cap_tok,
                                                                 int64_t n_tokens, int G, float tau, float2* part) {
    __shared__ float qs[ZHA_D];
    __shared__ float red[kFidThreads / 64];
    const int h = blockIdx.y, g = h / G;
    load_query<BF16>(q, h, qs);
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    float z[kFidPer];
    float m = zha_neg_inf();
#pragma unroll
    for (int k = 0; k < kFidPer; ++k) {
        const int64_t t = t0 + threadIdx.x + (int64_t)k * kFidThreads;
        z[k] = t < n_tokens ? logit<BF16>(K, (size_t)g * cap_tok + (size_t)t, qs, tau) : zha_neg_inf();
        m = fmaxf(m, z[k]);
    }
    const float M = block_max(m, red);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kFidPer; ++k) s += z[k] == zha_neg_inf() ? 0.f : __expf(z[k] - M);
    const float S = block_sum(s, red);
    if (threadIdx.x == 0) part[(size_t)h * gridDim.x + blockIdx.x] = make_float2(M, S);
}

// grid (H_q), 256 threads: lse[h] from the partials (in double: the sums of many
// workgroups' terms rescaled to one maximum).
__global__ __launch_bounds__(kFidThreads) void zha_fid_lse_reduce_kernel(const float2* part, int nblk, float* lse) {
    __shared__ double rd[kFidThreads];
    __shared__ float red[kFidThreads / 64];
    const int h = blockIdx.x;
    float m = zha_neg_inf();
    for (int b = threadIdx.x; b < nblk; b += kFidThreads) m = fmaxf(m, part[(size_t)h * nblk + b].x);
    const float M = block_max(m, red);
    double s = 0.0;
    for (int b = threadIdx.x; b < nblk; b += kFidThreads) {
        const float2 p = part[(size_t)h * nblk + b];
        if (p.y > 0.f) s += (double)p.y * exp((double)p.x - (double)M);
    }
    rd[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < kFidThreads; ++i) t += rd[i];
        lse[h] = (float)((double)M + log(t));
    }
}

// grid (H_kv), 256 threads: per-head kept bitmaps over node ids of a level below the
// chain, from its group kept list (nkept entries, head masks): words cleared, then set.
__global__ __launch_bounds__(kFidThreads) void zha_fid_bitmap_kernel(const int32_t* klist, const uint32_t* kmask,
                                                                    const int32_t* nkept, int64_t cap, uint64_t* kbm,
                                                                    int64_t wcap, int G) {
    const int g = blockIdx.x;
    uint64_t* bm = kbm + (size_t)g * G * wcap;
    for (int64_t i = threadIdx.x; i < (int64_t)G * wcap; i += kFidThreads) bm[i] = 0ull;
    __threadfence();                                   // every clearing store completed before any bit is set
    __syncthreads();
    const int nk = nkept[g];
    for (int i = threadIdx.x; i < nk; i += kFidThreads) {
        const int32_t node = klist[(size_t)g * cap + i];
        const uint32_t msk = kmask[(size_t)g * cap + i];
        for (int hl = 0; hl < G; ++hl)
            if ((msk >> hl) & 1u)
                atomicOr((unsigned long long*)&bm[(size_t)hl * wcap + (node >> 6)], 1ull << (node & 63));
    }
}

// grid (blocks, H_q): per workgroup, sum of p_t over tokens kept at each level, and
// over the attended set; sums[h][b][0 .. L] (L + 1 floats, level l at index l - 1).
template <bool BF16>
__global__ __launch_bounds__(kFidThreads) void zha_fid_recall_kernel(const void* K, const void* q, int64_t cap_tok,
                                                                    int64_t n_tokens, int G, float tau,
                                                                    const float* lse, ZhaFidLevels lv,
                                                                    float* sums) {
    __shared__ float qs[ZHA_D];
    __shared__ float red[kFidThreads / 64];
    const int h = blockIdx.y, g = h / G, hl = h - g * G;
    load_query<BF16>(q, h, qs);
    const float L0 = lse[h];
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    float acc[ZHA_FID_MAXL + 1];
#pragma unroll
    for (int l = 0; l <= ZHA_FID_MAXL; ++l) acc[l] = 0.f;
    for (int k = 0; k < kFidPer; ++k) {
        const int64_t t = t0 + threadIdx.x + (int64_t)k * kFidThreads;
        if (t >= n_tokens) break;
        const float p = __expf(logit<BF16>(K, (size_t)g * cap_tok + (size_t)t, qs, tau) - L0);
        // level l: kept when its node is incomplete or in the head's bitmap
        bool kept1 = true;
#pragma unroll
        for (int l = 0; l < ZHA_FID_MAXL; ++l) {
            if (l < lv.n) {
                const int64_t node = t / lv.span[l];
                bool kept = node >= lv.n_nodes[l];
                if (!kept) {
                    const uint64_t w = lv.kbm[l][((size_t)g * G + hl) * lv.wcap[l] + (size_t)(node >> 6)];
                    kept = (w >> (node & 63)) & 1ull;
                }
                acc[l] += kept ? p : 0.f;
                if (l == 0) kept1 = kept;
            }
        }
        // the attended set: token 0, the raw tail, tokens of kept level-1 chunks
        const bool att = t == 0 || kept1;
        acc[ZHA_FID_MAXL] += att ? p : 0.f;
    }
    for (int l = 0; l <= ZHA_FID_MAXL; ++l) {
        if (l < lv.n || l == ZHA_FID_MAXL) {
            const float s = block_sum(acc[l], red);
            if (threadIdx.x == 0)
                sums[((size_t)h * gridDim.x + blockIdx.x) * (ZHA_FID_MAXL + 1) + (l < lv.n ? l : lv.n)] = s;
        }
    }
}

// grid (H_q), 64 threads: recall[h][l] = sum over workgroups (double accumulation).
__global__ void zha_fid_recall_reduce_kernel(const float* sums, int nblk, int nl, float* recall) {
    const int h = blockIdx.x;
    for (int l = threadIdx.x; l <= nl; l += blockDim.x) {
        double t = 0.0;
        for (int b = 0; b < nblk; ++b) t += sums[((size_t)h * nblk + b) * (ZHA_FID_MAXL + 1) + l];
        recall[(size_t)h * (nl + 1) + l] = (float)t;
    }
}

}  // namespace

size_t zha_fid_work_bytes(int H_q, int64_t n_tokens) {
    const size_t nblk = (size_t)((n_tokens + kTok - 1) / kTok);
    return 256 + sizeof(float2) * H_q * nblk + sizeof(float) * H_q + sizeof(float) * H_q * nblk * (ZHA_FID_MAXL + 1);
}

hipError_t zha_launch_fid_bitmap(const int32_t* klist, const uint32_t* kmask, const int32_t* nkept, int64_t cap,
                                 uint64_t* kbm, int64_t wcap, int H_kv, int G, hipStream_t stream) {
    hipLaunchKernelGGL(zha_fid_bitmap_kernel, dim3((unsigned)H_kv), dim3(kFidThreads), 0, stream, klist, kmask, nkept,
                       cap, kbm, wcap, G);
    return hipGetLastError();
}

hipError_t zha_launch_fidelity(int kv_dtype, const void* K, const void* q, int64_t cap_tok, int64_t n_tokens,
                               int H_kv, int G, float tau, const ZhaFidLevels& lv, void* work, float* recall,
                               hipStream_t stream) {
    if (lv.n < 0 || lv.n > ZHA_FID_MAXL || n_tokens < 1) return hipErrorInvalidValue;
    const int H = H_kv * G;
    const int nblk = (int)((n_tokens + kTok - 1) / kTok);
    char* w = static_cast<char*>(work);
    float2* part = reinterpret_cast<float2*>(w + 256);
    float* lse = reinterpret_cast<float*>(part + (size_t)H * nblk);
    float* sums = lse + H;
    const dim3 grid((unsigned)nblk, (unsigned)H);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_fid_lse_kernel<true>, grid, dim3(kFidThreads), 0, stream, K, q, cap_tok, n_tokens, G,
                           tau, part);
    else
        hipLaunchKernelGGL(zha_fid_lse_kernel<false>, grid, dim3(kFidThreads), 0, stream, K, q, cap_tok, n_tokens, G,
                           tau, part);
    hipLaunchKernelGGL(zha_fid_lse_reduce_kernel, dim3((unsigned)H), dim3(kFidThreads), 0, stream, part, nblk, lse);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(zha_fid_recall_kernel<true>, grid, dim3(kFidThreads), 0, stream, K, q, cap_tok, n_tokens,
                           G, tau, lse, lv, sums);
    else
        hipLaunchKernelGGL(zha_fid_recall_kernel<false>, grid, dim3(kFidThreads), 0, stream, K, q, cap_tok, n_tokens,
                           G, tau, lse, lv, sums);
    hipLaunchKernelGGL(zha_fid_recall_reduce_kernel, dim3((unsigned)H), dim3(64), 0, stream, sums, nblk, lv.n,
                       recall);
    return hipGetLastError();
}
