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

// grid (ceil(n_parents / parents_per_block), H_kv), 256 threads.
__global__ __launch_bounds__(256) void zha_merge_kernel(
    const float* __restrict__ Sc, const float* __restrict__ Bc, const float* __restrict__ Lc,
    float* __restrict__ Sp, float* __restrict__ Bp, float* __restrict__ Lp,
    int64_t cap_c, int64_t cap_p, int c, int R, int64_t first_parent, int64_t n_parents) {
    extern __shared__ float a_s[];                       // [ppb][R][c]
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int per_parent = R * (ZHA_D / 4);              // float4 outputs per parent
    const int ppb = per_parent >= 256 ? 1 : 256 / per_parent;
    const int64_t p0 = first_parent + (int64_t)blockIdx.x * ppb;
    const int64_t end = first_parent + n_parents;
    if (p0 >= end) return;
    const int np = (int)min((int64_t)ppb, end - p0);
    for (int pr = tid; pr < np * R; pr += blockDim.x) {
        int pl = pr / R, r = pr - pl * R;
        int64_t child0 = (p0 + pl) * c;
        float m = zha_neg_inf();
        for (int j = 0; j < c; ++j) m = fmaxf(m, Lc[((size_t)g * cap_c + (size_t)(child0 + j)) * R + r]);
        float sum = 0.f;
        for (int j = 0; j < c; ++j) sum += expf(Lc[((size_t)g * cap_c + (size_t)(child0 + j)) * R + r] - m);
        float lse = m + logf(sum);
        float bp = 0.f;
        float* a = a_s + (pl * R + r) * c;
        for (int j = 0; j < c; ++j) {
            size_t o = ((size_t)g * cap_c + (size_t)(child0 + j)) * R + r;
            float la = Lc[o] - lse;                          // log a_j
            float aj = expf(la);
            a[j] = aj;
            bp = fmaf(aj, Bc[o] - la, bp);
        }
        size_t op = ((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r;
        Lp[op] = lse;
        Bp[op] = bp;
    }
    __syncthreads();
    for (int o = tid; o < np * per_parent; o += blockDim.x) {
        int pl = o / per_parent, rem = o - pl * per_parent;
        int r = rem / (ZHA_D / 4), d4 = rem - r * (ZHA_D / 4);
        int64_t child0 = (p0 + pl) * c;
        const float* a = a_s + (pl * R + r) * c;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < c; ++j) {
            float4 s = reinterpret_cast<const float4*>(Sc + (((size_t)g * cap_c + (size_t)(child0 + j)) * R + r) * ZHA_D)[d4];
            acc.x = fmaf(a[j], s.x, acc.x);
            acc.y = fmaf(a[j], s.y, acc.y);
            acc.z = fmaf(a[j], s.z, acc.z);
            acc.w = fmaf(a[j], s.w, acc.w);
        }
        reinterpret_cast<float4*>(Sp + (((size_t)g * cap_p + (size_t)(p0 + pl)) * R + r) * ZHA_D)[d4] = acc;
    }
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
                                   int64_t first_leaf, int64_t n_leaves, float tau, hipStream_t stream) {
    if (n_leaves <= 0) return hipSuccess;
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
    hipLaunchKernelGGL(zha_merge_kernel, grid, dim3(256), zha_merge_lds_bytes(c, R), stream, Sc, Bc, Lc, Sp,
                       Bp, Lp, cap_c, cap_p, c, R, first_parent, n_parents);
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
