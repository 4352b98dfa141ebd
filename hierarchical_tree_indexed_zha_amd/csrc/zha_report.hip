// Optional outputs of a decode step: each query head's kept level-1 chunk list
// (`sel`) and the step's per-level counts and byte totals (`stats`), both
// formed on the device from the routing the step left in scratch.
#include "../../include/zha.h"
#include "zha_common.h"
#include "zha_internal.h"

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// grid (H_q), 1024 threads: row h of sel = [k, chunk_0, ..., chunk_{k-1}], the
// chunks of the group's kept list (ascending) whose head mask holds head h.
__global__ __launch_bounds__(kSelThreads) void zha_sel_kernel(const int32_t* __restrict__ klist,
                                                              const uint32_t* __restrict__ kmask,
                                                              const int32_t* __restrict__ nkept, int64_t cap1,
                                                              int G, int32_t* __restrict__ sel) {
    __shared__ uint32_t s_wave[kSelWaves];
    __shared__ uint32_t s_run;
    const int h = blockIdx.x, g = h / G, hl = h - g * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nk = cap1 > 0 ? nkept[g] : 0;
    int32_t* row = sel + (size_t)h * (size_t)(cap1 + 1);
    const int32_t* kl = klist + (size_t)g * cap1;
    const uint32_t* km = kmask + (size_t)g * cap1;
    if (tid == 0) s_run = 0;
    __syncthreads();
    for (int base = 0; base < nk; base += kSelThreads) {
        const int i = base + tid;
        const bool mine = i < nk && ((km[i] >> hl) & 1u);
        const int32_t node = i < nk ? kl[i] : 0;
        const uint64_t b = __ballot(mine);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (lane == 0) s_wave[wave] = (uint32_t)__popcll(b);
        __syncthreads();
        uint32_t off = s_run, tot = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const uint32_t x = s_wave[w];
            off += w < wave ? x : 0u;
            tot += x;
        }
        if (mine) row[1 + off + below] = node;
        __syncthreads();
        if (tid == 0) s_run += tot;
        __syncthreads();
    }
    if (tid == 0) row[0] = (int32_t)s_run;
}

// grid 1, 256 threads: the step's zha_stats from the per-level counts.  At a
// chained level (every node scored, per-head kept bitmaps over node ids) the group
// kept nodes are the popcount of the OR of the group's head bitmaps, and the group
// candidates are the children of the level above's group kept nodes plus the
// orphans (every node at the top).
__global__ __launch_bounds__(256) void zha_stats_kernel(ZhaReportArgs r, zha_stats* __restrict__ out) {
    __shared__ unsigned long long s_gk[ZHA_STATS_MAX_LEVELS];
    const int tid = threadIdx.x;
    const int Hq = r.H * r.G;
    if (tid < ZHA_STATS_MAX_LEVELS) s_gk[tid] = 0ull;
    __syncthreads();
    for (int l = 0; l < r.levels; ++l) {
        if (!r.routed[l] || r.all_nodes[l] == 0) continue;   // uniform
        unsigned long long cnt = 0;
        const int wc = r.wcap[l];                         // row stride
        const int nw = (int)((r.n_nodes[l] + 63) / 64);   // words holding complete nodes
        for (int i = tid; i < r.H * nw; i += 256) {
            const int g = i / nw, w = i - g * nw;
            uint64_t u = 0;
            for (int hh = 0; hh < r.G; ++hh) u |= r.kbm[l][((size_t)g * r.G + hh) * wc + w];
            cnt += (unsigned long long)__popcll(u);
        }
        if (cnt) atomicAdd(&s_gk[l], cnt);
    }
    __syncthreads();
    if (tid < ZHA_STATS_MAX_LEVELS) {
        const int l = tid;
        int64_t cand = 0, kept = 0, gc = 0, gk = 0, streamed = 0;
        if (l < r.levels && r.routed[l]) {
            for (int h = 0; h < Hq; ++h) {
                cand += r.hstats[l][2 * h + 0];
                kept += r.hstats[l][2 * h + 1];
            }
            if (r.all_nodes[l] > 0) {
                gk = (int64_t)s_gk[l];
                if (l + 1 == r.top) gc = r.n_nodes[l] * r.H;
                else gc = (int64_t)r.c * (int64_t)s_gk[l + 1] + (int64_t)r.H * (r.n_nodes[l] - r.c * r.n_nodes[l + 1]);
                streamed = r.all_nodes[l] * r.H * r.plane_bytes;
            } else {
                for (int g = 0; g < r.H; ++g) {
                    gc += r.ncand[l][g];
                    gk += r.nkept[l][g];
                }
                // (a level scored whole during the chain streamed every node's planes)
                streamed = r.spec_nodes[l] > 0 ? r.spec_nodes[l] * r.H * r.plane_bytes : gc * r.plane_bytes;
            }
        }
        out->cand[l] = cand;
        out->kept[l] = kept;
        out->group_cand[l] = gc;
        out->group_kept[l] = gk;
        out->bytes_read[l] = gc * r.plane_bytes;
        out->bytes_streamed[l] = streamed;
    }
    if (tid == 0) {
        // tokens attended per group: kept chunks, the sink unless chunk 0 is kept, the tail
        const int64_t n1 = r.n_tokens / r.c;
        int64_t toks = 0;
        for (int g = 0; g < r.H; ++g) {
            const int64_t nk = r.cap1 > 0 ? r.nkept[0][g] : 0;
            const bool kept0 = nk > 0 && r.klist1[(size_t)g * r.cap1] == 0;
            toks += nk * r.c + ((n1 > 0 && !kept0) ? 1 : 0) + (r.n_tokens - r.c * n1);
        }
        out->n_tokens = r.n_tokens;
        out->top_level = r.top;
        out->levels = r.levels;
        out->gather_tokens = toks;
        out->gather_bytes = toks * r.kv_row_bytes;
    }
}

}  // namespace

hipError_t zha_launch_sel(const int32_t* klist, const uint32_t* kmask, const int32_t* nkept, int64_t cap1, int H_kv,
                          int G, int32_t* sel, hipStream_t stream) {
    hipLaunchKernelGGL(zha_sel_kernel, dim3((unsigned)(H_kv * G)), dim3(kSelThreads), 0, stream, klist, kmask, nkept,
                       cap1, G, sel);
    return hipGetLastError();
}

hipError_t zha_launch_stats(const ZhaReportArgs& r, zha_stats* out, hipStream_t stream) {
    hipLaunchKernelGGL(zha_stats_kernel, dim3(1), dim3(256), 0, stream, r, out);
    return hipGetLastError();
}
