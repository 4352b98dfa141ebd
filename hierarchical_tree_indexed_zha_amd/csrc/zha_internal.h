// Host-side launchers of the ZHA HIP kernels (internal to libzha.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// ---- summary tree (zha_summary.hip)
size_t zha_leaf_summary_lds_bytes(int R);
size_t zha_merge_lds_bytes(int c, int R);
hipError_t zha_launch_leaf_summary(int kv_dtype, const void* K, const float* Qref, float* S, float* B,
                                   float* LSE, int H_kv, int64_t cap_tok, int64_t cap1, int c, int R,
                                   int64_t first_leaf, int64_t n_leaves, float tau, hipStream_t stream);
hipError_t zha_launch_merge(const float* Sc, const float* Bc, const float* Lc, float* Sp, float* Bp, float* Lp,
                            int H_kv, int64_t cap_c, int64_t cap_p, int c, int R, int64_t first_parent,
                            int64_t n_parents, hipStream_t stream);
hipError_t zha_launch_kv_write(int kv_dtype, void* K, void* V, const void* kn, const void* vn, int H_kv,
                               int64_t cap_tok, int64_t row, hipStream_t stream);

// ---- per-level routing (zha_route.hip)
// Unsigned 32-bit division by a divisor fixed per launch (the chunk size),
// by multiplication with a precomputed reciprocal: the round-up method of
// Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication" (PLDI 1994), section 4.  With l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)
// where t = mulhi(m, n), exact for every 32-bit n and 1 <= d < 2^31.
struct ZhaDiv {
    uint32_t d, m, s1, s2;
};
inline ZhaDiv zha_make_div(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    ZhaDiv r;
    r.d = d;
    r.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    r.s1 = l < 1 ? l : 1;
    r.s2 = l > 1 ? l - 1 : 0;
    return r;
}
__device__ __forceinline__ uint32_t zha_div(uint32_t n, const ZhaDiv& v) {
    const uint32_t t = __umulhi(n, v.m);
    return (t + ((n - t) >> v.s1)) >> v.s2;
}

// Level l's candidates sit at positions 0..n-1 in ascending node order: at the
// first routed level they are nodes 0..n_top-1 seen by every head; below it they
// are the children of the level above's kept nodes (its kept list, ascending,
// with the heads that kept each) followed by this level's orphans, nodes
// [orph_lo, orph_hi) seen by every head.
// The selection cut of one query head at a sliced level, as far as the digit
// passes have found it (one per head, written by the last slice of each pass).
struct HugeCut {
    uint32_t done;                        // 1 when the cut key is known
    uint32_t ustar, ties;                 // the cut: largest kept key, keys equal to it
    uint32_t mshift, mval, bshift, bmask; // the next pass's digit, when not done
    uint32_t pad;
    uint64_t need;                        // mass still needed inside the current prefix
};
static_assert(sizeof(HugeCut) == 40, "HugeCut layout");

struct ZhaLevelArgs {
    const float* S;            // level planes [H_kv][cap][R][128]
    const float* B;            // [H_kv][cap][R]
    int64_t cap;               // node slots per head at this level
    int top;                   // 1 at the first routed level
    int64_t n_top;             // candidates at the first routed level (all its nodes)
    // the level above: its kept nodes are this level's parents (at the first routed
    // level: readable memory with pcap 1, whose values go unused)
    const int32_t* pklist;     // [H_kv][pcap]
    const uint32_t* pkmask;    // [H_kv][pcap]
    const int32_t* pnkept;     // [H_kv]
    int64_t pcap;
    int64_t orph_lo, orph_hi;  // this level's orphans
    ZhaDiv dc;                 // division by the chunk size
    int32_t* ncand;            // out [H_kv]: candidates at this level
    float* sig;                // [H_kv][G][cap]
    uint64_t* kbm;             // per-head kept bitmaps [H_kv][G][wcap]
    int64_t wcap;              // bitmap words per head
    int32_t* stats;            // out [H_q][2]
    int32_t* klist;            // out: kept nodes [H_kv][cap], ascending
    uint32_t* kmask;           // out: their head masks
    int32_t* nkept;            // out [H_kv]
    // Levels with more than ZHA_SLICED_MIN_CAP node slots select over slices of
    // ZHA_SLICE positions spread over the whole GPU (null otherwise):
    float* hblk;               // [H_q][ZHA_SCORE_MAXB] largest score per head in each score block
    int score_blocks;          // score blocks per group (entries of hblk per head)
    HugeCut* hstate;           // [H_q] the cut found so far per head
    uint32_t* hdone;           // [3][H_q] slices done per pass
    uint64_t* hmass;           // [3][H_q][2048] per-pass digit histograms: fixed-point mass
    uint32_t* hcnt;            // [3][H_q][2048] and count
    uint64_t* tiem;            // [H_q][slices] mass of cut-equal keys per slice
    uint32_t* chunk_cnt;       // [H_kv][wcap / 512] kept nodes per 512-word chunk
    int slices;                // slices per head
};
// One field in each 64-byte line of a level's arguments, and the arguments that
// follow them, demanded at kernel entry: the argument loads then go out in one
// batch (the compiler otherwise fetches them in dependent rounds behind uniform
// branches, each a memory round trip on a cold argument line).
#define ZHA_LEVEL_ARGS_READY(a, ...) \
    asm volatile("" ::"s"((a).S), "s"((a).pcap), "s"((a).wcap), "s"((a).hdone), "s"((a).slices), __VA_ARGS__)
#define ZHA_LDS_KEYS 32768     // candidates per head selected in one workgroup's LDS
#define ZHA_SLICE 32768        // positions per slice workgroup of a sliced level
#define ZHA_SLICED_MIN_CAP 262144   // levels with more node slots select over slices
// A large level (more than ZHA_SMALL_SLOTS node slots, not sliced) whose G heads'
// bitmap words together number at most ZHA_DEFER_WORDS and whose parents at most
// ZHA_DEFER_PARENTS is selected without a merge launch: the score kernel of the
// level below (`defer` = the level above's arguments) derives its kept list from
// the bitmaps in LDS and writes it.
#define ZHA_DEFER_WORDS 2048
#define ZHA_DEFER_PARENTS 4096
bool zha_defer_fits(int G, int64_t wcap, int64_t pcap);
size_t zha_defer_lds_bytes(int G, int64_t wcap, int64_t pcap);
hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream,
                                  const ZhaLevelArgs* defer = nullptr);
// merge = false leaves a large, unsliced level's kept list to the next level's
// score kernel (zha_launch_route_score with `defer`)
hipError_t zha_launch_route_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream,
                                   bool merge = true);
int zha_score_blocks(int64_t max_cand, int R);
// The first routed levels while they are small (node slots <= ZHA_SMALL_SLOTS,
// together at most ZHA_CHAIN_PLANES planes per group): every node scored by one
// launch, then the levels selected one after the other by one workgroup per group.
#define ZHA_SMALL_SLOTS 1024
#define ZHA_MAX_CHAIN 6
#define ZHA_CHAIN_PLANES 32768
struct ZhaChainArgs {
    ZhaLevelArgs lv[ZHA_MAX_CHAIN];   // lv[0] is the first routed level
    int blocks[ZHA_MAX_CHAIN];        // score workgroups per group for each level
    int n;
};
hipError_t zha_launch_route_chain(int kv_dtype, const void* q, const ZhaChainArgs& m, int H_kv, int G, int c, int R,
                                  float tau, float top_p, hipStream_t stream);

// ---- attention (zha_attn.hip)
struct ZhaAttnArgs {
    const void* K;
    const void* V;
    int64_t cap_tok;
    const void* q;             // [H_q][128]
    const int32_t* klist;      // kept level-1 chunks [H_kv][cap1] (sparse mode: always readable)
    const uint32_t* kmask;
    const int32_t* nkept;      // [H_kv]
    int64_t cap1;              // 0 when no level is routed (the lists then hold nothing)
    int64_t n_tokens;
    float* pm;                 // [H_kv][Bg][G]
    float* pl;                 // [H_kv][Bg][G]
    float* po;                 // [H_kv][Bg][G][128]
    int32_t* nact;             // [H_kv]
};
#define ZHA_ATTN_ARGS_READY(a, ...) asm volatile("" ::"s"((a).K), "s"((a).n_tokens), __VA_ARGS__)
hipError_t zha_launch_attention(int kv_dtype, bool dense, const ZhaAttnArgs& a, int H_kv, int G, int c,
                                float tau, int Bg, hipStream_t stream, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);
hipError_t zha_launch_combine(const ZhaAttnArgs& a, int H_kv, int G, int Bg, float* out, hipStream_t stream);
