// Host-side launchers of the ZHA HIP kernels (internal to libzha.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// ---- summary tree (zha_summary.hip)
size_t zha_leaf_summary_lds_bytes(int R);
size_t zha_merge_lds_bytes(int c, int R);
// Leaves [first_leaf, first_leaf + n_leaves).  With Sp non-null and first_leaf a
// multiple of c, a kernel that holds whole level-2 nodes (the matrix-core kernel at
// 4 <= R <= 16 with c in {2, 4}) also writes the summaries of the
// level-2 nodes made wholly of these leaves into Sp, Bp, Lp (capacity cap2) and sets
// *fused to 1; otherwise *fused is 0 and the caller merges them.
hipError_t zha_launch_leaf_summary(int kv_dtype, const void* K, const float* Qref, float* S, float* B,
                                   float* LSE, int H_kv, int64_t cap_tok, int64_t cap1, int c, int R,
                                   int64_t first_leaf, int64_t n_leaves, float tau, float* Sp, float* Bp, float* Lp,
                                   int64_t cap2, int* fused, hipStream_t stream);
hipError_t zha_launch_merge(const float* Sc, const float* Bc, const float* Lc, float* Sp, float* Bp, float* Lp,
                            int H_kv, int64_t cap_c, int64_t cap_p, int c, int R, int64_t first_parent,
                            int64_t n_parents, hipStream_t stream);
// Two levels at once: the middle level's nodes c * first_grand .. c * (first_grand
// + n_grand) - 1 (written to Sp/Bp/Lp) and their parents first_grand .. + n_grand
// (Sg/Bg/Lg), the same values as two zha_launch_merge calls.
size_t zha_merge2_lds_bytes(int c, int R);
hipError_t zha_launch_merge2(const float* Sc, const float* Bc, const float* Lc, float* Sp, float* Bp, float* Lp,
                             float* Sg, float* Bg, float* Lg, int H_kv, int64_t cap_c, int64_t cap_p, int64_t cap_g,
                             int c, int R, int64_t first_grand, int64_t n_grand, hipStream_t stream);
// the router's bfloat16 copy (round-to-nearest-even) of planes s of nodes
// [first, first + n) of one level, every KV head
hipError_t zha_launch_planes16(const float* S, uint16_t* S16, int H_kv, int64_t cap, int R, int64_t first, int64_t n,
                               hipStream_t stream);
// the router's 8-bit copy of planes s of nodes [first, first + n) of one level,
// every KV head: per plane a power-of-two scale SC and FP8 E4M3 codes S8
hipError_t zha_launch_planes8(const float* S, uint8_t* S8, float* SC, int H_kv, int64_t cap, int R, int64_t first,
                              int64_t n, hipStream_t stream);
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
#define ZHA_HIST_BINS 2048     // bins of a selection digit histogram

struct ZhaLevelArgs {
    const float* S;            // level planes [H_kv][cap][R][128]
    const uint16_t* S16;       // their bfloat16 copy, read instead when non-null
    const uint8_t* S8;         // their 8-bit copy (FP8 E4M3 codes), read instead when non-null
    const float* SC;           // [H_kv][cap][R] the 8-bit planes' scales (powers of two)
    int hkv;                   // KV groups of the tree: virtual group g reads the planes of g % hkv
    const float* B;            // [H_kv][cap][R]
    int64_t cap;               // node slots per head at this level
    int top;                   // 1 at the first routed level (positions are node ids)
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
    float* sig;                // [H_kv][G][sstride]
    int64_t sstride;           // row stride of sig: cap rounded up to a multiple of 4 (16-byte rows)
    uint64_t* kbm;             // per-head kept bitmaps [H_kv][G][wcap]
    int64_t wcap;              // bitmap words per head
    int32_t* stats;            // out [H_q][2]
    int32_t* klist;            // out: kept nodes [H_kv][cap], ascending
    uint32_t* kmask;           // out: their head masks
    int32_t* nkept;            // out [H_kv]
    // selection state of a level below the chain (null at chained levels):
    float* hblk;               // [H_q][ZHA_SCORE_MAXB] largest score per head in each score block
    int score_blocks;          // score blocks per group (entries of hblk per head)
    uint64_t* ghist;           // [H_q][ZHA_HIST_BINS] first-digit mass histograms of the select slices
    uint32_t* hdone;           // [H_q] select slice workgroups done
    void* hcut;                // [H_q] each head's cut (16 bytes)
    // frontiers beyond ZHA_LDS_KEYS candidates per head (null when the level's
    // capacity never exceeds it): the select kernel publishes each head's first
    // crossing bin, the cross kernel lists that bin's keys, the resolve kernel cuts
    uint4* pub;                // [H_q] {crossing bin, mass still needed (lo, hi), head max bits}
    uint4* gcnt;               // [H_q] {listed keys, -, -, overflow}
    uint2* gpart;              // [H_q][ZHA_CROSS_MAXW] per cross workgroup {keys below the bin, candidates}
    uint2* glist;              // [H_q][ZHA_GLIST] listed keys {key, position}
    uint32_t* tick;            // [H_kv] apply chunks started
    uint32_t* desc;            // [H_kv][ndesc] look-back descriptors of the apply chunks
    int ndesc;                 // apply chunks per group at this level's capacity
    // the level's every node already scored (node-indexed [H_kv][G][nstride], or
    // null): the score kernel then copies its candidates' scores from there
    const float* sigN;
    int64_t nstride;
};
// One field in each 64-byte line of a level's arguments, and the arguments that
// follow them, demanded at kernel entry: the argument loads then go out in one
// batch (the compiler otherwise fetches them in dependent rounds behind uniform
// branches, each a memory round trip on a cold argument line).
#define ZHA_LEVEL_ARGS_READY(a, ...) \
    asm volatile("" ::"s"((a).S), "s"((a).pcap), "s"((a).wcap), "s"((a).hblk), "s"((a).nstride), __VA_ARGS__)
#define ZHA_LDS_KEYS 32768     // a head's keys staged in LDS by the workgroup that cuts it
#define ZHA_GLIST 16384        // a large frontier's crossing-bin keys listed per head
#define ZHA_CROSS_MAXW 32      // cross workgroups per head
#define ZHA_CROSS_MIN_NODES (2 * ZHA_LDS_KEYS)   // levels of more complete nodes take the cross path
// Cross workgroups per head for a level of `cap` node slots: 4 slices of 1024
// positions each at least, at most ZHA_CROSS_MAXW.
__host__ __device__ inline int zha_cross_blocks(int64_t cap) {
    int64_t w = (cap + 4 * 1024 - 1) / (4 * 1024);
    return (int)(w < 1 ? 1 : w > ZHA_CROSS_MAXW ? ZHA_CROSS_MAXW : w);
}
// The level below the chain derives the chain's last level's group kept list from
// the chain's per-head bitmaps (`defer` = that level's arguments: top = 1, n_top
// its complete nodes, bitmaps over node ids) in its score kernel; at most
// ZHA_DEFER_WORDS head words staged.
#define ZHA_DEFER_WORDS 2048
size_t zha_defer_lds_bytes(int G, int64_t n);
hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream,
                                  const ZhaLevelArgs* defer = nullptr);
hipError_t zha_launch_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream);
hipError_t zha_launch_apply(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream);
// frontiers beyond ZHA_LDS_KEYS: list the crossing bin's keys over many workgroups,
// then cut each head from its list (both return at once for other heads)
hipError_t zha_launch_cross(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream);
hipError_t zha_launch_resolve(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream);
int zha_apply_chunks(int64_t cap);
int zha_score_blocks(int64_t max_cand, int R);
// The chain: the first routed levels while each has at most ZHA_CHAIN_SLOTS node
// slots and together at most ZHA_CHAIN_PLANES planes per group; every node scored
// by one launch, then each query head's workgroup selects them one after the other.
#define ZHA_CHAIN_SLOTS 8192
#define ZHA_MAX_CHAIN 8
#define ZHA_CHAIN_PLANES 32768
struct ZhaChainArgs {                 // scoring every node of the chained levels
    ZhaLevelArgs lv[ZHA_MAX_CHAIN];   // lv[0] is the first routed level
    int blocks[ZHA_MAX_CHAIN];        // score workgroups per group for each level
    int n;
};
struct ZhaChainLevel {                // selecting one chained level
    const float* sig;                 // node-indexed scores [H_kv][G][sstride]
    uint64_t* kbm;                    // out: per-head kept bitmaps over node ids [H_kv][G][wcap]
    int32_t* stats;                   // out [H_q][2]: candidates, kept
    int32_t cap, n_nodes, orph_lo, orph_hi, wcap, sstride;
};
struct ZhaChainSel {
    ZhaChainLevel lv[ZHA_MAX_CHAIN];
    int n;
    // spec_blocks > 0: workgroups past the H_kv x G selecting ones score every
    // node of the level below the chain (spec: its arguments as a first routed
    // level, sig = the node-indexed scores), spec_blocks per KV group, on the
    // compute units the selection leaves idle
    int nsel;                          // selecting workgroups: (virtual) KV groups x G
    int spec_blocks;
    ZhaLevelArgs spec;
    const void* q;
    int R;
    float tau;
};
hipError_t zha_launch_score_all(int kv_dtype, const void* q, const ZhaChainArgs& m, int H_kv, int G, int c, int R,
                                float tau, hipStream_t stream);
hipError_t zha_launch_chain(int kv_dtype, const ZhaChainSel& m, int H_kv, int G, int c, float top_p,
                            hipStream_t stream);
// the group kept list of a chained level 1 (bitmaps over node ids; a.top = 1)
hipError_t zha_launch_merge_ids(const ZhaLevelArgs& a, int H_kv, int G, int c, hipStream_t stream);

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
    int hkv;                   // KV groups of the cache: virtual group g reads the rows of g % hkv
};
#define ZHA_ATTN_ARGS_READY(a, ...) asm volatile("" ::"s"((a).K), "s"((a).n_tokens), __VA_ARGS__)
hipError_t zha_launch_attention(int kv_dtype, bool dense, const ZhaAttnArgs& a, int H_kv, int G, int c,
                                float tau, int Bg, hipStream_t stream, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);
hipError_t zha_launch_combine(const ZhaAttnArgs& a, int H_kv, int G, int Bg, float* out, hipStream_t stream);

// ---- router fidelity (zha_fidelity.hip)
#define ZHA_FID_MAXL 32
struct ZhaFidLevels {                  // level l at index l - 1
    const uint64_t* kbm[ZHA_FID_MAXL]; // per-head kept bitmaps over node ids [H_kv][G][wcap]
    int64_t wcap[ZHA_FID_MAXL];
    int64_t span[ZHA_FID_MAXL];        // tokens per node, c^l
    int64_t n_nodes[ZHA_FID_MAXL];     // complete nodes (tokens past them count as kept)
    int n;                             // levels
};
size_t zha_fid_work_bytes(int H_q, int64_t n_tokens);
hipError_t zha_launch_fid_bitmap(const int32_t* klist, const uint32_t* kmask, const int32_t* nkept, int64_t cap,
                                 uint64_t* kbm, int64_t wcap, int H_kv, int G, hipStream_t stream);
hipError_t zha_launch_fidelity(int kv_dtype, const void* K, const void* q, int64_t cap_tok, int64_t n_tokens,
                               int H_kv, int G, float tau, const ZhaFidLevels& lv, void* work, float* recall,
                               hipStream_t stream);

// ---- optional outputs of a decode step (zha_report.hip)
struct zha_stats;
struct ZhaReportArgs {
    const int32_t* ncand[32];    // per level l (index l-1): [H_kv] union candidates
    const int32_t* nkept[32];    // [H_kv] nodes kept by some head
    const int32_t* hstats[32];   // [H_q][2] per head: candidates, kept
    int64_t all_nodes[32];       // > 0: a chained level, its every node scored (its count per head)
    int64_t spec_nodes[32];      // > 0: the level below the chain, its every node scored during the chain
    int64_t n_nodes[32];         // complete nodes per head
    const uint64_t* kbm[32];     // chained levels: per-head kept bitmaps over node ids [H_kv][G][wcap]
    int32_t wcap[32];
    int32_t routed[32];          // 1 when the level has a complete node
    const int32_t* klist1;       // level-1 kept list [H_kv][cap1]
    int64_t cap1;                // 0 when no level was routed
    int64_t n_tokens;
    int64_t plane_bytes;         // R (d e + 4), e = 4 or 2 (bfloat16 planes): summary bytes of one node
    int64_t kv_row_bytes;        // 2 d e_kv: K and V bytes of one token
    int H, G, c, levels, top;
};
hipError_t zha_launch_sel(const int32_t* klist, const uint32_t* kmask, const int32_t* nkept, int64_t cap1, int H_kv,
                          int G, int32_t* sel, hipStream_t stream);
hipError_t zha_launch_stats(const ZhaReportArgs& r, zha_stats* out, hipStream_t stream);
