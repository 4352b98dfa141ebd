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
// Level l's candidates sit at positions 0..n-1 in ascending node order: at the
// first routed level they are nodes 0..n_top-1 seen by every head; below it,
// cand_node/cand_mask/ncand were written by the level above (children of its
// kept nodes, then the orphans of this level).
struct ZhaLevelArgs {
    const float* S;            // level planes [H_kv][cap][R][128]
    const float* B;            // [H_kv][cap][R]
    int64_t cap;               // node slots per head at this level
    int top;                   // 1 at the first routed level
    int64_t n_top;             // candidates at the first routed level (all its nodes)
    const int32_t* cand_node;  // [H_kv][cap] (unused when top)
    const uint32_t* cand_mask; // [H_kv][cap]
    int32_t* ncand;            // [H_kv] (written when top, read otherwise)
    float* sig;                // [H_kv][G][cap]
    uint64_t* kbm;             // per-head kept bitmaps [H_kv][G][wcap]
    int64_t wcap;              // bitmap words per head
    int32_t* done;             // [H_kv]
    int32_t* stats;            // out [H_q][2]
    int32_t* klist;            // out: kept nodes [H_kv][cap], ascending
    uint32_t* kmask;           // out: their head masks
    int32_t* nkept;            // out [H_kv]
    // candidates of the level below (not written at level 1)
    int32_t* next_node;        // [H_kv][next_cap]
    uint32_t* next_mask;
    int32_t* next_ncand;       // [H_kv]
    int64_t next_cap;
    int64_t orph_lo, orph_hi;  // orphan nodes of the level below
};
hipError_t zha_launch_route_score(int kv_dtype, const void* q, const ZhaLevelArgs& a, int H_kv, int G, int c,
                                  int R, float tau, int blocks, hipStream_t stream);
hipError_t zha_launch_route_select(const ZhaLevelArgs& a, int H_kv, int G, int c, float top_p, hipStream_t stream);
int zha_score_blocks(int64_t max_cand, int R);

// ---- attention (zha_attn.hip)
struct ZhaAttnArgs {
    const void* K;
    const void* V;
    int64_t cap_tok;
    const void* q;             // [H_q][128]
    const int32_t* klist;      // kept level-1 chunks [H_kv][cap1] (sparse mode; nullptr = none)
    const uint32_t* kmask;
    const int32_t* nkept;      // [H_kv]
    int64_t cap1;
    int64_t n_tokens;
    float* pm;                 // [H_kv][Bg][G]
    float* pl;                 // [H_kv][Bg][G]
    float* po;                 // [H_kv][Bg][G][128]
    int32_t* nact;             // [H_kv]
};
hipError_t zha_launch_attention(int kv_dtype, bool dense, const ZhaAttnArgs& a, int H_kv, int G, int c,
                                float tau, int Bg, hipStream_t stream);
hipError_t zha_launch_combine(const ZhaAttnArgs& a, int H_kv, int G, int Bg, float* out, hipStream_t stream);
