/*
 * zha.h — C ABI of libzha.so: one ZHA (Zyphra Hierarchical Attention) decode
 * step over a full KV cache on an MI355X (gfx950), the summary tree that feeds
 * it, and a dense-decode baseline.
 *
 * Method, as the source pages describe it:
 *   - Contiguous keys are cut into chunks of c tokens; each chunk is summarised,
 *     and summaries are grouped c at a time level after level (page "Zyphra
 *     分层注意力（ZHA）：通向真次二次注意力的新路径…", section 机制拆解; page
 *     "ZHA 用树形稀疏注意力改造现有大模型", section 稀疏注意力为什么还会被索引拖慢:
 *     chunk 4 with 6 levels gives a 4,096-token top node).
 *   - A node's summary holds, for each of R reference queries q_r, a tangent
 *     plane of the log attention mass: s_r (softmax-weighted mean of the node's
 *     keys at q_r) and b_r = LSE_r - tau q_r.s_r; a query q scores the node as
 *     max_r (tau q.s_r + b_r) (same page, same section).  tau = 1/sqrt(d).
 *   - A decode step scores the top level, keeps the minimal set of nodes whose
 *     cumulative softmax probability reaches top_p, expands only their children
 *     and repeats down to raw KV chunks (same sections; page rit.work
 *     "zha-tree-indexer-long-context", section "Дерево сокращает сам поиск
 *     нужных ключей"), then attends exactly over the raw keys of the kept
 *     chunks, token 0 (the attention sink) and the raw tail of fewer than c
 *     tokens that no chunk covers yet.
 *   - The full KV cache is kept; the tree sits beside it (page "Zyphra 分层注意力",
 *     section 局限与权衡).
 *
 * Conventions for every entry point:
 *   - All buffers are device pointers owned by the caller; the library
 *     allocates nothing and keeps no state besides a thread-local error string.
 *   - Work is enqueued on `stream` (a hipStream_t, or NULL for the default
 *     stream) and is asynchronous: a return of ZHA_OK means the launches were
 *     accepted, not that they finished.  No call synchronises the device.
 *   - Errors are returned as negative codes and described by zha_last_error();
 *     arguments are validated before anything is enqueued.
 *   - Calls that share a `scratch` buffer must not overlap in time.
 *
 * Layouts (row-major, d = head_dim):
 *   K, V    [n_kv_heads][capacity][d] of kv_dtype; row t holds token t.
 *   ref_q   [n_kv_heads][n_ref][d] float32; one set per KV head, shared by all
 *           levels.
 *   q       [n_q_heads][d] of kv_dtype; query head h reads KV head
 *           h / (n_q_heads / n_kv_heads).
 *   out     [n_q_heads][d] float32.
 *   tree    opaque, zha_tree_bytes(); level l occupies, per KV head, one slot
 *           per node index < capacity / c^l (see zha_tree_level_offsets).
 *   scratch opaque, zha_scratch_bytes(); holds the per-level candidate scores,
 *           kept lists and split-attention partials of the last decode step
 *           (see zha_route_level_offsets).
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ZHA_OK               0
#define ZHA_ERR_ARG         -1   /* null pointer, bad config value, level out of range */
#define ZHA_ERR_CAPACITY    -2   /* n_tokens (or n_tokens + 1 on append) exceeds capacity */
#define ZHA_ERR_UNSUPPORTED -3   /* valid but not implemented: head_dim != 128, group > 16, n_ref not in {1,2,4,8,16,32}, sink != 1 */
#define ZHA_ERR_HIP         -4   /* a HIP launch or runtime call failed */

/* kv_dtype values. */
#define ZHA_BF16 0
#define ZHA_F32  1

typedef struct zha_config {
    int32_t n_kv_heads;  /* H_kv >= 1 */
    int32_t n_q_heads;   /* H_q, a multiple of H_kv; group G = H_q / H_kv, 1 <= G <= 16 */
    int32_t head_dim;    /* d; 128 */
    int32_t chunk;       /* c >= 2: tokens per leaf chunk and fanout of every level */
    int32_t levels;      /* L >= 1: summary levels; a level-l node covers c^l tokens */
    int32_t n_ref;       /* R reference queries per KV head: 1, 2, 4, 8, 16 or 32 */
    float   top_p;       /* p in (0, 1]; p = 1 keeps every node */
    int32_t kv_dtype;    /* ZHA_BF16 or ZHA_F32 (K, V and q) */
    int64_t capacity;    /* rows of K and V per KV head; 1 <= capacity < 2^31 */
    int32_t sink;        /* 1: token 0 is always attended (the attention sink).  0 (no sink)
                          * is valid but not implemented (ZHA_ERR_UNSUPPORTED); other values
                          * are ZHA_ERR_ARG */
    int32_t plane_format;/* format of the planes s the router reads: ZHA_PLANES_F32 (0, the
                          * float32 planes themselves), ZHA_PLANES_BF16 (1, a bfloat16 copy
                          * of them, round-to-nearest-even) or ZHA_PLANES_FP8 (2, an 8-bit
                          * copy: per plane a power-of-two scale 2^k, the smallest with
                          * max_d |s_d| <= 448 * 2^k (k >= -126), and the FP8 E4M3 codes
                          * (sign, 4 exponent bits of bias 7, 3 mantissa bits, subnormals,
                          * largest 448) of s_d / 2^k rounded to nearest even).  Narrow
                          * copies sit beside the float32 planes that the tree's merges use;
                          * b stays float32.  Page "ZHA 用树形稀疏注意力改造现有大模型",
                          * section 几百倍加速 (a narrow-format router variant). */
} zha_config;

#define ZHA_PLANES_F32  0
#define ZHA_PLANES_BF16 1
#define ZHA_PLANES_FP8  2

typedef struct zha_buffers {
    void*        k;        /* device K [H_kv][capacity][d] */
    void*        v;        /* device V [H_kv][capacity][d] */
    const float* ref_q;    /* device [H_kv][R][d] float32 */
    void*        tree;     /* device, zha_tree_bytes(cfg) bytes */
    void*        scratch;  /* device, zha_scratch_bytes(cfg) bytes; contents need no initialisation */
} zha_buffers;

/* Validates a configuration without touching the device.  ZHA_OK or an error code. */
int zha_check_config(const zha_config* cfg);

/* Bytes of summary storage for a tree over `capacity` tokens (0 if cfg is invalid).
 * Per level l and KV head: float32 planes s[n][R][d], b[n][R] and log-sum-exp
 * lse[n][R] for n < capacity / c^l, and with plane_format = ZHA_PLANES_BF16 a
 * bfloat16 copy of s, with ZHA_PLANES_FP8 an 8-bit copy of s and its per-plane
 * float32 scales. */
size_t zha_tree_bytes(const zha_config* cfg);

/* Bytes of decode scratch (0 if cfg is invalid): candidate scores and kept
 * lists for every level at the worst-case frontier, plus split-attention
 * partials. */
size_t zha_scratch_bytes(const zha_config* cfg);

/* Bytes of scratch dense_decode needs (0 if cfg is invalid). */
size_t zha_dense_scratch_bytes(const zha_config* cfg);

/* Byte offsets, inside `tree`, of level `level` (1..L):
 *   s   float32 [H_kv][n_cap][R][d]
 *   b   float32 [H_kv][n_cap][R]
 *   lse float32 [H_kv][n_cap][R]
 *   s16 bfloat16 [H_kv][n_cap][R][d], the router's copy of s when plane_format is
 *       ZHA_PLANES_BF16 (*s16_off = -1 otherwise)
 *   s8  uint8 [H_kv][n_cap][R][d] FP8 E4M3 codes and
 *   sc  float32 [H_kv][n_cap][R] their per-plane scales (powers of two), the router's
 *       8-bit copy of s when plane_format is ZHA_PLANES_FP8 (*s8_off = *sc_off = -1
 *       otherwise)
 * with n_cap = capacity / c^level.  Any output pointer may be NULL.  Host-only;
 * ZHA_OK or ZHA_ERR_ARG. */
int zha_tree_level_offsets(const zha_config* cfg, int32_t level,
                           int64_t* s_off, int64_t* b_off, int64_t* lse_off, int64_t* n_cap,
                           int64_t* s16_off, int64_t* s8_off, int64_t* sc_off);

/* Where a decode step over n_tokens tokens leaves its routing of level `level`
 * inside `scratch` (byte offsets; host-only).  `chained` tells which layout holds:
 *   chained = 0 (a level scored over its group candidates):
 *     n_cand  int32  [H_kv]          candidates scored at this level, per KV group
 *     sigma   float32[H_kv][G][sig_stride] score of candidate position i for query head
 *                                     g*G+j (-inf where the candidate is not the
 *                                     head's); candidate positions follow ascending
 *                                     node index
 *     n_kept  int32  [H_kv]          nodes kept by at least one head of the group
 *     kept    int32  [H_kv][n_cap]   those node indices, ascending
 *     mask    uint32 [H_kv][n_cap]   bit j set when query head g*G+j kept the node
 *     stats   int32  [H_q][2]        per query head: candidates, kept
 *   chained = 1 (one of the first, small levels, every node scored):
 *     sigma   float32[H_kv][G][sig_stride] score of node i for query head g*G+j
 *     kbm     uint64 [H_kv][G][wcap] per-head kept bitmap over node ids
 *     stats   int32  [H_q][2]        per query head: candidates, kept
 *     (n_kept, kept and mask hold the group kept list only at the last chained
 *     level)
 * Values are valid only for levels the step routed (levels with at least one
 * complete node).  ZHA_OK or ZHA_ERR_ARG. */
typedef struct zha_route_offsets {
    int64_t n_cand, sigma, n_kept, kept, mask, stats, kbm;
    int64_t n_cap, wcap;
    int64_t chained;
    int64_t sig_stride;        /* row stride of sigma: n_cap rounded up to a multiple of 4 */
} zha_route_offsets;
int zha_route_level_offsets(const zha_config* cfg, int64_t n_tokens, int32_t level, zha_route_offsets* out);

/* Summarise every complete node over tokens [0, n_tokens) of K (levels 1..L):
 * leaves from raw keys, higher levels by the exact log-sum-exp merge of their
 * c children (equal to summarising the raw keys, since reference queries are
 * shared across levels).  0 <= n_tokens <= capacity.  Overwrites those tree
 * slots; leaves other slots untouched.
 * Defined by: page "Zyphra 分层注意力（ZHA）…", section 机制拆解 (chunk
 * summaries compressed again level by level); page "ZHA 用树形稀疏注意力改造现有大模型",
 * section 稀疏注意力为什么还会被索引拖慢 (tangent planes at reference queries). */
int zha_build_tree(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, void* stream);

/* Append one token: write k_new, v_new (device [H_kv][d] of kv_dtype) into row
 * n_before of K and V, then summarise each node the token completes (levels l
 * with (n_before + 1) % c^l == 0).  The caller then holds n_before + 1 tokens.
 * Requires n_before + 1 <= capacity and a tree that is current for n_before.
 * Defined by: page rit.work "zha-tree-indexer-long-context", section "Дерево
 * сокращает сам поиск нужных ключей" (the tree grows with the context; the
 * full cache is kept). */
int zha_append_token(const zha_config* cfg, const zha_buffers* bufs, int64_t n_before,
                     const void* k_new, const void* v_new, void* stream);

/* Per-step statistics a decode step writes to device memory when asked (see
 * zha_decode_step).  Index l-1 holds level l; levels above levels, and levels the
 * step did not route, hold zero.  A KV group's candidates at a level are the union
 * of its query heads' candidates: the nodes whose summary planes the router must
 * read once for the whole group. */
#define ZHA_STATS_MAX_LEVELS 32
typedef struct zha_stats {
    int64_t n_tokens;                                /* tokens the step attended over */
    int32_t top_level;                               /* highest level with a complete node (0: none) */
    int32_t levels;                                  /* cfg->levels */
    int64_t cand[ZHA_STATS_MAX_LEVELS];              /* candidates, summed over query heads */
    int64_t kept[ZHA_STATS_MAX_LEVELS];              /* kept nodes, summed over query heads */
    int64_t group_cand[ZHA_STATS_MAX_LEVELS];        /* union candidates, summed over KV groups */
    int64_t group_kept[ZHA_STATS_MAX_LEVELS];        /* nodes kept by some head of a group, summed over groups */
    int64_t bytes_read[ZHA_STATS_MAX_LEVELS];        /* summary bytes the level's routing needs:
                                                        group_cand * n_ref * (head_dim * e + 4), e = 4
                                                        (float32 planes) or 2 (ZHA_PLANES_BF16); with
                                                        ZHA_PLANES_FP8 group_cand * n_ref * (head_dim + 8)
                                                        (codes, scale and b) */
    int64_t bytes_streamed[ZHA_STATS_MAX_LEVELS];    /* summary bytes the kernels streamed for the level:
                                                        equal to bytes_read, except at the small top levels
                                                        whose every complete node is scored ahead of their
                                                        selection, and at the level below them when its
                                                        every node is scored while they are selected (then
                                                        n_nodes * n_kv_heads times the same bytes per node) */
    int64_t gather_tokens;                           /* distinct tokens attended, summed over KV groups */
    int64_t gather_bytes;                            /* K and V bytes those tokens occupy */
} zha_stats;

/* Bytes of the `sel` output of zha_decode_step: int32 [n_q_heads][1 + capacity / chunk]. */
size_t zha_sel_bytes(const zha_config* cfg);

/* One decode step for all query heads over tokens [0, n_tokens) (1 <= n_tokens
 * <= capacity) with a tree current for n_tokens.  Routes every query head
 * independently from the top level down, then attends exactly over its
 * selected raw tokens; writes out [H_q][d] float32.  The routing of each level
 * stays in scratch until the next call (zha_route_level_offsets).
 *   sel    NULL, or device int32 [H_q][1 + capacity / chunk] (zha_sel_bytes):
 *          row h receives head h's kept level-1 chunk count k, then the k chunk
 *          indices in ascending order (chunk j covers tokens [j c, j c + c)).
 *          Head h attends over those chunks, token 0 and the tail
 *          [c (n_tokens / c), n_tokens).  Entries past k are left as they were.
 *   stats  NULL, or a device zha_stats, written by the step's last kernel.
 * Defined by: page "ZHA 用树形稀疏注意力改造现有大模型", section
 * 稀疏注意力为什么还会被索引拖慢 (top-level scoring, minimal top-p node set,
 * expansion down to raw KV entries, token 0 always kept). */
int zha_decode_step(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                    const void* q, float* out, int32_t* sel, zha_stats* stats, void* stream);

/* zha_decode_step, plus HIP events recorded on `stream` around its phases:
 * events[0] before the first routing kernel; events[1] and events[2] at the
 * start and the end of the gather-attention kernel itself (recorded by its
 * dispatch, so events[1] -> events[2] is that kernel's execution time);
 * events[3] after the combine kernel.  `events` may be NULL and any entry may be
 * NULL (hipEvent_t values created by the caller).  Used to time the phases of a
 * step separately.  Same definition as zha_decode_step. */
int zha_decode_step_timed(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                          const void* q, float* out, int32_t* sel, zha_stats* stats,
                          void* const* events, void* stream);

/* A batch of n_queries decode queries over the same cache and tree, routed
 * together: every launch of the step serves all of them (each query keeps its
 * own frontiers, cuts and token sets; its results equal those of
 * zha_decode_step on that query alone up to the attention's summation order).
 *   q      [n_queries][n_q_heads][d] in kv_dtype.
 *   out    [n_queries][n_q_heads][d] float32.
 *   sel    NULL, or int32 [n_queries][n_q_heads][1 + capacity / chunk], as
 *          zha_decode_step's per query.
 *   bufs->scratch must hold zha_batch_scratch_bytes(cfg, n_queries) bytes.
 * Returns ZHA_ERR_ARG for n_queries < 1.  Defined by: page rit.work
 * "zha-tree-indexer-long-context", section "Дерево сокращает сам поиск нужных
 * ключей" (the tree serves every query: the search is sub-quadratic over a
 * sequence of queries, not one). */
size_t zha_batch_scratch_bytes(const zha_config* cfg, int32_t n_queries);
int zha_decode_batch(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, int32_t n_queries,
                     const void* q, float* out, int32_t* sel, void* stream);

/* zha_decode_step with a HIP event recorded on `stream` before the step's first
 * kernel (events[0]) and after each kernel it launches (events[1], events[2],
 * ...), up to max_events events in all; kinds[i] names the kernel that ends at
 * events[i] as 100 * kind + level (kinds[0] = 100 * 0 + the first routed
 * level).  *n_events receives how many events were recorded.  The step then
 * writes no sel/stats.  The event packets between kernels take a little time of
 * their own: for a per-kernel breakdown, not for the step's latency.  Returns
 * ZHA_ERR_ARG when events, kinds or n_events is NULL, max_events < 1 or one of
 * events[0 .. max_events) is NULL (hipEvent_t values created by the caller).
 * Same definition as zha_decode_step. */
enum {
    ZHA_TRACE_SCORE_ALL = 1,   /* scores of every node of the chained levels */
    ZHA_TRACE_CHAIN = 2,       /* per-head selection of the chained levels */
    ZHA_TRACE_MERGE_IDS = 3,   /* level-1 group list when the chain reaches level 1 */
    ZHA_TRACE_SCORE = 4,       /* a level's candidate scores */
    ZHA_TRACE_SELECT = 5,      /* a level's per-head cut */
    ZHA_TRACE_APPLY = 6,       /* a level's head masks and group kept list */
    ZHA_TRACE_GATHER = 7,      /* sparse attention over the kept chunks, sink and tail */
    ZHA_TRACE_COMBINE = 8,     /* merge of the gather's split partials */
    ZHA_TRACE_CROSS = 9,       /* a large frontier's crossing-bin keys listed */
    ZHA_TRACE_RESOLVE = 10     /* a large frontier's cut from that list */
};
int zha_decode_step_traced(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                           const void* q, float* out, void* const* events, int32_t max_events,
                           int32_t* kinds, int32_t* n_events, void* stream);

/* Dense baseline: exact softmax attention of every query head over all
 * n_tokens tokens (1 <= n_tokens <= capacity); scratch of
 * zha_dense_scratch_bytes(cfg) bytes (its split partials: the library
 * allocates nothing).  cfg's tree fields are ignored apart from validation.
 * Defined by: page rit.work "zha-tree-indexer-long-context", section "Дерево
 * сокращает сам поиск нужных ключей" (full attention reads the whole cache for
 * every new token). */
int dense_decode(const zha_config* cfg, const void* k, const void* v, int64_t n_tokens,
                 const void* q, float* out, void* scratch, void* stream);

/* Router fidelity of the last decode step, a diagnostic beside the hot path: for
 * query head h and level l (1..L), recall[h][l - 1] is the exact attention
 * probability mass at q (softmax over all n_tokens tokens) of the tokens whose
 * level-l node the head kept, tokens under no complete level-l node counting as
 * kept; recall[h][L] is the mass of the token set the step attended (its kept
 * level-1 chunks, token 0 and the raw tail).  recall: device float32
 * [n_q_heads][levels + 1].  work: device, zha_fidelity_work_bytes(cfg, n_tokens)
 * bytes.  Reads the routing a zha_decode_step with the same cfg, bufs, n_tokens
 * and q left in scratch, and rewrites the per-head kept bitmaps of the levels it
 * selected below its first small levels there.  Runs three passes over the
 * cache.  Defined by: page "ZHA 用树形稀疏注意力改造现有大模型", section
 * 256K 的质量结果 (how much of the true attention the router keeps). */
size_t zha_fidelity_work_bytes(const zha_config* cfg, int64_t n_tokens);
int zha_route_fidelity(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                       const void* q, float* recall, void* work, void* stream);

/* zha_decode_step without caller scratch, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The step's scratch is a device array inside the
 * library of ZHA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends; configurations whose zha_scratch_bytes() exceeds it are rejected
 * with ZHA_ERR_UNSUPPORTED before anything is enqueued.  Every call on a GPU
 * shares that GPU's array and leaves the step's routing in it: calls that
 * overlap in time on one GPU (several streams or threads) race and must be
 * serialised by the caller.  Allocates nothing; no sel/stats outputs. */
#define ZHA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int zha_decode_step_noalloc(const zha_config* cfg, const void* k, const void* v, const void* tree,
                            int64_t n_tokens, const void* q, float* out, void* stream);

/* Message for the last error returned on this thread ("" if none). */
const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
