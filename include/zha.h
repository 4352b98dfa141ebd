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
#define ZHA_ERR_UNSUPPORTED -3   /* valid but not implemented: head_dim != 128, group > 16, n_ref not in {1,2,4,8,16,32} */
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
} zha_config;

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
 * lse[n][R] for n < capacity / c^l. */
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
 * with n_cap = capacity / c^level.  Host-only; ZHA_OK or ZHA_ERR_ARG. */
int zha_tree_level_offsets(const zha_config* cfg, int32_t level,
                           int64_t* s_off, int64_t* b_off, int64_t* lse_off, int64_t* n_cap);

/* Where the last decode step left its routing of level `level` inside `scratch`
 * (byte offsets; host-only):
 *   n_cand  int32  [H_kv]          candidates scored at this level, per KV group
 *   sigma   float32[H_kv][G][n_cap] score of candidate position i for query head
 *                                   g*G+j (-inf where the candidate is not the
 *                                   head's); candidate positions follow ascending
 *                                   node index
 *   n_kept  int32  [H_kv]          nodes kept by at least one head of the group
 *   kept    int32  [H_kv][n_cap]   those node indices, ascending
 *   mask    uint32 [H_kv][n_cap]   bit j set when query head g*G+j kept the node
 *   stats   int32  [H_q][2]        per query head: candidates, kept
 * Values are valid only for levels the step routed (levels with at least one
 * complete node).  ZHA_OK or ZHA_ERR_ARG. */
typedef struct zha_route_offsets {
    int64_t n_cand, sigma, n_kept, kept, mask, stats;
    int64_t n_cap;
} zha_route_offsets;
int zha_route_level_offsets(const zha_config* cfg, int32_t level, zha_route_offsets* out);

/* Summarise every complete node over tokens [0, n_tokens) of K (levels 1..L):
 * leaves from raw keys, higher levels by the exact log-sum-exp merge of their
 * c children (equal to summarising the raw keys, since reference queries are
 * shared across levels).  0 <= n_tokens <= capacity.  Overwrites those tree
 * slots; leaves other slots untouched. */
int zha_build_tree(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, void* stream);

/* Append one token: write k_new, v_new (device [H_kv][d] of kv_dtype) into row
 * n_before of K and V, then summarise each node the token completes (levels l
 * with (n_before + 1) % c^l == 0).  The caller then holds n_before + 1 tokens.
 * Requires n_before + 1 <= capacity and a tree that is current for n_before. */
int zha_append_token(const zha_config* cfg, const zha_buffers* bufs, int64_t n_before,
                     const void* k_new, const void* v_new, void* stream);

/* One decode step for all query heads over tokens [0, n_tokens) (1 <= n_tokens
 * <= capacity) with a tree current for n_tokens.  Routes every query head
 * independently from the top level down, then attends exactly over its
 * selected raw tokens; writes out [H_q][d] float32.  The routing of each level
 * stays in scratch until the next call (zha_route_level_offsets). */
int zha_decode_step(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                    const void* q, float* out, void* stream);

/* zha_decode_step, plus HIP events recorded on `stream` around its phases:
 * events[0] before the first routing kernel; events[1] and events[2] at the
 * start and the end of the gather-attention kernel itself (recorded by its
 * dispatch, so events[1] -> events[2] is that kernel's execution time);
 * events[3] after the combine kernel.  `events` may be NULL and any entry may be
 * NULL (hipEvent_t values created by the caller).  Used to time the phases of a
 * step separately. */
int zha_decode_step_timed(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens,
                          const void* q, float* out, void* const* events, void* stream);

/* Dense baseline: exact softmax attention of every query head over all
 * n_tokens tokens (1 <= n_tokens <= capacity); scratch of
 * zha_dense_scratch_bytes(cfg) bytes.  cfg's tree fields are ignored apart
 * from validation. */
int dense_decode(const zha_config* cfg, const void* k, const void* v, int64_t n_tokens,
                 const void* q, float* out, void* scratch, void* stream);

/* Message for the last error returned on this thread ("" if none). */
const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
