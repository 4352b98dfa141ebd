// C ABI of libzha.so: argument validation, tree and scratch layouts, and the
// launch sequence of each entry point.  See include/zha.h for the contract.
#include "../../include/zha.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "zha_common.h"
#include "zha_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return ZHA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(ZHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int validate(const zha_config* cfg) {
    if (!cfg) return fail(ZHA_ERR_ARG, "config is NULL");
    if (cfg->n_kv_heads < 1) return fail(ZHA_ERR_ARG, "n_kv_heads must be >= 1 (got %d)", cfg->n_kv_heads);
    if (cfg->n_q_heads < cfg->n_kv_heads || cfg->n_q_heads % cfg->n_kv_heads != 0)
        return fail(ZHA_ERR_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", cfg->n_q_heads,
                    cfg->n_kv_heads);
    if (cfg->n_q_heads / cfg->n_kv_heads > ZHA_MAX_GROUP)
        return fail(ZHA_ERR_UNSUPPORTED, "query heads per KV head must be <= %d (got %d)", ZHA_MAX_GROUP,
                    cfg->n_q_heads / cfg->n_kv_heads);
    if (cfg->head_dim < 1) return fail(ZHA_ERR_ARG, "head_dim must be >= 1 (got %d)", cfg->head_dim);
    if (cfg->head_dim != ZHA_D) return fail(ZHA_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", ZHA_D, cfg->head_dim);
    if (cfg->chunk < 2) return fail(ZHA_ERR_ARG, "chunk must be >= 2 (got %d)", cfg->chunk);
    if (cfg->chunk > 1024) return fail(ZHA_ERR_UNSUPPORTED, "chunk must be <= 1024 (got %d)", cfg->chunk);
    if (cfg->levels < 1) return fail(ZHA_ERR_ARG, "levels must be >= 1 (got %d)", cfg->levels);
    if (cfg->levels > 32) return fail(ZHA_ERR_UNSUPPORTED, "levels must be <= 32 (got %d)", cfg->levels);
    if (cfg->n_ref < 1) return fail(ZHA_ERR_ARG, "n_ref must be >= 1 (got %d)", cfg->n_ref);
    {
        const int r = cfg->n_ref;
        if (r > 32 || (r & (r - 1)) != 0)
            return fail(ZHA_ERR_UNSUPPORTED, "n_ref must be 1, 2, 4, 8, 16 or 32 (got %d)", r);
    }
    if (!(cfg->top_p > 0.0f && cfg->top_p <= 1.0f))
        return fail(ZHA_ERR_ARG, "top_p must lie in (0, 1] (got %g)", (double)cfg->top_p);
    if (cfg->kv_dtype != ZHA_BF16 && cfg->kv_dtype != ZHA_F32)
        return fail(ZHA_ERR_ARG, "kv_dtype must be ZHA_BF16 or ZHA_F32 (got %d)", cfg->kv_dtype);
    if (cfg->capacity < 1) return fail(ZHA_ERR_ARG, "capacity must be >= 1 (got %lld)", (long long)cfg->capacity);
    if (cfg->capacity >= (int64_t(1) << 31))
        return fail(ZHA_ERR_UNSUPPORTED, "capacity must be < 2^31 (got %lld)", (long long)cfg->capacity);
    if (cfg->sink == 0) return fail(ZHA_ERR_UNSUPPORTED, "sink = 0 (no attention sink) is not implemented");
    if (cfg->sink != 1) return fail(ZHA_ERR_ARG, "sink must be 1 (got %d)", cfg->sink);
    if (cfg->plane_format != ZHA_PLANES_F32 && cfg->plane_format != ZHA_PLANES_BF16 &&
        cfg->plane_format != ZHA_PLANES_FP8)
        return fail(ZHA_ERR_ARG, "plane_format must be ZHA_PLANES_F32, ZHA_PLANES_BF16 or ZHA_PLANES_FP8 (got %d)",
                    cfg->plane_format);
    return ZHA_OK;
}

// Tokens covered by a level-l node, saturated above capacity (no overflow).
int64_t span_of(const zha_config* cfg, int level) {
    int64_t s = 1;
    for (int i = 0; i < level; ++i) {
        if (s > cfg->capacity) return cfg->capacity + 1;
        s *= cfg->chunk;
    }
    return s;
}

int64_t n_nodes(const zha_config* cfg, int64_t n_tokens, int level) { return n_tokens / span_of(cfg, level); }

struct Layout {
    int L = 0, G = 0, H = 0, R = 0;
    std::vector<int64_t> cap;             // node slots per level (index 1..L)
    // tree
    std::vector<size_t> t_s, t_b, t_l, t_s16;   // t_s16: bfloat16 router copy of s (0: none)
    std::vector<size_t> t_s8, t_sc;             // 8-bit router copy of s and its per-plane scales (0: none)
    size_t tree_bytes = 0;
    // decode scratch
    std::vector<size_t> sig, kbm, klist, kmask, ncand, nkept, stats;
    std::vector<size_t> hblk, ghist, hdone, hcut, tick, desc;   // selection state of a level below the chain
    std::vector<size_t> pub, gcnt, gpart, glist;  // frontiers beyond ZHA_LDS_KEYS (glist 0: the level never has one)
    std::vector<size_t> sign;             // node-indexed scores of a level scored during the chain (0: none)
    std::vector<int64_t> wcap;            // bitmap words per head per level
    std::vector<int64_t> sstr;            // score row stride per level (slots rounded up to 4)
    size_t pm = 0, pl = 0, po = 0, nact = 0;
    size_t noparent = 0;                  // readable, never written: the first routed level's parent arrays
    size_t scratch_bytes = 0;
    size_t dense_bytes = 0;
};

void attn_partials(const zha_config* cfg, size_t& off, size_t& pm, size_t& pl, size_t& po, size_t& nact) {
    const size_t H = cfg->n_kv_heads, G = cfg->n_q_heads / cfg->n_kv_heads;
    pm = off; off = align_up(off + sizeof(float) * H * ZHA_ATTN_MAXB * G);
    pl = off; off = align_up(off + sizeof(float) * H * ZHA_ATTN_MAXB * G);
    po = off; off = align_up(off + sizeof(float) * H * ZHA_ATTN_MAXB * G * ZHA_D);
    nact = off; off = align_up(off + sizeof(int32_t) * H);
}

// A level of n nodes per KV group may be scored whole while the chain above it
// selects: its float32 planes over every group within kSpecBytes, and compute
// units left over by the chain's H x G selecting workgroups.
#ifndef ZHA_COPY_CAP
#define ZHA_COPY_CAP 192
#endif
#ifndef ZHA_SPEC_MIB
#define ZHA_SPEC_MIB 96
#endif
constexpr size_t kSpecBytes = (size_t)ZHA_SPEC_MIB << 20;
constexpr int kSpecCUs = 256;
bool spec_fits(size_t n, size_t R, size_t H, size_t G) {
    return n * R * (sizeof(float) * ZHA_D + sizeof(float)) * H <= kSpecBytes && H * G + H <= (size_t)kSpecCUs;
}

Layout make_layout(const zha_config* cfg) {
    Layout y;
    y.L = cfg->levels;
    y.H = cfg->n_kv_heads;
    y.G = cfg->n_q_heads / cfg->n_kv_heads;
    y.R = cfg->n_ref;
    const size_t H = y.H, G = y.G, R = y.R;
    y.cap.assign(y.L + 2, 0);
    for (int l = 1; l <= y.L; ++l) y.cap[l] = n_nodes(cfg, cfg->capacity, l);
    y.t_s.assign(y.L + 1, 0); y.t_b.assign(y.L + 1, 0); y.t_l.assign(y.L + 1, 0); y.t_s16.assign(y.L + 1, 0);
    y.t_s8.assign(y.L + 1, 0); y.t_sc.assign(y.L + 1, 0);
    size_t off = 0;
    for (int l = 1; l <= y.L; ++l) {
        const size_t n = (size_t)y.cap[l];
        y.t_s[l] = off; off = align_up(off + sizeof(float) * H * n * R * ZHA_D);
        y.t_b[l] = off; off = align_up(off + sizeof(float) * H * n * R);
        y.t_l[l] = off; off = align_up(off + sizeof(float) * H * n * R);
        if (cfg->plane_format == ZHA_PLANES_BF16) {
            y.t_s16[l] = off; off = align_up(off + sizeof(uint16_t) * H * n * R * ZHA_D);
        }
        if (cfg->plane_format == ZHA_PLANES_FP8) {
            y.t_s8[l] = off; off = align_up(off + sizeof(uint8_t) * H * n * R * ZHA_D);
            y.t_sc[l] = off; off = align_up(off + sizeof(float) * H * n * R);
        }
    }
    y.tree_bytes = off;

    off = 0;
    for (auto* v : {&y.sig, &y.kbm, &y.klist, &y.kmask, &y.ncand, &y.nkept, &y.stats, &y.hblk, &y.ghist, &y.hdone, &y.hcut,
                    &y.tick, &y.desc, &y.pub, &y.gcnt, &y.gpart, &y.glist, &y.sign})
        v->assign(y.L + 1, 0);
    y.wcap.assign(y.L + 1, 0);
    y.sstr.assign(y.L + 1, 0);
    for (int l = 1; l <= y.L; ++l) {
        const size_t n = (size_t)y.cap[l];
        y.wcap[l] = (int64_t)((n + 63) / 64);
        y.sstr[l] = (int64_t)((n + 3) / 4 * 4);
        y.sig[l] = off;   off = align_up(off + sizeof(float) * H * G * (size_t)y.sstr[l]);
        y.kbm[l] = off;   off = align_up(off + sizeof(uint64_t) * H * G * (size_t)y.wcap[l]);
        y.klist[l] = off; off = align_up(off + sizeof(int32_t) * H * n);
        y.kmask[l] = off; off = align_up(off + sizeof(uint32_t) * H * n);
        y.ncand[l] = off; off = align_up(off + sizeof(int32_t) * H);
        y.nkept[l] = off; off = align_up(off + sizeof(int32_t) * H);
        y.stats[l] = off; off = align_up(off + sizeof(int32_t) * 2 * H * G);
        y.hblk[l] = off;  off = align_up(off + sizeof(float) * H * G * ZHA_SCORE_MAXB);
        y.ghist[l] = off; off = align_up(off + sizeof(uint64_t) * H * G * ZHA_HIST_BINS);
        y.hdone[l] = off; off = align_up(off + sizeof(uint32_t) * H * G);
        y.hcut[l] = off;  off = align_up(off + 16 * H * G);
        y.tick[l] = off;  off = align_up(off + sizeof(uint32_t) * H);
        y.desc[l] = off;  off = align_up(off + sizeof(uint32_t) * H * (size_t)zha_apply_chunks((int64_t)n));
        if (spec_fits(n, R, H, G)) {
            y.sign[l] = off; off = align_up(off + sizeof(float) * H * G * (size_t)y.sstr[l]);
        }
        if (n > (size_t)ZHA_LDS_KEYS) {
            y.pub[l] = off;   off = align_up(off + 16 * H * G);
            y.gcnt[l] = off;  off = align_up(off + 16 * H * G);
            y.gpart[l] = off; off = align_up(off + 8 * H * G * (size_t)ZHA_CROSS_MAXW);
            y.glist[l] = off; off = align_up(off + 8 * H * G * (size_t)ZHA_GLIST);
        }
    }
    attn_partials(cfg, off, y.pm, y.pl, y.po, y.nact);
    y.noparent = off; off = align_up(off + sizeof(int32_t) * std::max<size_t>(64, H));   // one entry per group
    y.scratch_bytes = off;

    size_t doff = 0, a, b, c, d;
    attn_partials(cfg, doff, a, b, c, d);
    y.dense_bytes = doff;
    return y;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// The router's narrow copy of level l's planes s for nodes [first, first + n):
// bfloat16, or 8-bit with per-plane scales (nothing for float32 planes).
int planes16(const zha_config* cfg, const Layout& y, void* T, int l, int64_t first, int64_t n, hipStream_t s) {
    if (n <= 0) return ZHA_OK;
    hipError_t e = hipSuccess;
    if (cfg->plane_format == ZHA_PLANES_BF16)
        e = zha_launch_planes16((const float*)at(T, y.t_s[l]), (uint16_t*)at(T, y.t_s16[l]), y.H, y.cap[l],
                                cfg->n_ref, first, n, s);
    else if (cfg->plane_format == ZHA_PLANES_FP8)
        e = zha_launch_planes8((const float*)at(T, y.t_s[l]), (uint8_t*)at(T, y.t_s8[l]), (float*)at(T, y.t_sc[l]),
                               y.H, y.cap[l], cfg->n_ref, first, n, s);
    return e == hipSuccess ? ZHA_OK : hip_fail(e, "plane copy launch");
}

// Attention workgroups per KV group: one per 8 tiles of 32 slots over every
// cached token, at most one resident round of the whole device (768 workgroups:
// 256 CUs x 3 resident) so that no partial second round trails the launch.  The
// kernel then activates one of them per 4 tiles of the slots it actually reads
// (kMinTilesPerBlock), up to this grid.
int attn_blocks(int64_t n_slots, int H, int kv_dtype) {
    const int64_t tiles = (n_slots + 31) / 32;
    int64_t b = (tiles + 7) / 8;
    if (b < 1) b = 1;
    if (b > ZHA_ATTN_MAXB) b = ZHA_ATTN_MAXB;
    // one resident round on 256 compute units
    const int64_t round = 256 * (kv_dtype == ZHA_BF16 ? ZHA_ATTN_BLOCKS_BF16 : ZHA_ATTN_BLOCKS_F32) / H;
    if (b > round) b = round > 0 ? round : 1;
    return (int)b;
}

float tau_of(const zha_config* cfg) { return 1.0f / std::sqrt((float)cfg->head_dim); }

// Highest level with a complete node over n_tokens tokens (0: none).
int top_level(const zha_config* cfg, int64_t n_tokens) {
    for (int l = cfg->levels; l >= 1; --l)
        if (n_nodes(cfg, n_tokens, l) > 0) return l;
    return 0;
}

// Levels of the chain, counted from the top: each at most ZHA_CHAIN_SLOTS complete
// nodes, together at most ZHA_CHAIN_PLANES planes per group.
int chain_levels(const zha_config* cfg, int64_t n_tokens, int top) {
    int nchain = 0;
    int64_t planes = 0;
    for (int l = top; l >= 1 && nchain < ZHA_MAX_CHAIN; --l) {
        if (n_nodes(cfg, n_tokens, l) > ZHA_CHAIN_SLOTS) break;
        planes += n_nodes(cfg, n_tokens, l) * (int64_t)cfg->n_ref;
        if (planes > ZHA_CHAIN_PLANES) break;
        ++nchain;
    }
    return nchain;
}

}  // namespace

extern "C" {

const char* zha_last_error(void) { return g_err; }

int zha_check_config(const zha_config* cfg) {
    int rc = validate(cfg);
    return rc == ZHA_OK ? ok() : rc;
}

size_t zha_tree_bytes(const zha_config* cfg) {
    if (validate(cfg) != ZHA_OK) return 0;
    ok();
    return make_layout(cfg).tree_bytes;
}

size_t zha_scratch_bytes(const zha_config* cfg) {
    if (validate(cfg) != ZHA_OK) return 0;
    ok();
    return make_layout(cfg).scratch_bytes;
}

size_t zha_dense_scratch_bytes(const zha_config* cfg) {
    if (validate(cfg) != ZHA_OK) return 0;
    ok();
    return make_layout(cfg).dense_bytes;
}

size_t zha_sel_bytes(const zha_config* cfg) {
    if (validate(cfg) != ZHA_OK) return 0;
    ok();
    return sizeof(int32_t) * (size_t)cfg->n_q_heads * (size_t)(cfg->capacity / cfg->chunk + 1);
}

int zha_tree_level_offsets(const zha_config* cfg, int32_t level, int64_t* s_off, int64_t* b_off, int64_t* lse_off,
                           int64_t* n_cap, int64_t* s16_off, int64_t* s8_off, int64_t* sc_off) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (level < 1 || level > cfg->levels) return fail(ZHA_ERR_ARG, "level %d outside 1..%d", level, cfg->levels);
    Layout y = make_layout(cfg);
    if (s_off) *s_off = (int64_t)y.t_s[level];
    if (b_off) *b_off = (int64_t)y.t_b[level];
    if (lse_off) *lse_off = (int64_t)y.t_l[level];
    if (n_cap) *n_cap = y.cap[level];
    if (s16_off) *s16_off = cfg->plane_format == ZHA_PLANES_BF16 ? (int64_t)y.t_s16[level] : -1;
    if (s8_off) *s8_off = cfg->plane_format == ZHA_PLANES_FP8 ? (int64_t)y.t_s8[level] : -1;
    if (sc_off) *sc_off = cfg->plane_format == ZHA_PLANES_FP8 ? (int64_t)y.t_sc[level] : -1;
    return ok();
}

int zha_route_level_offsets(const zha_config* cfg, int64_t n_tokens, int32_t level, zha_route_offsets* out) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(ZHA_ERR_ARG, "out is NULL");
    if (level < 1 || level > cfg->levels) return fail(ZHA_ERR_ARG, "level %d outside 1..%d", level, cfg->levels);
    if (n_tokens < 1 || n_tokens > cfg->capacity)
        return fail(ZHA_ERR_ARG, "n_tokens %lld outside 1..capacity", (long long)n_tokens);
    Layout y = make_layout(cfg);
    const int top = top_level(cfg, n_tokens);
    const int nchain = chain_levels(cfg, n_tokens, top);
    out->chained = (level <= top && top - level < nchain) ? 1 : 0;
    out->kbm = (int64_t)y.kbm[level];
    out->wcap = y.wcap[level];
    out->n_cand = (int64_t)y.ncand[level];
    out->sigma = (int64_t)y.sig[level];
    out->n_kept = (int64_t)y.nkept[level];
    out->kept = (int64_t)y.klist[level];
    out->mask = (int64_t)y.kmask[level];
    out->stats = (int64_t)y.stats[level];
    out->n_cap = y.cap[level];
    out->sig_stride = y.sstr[level];
    return ok();
}

int zha_build_tree(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!bufs || !bufs->k || !bufs->ref_q || !bufs->tree)
        return fail(ZHA_ERR_ARG, "buffers: k, ref_q and tree must be non-NULL");
    if (n_tokens < 0) return fail(ZHA_ERR_ARG, "n_tokens must be >= 0 (got %lld)", (long long)n_tokens);
    if (n_tokens > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)n_tokens,
                    (long long)cfg->capacity);
    Layout y = make_layout(cfg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int c = cfg->chunk, R = cfg->n_ref;
    float* T = static_cast<float*>(bufs->tree);
    // the leaf kernels that hold whole level-2 nodes write those as well (fused = 1)
    const bool two = y.L >= 2 && n_nodes(cfg, n_tokens, 2) > 0;
    int fused = 0;
    hipError_t e = zha_launch_leaf_summary(
        cfg->kv_dtype, bufs->k, bufs->ref_q, (float*)at(T, y.t_s[1]), (float*)at(T, y.t_b[1]), (float*)at(T, y.t_l[1]),
        y.H, cfg->capacity, y.cap[1], c, R, 0, n_nodes(cfg, n_tokens, 1), tau_of(cfg),
        two ? (float*)at(T, y.t_s[2]) : nullptr, two ? (float*)at(T, y.t_b[2]) : nullptr,
        two ? (float*)at(T, y.t_l[2]) : nullptr, two ? y.cap[2] : 0, &fused, s);
    if (e != hipSuccess) return hip_fail(e, "leaf summary launch");
    if ((rc = planes16(cfg, y, T, 1, 0, n_nodes(cfg, n_tokens, 1), s))) return rc;
    auto merge = [&](int l, int64_t first, int64_t n) {
        return zha_launch_merge((float*)at(T, y.t_s[l - 1]), (float*)at(T, y.t_b[l - 1]), (float*)at(T, y.t_l[l - 1]),
                                (float*)at(T, y.t_s[l]), (float*)at(T, y.t_b[l]), (float*)at(T, y.t_l[l]), y.H,
                                y.cap[l - 1], y.cap[l], c, R, first, n, s);
    };
    for (int l = 2; l <= y.L;) {
        const int64_t n = n_nodes(cfg, n_tokens, l);
        if (n == 0) break;
        if (l == 2 && fused) {                 // written by the leaf kernel
            if ((rc = planes16(cfg, y, T, l, 0, n, s))) return rc;
            ++l;
            continue;
        }
        const int64_t ng = l < y.L ? n_nodes(cfg, n_tokens, l + 1) : 0;
        if (ng > 0 && zha_merge2_lds_bytes(c, R) <= 64 * 1024) {
            // levels l and l + 1 in one launch for the nodes under complete level-(l + 1)
            // nodes, then level l's right-edge nodes (orphans one level up) alone
            e = zha_launch_merge2((float*)at(T, y.t_s[l - 1]), (float*)at(T, y.t_b[l - 1]),
                                  (float*)at(T, y.t_l[l - 1]), (float*)at(T, y.t_s[l]), (float*)at(T, y.t_b[l]),
                                  (float*)at(T, y.t_l[l]), (float*)at(T, y.t_s[l + 1]), (float*)at(T, y.t_b[l + 1]),
                                  (float*)at(T, y.t_l[l + 1]), y.H, y.cap[l - 1], y.cap[l], y.cap[l + 1], c, R, 0, ng,
                                  s);
            if (e != hipSuccess) return hip_fail(e, "merge launch (two levels)");
            if (n > (int64_t)c * ng && (e = merge(l, (int64_t)c * ng, n - (int64_t)c * ng)) != hipSuccess)
                return hip_fail(e, "merge launch");
            if ((rc = planes16(cfg, y, T, l, 0, n, s))) return rc;
            if ((rc = planes16(cfg, y, T, l + 1, 0, ng, s))) return rc;
            l += 2;
            continue;
        }
        if ((e = merge(l, 0, n)) != hipSuccess) return hip_fail(e, "merge launch");
        if ((rc = planes16(cfg, y, T, l, 0, n, s))) return rc;
        ++l;
    }
    return ok();
}

int zha_append_token(const zha_config* cfg, const zha_buffers* bufs, int64_t n_before, const void* k_new,
                     const void* v_new, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!bufs || !bufs->k || !bufs->v || !bufs->ref_q || !bufs->tree || !k_new || !v_new)
        return fail(ZHA_ERR_ARG, "buffers k, v, ref_q, tree and k_new, v_new must be non-NULL");
    if (n_before < 0) return fail(ZHA_ERR_ARG, "n_before must be >= 0 (got %lld)", (long long)n_before);
    if (n_before + 1 > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "appending token %lld exceeds capacity %lld", (long long)n_before,
                    (long long)cfg->capacity);
    Layout y = make_layout(cfg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int c = cfg->chunk, R = cfg->n_ref;
    hipError_t e = zha_launch_kv_write(cfg->kv_dtype, bufs->k, bufs->v, k_new, v_new, y.H, cfg->capacity, n_before, s);
    if (e != hipSuccess) return hip_fail(e, "kv write launch");
    const int64_t n = n_before + 1;
    if (n % c != 0) return ok();
    float* T = static_cast<float*>(bufs->tree);
    e = zha_launch_leaf_summary(cfg->kv_dtype, bufs->k, bufs->ref_q, (float*)at(T, y.t_s[1]), (float*)at(T, y.t_b[1]),
                                (float*)at(T, y.t_l[1]), y.H, cfg->capacity, y.cap[1], c, R, n / c - 1, 1,
                                tau_of(cfg), nullptr, nullptr, nullptr, 0, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "leaf summary launch");
    if ((rc = planes16(cfg, y, T, 1, n / c - 1, 1, s))) return rc;
    for (int l = 2; l <= y.L; ++l) {
        const int64_t span = span_of(cfg, l);
        if (span > cfg->capacity || n % span != 0) break;
        e = zha_launch_merge((float*)at(T, y.t_s[l - 1]), (float*)at(T, y.t_b[l - 1]), (float*)at(T, y.t_l[l - 1]),
                             (float*)at(T, y.t_s[l]), (float*)at(T, y.t_b[l]), (float*)at(T, y.t_l[l]), y.H,
                             y.cap[l - 1], y.cap[l], c, R, n / span - 1, 1, s);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
        if ((rc = planes16(cfg, y, T, l, n / span - 1, 1, s))) return rc;
    }
    return ok();
}

}  // extern "C"

namespace {
int record(void* const* events, int i, hipStream_t s) {
    if (!events || !events[i]) return ZHA_OK;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    return e == hipSuccess ? ZHA_OK : hip_fail(e, "event record");
}

// An event after each kernel of a traced step (none when ev is null).
struct Trace {
    void* const* ev = nullptr;
    int32_t* kinds = nullptr;
    int max = 0, n = 0;
    int mark(int kind, int level, hipStream_t s) {
        if (!ev || n >= max) return ZHA_OK;
        if (kinds) kinds[n] = kind * 100 + level;
        return record(ev, n++, s);
    }
};

// A batch of n_queries decode queries routes as n_queries x H_kv virtual KV groups:
// virtual group v = query * H_kv + g has its own frontiers, kept lists and
// partials in scratch (laid out for n_queries x H_kv groups), while the tree
// planes and the cache rows it reads are those of group g = v % H_kv.
zha_config virtual_config(const zha_config* cfg, int n_queries) {
    zha_config v = *cfg;
    v.n_kv_heads = cfg->n_kv_heads * n_queries;
    v.n_q_heads = cfg->n_q_heads * n_queries;
    return v;
}

int decode_impl(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q, float* out,
                int32_t* sel, zha_stats* stats, void* const* events, void* stream, Trace* tr = nullptr,
                int n_queries = 1) {
    Trace untraced;
    Trace& TR = tr ? *tr : untraced;
    int rc = validate(cfg);
    if (rc) return rc;
    if (n_queries < 1) return fail(ZHA_ERR_ARG, "n_queries must be >= 1 (got %d)", n_queries);
    if (!bufs || !bufs->k || !bufs->v || !bufs->tree || !bufs->scratch || !q || !out)
        return fail(ZHA_ERR_ARG, "buffers k, v, tree, scratch and q, out must be non-NULL");
    if (n_tokens < 1) return fail(ZHA_ERR_ARG, "n_tokens must be >= 1 (got %lld)", (long long)n_tokens);
    if (n_tokens > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)n_tokens,
                    (long long)cfg->capacity);
    const zha_config vcfg = virtual_config(cfg, n_queries);
    Layout y = make_layout(&vcfg);             // scratch: every virtual group
    Layout yt = make_layout(cfg);              // tree: the real groups
    const int hkv = cfg->n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int c = cfg->chunk, R = cfg->n_ref;
    const float tau = tau_of(cfg);
    char* T = static_cast<char*>(bufs->tree);
    char* X = static_cast<char*>(bufs->scratch);

    const int top = top_level(cfg, n_tokens);
    if ((rc = record(events, 0, s))) return rc;

    // Arguments of level l (parents: the kept list of level l + 1, or, at the first
    // routed level, a small scratch region that no kernel writes, so that a kernel
    // may issue its parent reads before it knows whether the level is the first).
    auto level_args = [&](int l) {
        ZhaLevelArgs a{};
        a.S = (const float*)(T + yt.t_s[l]);
        a.S16 = cfg->plane_format == ZHA_PLANES_BF16 ? (const uint16_t*)(T + yt.t_s16[l]) : nullptr;
        a.S8 = cfg->plane_format == ZHA_PLANES_FP8 ? (const uint8_t*)(T + yt.t_s8[l]) : nullptr;
        a.SC = cfg->plane_format == ZHA_PLANES_FP8 ? (const float*)(T + yt.t_sc[l]) : nullptr;
        a.B = (const float*)(T + yt.t_b[l]);
        a.hkv = hkv;
        a.cap = y.cap[l];
        a.top = l == top ? 1 : 0;
        a.n_top = n_nodes(cfg, n_tokens, l);
        a.dc = zha_make_div((uint32_t)c);
        a.ncand = (int32_t*)(X + y.ncand[l]);
        a.sig = (float*)(X + y.sig[l]);
        a.sstride = y.sstr[l];
        a.kbm = (uint64_t*)(X + y.kbm[l]);
        a.wcap = y.wcap[l];
        a.stats = (int32_t*)(X + y.stats[l]);
        a.klist = (int32_t*)(X + y.klist[l]);
        a.kmask = (uint32_t*)(X + y.kmask[l]);
        a.nkept = (int32_t*)(X + y.nkept[l]);
        if (l < top) {
            a.pklist = (const int32_t*)(X + y.klist[l + 1]);
            a.pkmask = (const uint32_t*)(X + y.kmask[l + 1]);
            a.pnkept = (const int32_t*)(X + y.nkept[l + 1]);
            a.pcap = y.cap[l + 1];
            a.orph_lo = (int64_t)c * n_nodes(cfg, n_tokens, l + 1);
            a.orph_hi = n_nodes(cfg, n_tokens, l);
        } else {
            a.pklist = (const int32_t*)(X + y.noparent);
            a.pkmask = (const uint32_t*)(X + y.noparent);
            a.pnkept = (const int32_t*)(X + y.noparent);
            a.pcap = 1;
            a.orph_lo = a.orph_hi = 0;
        }
        return a;
    };

    // The chain: the first small levels, every node scored by one launch, then each
    // query head's workgroup selects them top-down.
    const int nchain = chain_levels(cfg, n_tokens, top);
    const int below = top - nchain;            // the next level to route (0: none)
    // the level below the chain, scored whole during the chain when it fits
    const int spec = (nchain > 0 && below >= 1 && y.sign[below] &&
                      spec_fits((size_t)n_nodes(cfg, n_tokens, below), R, y.H, y.G)) ? below : 0;
    if (nchain > 0) {
        ZhaChainArgs sa{};
        ZhaChainSel cs{};
        sa.n = cs.n = nchain;
        for (int i = 0; i < nchain; ++i) {
            const int l = top - i;
            sa.lv[i] = level_args(l);
            sa.blocks[i] = zha_score_blocks(n_nodes(cfg, n_tokens, l), R);
            ZhaChainLevel& cl = cs.lv[i];
            cl.sig = (const float*)(X + y.sig[l]);
            cl.kbm = (uint64_t*)(X + y.kbm[l]);
            cl.stats = (int32_t*)(X + y.stats[l]);
            cl.cap = (int32_t)y.cap[l];
            cl.n_nodes = (int32_t)n_nodes(cfg, n_tokens, l);
            cl.orph_lo = l < top ? (int32_t)(c * n_nodes(cfg, n_tokens, l + 1)) : 0;
            cl.orph_hi = l < top ? (int32_t)n_nodes(cfg, n_tokens, l) : 0;
            cl.wcap = (int32_t)y.wcap[l];
            cl.sstride = (int32_t)y.sstr[l];
        }
        cs.nsel = y.H * y.G;
        cs.q = q;
        cs.R = R;
        cs.tau = tau;
        if (spec >= 1) {
            // the level below scored whole by the chain launch's other workgroups
            ZhaLevelArgs& sp = cs.spec;
            sp = level_args(spec);
            sp.top = 1;
            sp.n_top = n_nodes(cfg, n_tokens, spec);
            sp.pklist = (const int32_t*)(X + y.noparent);
            sp.pkmask = (const uint32_t*)(X + y.noparent);
            sp.pnkept = (const int32_t*)(X + y.noparent);
            sp.pcap = 1;
            sp.orph_lo = sp.orph_hi = 0;
            sp.sig = (float*)(X + y.sign[spec]);
            // (its count as a first routed level, rewritten by the level's score kernel)
            sp.ncand = (int32_t*)(X + y.ncand[spec]);
            // workgroups of 16 waves (one item of 16 / R nodes per wave and round), at
            // most the compute units the selecting workgroups leave
            const int64_t U = R <= 16 ? 16 / R : 1;
            const int64_t items = (sp.n_top + U - 1) / U;
            cs.spec_blocks = (int)std::min<int64_t>((kSpecCUs - y.H * y.G) / y.H, (items + 15) / 16);
        }
        if ((rc = TR.mark(0, top, s))) return rc;
        hipError_t e = zha_launch_score_all(cfg->kv_dtype, q, sa, y.H, y.G, c, R, tau, s);
        if (e != hipSuccess) return hip_fail(e, "score launch (chain)");
        if ((rc = TR.mark(ZHA_TRACE_SCORE_ALL, top, s))) return rc;
        e = zha_launch_chain(cfg->kv_dtype, cs, y.H, y.G, c, cfg->top_p, s);
        if (e != hipSuccess) return hip_fail(e, "chain launch");
        if ((rc = TR.mark(ZHA_TRACE_CHAIN, top, s))) return rc;
        if (below == 0) {
            // the chain reached level 1: its group kept list for the gather
            ZhaLevelArgs a1 = level_args(1);
            a1.top = 1;
            a1.n_top = n_nodes(cfg, n_tokens, 1);
            e = zha_launch_merge_ids(a1, y.H, y.G, c, s);
            if (e != hipSuccess) return hip_fail(e, "merge launch (chain)");
            if ((rc = TR.mark(ZHA_TRACE_MERGE_IDS, 1, s))) return rc;
        }
    }
    // Every level below: score over the group's candidates, then select.  The first
    // of them derives the chain's last level's group kept list in its score kernel.
    for (int l = below; l >= 1; --l) {
        ZhaLevelArgs a = level_args(l);
        a.hblk = (float*)(X + y.hblk[l]);
        a.ghist = (uint64_t*)(X + y.ghist[l]);
        a.hdone = (uint32_t*)(X + y.hdone[l]);
        a.hcut = (void*)(X + y.hcut[l]);
        a.tick = (uint32_t*)(X + y.tick[l]);
        a.desc = (uint32_t*)(X + y.desc[l]);
        // the cross and resolve kernels, when this level may hold frontiers well past
        // the keys one workgroup stages (else a head past them is cut by the select
        // kernel over every key, which stays rare)
        if (y.glist[l] && n_nodes(cfg, n_tokens, l) > ZHA_CROSS_MIN_NODES) {
            a.pub = (uint4*)(X + y.pub[l]);
            a.gcnt = (uint4*)(X + y.gcnt[l]);
            a.gpart = (uint2*)(X + y.gpart[l]);
            a.glist = (uint2*)(X + y.glist[l]);
        }
        a.ndesc = zha_apply_chunks(y.cap[l]);
        int blocks = zha_score_blocks(n_nodes(cfg, n_tokens, l), R);
        if (l == spec) blocks = std::min(blocks, ZHA_COPY_CAP);   // copying scores: fewer workgroups
        a.score_blocks = blocks;
        ZhaLevelArgs pa{};
        const bool defer = nchain > 0 && l == below;
        if (l == spec) {
            a.sigN = (const float*)(X + y.sign[l]);
            a.nstride = y.sstr[l];
        }
        if (defer) {
            // the chain's last level: positions are node ids, per-head bitmaps over them
            pa = level_args(l + 1);
            pa.top = 1;
            pa.n_top = n_nodes(cfg, n_tokens, l + 1);
            pa.pklist = (const int32_t*)(X + y.noparent);
            pa.pkmask = (const uint32_t*)(X + y.noparent);
            pa.pnkept = (const int32_t*)(X + y.noparent);
            pa.pcap = 1;
        }
        if (nchain == 0 && l == top && (rc = TR.mark(0, l, s))) return rc;
        hipError_t e = zha_launch_route_score(cfg->kv_dtype, q, a, y.H, y.G, c, R, tau, blocks, s,
                                              defer ? &pa : nullptr);
        if (e != hipSuccess) return hip_fail(e, "route score launch");
        if ((rc = TR.mark(ZHA_TRACE_SCORE, l, s))) return rc;
        e = zha_launch_select(a, y.H, y.G, c, cfg->top_p, s);
        if (e != hipSuccess) return hip_fail(e, "route select launch");
        if ((rc = TR.mark(ZHA_TRACE_SELECT, l, s))) return rc;
        if (a.glist) {
            e = zha_launch_cross(a, y.H, y.G, c, s);
            if (e != hipSuccess) return hip_fail(e, "route cross launch");
            if ((rc = TR.mark(ZHA_TRACE_CROSS, l, s))) return rc;
            e = zha_launch_resolve(a, y.H, y.G, c, cfg->top_p, s);
            if (e != hipSuccess) return hip_fail(e, "route resolve launch");
            if ((rc = TR.mark(ZHA_TRACE_RESOLVE, l, s))) return rc;
        }
        e = zha_launch_apply(a, y.H, y.G, c, s);
        if (e != hipSuccess) return hip_fail(e, "route apply launch");
        if ((rc = TR.mark(ZHA_TRACE_APPLY, l, s))) return rc;
    }

    ZhaAttnArgs at_;
    at_.K = bufs->k;
    at_.V = bufs->v;
    at_.cap_tok = cfg->capacity;
    at_.q = q;
    // the level-1 lists are readable even when no level is routed (cap1 = 0 then
    // says they hold nothing)
    at_.klist = (const int32_t*)(X + y.klist[1]);
    at_.kmask = (const uint32_t*)(X + y.kmask[1]);
    at_.nkept = (const int32_t*)(X + y.nkept[1]);
    at_.cap1 = top >= 1 ? y.cap[1] : 0;
    at_.n_tokens = n_tokens;
    at_.pm = (float*)(X + y.pm);
    at_.pl = (float*)(X + y.pl);
    at_.po = (float*)(X + y.po);
    at_.nact = (int32_t*)(X + y.nact);
    at_.hkv = hkv;
    const int Bg = attn_blocks(n_tokens + 1, y.H, cfg->kv_dtype);
    if (top == 0 && (rc = TR.mark(0, 0, s))) return rc;
    // events 1 and 2 bracket the gather kernel's own execution
    hipError_t e = zha_launch_attention(cfg->kv_dtype, false, at_, y.H, y.G, c, tau, Bg, s,
                                        events ? static_cast<hipEvent_t>(events[1]) : nullptr,
                                        events ? static_cast<hipEvent_t>(events[2]) : nullptr);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if ((rc = TR.mark(ZHA_TRACE_GATHER, 0, s))) return rc;
    e = zha_launch_combine(at_, y.H, y.G, Bg, out, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    if ((rc = TR.mark(ZHA_TRACE_COMBINE, 0, s))) return rc;
    if ((rc = record(events, 3, s))) return rc;
    if (sel) {
        e = zha_launch_sel(at_.klist, at_.kmask, at_.nkept, at_.cap1, y.H, y.G, sel, s);
        if (e != hipSuccess) return hip_fail(e, "sel launch");
    }
    if (stats) {
        ZhaReportArgs r{};
        for (int l = 1; l <= y.L; ++l) {
            r.ncand[l - 1] = (const int32_t*)(X + y.ncand[l]);
            r.nkept[l - 1] = (const int32_t*)(X + y.nkept[l]);
            r.hstats[l - 1] = (const int32_t*)(X + y.stats[l]);
            r.routed[l - 1] = n_nodes(cfg, n_tokens, l) > 0 ? 1 : 0;
            r.all_nodes[l - 1] = (l <= top && top - l < nchain) ? n_nodes(cfg, n_tokens, l) : 0;
            r.spec_nodes[l - 1] = l == spec ? n_nodes(cfg, n_tokens, l) : 0;
            r.kbm[l - 1] = (const uint64_t*)(X + y.kbm[l]);
            r.wcap[l - 1] = (int32_t)y.wcap[l];
            r.n_nodes[l - 1] = n_nodes(cfg, n_tokens, l);
        }
        r.klist1 = at_.klist;
        r.cap1 = at_.cap1;
        r.n_tokens = n_tokens;
        // one node's summary bytes the router reads: planes s (float32, or their
        // bfloat16 copy, or their 8-bit copy and its per-plane scale) and offsets b
        r.plane_bytes = cfg->plane_format == ZHA_PLANES_FP8 ? (int64_t)R * (ZHA_D + 8)
                        : (int64_t)R * (ZHA_D * (cfg->plane_format == ZHA_PLANES_BF16 ? 2 : 4) + 4);
        r.kv_row_bytes = 2 * ZHA_D * (cfg->kv_dtype == ZHA_BF16 ? 2 : 4);
        r.H = y.H;
        r.G = y.G;
        r.c = c;
        r.levels = y.L;
        r.top = top;
        e = zha_launch_stats(r, stats, s);
        if (e != hipSuccess) return hip_fail(e, "stats launch");
    }
    return ok();
}
}  // namespace

extern "C" {

int zha_decode_step(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q, float* out,
                    int32_t* sel, zha_stats* stats, void* stream) {
    return decode_impl(cfg, bufs, n_tokens, q, out, sel, stats, nullptr, stream);
}

int zha_decode_step_timed(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q,
                          float* out, int32_t* sel, zha_stats* stats, void* const* events, void* stream) {
    return decode_impl(cfg, bufs, n_tokens, q, out, sel, stats, events, stream);
}

size_t zha_batch_scratch_bytes(const zha_config* cfg, int32_t n_queries) {
    if (validate(cfg)) return 0;
    if (n_queries < 1) {
        fail(ZHA_ERR_ARG, "n_queries must be >= 1 (got %d)", n_queries);
        return 0;
    }
    const zha_config v = virtual_config(cfg, n_queries);
    if (validate(&v)) return 0;
    return make_layout(&v).scratch_bytes;
}

int zha_decode_batch(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, int32_t n_queries,
                     const void* q, float* out, int32_t* sel, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (n_queries < 1) return fail(ZHA_ERR_ARG, "n_queries must be >= 1 (got %d)", n_queries);
    const zha_config v = virtual_config(cfg, n_queries);
    if ((rc = validate(&v))) return rc;
    return decode_impl(cfg, bufs, n_tokens, q, out, sel, nullptr, nullptr, stream, nullptr, n_queries);
}

int zha_decode_step_traced(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q,
                           float* out, void* const* events, int32_t max_events, int32_t* kinds, int32_t* n_events,
                           void* stream) {
    if (!events || max_events < 1 || !kinds || !n_events)
        return fail(ZHA_ERR_ARG, "traced step: events, kinds and n_events must be non-NULL, max_events >= 1");
    for (int32_t i = 0; i < max_events; ++i)
        if (!events[i]) return fail(ZHA_ERR_ARG, "traced step: every one of the max_events events must be non-NULL");
    Trace tr;
    tr.ev = events;
    tr.kinds = kinds;
    tr.max = max_events;
    *n_events = 0;
    const int rc = decode_impl(cfg, bufs, n_tokens, q, out, nullptr, nullptr, nullptr, stream, &tr);
    *n_events = tr.n;
    return rc;
}

size_t zha_fidelity_work_bytes(const zha_config* cfg, int64_t n_tokens) {
    if (validate(cfg) || n_tokens < 1) return 0;
    return zha_fid_work_bytes(cfg->n_q_heads, n_tokens);
}

int zha_route_fidelity(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q, float* recall,
                       void* work, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!bufs || !bufs->k || !bufs->scratch || !q || !recall || !work)
        return fail(ZHA_ERR_ARG, "buffers k and scratch and q, recall, work must be non-NULL");
    if (n_tokens < 1) return fail(ZHA_ERR_ARG, "n_tokens must be >= 1 (got %lld)", (long long)n_tokens);
    if (n_tokens > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)n_tokens,
                    (long long)cfg->capacity);
    Layout y = make_layout(cfg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* X = static_cast<char*>(bufs->scratch);
    const int top = top_level(cfg, n_tokens);
    const int below = top - chain_levels(cfg, n_tokens, top);
    // levels below the chain: their per-head bitmaps from the group kept lists
    for (int l = below; l >= 1; --l) {
        hipError_t e = zha_launch_fid_bitmap((const int32_t*)(X + y.klist[l]), (const uint32_t*)(X + y.kmask[l]),
                                             (const int32_t*)(X + y.nkept[l]), y.cap[l], (uint64_t*)(X + y.kbm[l]),
                                             y.wcap[l], y.H, y.G, s);
        if (e != hipSuccess) return hip_fail(e, "fidelity bitmap launch");
    }
    ZhaFidLevels lv{};
    lv.n = y.L;
    for (int l = 1; l <= y.L; ++l) {
        lv.kbm[l - 1] = (const uint64_t*)(X + y.kbm[l]);
        lv.wcap[l - 1] = y.wcap[l];
        lv.span[l - 1] = span_of(cfg, l);
        lv.n_nodes[l - 1] = n_nodes(cfg, n_tokens, l);
    }
    hipError_t e = zha_launch_fidelity(cfg->kv_dtype, bufs->k, q, cfg->capacity, n_tokens, y.H, y.G, tau_of(cfg), lv,
                                       work, recall, s);
    if (e != hipSuccess) return hip_fail(e, "fidelity launch");
    return ok();
}

int dense_decode(const zha_config* cfg, const void* k, const void* v, int64_t n_tokens, const void* q, float* out,
                 void* scratch, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!k || !v || !q || !out || !scratch) return fail(ZHA_ERR_ARG, "k, v, q, out and scratch must be non-NULL");
    if (n_tokens < 1) return fail(ZHA_ERR_ARG, "n_tokens must be >= 1 (got %lld)", (long long)n_tokens);
    if (n_tokens > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)n_tokens,
                    (long long)cfg->capacity);
    const int H = cfg->n_kv_heads, G = cfg->n_q_heads / cfg->n_kv_heads;
    size_t off = 0, pm, pl, po, nact;
    attn_partials(cfg, off, pm, pl, po, nact);
    char* X = static_cast<char*>(scratch);
    ZhaAttnArgs a;
    a.K = k;
    a.V = v;
    a.cap_tok = cfg->capacity;
    a.q = q;
    a.klist = nullptr;
    a.kmask = nullptr;
    a.nkept = nullptr;
    a.cap1 = 0;
    a.n_tokens = n_tokens;
    a.pm = (float*)(X + pm);
    a.pl = (float*)(X + pl);
    a.po = (float*)(X + po);
    a.nact = (int32_t*)(X + nact);
    a.hkv = cfg->n_kv_heads;
    const int Bg = attn_blocks(n_tokens, H, cfg->kv_dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = zha_launch_attention(cfg->kv_dtype, true, a, H, G, cfg->chunk, tau_of(cfg), Bg, s);
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
    e = zha_launch_combine(a, H, G, Bg, out, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

}  // extern "C"

// ---- decode without caller scratch, for callers that cannot allocate
//
// The step's scratch is a file-scope device array.  Host code never uses the
// array's name as an address: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept per device.
namespace {

static __device__ __align__(256) unsigned char scratch[ZHA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(ZHA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(ZHA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_noalloc_ptr[dev] = p;
    }
    *out = g_noalloc_ptr[dev];
    return ZHA_OK;
}

}  // namespace

extern "C" int zha_decode_step_noalloc(const zha_config* cfg, const void* k, const void* v, const void* tree,
                                       int64_t n_tokens, const void* q, float* out, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!k || !v || !tree || !q || !out) return fail(ZHA_ERR_ARG, "k, v, tree, q and out must be non-NULL");
    const size_t need = make_layout(cfg).scratch_bytes;
    if (need > (size_t)ZHA_NOALLOC_SCRATCH_BYTES)
        return fail(ZHA_ERR_UNSUPPORTED,
                    "this configuration needs %zu bytes of decode scratch, more than the %zu the no-allocation "
                    "entry point holds (use zha_decode_step with caller scratch)",
                    need, (size_t)ZHA_NOALLOC_SCRATCH_BYTES);
    void* x = nullptr;
    if ((rc = noalloc_scratch(&x))) return rc;
    zha_buffers b;
    b.k = const_cast<void*>(k);
    b.v = const_cast<void*>(v);
    b.ref_q = nullptr;
    b.tree = const_cast<void*>(tree);
    b.scratch = x;
    return decode_impl(cfg, &b, n_tokens, q, out, nullptr, nullptr, nullptr, stream);
}
