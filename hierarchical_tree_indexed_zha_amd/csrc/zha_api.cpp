// C ABI of libzha.so: argument validation, tree and scratch layouts, and the
// launch sequence of each entry point.  See include/zha.h for the contract.
#include "../../include/zha.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
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
    std::vector<size_t> t_s, t_b, t_l;
    size_t tree_bytes = 0;
    // decode scratch
    std::vector<size_t> sig, kbm, klist, kmask, ncand, nkept, stats;
    std::vector<size_t> hmax, hcut, hdone, hmass, hcnt, tiem, chunk;   // sliced levels only
    std::vector<int> slices;                               // 0 when the level is not sliced
    std::vector<int64_t> wcap;            // bitmap words per head per level
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

Layout make_layout(const zha_config* cfg) {
    Layout y;
    y.L = cfg->levels;
    y.H = cfg->n_kv_heads;
    y.G = cfg->n_q_heads / cfg->n_kv_heads;
    y.R = cfg->n_ref;
    const size_t H = y.H, G = y.G, R = y.R;
    y.cap.assign(y.L + 2, 0);
    for (int l = 1; l <= y.L; ++l) y.cap[l] = n_nodes(cfg, cfg->capacity, l);
    y.t_s.assign(y.L + 1, 0); y.t_b.assign(y.L + 1, 0); y.t_l.assign(y.L + 1, 0);
    size_t off = 0;
    for (int l = 1; l <= y.L; ++l) {
        const size_t n = (size_t)y.cap[l];
        y.t_s[l] = off; off = align_up(off + sizeof(float) * H * n * R * ZHA_D);
        y.t_b[l] = off; off = align_up(off + sizeof(float) * H * n * R);
        y.t_l[l] = off; off = align_up(off + sizeof(float) * H * n * R);
    }
    y.tree_bytes = off;

    off = 0;
    for (auto* v : {&y.sig, &y.kbm, &y.klist, &y.kmask, &y.ncand, &y.nkept, &y.stats, &y.hmax, &y.hcut, &y.hdone, &y.hmass, &y.hcnt,
                    &y.tiem, &y.chunk})
        v->assign(y.L + 1, 0);
    y.slices.assign(y.L + 1, 0);
    y.wcap.assign(y.L + 1, 0);
    for (int l = 1; l <= y.L; ++l) {
        const size_t n = (size_t)y.cap[l];
        y.wcap[l] = (int64_t)((n + 63) / 64);
        y.sig[l] = off;   off = align_up(off + sizeof(float) * H * G * n);
        y.kbm[l] = off;   off = align_up(off + sizeof(uint64_t) * H * G * (size_t)y.wcap[l]);
        y.klist[l] = off; off = align_up(off + sizeof(int32_t) * H * n);
        y.kmask[l] = off; off = align_up(off + sizeof(uint32_t) * H * n);
        y.ncand[l] = off; off = align_up(off + sizeof(int32_t) * H);
        y.nkept[l] = off; off = align_up(off + sizeof(int32_t) * H);
        y.stats[l] = off; off = align_up(off + sizeof(int32_t) * 2 * H * G);
        if (n > (size_t)ZHA_SLICED_MIN_CAP) {
            // the widest levels select over slices of the whole GPU
            const size_t sl = (n + ZHA_SLICE - 1) / ZHA_SLICE;
            const size_t nch = ((size_t)y.wcap[l] + 511) / 512;
            y.slices[l] = (int)sl;
            y.hmax[l] = off;  off = align_up(off + sizeof(float) * H * G * ZHA_SCORE_MAXB);
            y.hcut[l] = off;  off = align_up(off + sizeof(HugeCut) * H * G);
            y.hdone[l] = off; off = align_up(off + sizeof(uint32_t) * 3 * H * G);
            y.hmass[l] = off; off = align_up(off + sizeof(uint64_t) * 3 * H * G * 2048);
            y.hcnt[l] = off;  off = align_up(off + sizeof(uint32_t) * 3 * H * G * 2048);
            y.tiem[l] = off;  off = align_up(off + sizeof(uint64_t) * H * G * sl);
            y.chunk[l] = off; off = align_up(off + sizeof(uint32_t) * H * nch);
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

// Attention workgroups per KV group: about 8 tiles of 32 slots each, at most one
// resident round of the whole device (768 workgroups: 256 CUs x 3 resident) so
// that no partial second round trails the launch.
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

int zha_tree_level_offsets(const zha_config* cfg, int32_t level, int64_t* s_off, int64_t* b_off, int64_t* lse_off,
                           int64_t* n_cap) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (level < 1 || level > cfg->levels) return fail(ZHA_ERR_ARG, "level %d outside 1..%d", level, cfg->levels);
    Layout y = make_layout(cfg);
    if (s_off) *s_off = (int64_t)y.t_s[level];
    if (b_off) *b_off = (int64_t)y.t_b[level];
    if (lse_off) *lse_off = (int64_t)y.t_l[level];
    if (n_cap) *n_cap = y.cap[level];
    return ok();
}

int zha_route_level_offsets(const zha_config* cfg, int32_t level, zha_route_offsets* out) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(ZHA_ERR_ARG, "out is NULL");
    if (level < 1 || level > cfg->levels) return fail(ZHA_ERR_ARG, "level %d outside 1..%d", level, cfg->levels);
    Layout y = make_layout(cfg);
    out->n_cand = (int64_t)y.ncand[level];
    out->sigma = (int64_t)y.sig[level];
    out->n_kept = (int64_t)y.nkept[level];
    out->kept = (int64_t)y.klist[level];
    out->mask = (int64_t)y.kmask[level];
    out->stats = (int64_t)y.stats[level];
    out->n_cap = y.cap[level];
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
    hipError_t e = zha_launch_leaf_summary(
        cfg->kv_dtype, bufs->k, bufs->ref_q, (float*)at(T, y.t_s[1]), (float*)at(T, y.t_b[1]), (float*)at(T, y.t_l[1]),
        y.H, cfg->capacity, y.cap[1], c, R, 0, n_nodes(cfg, n_tokens, 1), tau_of(cfg), s);
    if (e != hipSuccess) return hip_fail(e, "leaf summary launch");
    for (int l = 2; l <= y.L; ++l) {
        const int64_t n = n_nodes(cfg, n_tokens, l);
        if (n == 0) break;
        e = zha_launch_merge((float*)at(T, y.t_s[l - 1]), (float*)at(T, y.t_b[l - 1]), (float*)at(T, y.t_l[l - 1]),
                             (float*)at(T, y.t_s[l]), (float*)at(T, y.t_b[l]), (float*)at(T, y.t_l[l]), y.H,
                             y.cap[l - 1], y.cap[l], c, R, 0, n, s);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
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
                                tau_of(cfg), s);
    if (e != hipSuccess) return hip_fail(e, "leaf summary launch");
    for (int l = 2; l <= y.L; ++l) {
        const int64_t span = span_of(cfg, l);
        if (span > cfg->capacity || n % span != 0) break;
        e = zha_launch_merge((float*)at(T, y.t_s[l - 1]), (float*)at(T, y.t_b[l - 1]), (float*)at(T, y.t_l[l - 1]),
                             (float*)at(T, y.t_s[l]), (float*)at(T, y.t_b[l]), (float*)at(T, y.t_l[l]), y.H,
                             y.cap[l - 1], y.cap[l], c, R, n / span - 1, 1, s);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
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

int decode_impl(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q, float* out,
                void* const* events, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!bufs || !bufs->k || !bufs->v || !bufs->tree || !bufs->scratch || !q || !out)
        return fail(ZHA_ERR_ARG, "buffers k, v, tree, scratch and q, out must be non-NULL");
    if (n_tokens < 1) return fail(ZHA_ERR_ARG, "n_tokens must be >= 1 (got %lld)", (long long)n_tokens);
    if (n_tokens > cfg->capacity)
        return fail(ZHA_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)n_tokens,
                    (long long)cfg->capacity);
    Layout y = make_layout(cfg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int c = cfg->chunk, R = cfg->n_ref;
    const float tau = tau_of(cfg);
    char* T = static_cast<char*>(bufs->tree);
    char* X = static_cast<char*>(bufs->scratch);

    int top = 0;
    for (int l = y.L; l >= 1; --l)
        if (n_nodes(cfg, n_tokens, l) > 0) { top = l; break; }
    if ((rc = record(events, 0, s))) return rc;

    // The first routed levels, while small, form one chain: all their nodes scored
    // in one launch, then selected level after level by one workgroup per group.
    int nchain = 0;
    {
        int64_t planes = 0;
        for (int l = top; l >= 1 && nchain < ZHA_MAX_CHAIN; --l) {
            if (y.cap[l] > ZHA_SMALL_SLOTS || y.slices[l]) break;
            planes += n_nodes(cfg, n_tokens, l) * (int64_t)R;
            if (planes > ZHA_CHAIN_PLANES) break;
            ++nchain;
        }
        if (nchain < 2) nchain = 0;   // a lone small level gains nothing
    }
    ZhaChainArgs chain;
    chain.n = nchain;
    // a large level above a routed one may leave its merge to the level below's
    // score kernel
    ZhaLevelArgs above;
    bool defer_above = false;
    for (int l = top; l >= 1; --l) {
        ZhaLevelArgs a;
        a.S = (const float*)(T + y.t_s[l]);
        a.B = (const float*)(T + y.t_b[l]);
        a.cap = y.cap[l];
        a.top = l == top ? 1 : 0;
        a.n_top = n_nodes(cfg, n_tokens, l);
        a.dc = zha_make_div((uint32_t)c);
        a.ncand = (int32_t*)(X + y.ncand[l]);
        a.sig = (float*)(X + y.sig[l]);
        a.kbm = (uint64_t*)(X + y.kbm[l]);
        a.wcap = y.wcap[l];
        a.stats = (int32_t*)(X + y.stats[l]);
        a.klist = (int32_t*)(X + y.klist[l]);
        a.kmask = (uint32_t*)(X + y.kmask[l]);
        a.nkept = (int32_t*)(X + y.nkept[l]);
        if (y.slices[l]) {
            a.hblk = (float*)(X + y.hmax[l]);
            a.hstate = (HugeCut*)(X + y.hcut[l]);
            a.hdone = (uint32_t*)(X + y.hdone[l]);
            a.hmass = (uint64_t*)(X + y.hmass[l]);
            a.hcnt = (uint32_t*)(X + y.hcnt[l]);
            a.tiem = (uint64_t*)(X + y.tiem[l]);
            a.chunk_cnt = (uint32_t*)(X + y.chunk[l]);
            a.slices = y.slices[l];
        } else {
            a.hblk = nullptr;
            a.hstate = nullptr;
            a.hdone = nullptr;
            a.hmass = nullptr;
            a.hcnt = nullptr;
            a.tiem = nullptr;
            a.chunk_cnt = nullptr;
            a.slices = 0;
        }
        if (l < top) {
            a.pklist = (const int32_t*)(X + y.klist[l + 1]);
            a.pkmask = (const uint32_t*)(X + y.kmask[l + 1]);
            a.pnkept = (const int32_t*)(X + y.nkept[l + 1]);
            a.pcap = y.cap[l + 1];
            a.orph_lo = (int64_t)c * n_nodes(cfg, n_tokens, l + 1);
            a.orph_hi = n_nodes(cfg, n_tokens, l);
        } else {
            // the first routed level has no parents: the parent arrays point at a
            // small scratch region that no kernel writes (their values go unused), so
            // that a kernel may issue its parent reads before it knows whether the
            // level is the first
            a.pklist = (const int32_t*)(X + y.noparent);
            a.pkmask = (const uint32_t*)(X + y.noparent);
            a.pnkept = (const int32_t*)(X + y.noparent);
            a.pcap = 1;
            a.orph_lo = a.orph_hi = 0;
        }
        const int blocks = zha_score_blocks(n_nodes(cfg, n_tokens, l), R);
        a.score_blocks = blocks;
        if (top - l < nchain) {
            chain.lv[top - l] = a;
            chain.blocks[top - l] = blocks;
            if (top - l == nchain - 1) {
                hipError_t e = zha_launch_route_chain(cfg->kv_dtype, q, chain, y.H, y.G, c, R, tau, cfg->top_p, s);
                if (e != hipSuccess) return hip_fail(e, "route chain launch");
            }
            continue;
        }
        const bool defer = l >= 2 && y.cap[l] > ZHA_SMALL_SLOTS && !y.slices[l] &&
                           zha_defer_fits(y.G, y.wcap[l], a.top ? 0 : a.pcap);
        hipError_t e = zha_launch_route_score(cfg->kv_dtype, q, a, y.H, y.G, c, R, tau, blocks, s,
                                              defer_above ? &above : nullptr);
        if (e != hipSuccess) return hip_fail(e, "route score launch");
        e = zha_launch_route_select(a, y.H, y.G, c, cfg->top_p, s, !defer);
        if (e != hipSuccess) return hip_fail(e, "route select launch");
        above = a;
        defer_above = defer;
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
    const int Bg = attn_blocks(n_tokens + 1, y.H, cfg->kv_dtype);
    // events 1 and 2 bracket the gather kernel's own execution
    hipError_t e = zha_launch_attention(cfg->kv_dtype, false, at_, y.H, y.G, c, tau, Bg, s,
                                        events ? static_cast<hipEvent_t>(events[1]) : nullptr,
                                        events ? static_cast<hipEvent_t>(events[2]) : nullptr);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    e = zha_launch_combine(at_, y.H, y.G, Bg, out, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    if ((rc = record(events, 3, s))) return rc;
    return ok();
}
}  // namespace

extern "C" {

int zha_decode_step(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q, float* out,
                    void* stream) {
    return decode_impl(cfg, bufs, n_tokens, q, out, nullptr, stream);
}

int zha_decode_step_timed(const zha_config* cfg, const zha_buffers* bufs, int64_t n_tokens, const void* q,
                          float* out, void* const* events, void* stream) {
    return decode_impl(cfg, bufs, n_tokens, q, out, events, stream);
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
    const int Bg = attn_blocks(n_tokens, H, cfg->kv_dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = zha_launch_attention(cfg->kv_dtype, true, a, H, G, cfg->chunk, tau_of(cfg), Bg, s);
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
    e = zha_launch_combine(a, H, G, Bg, out, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

}  // extern "C"
