// santa_api.cpp -- the C ABI of libsanta: host-side validation, workspace
// sizing and carving, and launch sequencing.  See include/santa.h for the
// contract of every entry point.
#include "../../include/santa.h"

#include <hip/hip_runtime.h>

#include "santa_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kHeadDimBuilt = 128;
constexpr int kMaxTiles = 1024;       // reducer and merge: one thread per tile
constexpr int kMaxSamplesProp = 4096; // prop keeps the selected rows of a head in LDS
constexpr int kMaxSamples = 65536;
constexpr int kMaxDraws = 64;         // Bernoulli scoring: ternary draws per query

thread_local void *g_ev_begin = nullptr;
thread_local void *g_ev_end = nullptr;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// whether the byte ranges [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// `out` must not overlap the query or the per-head offsets: prop's pass 1
// clears output rows while other workgroups of the call still read q
bool out_aliases_inputs(const santa_problem *p, const void *q, const float *u, const float *out) {
    const size_t rows = (size_t)p->batch * p->num_q_heads;
    const size_t out_bytes = rows * p->head_dim * sizeof(float);
    const size_t q_bytes = rows * p->head_dim * (p->q_dtype == SANTA_F32 ? 4 : 2);
    return overlaps(out, out_bytes, q, q_bytes) || (u && overlaps(out, out_bytes, u, rows * sizeof(float)));
}

struct Derived {
    int group = 0;
    int max_nt = 0;
    int kmax = 0;   // prop: capacity of the per-head visit list, min(S, n_t)
};

bool tile_len_built(int T) { return T == 64 || T == 128 || T == 256 || T == 512 || T == 1024; }

// Shape/layout checks shared by every variant.  S is checked for prop/flash.
int validate(const santa_problem *p, int variant, int S, Derived *d) {
    if (!p) return SANTA_ERR_INVALID;
    if (variant < SANTA_VARIANT_PROP || variant > SANTA_VARIANT_EXACT) return SANTA_ERR_INVALID;
    if (p->batch < 0 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 ||
        p->max_seq_len < 1 || p->tile_len < 1)
        return SANTA_ERR_INVALID;
    if (p->num_q_heads % p->num_kv_heads) return SANTA_ERR_INVALID;
    if (p->tile_len % 64) return SANTA_ERR_INVALID;
    if (p->q_dtype != SANTA_F32 && p->q_dtype != SANTA_BF16) return SANTA_ERR_INVALID;
    if (p->kv_dtype != SANTA_F32 && p->kv_dtype != SANTA_BF16 && p->kv_dtype != SANTA_FP8_E4M3)
        return SANTA_ERR_INVALID;
    if (!(p->scale > 0.0f) || p->scale != p->scale) return SANTA_ERR_INVALID;
    if (p->page_size < 0) return SANTA_ERR_INVALID;
    if (p->page_size > 0) {
        if (p->page_size % 16) return SANTA_ERR_INVALID;
        if (!p->page_table) return SANTA_ERR_INVALID;
        const long need = ((long)p->max_seq_len + p->page_size - 1) / p->page_size;
        if (p->max_pages_per_seq < need) return SANTA_ERR_INVALID;
    }
    const int G = p->num_q_heads / p->num_kv_heads;
    if (p->head_dim != kHeadDimBuilt) return SANTA_ERR_UNSUPPORTED;
    // built pairs: fp32/fp32, bf16/bf16 and bf16 queries with e4m3 KV
    const bool pair_built = p->q_dtype == p->kv_dtype ||
                            (p->q_dtype == SANTA_BF16 && p->kv_dtype == SANTA_FP8_E4M3);
    if (!pair_built) return SANTA_ERR_UNSUPPORTED;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return SANTA_ERR_UNSUPPORTED;
    if (!tile_len_built(p->tile_len)) return SANTA_ERR_UNSUPPORTED;
    const long nt = ((long)p->max_seq_len + p->tile_len - 1) / p->tile_len;
    if (nt > kMaxTiles) return SANTA_ERR_UNSUPPORTED;
    if ((long)p->batch * p->num_kv_heads * nt > 0x7fffffffL) return SANTA_ERR_UNSUPPORTED;
    if ((long)p->batch * p->num_q_heads * 8 > 0x7fffffffL) return SANTA_ERR_UNSUPPORTED;
    if (variant != SANTA_VARIANT_EXACT) {
        if (S < 1 || S > kMaxSamples) return SANTA_ERR_INVALID;
    }
    if (variant == SANTA_VARIANT_PROP && S > kMaxSamplesProp) return SANTA_ERR_UNSUPPORTED;
    if (variant == SANTA_VARIANT_FLASH) {
        if (p->seq_lens) return SANTA_ERR_INVALID;
        if (S % nt) return SANTA_ERR_INVALID;
        if (S / nt > p->tile_len) return SANTA_ERR_UNSUPPORTED;   // local list lives in the tile's LDS
    }
    d->group = G;
    d->max_nt = (int)nt;
    d->kmax = (variant == SANTA_VARIANT_PROP) ? (S < nt ? S : (int)nt) : 0;
    return SANTA_OK;
}

// Workspace layout (each region 256-byte aligned).  With base == nullptr it
// only sizes.
size_t carve(const santa_problem *p, int variant, const Derived &d, char *base, santa::Workspace *ws) {
    const size_t BH = (size_t)p->batch * p->num_q_heads;
    size_t off = 0;
    auto take = [&](size_t bytes) -> void * {
        void *ptr = base ? base + off : nullptr;
        off += align_up(bytes);
        return ptr;
    };
    santa::Workspace w{};
    // every variant's layout starts with the single-launch prop's counters,
    // so that no other call ever writes over them
    w.sync = take(santa::kSyncBytes);
    if (variant == SANTA_VARIANT_PROP) {
        // every tile in full, also the short last one (aligned wide stores,
        // and whole-tile reads in pass 2)
        w.stash = take(BH * (size_t)d.max_nt * p->tile_len * sizeof(float));
        w.stats = take(BH * (size_t)d.max_nt * 2 * sizeof(float));
    } else {
        w.part_m = take(BH * (size_t)d.max_nt * sizeof(float));
        w.part_l = take(BH * (size_t)d.max_nt * sizeof(float));
        w.part_o = take(BH * (size_t)d.max_nt * kHeadDimBuilt * sizeof(float));
    }
    if (ws) *ws = w;
    return off;
}

int check_workspace(const santa_problem *p, int variant, const Derived &d, void *workspace,
                    size_t workspace_bytes, santa::Workspace *ws) {
    const size_t need = carve(p, variant, d, nullptr, nullptr);
    if (!workspace || workspace_bytes < need) return SANTA_ERR_WORKSPACE;
    if (((uintptr_t)workspace) % kAlign) return SANTA_ERR_WORKSPACE;
    carve(p, variant, d, (char *)workspace, ws);
    return SANTA_OK;
}

santa::LaunchArgs make_args(const santa_problem *p, const Derived &d, const void *q, const void *k,
                            const void *v, int S, const float *u, float *out, int *sample_idx,
                            int *tile_budget, const santa::Workspace &ws, void *stream) {
    santa::LaunchArgs a{};
    a.batch = p->batch;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.group = d.group;
    a.max_seq_len = p->max_seq_len;
    a.max_nt = d.max_nt;
    a.tile_len = p->tile_len;
    a.seq_lens = p->seq_lens;
    a.page_size = p->page_size;
    a.page_table = p->page_table;
    a.max_pages = p->max_pages_per_seq;
    a.kv_dtype = p->kv_dtype;
    a.scale = p->scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.S = S;
    a.u = u;
    a.out = out;
    a.sample_idx = sample_idx;
    a.tile_budget = tile_budget;
    a.kmax = d.kmax;
    a.ws = ws;
    a.stream = stream;
    return a;
}

int run_sampled(int variant, const santa_problem *p, const void *q, const void *k, const void *v,
                int32_t S, int32_t sampler, const float *u, float *out, int32_t *sample_idx,
                int32_t *tile_budget, void *workspace, size_t workspace_bytes, void *stream) {
    Derived d;
    int st = validate(p, variant, S, &d);
    if (st != SANTA_OK) return st;
    if (sampler != SANTA_SAMPLER_SYS && sampler != SANTA_SAMPLER_STRAT && sampler != SANTA_SAMPLER_IID)
        return SANTA_ERR_INVALID;
    if (p->batch == 0) return SANTA_OK;
    if (!q || !k || !v || !u || !out) return SANTA_ERR_INVALID;
    if (out_aliases_inputs(p, q, u, out)) return SANTA_ERR_INVALID;
    santa::Workspace ws;
    st = check_workspace(p, variant, d, workspace, workspace_bytes, &ws);
    if (st != SANTA_OK) return st;
    santa::LaunchArgs a =
        make_args(p, d, q, k, v, S, u, out, sample_idx,
                  variant == SANTA_VARIANT_PROP ? tile_budget : nullptr, ws, stream);
    a.sampler = sampler;
    const santa::TimingHook hook{g_ev_begin, g_ev_end};
    const hipError_t e = variant == SANTA_VARIANT_PROP ? santa::launch_prop(a, hook)
                                                       : santa::launch_flash(a, hook);
    return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

}  // namespace

extern "C" {

int santa_workspace_size(const santa_problem *p, int32_t variant, int32_t S, size_t *bytes) {
    if (!bytes) return SANTA_ERR_INVALID;
    Derived d;
    const int st = validate(p, variant, variant == SANTA_VARIANT_EXACT ? 1 : S, &d);
    if (st != SANTA_OK) return st;
    *bytes = carve(p, variant, d, nullptr, nullptr);
    return SANTA_OK;
}

int santa_decode_prop(const santa_problem *p, const void *q, const void *k, const void *v, int32_t S,
                      const float *u, float *out, int32_t *sample_idx, int32_t *tile_budget,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return run_sampled(SANTA_VARIANT_PROP, p, q, k, v, S, SANTA_SAMPLER_SYS, u, out, sample_idx, tile_budget,
                       workspace, workspace_bytes, stream);
}

int santa_decode_prop_fused(const santa_problem *p, const void *q, const void *k, const void *v, int32_t S,
                            const float *u, float *out, int32_t *sample_idx, int32_t *tile_budget,
                            void *workspace, size_t workspace_bytes, void *stream) {
    Derived d;
    int st = validate(p, SANTA_VARIANT_PROP, S, &d);
    if (st != SANTA_OK) return st;
    if ((long)p->batch * p->num_kv_heads > santa::kMaxSyncGroups) return SANTA_ERR_UNSUPPORTED;
    if (p->batch == 0) return SANTA_OK;
    if (!q || !k || !v || !u || !out) return SANTA_ERR_INVALID;
    if (out_aliases_inputs(p, q, u, out)) return SANTA_ERR_INVALID;
    santa::Workspace ws;
    st = check_workspace(p, SANTA_VARIANT_PROP, d, workspace, workspace_bytes, &ws);
    if (st != SANTA_OK) return st;
    santa::LaunchArgs a = make_args(p, d, q, k, v, S, u, out, sample_idx, tile_budget, ws, stream);
    a.sampler = SANTA_SAMPLER_SYS;
    const santa::TimingHook hook{g_ev_begin, g_ev_end};
    return santa::launch_prop_fused(a, hook) == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_decode_prop_sampler(const santa_problem *p, const void *q, const void *k, const void *v,
                              int32_t S, int32_t sampler, const float *u, float *out,
                              int32_t *sample_idx, int32_t *tile_budget, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return run_sampled(SANTA_VARIANT_PROP, p, q, k, v, S, sampler, u, out, sample_idx, tile_budget,
                       workspace, workspace_bytes, stream);
}

int santa_decode_flash(const santa_problem *p, const void *q, const void *k, const void *v, int32_t S,
                       const float *u, float *out, int32_t *sample_idx, int32_t *tile_budget,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return run_sampled(SANTA_VARIANT_FLASH, p, q, k, v, S, SANTA_SAMPLER_SYS, u, out, sample_idx, tile_budget,
                       workspace, workspace_bytes, stream);
}

int santa_decode_flash_sampler(const santa_problem *p, const void *q, const void *k, const void *v,
                               int32_t S, int32_t sampler, const float *u, float *out,
                               int32_t *sample_idx, int32_t *tile_budget, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return run_sampled(SANTA_VARIANT_FLASH, p, q, k, v, S, sampler, u, out, sample_idx, tile_budget,
                       workspace, workspace_bytes, stream);
}

int exact_decode_ref(const santa_problem *p, const void *q, const void *k, const void *v, float *out,
                     void *workspace, size_t workspace_bytes, void *stream) {
    Derived d;
    int st = validate(p, SANTA_VARIANT_EXACT, 1, &d);
    if (st != SANTA_OK) return st;
    if (p->batch == 0) return SANTA_OK;
    if (!q || !k || !v || !out) return SANTA_ERR_INVALID;
    if (out_aliases_inputs(p, q, nullptr, out)) return SANTA_ERR_INVALID;
    santa::Workspace ws;
    st = check_workspace(p, SANTA_VARIANT_EXACT, d, workspace, workspace_bytes, &ws);
    if (st != SANTA_OK) return st;
    const santa::LaunchArgs a = make_args(p, d, q, k, v, 0, nullptr, out, nullptr, nullptr, ws, stream);
    const santa::TimingHook hook{g_ev_begin, g_ev_end};
    return santa::launch_exact(a, hook) == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_decode_prop_bernoulli(const santa_problem *p, const void *q, const void *k_features,
                                const void *v, int32_t S, const float *u, int32_t draws,
                                int32_t group_mean, const float *u_bern, float *out,
                                int32_t *sample_idx, int32_t *tile_budget, int32_t *features_read,
                                void *workspace, size_t workspace_bytes, void *stream) {
    Derived d;
    int st = validate(p, SANTA_VARIANT_PROP, S, &d);
    if (st != SANTA_OK) return st;
    if (draws < 1 || draws > kMaxDraws || (group_mean != 0 && group_mean != 1)) return SANTA_ERR_INVALID;
    if (p->q_dtype != SANTA_BF16 || (p->kv_dtype != SANTA_BF16 && p->kv_dtype != SANTA_FP8_E4M3) ||
        p->page_size != 0 || p->max_seq_len % 4)
        return SANTA_ERR_UNSUPPORTED;
    if (p->batch == 0) return SANTA_OK;
    if (!q || !k_features || !v || !u || !u_bern || !out) return SANTA_ERR_INVALID;
    // 4 keys of a feature per lane load: 8 bytes of bf16, 4 of e4m3
    if (((uintptr_t)k_features) % (p->kv_dtype == SANTA_BF16 ? 8 : 4)) return SANTA_ERR_INVALID;
    if (out_aliases_inputs(p, q, u, out)) return SANTA_ERR_INVALID;
    santa::Workspace ws;
    st = check_workspace(p, SANTA_VARIANT_PROP, d, workspace, workspace_bytes, &ws);
    if (st != SANTA_OK) return st;
    santa::LaunchArgs a = make_args(p, d, q, k_features, v, S, u, out, sample_idx, tile_budget, ws, stream);
    a.sampler = santa::kSamplerSys;
    a.draws = draws;
    a.group_mean = group_mean;
    a.u_bern = u_bern;
    a.features_read = features_read;
    // with the mean query the group's heads share its first head's stash row
    a.stash_shift = group_mean ? (d.group == 8 ? 3 : d.group == 4 ? 2 : d.group == 2 ? 1 : 0) : 0;
    const santa::TimingHook hook{g_ev_begin, g_ev_end};
    return santa::launch_prop_bernoulli(a, hook) == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_set_timing_events(void *begin_event, void *end_event) {
    if (begin_event && end_event) {
        g_ev_begin = begin_event;
        g_ev_end = end_event;
    } else {
        g_ev_begin = nullptr;
        g_ev_end = nullptr;
    }
    return SANTA_OK;
}

const char *santa_status_string(int status) {
    switch (status) {
        case SANTA_OK: return "ok";
        case SANTA_ERR_INVALID: return "invalid argument";
        case SANTA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SANTA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case SANTA_ERR_HIP: return "HIP launch error";
        case SANTA_ERR_TOO_LARGE: return "problem needs more workspace than the static scratch holds";
        default: return "unknown status";
    }
}

int santa_abi_version(void) { return 6; }

}  // extern "C"
