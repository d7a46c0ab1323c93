// The C ABI (include/mbert.h): argument validation, workspace layout, layer sequencing,
// HIP graph capture and per-kernel timing. Host code only; every step of the forward runs
// in the kernels of k_meta / k_norm / k_gemm / k_attn.
#include <algorithm>
#include <climits>
#include <mutex>
#include <new>
#include <vector>

#include "common.hpp"

using namespace mb;

namespace {

constexpr int kVersion = 100;  // 1.00

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_dtype(mbert_dtype dt) {
    return (dt == MBERT_F32 || dt == MBERT_BF16 || dt == MBERT_F16) ? MBERT_OK : MBERT_EUNSUPPORTED;
}
size_t dsize(mbert_dtype dt) { return dt == MBERT_F32 ? 4 : (dt == MBERT_BF16 || dt == MBERT_F16) ? 2 : 0; }

int check_cfg(const mbert_config* c) {
    if (!c) return MBERT_EINVAL;
    if (c->hidden != D || c->n_heads != NH || c->head_dim != HD || c->intermediate != FF)
        return MBERT_EUNSUPPORTED;
    if (c->n_layers < 1 || c->n_layers > 4096 || c->vocab < 1 || c->global_every < 1)
        return MBERT_EINVAL;
    if (c->half_window < 0 || c->half_window > 65536) return MBERT_EINVAL;
    if (c->max_positions < 1 || c->max_positions > (1 << 20)) return MBERT_ERANGE;
    if (!(c->theta_global > 0.0) || !(c->theta_local > 0.0) || !(c->norm_eps >= 0.0f))
        return MBERT_EINVAL;
    return MBERT_OK;
}

// Rows are addressed with 32-bit products of row and 2304 columns in places; keep totals small
// enough that every element offset fits comfortably in size_t and every count in int.
constexpr long kMaxRows = (long)INT_MAX / QKV;

int check_sizes(int total, int n_seqs) {
    if (total < 0 || n_seqs < 0) return MBERT_EINVAL;
    if (total > kMaxRows) return MBERT_ERANGE;
    return MBERT_OK;
}

int check_weights(const mbert_weights* w) {
    if (!w) return MBERT_EINVAL;
    int rc = check_cfg(&w->cfg);
    if (rc) return rc;
    if ((rc = check_dtype(w->dtype))) return rc;
    if (!w->tok_emb || !w->emb_norm || !w->final_norm || !w->layers || !w->rope) return MBERT_EINVAL;
    for (int l = 0; l < w->cfg.n_layers; ++l) {
        const mbert_layer_weights& L = w->layers[l];
        if (!L.Wqkv || !L.attn_Wo || !L.mlp_norm || !L.Wi || !L.mlp_Wo) return MBERT_EINVAL;
        if ((l == 0) != (L.attn_norm == nullptr)) return MBERT_EINVAL;  // identity on layer 0 only
    }
    return MBERT_OK;
}

mbert_ws_layout make_layout(mbert_dtype dt, int total_max, int n_seqs) {
    mbert_ws_layout L{};
    const size_t T = (size_t)total_max;
    const size_t ds = dsize(dt);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.resid = take(T * D * 4);
    L.h = take(T * D * ds);
    L.qkv = take(T * QKV * ds);
    L.meta = take(meta_ints(total_max, n_seqs) * 4);
    L.partials = take(tiles_max_for(total_max, n_seqs) * FPARTS * D * 4);
    L.ids = take(T * 4);
    L.indices = take(T * 4);
    L.rowmap = take(T * 4);
    L.cu = take(((size_t)n_seqs + 1) * 4);
    L.xs = take(T * D * ds);
    L.rstats = take(T * 12 * 8);
    L.total_bytes = off;
    return L;
}

// ---------------------------------------------------------------- per-kernel timing
struct Recorder {
    mbert_timer* t = nullptr;
    int kind = -1;
};

}  // namespace

struct mbert_timer {
    std::vector<hipEvent_t> ev;  // 2 per launch
    int used = 0;                // launches recorded since the last reset
};

struct mbert_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace mb {
LaunchEvents& launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}
}  // namespace mb

namespace {

// Arm the thread's launch events with the next slot of the timer (see MB_LAUNCH); a step that
// launched nothing records both events back to back.
inline void rec_begin(Recorder* r, int kind, hipStream_t) {
    if (r && r->t && r->kind == kind && 2 * r->t->used + 1 < (int)r->t->ev.size()) {
        mb::LaunchEvents& ev = mb::launch_events();
        ev.start = r->t->ev[2 * r->t->used];
        ev.stop = r->t->ev[2 * r->t->used + 1];
    }
}
inline void rec_end(Recorder* r, int kind, hipStream_t s) {
    if (r && r->t && r->kind == kind && 2 * r->t->used + 1 < (int)r->t->ev.size()) {
        mb::LaunchEvents& ev = mb::launch_events();
        if (ev.start != nullptr) {
            (void)hipEventRecord(ev.start, s);
            (void)hipEventRecord(ev.stop, s);
        }
        ev = mb::LaunchEvents{};
        r->t->used++;
    }
}

#define MB_TRY(expr)                  \
    do {                              \
        const int _rc = (expr);       \
        if (_rc != MBERT_OK) return _rc; \
    } while (0)

#define MB_TIMED(rec, kind, s, expr)  \
    do {                              \
        rec_begin(rec, kind, s);      \
        const int _rc = (expr);       \
        rec_end(rec, kind, s);        \
        if (_rc != MBERT_OK) return _rc; \
    } while (0)

// Folded weights of one layer: {Wqkv o attn_norm, c, Wi o mlp_norm, c}, 256-byte aligned.
struct FoldLayout {
    size_t wq, cq, wi, ci, stride;
};
FoldLayout fold_layout(mbert_dtype dt) {
    FoldLayout f{};
    const size_t wbytes = align256((size_t)QKV * D * dsize(dt)), cbytes = align256((size_t)QKV * 4);
    f.wq = 0;
    f.cq = wbytes;
    f.wi = wbytes + cbytes;
    f.ci = 2 * wbytes + cbytes;
    f.stride = 2 * (wbytes + cbytes);
    return f;
}
bool use_fold(const mbert_weights* w) { return w->folded != nullptr; }

// One layer with the pre-norm LayerNorms folded into the QKV and Wi GEMMs: the residual
// GEMMs leave the residual rounded to dtype (xs; for fp32 the residual itself) and its chunk
// statistics, which the next GEMM normalises in its epilogue. Layer 0's QKV reads the
// embedding norm output (no attention norm there); the last MLP residual feeds the final norm.
int run_layer_folded(const mbert_weights* w, int layer, int total, int n_seqs, char* ws,
                     const mbert_ws_layout& L, hipStream_t s, Recorder* rec, bool host_rows) {
    const mbert_config& c = w->cfg;
    const mbert_layer_weights& lw = w->layers[layer];
    const mbert_dtype dt = w->dtype;
    const int32_t* meta = reinterpret_cast<const int32_t*>(ws + L.meta);
    float* resid = reinterpret_cast<float*>(ws + L.resid);
    void* h = ws + L.h;
    void* qkv = ws + L.qkv;
    void* xs = dt == MBERT_F32 ? nullptr : ws + L.xs;
    const void* xa = dt == MBERT_F32 ? static_cast<const void*>(resid) : xs;  // raw residual
    float2* st = reinterpret_cast<float2*>(ws + L.rstats);
    const FoldLayout F = fold_layout(dt);
    const char* fb = static_cast<const char*>(w->folded) + (size_t)layer * F.stride;
    const bool glob = (layer % c.global_every) == 0;
    if (layer == 0) {
        MB_TIMED(rec, MBERT_K_QKV_ROPE, s,
                 mbh::launch_qkv(dt, h, total, meta, lw.Wqkv, w->rope, c.max_positions, glob ? 0 : 1,
                                 1, qkv, s, nullptr, host_rows));
    } else {
        const mbh::FoldArgs fa{reinterpret_cast<const float*>(fb + F.cq), st, c.norm_eps};
        MB_TIMED(rec, MBERT_K_QKV_ROPE, s,
                 mbh::launch_qkv(dt, xa, total, meta, fb + F.wq, w->rope, c.max_positions,
                                 glob ? 0 : 1, 1, qkv, s, &fa, host_rows));
    }
    MB_TIMED(rec, glob ? MBERT_K_ATTN_GLOBAL : MBERT_K_ATTN_LOCAL, s,
             mbh::launch_attention(dt, qkv, total, meta, n_seqs, glob ? 1 : 0, c.half_window, h, s));
    MB_TIMED(rec, MBERT_K_WO_RESID, s,
             mbh::launch_linear_residual(dt, h, D, total, meta, lw.attn_Wo, resid, s, xs, st,
                                         host_rows));
    const mbh::FoldArgs fm{reinterpret_cast<const float*>(fb + F.ci), st, c.norm_eps};
    MB_TIMED(rec, MBERT_K_WI_GEGLU, s,
             mbh::launch_geglu(dt, xa, total, meta, fb + F.wi, qkv, s, &fm, host_rows));
    const bool last = layer + 1 == c.n_layers;
    MB_TIMED(rec, MBERT_K_WO2_RESID, s,
             mbh::launch_linear_residual(dt, qkv, FF, total, meta, lw.mlp_Wo, resid, s,
                                         last ? nullptr : xs, last ? nullptr : st, host_rows));
    return MBERT_OK;
}

// host_rows: total is the exact row count (a packed batch), so the GEMMs need not load it.
int run_layer(const mbert_weights* w, int layer, int total, int n_seqs, char* ws,
              const mbert_ws_layout& L, hipStream_t s, Recorder* rec, bool fold = false,
              bool host_rows = false) {
    if (fold) return run_layer_folded(w, layer, total, n_seqs, ws, L, s, rec, host_rows);
    const mbert_config& c = w->cfg;
    const mbert_layer_weights& lw = w->layers[layer];
    const mbert_dtype dt = w->dtype;
    const int32_t* meta = reinterpret_cast<const int32_t*>(ws + L.meta);
    float* resid = reinterpret_cast<float*>(ws + L.resid);
    void* h = ws + L.h;
    void* qkv = ws + L.qkv;
    const bool glob = (layer % c.global_every) == 0;
    if (layer > 0)
        MB_TIMED(rec, MBERT_K_LAYERNORM, s,
                 mbh::launch_layernorm(dt, resid, total, meta, lw.attn_norm, c.norm_eps, h, s));
    MB_TIMED(rec, MBERT_K_QKV_ROPE, s,
             mbh::launch_qkv(dt, h, total, meta, lw.Wqkv, w->rope, c.max_positions, glob ? 0 : 1, 1,
                             qkv, s, nullptr, host_rows));
    MB_TIMED(rec, glob ? MBERT_K_ATTN_GLOBAL : MBERT_K_ATTN_LOCAL, s,
             mbh::launch_attention(dt, qkv, total, meta, n_seqs, glob ? 1 : 0, c.half_window, h, s));
    MB_TIMED(rec, MBERT_K_WO_RESID, s,
             mbh::launch_linear_residual(dt, h, D, total, meta, lw.attn_Wo, resid, s, nullptr,
                                         nullptr, host_rows));
    MB_TIMED(rec, MBERT_K_LAYERNORM, s,
             mbh::launch_layernorm(dt, resid, total, meta, lw.mlp_norm, c.norm_eps, h, s));
    MB_TIMED(rec, MBERT_K_WI_GEGLU, s,
             mbh::launch_geglu(dt, h, total, meta, lw.Wi, qkv, s, nullptr, host_rows));
    MB_TIMED(rec, MBERT_K_WO2_RESID, s,
             mbh::launch_linear_residual(dt, qkv, FF, total, meta, lw.mlp_Wo, resid, s, nullptr,
                                         nullptr, host_rows));
    return MBERT_OK;
}

int encode_impl(const mbert_weights* w, const int32_t* ids, const int32_t* cu, int n_seqs,
                int total, void* ws, size_t ws_bytes, float* out, float* pooled, hipStream_t s,
                Recorder* rec) {
    MB_TRY(check_weights(w));
    MB_TRY(check_sizes(total, n_seqs));
    if (!ws || !out || !ids || !cu) return MBERT_EINVAL;
    const mbert_ws_layout L = make_layout(w->dtype, total, n_seqs);
    if (ws_bytes < L.total_bytes) return MBERT_ENOSPC;
    char* base = static_cast<char*>(ws);
    int32_t* meta = reinterpret_cast<int32_t*>(base + L.meta);
    float* resid = reinterpret_cast<float*>(base + L.resid);
    MB_TIMED(rec, MBERT_K_META, s,
             mbh::launch_pack_meta(cu, n_seqs, total, w->cfg.max_positions, meta, s));
    if (total == 0) {
        if (pooled && n_seqs > 0)
            MB_TRY(mbh::launch_final_ln_pool(resid, 0, meta, n_seqs, w->dtype, w->final_norm,
                                             w->cfg.norm_eps, out, pooled,
                                             reinterpret_cast<float*>(base + L.partials), s));
        return MBERT_OK;
    }
    MB_TIMED(rec, MBERT_K_EMBED_LN, s,
             mbh::launch_embed_ln(w->dtype, ids, total, meta, w->tok_emb, w->cfg.vocab,
                                  w->emb_norm, w->cfg.norm_eps, resid, base + L.h, s));
    for (int l = 0; l < w->cfg.n_layers; ++l)
        MB_TRY(run_layer(w, l, total, n_seqs, base, L, s, rec, use_fold(w), true));
    MB_TIMED(rec, MBERT_K_FINAL_POOL, s,
             mbh::launch_final_ln_pool(resid, total, meta, n_seqs, w->dtype, w->final_norm,
                                       w->cfg.norm_eps, out, pooled,
                                       reinterpret_cast<float*>(base + L.partials), s));
    return MBERT_OK;
}

// The padded batch run as is, every row at its full width (the non-unpadded path): keys are
// each row's real tokens, pad rows are computed and then zeroed, pooling covers real tokens.
int encode_padded_keymask_impl(const mbert_weights* w, const int32_t* ids_pad,
                               const int32_t* mask, int B, int Tpad, void* ws, size_t ws_bytes,
                               float* out_pad, float* pooled, hipStream_t s) {
    MB_TRY(check_weights(w));
    if (B < 0 || Tpad < 0) return MBERT_EINVAL;
    if ((long)B * (long)Tpad > kMaxRows) return MBERT_ERANGE;
    if (!ws || !out_pad || !ids_pad || !mask) return MBERT_EINVAL;
    const int total_max = B * Tpad;
    const mbert_ws_layout L = make_layout(w->dtype, total_max, B);
    if (ws_bytes < L.total_bytes) return MBERT_ENOSPC;
    char* base = static_cast<char*>(ws);
    int32_t* meta = reinterpret_cast<int32_t*>(base + L.meta);
    float* resid = reinterpret_cast<float*>(base + L.resid);
    MB_TRY(mbh::launch_padded_meta(mask, B, Tpad, w->cfg.max_positions, meta, s));
    if (total_max > 0) {
        MB_TRY(mbh::launch_embed_ln(w->dtype, ids_pad, total_max, meta, w->tok_emb, w->cfg.vocab,
                                    w->emb_norm, w->cfg.norm_eps, resid, base + L.h, s));
        for (int l = 0; l < w->cfg.n_layers; ++l)
            MB_TRY(run_layer(w, l, total_max, B, base, L, s, nullptr, use_fold(w)));
    }
    return mbh::launch_final_ln_pool(resid, total_max, meta, B, w->dtype, w->final_norm,
                                     w->cfg.norm_eps, out_pad, pooled,
                                     reinterpret_cast<float*>(base + L.partials), s);
}

int encode_padded_impl(const mbert_weights* w, const int32_t* ids_pad, const int32_t* mask, int B,
                       int Tpad, void* ws, size_t ws_bytes, float* out_pad, float* pooled,
                       hipStream_t s, Recorder* rec) {
    MB_TRY(check_weights(w));
    if (B < 0 || Tpad < 0) return MBERT_EINVAL;
    if ((long)B * (long)Tpad > kMaxRows) return MBERT_ERANGE;
    if (!ws || !out_pad || !ids_pad || !mask) return MBERT_EINVAL;
    const int total_max = B * Tpad;
    const mbert_ws_layout L = make_layout(w->dtype, total_max, B);
    if (ws_bytes < L.total_bytes) return MBERT_ENOSPC;
    char* base = static_cast<char*>(ws);
    int32_t* meta = reinterpret_cast<int32_t*>(base + L.meta);
    int32_t* ids = reinterpret_cast<int32_t*>(base + L.ids);
    float* resid = reinterpret_cast<float*>(base + L.resid);
    MB_TIMED(rec, MBERT_K_META, s,
             mbh::launch_unpad(ids_pad, mask, B, Tpad, w->cfg.max_positions, ids,
                               reinterpret_cast<int32_t*>(base + L.indices),
                               reinterpret_cast<int32_t*>(base + L.rowmap),
                               reinterpret_cast<int32_t*>(base + L.cu), meta, s));
    if (total_max > 0) {
        MB_TIMED(rec, MBERT_K_EMBED_LN, s,
                 mbh::launch_embed_ln(w->dtype, ids, total_max, meta, w->tok_emb, w->cfg.vocab,
                                      w->emb_norm, w->cfg.norm_eps, resid, base + L.h, s));
        for (int l = 0; l < w->cfg.n_layers; ++l)
            MB_TRY(run_layer(w, l, total_max, B, base, L, s, rec, use_fold(w)));
    }
    // the final norm writes the padded output directly (rows by their slot; pads zeroed)
    MB_TIMED(rec, MBERT_K_FINAL_POOL, s,
             mbh::launch_final_ln_pool(resid, total_max, meta, B, w->dtype, w->final_norm,
                                       w->cfg.norm_eps, out_pad, pooled,
                                       reinterpret_cast<float*>(base + L.partials), s,
                                       reinterpret_cast<int32_t*>(base + L.indices),
                                       reinterpret_cast<int32_t*>(base + L.rowmap), total_max));
    return MBERT_OK;
}

// A padded batch split into groups of consecutive rows (whole sequences), each group's whole
// forward on its own stream, forked from and joined back into `s` with events. Rows never
// interact across sequences, so every output row is computed exactly as in one forward; the
// groups' kernels overlap, which fills the GPU when one batch's kernels are latency-bound.
struct GroupSplit {
    int groups, per;  // number of groups, batch rows per group (the last may hold fewer)
};
GroupSplit group_split(int B, int n_groups) {
    GroupSplit g{1, B};
    if (n_groups <= 1 || B <= 1) return g;
    g.per = (B + n_groups - 1) / n_groups;
    g.groups = (B + g.per - 1) / g.per;
    return g;
}

int encode_padded_grouped_impl(const mbert_weights* w, const int32_t* ids_pad,
                               const int32_t* mask, int B, int Tpad, int n_groups, void* ws,
                               size_t ws_bytes, float* out_pad, float* pooled,
                               const hipStream_t* extra, hipStream_t s) {
    MB_TRY(check_weights(w));
    if (B < 0 || Tpad < 0 || n_groups < 1) return MBERT_EINVAL;
    if ((long)B * (long)Tpad > kMaxRows) return MBERT_ERANGE;
    const GroupSplit g = group_split(B, n_groups);
    if (g.groups == 1)
        return encode_padded_impl(w, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled, s,
                                  nullptr);
    if (!ws || !out_pad || !ids_pad || !mask || !extra) return MBERT_EINVAL;
    for (int i = 0; i < g.groups - 1; ++i)
        if (extra[i] == nullptr || extra[i] == s) return MBERT_EINVAL;
    const size_t per_ws = make_layout(w->dtype, g.per * Tpad, g.per).total_bytes;
    if (ws_bytes < per_ws * (size_t)g.groups) return MBERT_ENOSPC;
    std::vector<hipEvent_t> ev(g.groups, nullptr);  // ev[0]: fork; ev[i]: join of group i
    for (auto& e : ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            for (auto& f : ev)
                if (f) (void)hipEventDestroy(f);
            return MBERT_EHIP;
        }
    int rc = hipEventRecord(ev[0], s) == hipSuccess ? MBERT_OK : MBERT_EHIP;
    for (int i = 1; i < g.groups && rc == MBERT_OK; ++i)
        if (hipStreamWaitEvent(extra[i - 1], ev[0], 0) != hipSuccess) rc = MBERT_EHIP;
    for (int i = 0; i < g.groups && rc == MBERT_OK; ++i) {
        const int b0 = i * g.per, nb = std::min(g.per, B - b0);
        const size_t r0 = (size_t)b0 * Tpad;
        rc = encode_padded_impl(w, ids_pad + r0, mask + r0, nb, Tpad,
                                static_cast<char*>(ws) + per_ws * i, per_ws, out_pad + r0 * D,
                                pooled ? pooled + (size_t)b0 * D : nullptr,
                                i == 0 ? s : extra[i - 1], nullptr);
    }
    // join every forked stream back, also after an error (a capture must end joined)
    for (int i = 1; i < g.groups; ++i) {
        (void)hipEventRecord(ev[i], extra[i - 1]);
        (void)hipStreamWaitEvent(s, ev[i], 0);
    }
    for (auto& e : ev) (void)hipEventDestroy(e);
    return rc;
}


}  // namespace

extern "C" {

int mbert_version(void) { return kVersion; }

const char* mbert_strerror(int code) {
    switch (code) {
        case MBERT_OK: return "ok";
        case MBERT_EINVAL: return "invalid argument";
        case MBERT_EUNSUPPORTED: return "unsupported dims or dtype";
        case MBERT_ERANGE: return "size out of range";
        case MBERT_ENOSPC: return "workspace too small";
        case MBERT_EHIP: return "HIP launch or runtime error";
        default: return "unknown error";
    }
}

int mbert_default_config(mbert_config* c) {
    if (!c) return MBERT_EINVAL;
    c->n_layers = 22;
    c->hidden = D;
    c->n_heads = NH;
    c->head_dim = HD;
    c->intermediate = FF;
    c->vocab = 50368;
    c->global_every = 3;
    c->half_window = 64;
    c->max_positions = 8192;
    c->theta_global = 160000.0;
    c->theta_local = 10000.0;
    c->norm_eps = 1e-5f;
    return MBERT_OK;
}

int mbert_check_config(const mbert_config* c) { return check_cfg(c); }
int mbert_tile_tokens(void) { return TILE; }
size_t mbert_meta_ints(int total_max, int n_seqs) {
    if (total_max < 0 || n_seqs < 0) return 0;
    return meta_ints(total_max, n_seqs);
}
size_t mbert_dtype_size(mbert_dtype dt) { return dsize(dt); }

size_t mbert_rope_table_floats(const mbert_config* c) {
    if (check_cfg(c)) return 0;
    return (size_t)2 * c->max_positions * (HD / 2) * 2;
}

int mbert_build_rope_tables(const mbert_config* c, float* table, void* stream) {
    MB_TRY(check_cfg(c));
    if (!table) return MBERT_EINVAL;
    return mbh::launch_rope_tables(table, c->max_positions, c->theta_global, c->theta_local,
                                   as_stream(stream));
}

int mbert_pack_meta(const int32_t* cu, int n_seqs, int total, int max_positions, int32_t* meta,
                    void* stream) {
    MB_TRY(check_sizes(total, n_seqs));
    if (!cu || !meta || max_positions < 1) return MBERT_EINVAL;
    return mbh::launch_pack_meta(cu, n_seqs, total, max_positions, meta, as_stream(stream));
}

int mbert_unpad(const int32_t* ids_pad, const int32_t* mask, int B, int Tpad, int max_positions,
                int32_t* ids, int32_t* indices, int32_t* rowmap, int32_t* cu, int32_t* meta,
                void* stream) {
    if (B < 0 || Tpad < 0 || max_positions < 1) return MBERT_EINVAL;
    if ((long)B * Tpad > kMaxRows) return MBERT_ERANGE;
    if (!cu || !meta) return MBERT_EINVAL;
    if ((long)B * Tpad > 0 && (!ids_pad || !mask || !ids || !indices || !rowmap)) return MBERT_EINVAL;
    return mbh::launch_unpad(ids_pad, mask, B, Tpad, max_positions, ids, indices, rowmap, cu, meta,
                             as_stream(stream));
}

int mbert_attn_key_ranges(const int32_t* meta, int total_max, int n_seqs, int is_global,
                          int half_window, int32_t* lo, int32_t* hi, void* stream) {
    MB_TRY(check_sizes(total_max, n_seqs));
    if (!meta || !lo || !hi || half_window < 0) return MBERT_EINVAL;
    return mbh::launch_key_ranges(meta, total_max, n_seqs, is_global ? 1 : 0, half_window, lo, hi,
                                  as_stream(stream));
}

int mbert_read_status(const int32_t* meta, int32_t* out4, void* stream) {
    if (!meta || !out4) return MBERT_EINVAL;
    const hipStream_t s = as_stream(stream);
    if (hipMemcpyAsync(out4, meta, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return MBERT_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MBERT_EHIP;
    return MBERT_OK;
}

int mbert_embed_ln(mbert_dtype dt, const int32_t* ids, int total, const int32_t* meta,
                   const void* tok_emb, int vocab, const void* norm_w, float eps, float* resid,
                   void* h, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (total > 0 && (!ids || !tok_emb || !norm_w || !resid || vocab < 1)) return MBERT_EINVAL;
    if (dt != MBERT_F32 && total > 0 && !h) return MBERT_EINVAL;
    return mbh::launch_embed_ln(dt, ids, total, meta, tok_emb, vocab, norm_w, eps, resid, h,
                                as_stream(stream));
}

int mbert_mfma_probe(mbert_dtype dt, int blocks, int iters, float* out, void* stream) {
    MB_TRY(check_dtype(dt));
    if (blocks < 1 || blocks > (1 << 16) || iters < 1 || iters > (1 << 20) || !out) return MBERT_EINVAL;
    return mbh::launch_mfma_probe(dt, blocks, iters, out, as_stream(stream));
}

int mbert_layernorm(mbert_dtype dt, const float* x, int total, const int32_t* meta, const void* w,
                    float eps, void* y, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (total > 0 && (!x || !w || !y)) return MBERT_EINVAL;
    return mbh::launch_layernorm(dt, x, total, meta, w, eps, y, as_stream(stream));
}

int mbert_qkv_rope(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* Wqkv,
                   const float* rope, int max_positions, int table, int apply_rope, void* qkv,
                   void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (total > 0 && (!h || !Wqkv || !qkv)) return MBERT_EINVAL;
    if (apply_rope && (!meta || !rope || max_positions < 1 || (table != 0 && table != 1)))
        return MBERT_EINVAL;
    return mbh::launch_qkv(dt, h, total, meta, Wqkv, rope, max_positions, table, apply_rope, qkv,
                           as_stream(stream));
}

int mbert_rope(mbert_dtype dt, void* qkv, int total, const int32_t* meta, const float* rope,
               int max_positions, int table, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (!meta || !rope || max_positions < 1 || (table != 0 && table != 1)) return MBERT_EINVAL;
    if (total > 0 && !qkv) return MBERT_EINVAL;
    return mbh::launch_rope(dt, qkv, total, meta, rope, max_positions, table, as_stream(stream));
}

int mbert_attention(mbert_dtype dt, const void* qkv, int total, const int32_t* meta, int n_seqs,
                    int is_global, int half_window, void* o, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, n_seqs));
    if (!meta || half_window < 0) return MBERT_EINVAL;
    if (total > 0 && (!qkv || !o)) return MBERT_EINVAL;
    return mbh::launch_attention(dt, qkv, total, meta, n_seqs, is_global ? 1 : 0, half_window, o,
                                 as_stream(stream));
}

int mbert_linear_residual(mbert_dtype dt, const void* a, int K, int total, const int32_t* meta,
                          const void* W, float* resid, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (K != D && K != FF) return MBERT_EUNSUPPORTED;
    if (total > 0 && (!a || !W || !resid)) return MBERT_EINVAL;
    return mbh::launch_linear_residual(dt, a, K, total, meta, W, resid, as_stream(stream));
}

int mbert_mlp_in_geglu(mbert_dtype dt, const void* h, int total, const int32_t* meta,
                       const void* Wi, void* m, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (total > 0 && (!h || !Wi || !m)) return MBERT_EINVAL;
    return mbh::launch_geglu(dt, h, total, meta, Wi, m, as_stream(stream));
}

int mbert_linear_residual_stats(mbert_dtype dt, const void* a, int K, int total,
                                const int32_t* meta, const void* W, float* resid, void* xs,
                                float* stats, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (K != D && K != FF) return MBERT_EUNSUPPORTED;
    if (total > 0 && (!a || !W || !resid || !stats || (dt != MBERT_F32 && !xs))) return MBERT_EINVAL;
    return mbh::launch_linear_residual(dt, a, K, total, meta, W, resid, as_stream(stream),
                                       dt == MBERT_F32 ? nullptr : xs,
                                       reinterpret_cast<float2*>(stats));
}

int mbert_fold_weight(mbert_dtype dt, const void* W, const void* w, int rows, void* Wf, float* c,
                      void* stream) {
    MB_TRY(check_dtype(dt));
    if (rows < 0) return MBERT_EINVAL;
    if (rows > 0 && (!W || !w || !Wf || !c)) return MBERT_EINVAL;
    if (rows == 0) return MBERT_OK;
    return mbh::launch_fold_weight(dt, W, w, rows, Wf, c, as_stream(stream));
}

int mbert_folded_gemm(mbert_dtype dt, int kind, const void* xs, const float* stats, int total,
                      const int32_t* meta, const void* Wf, const float* c, float eps,
                      const float* rope, int max_positions, int table, void* out, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (kind != MBERT_FOLD_QKV_ROPE && kind != MBERT_FOLD_GEGLU) return MBERT_EINVAL;
    if (total > 0 && (!xs || !stats || !Wf || !c || !out)) return MBERT_EINVAL;
    const mbh::FoldArgs fa{c, reinterpret_cast<const float2*>(stats), eps};
    if (kind == MBERT_FOLD_QKV_ROPE) {
        if (!meta || !rope || max_positions < 1 || (table != 0 && table != 1)) return MBERT_EINVAL;
        return mbh::launch_qkv(dt, xs, total, meta, Wf, rope, max_positions, table, 1, out,
                               as_stream(stream), &fa);
    }
    return mbh::launch_geglu(dt, xs, total, meta, Wf, out, as_stream(stream), &fa);
}

size_t mbert_pool_partial_floats(int total_max, int n_seqs) {
    if (total_max < 0 || n_seqs < 0) return 0;
    return tiles_max_for(total_max, n_seqs) * FPARTS * D;
}

int mbert_final_ln_pool(const float* resid, int total, const int32_t* meta, int n_seqs,
                        mbert_dtype dt, const void* w, float eps, float* out, float* pooled,
                        float* partials, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, n_seqs));
    if (!meta || !w || (total > 0 && (!resid || !out)) || (pooled && !partials)) return MBERT_EINVAL;
    return mbh::launch_final_ln_pool(resid, total, meta, n_seqs, dt, w, eps, out, pooled, partials,
                                     as_stream(stream));
}

int mbert_encode_padded_keymask(const mbert_weights* w, const int32_t* ids_pad,
                                const int32_t* mask, int B, int Tpad, void* ws, size_t ws_bytes,
                                float* out_pad, float* pooled, void* stream) {
    return encode_padded_keymask_impl(w, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                                      as_stream(stream));
}

int mbert_attention_probs(mbert_dtype dt, const void* qkv, int total, int row0, int n_q, int n_k,
                          int is_global, int half_window, float* probs, void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (row0 < 0 || n_q < 0 || n_k < 0 || n_k > n_q || (long)row0 + n_q > total || half_window < 0)
        return MBERT_EINVAL;
    if (n_q > 65535 * 16) return MBERT_ERANGE;
    if (n_q > 0 && (!qkv || !probs)) return MBERT_EINVAL;
    return mbh::launch_attention_probs(dt, qkv, row0, n_q, n_k, is_global ? 1 : 0, half_window,
                                       probs, as_stream(stream));
}

int mbert_pool(const float* out, int total, const int32_t* meta, int n_seqs, int mode,
               float* pooled, float* partials, void* stream) {
    MB_TRY(check_sizes(total, n_seqs));
    if (mode < 0 || mode > 3) return MBERT_EINVAL;
    if (n_seqs > 0 && (!meta || !pooled || (total > 0 && !out))) return MBERT_EINVAL;
    if (n_seqs > 0 && (mode & 1) == MBERT_POOL_MEAN && !partials) return MBERT_EINVAL;
    return mbh::launch_pool(out, total, meta, n_seqs, mode, pooled, partials, as_stream(stream));
}

namespace {
struct HeadLayout {
    size_t h0, u, h2, total;
};
HeadLayout head_layout(mbert_dtype dt, int rows) {
    const size_t R = (size_t)(rows > 0 ? rows : 0), ds = dsize(dt);
    HeadLayout L{};
    L.h0 = 0;
    L.u = align256(R * D * ds);
    L.h2 = align256(L.u + R * D * 4);
    L.total = align256(L.h2 + R * D * ds);
    return L;
}
// h2 = LN(gelu(cast(x[rows]) . W_dense^T); norm_w): the prediction head, in the workspace.
int prediction_head(mbert_dtype dt, const float* x, int total, const int32_t* rows, int R,
                    const void* Wd, const void* nw, float eps, char* ws, const HeadLayout& L,
                    hipStream_t s) {
    MB_TRY(mbh::launch_gather_cast(dt, x, total, rows, R, ws + L.h0, s));
    MB_TRY(mbh::launch_linear_f32(dt, ws + L.h0, R, Wd, D, D, 1, nullptr,
                                  reinterpret_cast<float*>(ws + L.u), s));
    return mbh::launch_layernorm(dt, reinterpret_cast<float*>(ws + L.u), R, nullptr, nw, eps,
                                 ws + L.h2, s);
}
}  // namespace

size_t mbert_head_workspace_bytes(mbert_dtype dt, int rows) {
    if (check_dtype(dt) != MBERT_OK || rows < 0) return 0;
    return head_layout(dt, rows).total;
}

int mbert_mlm_head(mbert_dtype dt, const float* x, int total, const int32_t* rows, int n_rows,
                   const void* W_dense, const void* norm_w, float eps, const void* decoder_w,
                   const void* decoder_b, int vocab, void* ws, size_t ws_bytes, float* logits,
                   void* stream) {
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total, 0));
    if (n_rows < 0 || vocab <= 0) return MBERT_EINVAL;
    if (vocab % 64 != 0) return MBERT_EUNSUPPORTED;
    MB_TRY(check_sizes(n_rows, 0));
    if (n_rows == 0) return MBERT_OK;
    if (!x || !W_dense || !norm_w || !decoder_w || !decoder_b || !ws || !logits) return MBERT_EINVAL;
    if (!rows && n_rows > total) return MBERT_EINVAL;
    const HeadLayout L = head_layout(dt, n_rows);
    if (ws_bytes < L.total) return MBERT_ENOSPC;
    const hipStream_t s = as_stream(stream);
    char* w = static_cast<char*>(ws);
    MB_TRY(prediction_head(dt, x, total, rows, n_rows, W_dense, norm_w, eps, w, L, s));
    return mbh::launch_linear_f32(dt, w + L.h2, n_rows, decoder_w, vocab, D, 0, decoder_b, logits, s);
}

int mbert_classifier_head(mbert_dtype dt, const float* pooled, int n_seqs, const void* W_dense,
                          const void* norm_w, float eps, const void* W_cls, const void* b_cls,
                          int n_labels, void* ws, size_t ws_bytes, float* logits, void* stream) {
    MB_TRY(check_dtype(dt));
    if (n_seqs < 0 || n_labels < 1 || n_labels > 4096) return MBERT_EINVAL;
    if (n_seqs > kMaxRows) return MBERT_ERANGE;
    if (n_seqs == 0) return MBERT_OK;
    if (!pooled || !W_dense || !norm_w || !W_cls || !b_cls || !ws || !logits) return MBERT_EINVAL;
    const HeadLayout L = head_layout(dt, n_seqs);
    if (ws_bytes < L.total) return MBERT_ENOSPC;
    const hipStream_t s = as_stream(stream);
    char* w = static_cast<char*>(ws);
    MB_TRY(prediction_head(dt, pooled, n_seqs, nullptr, n_seqs, W_dense, norm_w, eps, w, L, s));
    return mbh::launch_small_linear(dt, w + L.h2, W_cls, b_cls, n_seqs, n_labels, logits, s);
}

int mbert_repad(const float* out, const int32_t* rowmap, int B, int Tpad, float* out_pad,
                void* stream) {
    if (B < 0 || Tpad < 0) return MBERT_EINVAL;
    if ((long)B * Tpad > kMaxRows) return MBERT_ERANGE;
    if ((long)B * Tpad > 0 && (!out || !rowmap || !out_pad)) return MBERT_EINVAL;
    return mbh::launch_repad(out, rowmap, B, Tpad, out_pad, as_stream(stream));
}

size_t mbert_workspace_bytes(const mbert_config* c, mbert_dtype dt, int total_max, int n_seqs) {
    if (check_cfg(c) || check_dtype(dt) || check_sizes(total_max, n_seqs)) return 0;
    return make_layout(dt, total_max, n_seqs).total_bytes;
}

size_t mbert_workspace_bytes_grouped(const mbert_config* c, mbert_dtype dt, int B, int Tpad,
                                     int n_groups) {
    if (check_cfg(c) || check_dtype(dt) || B < 0 || Tpad < 0 || n_groups < 1) return 0;
    if ((long)B * (long)Tpad > kMaxRows) return 0;
    const GroupSplit g = group_split(B, n_groups);
    return make_layout(dt, g.per * Tpad, g.per).total_bytes * (size_t)g.groups;
}

int mbert_workspace_layout(const mbert_config* c, mbert_dtype dt, int total_max, int n_seqs,
                           mbert_ws_layout* layout) {
    MB_TRY(check_cfg(c));
    MB_TRY(check_dtype(dt));
    MB_TRY(check_sizes(total_max, n_seqs));
    if (!layout) return MBERT_EINVAL;
    *layout = make_layout(dt, total_max, n_seqs);
    return MBERT_OK;
}

size_t mbert_folded_bytes(const mbert_config* c, mbert_dtype dt) {
    if (check_cfg(c) || check_dtype(dt)) return 0;
    return fold_layout(dt).stride * (size_t)c->n_layers;
}

int mbert_fold_norms(const mbert_weights* w, void* folded, size_t bytes, void* stream) {
    MB_TRY(check_weights(w));
    if (!folded) return MBERT_EINVAL;
    if (bytes < mbert_folded_bytes(&w->cfg, w->dtype)) return MBERT_ENOSPC;
    const FoldLayout F = fold_layout(w->dtype);
    hipStream_t s = as_stream(stream);
    for (int l = 0; l < w->cfg.n_layers; ++l) {
        char* fb = static_cast<char*>(folded) + (size_t)l * F.stride;
        const mbert_layer_weights& lw = w->layers[l];
        if (l > 0)
            MB_TRY(mbh::launch_fold_weight(w->dtype, lw.Wqkv, lw.attn_norm, QKV, fb + F.wq,
                                           reinterpret_cast<float*>(fb + F.cq), s));
        MB_TRY(mbh::launch_fold_weight(w->dtype, lw.Wi, lw.mlp_norm, 2 * FF, fb + F.wi,
                                       reinterpret_cast<float*>(fb + F.ci), s));
    }
    return MBERT_OK;
}

int mbert_layer(const mbert_weights* w, int layer, int total, int n_seqs, void* ws,
                size_t ws_bytes, void* stream) {
    MB_TRY(check_weights(w));
    MB_TRY(check_sizes(total, n_seqs));
    if (!ws || layer < 0 || layer >= w->cfg.n_layers) return MBERT_EINVAL;
    const mbert_ws_layout L = make_layout(w->dtype, total, n_seqs);
    if (ws_bytes < L.total_bytes) return MBERT_ENOSPC;
    if (total == 0) return MBERT_OK;
    return run_layer(w, layer, total, n_seqs, static_cast<char*>(ws), L, as_stream(stream), nullptr);
}

int mbert_encode(const mbert_weights* w, const int32_t* ids, const int32_t* cu, int n_seqs,
                 int total, void* ws, size_t ws_bytes, float* out, float* pooled, void* stream) {
    return encode_impl(w, ids, cu, n_seqs, total, ws, ws_bytes, out, pooled, as_stream(stream),
                       nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------- forward without allocation
// The workspace of mbert_encode_noalloc: a fixed device array owned by the library (one copy
// per GPU, held until the process ends). Host code never passes this name to a kernel or a
// copy: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MBERT_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MBERT_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MBERT_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MBERT_OK;
}
}  // namespace

extern "C" {

size_t mbert_noalloc_max_bytes(void) { return MBERT_NOALLOC_WORKSPACE_BYTES; }

int mbert_encode_noalloc(const mbert_weights* w, const int32_t* ids, const int32_t* cu,
                         int n_seqs, int total, float* out, float* pooled, void* stream) {
    MB_TRY(check_weights(w));
    MB_TRY(check_sizes(total, n_seqs));
    if (make_layout(w->dtype, total, n_seqs).total_bytes > MBERT_NOALLOC_WORKSPACE_BYTES)
        return MBERT_ENOSPC;
    void* ws = nullptr;
    MB_TRY(scratch_address(&ws));
    return encode_impl(w, ids, cu, n_seqs, total, ws, MBERT_NOALLOC_WORKSPACE_BYTES, out, pooled,
                       as_stream(stream), nullptr);
}

int mbert_encode_padded(const mbert_weights* w, const int32_t* ids_pad, const int32_t* mask, int B,
                        int Tpad, void* ws, size_t ws_bytes, float* out_pad, float* pooled,
                        void* stream) {
    return encode_padded_impl(w, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                              as_stream(stream), nullptr);
}

int mbert_encode_padded_grouped(const mbert_weights* w, const int32_t* ids_pad,
                                const int32_t* mask, int B, int Tpad, int n_groups, void* ws,
                                size_t ws_bytes, float* out_pad, float* pooled,
                                void* const* streams, void* stream) {
    return encode_padded_grouped_impl(w, ids_pad, mask, B, Tpad, n_groups, ws, ws_bytes, out_pad,
                                      pooled, reinterpret_cast<const hipStream_t*>(streams),
                                      as_stream(stream));
}

// ---------------------------------------------------------------- graphs
static int capture_common(hipStream_t s, mbert_graph** graph, int (*body)(void*), void* ctx) {
    if (!graph || s == nullptr) return MBERT_EINVAL;
    *graph = nullptr;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) return MBERT_EHIP;
    const int rc = body(ctx);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (rc != MBERT_OK) {
        if (g) (void)hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess || !g) return MBERT_EHIP;
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(g);
        return MBERT_EHIP;
    }
    mbert_graph* G = new (std::nothrow) mbert_graph;
    if (!G) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(g);
        return MBERT_EINVAL;
    }
    G->graph = g;
    G->exec = exec;
    *graph = G;
    return MBERT_OK;
}

struct PackedCtx {
    const mbert_weights* w;
    const int32_t *ids, *cu;
    int n_seqs, total;
    void* ws;
    size_t ws_bytes;
    float *out, *pooled;
    hipStream_t s;
};
struct PaddedCtx {
    const mbert_weights* w;
    const int32_t *ids_pad, *mask;
    int B, Tpad;
    void* ws;
    size_t ws_bytes;
    float *out_pad, *pooled;
    hipStream_t s;
};

int mbert_graph_capture(const mbert_weights* w, const int32_t* ids, const int32_t* cu, int n_seqs,
                        int total, void* ws, size_t ws_bytes, float* out, float* pooled,
                        void* stream, mbert_graph** graph) {
    MB_TRY(check_weights(w));  // fail before capture starts
    PackedCtx c{w, ids, cu, n_seqs, total, ws, ws_bytes, out, pooled, as_stream(stream)};
    return capture_common(as_stream(stream), graph, [](void* p) {
        PackedCtx* x = static_cast<PackedCtx*>(p);
        return encode_impl(x->w, x->ids, x->cu, x->n_seqs, x->total, x->ws, x->ws_bytes, x->out,
                           x->pooled, x->s, nullptr);
    }, &c);
}

int mbert_graph_capture_padded(const mbert_weights* w, const int32_t* ids_pad, const int32_t* mask,
                               int B, int Tpad, void* ws, size_t ws_bytes, float* out_pad,
                               float* pooled, void* stream, mbert_graph** graph) {
    MB_TRY(check_weights(w));
    PaddedCtx c{w, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled, as_stream(stream)};
    return capture_common(as_stream(stream), graph, [](void* p) {
        PaddedCtx* x = static_cast<PaddedCtx*>(p);
        return encode_padded_impl(x->w, x->ids_pad, x->mask, x->B, x->Tpad, x->ws, x->ws_bytes,
                                  x->out_pad, x->pooled, x->s, nullptr);
    }, &c);
}

struct GroupedCtx {
    const mbert_weights* w;
    const int32_t *ids_pad, *mask;
    int B, Tpad, n_groups;
    void* ws;
    size_t ws_bytes;
    float *out_pad, *pooled;
    const hipStream_t* extra;
    hipStream_t s;
};

int mbert_graph_capture_padded_grouped(const mbert_weights* w, const int32_t* ids_pad,
                                       const int32_t* mask, int B, int Tpad, int n_groups,
                                       void* ws, size_t ws_bytes, float* out_pad, float* pooled,
                                       void* const* streams, void* stream, mbert_graph** graph) {
    MB_TRY(check_weights(w));
    GroupedCtx c{w, ids_pad, mask, B, Tpad, n_groups, ws, ws_bytes, out_pad, pooled,
                 reinterpret_cast<const hipStream_t*>(streams), as_stream(stream)};
    return capture_common(as_stream(stream), graph, [](void* p) {
        GroupedCtx* x = static_cast<GroupedCtx*>(p);
        return encode_padded_grouped_impl(x->w, x->ids_pad, x->mask, x->B, x->Tpad, x->n_groups,
                                          x->ws, x->ws_bytes, x->out_pad, x->pooled, x->extra,
                                          x->s);
    }, &c);
}

int mbert_graph_launch(mbert_graph* graph, void* stream) {
    if (!graph || !graph->exec) return MBERT_EINVAL;
    return hipGraphLaunch(graph->exec, as_stream(stream)) == hipSuccess ? MBERT_OK : MBERT_EHIP;
}

int mbert_graph_destroy(mbert_graph* graph) {
    if (!graph) return MBERT_EINVAL;
    if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
    if (graph->graph) (void)hipGraphDestroy(graph->graph);
    delete graph;
    return MBERT_OK;
}

// ---------------------------------------------------------------- timing
int mbert_timer_create(int max_launches, mbert_timer** timer) {
    if (!timer || max_launches < 1 || max_launches > (1 << 20)) return MBERT_EINVAL;
    *timer = nullptr;
    mbert_timer* t = new (std::nothrow) mbert_timer;
    if (!t) return MBERT_EINVAL;
    t->ev.resize(2 * (size_t)max_launches, nullptr);
    for (auto& e : t->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto& f : t->ev)
                if (f) (void)hipEventDestroy(f);
            delete t;
            return MBERT_EHIP;
        }
    }
    *timer = t;
    return MBERT_OK;
}

int mbert_timer_reset(mbert_timer* t) {
    if (!t) return MBERT_EINVAL;
    t->used = 0;
    return MBERT_OK;
}

int mbert_timer_read(mbert_timer* t, int* launches, double* total_ms) {
    if (!t || !launches || !total_ms) return MBERT_EINVAL;
    *launches = t->used;
    *total_ms = 0.0;
    if (t->used == 0) return MBERT_OK;
    if (hipEventSynchronize(t->ev[2 * t->used - 1]) != hipSuccess) return MBERT_EHIP;
    double sum = 0.0;
    for (int i = 0; i < t->used; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess) return MBERT_EHIP;
        sum += ms;
    }
    *total_ms = sum;
    return MBERT_OK;
}

int mbert_timer_destroy(mbert_timer* t) {
    if (!t) return MBERT_EINVAL;
    for (auto& e : t->ev)
        if (e) (void)hipEventDestroy(e);
    delete t;
    return MBERT_OK;
}

int mbert_encode_timed(const mbert_weights* w, const int32_t* ids, const int32_t* cu, int n_seqs,
                       int total, void* ws, size_t ws_bytes, float* out, float* pooled,
                       void* stream, int kind, mbert_timer* timer) {
    if (!timer || kind < 0 || kind >= MBERT_K_COUNT) return MBERT_EINVAL;
    Recorder rec{timer, kind};
    return encode_impl(w, ids, cu, n_seqs, total, ws, ws_bytes, out, pooled, as_stream(stream), &rec);
}

int mbert_encode_padded_timed(const mbert_weights* w, const int32_t* ids_pad, const int32_t* mask,
                              int B, int Tpad, void* ws, size_t ws_bytes, float* out_pad,
                              float* pooled, void* stream, int kind, mbert_timer* timer) {
    if (!timer || kind < 0 || kind >= MBERT_K_COUNT) return MBERT_EINVAL;
    Recorder rec{timer, kind};
    return encode_padded_impl(w, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                              as_stream(stream), &rec);
}

}  // extern "C"
