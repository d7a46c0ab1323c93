/*
 * mbert.h — C ABI of the MI355X (gfx950) ModernBERT-base encoder forward.
 *
 * What is computed (the pages this library follows, by title and section):
 *   kgptalkie.com "ModernBERT-base Architecture Teardown: Every Layer With Real Code"
 *   candding docs "ModernBERT", safebydesign.ai "ModernBertModel 22L 768d",
 *   nest.franknoh.dev "modernbert-base", rayaq.ca "Encoder-only models".
 *   The encoder: embedding row gather + weight-only LayerNorm; 22 pre-norm layers (layer 0
 *   without attention norm) of fused Wqkv -> rotate-half RoPE (base 160000 on global layers
 *   i % 3 == 0, 10000 on local ones) -> bidirectional softmax attention (local layers keep
 *   key j for query i iff |i - j| <= 64) -> Wo + residual -> LayerNorm -> Wi -> exact-erf
 *   GeGLU (first half activated, second half the multiplier) -> Wo + residual; the final
 *   LayerNorm; masked mean pooling with L2 normalisation. Batches are unpadded: sequences
 *   are packed back to back and delimited by cu_seqlens.
 *
 * Conventions (every entry point):
 *   - Pointers named "device" are HIP device pointers; "host" pointers are ordinary memory.
 *     The caller owns every buffer. The library never allocates or frees device memory and
 *     keeps no mutable global state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls only enqueue
 *     work and return; synchronisation is the caller's job. No call synchronises the device
 *     except mbert_read_status and mbert_build_rope_tables (documented there).
 *   - Return value: MBERT_OK (0) or one of the error codes below. Nothing is thrown across the
 *     ABI. Host-detectable errors are reported before anything is enqueued.
 *   - Data that lives on the device (token ids, cu_seqlens, masks) is validated on the device
 *     by the meta kernels; problems set bits in the status word of the meta buffer (read it
 *     with mbert_read_status). A batch with invalid cu_seqlens gets no attention work at all
 *     and its outputs are unspecified, but no kernel reads or writes out of bounds.
 *   - Dtypes: ids, cu_seqlens, indices and all meta are int32. Weights and GEMM inputs use
 *     `dtype`; the residual stream, per-token outputs and pooled vectors are always float32.
 *   - Kernels are specialised to ModernBERT-base's shapes: hidden 768, 12 heads of 64,
 *     intermediate 1152. Other dims return MBERT_EUNSUPPORTED.
 *   - Calls on different streams are safe when they use different workspaces and outputs.
 */
#ifndef MBERT_H
#define MBERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- error codes */
#define MBERT_OK 0
#define MBERT_EINVAL 1       /* NULL pointer, negative or inconsistent size, bad argument */
#define MBERT_EUNSUPPORTED 2 /* dims other than 768/12/64/1152, or an unknown dtype        */
#define MBERT_ERANGE 3       /* a size beyond a documented limit (e.g. max_positions)       */
#define MBERT_ENOSPC 4       /* workspace smaller than mbert_workspace_bytes()             */
#define MBERT_EHIP 5         /* a HIP launch or runtime call failed                         */

/* status bits written by the meta kernels (counts[MBERT_META_STATUS]) */
#define MBERT_STATUS_BAD_CU 1        /* cu_seqlens[0] != 0, decreasing, or cu[S] != total  */
#define MBERT_STATUS_TOO_LONG 2      /* a sequence longer than max_positions                */
#define MBERT_STATUS_BAD_MASK 4      /* a padding-mask entry other than 0 or 1              */
#define MBERT_STATUS_BAD_ID 8        /* a token id outside [0, vocab); that row reads row 0 */

typedef enum { MBERT_F32 = 0, MBERT_BF16 = 1, MBERT_F16 = 2 } mbert_dtype;

/* Hyper-parameters (kgptalkie §"What Is ModernBERT-base?"; candding §"What it is",
 * §"The alternating attention", §"The two rope tables"). */
typedef struct {
    int n_layers;        /* 22                                                     */
    int hidden;          /* 768  (fixed)                                           */
    int n_heads;         /* 12   (fixed)                                           */
    int head_dim;        /* 64   (fixed)                                           */
    int intermediate;    /* 1152 (fixed)                                           */
    int vocab;           /* 50368                                                  */
    int global_every;    /* 3: layer i is global iff i % global_every == 0         */
    int half_window;     /* 64: local layers keep |i - j| <= half_window (0..4096) */
    int max_positions;   /* 8192: longest accepted sequence; RoPE table length     */
    double theta_global; /* 160000                                                 */
    double theta_local;  /* 10000                                                  */
    float norm_eps;      /* 1e-5                                                   */
} mbert_config;

/* One layer's weights: device pointers, `dtype` elements, Linear weights [out, in]
 * row-major (candding §"The tensors"). */
typedef struct {
    const void* attn_norm; /* [768]; must be NULL on layer 0 (no attention norm there) */
    const void* Wqkv;      /* [2304, 768]: rows 0-767 query, 768-1535 key, 1536-2303 value */
    const void* attn_Wo;   /* [768, 768]                                               */
    const void* mlp_norm;  /* [768]                                                    */
    const void* Wi;        /* [2304, 768]: rows 0-1151 GELU branch, 1152-2303 multiplier */
    const void* mlp_Wo;    /* [768, 1152]                                              */
} mbert_layer_weights;

typedef struct {
    mbert_config cfg;
    mbert_dtype dtype;
    const void* tok_emb;               /* device [vocab, 768]                          */
    const void* emb_norm;              /* device [768]                                 */
    const void* final_norm;            /* device [768]                                 */
    const mbert_layer_weights* layers; /* HOST array [cfg.n_layers]                    */
    const float* rope;                 /* device tables from mbert_build_rope_tables   */
    const void* folded;                /* device buffer from mbert_fold_norms, or NULL */
} mbert_weights;

/* ---------------------------------------------------------------- folded LayerNorms
 * The pre-norm LayerNorms inside the stack (attn_norm of layers >= 1, mlp_norm of every
 * layer; candding §"The pre-norm layer and the final norm") can be folded into the GEMM that
 * reads them: LN(x) . W^T = rstd * (x . (W o w)^T - mean * c), c_r = sum_k (W o w)[r][k],
 * with mean and rstd of each row of x (biased variance, eps inside the square root). The
 * residual GEMMs then also write each row's statistics per 64-column chunk and the residual
 * rounded to dtype, and no separate LayerNorm kernel runs between them. Only the rounding
 * point moves: dtype(x) enters the GEMM instead of dtype(LN(x)). The rounding error of x is
 * relative to |x|, that of LN(x) to the row's spread, so the two agree while a row's mean is
 * small against its spread: the normalised error grows like |mean| / std times one unit of
 * the dtype (2^-9 bf16, 2^-12 fp16), i.e. cancellation in x - mean, not range. Magnitude
 * alone is harmless: the fp32 residual and its chunk statistics stay exact, and a trained
 * model's residual stream peaks near 81 % of the fp16 maximum (candding §"Dtype headroom"),
 * which fp16 holds; a residual beyond 65,504 would overflow the fp16 copy, and such a model
 * must run with folded = NULL (separate LayerNorms from the fp32 residual).
 * mbert_fold_norms fills `folded` (mbert_folded_bytes(cfg, dtype) bytes, device) from w's
 * current weights; setting w->folded to it makes mbert_encode, mbert_encode_padded and
 * mbert_encode_padded_keymask (and their graph captures) use the folded path; mbert_layer
 * always runs the separate LayerNorm. Re-run after changing a Wqkv, Wi or norm weight.
 * Layout per layer l: Wqkv o attn_norm [2304,768] dtype, its c [2304] f32, Wi o mlp_norm
 * [2304,768] dtype, its c [2304] f32, each 256-byte aligned (layer 0's first two unused).
 * Returns MBERT_ENOSPC if bytes is too small. */
size_t mbert_folded_bytes(const mbert_config* cfg, mbert_dtype dtype);
int mbert_fold_norms(const mbert_weights* w, void* folded, size_t bytes, void* stream);

/* ---------------------------------------------------------------- meta buffer layout
 * One int32 device buffer of mbert_meta_ints(total_max, n_seqs) elements:
 *   [0, 8)                 counts: [0] total tokens T, [1] max_seqlen, [2] n_tiles,
 *                                  [3] status bits, [4..7] reserved (0)
 *   [8, 8+total_max)       pos: position of every token inside its sequence (0 .. L-1)
 *   then S+1               seq_tile0: first work tile of each sequence; [S] = n_tiles
 *   then (16-byte aligned) 4 * tiles_max ints: {q0, qn, s0, s1} per work tile: tokens
 *                          [q0, q0+qn) of the sequence [s0, s1); tiles never cross sequences;
 *                          qn <= mbert_tile_tokens()
 *   then tiles_max ints    order: a permutation of [0, n_tiles), the order in which the
 *                          attention takes the tiles (tiles of longer sequences first; in
 *                          row order for the full-width padded path)
 * tiles_max = ceil(total_max / tile_tokens) + n_seqs. */
#define MBERT_META_TOTAL 0
#define MBERT_META_MAXLEN 1
#define MBERT_META_NTILES 2
#define MBERT_META_STATUS 3

/* ---------------------------------------------------------------- library info */
int mbert_version(void);                     /* 100 * major + minor                    */
const char* mbert_strerror(int code);        /* static string, never NULL              */
int mbert_default_config(mbert_config* cfg); /* fills the ModernBERT-base values       */
int mbert_check_config(const mbert_config* cfg);
int mbert_tile_tokens(void);                 /* query rows per work tile (128)         */
size_t mbert_meta_ints(int total_max, int n_seqs);
size_t mbert_dtype_size(mbert_dtype dtype);  /* 4, 2, 2; 0 for an unknown dtype        */

/* ---------------------------------------------------------------- RoPE tables
 * float2 {cos, sin} tables [2][max_positions][head_dim/2]: table 0 uses theta_global,
 * table 1 theta_local; entry [p][i] is the angle p * theta^(-2i/64) (kgptalkie §"How Does
 * RoPE Work With Two Bases?"), evaluated in float64 on the device and rounded once to
 * float32. `table` holds mbert_rope_table_floats(cfg) floats. Enqueued on `stream`. */
size_t mbert_rope_table_floats(const mbert_config* cfg);
int mbert_build_rope_tables(const mbert_config* cfg, float* table, void* stream);

/* ---------------------------------------------------------------- batch meta
 * mbert_pack_meta: packed batch. From device cu_seqlens [n_seqs+1] (cu[0] = 0,
 * non-decreasing, cu[n_seqs] = total) build the meta buffer: counts, work tiles, positions.
 * Validates cu_seqlens on the device (status bits). max_positions bounds every length. */
int mbert_pack_meta(const int32_t* cu_seqlens, int n_seqs, int total, int max_positions,
                    int32_t* meta, void* stream);

/* mbert_unpad: padded batch ids_pad/mask [B, Tpad] (device, row-major, mask 1 = real token;
 * kgptalkie §"How Does Text Become Tokens?") -> packed ids [B*Tpad max], indices [B*Tpad max]
 * (flat b*Tpad+t of each real token, ascending), rowmap [B*Tpad] (packed index of each padded
 * slot or -1), cu_seqlens [B+1], and the meta buffer (sized for total_max = B*Tpad, n_seqs =
 * B). A token's position is its rank among the real tokens of its row. */
int mbert_unpad(const int32_t* ids_pad, const int32_t* mask, int B, int Tpad,
                int max_positions, int32_t* ids, int32_t* indices, int32_t* rowmap,
                int32_t* cu_seqlens, int32_t* meta, void* stream);

/* mbert_attn_key_ranges: for every token t < T, the first and last token index (inclusive)
 * its query reads on a global (is_global = 1) or local layer; computed by the same device
 * function the attention kernel uses (candding §"The alternating attention"). Debug/test. */
int mbert_attn_key_ranges(const int32_t* meta, int total_max, int n_seqs, int is_global,
                          int half_window, int32_t* lo, int32_t* hi, void* stream);

/* mbert_read_status: copies counts[0..3] of a meta buffer to host `out4`, synchronising
 * `stream` first. */
int mbert_read_status(const int32_t* meta, int32_t* out4, void* stream);

/* ---------------------------------------------------------------- per-step entry points
 * Row counts: `total` is the number of token rows the buffers hold (host value). When `meta`
 * is not NULL the kernels process only counts[MBERT_META_TOTAL] <= total rows (the padded
 * path sizes buffers for B*Tpad and learns T on the device). Row strides are dense. */

/* Embedding gather + LayerNorm (kgptalkie §"How Do Token Ids Become Vectors?",
 * §"What Does LayerNorm Do?"): resid [T,768] f32 = LN(tok_emb[ids]; w); h [T,768] dtype is
 * the same values rounded to dtype (for MBERT_F32, h may equal resid or be NULL). */
int mbert_embed_ln(mbert_dtype dtype, const int32_t* ids, int total, const int32_t* meta,
                   const void* tok_emb, int vocab, const void* norm_w, float eps,
                   float* resid, void* h, void* stream);

/* Weight-only LayerNorm, biased variance, eps inside the square root: x f32 [T,768] ->
 * y dtype [T,768] (candding §"The pre-norm layer and the final norm"). */
int mbert_layernorm(mbert_dtype dtype, const float* x, int total, const int32_t* meta,
                    const void* w, float eps, void* y, void* stream);

/* qkv [T,2304] = h [T,768] . Wqkv^T; with apply_rope, columns 0-1535 (query and key, head by
 * head) are rotated in the epilogue with table `table` (0 = global base, 1 = local) at
 * each row's position (meta pos). Rotate-half: y_i = x_i c - x_{i+32} s,
 * y_{i+32} = x_{i+32} c + x_i s (candding §"The two rope tables"). meta is required. */
int mbert_qkv_rope(mbert_dtype dtype, const void* h, int total, const int32_t* meta,
                   const void* Wqkv, const float* rope, int max_positions, int table,
                   int apply_rope, void* qkv, void* stream);

/* Standalone rotate-half RoPE, in place on the query and key columns of qkv [T,2304]. */
int mbert_rope(mbert_dtype dtype, void* qkv, int total, const int32_t* meta,
               const float* rope, int max_positions, int table, void* stream);

/* Varlen attention: o [T,768] = per head softmax(q k^T / 8) v over the keys of the same
 * sequence; on local layers (is_global = 0) only keys with |i - j| <= half_window
 * (kgptalkie §"How Does Self-Attention Work?", §"What Are Local and Global Attention?").
 * Work comes from the meta tiles; no row ever reads another sequence. */
int mbert_attention(mbert_dtype dtype, const void* qkv, int total, const int32_t* meta,
                    int n_seqs, int is_global, int half_window, void* o, void* stream);

/* resid [T,768] f32 += a [T,K] . W^T, W [768,K]; K = 768 (attention Wo) or 1152 (MLP Wo). */
int mbert_linear_residual(mbert_dtype dtype, const void* a, int K, int total,
                          const int32_t* meta, const void* W, float* resid, void* stream);

/* m [T,1152] = gelu_erf(u[:, :1152]) * u[:, 1152:], u = h [T,768] . Wi^T (candding §"The
 * feed-forward halves"; kgptalkie §"What Does the GeGLU MLP Do?"). */
int mbert_mlp_in_geglu(mbert_dtype dtype, const void* h, int total, const int32_t* meta,
                       const void* Wi, void* m, void* stream);

/* The folded path one step at a time (the same kernels the folded forward runs).
 * mbert_linear_residual_stats: resid += a . W^T as mbert_linear_residual, and also
 * stats [T,12,2] f32 = {mean, sum of squared deviations from it} of each 64-column chunk of
 * each new residual row, and xs [T,768] dtype = the new residual rounded once to dtype
 * (16-bit types; ignored for MBERT_F32, whose folded GEMM reads resid itself).
 * mbert_fold_weight: Wf [rows,768] dtype = W o w (each column k scaled by the norm weight
 * w[k], rounded once), c [rows] f32 = the sum of each rounded row of Wf.
 * mbert_folded_gemm: LN(x; w) . W^T computed as rstd * (xs . Wf^T - mean * c), mean and rstd
 * merged from the chunk statistics (Chan et al.'s pairwise formula; biased variance, eps
 * inside the square root). kind MBERT_FOLD_QKV_ROPE: Wf from Wqkv, out = qkv [T,2304] with
 * RoPE as mbert_qkv_rope (apply_rope = 1; meta, rope, table required); kind
 * MBERT_FOLD_GEGLU: Wf from Wi, out = m [T,1152] as mbert_mlp_in_geglu. For MBERT_F32 pass
 * the fp32 residual as xs. */
#define MBERT_FOLD_QKV_ROPE 0
#define MBERT_FOLD_GEGLU 1
int mbert_linear_residual_stats(mbert_dtype dtype, const void* a, int K, int total,
                                const int32_t* meta, const void* W, float* resid, void* xs,
                                float* stats, void* stream);
int mbert_fold_weight(mbert_dtype dtype, const void* W, const void* w, int rows, void* Wf,
                      float* c, void* stream);
int mbert_folded_gemm(mbert_dtype dtype, int kind, const void* xs, const float* stats, int total,
                      const int32_t* meta, const void* Wf, const float* c, float eps,
                      const float* rope, int max_positions, int table, void* out, void* stream);

/* Final LayerNorm and pooling: out [T,768] f32 = LN(resid; w); pooled [S,768] f32 = the mean
 * of each sequence's rows of out divided by max(L2 norm, 1e-12); an empty sequence pools to
 * 0 (kgptalkie §"How Do We Get One Vector per Text?"; safebydesign §"Implementing it").
 * `partials` is scratch of mbert_pool_partial_floats(total, n_seqs) floats. pooled may be
 * NULL (then partials may be NULL too). meta is required. Deterministic: no atomics. */
size_t mbert_pool_partial_floats(int total_max, int n_seqs);
int mbert_final_ln_pool(const float* resid, int total, const int32_t* meta, int n_seqs,
                        mbert_dtype dtype, const void* w, float eps, float* out,
                        float* pooled, float* partials, void* stream);

/* Attention probabilities of one sequence, every head, for inspection (not used by the
 * forward): probs [12][n_q][n_k] f32, probs[h][i][j] = softmax over allowed keys of
 * q_i . k_j / 8 for query rows row0 + i (i < n_q) and key rows row0 + j (j < n_k <= n_q) of
 * qkv [total,2304] (RoPE already applied), positions counted from row0; a local layer
 * (is_global = 0) allows |i - j| <= half_window (kgptalkie §"How Does Self-Attention
 * Work?", §"What Are Local and Global Attention?"). Disallowed keys, and all keys of a query
 * without any, are 0. n_k < n_q is a padded row: its keys are the real tokens. */
int mbert_attention_probs(mbert_dtype dtype, const void* qkv, int total, int row0, int n_q,
                          int n_k, int is_global, int half_window, float* probs, void* stream);

/* Pooling of finished rows out [T,768] f32 (after the final LayerNorm), per sequence of the
 * meta buffer: MBERT_POOL_MEAN, the mean of the sequence's rows (kgptalkie §"How Do We Get
 * One Vector per Text?"), or MBERT_POOL_CLS, its first row (candding §"Pooling and
 * normalization": index 0); with MBERT_POOL_L2 or'ed in, each pooled vector is divided by
 * max(L2 norm, 1e-12). An empty sequence pools to 0. `partials` is scratch of
 * mbert_pool_partial_floats(total, n_seqs) floats (unused, may be NULL, for CLS). Deterministic. */
enum { MBERT_POOL_MEAN = 0, MBERT_POOL_CLS = 1, MBERT_POOL_L2 = 2 };
int mbert_pool(const float* out, int total, const int32_t* meta, int n_seqs, int mode,
               float* pooled, float* partials, void* stream);

/* ---- heads (kgptalkie §"The Masked-LM Head", §"How Do We Put a Classifier on Top?")
 * Both start with the prediction head: h = LN(gelu_erf(x . W_dense^T); norm_w, eps), W_dense
 * [768,768] without bias, LayerNorm weight-only like the encoder's.
 * mbert_mlm_head: x is the final hidden state [total,768] f32; rows (device int32 [n_rows], or
 * NULL for rows 0..n_rows-1) selects the positions to score (e.g. the [MASK] tokens); a row
 * index outside [0, total) scores a zero vector. logits [n_rows, vocab] f32 = h . decoder_w^T
 * + decoder_b, decoder_w [vocab,768] (the tied embedding table), decoder_b [vocab]; vocab must
 * be a multiple of 64 (50,368 is).
 * mbert_classifier_head: pooled [n_seqs,768] f32 (mbert_pool, MBERT_POOL_MEAN without L2 for
 * ModernBERT's classifier); logits [n_seqs, n_labels] f32 = h . W_cls^T + b_cls, W_cls
 * [n_labels,768], b_cls [n_labels], 1 <= n_labels <= 4096.
 * Weights are of `dtype`. `ws` is device scratch of mbert_head_workspace_bytes(dtype, rows)
 * bytes, rows = n_rows or n_seqs. */
size_t mbert_head_workspace_bytes(mbert_dtype dtype, int rows);
int mbert_mlm_head(mbert_dtype dtype, const float* x, int total, const int32_t* rows, int n_rows,
                   const void* W_dense, const void* norm_w, float eps, const void* decoder_w,
                   const void* decoder_b, int vocab, void* ws, size_t ws_bytes, float* logits,
                   void* stream);
int mbert_classifier_head(mbert_dtype dtype, const float* pooled, int n_seqs, const void* W_dense,
                          const void* norm_w, float eps, const void* W_cls, const void* b_cls,
                          int n_labels, void* ws, size_t ws_bytes, float* logits, void* stream);

/* Re-pad: out_pad [B,Tpad,768] f32 gets row rowmap[b*Tpad+t] of out, or zeros where
 * rowmap is -1 (the zero-filled unpacking of rayaq §"Padding and the key padding mask"). */
int mbert_repad(const float* out, const int32_t* rowmap, int B, int Tpad, float* out_pad,
                void* stream);

/* ---------------------------------------------------------------- workspace
 * Device scratch for one forward; the caller allocates mbert_workspace_bytes() bytes
 * (256-byte aligned). Layout (byte offsets from mbert_workspace_layout): resid f32
 * [Tmax,768], h dtype [Tmax,768] (also the attention output), qkv dtype [Tmax,2304] (also the
 * GeGLU output), meta, pool partials, for the padded path ids/indices/rowmap/cu, and for
 * folded LayerNorms xs dtype [Tmax,768] (the residual rounded) and rstats f32 [Tmax,12,2].
 * (The padded path's final norm writes the caller's padded output directly.) */
typedef struct {
    size_t resid, h, qkv, meta, partials, ids, indices, rowmap, cu, xs, rstats, total_bytes;
} mbert_ws_layout;
size_t mbert_workspace_bytes(const mbert_config* cfg, mbert_dtype dtype, int total_max,
                             int n_seqs);
int mbert_workspace_layout(const mbert_config* cfg, mbert_dtype dtype, int total_max,
                           int n_seqs, mbert_ws_layout* layout);

/* One encoder layer `layer` on the workspace's residual stream (resid in, resid out;
 * h must hold LN(resid) only for layer 0, where the embedding norm output is used as is). */
int mbert_layer(const mbert_weights* w, int layer, int total, int n_seqs, void* ws,
                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- the forward
 * mbert_encode: packed batch. ids [total], cu_seqlens [n_seqs+1] on the device. Writes
 * out [total,768] f32 (after the final LayerNorm) and, if not NULL, pooled [n_seqs,768]. */
int mbert_encode(const mbert_weights* w, const int32_t* ids, const int32_t* cu_seqlens,
                 int n_seqs, int total, void* ws, size_t ws_bytes, float* out,
                 float* pooled, void* stream);

/* mbert_encode_noalloc: mbert_encode without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc). The workspace is a fixed device array inside the
 * library, MBERT_NOALLOC_WORKSPACE_BYTES (64 MiB) on each GPU the library runs on, held
 * until the process ends; its address is looked up once per device (the device current at
 * the call; `stream` must belong to it). Returns MBERT_ENOSPC when
 * mbert_workspace_bytes(cfg, dtype, total, n_seqs) exceeds it (about 6,000 tokens in bf16 or
 * fp16, 3,500 in fp32), before any work is enqueued. Every part of the array is written
 * before it is read within one call, so nothing needs clearing between calls; the array
 * keeps the last call's contents. All calls on one GPU share the array: calls that overlap
 * in time on one GPU (different streams or threads without ordering between them) race and
 * corrupt each other's results. Same outputs as mbert_encode on the same inputs. */
#define MBERT_NOALLOC_WORKSPACE_BYTES (64ull << 20)
size_t mbert_noalloc_max_bytes(void);
int mbert_encode_noalloc(const mbert_weights* w, const int32_t* ids, const int32_t* cu_seqlens,
                         int n_seqs, int total, float* out, float* pooled, void* stream);

/* mbert_encode_padded: padded batch ids_pad/mask [B,Tpad] on the device: unpad, encode,
 * re-pad. out_pad [B,Tpad,768] f32 with zeros at pads (the final LayerNorm writes each token's
 * row to its padded slot); pooled [B,768] (may be NULL). The packed cu_seqlens/indices stay
 * in the workspace (layout.cu/layout.indices). No host synchronisation: the token count stays
 * on the device. Workspace from mbert_workspace_bytes(cfg, dtype, B*Tpad, B). */
int mbert_encode_padded(const mbert_weights* w, const int32_t* ids_pad, const int32_t* mask,
                        int B, int Tpad, void* ws, size_t ws_bytes, float* out_pad,
                        float* pooled, void* stream);

/* The padded batch run as is, without unpadding (what a caller without varlen support
 * computes): every one of the B*Tpad rows goes through the layers, row b's keys are its
 * first L_b rows (mask rows must be right-padded: ones, then zeros; otherwise
 * MBERT_STATUS_BAD_MASK is set and the leading run of ones is used), a query with no key in
 * its window outputs zeros. out_pad [B,Tpad,768] f32 with zeros at the pads; pooled [B,768]
 * over the real tokens as in mbert_encode. Real rows agree with mbert_encode_padded (the key
 * padding mask hides pads exactly: rayaq §"Padding and the key padding mask"); it does
 * B*Tpad/T times the work. Workspace as mbert_encode_padded. */
int mbert_encode_padded_keymask(const mbert_weights* w, const int32_t* ids_pad,
                                const int32_t* mask, int B, int Tpad, void* ws, size_t ws_bytes,
                                float* out_pad, float* pooled, void* stream);

/* The padded batch split into n_groups groups of consecutive rows (whole sequences; the last
 * group may hold fewer), each group's forward (as mbert_encode_padded) enqueued on its own
 * stream: group 0 on `stream`, group g on streams[g-1] (n_groups-1 distinct streams, none of
 * them `stream`), forked from `stream` and joined back into it with events, so the call is
 * ordered on `stream` like any other. Sequences never interact, so every output is the
 * same as mbert_encode_padded's up to rounding; the groups' kernels overlap on the GPU. (The
 * attention kernel splits each workgroup's key tiles over two wave sets, merging their softmax
 * states, when its grid has at most 256 workgroups; a group's grid may be below that bound
 * where the whole batch's is not. Every call with the same groups gives bitwise the same
 * result.) The workspace holds one region per group: mbert_workspace_bytes_grouped() bytes.
 * n_groups is clamped to B. */
size_t mbert_workspace_bytes_grouped(const mbert_config* cfg, mbert_dtype dtype, int B, int Tpad,
                                     int n_groups);
int mbert_encode_padded_grouped(const mbert_weights* w, const int32_t* ids_pad,
                                const int32_t* mask, int B, int Tpad, int n_groups, void* ws,
                                size_t ws_bytes, float* out_pad, float* pooled,
                                void* const* streams, void* stream);

/* ---------------------------------------------------------------- graphs and timing
 * mbert_graph_capture: records mbert_encode (packed) with the given buffers into a HIP graph
 * on `stream` and instantiates it; mbert_graph_launch replays it on `stream`. The buffers
 * must stay alive and unchanged in address while the graph exists. */
typedef struct mbert_graph mbert_graph;
int mbert_graph_capture(const mbert_weights* w, const int32_t* ids, const int32_t* cu_seqlens,
                        int n_seqs, int total, void* ws, size_t ws_bytes, float* out,
                        float* pooled, void* stream, mbert_graph** graph);
int mbert_graph_capture_padded(const mbert_weights* w, const int32_t* ids_pad,
                               const int32_t* mask, int B, int Tpad, void* ws, size_t ws_bytes,
                               float* out_pad, float* pooled, void* stream, mbert_graph** graph);
/* As mbert_graph_capture_padded for mbert_encode_padded_grouped: the captured graph has one
 * branch per group. */
int mbert_graph_capture_padded_grouped(const mbert_weights* w, const int32_t* ids_pad,
                                       const int32_t* mask, int B, int Tpad, int n_groups,
                                       void* ws, size_t ws_bytes, float* out_pad, float* pooled,
                                       void* const* streams, void* stream, mbert_graph** graph);
int mbert_graph_launch(mbert_graph* graph, void* stream);
int mbert_graph_destroy(mbert_graph* graph);

/* Calibration (not part of the forward): the sustained dense MFMA rate of this GPU. Launches
 * `blocks` workgroups of 4 wave64s on `stream`; every wave runs `iters` rounds of four
 * independent 32x32 MFMA accumulations on operands held in registers (one
 * v_mfma_f32_32x32x16 per slot for bf16 / fp16: 32,768 flops; four v_mfma_f32_32x32x2_f32 per
 * slot for fp32: 16,384 flops), so the launch does blocks * 4 * iters * 4 * (flops per slot)
 * flops and its duration gives the rate.
 * `out`: device floats [blocks * 256] (written; values meaningless). Asynchronous.
 * Errors: MBERT_EINVAL for blocks outside [1, 65536], iters outside [1, 2^20] or a null
 * `out`; MBERT_EUNSUPPORTED for another dtype. */
int mbert_mfma_probe(mbert_dtype dtype, int blocks, int iters, float* out, void* stream);

/* Kernel kinds for per-kernel timing. */
#define MBERT_K_EMBED_LN 0
#define MBERT_K_LAYERNORM 1
#define MBERT_K_QKV_ROPE 2
#define MBERT_K_ATTN_GLOBAL 3
#define MBERT_K_ATTN_LOCAL 4
#define MBERT_K_WO_RESID 5
#define MBERT_K_WI_GEGLU 6
#define MBERT_K_WO2_RESID 7
#define MBERT_K_FINAL_POOL 8
#define MBERT_K_META 9
#define MBERT_K_COUNT 10

/* Per-kernel timing of an eager forward: mbert_timer_create makes an opaque recorder of
 * hipEvents (host object; no device memory); mbert_encode_timed / _padded_timed run the
 * same forward as mbert_encode / _padded and record an event pair around every launch of
 * kernel kind `kind`; mbert_timer_read synchronises on the last event and returns the number
 * of launches timed and their total milliseconds since the last reset. */
typedef struct mbert_timer mbert_timer;
int mbert_timer_create(int max_launches, mbert_timer** timer);
int mbert_timer_reset(mbert_timer* timer);
int mbert_timer_read(mbert_timer* timer, int* launches, double* total_ms);
int mbert_timer_destroy(mbert_timer* timer);
int mbert_encode_timed(const mbert_weights* w, const int32_t* ids, const int32_t* cu_seqlens,
                       int n_seqs, int total, void* ws, size_t ws_bytes, float* out,
                       float* pooled, void* stream, int kind, mbert_timer* timer);
int mbert_encode_padded_timed(const mbert_weights* w, const int32_t* ids_pad,
                              const int32_t* mask, int B, int Tpad, void* ws, size_t ws_bytes,
                              float* out_pad, float* pooled, void* stream, int kind,
                              mbert_timer* timer);

#ifdef __cplusplus
}
#endif
#endif /* MBERT_H */
