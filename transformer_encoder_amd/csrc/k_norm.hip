// Bandwidth-bound row kernels: embedding gather + LayerNorm, LayerNorm, final LayerNorm with
// pooling partial sums, pooling, standalone RoPE. One wave64 per 768-wide row: 12 elements
// per lane, read as three coalesced 4-element chunks, statistics in fp32 by wave reductions.
#include "common.hpp"

namespace mb {

// Non-temporal forms (loads and stores that do not keep the lines in the caches), for rows
// streamed once through batches far larger than the caches: the embedding LayerNorm's two
// outputs at 262,144 rows went from 5.2 to 7.1 TB/s with them (its rows also come from a table
// the caches do hold), the final LayerNorm's from 4.8 to 5.1 TB/s including its pooling.
__device__ __forceinline__ void load_row12_nt(const float* row, int lane, float v[12]) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * (lane + 64 * c)));
        v[4 * c + 0] = x[0];
        v[4 * c + 1] = x[1];
        v[4 * c + 2] = x[2];
        v[4 * c + 3] = x[3];
    }
}
template <typename T>
__device__ __forceinline__ void store_row12_nt(T* row, int lane, const float v[12]) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        if constexpr (sizeof(T) == 4) {
            const f32x4 o = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(row + 4 * (lane + 64 * c)));
        } else {
            typedef T t4 __attribute__((ext_vector_type(4)));
            const t4 o = {(T)v[4 * c], (T)v[4 * c + 1], (T)v[4 * c + 2], (T)v[4 * c + 3]};
            __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, o),
                                        reinterpret_cast<unsigned long long*>(row + 4 * (lane + 64 * c)));
        }
    }
}
// Rows from which a launch streams with non-temporal accesses (below, the outputs are left
// in L2 for the next kernel, which reads them right away).
constexpr int NT_ROWS = 16384;

template <typename T>
__device__ __forceinline__ void load_row12(const T* row, int lane, float v[12]) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const float4 x = Vec4<T>::load(row + 4 * (lane + 64 * c));
        v[4 * c + 0] = x.x;
        v[4 * c + 1] = x.y;
        v[4 * c + 2] = x.z;
        v[4 * c + 3] = x.w;
    }
}

template <typename T>
__device__ __forceinline__ void store_row12(T* row, int lane, const float v[12]) {
#pragma unroll
    for (int c = 0; c < 3; ++c)
        Vec4<T>::store(row + 4 * (lane + 64 * c),
                       make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]));
}

// The same row written through to memory as it retires (buffer stores with sc1): each store
// instruction covers whole 128-byte lines, so no dirty line is left in L2 for the write-back
// at the end of the kernel, which the next kernel would wait for.
template <typename T>
__device__ __forceinline__ void store_row12_wt(T* row, int lane, const float v[12]) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const unsigned off = (unsigned)(sizeof(T) * 4 * (lane + 64 * c));
        if constexpr (sizeof(T) == 4) {
            const f32x4 o = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
            buf_store16(__builtin_bit_cast(u32x4, o), row, D * 4, off);
        } else {
            typedef T t4 __attribute__((ext_vector_type(4)));
            const t4 o = {(T)v[4 * c], (T)v[4 * c + 1], (T)v[4 * c + 2], (T)v[4 * c + 3]};
            buf_store8b(__builtin_bit_cast(unsigned long long, o), row, D * (unsigned)sizeof(T), off);
        }
    }
}

// Weight-only LayerNorm of one row held by a wave: mean, biased variance from a second pass,
// eps inside the square root, times the weight (kgptalkie, "ModernBERT-base Architecture
// Teardown", §"What Does LayerNorm Do?"; candding, "ModernBERT", §"The pre-norm layer and the
// final norm").
template <typename TW>
__device__ __forceinline__ void layernorm12(float v[12], const TW* w, int lane, float eps) {
    float wv[12];
    load_row12(w, lane, wv);  // issued before the reductions, so its latency overlaps them
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 12; ++i) s += v[i];
    const float mean = wave_sum(s) * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        v[i] -= mean;
        q += v[i] * v[i];
    }
    const float var = wave_sum(q) * (1.0f / D);
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < 12; ++i) v[i] = v[i] * rstd * wv[i];
}

// Two rows per wave: both rows' ids in one load, both embedding rows in flight before either
// is normalised.
constexpr int EMB_R = 2;
template <typename T>
__global__ __launch_bounds__(256) void embed_ln_kernel(const int* __restrict__ ids, int total,
                                                       int* counts, const T* __restrict__ emb,
                                                       int vocab, const T* __restrict__ w,
                                                       float eps, float* __restrict__ resid,
                                                       T* __restrict__ h) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long row0 = ((long)blockIdx.x * 4 + wv) * EMB_R;
    if (row0 >= total) return;
    // lane k holds the id of row row0 + k; loaded before the device row count is known
    const int my = lane < EMB_R && row0 + lane < total ? ids[row0 + lane] : 0;
    const int nrows = rows_of(counts, total);
    if (row0 >= nrows) return;
    int id[EMB_R];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < EMB_R; ++k) {
        id[k] = __builtin_amdgcn_readlane(my, k);
        if (id[k] < 0 || id[k] >= vocab) {  // out of range: row 0, and (a real row) a status bit
            bad |= row0 + k < nrows;
            id[k] = 0;
        }
    }
    if (bad && lane == 0 && counts) atomicOr(counts + MBERT_META_STATUS, MBERT_STATUS_BAD_ID);
    float v[EMB_R][12];
#pragma unroll
    for (int k = 0; k < EMB_R; ++k) load_row12(emb + (long)id[k] * D, lane, v[k]);
    const bool nt = total >= NT_ROWS;
#pragma unroll
    for (int k = 0; k < EMB_R; ++k) {
        if (row0 + k >= nrows) break;
        layernorm12(v[k], w, lane, eps);
        float* rr = resid + (row0 + k) * D;
        T* hr = h != nullptr && (void*)h != (void*)resid ? h + (row0 + k) * D : nullptr;
        if (nt) {
            store_row12_nt(rr, lane, v[k]);
            if (hr) store_row12_nt(hr, lane, v[k]);
        } else {
            store_row12_wt(rr, lane, v[k]);
            if (hr) store_row12_wt(hr, lane, v[k]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x, int total,
                                                        const int* __restrict__ counts,
                                                        const T* __restrict__ w, float eps,
                                                        T* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows_of(counts, total)) return;
    float v[12];
    load_row12(x + row * D, lane, v);
    layernorm12(v, w, lane, eps);
    store_row12(y + row * D, lane, v);
}

// Final LayerNorm plus pooling partial sums. Work unit: one quarter of a work tile (<= 32 rows
// of one sequence), 16 waves of 2 rows each, both rows' loads in flight before either is
// normalised (16 waves of 2 rows streamed 262,144 rows 6.5 % faster than 4 waves of 8, and
// 8 waves of 4 sat between); the unit's column sums of its normalised rows are reduced over
// the waves in a fixed order into partials[(tile * FPARTS + quarter) * 768] (no atomics:
// bitwise reproducible). Rows at or past the sequence's key end (the pad rows of a padded batch run at
// full width) are written as zeros and left out of the sums.
// With `scatter`, packed row k is written to row scatter[k] of `out` (the padded output), and
// the workgroups after the LayerNorm ones write zeros to every row whose rowmap entry is
// negative (the pads): the re-pad is part of this launch. There a wave takes ZSLOTS consecutive
// slots, reads their rowmap entries with one load and zeroes the pad rows among them, so no
// wave waits on more than one load. 16 slots a wave spread the zeroing of a 4096-slot batch
// over 16 workgroups: with 64 (4 workgroups of 16 waves) the stores of the few CUs that held
// them set the launch's time (9.5 -> 19.5 us).
constexpr int FROWS = TILE / FPARTS;    // rows per workgroup
constexpr int FWAVES = 16;
constexpr int FRW = FROWS / FWAVES;     // rows per wave
constexpr int ZSLOTS = 16;              // padded-output slots a wave checks for pad rows

template <typename T>
__global__ __launch_bounds__(64 * FWAVES) void final_ln_kernel(const float* __restrict__ resid,
                                                               const int* __restrict__ meta,
                                                               int total_max, int S,
                                                               const T* __restrict__ w, float eps,
                                                               float* __restrict__ out,
                                                               float* __restrict__ partials,
                                                               int ln_blocks,
                                                               const int* __restrict__ scatter,
                                                               const int* __restrict__ rowmap,
                                                               int n_slots) {
    __shared__ float red[FWAVES][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x >= ln_blocks) {  // pad rows of the padded output
        const int r0 = (((int)blockIdx.x - ln_blocks) * FWAVES + wave) * ZSLOTS;
        if (r0 >= n_slots) return;
        unsigned long long pads =
            __ballot(lane < ZSLOTS && r0 + lane < n_slots && rowmap[r0 + lane] < 0);
        const float z[12] = {};
        while (pads) {  // wave-uniform
            const int j = __builtin_ctzll(pads);
            pads &= pads - 1;
            store_row12(out + (long)(r0 + j) * D, lane, z);
        }
        return;
    }
    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    const int b = blockIdx.x / FPARTS, q = blockIdx.x % FPARTS;
    // the tile entry (b < tiles_max: in bounds) is read beside the tile count, not after it;
    // a real tile never has fewer than one row, so the second test only keeps both loads
    // ahead of the branch
    const int4 tl = mv.tiles[b];
    if ((b >= mv.counts[MBERT_META_NTILES]) | (tl.y < 1)) return;
    const int r0 = q * FROWS;
    if (r0 >= tl.y) {  // an empty quarter still leaves its (zero) partial sums
        if (partials)
            for (int col = threadIdx.x; col < D; col += 64 * FWAVES) partials[(long)blockIdx.x * D + col] = 0.f;
        return;
    }
    const int real = min(tl.y, tl.w - tl.x);
    const bool nt = total_max >= NT_ROWS;
    float v[FRW][12];
    long dst[FRW];  // output rows, loaded with the input rows
#pragma unroll
    for (int k = 0; k < FRW; ++k) {
        const int r = tl.x + min(r0 + wave + FWAVES * k, tl.y - 1);
        if (nt) load_row12_nt(resid + (long)r * D, lane, v[k]);
        else load_row12(resid + (long)r * D, lane, v[k]);
        dst[k] = scatter ? (long)scatter[r] : (long)r;
    }
    float acc[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < FRW; ++k) {
        const int r = r0 + wave + FWAVES * k;
        if (r >= tl.y) break;
        if (r < real) {
            layernorm12(v[k], w, lane, eps);
#pragma unroll
            for (int i = 0; i < 12; ++i) acc[i] += v[k][i];
        } else {
#pragma unroll
            for (int i = 0; i < 12; ++i) v[k][i] = 0.f;
        }
        if (nt) store_row12_nt(out + dst[k] * D, lane, v[k]);
        else store_row12(out + dst[k] * D, lane, v[k]);
    }
    if (partials == nullptr) return;
#pragma unroll
    for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][4 * (lane + 64 * c) + e] = acc[4 * c + e];
    __syncthreads();
    for (int col = threadIdx.x; col < D; col += 64 * FWAVES) {
        float sum = 0.f;
#pragma unroll
        for (int qq = 0; qq < FWAVES; ++qq) sum += red[qq][col];
        partials[(long)blockIdx.x * D + col] = sum;
    }
}

// Mean over the sequence from the tile partials, then L2 normalisation (kgptalkie, §"How Do We
// Get One Vector per Text?"; safebydesign, "ModernBertModel 22L 768d", §"Implementing it":
// normalize(pool(x))). An empty sequence pools to zero. Four groups of 256 threads: group g
// sums partial rows g, g + 4, g + 8, ... of the sequence (each thread three columns, batches of
// 8 rows in flight), then the four group sums are added in group order: a fixed order, so the
// result is bitwise reproducible.
constexpr int POOL_GROUPS = 4;
static_assert(POOL_GROUPS == 4, "the group sums are added as four terms");
__global__ __launch_bounds__(256 * POOL_GROUPS) void pool_kernel(const int* __restrict__ meta,
                                                                 int total_max, int S,
                                                                 const float* __restrict__ partials,
                                                                 float* __restrict__ pooled,
                                                                 int normalize) {
    __shared__ float gsum[POOL_GROUPS][D];
    __shared__ float red[4];
    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    const int s = blockIdx.x;
    const int t0 = mv.seq_tile0[s], t1 = mv.seq_tile0[s + 1];
    const int L = t1 > t0 ? mv.tiles[t0].w - mv.tiles[t0].z : 0;
    const int g = threadIdx.x >> 8, ct = threadIdx.x & 255;
    const long base = (long)t0 * FPARTS;
    const int n = (t1 - t0) * FPARTS;
    constexpr int PB = 8;
    float acc[3] = {0.f, 0.f, 0.f};
    for (int j0 = g; j0 < n; j0 += POOL_GROUPS * PB) {
        float x[PB][3];
#pragma unroll
        for (int j = 0; j < PB; ++j)
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const int r = j0 + POOL_GROUPS * j;
                x[j][c] = r < n ? partials[(base + r) * D + ct + 256 * c] : 0.f;
            }
#pragma unroll
        for (int j = 0; j < PB; ++j)
#pragma unroll
            for (int c = 0; c < 3; ++c) acc[c] += x[j][c];
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) gsum[g][ct + 256 * c] = acc[c];
    __syncthreads();
    float m[3];
    if (g == 0) {
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const int col = ct + 256 * c;
            const float t = ((gsum[0][col] + gsum[1][col]) + gsum[2][col]) + gsum[3][col];
            m[c] = L > 0 ? t / (float)L : 0.f;
            sq += m[c] * m[c];
        }
        sq = wave_sum(sq);
        if ((ct & 63) == 0) red[ct >> 6] = sq;
    }
    __syncthreads();
    if (g != 0) return;
    const float nrm = sqrtf(((red[0] + red[1]) + red[2]) + red[3]);
    const float inv = normalize ? 1.0f / fmaxf(nrm, 1e-12f) : 1.0f;
#pragma unroll
    for (int c = 0; c < 3; ++c) pooled[(long)s * D + ct + 256 * c] = m[c] * inv;
}

// Column sums of already-normalised rows (the mean pooling of a finished forward), per quarter
// work tile and in the same fixed order as the final-norm kernel's partials.
__global__ __launch_bounds__(64 * FWAVES) void colsum_kernel(const float* __restrict__ out,
                                                             const int* __restrict__ meta,
                                                             int total_max, int S,
                                                             float* __restrict__ partials) {
    __shared__ float red[FWAVES][D];
    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    const int b = blockIdx.x / FPARTS, q = blockIdx.x % FPARTS;
    if (b >= mv.counts[MBERT_META_NTILES]) return;
    const int4 tl = mv.tiles[b];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) acc[i] = 0.f;
    for (int r = q * FROWS + wave; r < min(tl.y, (q + 1) * FROWS); r += FWAVES) {
        float v[12];
        load_row12(out + (long)(tl.x + r) * D, lane, v);
#pragma unroll
        for (int i = 0; i < 12; ++i) acc[i] += v[i];
    }
#pragma unroll
    for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][4 * (lane + 64 * c) + e] = acc[4 * c + e];
    __syncthreads();
    for (int col = threadIdx.x; col < D; col += 64 * FWAVES) {
        float sum = 0.f;
#pragma unroll
        for (int qq = 0; qq < FWAVES; ++qq) sum += red[qq][col];
        partials[(long)blockIdx.x * D + col] = sum;
    }
}

// CLS pooling: the first row of each sequence (candding, "ModernBERT", §"Pooling and
// normalization": index 0), optionally divided by max(L2 norm, 1e-12); an empty sequence
// pools to zero. One wave per sequence.
__global__ __launch_bounds__(256) void cls_kernel(const float* __restrict__ out,
                                                  const int* __restrict__ meta, int total_max,
                                                  int S, float* __restrict__ pooled,
                                                  int normalize) {
    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (s >= S) return;
    const int t0 = mv.seq_tile0[s], t1 = mv.seq_tile0[s + 1];
    float v[12];
    if (t1 > t0) {
        load_row12(out + (long)mv.tiles[t0].z * D, lane, v);
    } else {
#pragma unroll
        for (int i = 0; i < 12; ++i) v[i] = 0.f;
    }
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 12; ++i) sq += v[i] * v[i];
    sq = wave_sum(sq);
    const float inv = normalize ? 1.0f / fmaxf(sqrtf(sq), 1e-12f) : 1.0f;
#pragma unroll
    for (int i = 0; i < 12; ++i) v[i] *= inv;
    store_row12(pooled + (long)s * D, lane, v);
}

// Standalone rotate-half RoPE on the query and key columns of one qkv row per workgroup
// (candding, "ModernBERT", §"The two rope tables").
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ qkv, int total,
                                                   const int* __restrict__ meta,
                                                   const float2* __restrict__ tab, int max_pos) {
    const long row = blockIdx.x;
    if (row >= rows_of(meta, total)) return;
    const int p = min(max(meta[8 + row], 0), max_pos - 1);  // pos follows the 8 counts
    T* r = qkv + row * QKV;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const int j = threadIdx.x + 256 * c;  // 24 heads (q then k) x 32 pairs
        const int i = j & 31;
        const int col = (j >> 5) * HD + i;
        const float2 cs = tab[(long)p * (HD / 2) + i];
        const float x1 = to_f(r[col]), x2 = to_f(r[col + 32]);
        r[col] = from_f<T>(x1 * cs.x - x2 * cs.y);
        r[col + 32] = from_f<T>(x2 * cs.x + x1 * cs.y);
    }
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_embed_ln(mbert_dtype dt, const int32_t* ids, int total, const int32_t* meta,
                    const void* emb, int vocab, const void* w, float eps, float* resid, void* h,
                    hipStream_t s) {
    if (total == 0) return MBERT_OK;
    const unsigned grid = (unsigned)((total + 4 * EMB_R - 1) / (4 * EMB_R));
    int* counts = const_cast<int*>(meta);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((embed_ln_kernel<float>), grid, 256, 0, s, ids, total, counts, (const float*)emb, vocab,
                                                        (const float*)w, eps, resid, (float*)h);
            break;
        case MBERT_BF16:
            MB_LAUNCH((embed_ln_kernel<bf16>), grid, 256, 0, s, ids, total, counts, (const bf16*)emb, vocab,
                                                       (const bf16*)w, eps, resid, (bf16*)h);
            break;
        case MBERT_F16:
            MB_LAUNCH((embed_ln_kernel<f16>), grid, 256, 0, s, ids, total, counts, (const f16*)emb, vocab,
                                                      (const f16*)w, eps, resid, (f16*)h);
            break;
        default:
            return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_layernorm(mbert_dtype dt, const float* x, int total, const int32_t* meta,
                     const void* w, float eps, void* y, hipStream_t s) {
    if (total == 0) return MBERT_OK;
    const unsigned grid = (unsigned)((total + 3) / 4);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((layernorm_kernel<float>), grid, 256, 0, s, x, total, meta, (const float*)w, eps, (float*)y);
            break;
        case MBERT_BF16:
            MB_LAUNCH((layernorm_kernel<bf16>), grid, 256, 0, s, x, total, meta, (const bf16*)w, eps, (bf16*)y);
            break;
        case MBERT_F16:
            MB_LAUNCH((layernorm_kernel<f16>), grid, 256, 0, s, x, total, meta, (const f16*)w, eps, (f16*)y);
            break;
        default:
            return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_final_ln_pool(const float* resid, int total, const int32_t* meta, int n_seqs,
                         mbert_dtype dt, const void* w, float eps, float* out, float* pooled,
                         float* partials, hipStream_t s, const int32_t* scatter,
                         const int32_t* rowmap, int n_slots) {
    const size_t tmax = tiles_max_for(total, n_seqs);
    const int ln_blocks = (int)tmax * FPARTS;
    // pad rows of the padded output: a wave per ZSLOTS slots
    const int zero_blocks =
        (scatter && n_slots > 0) ? (n_slots + ZSLOTS * FWAVES - 1) / (ZSLOTS * FWAVES) : 0;
    const unsigned grid = (unsigned)(ln_blocks + zero_blocks);
    if (grid > 0) {
        float* part = pooled ? partials : nullptr;
        switch (dt) {
            case MBERT_F32:
                MB_LAUNCH((final_ln_kernel<float>), grid, 64 * FWAVES, 0, s, resid, meta, total, n_seqs,
                          (const float*)w, eps, out, part, ln_blocks, scatter, rowmap, n_slots);
                break;
            case MBERT_BF16:
                MB_LAUNCH((final_ln_kernel<bf16>), grid, 64 * FWAVES, 0, s, resid, meta, total, n_seqs,
                          (const bf16*)w, eps, out, part, ln_blocks, scatter, rowmap, n_slots);
                break;
            case MBERT_F16:
                MB_LAUNCH((final_ln_kernel<f16>), grid, 64 * FWAVES, 0, s, resid, meta, total, n_seqs,
                          (const f16*)w, eps, out, part, ln_blocks, scatter, rowmap, n_slots);
                break;
            default:
                return MBERT_EUNSUPPORTED;
        }
        MB_CHECK_LAUNCH();
    }
    if (pooled && n_seqs > 0) {
        MB_LAUNCH((pool_kernel), n_seqs, 256 * POOL_GROUPS, 0, s, meta, total, n_seqs, partials, pooled, 1);
        MB_CHECK_LAUNCH();
    }
    return MBERT_OK;
}

int launch_rope(mbert_dtype dt, void* qkv, int total, const int32_t* meta, const float* rope,
                int max_pos, int table, hipStream_t s) {
    if (total == 0) return MBERT_OK;
    const float2* tab = reinterpret_cast<const float2*>(rope) + (size_t)table * max_pos * (HD / 2);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((rope_kernel<float>), total, 256, 0, s, (float*)qkv, total, meta, tab, max_pos);
            break;
        case MBERT_BF16:
            MB_LAUNCH((rope_kernel<bf16>), total, 256, 0, s, (bf16*)qkv, total, meta, tab, max_pos);
            break;
        case MBERT_F16:
            MB_LAUNCH((rope_kernel<f16>), total, 256, 0, s, (f16*)qkv, total, meta, tab, max_pos);
            break;
        default:
            return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

}  // namespace mbh

namespace mbh {
using namespace mb;

int launch_pool(const float* out, int total, const int32_t* meta, int n_seqs, int mode,
                float* pooled, float* partials, hipStream_t s) {
    if (n_seqs == 0) return MBERT_OK;
    const int normalize = (mode & MBERT_POOL_L2) != 0;
    if ((mode & 1) == MBERT_POOL_CLS) {
        MB_LAUNCH((cls_kernel), (n_seqs + 3) / 4, 256, 0, s, out, meta, total, n_seqs, pooled, normalize);
        MB_CHECK_LAUNCH();
        return MBERT_OK;
    }
    const size_t tmax = tiles_max_for(total, n_seqs);
    if (tmax > 0) {
        MB_LAUNCH((colsum_kernel), (unsigned)(tmax * FPARTS), 64 * FWAVES, 0, s, out, meta, total, n_seqs,
                  partials);
        MB_CHECK_LAUNCH();
    }
    MB_LAUNCH((pool_kernel), n_seqs, 256 * POOL_GROUPS, 0, s, meta, total, n_seqs, partials, pooled, normalize);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}
}  // namespace mbh
