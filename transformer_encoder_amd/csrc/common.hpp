// Shared device-side definitions for the gfx950 ModernBERT-base encoder kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mbert.h"

namespace mb {

// ModernBERT-base shapes the kernels are specialised to (kgptalkie, "ModernBERT-base
// Architecture Teardown", §"What Is ModernBERT-base?").
constexpr int D = 768;        // hidden width
constexpr int NH = 12;        // heads
constexpr int HD = 64;        // head width
constexpr int FF = 1152;      // GeGLU intermediate width
constexpr int QKV = 3 * D;    // fused projection width
constexpr int TILE = 128;     // query rows per attention / pooling work tile
constexpr int FPARTS = 4;     // pooling partial sums per work tile (one per 32 rows)
constexpr int NXCD = 8;       // accelerator complex dies on MI355X

typedef __bf16 bf16;
typedef _Float16 f16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- wait counts, LDS DMA
// s_waitcnt immediates (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// wait until at most n vector-memory operations are outstanding / until LDS operations drain.
constexpr unsigned vmcnt_imm(int n) {
    return (unsigned)(n & 15) | ((unsigned)((n >> 4) & 3) << 14) | (7u << 4) | (15u << 8);
}
constexpr unsigned lgkmcnt0_imm() { return 63u | (3u << 14) | (7u << 4); }

// 16 bytes per lane from global memory straight into LDS through a buffer load (MUBUF, offset
// = voff + soff from an SGPR base): lane i's bytes land at lds + 16 i (lds is the same for the
// whole wave). A buffer load, not a global (FLAT) one: after a FLAT load into LDS the compiler
// waits for every LDS operation before any use, with this one its LDS wait counts stay exact.
// The builtin exists only for the device target; the host pass, which never runs this, would
// otherwise drop every kernel that uses it.
__device__ __forceinline__ void lds_dma16_buf(const void* base, unsigned extent, unsigned voff,
                                              unsigned soff, unsigned char* lds) {
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, extent, 0x00020000),
        (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

// ---------------------------------------------------------------- buffer stores
// Stores through a buffer descriptor (base, extent in bytes): a store at or beyond the extent
// is dropped by the hardware, so rows past the end need no branch (a branch around a store
// leaves the compiler unsure how many stores are in flight, and it then waits for all).
// The stores carry the device-scope coherence bit (sc1): they are written through the XCD's
// L2 as they retire, rather than left dirty there for the end-of-kernel write-back, which
// otherwise delays the next kernel (0.6 % per forward on a 2445-token batch when the GEMM
// epilogues use it). Only for stores whose lanes cover whole 128-byte lines: the attention
// output's 16-byte row pieces, written through, made the forward 2.7 % slower.
constexpr int STORE_CPOL = 16;  // sc1
__device__ __forceinline__ void buf_store8b(unsigned long long v, const void* base, unsigned extent,
                                            unsigned off) {
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_raw_buffer_store_b64(
        __builtin_bit_cast(u32x2, v),
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, extent, 0x00020000),
        off, 0, STORE_CPOL);
#endif
}
__device__ __forceinline__ void buf_store16(u32x4 v, const void* base, unsigned extent, unsigned off) {
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_raw_buffer_store_b128(
        v, __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, extent, 0x00020000),
        off, 0, STORE_CPOL);
#endif
}

// ---------------------------------------------------------------- element conversion
template <typename T> __device__ __forceinline__ float to_f(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return static_cast<T>(x); }

// Four consecutive elements <-> float4 (8-byte loads for 16-bit types, 16-byte for fp32).
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    typedef float4 raw;
    __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct Vec4<bf16> {
    __device__ static float4 load(const bf16* p) {
        bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
        return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    }
    __device__ static void store(bf16* p, float4 v) {
        bf16x4 o = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
        *reinterpret_cast<bf16x4*>(p) = o;
    }
};
template <> struct Vec4<f16> {
    __device__ static float4 load(const f16* p) {
        f16x4 v = *reinterpret_cast<const f16x4*>(p);
        return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    }
    __device__ static void store(f16* p, float4 v) {
        f16x4 o = {(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
        *reinterpret_cast<f16x4*>(p) = o;
    }
};

// ---------------------------------------------------------------- wave reductions (wave64)
// Sum over the 64 lanes, the same value in every lane, in a fixed order. Within each row of
// 16 lanes the data-parallel-primitive (DPP) lane swaps run on the VALU: swap neighbours, swap
// pairs, mirror within 8, mirror within 16; the four row sums are then read as scalars and
// added in row order.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return ((r0 + r1) + r2) + r3;
}

// ---------------------------------------------------------------- work distribution
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Remap the
// hardware id so that each XCD receives one contiguous range of logical tiles: neighbouring
// tiles share operands (the same activation rows, the same head's keys), so they hit in the
// same L2. `n` is the grid size; ids at or beyond n never occur.
__device__ __forceinline__ int xcd_remap(int hw_id, int n) {
    const int per = (n + NXCD - 1) / NXCD;
    const int xcd = hw_id % NXCD;
    const int local = hw_id / NXCD;
    return xcd * per + local;  // may be >= n when n % 8 != 0: the caller returns early
}
__host__ __device__ inline int xcd_grid(int n) { return ((n + NXCD - 1) / NXCD) * NXCD; }

// ---------------------------------------------------------------- the attention band
// Keys a query may read, inclusive [lo, hi], as packed token indices: the whole sequence
// [s0, s1) on a global layer, |i - j| <= W clipped to the sequence on a local layer
// (candding, "ModernBERT", §"The alternating attention"). Shared by the attention kernel
// and the key-range debug kernel so the band can be checked exactly.
__device__ __forceinline__ void key_range(int q, int s0, int s1, int is_global, int W,
                                          int& lo, int& hi) {
    if (is_global) {
        lo = s0;
        hi = s1 - 1;
    } else {
        lo = max(s0, q - W);
        hi = min(s1 - 1, q + W);
    }
}

// Meta buffer offsets (see mbert.h).
struct MetaView {
    int* counts;
    int* seq_tile0;
    int4* tiles;
    int* pos;
    int* order;  // the attention's dispatch order of the tiles (a permutation of [0, n_tiles))
};
__host__ __device__ inline size_t tiles_max_for(int total_max, int n_seqs) {
    return (size_t)((total_max + TILE - 1) / TILE) + (size_t)n_seqs;
}
__host__ __device__ inline MetaView meta_view(int* meta, int total_max, int n_seqs) {
    MetaView v;
    v.counts = meta;
    v.pos = meta + 8;
    v.seq_tile0 = meta + 8 + total_max;
    size_t off = 8 + (size_t)total_max + (size_t)n_seqs + 1;
    off = (off + 3) & ~(size_t)3;  // 16-byte alignment for int4 tiles
    v.tiles = reinterpret_cast<int4*>(meta + off);
    v.order = meta + off + 4 * tiles_max_for(total_max, n_seqs);
    return v;
}
__host__ __device__ inline size_t meta_ints(int total_max, int n_seqs) {
    size_t off = 8 + (size_t)total_max + (size_t)n_seqs + 1;
    off = (off + 3) & ~(size_t)3;
    return off + 5 * tiles_max_for(total_max, n_seqs);
}

// Rows to process: the device count when a meta buffer is given, else the host count.
__device__ __forceinline__ int rows_of(const int* counts, int total) {
    return counts ? min(total, counts[MBERT_META_TOTAL]) : total;
}

}  // namespace mb

// Host-side launch helpers (defined in the .hip files; called by api.cpp).
namespace mbh {
using mbert_dtype_t = mbert_dtype;
int launch_rope_tables(float* table, int max_pos, double theta_g, double theta_l, hipStream_t s);
int launch_pack_meta(const int32_t* cu, int n_seqs, int total, int max_pos, int32_t* meta,
                     hipStream_t s);
int launch_unpad(const int32_t* ids_pad, const int32_t* mask, int B, int Tpad, int max_pos,
                 int32_t* ids, int32_t* indices, int32_t* rowmap, int32_t* cu, int32_t* meta,
                 hipStream_t s);
int launch_key_ranges(const int32_t* meta, int total_max, int n_seqs, int is_global, int W,
                      int32_t* lo, int32_t* hi, hipStream_t s);
int launch_repad(const float* out, const int32_t* rowmap, int B, int Tpad, float* out_pad,
                 hipStream_t s);
int launch_embed_ln(mbert_dtype dt, const int32_t* ids, int total, const int32_t* meta,
                    const void* emb, int vocab, const void* w, float eps, float* resid, void* h,
                    hipStream_t s);
int launch_layernorm(mbert_dtype dt, const float* x, int total, const int32_t* meta,
                     const void* w, float eps, void* y, hipStream_t s);
// Pooling of finished rows: mode = MBERT_POOL_MEAN or MBERT_POOL_CLS, | MBERT_POOL_L2.
int launch_pool(const float* out, int total, const int32_t* meta, int n_seqs, int mode,
                float* pooled, float* partials, hipStream_t s);
// out (fp32 [M, N]) = gelu(a . W^T) (gelu != 0) or a . W^T + bias; K = 768, N % 64 == 0.
int launch_linear_f32(mbert_dtype dt, const void* a, int M, const void* W, int N, int K, int gelu,
                      const void* bias, float* out, hipStream_t s);
int launch_gather_cast(mbert_dtype dt, const float* x, int total, const int32_t* rows, int R,
                       void* out, hipStream_t s);
int launch_small_linear(mbert_dtype dt, const void* h, const void* W, const void* b, int S, int C,
                        float* out, hipStream_t s);
// Meta of a padded batch run at full width: B sequences of Tpad rows, keys cut at L_b.
int launch_padded_meta(const int32_t* mask, int B, int Tpad, int max_pos, int32_t* meta,
                       hipStream_t s);
int launch_attention_probs(mbert_dtype dt, const void* qkv, int row0, int n_q, int n_k,
                           int is_global, int W, float* probs, hipStream_t s);
// Final LayerNorm (+ pooling partials and mean pooling when pooled != NULL). With `scatter`,
// packed row k goes to row scatter[k] of `out` and the n_slots rows whose rowmap entry is
// negative are zeroed in the same launch (the padded output written directly).
int launch_final_ln_pool(const float* resid, int total, const int32_t* meta, int n_seqs,
                         mbert_dtype dt, const void* w, float eps, float* out, float* pooled,
                         float* partials, hipStream_t s, const int32_t* scatter = nullptr,
                         const int32_t* rowmap = nullptr, int n_slots = 0);
// A LayerNorm folded into the GEMM that follows it: the A operand is the raw residual (in
// dtype; the fp32 residual itself for MBERT_F32), W is the folded weight (W o w), and the
// epilogue applies rstd * (acc - mean * c) from the producer's chunk statistics.
struct FoldArgs {
    const float* c;        // [rows of W]
    const float2* stats;   // [rows][12] {mean, M2} per 64-column chunk
    float eps;
};
int launch_mfma_probe(mbert_dtype dt, int blocks, int iters, float* out, hipStream_t s);
// GEMM launches take their row count from meta's device count unless host_rows is set: then
// total is exact (a packed batch, whose meta count is total itself) and the kernels start
// without loading the count first.
int launch_qkv(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* W,
               const float* rope, int max_pos, int table, int apply_rope, void* qkv,
               hipStream_t s, const FoldArgs* fold = nullptr, bool host_rows = false);
// Folded weight of one norm: Wf [rows,768] = W o w rounded to dtype, c [rows] = row sums of Wf.
int launch_fold_weight(mbert_dtype dt, const void* W, const void* w, int rows, void* Wf,
                       float* c, hipStream_t s);
int launch_rope(mbert_dtype dt, void* qkv, int total, const int32_t* meta, const float* rope,
                int max_pos, int table, hipStream_t s);
// With stats_out, the residual epilogue also writes the new residual's chunk statistics and
// (xs_out, 16-bit types) the residual rounded to dtype, for a folded LayerNorm next.
int launch_linear_residual(mbert_dtype dt, const void* a, int K, int total, const int32_t* meta,
                           const void* W, float* resid, hipStream_t s, void* xs_out = nullptr,
                           float2* stats_out = nullptr, bool host_rows = false);
int launch_geglu(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* Wi,
                 void* m, hipStream_t s, const FoldArgs* fold = nullptr, bool host_rows = false);
int launch_attention(mbert_dtype dt, const void* qkv, int total, const int32_t* meta, int n_seqs,
                     int is_global, int W, void* o, hipStream_t s);
}  // namespace mbh

// Per-kernel timing: while a timer slot is armed on this thread (the *_timed entry points),
// launches carry its start / stop events on the kernel dispatch itself
// (hipExtLaunchKernelGGL), so the elapsed time is the kernels' own, without the launch gap an
// event recorded before the launch would add. The first launch takes the start event; every
// launch takes the stop event, so a step of several kernels is timed from the first to the
// last.
namespace mb {
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();
}  // namespace mb

// A launch first clears the thread's HIP error state, so that MB_CHECK_LAUNCH reports this
// launch's error and not one left behind by an unrelated earlier HIP call of the caller.
#define MB_LAUNCH(kernel, grid, block, shmem, stream, ...)                                    \
    do {                                                                                      \
        (void)hipGetLastError();                                                              \
        ::mb::LaunchEvents& ev_ = ::mb::launch_events();                                      \
        if (ev_.stop != nullptr) {                                                            \
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), shmem, stream, ev_.start,  \
                                  ev_.stop, 0, __VA_ARGS__);                                  \
            ev_.start = nullptr;                                                              \
        } else {                                                                              \
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), shmem, stream, __VA_ARGS__);  \
        }                                                                                     \
    } while (0)

#define MB_CHECK_LAUNCH()                                   \
    do {                                                    \
        if (hipGetLastError() != hipSuccess) return MBERT_EHIP; \
    } while (0)
