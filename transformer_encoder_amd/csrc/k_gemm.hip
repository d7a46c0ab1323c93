// MFMA GEMM for the encoder's four projections: C[M, N] = A[M, K] . B[N, K]^T, both operands
// K-contiguous (activations row-major, Linear weights stored [out, in]), fp32 accumulation.
//
// Main loop: 4 (or 8) wave64s in a 2x2 (2x4) arrangement; each wave owns a sub-tile made of
// 32x32 MFMA blocks (v_mfma_f32_32x32x16_{bf16,f16}; fp32 inputs use v_mfma_f32_32x32x2_f32,
// four per 16-byte operand). K is consumed 128 bytes at a time (64 16-bit or 32 fp32
// elements; 64 bytes is a compile-time option); K is only 768 or 1152, so a workgroup's whole
// life is a dozen K-steps and the load latency has to be covered by loads in flight, not by a
// long loop. Operand tiles go from global memory straight into LDS (buffer loads with the LDS
// destination, 16 bytes per lane) into DS stages, with explicit wait counts and one raw
// barrier per K-step. LDS rows are unpadded and XOR-swizzled by 16-byte chunk (see lds_off),
// which keeps the 16-byte operand reads conflict-free. The fragment reads are software-
// pipelined: those of k-substep s + 1 are issued before (or between) the MFMAs of substep s.
//
// Epilogue: the fp32 accumulator tile is staged through LDS (row pitch BN + 8 floats, which
// keeps the two half-waves of an MFMA block on disjoint banks) and then processed row-major,
// so every global access is a coalesced 16-byte vector:
//   STORE : C (dtype) = acc
//   ROPE  : query/key columns rotated rotate-half style at each row's position, then stored
//           (candding, "ModernBERT", §"The two rope tables"); one position load per row and
//           contiguous {cos, sin} reads from the float64-built table
//   RESID : resid (fp32) += acc (kgptalkie, §"What Does LayerNorm Do?": the block output is
//           added back to its input)
//   GEGLU : m = gelu_erf(u_gate) * u_mult; the B tile takes BN/2 rows from the GELU-branch
//           half of Wi and the same BN/2 rows of the multiplier half, so the pair of every
//           output column sits in one tile (candding, §"The feed-forward halves").
//   GELU_F32 / BIAS_F32 : C (fp32, row pitch N) = gelu_erf(acc) or acc + bias[col], the dense
//           layer of the prediction head and the biased decoder / classifier Linear
//           (kgptalkie, §"The Masked-LM Head")
// Epilogues that read memory issue all their loads first, from rows clamped into range, and
// each pass issues the next pass's loads before its own stores; stores go through buffer
// descriptors that drop rows past the end. With a folded LayerNorm (cfold / stats_in) the
// output is rstd * (acc - mean * c): the accumulators start at -mean * c (set while the first
// operand stage lands) and the epilogue scales them by rstd; the residual epilogue can also
// write the new residual's chunk statistics and its dtype copy for the next such GEMM.
// Work distribution: tiles are spread over the 8 XCDs in contiguous ranges counted from the
// real row count read on the device (the padded path sizes its grid for B * Tpad rows). The
// 256x256 tiles of the QKV and Wi GEMMs are persistent: one workgroup per CU walks its XCD's
// tile slots and issues the next tile's loads during the current tile's epilogue.
#include "common.hpp"

// Operand staging: the number of LDS stages per tile shape (two for the 2304-wide GEMMs, three
// for the 768-wide ones, measured on whole forwards of the padded batch-8 workload; deeper
// stages or 64-byte K-steps were slower at 1k-262k rows).
#ifndef MB_GEMM_DMA
#define MB_GEMM_DMA 2
#endif
#ifndef MB_GEMM_DMA_N768
#define MB_GEMM_DMA_N768 3
#endif
#ifndef MB_GEMM_MID_DS
#define MB_GEMM_MID_DS MB_GEMM_DMA
#endif
#ifndef MB_GEMM_MID_OCC
#define MB_GEMM_MID_OCC 2
#endif
#ifndef MB_GEMM_MID_RB
#define MB_GEMM_MID_RB 128
#endif
#ifndef MB_GEMM_SMALL_DS
#define MB_GEMM_SMALL_DS MB_GEMM_DMA
#endif
#ifndef MB_GEMM_SMALL_OCC
#define MB_GEMM_SMALL_OCC 3
#endif
#ifndef MB_GEMM_SMALL_RB
#define MB_GEMM_SMALL_RB 128
#endif
#ifndef MB_GEMM_N768_OCC
#define MB_GEMM_N768_OCC 4
#endif
#ifndef MB_GEMM_N768_RB
#define MB_GEMM_N768_RB 128
#endif
#ifndef MB_GEMM_BIG_DS
#define MB_GEMM_BIG_DS 2
#endif
#ifndef MB_GEMM_BIG_RB
#define MB_GEMM_BIG_RB 128
#endif
// 32-row block-rows of each wave staged per epilogue pass on non-persistent 256x256 QKV and
// Wi tiles (the persistent layout has no LDS for it): two passes of 128 rows instead of four
// of 64, half the barriers and twice the independent work between them.
#ifndef MB_GEMM_EPB
#define MB_GEMM_EPB 2
#endif
// Persistent 256x256 tiles: one workgroup per CU takes its XCD's tile slots in turn and issues
// the next tile's row statistics, positions and first K-step while the current tile's
// epilogue runs (the epilogue then stages in four passes, above the first operand stage).
#ifndef MB_GEMM_PERSIST
#define MB_GEMM_PERSIST 1
#endif
#ifndef MB_GEMM_BIG_MIN_TILES
#define MB_GEMM_BIG_MIN_TILES 512
#endif
#ifndef MB_GEMM_SMALL_MAX_TILES
#define MB_GEMM_SMALL_MAX_TILES 1024
#endif

namespace mb {

enum { EPI_STORE = 0, EPI_ROPE = 1, EPI_RESID = 2, EPI_GEGLU = 3, EPI_GELU_F32 = 4, EPI_BIAS_F32 = 5 };


struct GemmArgs {
    const void* A;       // [M, K] dtype
    const void* B;       // [N, K] dtype
    int M;               // host row bound (grid size)
    const int* counts;   // device row count (meta counts) or null
    int K;               // 768 or 1152
    int N;               // rows of B that this GEMM uses
    void* C;             // STORE/ROPE: dtype [M, N]; RESID: f32 [M, 768]; GEGLU: dtype [M, N/2]
    const int* pos;      // ROPE: positions [M]
    const float2* rope;  // ROPE: {cos, sin} table [max_pos][32] of the layer kind
    int max_pos;
    const void* bias;    // BIAS_F32: [N] dtype
    // LayerNorm folded into this GEMM (STORE / ROPE / GEGLU): A holds the raw residual in
    // dtype and B the weight with its columns scaled by the norm weight, W o w; the output is
    // rstd * (acc - mean * cfold[col]), mean and rstd merged from stats_in. Off when null.
    const float* cfold;      // [rows of B] sums over k of (W o w)[row][k]
    const float2* stats_in;  // [M][NCHUNK] {mean, M2} of each 64-column chunk of each row
    float eps;
    // RESID extras: the new residual rounded to dtype (xs_out, [M, 768], may be null) and its
    // per-chunk statistics (stats_out) for the next folded GEMM. Off when stats_out is null.
    void* xs_out;
    float2* stats_out;
};

template <typename T> struct MfmaOp;
template <> struct MfmaOp<bf16> {
    __device__ __forceinline__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<f16> {
    __device__ __forceinline__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaOp<float> {
    __device__ __forceinline__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
        const f32x4 av = __builtin_bit_cast(f32x4, a), bv = __builtin_bit_cast(f32x4, b);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[3], bv[3], c, 0, 0, 0);
    }
};

// Barrier for LDS reuse only: waits for this wave's LDS operations, not for its global stores
// (__syncthreads would also wait for every store in flight, serialising the epilogue passes).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The erf form of GELU, z * Phi(z) with Phi(z) = (1 + erf(z / sqrt 2)) / 2 (candding, §"The
// feed-forward halves"; not the tanh form). erfc(x), x >= 0, comes from the rational-exponential
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (|error| <= 1.5e-7): erfc(x) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x). For either sign of z, z Phi(z) = max(z, 0) - |z| erfc(|z| / sqrt 2) / 2,
// which needs no select; the halving sits in the coefficients (a_i / 2) and exp(-x^2) is
// exp2(z * (z * -log2(e) / 2)). The result is within 3.3e-7 of the exact GELU in float32 over
// all z (the direct form Phi = 1 - erfc / 2 or erfc / 2 by sign: 4.3e-7, three more operations).
__device__ __forceinline__ float gelu_erf(float z) {
    const float x = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
    float q = fmaf(t, 0.5307027145f, -0.7265760135f);
    q = fmaf(t, q, 0.7107068705f);
    q = fmaf(t, q, -0.142248368f);
    q = fmaf(t, q, 0.127414796f);
    const float h = q * t * __builtin_amdgcn_exp2f(z * (z * -0.7213475204444817f));
    return fmaf(-fabsf(z), h, fmaxf(z, 0.0f));
}

// Tiles over the 8 XCDs (each with its own L2): the (row-tile, column-tile) grid is cut into
// a x b blocks, a * b = 8, one block per XCD, so an XCD fetches only its rows of A and its
// columns of B. The split balances tiles per XCD first, then minimises the bytes the XCDs
// fetch between them, proportional to M/a + N/b (K is common). Within a block, consecutive
// workgroups share rows of A.
__host__ __device__ inline void xcd_split(int nbm, int nbn, int M, int N, int& a, int& bmper,
                                          int& bnper) {
    int best_tiles = 0x7fffffff;
    long best_bytes = 0x7fffffffffffL;
    a = NXCD;
    for (int aa = NXCD; aa >= 1; aa >>= 1) {
        const int bb = NXCD / aa;
        const int tiles = ((nbm + aa - 1) / aa) * ((nbn + bb - 1) / bb);
        const long bytes = (long)M / aa + (long)N / bb;
        if (tiles < best_tiles || (tiles == best_tiles && bytes < best_bytes)) {
            best_tiles = tiles;
            best_bytes = bytes;
            a = aa;
        }
    }
    bmper = (nbm + a - 1) / a;
    bnper = (nbn + (NXCD / a) - 1) / (NXCD / a);
}

__device__ __forceinline__ bool xcd_tile(int hw_id, int nbm, int nbn, int M, int N, int& bm,
                                         int& bn) {
    int a, bmper, bnper;
    xcd_split(nbm, nbn, M, N, a, bmper, bnper);
    const int xcd = hw_id % NXCD, local = hw_id / NXCD;
    if (local >= bmper * bnper) return false;
    const int b = NXCD / a;
    bm = (xcd / b) * bmper + local / bnper;
    bn = (xcd % b) * bnper + local % bnper;
    return bm < nbm && bn < nbn;
}

// Workgroups of a persistent GEMM launch: one per CU of the MI355X (256 CUs in 8 XCDs).
constexpr int GEMM_PERSIST_WG = 256;
// Persistent on the 256x256 tiles of the forward's QKV and Wi GEMMs (RoPE and GeGLU
// epilogues); not the residual epilogue (its prefetched old residual leaves no registers for
// the next tile's loads; a persistent build spilled), the plain store (spilled too) nor the
// heads' fp32 epilogues.
constexpr bool gemm_persistent(int bm, int epi) {
    return MB_GEMM_PERSIST && bm == 256 && (epi == EPI_ROPE || epi == EPI_GEGLU);
}

// Grid size covering every split the device may choose for any row count up to M.
inline int xcd_gemm_grid(int M, int BM, int N, int BN) {
    const int nbm = (M + BM - 1) / BM, nbn = N / BN;
    int worst = 0;
    for (int aa = NXCD; aa >= 1; aa >>= 1) {
        const int bb = NXCD / aa;
        worst = max(worst, ((nbm + aa - 1) / aa) * ((nbn + bb - 1) / bb));
    }
    return NXCD * worst;
}

// LDS position of 16-byte chunk c of stage row r. Rows are RB bytes (128 or 64), unpadded.
// RB = 128: chunk c (0..7) is stored at slot c ^ ((r >> 1) & 7); rows r and r+1 differ by half
// of the 256-byte bank window, pairs of rows by the slot. RB = 64: chunk c (0..3) at slot
// c ^ ((r >> 2) & 3); four consecutive rows fill the window, groups of four differ by the slot.
// Either way sixteen consecutive rows read at one logical chunk cover all 64 banks, and the
// lanes that store one row write it contiguously.
template <int RB = 128>
__device__ __forceinline__ int lds_off(int r, int c) {
    if constexpr (RB == 128) return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    else return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

template <int EPI, int BN>
__device__ __forceinline__ int b_row(int bn, int r) {
    if constexpr (EPI == EPI_GEGLU) {
        // first BN/2 rows: GELU branch rows bn*BN/2 + r; next BN/2: the multiplier half
        return (r < BN / 2) ? bn * (BN / 2) + r : FF + bn * (BN / 2) + (r - BN / 2);
    } else {
        return bn * BN + r;
    }
}

// Residual statistics come in 64-column chunks: 12 per 768-wide row.
constexpr int NCHUNK = 768 / 64;

// Sum over each row of 16 lanes (the same value in all 16), by DPP lane swaps.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return v;
}

// Eight floats as dtype T to byte offset off of a buffer (16 bytes, or 32 for fp32).
template <typename T>
__device__ __forceinline__ void buf_store8(const void* base, unsigned extent, unsigned off, const float* v) {
    if constexpr (sizeof(T) == 4) {
        buf_store16(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), base, extent, off);
        buf_store16(__builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}), base, extent, off + 16);
    } else {
        typedef T t8 __attribute__((ext_vector_type(8)));
        t8 o = {(T)v[0], (T)v[1], (T)v[2], (T)v[3], (T)v[4], (T)v[5], (T)v[6], (T)v[7]};
        buf_store16(__builtin_bit_cast(u32x4, o), base, extent, off);
    }
}

__device__ __forceinline__ void load8(const float* src, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T, int BM, int BN, int NWM, int NWN, int EPI, int OCC, int DS, int RB = 128>
__global__ __launch_bounds__(64 * NWM * NWN, OCC) void gemm_kernel(GemmArgs p) {
    // Operand tiles go from global memory straight into DS LDS stages (16 bytes per lane),
    // with explicit wait counts and raw barriers. RB: bytes of K per row and K-step (128, or
    // 64 for more stages in the same LDS).
    constexpr int NT = 64 * NWM * NWN;                    // threads
    constexpr int ROWB = RB;   // bytes of K per row per stage; rows are unpadded (swizzled)
    static_assert(RB == 128 || RB == 64, "K-steps of 128 or 64 bytes");
    constexpr int SUB = ROWB / 32;                        // MFMA k-substeps per K-step
    constexpr int KT = ROWB / (int)sizeof(T);
    constexpr int WM = BM / NWM, WN = BN / NWN, FM = WM / 32, FN = WN / 32;
    constexpr int CP = BN + 8;                            // epilogue staging pitch (floats)
    constexpr bool PERSIST = gemm_persistent(BM, EPI);
    static_assert(!PERSIST || DS == 2, "persistent tiles prefetch into the first of two stages");
    constexpr int EPB = (!PERSIST && BM == 256 && (EPI == EPI_ROPE || EPI == EPI_STORE || EPI == EPI_GEGLU))
                            ? MB_GEMM_EPB : 1;  // block-rows a pass
    static_assert(FM % EPB == 0, "passes of whole block-rows");
    constexpr int NPASS = FM / EPB;                       // epilogue passes
    constexpr int EROWS = NWM * 32 * EPB;                 // rows staged per epilogue pass
    constexpr int MAIN_BYTES = DS * (BM + BN) * ROWB;
    constexpr int EPI_BYTES = EROWS * CP * 4;
    // folded GEMMs: mean and rstd per tile row and c per column, in LDS of their own beyond
    // the operand stages and the epilogue staging (they are written before the main loop)
    constexpr bool FOLDABLE = EPI == EPI_STORE || EPI == EPI_ROPE || EPI == EPI_GEGLU;
    // persistent tiles: the epilogue stages above stage 0 (which meanwhile takes the next
    // tile's first K-step), and the next tile's row statistics land in LDS of their own
    constexpr int STG_OFF = PERSIST ? (BM + BN) * RB : 0;
    constexpr int FOLD_OFF = MAIN_BYTES > STG_OFF + EPI_BYTES ? MAIN_BYTES : STG_OFF + EPI_BYTES;
    constexpr int SST_OFF = FOLD_OFF + (FOLDABLE ? BM * 8 + BN * 4 : 0);
    constexpr int SMEM = SST_OFF + (PERSIST && FOLDABLE ? BM * NCHUNK * 8 : 0);
    static_assert(EPI != EPI_ROPE || BN % 64 == 0, "RoPE tiles hold whole heads");
    __shared__ __align__(16) unsigned char smem[SMEM];

    const int nbn = p.N / BN;
    const int M = rows_of(p.counts, p.M);
    const int nbm = (M + BM - 1) / BM;
    int bm, bn;
    // persistent: slots blockIdx.x, + gridDim.x, ... (gridDim.x is a multiple of the XCD count,
    // so every slot of a workgroup lies on its own XCD), skipping slots without a tile
    int hw = blockIdx.x, nslots = 0;
    if constexpr (PERSIST) {
        int a_, bmp_, bnp_;
        xcd_split(nbm, nbn, M, p.N, a_, bmp_, bnp_);
        nslots = NXCD * bmp_ * bnp_;
        while (hw < nslots && !xcd_tile(hw, nbm, nbn, M, p.N, bm, bn)) hw += gridDim.x;
        if (hw >= nslots) return;
    } else {
        if (!xcd_tile(hw, nbm, nbn, M, p.N, bm, bn)) return;
    }
    const int tid0 = threadIdx.x;
    // staged epilogue row sr of pass i holds row sr % 32 of block-row EPB * i + (sr / 32) % EPB
    // of wave row sr / (32 EPB)
    auto tile_row_at = [](int mm0, int i, int sr) {
        return mm0 + (sr / (32 * EPB)) * (BM / NWM) + 32 * (EPB * i + (sr >> 5) % EPB) + (sr & 31);
    };
    // persistent: the next tile's RoPE positions and folded-norm column sum, loaded during the
    // previous tile's epilogue
    int rpos_c[NPASS];
    float fc_c = 0.f;
#pragma unroll
    for (int i = 0; i < NPASS; ++i) rpos_c[i] = 0;
    for (bool first = true;; first = false) {
        const int m0 = bm * BM;
        auto tile_row_of = [&](int i, int sr) { return tile_row_at(m0, i, sr); };
        constexpr int R_NHT = BN / HD > 0 ? BN / HD : 1;
        constexpr int R_IT = EPI == EPI_ROPE ? EROWS * R_NHT * 4 / (64 * NWM * NWN) : 1;
        constexpr int S_CH = BN / 4;
        constexpr int S_IT = EPI == EPI_RESID ? EROWS * S_CH / (64 * NWM * NWN) : 1;
        static_assert(EPI != EPI_ROPE || EROWS * R_NHT * 4 % (64 * NWM * NWN) == 0, "items split evenly");
        // RoPE epilogue items: item k of a thread is head (tid / 4) % R_HPT + R_HPT * k of staged row
        // tid / (4 R_HPT) at 8-frequency chunk tid % 4, so a thread's items share one {cos, sin} load
        constexpr int R_HPT = R_NHT / R_IT;
        static_assert(EPI != EPI_ROPE || R_NHT % R_IT == 0, "items of a thread share a row");
        static_assert(EPI != EPI_RESID || EROWS * S_CH % (64 * NWM * NWN) == 0, "items split evenly");
        const bool rot = EPI == EPI_ROPE && bn * BN < 2 * D;  // query and key columns are rotated
        int rpos[NPASS];
        float4 rcs[2][4];
        f32x4 rold[2][S_IT];
        float4 fbias[EPI == EPI_BIAS_F32 ? (NWM * 32) * S_CH / (64 * NWM * NWN) : 1];
        if constexpr (EPI == EPI_ROPE && !PERSIST) {  // raw positions; clamped after the main loop
#pragma unroll
            for (int i = 0; i < NPASS; ++i)
                rpos[i] = p.pos[min(tile_row_of(i, tid0 / (4 * R_HPT)), M - 1)];
        } else if constexpr (EPI == EPI_BIAS_F32) {
#pragma unroll
            for (int k = 0; k < (int)(sizeof(fbias) / sizeof(fbias[0])); ++k)
                fbias[k] = Vec4<T>::load((const T*)p.bias + bn * BN + 4 * ((tid0 + 64 * NWM * NWN * k) % S_CH));
        }
        // Folded LayerNorm: this tile's row statistics and column sums are loaded now, ahead of the
        // operand DMAs, and merged while the first stage lands
        const bool fold = FOLDABLE && p.stats_in != nullptr;
        // (unconditional loads, from the weights when there is no fold, so that no branch stands
        // between them and the main loop's wait counts)
        float2 fst[NCHUNK];
        float fc = 0.f;
        if constexpr (FOLDABLE && !PERSIST) {
            static_assert(BM <= 64 * NWM * NWN && BN <= 64 * NWM * NWN, "a thread per row and column");
            const float2* sp = fold ? p.stats_in : reinterpret_cast<const float2*>(p.B);
            const float* cp = fold ? p.cfold : reinterpret_cast<const float*>(p.B);
            const int r = fold ? min(m0 + min(tid0, BM - 1), M - 1) : 0;
#pragma unroll
            for (int j = 0; j < NCHUNK; ++j) fst[j] = sp[(size_t)r * NCHUNK + j];
            fc = cp[fold ? b_row<EPI, BN>(bn, min(tid0, BN - 1)) : 0];
        }

        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wm = wave / NWN, wn = wave % NWN;
        const size_t ld = (size_t)p.K * sizeof(T);

        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        const int nk = p.K / KT;
        const int lrow = lane & 31, lk = lane >> 5;  // lk: which 16-byte half of a 32-byte k-step
        static_assert(DS >= 2, "at least two LDS stages");
        constexpr int NW = NWM * NWN;
        constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
        constexpr int RPG = 64 / CPR;         // rows per 1 KB group (one DMA instruction)
        constexpr int G = (BM + BN) / RPG;    // groups of a stage
        static_assert(G % NW == 0, "groups split over the waves");
        constexpr int GW = G / NW;            // DMA instructions per wave and K-step
        constexpr int STAGE = (BM + BN) * ROWB;
        // Group g covers LDS rows RPG*g .. RPG*g + RPG-1 (A rows first, then B rows); lane L fills
        // row RPG*g + L/CPR at physical chunk L%CPR, which holds the logical chunk that lds_off
        // places there (the swizzle is its own inverse).
        // A groups (the first AJ of each wave) read from this tile's first row, B groups from the
        // weight base; offsets are 32-bit and stay inside each extent (rows are
        // clamped), the K-step goes into the scalar offset.
        constexpr int AJ = (BM / RPG) / NW;
        static_assert((BM / RPG) % NW == 0, "A and B groups split evenly over the waves");
        const int wu = __builtin_amdgcn_readfirstlane(wave);
        const unsigned char* abase = (const unsigned char*)p.A + (size_t)m0 * ld;
        const unsigned aext = (unsigned)min((size_t)(M - m0) * ld, (size_t)0xFFFFFFFFu);
        const unsigned bext = (unsigned)((size_t)(EPI == EPI_GEGLU ? 2 * FF : p.N) * ld);
        auto voff_of = [&](int tm0, int tbn, int jg) {
            const int g = wave + NW * jg, lrow8 = RPG * g + lane / CPR;
            const int c = (lds_off<ROWB>(lrow8, lane % CPR) - lrow8 * ROWB) >> 4;
            return jg < AJ ? (unsigned)((min(tm0 + lrow8, M - 1) - tm0) * ld + c * 16)
                           : (unsigned)(b_row<EPI, BN>(tbn, lrow8 - BM) * ld + c * 16);
        };
        unsigned voff[GW];
#pragma unroll
        for (int jg = 0; jg < GW; ++jg) voff[jg] = voff_of(m0, bn, jg);
        // Persistent tiles: what a tile needs before its main loop (positions, folded-norm column
        // sum, row statistics into LDS, K-step 0 into stage 0) is issued by the previous tile's
        // epilogue, or here for a workgroup's first tile. Without a next tile (live false) the
        // loads read row 0 and the DMAs an empty range, so no branch stands around them.
        auto prefetch = [&](int tbm, int tbn, bool live) {
            if constexpr (PERSIST) {
                const int tm0 = tbm * BM;
                if constexpr (EPI == EPI_ROPE) {
#pragma unroll
                    for (int i = 0; i < NPASS; ++i)
                        rpos_c[i] = p.pos[live ? min(tile_row_at(tm0, i, tid0 / (4 * R_HPT)), M - 1) : 0];
                }
                if constexpr (FOLDABLE) {
                    const float* cp = fold ? p.cfold : reinterpret_cast<const float*>(p.B);
                    fc_c = cp[fold && live ? b_row<EPI, BN>(tbn, min(tid0, BN - 1)) : 0];
                    // statistics of rows tm0 .. tm0 + BM - 1: BM * 96 contiguous bytes, 1 KB a DMA
                    constexpr int NSG = BM * NCHUNK * 8 / 1024;
                    static_assert(NSG % NW == 0, "statistics groups split over the waves");
                    const void* sb = fold && live ? static_cast<const void*>(p.stats_in + (size_t)tm0 * NCHUNK) : p.B;
                    const unsigned se = fold && live ? (unsigned)min((size_t)(M - tm0) * NCHUNK * 8, (size_t)0xFFFFFFFFu) : 0u;
#pragma unroll
                    for (int q = 0; q < NSG / NW; ++q)
                        lds_dma16_buf(sb, se, (unsigned)((wu + NW * q) * 1024 + 16 * lane), 0u,
                                      smem + SST_OFF + (wu + NW * q) * 1024);
                }
                const unsigned char* ab = (const unsigned char*)p.A + (size_t)(live ? tm0 : 0) * ld;
                const unsigned ae = live ? (unsigned)min((size_t)(M - tm0) * ld, (size_t)0xFFFFFFFFu) : 0u;
#pragma unroll
                for (int jg = 0; jg < GW; ++jg)
                    lds_dma16_buf(jg < AJ ? (const void*)ab : p.B, jg < AJ ? ae : (live ? bext : 0u),
                                  voff_of(tm0, tbn, jg), 0u, smem + (wu + NW * jg) * 1024);
            }
        };
        // Chan et al.'s pairwise merge of the 12 chunk statistics (equal counts of 64):
        // mean = mean of the means, M2 = sum of M2 + 64 * sum of squared mean deviations;
        // biased variance M2 / 768, eps inside the square root, as the LayerNorm kernel
        auto merge_stats = [&](const float2* fs, float& mean, float& rstd) {
            mean = 0.f;
#pragma unroll
            for (int j = 0; j < NCHUNK; ++j) mean += fs[j].x;
            mean *= 1.0f / NCHUNK;
            float m2 = 0.f, dev = 0.f;
#pragma unroll
            for (int j = 0; j < NCHUNK; ++j) {
                m2 += fs[j].y;
                dev += (fs[j].x - mean) * (fs[j].x - mean);
            }
            const float var = (m2 + 64.0f * dev) * (1.0f / D);
            rstd = 1.0f / sqrtf(var + p.eps);
        };
#define MB_DMA(KT_, ST_)                                                                  \
        do {                                                                          \
            _Pragma("unroll") for (int jg = 0; jg < GW; ++jg)                         \
                lds_dma16_buf(jg < AJ ? (const void*)abase : p.B, jg < AJ ? aext : bext, \
                              voff[jg], (unsigned)(KT_) * ROWB,                       \
                              smem + (ST_) * STAGE + (wu + NW * jg) * 1024);          \
        } while (0)
#define MB_FRAGS(ST_, S_, B_)                                                              \
        do {                                                                          \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) af[B_][i] =                \
                *(const u32x4*)((ST_) + lds_off<ROWB>(wm * WM + 32 * i + lrow, 2 * (S_) + lk)); \
            _Pragma("unroll") for (int j = 0; j < FN; ++j) bf[B_][j] =                \
                *(const u32x4*)((ST_) + lds_off<ROWB>(BM + wn * WN + 32 * j + lrow, 2 * (S_) + lk)); \
        } while (0)
        // Software pipeline: the fragments of k-substep s + 1 are read while the MFMAs of
        // substep s run; the wait and barrier that hand over the next stage sit before the last
        // substep's MFMAs, so the previous substep's MFMAs are still in the pipe meanwhile.
        float* rmean = reinterpret_cast<float*>(smem + FOLD_OFF);  // [BM]
        float* rrstd = rmean + BM;                                 // [BM]
        float* cst = rrstd + BM;                                   // [BN]
        if constexpr (PERSIST) {
            if (first) prefetch(bm, bn, true);
#pragma unroll
            for (int i = 0; i < NPASS; ++i) rpos[i] = rpos_c[i];
            fc = fc_c;
            MB_DMA(min(1, nk - 1), 1);  // K-step 1 into stage 1 (free since the last epilogue pass)
            if (first) {
                // everything but K-step 1 has landed (later tiles: the previous tile's last
                // epilogue pass waited for its prefetch, and its final barrier published it)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(GW));
                __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            if constexpr (FOLDABLE) {
                if (fold) {
                    if (tid < BM) {
                        const float4* sp = reinterpret_cast<const float4*>(smem + SST_OFF) + tid * (NCHUNK / 2);
                        float2 fs[NCHUNK];
#pragma unroll
                        for (int j = 0; j < NCHUNK / 2; ++j) {
                            const float4 v = sp[j];
                            fs[2 * j] = make_float2(v.x, v.y);
                            fs[2 * j + 1] = make_float2(v.z, v.w);
                        }
                        float mean, rstd;
                        merge_stats(fs, mean, rstd);
                        rmean[tid] = mean;
                        rrstd[tid] = rstd;
                    }
                    if (tid < BN) cst[tid] = fc;
                } else if (tid < BM) {
                    rrstd[tid] = 1.0f;  // the epilogue scales by rstd with or without a fold
                }
            }
            __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        } else {
#pragma unroll
            for (int st = 0; st < DS; ++st) MB_DMA(min(st, nk - 1), st);
            if constexpr (FOLDABLE) {
                if (fold) {
                    // the statistics were loaded before the DMAs: this wait leaves the DMAs in flight
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(GW * DS));
                    float mean, rstd;
                    merge_stats(fst, mean, rstd);
                    if (tid < BM) {
                        rmean[tid] = mean;
                        rrstd[tid] = rstd;
                    }
                    if (tid < BN) cst[tid] = fc;
                } else if (tid < BM) {
                    rrstd[tid] = 1.0f;  // the epilogue scales by rstd with or without a fold
                }
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(GW * (DS - 1)));
            __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());  // also retires scalar loads, so that the
                                                         // LDS wait counts in the loop are exact
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        if constexpr (FOLDABLE) {
            if (fold) {
                // out = rstd * (acc - mean * c): the accumulators start at -mean * c (row mean of
                // this lane's rows 8 (e / 4) + 4 (lane / 32) + e % 4 of each block, column sum of
                // its column), so the epilogue only scales by rstd
                const int rq0 = (lane >> 5) * 4;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 mv = *reinterpret_cast<const float4*>(rmean + wm * WM + 32 * i + 8 * q + rq0);
                        const float m4[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const float c = cst[wn * WN + 32 * j + lrow];
#pragma unroll
                            for (int t = 0; t < 4; ++t) acc[i][j][4 * q + t] = -m4[t] * c;
                        }
                    }
            }
        }
        static_assert(SUB % 2 == 0, "fragment buffers alternate by substep");
        u32x4 af[2][FM], bf[2][FN];
        MB_FRAGS(smem, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const unsigned char* St = smem + (kt % DS) * STAGE;
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                if (s + 1 < SUB) {
                    MB_FRAGS(St, s + 1, (s + 1) & 1);
                } else {
                    // every wave has read stage kt once its own reads have landed: after the
                    // barrier the stage takes K-step kt + DS, and stage kt + 1 (whose DMAs this
                    // wave has waited for) is visible to all
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(GW * (DS - 2)));
                    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    {
                        // past the last K-step the DMA's offset lies beyond both buffer extents:
                        // the range check drops it (no memory traffic, nothing for the epilogue
                        // to wait for; 0.5 % per forward of 28k tokens against re-reading the
                        // last K-step)
                        const unsigned soff = kt + DS < nk ? (unsigned)(kt + DS) * ROWB : 0x80000000u;
#pragma unroll
                        for (int jg = 0; jg < GW; ++jg)
                            lds_dma16_buf(jg < AJ ? (const void*)abase : p.B, jg < AJ ? aext : bext,
                                          voff[jg], soff, smem + (kt % DS) * STAGE + (wu + NW * jg) * 1024);
                    }
                    MB_FRAGS(smem + ((kt + 1) % DS) * STAGE, 0, 0);
                }
                // 8 MFMAs per substep (256x256 tiles): one fragment read (and on the last substep
                // one DMA) after each MFMA, so that the reads issue while the matrix core works
                // (0.2-1.5 % per forward at 28k-262k tokens). With fewer MFMAs per substep the
                // reads go first, in a block (interleaving them there was 1-4 % slower).
                constexpr int NMF = FM * FN, NRD = FM + FN;
                constexpr bool IL = NMF >= 8;
                if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) MfmaOp<T>::run(af[s & 1][i], bf[s & 1][j], acc[i][j]);
                if constexpr (IL) {
#pragma unroll
                    for (int q = 0; q < NMF; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
                        if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
                        if (s + 1 == SUB && q < GW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA
                    }
                    if (s + 1 == SUB && GW > NMF)
                        __builtin_amdgcn_sched_group_barrier(0x020, GW > NMF ? GW - NMF : 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#undef MB_FRAGS
#undef MB_DMA
        // the last DMAs (dropped by the range check) complete before the epilogue reuses the LDS
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        // ---- epilogue, in NPASS passes: pass i stages block-rows EPB i .. EPB i + EPB - 1 of every
        //      wave (EROWS tile rows) through LDS. A lane holds column (lane & 31) of each 32x32 block and rows
        //      8 * (e / 4) + 4 * (lane / 32) + (e % 4) for accumulator element e.
        // The vector-memory counter is shared by loads and stores and retires in order, so a pass
        // that waited for its own loads after the previous pass's stores would also wait for those
        // stores: every global load of pass i + 1 (the RoPE table rows, the old residual) is issued
        // before the stores of pass i, from rows clamped into [0, M), and only the stores test the
        // row. The RoPE positions are loaded before the main loop.
        float* Cs = reinterpret_cast<float*>(smem + STG_OFF);
        const int rq = (lane >> 5) * 4;
        // persistent: this workgroup's next tile
        int bm_n = bm, bn_n = bn;
        bool have_next = false;
        if constexpr (PERSIST) {
            int h = hw + gridDim.x, tb = 0, tn = 0;
            while (h < nslots && !xcd_tile(h, nbm, nbn, M, p.N, tb, tn)) h += gridDim.x;
            if (h < nslots) {
                have_next = true;
                bm_n = tb;
                bn_n = tn;
            }
            hw = h;
        }
        // output rows m0 .. M-1 as one buffer; offsets are relative to row m0
        const int cpitch = EPI == EPI_ROPE ? QKV * (int)sizeof(T)
                         : EPI == EPI_RESID ? D * 4
                         : EPI == EPI_GEGLU ? FF * (int)sizeof(T)
                         : EPI == EPI_STORE ? p.N * (int)sizeof(T)
                         : p.N * 4;
        const void* cbase = (const unsigned char*)p.C + (size_t)m0 * cpitch;
        const unsigned cext = (unsigned)min((size_t)(M - m0) * cpitch, (size_t)0xFFFFFFFFu);
        // residual extras: statistics [M][NCHUNK] float2 and the dtype copy [M, 768]
        const void* sbase = (const unsigned char*)p.stats_out + (size_t)m0 * NCHUNK * 8;
        const unsigned sext = (unsigned)min((size_t)(M - m0) * NCHUNK * 8, (size_t)0xFFFFFFFFu);
        const void* xbase = (const unsigned char*)p.xs_out + (size_t)m0 * D * sizeof(T);
        const unsigned xext = (unsigned)min((size_t)(M - m0) * D * sizeof(T), (size_t)0xFFFFFFFFu);
        auto issue_loads = [&](int i) {
            if constexpr (EPI == EPI_ROPE) {  // value tiles load (and ignore) the table too
                const float4* t = reinterpret_cast<const float4*>(p.rope + (size_t)rpos[i] * (HD / 2) + 8 * (tid & 3));
#pragma unroll
                for (int q = 0; q < 4; ++q) rcs[i & 1][q] = t[q];
            } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
                for (int k = 0; k < S_IT; ++k) {
                    const int idx = tid + NT * k, sr = idx / S_CH, c = idx % S_CH;
                    const f32x4* src = reinterpret_cast<const f32x4*>(
                        (const float*)p.C + (size_t)min(tile_row_of(i, sr), M - 1) * D + bn * BN + 4 * c);
                    // the old residual is read once: on the largest tiles (only used for long
                    // batches, far beyond the caches) non-temporally, 3-5 % faster at 262,144 rows
                    if constexpr (BM == 256) rold[i & 1][k] = __builtin_nontemporal_load(src);
                    else rold[i & 1][k] = *src;
                }
            }
        };
        // Values loaded before the main loop are first used here: the empty asm statements keep
        // the compiler from starting their arithmetic (and so waiting for them) before the loop.
        if constexpr (EPI == EPI_ROPE) {
#pragma unroll
            for (int i = 0; i < NPASS; ++i) {
                asm volatile("" : "+v"(rpos[i]));
                rpos[i] = min(max(rpos[i], 0), p.max_pos - 1);
            }
        }
        // out = rstd * acc for tile row tr (0 .. BM-1); acc started at -mean * c. Unconditional
        // (rstd is 1 without a fold): no branch keeps the rstd reads from being issued early
        auto fold8 = [&](float* v, int tr, int tc) {
            (void)tc;
            const float r = rrstd[tr];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= r;
        };
        issue_loads(0);
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
#pragma unroll
            for (int b = 0; b < EPB; ++b)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        Cs[(wm * 32 * EPB + 32 * b + 8 * (e >> 2) + rq + (e & 3)) * CP + wn * WN + 32 * j + lrow] =
                            acc[EPB * i + b][j][e];
            lds_barrier();
            if (i + 1 < NPASS) issue_loads(i + 1);
            if constexpr (PERSIST) {
                // the next tile's prefetch goes after this pass's loads (waiting for those then does
                // not wait for it); the last pass waits for it, so that the pass's final barrier
                // publishes the prefetched LDS data
                if (i == 0) prefetch(bm_n, bn_n, have_next);
                if (i + 1 == NPASS) {
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    asm volatile("" ::: "memory");
                }
            }
            auto tile_row = [&](int sr) { return tile_row_of(i, sr); };
            if constexpr (EPI == EPI_STORE) {
                constexpr int CH = BN / 8, IT = EROWS * CH / NT;
                static_assert(EROWS * CH % NT == 0, "items split evenly");
#pragma unroll
                for (int k = 0; k < IT; ++k) {
                    const int idx = tid + NT * k, sr = idx / CH, c = idx % CH, row = tile_row(sr);
                    float v[8];
                    load8(Cs + sr * CP + 8 * c, v);
                    fold8(v, row - m0, 8 * c);
                    buf_store8<T>(cbase, cext, (unsigned)((row - m0) * cpitch + (bn * BN + 8 * c) * (int)sizeof(T)), v);
                }
            } else if constexpr (EPI == EPI_ROPE) {
                const int c0 = bn * BN;
#pragma unroll
                for (int k = 0; k < R_IT; ++k) {
                    const int pc = tid & 3, hh = (tid >> 2) % R_HPT + R_HPT * k, sr = tid / (4 * R_HPT);
                    const int row = tile_row(sr);
                    float x1[8], x2[8];
                    const float* x = Cs + sr * CP + HD * hh + 8 * pc;
                    load8(x, x1);
                    load8(x + 32, x2);
                    fold8(x1, row - m0, HD * hh + 8 * pc);
                    fold8(x2, row - m0, HD * hh + 8 * pc + 32);
                    if (rot) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 t = rcs[i & 1][q];
                            const float a0 = x1[2 * q], b0 = x2[2 * q], a1 = x1[2 * q + 1], b1 = x2[2 * q + 1];
                            x1[2 * q] = a0 * t.x - b0 * t.y;
                            x2[2 * q] = b0 * t.x + a0 * t.y;
                            x1[2 * q + 1] = a1 * t.z - b1 * t.w;
                            x2[2 * q + 1] = b1 * t.z + a1 * t.w;
                        }
                    }
                    const unsigned off = (unsigned)(((row - m0) * QKV + c0 + HD * hh + 8 * pc) * (int)sizeof(T));
                    buf_store8<T>(cbase, cext, off, x1);
                    buf_store8<T>(cbase, cext, off + 32 * (unsigned)sizeof(T), x2);
                }
            } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
                for (int k = 0; k < S_IT; ++k) {
                    const int idx = tid + NT * k, sr = idx / S_CH, c = idx % S_CH, row = tile_row(sr);
                    const f32x4 a = *reinterpret_cast<const f32x4*>(Cs + sr * CP + 4 * c);
                    const f32x4 v = rold[i & 1][k] + a;
                    buf_store16(__builtin_bit_cast(u32x4, v), cbase, cext,
                                (unsigned)(((row - m0) * D + bn * BN + 4 * c) * 4));
                    if (p.stats_out) {
                        // the 16 lanes of this DPP row hold one 64-column chunk of this row:
                        // its mean, then the sum of squared deviations from it (two passes)
                        const float mean = row16_sum((v.x + v.y) + (v.z + v.w)) * (1.0f / 64);
                        const f32x4 d = v - mean;
                        const float m2 = row16_sum((d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w));
                        if ((lane & 15) == 0)
                            buf_store8b(__builtin_bit_cast(unsigned long long, make_float2(mean, m2)),
                                        sbase, sext,
                                        (unsigned)(((row - m0) * NCHUNK + (bn * BN + 4 * c) / 64) * 8));
                        if constexpr (sizeof(T) == 2) {
                            if (p.xs_out) {
                                typedef T t4 __attribute__((ext_vector_type(4)));
                                const t4 o = {(T)v.x, (T)v.y, (T)v.z, (T)v.w};
                                buf_store8b(__builtin_bit_cast(unsigned long long, o), xbase, xext,
                                            (unsigned)(((row - m0) * D + bn * BN + 4 * c) * 2));
                            }
                        }
                    }
                }
            } else if constexpr (EPI == EPI_GELU_F32 || EPI == EPI_BIAS_F32) {
                constexpr int CH = BN / 4, IT = EROWS * CH / NT;
                static_assert(EROWS * CH % NT == 0, "items split evenly");
#pragma unroll
                for (int k = 0; k < IT; ++k) {
                    const int idx = tid + NT * k, sr = idx / CH, c = idx % CH, row = tile_row(sr);
                    float4 v = *reinterpret_cast<const float4*>(Cs + sr * CP + 4 * c);
                    if constexpr (EPI == EPI_GELU_F32) {
                        v.x = gelu_erf(v.x);
                        v.y = gelu_erf(v.y);
                        v.z = gelu_erf(v.z);
                        v.w = gelu_erf(v.w);
                    } else {
                        v.x += fbias[k].x;
                        v.y += fbias[k].y;
                        v.z += fbias[k].z;
                        v.w += fbias[k].w;
                    }
                    buf_store16(__builtin_bit_cast(u32x4, v), cbase, cext,
                                (unsigned)((row - m0) * cpitch + (bn * BN + 4 * c) * 4));
                }
            } else {  // EPI_GEGLU
                constexpr int HALF = BN / 2, CH = HALF / 8, IT = EROWS * CH / NT;
                static_assert(EROWS * CH % NT == 0, "items split evenly");
#pragma unroll
                for (int k = 0; k < IT; ++k) {
                    const int idx = tid + NT * k, sr = idx / CH, c = idx % CH, row = tile_row(sr);
                    float g[8], u[8];
                    load8(Cs + sr * CP + 8 * c, g);
                    load8(Cs + sr * CP + HALF + 8 * c, u);
                    fold8(g, row - m0, 8 * c);
                    fold8(u, row - m0, HALF + 8 * c);
#pragma unroll
                    for (int q = 0; q < 8; ++q) g[q] = gelu_erf(g[q]) * u[q];
                    buf_store8<T>(cbase, cext, (unsigned)((row - m0) * cpitch + (bn * HALF + 8 * c) * (int)sizeof(T)), g);
                }
            }
            lds_barrier();
        }
        if constexpr (!PERSIST) return;
        if (!have_next) return;
        bm = bm_n;
        bn = bn_n;
    }
}




// Calibration of the matrix cores (not part of the forward): every wave runs `iters` rounds of
// four independent 32x32 MFMA accumulations on operands held in registers, so the kernel's
// duration gives the sustained dense MFMA rate of this chip for type T (16-bit: one 32x32x16,
// 32,768 flops, per slot; fp32: four 32x32x2, 16,384 flops, per slot). Each
// thread writes one float (the sum of its accumulators) so that nothing is optimised away.
template <typename T>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* out) {
    const unsigned lane = threadIdx.x & 63;
    const u32x4 a = {0x3f803f80u ^ lane, 0x3f803f80u, 0x3c003c00u, 0x3f803f80u ^ (lane << 16)};
    const u32x4 b = {0x3c003c00u, 0x3f803f80u ^ lane, 0x3c003c00u, 0x3f803f80u};
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) MfmaOp<T>::run(a, b, acc[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Tile shapes, by grid size (K is 768 or 1152, so a tile lives for only 12-36 K-steps and a
// small grid is bound by per-workgroup latency and by how evenly the tiles cover 256 CUs):
//   256x256, 8 waves of 128x64  - many rows: twice the MFMA work per wave per K-step
//   128x128, 4 waves of 64x64   - mid-sized grids
//   64x128 (N = 2304) / 64x64 (N = 768), 4 waves - few rows: more, shorter workgroups spread
//   over more CUs (64x128 measured 0.7 % faster per forward than 128x64 on 2445 rows)
template <typename T, int BM, int BN, int NWM, int NWN, int EPI, int OCC, int DS = MB_GEMM_DMA,
          int RB = 128>
int launch_tiles(const GemmArgs& a, hipStream_t s) {
    const int n = ((a.M + BM - 1) / BM) * (a.N / BN);
    if (n == 0) return MBERT_OK;
    int grid = xcd_gemm_grid(a.M, BM, a.N, BN);
    // persistent 256x256 tiles: one workgroup per CU (a multiple of the XCD count)
    if (gemm_persistent(BM, EPI)) grid = min(grid, GEMM_PERSIST_WG);
    MB_LAUNCH((gemm_kernel<T, BM, BN, NWM, NWN, EPI, OCC, DS, RB>), grid, 64 * NWM * NWN, 0, s, a);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

template <typename T, int EPI>
int run_gemm(const GemmArgs& a, hipStream_t s) {
    if ((a.K * (int)sizeof(T)) % 128 != 0) return MBERT_EUNSUPPORTED;
    const int t128 = ((a.M + 127) / 128) * (a.N / 128);
    const int t256 = ((a.M + 255) / 256) * (a.N / 256);
    if (a.N % 256 == 0 && t256 >= MB_GEMM_BIG_MIN_TILES)
        return launch_tiles<T, 256, 256, 2, 4, EPI, 1, MB_GEMM_BIG_DS, MB_GEMM_BIG_RB>(a, s);
    if (t128 >= MB_GEMM_SMALL_MAX_TILES)
        return launch_tiles<T, 128, 128, 2, 2, EPI, MB_GEMM_MID_OCC, MB_GEMM_MID_DS, MB_GEMM_MID_RB>(a, s);
    if (a.N == D)
        return launch_tiles<T, 64, 64, 2, 2, EPI, MB_GEMM_N768_OCC, MB_GEMM_DMA_N768, MB_GEMM_N768_RB>(a, s);
    return launch_tiles<T, 64, 128, 2, 2, EPI, MB_GEMM_SMALL_OCC, MB_GEMM_SMALL_DS, MB_GEMM_SMALL_RB>(a, s);
}

// fp32 outputs of any width that is a multiple of 64 (the heads: 768, or a vocabulary of
// 50,368 = 787 x 64 columns).
template <typename T, int EPI>
int run_gemm_f32(const GemmArgs& a, hipStream_t s) {
    if (a.N % 128 == 0) return run_gemm<T, EPI>(a, s);
    if ((a.K * (int)sizeof(T)) % 128 != 0) return MBERT_EUNSUPPORTED;
    if (a.M <= 512) return launch_tiles<T, 64, 64, 2, 2, EPI, 4>(a, s);
    return launch_tiles<T, 128, 64, 2, 2, EPI, 3>(a, s);
}

template <typename T>
int qkv_t(const GemmArgs& a, int apply_rope, hipStream_t s) {
    return apply_rope ? run_gemm<T, EPI_ROPE>(a, s) : run_gemm<T, EPI_STORE>(a, s);
}

template <typename T>
int resid_t(const GemmArgs& a, hipStream_t s) {
    return run_gemm<T, EPI_RESID>(a, s);
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_mfma_probe(mbert_dtype dt, int blocks, int iters, float* out, hipStream_t s) {
    switch (dt) {
        case MBERT_F32: MB_LAUNCH((mfma_probe_kernel<float>), blocks, 256, 0, s, iters, out); break;
        case MBERT_BF16: MB_LAUNCH((mfma_probe_kernel<bf16>), blocks, 256, 0, s, iters, out); break;
        case MBERT_F16: MB_LAUNCH((mfma_probe_kernel<f16>), blocks, 256, 0, s, iters, out); break;
        default: return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_qkv(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* W,
               const float* rope, int max_pos, int table, int apply_rope, void* qkv,
               hipStream_t s, const FoldArgs* fold, bool host_rows) {
    GemmArgs a{};
    if (fold) {
        a.cfold = fold->c;
        a.stats_in = fold->stats;
        a.eps = fold->eps;
    }
    a.A = h;
    a.B = W;
    a.M = total;
    a.counts = host_rows ? nullptr : meta;
    a.K = D;
    a.N = QKV;
    a.C = qkv;
    a.pos = meta ? meta + 8 : nullptr;
    a.rope = reinterpret_cast<const float2*>(rope) + (size_t)table * max_pos * (HD / 2);
    a.max_pos = max_pos;
    switch (dt) {
        case MBERT_F32: return qkv_t<float>(a, apply_rope, s);
        case MBERT_BF16: return qkv_t<bf16>(a, apply_rope, s);
        case MBERT_F16: return qkv_t<f16>(a, apply_rope, s);
        default: return MBERT_EUNSUPPORTED;
    }
}

int launch_linear_residual(mbert_dtype dt, const void* a_, int K, int total, const int32_t* meta,
                           const void* W, float* resid, hipStream_t s, void* xs_out,
                           float2* stats_out, bool host_rows) {
    GemmArgs a{};
    a.xs_out = xs_out;
    a.stats_out = stats_out;
    a.A = a_;
    a.B = W;
    a.M = total;
    a.counts = host_rows ? nullptr : meta;
    a.K = K;
    a.N = D;
    a.C = resid;
    switch (dt) {
        case MBERT_F32: return resid_t<float>(a, s);
        case MBERT_BF16: return resid_t<bf16>(a, s);
        case MBERT_F16: return resid_t<f16>(a, s);
        default: return MBERT_EUNSUPPORTED;
    }
}

int launch_geglu(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* Wi,
                 void* m, hipStream_t s, const FoldArgs* fold, bool host_rows) {
    GemmArgs a{};
    if (fold) {
        a.cfold = fold->c;
        a.stats_in = fold->stats;
        a.eps = fold->eps;
    }
    a.A = h;
    a.B = Wi;
    a.M = total;
    a.counts = host_rows ? nullptr : meta;
    a.K = D;
    a.N = 2 * FF;
    a.C = m;
    switch (dt) {
        case MBERT_F32: return run_gemm<float, EPI_GEGLU>(a, s);
        case MBERT_BF16: return run_gemm<bf16, EPI_GEGLU>(a, s);
        case MBERT_F16: return run_gemm<f16, EPI_GEGLU>(a, s);
        default: return MBERT_EUNSUPPORTED;
    }
}

}  // namespace mbh

namespace mbh {
int launch_linear_f32(mbert_dtype dt, const void* a_, int M, const void* W, int N, int K,
                      int gelu, const void* bias, float* out, hipStream_t s) {
    mb::GemmArgs a{};
    a.A = a_;
    a.B = W;
    a.M = M;
    a.K = K;
    a.N = N;
    a.C = out;
    a.bias = bias;
    if (N % 64 != 0 || K != mb::D || (!gelu && !bias)) return MBERT_EUNSUPPORTED;
    switch (dt) {
        case MBERT_F32:
            return gelu ? mb::run_gemm_f32<float, mb::EPI_GELU_F32>(a, s)
                        : mb::run_gemm_f32<float, mb::EPI_BIAS_F32>(a, s);
        case MBERT_BF16:
            return gelu ? mb::run_gemm_f32<mb::bf16, mb::EPI_GELU_F32>(a, s)
                        : mb::run_gemm_f32<mb::bf16, mb::EPI_BIAS_F32>(a, s);
        case MBERT_F16:
            return gelu ? mb::run_gemm_f32<mb::f16, mb::EPI_GELU_F32>(a, s)
                        : mb::run_gemm_f32<mb::f16, mb::EPI_BIAS_F32>(a, s);
        default: return MBERT_EUNSUPPORTED;
    }
}
}  // namespace mbh

namespace mb {
// Folded LayerNorm weight: Wf[r][k] = W[r][k] * w[k] rounded once to T, and c[r] the sum of
// the rounded row (so that rstd * (x . Wf_r - mean * c_r) is exactly sum_k (x_k - mean) rstd
// w_k W_rk up to the rounding of Wf). One wave per row, a fixed summation order.
template <typename T>
__global__ __launch_bounds__(256) void fold_weight_kernel(const T* __restrict__ W,
                                                          const T* __restrict__ w, int rows,
                                                          T* __restrict__ Wf, float* __restrict__ c) {
    const int lane = threadIdx.x & 63, r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int k = lane + 64 * j;
        const T v = (T)(to_f(W[(size_t)r * D + k]) * to_f(w[k]));
        Wf[(size_t)r * D + k] = v;
        acc += to_f(v);
    }
    acc = wave_sum(acc);
    if (lane == 0) c[r] = acc;
}
}  // namespace mb

namespace mbh {
int launch_fold_weight(mbert_dtype dt, const void* W, const void* w, int rows, void* Wf,
                       float* c, hipStream_t s) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((mb::fold_weight_kernel<float>), grid, 256, 0, s, (const float*)W, (const float*)w, rows,
                      (float*)Wf, c);
            break;
        case MBERT_BF16:
            MB_LAUNCH((mb::fold_weight_kernel<mb::bf16>), grid, 256, 0, s, (const mb::bf16*)W,
                      (const mb::bf16*)w, rows, (mb::bf16*)Wf, c);
            break;
        case MBERT_F16:
            MB_LAUNCH((mb::fold_weight_kernel<mb::f16>), grid, 256, 0, s, (const mb::f16*)W,
                      (const mb::f16*)w, rows, (mb::f16*)Wf, c);
            break;
        default:
            return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}
}  // namespace mbh
