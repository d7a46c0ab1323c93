// MFMA GEMM for the encoder's four projections: C[M, N] = A[M, K] . B[N, K]^T, both operands
// K-contiguous (activations row-major, Linear weights stored [out, in]), fp32 accumulation.
//
// Tiling: 256 threads = 4 wave64s in a 2x2 arrangement; each wave owns a (BM/2) x (BN/2)
// sub-tile made of 32x32 MFMA blocks (v_mfma_f32_32x32x16_{bf16,f16}; fp32 inputs use
// v_mfma_f32_32x32x2_f32, four per 16-byte operand). K is consumed 128 bytes at a time
// (64 16-bit or 32 fp32 elements) through two LDS stages: the next K-tile is fetched into
// registers while the current one feeds the MFMAs, so each iteration needs one barrier.
// LDS rows are padded to 144 bytes so the 16-byte operand reads of 8 consecutive lanes hit
// distinct banks.
//
// Epilogues (fused, applied to the fp32 accumulators before anything is rounded):
//   STORE : C (dtype) = acc
//   ROPE  : query/key head columns rotated rotate-half style at each row's position, then
//           stored (candding, "ModernBERT", §"The two rope tables"); a wave's two 32-column
//           blocks are dims i and i+32 of one head, so every pair sits in one lane.
//   RESID : resid (fp32) += acc (kgptalkie, §"What Does LayerNorm Do?": the block output is
//           added back to its input)
//   GEGLU : m = gelu_erf(u_gate) * u_mult; the B tile interleaves the GELU-branch rows
//           [n0, n0+32) and the multiplier rows [1152+n0, 1152+n0+32) per wave so the pair of
//           a column lands in one lane (candding, §"The feed-forward halves").
#include "common.hpp"

namespace mb {

enum { EPI_STORE = 0, EPI_ROPE = 1, EPI_RESID = 2, EPI_GEGLU = 3 };

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float gelu_erf(float z) {
    // z * Phi(z) with the exact error function (candding, §"The feed-forward halves")
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

template <int EPI, int BN>
__device__ __forceinline__ int b_row(int bn, int r) {
    if constexpr (EPI == EPI_GEGLU) {
        const int half = r / (BN / 2);            // which wave column
        const int within = r % (BN / 2);
        const int blk = within / 32, i = within % 32;  // blk 0: GELU branch, 1: multiplier
        return blk * FF + bn * (BN / 2) + half * 32 + i;
    } else {
        return bn * BN + r;
    }
}

template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs p) {
    constexpr int ROWB = 128, PITCH = 144;
    constexpr int KT = ROWB / (int)sizeof(T);
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    constexpr int ACH = BM / 32, BCH = BN / 32;
    static_assert(EPI != EPI_ROPE || FN == 2, "RoPE epilogue needs 64-column wave tiles");
    static_assert(EPI != EPI_GEGLU || FN == 2, "GeGLU epilogue needs 64-column wave tiles");
    __shared__ __align__(16) unsigned char smem[2 * (BM + BN) * PITCH];

    const int nbn = p.N / BN;
    const int nbm = (p.M + BM - 1) / BM;
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    if (tile >= nbn * nbm) return;
    const int bm = tile / nbn, bn = tile % nbn;
    const int M = rows_of(p.counts, p.M);
    const int m0 = bm * BM;
    if (m0 >= M) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int crow = tid >> 3, cchunk = tid & 7;
    const size_t ld = (size_t)p.K * sizeof(T);

    const unsigned char* a_ptr[ACH];
    const unsigned char* b_ptr[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int gr = min(m0 + crow + 32 * i, M - 1);
        a_ptr[i] = (const unsigned char*)p.A + (size_t)gr * ld + cchunk * 16;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        const int gr = b_row<EPI, BN>(bn, crow + 32 * i);
        b_ptr[i] = (const unsigned char*)p.B + (size_t)gr * ld + cchunk * 16;
    }

    u32x4 ra[ACH], rb[BCH];
    auto gload = [&](int kt) {
        const size_t off = (size_t)kt * ROWB;
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = *(const u32x4*)(a_ptr[i] + off);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = *(const u32x4*)(b_ptr[i] + off);
    };
    auto sstore = [&](int st) {
        unsigned char* base = smem + st * (BM + BN) * PITCH;
#pragma unroll
        for (int i = 0; i < ACH; ++i) *(u32x4*)(base + (crow + 32 * i) * PITCH + cchunk * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            *(u32x4*)(base + (BM + crow + 32 * i) * PITCH + cchunk * 16) = rb[i];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = p.K / KT;
    gload(0);
    sstore(0);
    __syncthreads();
    const int lrow = lane & 31, lk = (lane >> 5) * 16;
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload(kt + 1);
        const unsigned char* As = smem + (kt & 1) * (BM + BN) * PITCH;
        const unsigned char* Bs = As + BM * PITCH;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *(const u32x4*)(As + (wm * WM + 32 * i + lrow) * PITCH + s * 32 + lk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *(const u32x4*)(Bs + (wn * WN + 32 * j + lrow) * PITCH + s * 32 + lk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) MfmaOp<T>::run(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 31) of each 32x32 block and rows
    //      8 * (e / 4) + 4 * (lane / 32) + (e % 4) for accumulator element e.
    const int rq = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + rq + (e & 3);
            if (row >= M) continue;
            if constexpr (EPI == EPI_STORE) {
                T* C = (T*)p.C;
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    C[(size_t)row * p.N + bn * BN + wn * WN + 32 * j + lrow] = from_f<T>(acc[i][j][e]);
            } else if constexpr (EPI == EPI_RESID) {
                float* R = (float*)p.C;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    float* r = R + (size_t)row * D + bn * BN + wn * WN + 32 * j + lrow;
                    *r += acc[i][j][e];
                }
            } else if constexpr (EPI == EPI_ROPE) {
                T* C = (T*)p.C;
                const int c0 = bn * BN + wn * WN;  // first column of this wave's head
                float y1 = acc[i][0][e], y2 = acc[i][1][e];
                if (c0 < 2 * D) {
                    const int pp = min(max(p.pos[row], 0), p.max_pos - 1);
                    const float2 cs = p.rope[(size_t)pp * (HD / 2) + lrow];
                    const float x1 = y1, x2 = y2;
                    y1 = x1 * cs.x - x2 * cs.y;
                    y2 = x2 * cs.x + x1 * cs.y;
                }
                C[(size_t)row * QKV + c0 + lrow] = from_f<T>(y1);
                C[(size_t)row * QKV + c0 + 32 + lrow] = from_f<T>(y2);
            } else {  // EPI_GEGLU
                T* C = (T*)p.C;
                const int col = bn * (BN / 2) + wn * 32 + lrow;
                C[(size_t)row * FF + col] = from_f<T>(gelu_erf(acc[i][0][e]) * acc[i][1][e]);
            }
        }
    }
}

template <typename T, int BM, int BN, int EPI>
int run_gemm(const GemmArgs& a, hipStream_t s) {
    const int nbm = (a.M + BM - 1) / BM, nbn = a.N / BN;
    const int n = nbm * nbn;
    if (n == 0) return MBERT_OK;
    gemm_kernel<T, BM, BN, EPI><<<xcd_grid(n), 256, 0, s>>>(a);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

template <typename T>
int qkv_t(const GemmArgs& a, int apply_rope, hipStream_t s) {
    return apply_rope ? run_gemm<T, 128, 128, EPI_ROPE>(a, s) : run_gemm<T, 128, 128, EPI_STORE>(a, s);
}

template <typename T>
int resid_t(const GemmArgs& a, hipStream_t s) {
    // N = 768 gives only 6 column tiles: use 64-row tiles until there are enough row tiles
    // to fill 256 CUs twice over with 128-row ones.
    if ((a.M + 127) / 128 * 6 >= 1024) return run_gemm<T, 128, 128, EPI_RESID>(a, s);
    return run_gemm<T, 64, 128, EPI_RESID>(a, s);
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_qkv(mbert_dtype dt, const void* h, int total, const int32_t* meta, const void* W,
               const float* rope, int max_pos, int table, int apply_rope, void* qkv,
               hipStream_t s) {
    GemmArgs a{};
    a.A = h;
    a.B = W;
    a.M = total;
    a.counts = meta;
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
                           const void* W, float* resid, hipStream_t s) {
    GemmArgs a{};
    a.A = a_;
    a.B = W;
    a.M = total;
    a.counts = meta;
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
                 void* m, hipStream_t s) {
    GemmArgs a{};
    a.A = h;
    a.B = Wi;
    a.M = total;
    a.counts = meta;
    a.K = D;
    a.N = 2 * FF;
    a.C = m;
    switch (dt) {
        case MBERT_F32: return run_gemm<float, 128, 128, EPI_GEGLU>(a, s);
        case MBERT_BF16: return run_gemm<bf16, 128, 128, EPI_GEGLU>(a, s);
        case MBERT_F16: return run_gemm<f16, 128, 128, EPI_GEGLU>(a, s);
        default: return MBERT_EUNSUPPORTED;
    }
}

}  // namespace mbh
