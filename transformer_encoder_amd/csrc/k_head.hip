// Small kernels of the heads on top of the encoder (kgptalkie, "ModernBERT-base Architecture
// Teardown", §"The Masked-LM Head", §"How Do We Put a Classifier on Top?"): the row gather that
// feeds the prediction head, and the narrow classifier Linear. The dense layers, the
// LayerNorm and the 50,368-wide decoder run on the GEMM and norm kernels.
#include "common.hpp"

namespace mb {

// out[r] = dtype(x[rows[r]]) (or x[r] without a row list); a row index outside [0, total)
// gives a zero row. One wave per row, 12 values per lane.
template <typename T>
__global__ __launch_bounds__(256) void gather_cast_kernel(const float* __restrict__ x, int total,
                                                          const int* __restrict__ rows, int R,
                                                          T* __restrict__ out) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (r >= R) return;
    const int src = rows ? rows[r] : r;
    const bool ok = src >= 0 && src < total;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const float4 v = ok ? *reinterpret_cast<const float4*>(x + (long)src * D + 4 * (lane + 64 * c))
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        Vec4<T>::store(out + (long)r * D + 4 * (lane + 64 * c), v);
    }
}

// out[s, c] = h[s] . W[c] + b[c] for a handful of labels: one wave per (row, label).
template <typename T>
__global__ __launch_bounds__(256) void small_linear_kernel(const T* __restrict__ h,
                                                           const T* __restrict__ W,
                                                           const T* __restrict__ b, int S, int C,
                                                           float* __restrict__ out) {
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (idx >= S * C) return;
    const int s = idx / C, c = idx % C;
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float4 x = Vec4<T>::load(h + (long)s * D + 4 * (lane + 64 * q));
        const float4 w = Vec4<T>::load(W + (long)c * D + 4 * (lane + 64 * q));
        acc += x.x * w.x + x.y * w.y + x.z * w.z + x.w * w.w;
    }
    acc = wave_sum(acc);
    if (lane == 0) out[idx] = acc + to_f(b[c]);
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_gather_cast(mbert_dtype dt, const float* x, int total, const int32_t* rows, int R,
                       void* out, hipStream_t s) {
    if (R == 0) return MBERT_OK;
    const unsigned grid = (unsigned)((R + 3) / 4);
    switch (dt) {
        case MBERT_F32: MB_LAUNCH((gather_cast_kernel<float>), grid, 256, 0, s, x, total, rows, R, (float*)out); break;
        case MBERT_BF16: MB_LAUNCH((gather_cast_kernel<bf16>), grid, 256, 0, s, x, total, rows, R, (bf16*)out); break;
        case MBERT_F16: MB_LAUNCH((gather_cast_kernel<f16>), grid, 256, 0, s, x, total, rows, R, (f16*)out); break;
        default: return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_small_linear(mbert_dtype dt, const void* h, const void* W, const void* b, int S, int C,
                        float* out, hipStream_t s) {
    if (S == 0 || C == 0) return MBERT_OK;
    const unsigned grid = (unsigned)(((long)S * C + 3) / 4);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((small_linear_kernel<float>), grid, 256, 0, s, (const float*)h, (const float*)W, (const float*)b, S, C, out);
            break;
        case MBERT_BF16:
            MB_LAUNCH((small_linear_kernel<bf16>), grid, 256, 0, s, (const bf16*)h, (const bf16*)W, (const bf16*)b, S, C, out);
            break;
        case MBERT_F16:
            MB_LAUNCH((small_linear_kernel<f16>), grid, 256, 0, s, (const f16*)h, (const f16*)W, (const f16*)b, S, C, out);
            break;
        default: return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}
}  // namespace mbh
