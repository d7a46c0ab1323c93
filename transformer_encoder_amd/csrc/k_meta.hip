// Batch bookkeeping kernels: RoPE tables, unpadding, work tiles, positions, key ranges,
// re-padding. Integer work is exact; no floating point decides anything here.
#include "common.hpp"

namespace mb {

// ---------------------------------------------------------------- RoPE tables
// Entry [t][p][i] = {cos, sin} of p * theta_t^(-2i/64), evaluated in float64 and rounded once
// to float32 (kgptalkie, "ModernBERT-base Architecture Teardown", §"How Does RoPE Work With
// Two Bases?"; table 0 = global base, table 1 = local base).
__global__ void rope_table_kernel(float2* __restrict__ tab, int max_pos, double theta_g,
                                  double theta_l) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long n = 2L * max_pos * (HD / 2);
    if (idx >= n) return;
    const int i = (int)(idx % (HD / 2));
    const int p = (int)((idx / (HD / 2)) % max_pos);
    const int t = (int)(idx / ((long)(HD / 2) * max_pos));
    const double theta = t == 0 ? theta_g : theta_l;
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)HD);
    const double a = (double)p * inv_freq;
    tab[idx] = make_float2((float)cos(a), (float)sin(a));
}

// ---------------------------------------------------------------- block scan (1024 threads)
__device__ int block_excl_scan(int v, int* lds, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) lds[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = lane < nw ? lds[lane] : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(t, o, 64);
            if (lane >= o) t += y;
        }
        if (lane < nw) lds[lane] = t;
    }
    __syncthreads();
    const int prefix = w > 0 ? lds[w - 1] : 0;
    total = lds[nw - 1];
    __syncthreads();
    return prefix + x - v;
}

// Work tiles of TILE query rows; a tile never crosses a sequence. Shared by the packed and
// the padded path; cu must already hold valid offsets when ok is true.
__device__ void build_tiles(const int* cu, int S, bool ok, MetaView mv, int* lds) {
    int carry = 0;
    for (int base = 0; base < S; base += blockDim.x) {
        const int s = base + threadIdx.x;
        int a = 0, L = 0;
        if (s < S) {
            a = cu[s];
            L = cu[s + 1] - a;
        }
        const int nt = (ok && s < S) ? (L + TILE - 1) / TILE : 0;
        int tot;
        const int ex = block_excl_scan(nt, lds, tot);
        if (s < S) {
            mv.seq_tile0[s] = carry + ex;
            for (int j = 0; j < nt; ++j)
                mv.tiles[carry + ex + j] = make_int4(a + j * TILE, min(TILE, L - j * TILE), a, a + L);
        }
        carry += tot;
    }
    if (threadIdx.x == 0) {
        mv.seq_tile0[S] = carry;
        mv.counts[MBERT_META_NTILES] = carry;
    }
    // The attention's dispatch order: the tiles of longer sequences first (a global layer's
    // tile costs its sequence's length in key tiles), so that the longest workgroups do not
    // start last. A counting sort of the sequences by key tiles (64 keys each, capped at 128):
    // tile counts per key, start offsets in descending key order, then each sequence claims
    // its slots; within one key the order is whatever the atomics give (each tile's output is
    // its own, so the results do not depend on it).
    constexpr int KB = 129;
    __shared__ int bins[KB];
    for (int k = threadIdx.x; k < KB; k += blockDim.x) bins[k] = 0;
    __syncthreads();
    auto key_of = [](int L) { return min((L + 63) / 64, KB - 1); };
    for (int s = threadIdx.x; ok && s < S; s += blockDim.x) {
        const int L = cu[s + 1] - cu[s];
        if (L > 0) atomicAdd(&bins[key_of(L)], (L + TILE - 1) / TILE);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int k = KB - 1; k >= 0; --k) {
            const int c = bins[k];
            bins[k] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int s = threadIdx.x; ok && s < S; s += blockDim.x) {
        const int L = cu[s + 1] - cu[s];
        if (L <= 0) continue;
        const int nt = (L + TILE - 1) / TILE;
        const int p = atomicAdd(&bins[key_of(L)], nt), t0 = mv.seq_tile0[s];
        for (int j = 0; j < nt; ++j) mv.order[p + j] = t0 + j;
    }
}

// Packed path: validate cu_seqlens, then counts and tiles. One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void pack_meta_kernel(const int* __restrict__ cu, int S,
                                                         int total, int max_pos,
                                                         int* __restrict__ meta, int total_max) {
    __shared__ int lds[32];
    __shared__ int s_status, s_maxlen;
    const MetaView mv = meta_view(meta, total_max, S);
    if (threadIdx.x == 0) {
        s_status = (cu[0] != 0 || cu[S] != total) ? MBERT_STATUS_BAD_CU : 0;
        s_maxlen = 0;
    }
    __syncthreads();
    int status = 0, maxlen = 0;
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        const int a = cu[s], b = cu[s + 1];
        if (b < a || a < 0 || b > total) status |= MBERT_STATUS_BAD_CU;
        const int L = b - a;
        if (L > max_pos) status |= MBERT_STATUS_TOO_LONG;
        maxlen = max(maxlen, L);
    }
    if (status) atomicOr(&s_status, status);
    atomicMax(&s_maxlen, maxlen);
    __syncthreads();
    status = s_status;
    const bool ok = (status & (MBERT_STATUS_BAD_CU | MBERT_STATUS_TOO_LONG)) == 0;
    build_tiles(cu, S, ok, mv, lds);
    if (threadIdx.x == 0) {
        mv.counts[MBERT_META_TOTAL] = total;
        mv.counts[MBERT_META_MAXLEN] = ok ? s_maxlen : 0;
        mv.counts[MBERT_META_STATUS] = status;
        for (int i = 4; i < 8; ++i) mv.counts[i] = 0;
    }
}

// Padded batch run at full width (no unpadding): row b of the [B, Tpad] batch is one
// sequence of Tpad query rows whose keys are its first L_b rows, the real tokens of a
// right-padded mask (the key padding mask: rayaq, "Encoder-only models", §"Padding and the key
// padding mask"). Tiles {b*Tpad + 128k, rows, b*Tpad, b*Tpad + L_b}; a mask row that is not
// ones followed by zeros flags MBERT_STATUS_BAD_MASK and keeps its leading run of ones as keys.
// One workgroup of 1024 threads, a wave per batch row.
__global__ __launch_bounds__(1024) void padded_meta_kernel(const int* __restrict__ mask, int B,
                                                           int Tpad, int max_pos,
                                                           int* __restrict__ meta) {
    __shared__ int s_status;
    const int total_max = B * Tpad;
    const MetaView mv = meta_view(meta, total_max, B);
    const int nt = (Tpad + TILE - 1) / TILE;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (threadIdx.x == 0) s_status = Tpad > max_pos ? MBERT_STATUS_TOO_LONG : 0;
    __syncthreads();
    const bool too_long = s_status != 0;
    int status = 0;
    for (int b = wave; b < B; b += nw) {
        const int* m = mask + (long)b * Tpad;
        // leading run of ones: the first t with m[t] != 1 (Tpad if none)
        int first = Tpad, any_after = 0;
        for (int t = lane; t < Tpad; t += 64)
            if (m[t] != 1) first = min(first, t);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
        for (int t = first + lane; t < Tpad; t += 64) any_after |= m[t] != 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) any_after |= __shfl_xor(any_after, o, 64);
        if (any_after) status |= MBERT_STATUS_BAD_MASK;
        const int L = first;
        for (int k = lane; k < nt; k += 64) {
            mv.tiles[b * nt + k] = make_int4(b * Tpad + TILE * k, min(TILE, Tpad - TILE * k),
                                             b * Tpad, b * Tpad + L);
            mv.order[b * nt + k] = b * nt + k;  // every row is Tpad queries: in row order
        }
        if (lane == 0) mv.seq_tile0[b] = too_long ? 0 : b * nt;
    }
    if (status) atomicOr(&s_status, status);
    __syncthreads();
    if (threadIdx.x == 0) {
        mv.seq_tile0[B] = too_long ? 0 : B * nt;
        mv.counts[MBERT_META_TOTAL] = total_max;
        mv.counts[MBERT_META_MAXLEN] = too_long ? 0 : Tpad;
        mv.counts[MBERT_META_NTILES] = too_long ? 0 : B * nt;
        mv.counts[MBERT_META_STATUS] = s_status;
        for (int i = 4; i < 8; ++i) mv.counts[i] = 0;
    }
}

// Position of each token inside its sequence, one workgroup per tile.
__global__ __launch_bounds__(TILE) void pos_kernel(int* __restrict__ meta, int total_max, int S) {
    const MetaView mv = meta_view(meta, total_max, S);
    const int b = blockIdx.x;
    if (b >= mv.counts[MBERT_META_NTILES]) return;
    const int4 tl = mv.tiles[b];
    const int t = threadIdx.x;
    if (t < tl.y) mv.pos[tl.x + t] = tl.x + t - tl.z;
}

// Padded path, step 1: per row, count the real tokens (mask != 0). cu[b+1] temporarily holds
// L_b | (bad-mask flag << 30).
__global__ __launch_bounds__(256) void unpad_count_kernel(const int* __restrict__ mask, int Tpad,
                                                          int* __restrict__ cu) {
    __shared__ int red[4];
    const int b = blockIdx.x;
    int cnt = 0, bad = 0;
    for (int t = threadIdx.x; t < Tpad; t += blockDim.x) {
        const int m = mask[(long)b * Tpad + t];
        cnt += m != 0;
        bad |= (m != 0 && m != 1);
    }
    for (int o = 32; o > 0; o >>= 1) {
        cnt += __shfl_xor(cnt, o, 64);
        bad |= __shfl_xor(bad, o, 64);
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt | (bad << 30);
    __syncthreads();
    if (threadIdx.x == 0) {
        int c = 0, f = 0;
        for (int i = 0; i < 4; ++i) {
            c += red[i] & ((1 << 30) - 1);
            f |= red[i] >> 30;
        }
        cu[b + 1] = c | (f << 30);
    }
}

// Padded path, step 2: scan the row lengths into cu_seqlens, then counts and tiles.
__global__ __launch_bounds__(1024) void unpad_scan_kernel(int* __restrict__ cu, int B, int max_pos,
                                                          int* __restrict__ meta, int total_max) {
    __shared__ int lds[32];
    __shared__ int s_status, s_maxlen;
    const MetaView mv = meta_view(meta, total_max, B);
    if (threadIdx.x == 0) {
        s_status = 0;
        s_maxlen = 0;
    }
    __syncthreads();
    int carry = 0, status = 0, maxlen = 0;
    for (int base = 0; base < B; base += blockDim.x) {
        const int b = base + threadIdx.x;
        int L = 0;
        if (b < B) {
            const int v = cu[b + 1];
            L = v & ((1 << 30) - 1);
            if (v >> 30) status |= MBERT_STATUS_BAD_MASK;
            if (L > max_pos) status |= MBERT_STATUS_TOO_LONG;
            maxlen = max(maxlen, L);
        }
        int tot;
        const int ex = block_excl_scan(L, lds, tot);
        if (b < B) cu[b + 1] = carry + ex + L;
        carry += tot;
    }
    if (threadIdx.x == 0) cu[0] = 0;
    if (status) atomicOr(&s_status, status);
    atomicMax(&s_maxlen, maxlen);
    __syncthreads();
    status = s_status;
    const bool ok = (status & MBERT_STATUS_TOO_LONG) == 0;
    build_tiles(cu, B, ok, mv, lds);
    if (threadIdx.x == 0) {
        mv.counts[MBERT_META_TOTAL] = carry;
        mv.counts[MBERT_META_MAXLEN] = ok ? s_maxlen : 0;
        mv.counts[MBERT_META_STATUS] = status;
        for (int i = 4; i < 8; ++i) mv.counts[i] = 0;
    }
}

// Padded path, step 3: compact each row: ids, flat indices, positions (rank among the row's
// real tokens) and the padded-slot -> packed-row map (-1 at pads).
__global__ __launch_bounds__(256) void unpad_compact_kernel(const int* __restrict__ ids_pad,
                                                            const int* __restrict__ mask, int Tpad,
                                                            const int* __restrict__ cu,
                                                            int* __restrict__ ids,
                                                            int* __restrict__ indices,
                                                            int* __restrict__ rowmap,
                                                            int* __restrict__ meta, int total_max,
                                                            int B) {
    __shared__ int wsum[4];
    const MetaView mv = meta_view(meta, total_max, B);
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = cu[b];
    int carry = 0;
    for (int t0 = 0; t0 < Tpad; t0 += blockDim.x) {
        const int t = t0 + threadIdx.x;
        const long slot = (long)b * Tpad + t;
        const int real = (t < Tpad) ? (mask[slot] != 0) : 0;
        const unsigned long long bal = __ballot(real);
        const int below = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (lane == 0) wsum[w] = __popcll(bal);
        __syncthreads();
        int woff = 0, tot = 0;
        for (int i = 0; i < 4; ++i) {
            if (i < w) woff += wsum[i];
            tot += wsum[i];
        }
        const int rank = carry + woff + below;
        if (t < Tpad) {
            if (real) {
                const int k = base + rank;
                ids[k] = ids_pad[slot];
                indices[k] = (int)slot;
                mv.pos[k] = rank;
                rowmap[slot] = k;
            } else {
                rowmap[slot] = -1;
            }
        }
        carry += tot;
        __syncthreads();
    }
}

// Padded path in one workgroup (small batches): the three steps above in a single launch. One
// pass over the B x Tpad slots in row-major chunks of 1024: a block-wide exclusive scan of the
// real-token flags gives each real slot its packed row k (tokens are packed row by row, so k
// counts the real slots before it), the first slot of row b records cu[b], and the position is
// k - cu[b]. All mask and id loads are issued before the first scan; cu_seqlens and the packed
// rows stay in LDS and registers (no global round trip between the steps).
constexpr int UNPAD_FUSED_CHUNKS = 16;  // slots per thread: up to 16 x 1024 slots
constexpr int UNPAD_FUSED_SLOTS = UNPAD_FUSED_CHUNKS * 1024;
__global__ __launch_bounds__(1024) void unpad_fused_kernel(const int* __restrict__ ids_pad,
                                                           const int* __restrict__ mask, int B,
                                                           int Tpad, int max_pos,
                                                           int* __restrict__ ids,
                                                           int* __restrict__ indices,
                                                           int* __restrict__ rowmap,
                                                           int* __restrict__ cu,
                                                           int* __restrict__ meta, int total_max) {
    __shared__ int lds[32];
    __shared__ int wcnt[16];  // real slots per wave of the current chunk
    __shared__ int s_status, s_maxlen;
    __shared__ int s_cu[UNPAD_FUSED_SLOTS + 1];  // the launcher keeps B <= UNPAD_FUSED_SLOTS
    const MetaView mv = meta_view(meta, total_max, B);
    const int n = B * Tpad, tid = threadIdx.x;
    if (tid == 0) {
        s_status = 0;
        s_maxlen = 0;
    }
    int mv_[UNPAD_FUSED_CHUNKS] = {}, idv[UNPAD_FUSED_CHUNKS] = {}, kv[UNPAD_FUSED_CHUNKS] = {};
    if (n > 0) {
#pragma unroll
        for (int c = 0; c < UNPAD_FUSED_CHUNKS; ++c) {
            const int slot = min(c * 1024 + tid, n - 1);  // past the end: re-read the last slot
            mv_[c] = mask[slot];
            idv[c] = ids_pad[slot];
        }
    }
    if (Tpad == 0)  // B rows without a slot: B empty sequences
        for (int b = tid; b <= B; b += blockDim.x) {
            s_cu[b] = 0;
            cu[b] = 0;
        }
    __syncthreads();
    int carry = 0, bad = 0;
#pragma unroll
    for (int c = 0; c < UNPAD_FUSED_CHUNKS; ++c) {
        if (c * 1024 >= n) break;  // uniform
        const int slot = c * 1024 + tid;
        const bool in = slot < n;
        const int real = in && mv_[c] != 0;
        bad |= in && mv_[c] != 0 && mv_[c] != 1;
        // exclusive prefix of the 0/1 flags: ballot and population count within the wave, then
        // the counts of the waves before it
        const int lane = tid & 63, wv = tid >> 6;
        const unsigned long long bal = __ballot(real);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wcnt[wv] = __popcll(bal);
        __syncthreads();
        int woff = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int cw = wcnt[w];
            woff += w < wv ? cw : 0;
            tot += cw;
        }
        __syncthreads();  // wcnt is rewritten by the next chunk
        const int k = carry + woff + below;
        kv[c] = k;
        const int b = in ? slot / Tpad : 0;
        if (in && slot == b * Tpad) {
            s_cu[b] = k;
            cu[b] = k;
        }
        if (in) {
            rowmap[slot] = real ? k : -1;
            if (real) {
                ids[k] = idv[c];
                indices[k] = slot;
            }
        }
        carry += tot;
    }
    if (tid == 0 && Tpad > 0) {
        s_cu[B] = carry;
        cu[B] = carry;
    }
    __syncthreads();  // s_cu complete
    // positions: rank among the row's real tokens
#pragma unroll
    for (int c = 0; c < UNPAD_FUSED_CHUNKS; ++c) {
        const int slot = c * 1024 + tid;
        if (c * 1024 >= n) break;
        if (slot < n && mv_[c] != 0) mv.pos[kv[c]] = kv[c] - s_cu[slot / Tpad];
    }
    int status = bad ? MBERT_STATUS_BAD_MASK : 0, maxlen = 0;
    for (int b = tid; b < B; b += blockDim.x) {
        const int L = s_cu[b + 1] - s_cu[b];
        if (L > max_pos) status |= MBERT_STATUS_TOO_LONG;
        maxlen = max(maxlen, L);
    }
    if (status) atomicOr(&s_status, status);
    atomicMax(&s_maxlen, maxlen);
    __syncthreads();
    status = s_status;
    const bool ok = (status & MBERT_STATUS_TOO_LONG) == 0;
    build_tiles(s_cu, B, ok, mv, lds);
    if (tid == 0) {
        mv.counts[MBERT_META_TOTAL] = carry;
        mv.counts[MBERT_META_MAXLEN] = ok ? s_maxlen : 0;
        mv.counts[MBERT_META_STATUS] = status;
        for (int i = 4; i < 8; ++i) mv.counts[i] = 0;
    }
}

// Per-token key ranges through the attention kernel's own band function.
__global__ __launch_bounds__(TILE) void key_range_kernel(const int* __restrict__ meta, int total_max,
                                                         int S, int is_global, int W,
                                                         int* __restrict__ lo, int* __restrict__ hi) {
    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    const int b = blockIdx.x;
    if (b >= mv.counts[MBERT_META_NTILES]) return;
    const int4 tl = mv.tiles[b];
    const int t = threadIdx.x;
    if (t >= tl.y) return;
    int l, h;
    key_range(tl.x + t, tl.z, tl.w, is_global, W, l, h);
    lo[tl.x + t] = l;
    hi[tl.x + t] = h;
}

// Re-pad: 64 threads per padded row, 12 floats each.
__global__ __launch_bounds__(256) void repad_kernel(const float* __restrict__ out,
                                                    const int* __restrict__ rowmap, long rows,
                                                    float* __restrict__ out_pad) {
    const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const int k = rowmap[r];
    float4* dst = reinterpret_cast<float4*>(out_pad + r * D);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k >= 0) v = reinterpret_cast<const float4*>(out + (long)k * D)[lane + 64 * c];
        dst[lane + 64 * c] = v;
    }
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_rope_tables(float* table, int max_pos, double theta_g, double theta_l, hipStream_t s) {
    const long n = 2L * max_pos * (HD / 2);
    MB_LAUNCH((rope_table_kernel), (unsigned)((n + 255) / 256), 256, 0, s, reinterpret_cast<float2*>(table),
                                                                  max_pos, theta_g, theta_l);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_pack_meta(const int32_t* cu, int n_seqs, int total, int max_pos, int32_t* meta,
                     hipStream_t s) {
    MB_LAUNCH((pack_meta_kernel), 1, 1024, 0, s, cu, n_seqs, total, max_pos, meta, total);
    MB_CHECK_LAUNCH();
    const size_t tmax = tiles_max_for(total, n_seqs);
    if (tmax > 0) {
        MB_LAUNCH((pos_kernel), (unsigned)tmax, TILE, 0, s, meta, total, n_seqs);
        MB_CHECK_LAUNCH();
    }
    return MBERT_OK;
}

int launch_padded_meta(const int32_t* mask, int B, int Tpad, int max_pos, int32_t* meta,
                       hipStream_t s) {
    MB_LAUNCH((padded_meta_kernel), 1, 1024, 0, s, mask, B, Tpad, max_pos, meta);
    MB_CHECK_LAUNCH();
    const size_t tmax = tiles_max_for(B * Tpad, B);
    if (tmax > 0) {
        MB_LAUNCH((pos_kernel), (unsigned)tmax, TILE, 0, s, meta, B * Tpad, B);
        MB_CHECK_LAUNCH();
    }
    return MBERT_OK;
}

int launch_unpad(const int32_t* ids_pad, const int32_t* mask, int B, int Tpad, int max_pos,
                 int32_t* ids, int32_t* indices, int32_t* rowmap, int32_t* cu, int32_t* meta,
                 hipStream_t s) {
    const int total_max = B * Tpad;
    if ((long)B * Tpad <= UNPAD_FUSED_SLOTS && B <= UNPAD_FUSED_SLOTS) {
        MB_LAUNCH((unpad_fused_kernel), 1, 1024, 0, s, ids_pad, mask, B, Tpad, max_pos, ids, indices, rowmap,
                  cu, meta, total_max);
        MB_CHECK_LAUNCH();
        return MBERT_OK;
    }
    if (B > 0) {
        MB_LAUNCH((unpad_count_kernel), B, 256, 0, s, mask, Tpad, cu);
        MB_CHECK_LAUNCH();
    }
    MB_LAUNCH((unpad_scan_kernel), 1, 1024, 0, s, cu, B, max_pos, meta, total_max);
    MB_CHECK_LAUNCH();
    if (B > 0) {
        MB_LAUNCH((unpad_compact_kernel), B, 256, 0, s, ids_pad, mask, Tpad, cu, ids, indices, rowmap, meta,
                                              total_max, B);
        MB_CHECK_LAUNCH();
    }
    return MBERT_OK;
}

int launch_key_ranges(const int32_t* meta, int total_max, int n_seqs, int is_global, int W,
                      int32_t* lo, int32_t* hi, hipStream_t s) {
    const size_t tmax = tiles_max_for(total_max, n_seqs);
    if (tmax == 0) return MBERT_OK;
    MB_LAUNCH((key_range_kernel), (unsigned)tmax, TILE, 0, s, meta, total_max, n_seqs, is_global, W, lo, hi);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

int launch_repad(const float* out, const int32_t* rowmap, int B, int Tpad, float* out_pad,
                 hipStream_t s) {
    const long rows = (long)B * Tpad;
    if (rows == 0) return MBERT_OK;
    MB_LAUNCH((repad_kernel), (unsigned)((rows + 3) / 4), 256, 0, s, out, rowmap, rows, out_pad);
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

}  // namespace mbh
