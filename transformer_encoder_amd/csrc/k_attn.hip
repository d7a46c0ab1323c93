// Varlen bidirectional attention for one layer: o = softmax(q k^T / 8 + mask) v per head,
// keys restricted to the query's own sequence, and on local layers to |i - j| <= W
// (kgptalkie, "ModernBERT-base Architecture Teardown", §"How Does Self-Attention Work?",
// §"What Are Local and Global Attention?"; candding, "ModernBERT", §"The alternating
// attention").
//
// Work: one workgroup per (work tile of <= 128 query rows of one sequence, head); 4 wave64s,
// 32 query rows each. K/V tiles of 64 keys stream through two LDS stages, one tile ahead: the
// 16-bit types load them from global memory straight into the stage (buffer loads into LDS),
// fp32 through registers, with unconditional loads. The workgroup walks only the keys its
// band can reach: the whole sequence on a global layer, [q0 - W, q0 + qn - 1 + W] on a local
// one; a wave whose own band misses a key tile skips its MFMAs for it. On a grid of at most
// one workgroup per CU (16-bit types), the workgroup has 8 waves: the second four take the
// odd key tiles, two tiles are staged per step, and the two online-softmax states of each
// query are merged at the end (the usual rescale-and-add of partial softmax sums).
//
// Layout trick: each wave computes S^T = K Q^T (32x32 MFMA blocks: rows = keys,
// columns = queries), so every lane owns one query column: the row max, row sum and the
// rescaling of the output are per-lane, with one cross-lane exchange (lane ^ 32) for the max.
// The probabilities then feed O^T = V^T P^T directly as the MFMA B operand (no shuffle);
// V is staged in its natural [key][d] layout like K, and each lane's 8 keys at its d come
// from two transposed LDS reads (ds_read_b64_tr_b16). The MFMA k-slots of both operands
// follow the same key permutation (lane group g holds keys 4g..4g+3 and 8+4g..8+4g+3 of each
// 16-key slice), which leaves the product unchanged.
// Softmax is online in fp32 with exp2 and the scale 0.125 * log2(e) folded into one FMA; edge
// tiles are masked branch-free (a per-lane bit mask of the allowed keys); the running max is only
// raised (and the output rescaled) when a row's max grows by more than 2^8, and only then are
// the two half-row maxima of a query (lanes l and l ^ 32) exchanged.
// The fp32 variant uses v_mfma_f32_32x32x2_f32 and padded natural K and V rows.
#include "common.hpp"

// fp32: K/V tiles held in registers ahead of the LDS stage (with register staging for every
// type, a second register stage gained 2-3 % on 8192-key global layers and lost as much on
// short sequences).
#ifndef MB_ATTN_PREFETCH
#define MB_ATTN_PREFETCH 1
#endif
// Largest grid ((work tile, head) pairs) run with the key tiles split over two wave sets: one
// workgroup per CU at most. Beyond that some CUs hold two 8-wave workgroups and set the pace
// (a 2445-token batch in 264 workgroups: global layer 16.1 -> 17.2 us, while 132 workgroups
// of half of it gain 12.7 -> 11.1 us).
#ifndef MB_ATTN_SPLIT_MAX_WG
#define MB_ATTN_SPLIT_MAX_WG 256
#endif

namespace mb {
constexpr int ATTN_SPLIT_MAX_WG = MB_ATTN_SPLIT_MAX_WG;


template <typename T> struct AttnCfg {
    static constexpr bool F32 = sizeof(T) == 4;
    // K row pitch, elements ([key][d]); the 16-bit layout is unpadded (128-byte rows) and
    // XOR-swizzled by 16-byte chunk (kchunk): conflict-free both for the 16-byte row writes
    // and for the 16-byte reads of 16 rows at one chunk
    static constexpr int KP = F32 ? 68 : 64;
    static constexpr int VP = F32 ? 68 : 64;   // V pitch, [key][d]; 16-bit: unpadded, vchunk
    static constexpr int KSZ = 64 * KP;
    static constexpr int VSZ = 64 * VP;
};

// Byte offset of 16-byte chunk c (0..7) of K row r in the 16-bit layout: chunk c sits at slot
// c ^ ((r >> 1) & 7); rows r and r + 1 differ by half of the 256-byte bank window, pairs of
// rows by the slot.
__device__ __forceinline__ int kchunk(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Transposed 8-byte LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane j gets
// element j % 4 of the 4-element rows read by lanes j / 4, 4 + j / 4, 8 + j / 4, 12 + j / 4.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// Byte offset of 16-byte chunk c of V row (key) r in the 16-bit layout: chunk c at slot
// c ^ (4 * bit 1 of r). A transposed read takes four rows of 64 bytes (keys 4g.. of a 16-key
// slice, d 32 db..) per half wave: the two rows of one parity land on disjoint slots.
__device__ __forceinline__ int vchunk(int r, int c) { return r * 128 + ((c ^ (((r >> 1) & 1) << 2)) << 4); }

template <typename T> struct Mma;
template <> struct Mma<bf16> {
    __device__ __forceinline__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static u32x4 pack(const float* p) {
        bf16x8 v = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3],
                    (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
        return __builtin_bit_cast(u32x4, v);
    }
};
template <> struct Mma<f16> {
    __device__ __forceinline__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static u32x4 pack(const float* p) {
        f16x8 v = {(f16)p[0], (f16)p[1], (f16)p[2], (f16)p[3],
                   (f16)p[4], (f16)p[5], (f16)p[6], (f16)p[7]};
        return __builtin_bit_cast(u32x4, v);
    }
};

// KS: key-tile sets per workgroup (1: 4 waves; 2: 8 waves, split keys, 16-bit types only)
template <typename T, int KS>
__global__ __launch_bounds__(256 * KS, KS == 1 ? 2 : 1) void attn_kernel(
    const T* __restrict__ qkv, T* __restrict__ out, const int* __restrict__ meta, int total_max,
    int S, int tiles_max, int is_global, int W, float scale_log2) {
    using C = AttnCfg<T>;
    constexpr bool F32 = C::F32;
    static_assert(KS == 1 || (KS == 2 && !F32), "key halves for the 16-bit types");
    // [stage][key half]: with KS = 2 the workgroup stages two key tiles per step, one per half
    __shared__ __align__(16) T Ks[2][KS][C::KSZ];
    __shared__ __align__(16) T Vs[2][KS][C::VSZ];

    const MetaView mv = meta_view(const_cast<int*>(meta), total_max, S);
    // (head, tile) pairs of the real tile count, spread over the XCDs in contiguous ranges:
    // the query tiles of one head (which read the same keys) share an L2
    const int n_tiles = mv.counts[MBERT_META_NTILES];
    const int n_act = NH * n_tiles;
    const int per = (n_act + NXCD - 1) / NXCD;
    const int local = blockIdx.x / NXCD;
    if (local >= per) return;
    const int lin = (blockIdx.x % NXCD) * per + local;
    if (lin >= n_act) return;
    // On global layers whose grid takes more than one round of workgroup slots (3 per CU),
    // the tiles of each head in the meta block's dispatch order (longer sequences first), so
    // that the longest workgroups do not start last (a 64-sequence batch of 32-2048 tokens:
    // 3-5 % faster). Local tiles all cost about the same, and a grid that fits at once does not
    // wait for late starters: both keep the row order, which measured 1-5 % better for them.
    const int head = lin / n_tiles;
    const int tile = (is_global && n_act > 3 * 256) ? mv.order[lin % n_tiles] : lin % n_tiles;
    const int4 tl = mv.tiles[tile];
    const int q0 = tl.x, qn = tl.y, s0 = tl.z, s1 = tl.w;

    // wave w: queries 32 (w % 4) .. +31 of the tile, key tiles kh, kh + KS, kh + 2 KS, ...
    // (kh = w / 4); staging thread tid loads key tile KS i + sh of step i (sh = tid / 256)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qg = wave & 3, kh = wave >> 2;
    const int stid = tid & 255, sh = tid >> 8;
    const int n = lane & 31, g = lane >> 5;
    const int qw0 = q0 + 32 * qg;
    const int qcnt = min(32, qn - 32 * qg);

    int klo, khi, tmp;
    key_range(q0, s0, s1, is_global, W, klo, tmp);
    key_range(q0 + qn - 1, s0, s1, is_global, W, tmp, khi);
    if (khi < klo) {
        // no key for any query of the tile (pad rows of a padded batch run at full width,
        // beyond the window of every real key): zero outputs, as for fully masked rows
        for (int idx = threadIdx.x; idx < qn * (HD / 4); idx += blockDim.x)
            Vec4<T>::store(out + (size_t)(q0 + idx / (HD / 4)) * D + head * HD + 4 * (idx % (HD / 4)),
                           make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const int nkt = (khi - klo) / 64 + 1;

    // this lane's query (loads clamped into the tile) and its band
    const int qrow = q0 + min(32 * qg + n, qn - 1);
    int qlo, qhi;
    key_range(qw0 + n, s0, s1, is_global, W, qlo, qhi);
    // keys valid for every query of the wave: [lo of the last query, hi of the first]
    int wlo = 1, whi = 0, all_lo = 1, all_hi = 0;
    if (qcnt > 0) {
        key_range(qw0, s0, s1, is_global, W, wlo, all_hi);
        key_range(qw0 + qcnt - 1, s0, s1, is_global, W, all_lo, whi);
    }

    // ---- Q fragment (MFMA B operand: column = query, 16-byte k-chunks)
    constexpr int NQ = F32 ? 8 : 4;
    u32x4 qf[NQ];
    {
        const T* qp = qkv + (size_t)qrow * QKV + head * HD;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int d = F32 ? (8 * c + 4 * g) : (16 * c + 8 * g);
            qf[c] = *(const u32x4*)(qp + d);
        }
    }

    // ---- K/V staging
    constexpr int KCH = F32 ? 4 : 2;  // 16-byte chunks per thread for K (and V for fp32)
    constexpr int AP = MB_ATTN_PREFETCH;  // K/V tiles held in registers ahead of the LDS stage
    u32x4 rk[AP][KCH], rv[AP][KCH];
    auto gload = [&](int step, int u) {
        const int kb = klo + 64 * min(KS * step + sh, nkt - 1);
        if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int key = min(kb + (tid >> 4) + 16 * i, khi);
                const T* src = qkv + (size_t)key * QKV + head * HD + (tid & 15) * 4;
                rk[u][i] = *(const u32x4*)(src + D);
                rv[u][i] = *(const u32x4*)(src + 2 * D);
            }
        } else {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int key = min(kb + (stid >> 3) + 32 * i, khi);
                rk[u][i] = *(const u32x4*)(qkv + (size_t)key * QKV + D + head * HD + (stid & 7) * 8);
            }
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int key = min(kb + (stid >> 3) + 32 * i, khi);
                rv[u][i] = *(const u32x4*)(qkv + (size_t)key * QKV + 2 * D + head * HD + (stid & 7) * 8);
            }
        }
    };
    auto sstore = [&](int st, int u) {
        if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int off = ((tid >> 4) + 16 * i) * C::KP + (tid & 15) * 4;
                *(u32x4*)(&Ks[st][sh][off]) = rk[u][i];
                *(u32x4*)(&Vs[st][sh][off]) = rv[u][i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < KCH; ++i)
                *(u32x4*)(reinterpret_cast<unsigned char*>(&Ks[st][sh][0]) + kchunk((stid >> 3) + 32 * i, stid & 7)) = rk[u][i];
#pragma unroll
            for (int i = 0; i < KCH; ++i)
                *(u32x4*)(reinterpret_cast<unsigned char*>(&Vs[st][sh][0]) + vchunk((stid >> 3) + 32 * i, stid & 7)) = rv[u][i];
        }
    };

    // 16-bit types: the step's K/V tiles go from global memory straight into the LDS stage
    // (buffer loads into LDS, 16 bytes a lane, 1 KB a wave instruction), with no register
    // staging and no LDS stores (8192-token global layer 253 -> 241 us together with the
    // masking and max exchange below). A step holds 16 KS groups of 1 KB (per key tile 8 of
    // K, then 8 of V; group j = rows 8j .. 8j+7); wave w fills groups w, w + NWV, ...: lane L
    // row 8j + L / 8 at physical chunk L % 8, which holds the logical chunk that kchunk /
    // vchunk place there (both swizzles are their own inverses). One buffer descriptor per
    // key tile, based at its first key and ending at the sequence's last, so offsets stay small
    // for any sequence length and rows past the end load zeros.
    constexpr int NWV = 4 * KS, GPW = 16 * KS / NWV;
    static_assert(F32 || sizeof(Ks[0]) == sizeof(Vs[0]), "K and V stages of one size");
    constexpr unsigned SSTR = (unsigned)sizeof(Ks[0]);  // bytes between stages
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int drow[GPW];
    unsigned dcol[GPW];
    unsigned char* dst0[GPW];  // stage-0 destination of each group (wave-uniform)
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int hh = (NWV * i) / 16, within = wv + NWV * i - 16 * hh, j = within % 8;
        const bool isv = within >= 8;
        const int r = 8 * j + (lane >> 3), pc = lane & 7;
        const int c = isv ? (pc ^ (((r >> 1) & 1) << 2)) : (pc ^ ((r >> 1) & 7));
        drow[i] = r;
        dcol[i] = (unsigned)(((isv ? 2 * D : D) + head * HD + 8 * c) * (int)sizeof(T));
        dst0[i] = (isv ? reinterpret_cast<unsigned char*>(&Vs[0][hh][0])
                       : reinterpret_cast<unsigned char*>(&Ks[0][hh][0])) + 1024 * j;
    }
    // per-lane offsets within a key tile are loop constants; the tile's first key goes into the
    // descriptor base and its row count into the extent, so rows past the sequence's last key
    // (and a tile past the last) read as zeros, which the masking and the zero probabilities
    // of those keys leave without effect
    unsigned voffc[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) voffc[i] = (unsigned)drow[i] * (unsigned)(QKV * sizeof(T)) + dcol[i];
    auto dma = [&](int step, int st) {
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int hh = (NWV * i) / 16;
            const int tix = KS * step + hh;
            const int kbs = klo + 64 * min(tix, nkt - 1);
            const int nrows = tix < nkt ? min(64, khi - kbs + 1) : 0;
            lds_dma16_buf(qkv + (size_t)kbs * QKV, (unsigned)nrows * (unsigned)(QKV * sizeof(T)), voffc[i], 0u,
                          dst0[i] + st * SSTR);
        }
    };
    // the step's DMAs of this wave landed and its LDS reads are done, then the barrier: the
    // stage just filled is visible to all, the one just read may be refilled
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    f32x16 oacc[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        oacc[0][e] = 0.f;
        oacc[1][e] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    // Every load is unconditional (a tile past the last re-reads the last one on the fp32 path
    // and loads zeros on the DMA path): loads under a branch leave the wait-count pass unsure
    // of what is in flight. Step i's tiles are held in register slot i % AP; the loop is
    // unrolled AP times so the slots are static.
    const int nst = (nkt + KS - 1) / KS;  // steps of KS key tiles
    if constexpr (F32) {
#pragma unroll
        for (int u = 0; u < AP; ++u) gload(u, u);
        sstore(0, 0);
        __syncthreads();
    } else {
        // the LDS slots this wave's DMA lanes fill start as zeros, so that rows past a sequence's
        // end hold zeros or earlier keys whether or not the hardware writes its zeros for them
        // (a masked key's probability is 0, and 0 times a stale non-finite value is not)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < GPW; ++i) *(u32x4*)(dst0[i] + st * SSTR + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
        asm volatile("" ::: "memory");
        dma(0, 0);
        publish();
    }
    for (int it0 = 0; it0 < nst; it0 += AP) {
#pragma unroll
    for (int u = 0; u < AP; ++u) {
        const int it = it0 + u;
        if (it >= nst) break;  // uniform over the workgroup
        if constexpr (F32) gload(it + AP, u);
        else dma(it + 1, (it + 1) & 1);  // the stage read in the previous step
        const int t = KS * it + kh;  // this wave's key tile
        const int kb = klo + 64 * t;
        const bool active = t < nkt && qcnt > 0 && kb <= whi && kb + 63 >= wlo;
        if (active) {
            const int st = it & 1;
            // ---- S^T = K Q^T for keys kb .. kb+63 (two 32-key blocks)
            f32x16 sacc[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kk][e] = 0.f;
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const int d = F32 ? (8 * c + 4 * g) : (16 * c + 8 * g);
                    const u32x4 a = F32 ? *(const u32x4*)(&Ks[st][kh][(32 * kk + n) * C::KP + d])
                                        : *(const u32x4*)(reinterpret_cast<const unsigned char*>(&Ks[st][kh][0]) +
                                                          kchunk(32 * kk + n, d / 8));
                    if constexpr (F32) {
                        const f32x4 av = __builtin_bit_cast(f32x4, a), bv = __builtin_bit_cast(f32x4, qf[c]);
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            sacc[kk] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[x], bv[x], sacc[kk], 0, 0, 0);
                    } else {
                        Mma<T>::run(a, qf[c], sacc[kk]);
                    }
                }
            }
            // ---- online softmax (per lane = per query), branch-free masking
            const bool need_mask = is_global ? (kb + 63 > khi) : !(kb >= all_lo && kb + 63 <= all_hi);
            float sv[32];
            float mx = -INFINITY;
            if (need_mask) {
                // key of element e = kb + 4g + [32kk + 8(e/4) + (e%4)]: the allowed keys, relative
                // to kb + 4g, are lo_rel .. hi_rel; as bits of one word per 32-key block, each
                // element's bit sign-extended to a select mask (two VALU operations an element,
                // no compare results in SGPRs)
                const int lo_rel = qlo - (kb + 4 * g), hi_rel = qhi - (kb + 4 * g);
                unsigned wbits[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int lo = max(lo_rel - 32 * kk, 0), hi = min(hi_rel - 32 * kk, 31);
                    wbits[kk] = hi >= lo ? (0xffffffffu >> (31 - (hi - lo))) << lo : 0u;
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int rel = 8 * (e >> 2) + (e & 3);
                        const unsigned m = (unsigned)((int)(wbits[kk] << (31 - rel)) >> 31);
                        // through a scalar: a bit cast of the vector element itself reads
                        // element 0 with this compiler
                        const float sval = sacc[kk][e];
                        const float x = __builtin_bit_cast(
                            float, (__builtin_bit_cast(unsigned, sval) & m) | (~m & 0xff800000u));
                        sv[16 * kk + e] = x;
                        mx = fmaxf(mx, x);
                    }
            } else {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        sv[16 * kk + e] = sacc[kk][e];
                        mx = fmaxf(mx, sacc[kk][e]);
                    }
            }
            mx *= scale_log2;  // this lane's half of the row, log2 units
            // Lazy rescale: the running max only moves (and O, l are rescaled) when some lane's
            // max exceeds it by more than 8; otherwise exp2 arguments stay <= 8 (p <= 256).
            // Softmax is invariant to the subtracted constant, so the result is the same. The
            // two halves of a query's row (lanes l and l ^ 32) share m_run: it only moves to
            // the maximum over both, exchanged here (8192-token global layer: 1-3 % against an
            // exchange on every tile).
            if (__any(mx > m_run + 8.0f)) {
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    oacc[0][e] *= alpha;
                    oacc[1][e] *= alpha;
                }
                m_run = m_new;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2, -m_use));
                lsum += sv[i];
            }
            l_run += lsum;
            // ---- O^T += V^T P^T
            if constexpr (F32) {
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = 32 * kk + 8 * (e >> 2) + 4 * g + (e & 3);
                            const float a = Vs[st][kh][key * C::VP + 32 * db + n];
                            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sv[16 * kk + e], oacc[db], 0, 0, 0);
                        }
            } else {
                u32x4 pb[2][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int h = 0; h < 2; ++h) pb[kk][h] = Mma<T>::pack(&sv[16 * kk + 8 * h]);
                // V^T fragments by transposed reads: in each 16-lane group, lane m reads the
                // 4 values of V row 4g + m/4 (of the 16-key slice) at d 32 db + 16 (bit 4 of
                // the lane) + 4 (m % 4); the read hands lane n the 4 keys 4g..4g+3 at d 32 db + n
                const int m16 = lane & 15, q4 = lane >> 4;
                const int rowoff = 4 * (q4 >> 1) + (m16 >> 2);
                const int cb = 2 * (q4 & 1) + ((m16 >> 1) & 1), xsw = ((rowoff >> 1) & 1) << 2;
                const unsigned char* vb =
                    reinterpret_cast<const unsigned char*>(&Vs[st][kh][0]) + rowoff * 128 + (m16 & 1) * 8;
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const unsigned char* p = vb + (((4 * db + cb) ^ xsw) << 4) + (32 * kk + 16 * h) * 128;
                            const u32x2 lo = lds_read_tr16(p);            // keys 4g .. 4g+3
                            const u32x2 hi = lds_read_tr16(p + 8 * 128);  // keys 8+4g .. 8+4g+3
                            const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                            Mma<T>::run(a, pb[kk][h], oacc[db]);
                        }
            }
        }
        if constexpr (F32) {
            if (it + 1 < nst) sstore((it + 1) & 1, (u + 1) % AP);
            __syncthreads();
        } else {
            publish();
        }
    }
    }

    if constexpr (KS == 2) {
        // Merge the key halves (every wave is past the loop's last barrier, so the V stages
        // are free): waves 4-7 leave their running max, sum and output in LDS, waves 0-3 add
        // them in on the larger of the two maxima. A half that saw no key has max -inf and
        // weight 0.
        float* xs = reinterpret_cast<float*>(&Ks[0][0][0]) + qg * 2 * 64 + lane;  // max, sum
        float* xm = reinterpret_cast<float*>(&Vs[0][0][0]) + qg * 32 * 64 + lane;  // outputs
        static_assert(sizeof(Ks) >= 4 * 2 * 64 * sizeof(float) && sizeof(Vs) >= 4 * 32 * 64 * sizeof(float),
                      "merge area");
        if (kh == 1) {
            xs[0] = m_run;
            xs[64] = l_run;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) xm[(16 * db + e) * 64] = oacc[db][e];
        }
        __syncthreads();
        if (kh == 1) return;
        const float m1 = xs[0], l1 = xs[64];
        const float mm = fmaxf(m_run, m1);
        const float f0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
        const float f1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        l_run = l_run * f0 + l1 * f1;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] = oacc[db][e] * f0 + xm[(16 * db + e) * 64] * f1;
    }

    // ---- normalise and write: lane holds d = 32 db + 8 j + 4 g + i of its query
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (n < qcnt) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // a query with no key: zeros
        T* op = out + (size_t)(qw0 + n) * D + head * HD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 v = make_float4(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                                             oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
                Vec4<T>::store(op + 32 * db + 8 * j + 4 * g, v);
            }
    }
}

// Attention probabilities of one sequence, every head, written out in full (a debugging and
// inspection path, not the forward's): probs[h][i][j] = softmax over the allowed keys j of
// q_i . k_j / 8 for query rows row0 + i (i < n_q) and key rows row0 + j (j < n_k), positions
// counted from row0; a local layer allows |i - j| <= W (kgptalkie, "ModernBERT-base
// Architecture Teardown", §"How Does Self-Attention Work?", §"What Are Local and Global
// Attention?"). Keys outside the band, and every key of a query that has none, get 0.
// One workgroup per (query, head); each thread owns keys j = tid + 256 k of the row, which it
// keeps in the output row between the max, exponent and normalisation passes.
template <typename T>
__global__ __launch_bounds__(256) void attn_probs_kernel(const T* __restrict__ qkv, int row0,
                                                         int n_q, int n_k, int is_global, int W,
                                                         float* __restrict__ probs) {
    __shared__ float qs[HD];
    __shared__ float red[4];
    const int i = blockIdx.x, head = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    if (tid < HD) qs[tid] = to_f(qkv[(size_t)(row0 + i) * QKV + head * HD + tid]);
    __syncthreads();
    const int lo = is_global ? 0 : max(0, i - W);
    const int hi = is_global ? n_k - 1 : min(n_k - 1, i + W);
    float* row = probs + ((size_t)head * n_q + i) * n_k;
    float mx = -INFINITY;
    for (int j = tid; j < n_k; j += 256) {
        float sc = -INFINITY;
        if (j >= lo && j <= hi) {
            const T* kp = qkv + (size_t)(row0 + j) * QKV + D + head * HD;
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < HD; d += 4) {
                const float4 k4 = Vec4<T>::load(kp + d);
                acc += qs[d] * k4.x + qs[d + 1] * k4.y + qs[d + 2] * k4.z + qs[d + 3] * k4.w;
            }
            sc = acc * 0.125f;
        }
        row[j] = sc;
        mx = fmaxf(mx, sc);
    }
    // block max, then block sum (fixed order over the four waves)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int j = tid; j < n_k; j += 256) {
        const float p = row[j] == -INFINITY ? 0.f : expf(row[j] - mx);
        row[j] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[tid >> 6] = sum;
    __syncthreads();
    sum = ((red[0] + red[1]) + red[2]) + red[3];
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    for (int j = tid; j < n_k; j += 256) row[j] *= inv;
}

}  // namespace mb

namespace mbh {
using namespace mb;

int launch_attention(mbert_dtype dt, const void* qkv, int total, const int32_t* meta, int n_seqs,
                     int is_global, int W, void* o, hipStream_t s) {
    const int tmax = (int)tiles_max_for(total, n_seqs);
    if (tmax == 0) return MBERT_OK;
    const unsigned grid = (unsigned)xcd_grid(NH * tmax);
    const float scale_log2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
    // A grid of at most one workgroup per CU leaves most SIMDs with one wave or none: then
    // each workgroup splits its key tiles over two sets of four waves, which halves the chain
    // of tiles a wave walks (the sets merge their softmax states at the end).
    const bool split = NH * tmax <= ATTN_SPLIT_MAX_WG;
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((attn_kernel<float, 1>), grid, 256, 0, s, (const float*)qkv, (float*)o, meta, total,
                      n_seqs, tmax, is_global, W, scale_log2);
            break;
        case MBERT_BF16:
            if (split)
                MB_LAUNCH((attn_kernel<bf16, 2>), grid, 512, 0, s, (const bf16*)qkv, (bf16*)o, meta, total,
                          n_seqs, tmax, is_global, W, scale_log2);
            else
                MB_LAUNCH((attn_kernel<bf16, 1>), grid, 256, 0, s, (const bf16*)qkv, (bf16*)o, meta, total,
                          n_seqs, tmax, is_global, W, scale_log2);
            break;
        case MBERT_F16:
            if (split)
                MB_LAUNCH((attn_kernel<f16, 2>), grid, 512, 0, s, (const f16*)qkv, (f16*)o, meta, total,
                          n_seqs, tmax, is_global, W, scale_log2);
            else
                MB_LAUNCH((attn_kernel<f16, 1>), grid, 256, 0, s, (const f16*)qkv, (f16*)o, meta, total,
                          n_seqs, tmax, is_global, W, scale_log2);
            break;
        default:
            return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}

}  // namespace mbh

namespace mbh {
int launch_attention_probs(mbert_dtype dt, const void* qkv, int row0, int n_q, int n_k,
                           int is_global, int W, float* probs, hipStream_t s) {
    if (n_q == 0 || n_k == 0) return MBERT_OK;
    const dim3 grid((unsigned)n_q, mb::NH);
    switch (dt) {
        case MBERT_F32:
            MB_LAUNCH((mb::attn_probs_kernel<float>), grid, 256, 0, s, (const float*)qkv, row0, n_q, n_k, is_global, W, probs);
            break;
        case MBERT_BF16:
            MB_LAUNCH((mb::attn_probs_kernel<mb::bf16>), grid, 256, 0, s, (const mb::bf16*)qkv, row0, n_q, n_k, is_global, W, probs);
            break;
        case MBERT_F16:
            MB_LAUNCH((mb::attn_probs_kernel<mb::f16>), grid, 256, 0, s, (const mb::f16*)qkv, row0, n_q, n_k, is_global, W, probs);
            break;
        default: return MBERT_EUNSUPPORTED;
    }
    MB_CHECK_LAUNCH();
    return MBERT_OK;
}
}  // namespace mbh
