// Lightning-indexer scores on gfx950 MFMA.
//
// The DSA indexer named in "IndexCache: Accelerating Sparse Attention via
// Cross-Layer Index Reuse" (arXiv abstract) scores every visible key of
// every query; the blog "When the Optimizer Becomes the Bottleneck"
// (section "The Hidden Quadratic") shows it is the O(L^2) term.  Score:
//     I[t,s] = sum_j w[t,j] * max(0, q_I[t,j,:] . k_I[s,:]),   s <= p(t).
//
// Tiling.  One 16x16 MFMA output tile holds 16 indexer heads (rows) x 16
// keys (columns).  Lane l gets key l%16 and heads 4*(l/16)..+3, so the ReLU
// and the w-weighted head sum run in registers over that lane's heads, and
// two lane-row swaps finish the sum over the 64 heads.  A query's q_I slab
// stays in VGPRs for the whole key sweep; k_I rows stream through LDS in
// blocks of 64 keys shared by all waves of the workgroup.  Key blocks past
// the workgroup's last query are never loaded (causal skipping), and no
// L x L matrix exists: scores go to a [queries-of-chunk, visible keys] tile.
#include "common.h"

using namespace ic;

namespace {

constexpr int KB = 64;          // keys per LDS block

template <bool FP8, int D_I>
struct IdxGeom {
    static constexpr int ES = FP8 ? 1 : 2;          // bytes per element
    static constexpr int ROWB = D_I * ES;           // bytes per k_I / q_I head row
    static constexpr int NKC = FP8 ? 1 : D_I / 32;  // MFMAs along K per 16x16 tile
    static constexpr int LSTR = ROWB + 16;          // padded LDS row stride (bytes)
};

// A/B fragment of one 16-row slab (16 heads of q_I, or 16 keys of k_I).
template <bool FP8, int D_I>
struct Frag {
    static constexpr int NKC = IdxGeom<FP8, D_I>::NKC;
    // fp8: one i32x8 (32 bytes of K per lane); bf16: NKC x i32x4 (8 bf16 of each K=32 chunk)
    i32x8 f8;
    i32x4 b16[NKC > 0 ? NKC : 1];
};

// Load lane (r, g)'s K slice of a 16-row slab from row pointer `row` (NULL -> zeros).
template <bool FP8, int D_I>
__device__ __forceinline__ void load_frag(Frag<FP8, D_I>& f, const uint8_t* row, int g) {
    if constexpr (FP8) {
        i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        if (row != nullptr && 32 * g < D_I) {
            lo = *reinterpret_cast<const i32x4*>(row + 32 * g);
            hi = *reinterpret_cast<const i32x4*>(row + 32 * g + 16);
        }
        f.f8 = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
#pragma unroll
        for (int kc = 0; kc < Frag<FP8, D_I>::NKC; ++kc) {
            i32x4 v = {0, 0, 0, 0};
            if (row != nullptr) v = *reinterpret_cast<const i32x4*>(row + (32 * kc + 8 * g) * 2);
            f.b16[kc] = v;
        }
    }
}

template <bool FP8, int D_I>
__device__ __forceinline__ f32x4 tile_mma(const Frag<FP8, D_I>& a, const Frag<FP8, D_I>& b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FP8) {
        acc = mfma_fp8_k128(a.f8, b.f8, acc);
    } else {
#pragma unroll
        for (int kc = 0; kc < Frag<FP8, D_I>::NKC; ++kc) acc = mfma_bf16_k32(a.b16[kc], b.b16[kc], acc);
    }
    return acc;
}

// ReLU, head weights, sum over this lane's heads, then over the 4 lane rows.
template <int HT>
__device__ __forceinline__ float head_reduce(const f32x4 (&acc)[HT], const float (&wv)[HT][4]) {
    float s = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(wv[ht][e], fmaxf(acc[ht][e], 0.f), s);
    s = sum_xor16(s);
    s = sum_xor32(s);
    return s;
}

// ---------------------------------------------------------------------------
// Prefill: workgroup = QW*NW consecutive queries of a chunk, all their keys.
// ---------------------------------------------------------------------------
template <bool FP8, int D_I, int HT, int QW, int NW>
__global__ __launch_bounds__(NW * 64) void indexer_prefill_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    float* __restrict__ scores, int64_t row_stride, int q_begin, int nq, int pos_begin, int H_I) {
    using G = IdxGeom<FP8, D_I>;
    constexpr int QB = QW * NW;
    constexpr int NT = NW * 64;
    constexpr int CHUNKS = KB * G::ROWB / 16;                 // 16-byte pieces per key block
    constexpr int CPT = (CHUNKS + NT - 1) / NT;               // pieces per thread
    constexpr int CPR = G::ROWB / 16;                         // pieces per key row
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][KB * G::LSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nblk = (nq + QB - 1) / QB;
    const int blk = nblk - 1 - (int)blockIdx.x;               // late (long) query blocks first
    const int t0 = blk * QB;
    const int t_last = min(t0 + QB, nq) - 1;
    const int nkeys = pos_begin + t_last + 1;                 // keys visible to the block
    const int nkb = (nkeys + KB - 1) / KB;

    // This wave's queries: A fragments (q_I slabs) and head weights, kept in VGPRs.
    Frag<FP8, D_I> A[QW][HT];
    float wr[QW][HT][4];
    int pq[QW];                                               // absolute position, -1 if no query
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int t = t0 + wv * QW + q;
        const bool valid = t < nq;
        pq[q] = valid ? pos_begin + t : -1;
        const int64_t qrow = (int64_t)(q_begin + (valid ? t : 0)) * H_I;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + r;
            const uint8_t* p = (valid && h < H_I) ? qI + (qrow + h) * G::ROWB : nullptr;
            load_frag<FP8, D_I>(A[q][ht], p, g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int hh = 16 * ht + 4 * g + e;
                wr[q][ht][e] = (valid && hh < H_I) ? w[qrow + hh] : 0.f;
            }
        }
    }
    int p_wave = -1;
#pragma unroll
    for (int q = 0; q < QW; ++q) p_wave = max(p_wave, pq[q]);

    // Cooperative k_I block load: piece c -> key c / CPR, byte offset (c % CPR) * 16.
    i32x4 stage[CPT];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int key = kb * KB + c / CPR;
            i32x4 v = {0, 0, 0, 0};
            if (c < CHUNKS && key < nkeys)
                v = *reinterpret_cast<const i32x4*>(kI + (int64_t)key * G::ROWB + (c % CPR) * 16);
            stage[i] = v;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            if (c < CHUNKS)
                *reinterpret_cast<i32x4*>(&lds[buf][(c / CPR) * G::LSTR + (c % CPR) * 16]) = stage[i];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nkb) gload(kb + 1);
#pragma unroll
        for (int kt = 0; kt < KB / 16; ++kt) {
            const int s0 = kb * KB + kt * 16;
            if (s0 > p_wave) break;                           // every key of the tile is in the future
            Frag<FP8, D_I> Bf;
            const uint8_t* brow = &lds[buf][(kt * 16 + r) * G::LSTR];
            if constexpr (FP8) {
                i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
                if (32 * g < D_I) {
                    lo = *reinterpret_cast<const i32x4*>(brow + 32 * g);
                    hi = *reinterpret_cast<const i32x4*>(brow + 32 * g + 16);
                }
                Bf.f8 = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
#pragma unroll
                for (int kc = 0; kc < G::NKC; ++kc)
                    Bf.b16[kc] = *reinterpret_cast<const i32x4*>(brow + (32 * kc + 8 * g) * 2);
            }
            float val[QW];
#pragma unroll
            for (int q = 0; q < QW; ++q) {
                f32x4 acc[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[ht] = tile_mma<FP8, D_I>(A[q][ht], Bf);
                val[q] = head_reduce<HT>(acc, wr[q]);
            }
            // lane row g stores query g's 16 scores (keys s0 .. s0+15)
            const int s = s0 + r;
#pragma unroll
            for (int q = 0; q < QW; ++q) {
                if (g == q && pq[q] >= 0 && s <= pq[q]) {
                    const int t = t0 + wv * QW + q;
                    scores[(int64_t)t * row_stride + s] = val[q];
                }
            }
        }
        if (kb + 1 < nkb) lstore(buf ^ 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Decode: one query per sequence; workgroup = (key range, sequence).  Keys
// stream straight from HBM into B fragments (no reuse to stage in LDS).
// ---------------------------------------------------------------------------
constexpr int DEC_TILES_PER_WAVE = 4;                        // 64 keys per wave
constexpr int DEC_NW = 4;
constexpr int DEC_KEYS_PER_WG = DEC_NW * DEC_TILES_PER_WAVE * 16;

template <bool FP8, int D_I, int HT>
__global__ __launch_bounds__(DEC_NW * 64) void indexer_decode_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, int Lk, int H_I) {
    using G = IdxGeom<FP8, D_I>;
    const int b = blockIdx.y;
    const int n = max(1, min(seq_len[b], Lk));          // visible keys (clamped to the cache)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int key0 = blockIdx.x * DEC_KEYS_PER_WG + wv * DEC_TILES_PER_WAVE * 16;
    if (key0 >= n) return;

    Frag<FP8, D_I> A[HT];
    float wr[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = 16 * ht + r;
        load_frag<FP8, D_I>(A[ht], h < H_I ? qI + ((int64_t)b * H_I + h) * G::ROWB : nullptr, g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = 16 * ht + 4 * g + e;
            wr[ht][e] = hh < H_I ? w[(int64_t)b * H_I + hh] : 0.f;
        }
    }
    const uint8_t* kbase = kI + (int64_t)b * Lk * G::ROWB;
    Frag<FP8, D_I> Bf[DEC_TILES_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DEC_TILES_PER_WAVE; ++i) {
        const int s = key0 + 16 * i + r;
        load_frag<FP8, D_I>(Bf[i], s < n ? kbase + (int64_t)s * G::ROWB : nullptr, g);
    }
    float* srow = scores + (int64_t)b * Lk;
#pragma unroll
    for (int i = 0; i < DEC_TILES_PER_WAVE; ++i) {
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = tile_mma<FP8, D_I>(A[ht], Bf[i]);
        const float v = head_reduce<HT>(acc, wr);
        const int s = key0 + 16 * i + r;
        if (g == 0 && s < n) srow[s] = v;
    }
}

template <bool FP8, int D_I, int HT>
hipError_t prefill_dispatch(const ic_indexer_args& a, hipStream_t st) {
    constexpr int QW = FP8 ? 2 : 1;
    constexpr int NW = 8;
    constexpr int QB = QW * NW;
    const int nblk = (a.nq + QB - 1) / QB;
    hipLaunchKernelGGL((indexer_prefill_kernel<FP8, D_I, HT, QW, NW>), dim3(nblk), dim3(NW * 64), 0, st,
                       (const uint8_t*)a.q_I, a.w, (const uint8_t*)a.k_I, a.scores, a.row_stride,
                       a.q_begin, a.nq, a.pos_begin, a.H_I);
    return hipGetLastError();
}

template <bool FP8, int D_I, int HT>
hipError_t decode_dispatch(const ic_indexer_decode_args& a, hipStream_t st) {
    dim3 grid((a.Lk + DEC_KEYS_PER_WG - 1) / DEC_KEYS_PER_WG, a.B);
    hipLaunchKernelGGL((indexer_decode_kernel<FP8, D_I, HT>), grid, dim3(DEC_NW * 64), 0, st,
                       (const uint8_t*)a.q_I, a.w, (const uint8_t*)a.k_I, a.seq_len, a.scores, a.Lk, a.H_I);
    return hipGetLastError();
}

}  // namespace

#define IC_DISPATCH_SHAPE(FN, ARGS, ST)                                                     \
    do {                                                                                    \
        const bool big = (ARGS).H_I > 16;                                                   \
        if ((ARGS).fp8) {                                                                   \
            if ((ARGS).d_I == 128) return big ? FN<true, 128, 4>(ARGS, ST) : FN<true, 128, 1>(ARGS, ST); \
            if ((ARGS).d_I == 64) return big ? FN<true, 64, 4>(ARGS, ST) : FN<true, 64, 1>(ARGS, ST);    \
            if ((ARGS).d_I == 32) return big ? FN<true, 32, 4>(ARGS, ST) : FN<true, 32, 1>(ARGS, ST);    \
        } else {                                                                            \
            if ((ARGS).d_I == 128) return big ? FN<false, 128, 4>(ARGS, ST) : FN<false, 128, 1>(ARGS, ST); \
            if ((ARGS).d_I == 64) return big ? FN<false, 64, 4>(ARGS, ST) : FN<false, 64, 1>(ARGS, ST);    \
            if ((ARGS).d_I == 32) return big ? FN<false, 32, 4>(ARGS, ST) : FN<false, 32, 1>(ARGS, ST);    \
        }                                                                                   \
        return hipErrorInvalidValue;                                                        \
    } while (0)

hipError_t launch_indexer_prefill(const ic_indexer_args& a, hipStream_t st) {
    if (a.nq <= 0) return hipSuccess;
    IC_DISPATCH_SHAPE(prefill_dispatch, a, st);
}

hipError_t launch_indexer_decode(const ic_indexer_decode_args& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    IC_DISPATCH_SHAPE(decode_dispatch, a, st);
}
