// Lightning-indexer scores on gfx950 MFMA.
//
// DSA's lightning indexer scores every visible key of every query ("IndexCache:
// Accelerating Sparse Attention via Cross-Layer Index Reuse", arXiv abstract);
// the blog "When the Optimizer Becomes the Bottleneck" (section "The Hidden
// Quadratic") shows it is the O(L^2) term that IndexCache removes from S
// layers.  Score:
//     I[t,s] = sum_j w[t,j] * max(0, q_I[t,j,:] . k_I[s,:]),   s <= p(t).
//
// Tiling.  One 16x16 MFMA output tile holds 16 indexer heads (rows) x 16
// keys (columns).  Lane l gets key l%16 and heads 4*(l/16)..+3, so the ReLU
// (one v_med3) and the w-weighted head sum (one v_fmac) run in registers over
// that lane's 16 heads, and two lane-row swaps finish the sum over 64 heads.
// A query's q_I slab stays in VGPRs for the whole key sweep; k_I rows stream
// through LDS in blocks shared by all waves of the workgroup.  Key blocks past
// the workgroup's last query are never loaded (causal skipping), and no L x L
// matrix exists: scores go to a [queries-of-chunk, visible keys] tile, written
// 64 contiguous keys per store instruction.
#include "common.h"

using namespace ic;

namespace {

template <bool FP8, int D_I>
struct IdxGeom {
    static constexpr int ES = FP8 ? 1 : 2;          // bytes per element
    static constexpr int ROWB = D_I * ES;           // bytes per k_I / q_I head row
    static constexpr int NKC = FP8 ? 1 : D_I / 32;  // MFMAs along K per 16x16 tile
    static constexpr int LSTR = ROWB + 32;          // LDS row stride: 32-byte aligned, skewed banks
};

// A/B fragment of one 16-row slab (16 heads of q_I, or 16 keys of k_I).
//   fp8 : one i32x8, bytes 32*g .. 32*g+31 of the row (K = 128 in one MFMA; rows
//         shorter than 128 bytes are zero-padded in K)
//   bf16: NKC x i32x4, elements 32*kc + 8*g .. +7 (one K = 32 MFMA per kc)
template <bool FP8, int D_I>
struct Frag {
    static constexpr int NKC = IdxGeom<FP8, D_I>::NKC;
    i32x8 f8;
    i32x4 b16[NKC > 0 ? NKC : 1];
};

// Lane (r, g)'s K slice of a 16-row slab from row pointer `row` (NULL -> zeros).
template <bool FP8, int D_I>
__device__ __forceinline__ void load_frag(Frag<FP8, D_I>& f, const uint8_t* row, int g) {
    if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row != nullptr && (D_I >= 128 || 32 * g < D_I)) v = *reinterpret_cast<const i32x8*>(row + 32 * g);
        f.f8 = v;
    } else {
#pragma unroll
        for (int kc = 0; kc < Frag<FP8, D_I>::NKC; ++kc) {
            i32x4 v = {0, 0, 0, 0};
            if (row != nullptr) v = *reinterpret_cast<const i32x4*>(row + (32 * kc + 8 * g) * 2);
            f.b16[kc] = v;
        }
    }
}

// Same slice from a k_I row staged in LDS (always present).
template <bool FP8, int D_I>
__device__ __forceinline__ void load_frag_lds(Frag<FP8, D_I>& f, const uint8_t* row, int g) {
    if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (D_I >= 128 || 32 * g < D_I) v = *reinterpret_cast<const i32x8*>(row + 32 * g);
        f.f8 = v;
    } else {
#pragma unroll
        for (int kc = 0; kc < Frag<FP8, D_I>::NKC; ++kc)
            f.b16[kc] = *reinterpret_cast<const i32x4*>(row + (32 * kc + 8 * g) * 2);
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

// max(x, 0) in one instruction for the finite MFMA outputs.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

// ReLU, head weights, sum over this lane's heads, then over the 4 lane rows.
template <int HT>
__device__ __forceinline__ float head_reduce(const f32x4 (&acc)[HT], const float (&wv)[HT][4]) {
    float s = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(wv[ht][e], relu(acc[ht][e]), s);
    s = sum_xor16(s);
    s = sum_xor32(s);
    return s;
}

// v[g] for lane row g (g < 4).
__device__ __forceinline__ float pick4(float a, float b, float c, float d, int g) {
    return g < 2 ? (g == 0 ? a : b) : (g == 2 ? c : d);
}

// Head weights of this lane (heads 16*ht + 4g + e) for one query row (NULL -> zeros).
template <int HT>
__device__ __forceinline__ void load_w(float (&wr)[HT][4], const float* wrow, int H_I, int g) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = 16 * ht + 4 * g + e;
            wr[ht][e] = (wrow != nullptr && hh < H_I) ? wrow[hh] : 0.f;
        }
}

// ---------------------------------------------------------------------------
// Prefill: workgroup = QW*NW consecutive queries of a chunk, all their keys.
// ---------------------------------------------------------------------------
template <bool FP8, int D_I, int HT, int QW, int NW, int KB>
__global__ __launch_bounds__(NW * 64) void indexer_prefill_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    float* __restrict__ scores, int64_t row_stride, int q_begin, int nq, int pos_begin, int H_I) {
    using G = IdxGeom<FP8, D_I>;
    static_assert(KB % 64 == 0, "a key block is stored 64 keys per instruction");
    constexpr int QB = QW * NW;
    constexpr int NT = NW * 64;
    constexpr int NKT = KB / 16;                              // 16-key tiles per block
    constexpr int CHUNKS = KB * G::ROWB / 16;                 // 16-byte pieces per key block
    constexpr int CPT = (CHUNKS + NT - 1) / NT;               // pieces per thread
    constexpr int CPR = G::ROWB / 16;                         // pieces per key row
    __shared__ __attribute__((aligned(32))) uint8_t lds[2][KB * G::LSTR];

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
    float* srow[QW];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int t = t0 + wv * QW + q;
        const bool valid = t < nq;
        pq[q] = valid ? pos_begin + t : -1;
        srow[q] = scores + (int64_t)(valid ? t : 0) * row_stride + 16 * g + r;
        const int64_t qrow = (int64_t)(q_begin + (valid ? t : 0)) * H_I;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + r;
            load_frag<FP8, D_I>(A[q][ht], (valid && h < H_I) ? qI + (qrow + h) * G::ROWB : nullptr, g);
        }
        load_w<HT>(wr[q], valid ? w + qrow : nullptr, H_I, g);
    }

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
        // Software pipeline over the block's tiles: the MFMAs of tile kt are issued before
        // the ReLU / head-sum epilogue of tile kt-1, so matrix and vector units overlap.
        float val[QW][NKT];
        f32x4 acc[2][QW][HT];
#pragma unroll
        for (int kt = 0; kt <= NKT; ++kt) {
            if (kt < NKT) {
                Frag<FP8, D_I> Bf;
                load_frag_lds<FP8, D_I>(Bf, &lds[buf][(kt * 16 + r) * G::LSTR], g);
#pragma unroll
                for (int q = 0; q < QW; ++q)
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) acc[kt & 1][q][ht] = tile_mma<FP8, D_I>(A[q][ht], Bf);
            }
            if (kt > 0) {
#pragma unroll
                for (int q = 0; q < QW; ++q) val[q][kt - 1] = head_reduce<HT>(acc[(kt - 1) & 1][q], wr[q]);
            }
        }
        // Lane row g stores tile 4*grp + g: 64 consecutive keys per query per instruction.
#pragma unroll
        for (int grp = 0; grp < NKT / 4; ++grp) {
            const int s = kb * KB + 64 * grp + 16 * g + r;
#pragma unroll
            for (int q = 0; q < QW; ++q) {
                const float v = pick4(val[q][4 * grp], val[q][4 * grp + 1], val[q][4 * grp + 2],
                                      val[q][4 * grp + 3], g);
                if (s <= pq[q]) srow[q][kb * KB + 64 * grp] = v;
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
constexpr int DEC_TILES_PER_WAVE = 8;                        // 128 keys per wave
constexpr int DEC_NW = 4;
constexpr int DEC_KEYS_PER_WG = DEC_NW * DEC_TILES_PER_WAVE * 16;

template <bool FP8, int D_I, int HT>
__global__ __launch_bounds__(DEC_NW * 64) void indexer_decode_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, int64_t score_stride, int Lk, int H_I) {
    using G = IdxGeom<FP8, D_I>;
    const int b = blockIdx.y;
    const int n = max(1, min(seq_len[b], Lk));                // visible keys (clamped to the cache)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int key0 = blockIdx.x * DEC_KEYS_PER_WG + wv * DEC_TILES_PER_WAVE * 16;
    if (key0 >= n) return;

    const uint8_t* kbase = kI + (int64_t)b * Lk * G::ROWB;
    Frag<FP8, D_I> Bf[DEC_TILES_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DEC_TILES_PER_WAVE; ++i) {
        const int s = key0 + 16 * i + r;
        load_frag<FP8, D_I>(Bf[i], s < n ? kbase + (int64_t)s * G::ROWB : nullptr, g);
    }
    Frag<FP8, D_I> A[HT];
    float wr[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = 16 * ht + r;
        load_frag<FP8, D_I>(A[ht], h < H_I ? qI + ((int64_t)b * H_I + h) * G::ROWB : nullptr, g);
    }
    load_w<HT>(wr, w + (int64_t)b * H_I, H_I, g);
    float val[DEC_TILES_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DEC_TILES_PER_WAVE; ++i) {
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = tile_mma<FP8, D_I>(A[ht], Bf[i]);
        val[i] = head_reduce<HT>(acc, wr);
    }
    float* srow = scores + (int64_t)b * score_stride;
#pragma unroll
    for (int grp = 0; grp < DEC_TILES_PER_WAVE / 4; ++grp) {
        const int s = key0 + 64 * grp + 16 * g + r;
        const float v = pick4(val[4 * grp], val[4 * grp + 1], val[4 * grp + 2], val[4 * grp + 3], g);
        if (s < n) srow[s] = v;
    }
}

template <bool FP8, int D_I, int HT, int NW>
hipError_t prefill_launch(const ic_indexer_args& a, hipStream_t st) {
    constexpr int QW = FP8 ? 2 : 1;
    constexpr int KB = 64;
    constexpr int QB = QW * NW;
    const int nblk = (a.nq + QB - 1) / QB;
    hipLaunchKernelGGL((indexer_prefill_kernel<FP8, D_I, HT, QW, NW, KB>), dim3(nblk), dim3(NW * 64), 0, st,
                       (const uint8_t*)a.q_I, a.w, (const uint8_t*)a.k_I, a.scores, a.row_stride,
                       a.q_begin, a.nq, a.pos_begin, a.H_I);
    return hipGetLastError();
}

// 8-wave workgroups share each k_I block among 16 queries; when that leaves fewer than
// two workgroups per CU (a 4096-query chunk), 4-wave workgroups keep the CUs fed.
template <bool FP8, int D_I, int HT>
hipError_t prefill_dispatch(const ic_indexer_args& a, hipStream_t st) {
    constexpr int QW = FP8 ? 2 : 1;
    if ((a.nq + QW * 8 - 1) / (QW * 8) >= 512) return prefill_launch<FP8, D_I, HT, 8>(a, st);
    return prefill_launch<FP8, D_I, HT, 4>(a, st);
}

template <bool FP8, int D_I, int HT>
hipError_t decode_dispatch(const ic_indexer_decode_args& a, hipStream_t st) {
    dim3 grid((a.Lk + DEC_KEYS_PER_WG - 1) / DEC_KEYS_PER_WG, a.B);
    hipLaunchKernelGGL((indexer_decode_kernel<FP8, D_I, HT>), grid, dim3(DEC_NW * 64), 0, st,
                       (const uint8_t*)a.q_I, a.w, (const uint8_t*)a.k_I, a.seq_len, a.scores, a.score_stride,
                       a.Lk, a.H_I);
    return hipGetLastError();
}

}  // namespace

// H_I <= 16 uses one head tile; 17..64 heads use four (absent heads get zero rows and weights).
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
