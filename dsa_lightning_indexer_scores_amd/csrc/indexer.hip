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
// and the w-weighted head sum run in registers over that lane's 16 heads, and
// lane-row swaps finish the sum over 64 heads, four key tiles at a time.
//
// fp8 prefill epilogue.  ReLU(y) = (y + |y|) / 2 splits the score into
//     1/2 sum_j w_j |q_j . k|   +   1/2 (sum_j w_j q_j) . k.
// The first sum is one v_fma per (head, key) with |y| as a free input
// modifier (the plain form needs a max and an fma).  The second is linear in
// k, so it runs on the matrix core: the head-weighted query is split into
// e4m3 parts with an E8M0 scale per 32-channel block, one MFMA row per part,
// and each part carries the next 4 significant bits of what the earlier parts
// left, so 8 parts leave a residual below 2^-32 of the block's largest value.
// That halves the vector work per MFMA, which is what bounds this kernel on
// gfx950 (the matrix core hides about 4 VALU ops per fp8 MFMA, not 8).
// A query's q_I slab stays in VGPRs for the whole key sweep; k_I rows stream
// through LDS in blocks shared by all waves of the workgroup.  Key blocks past
// the workgroup's last query are never loaded (causal skipping), and no L x L
// matrix exists: scores go to a [queries-of-chunk, visible keys] tile, written
// 64 contiguous keys per store instruction.
#include <algorithm>

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

// ReLU and head weights over this lane's heads (its part of the 64-head sum).
template <int HT>
__device__ __forceinline__ float head_partial(const f32x4 (&acc)[HT], const float (&wv)[HT][4]) {
    float s = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(wv[ht][e], relu(acc[ht][e]), s);
    return s;
}

// Same in the |y| form: s0 + sum_e w'_e |y_e| (w' = w/2).
template <int HT>
__device__ __forceinline__ float head_partial_abs(const f32x4 (&acc)[HT], const float (&wv)[HT][4], float s) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(wv[ht][e], fabsf(acc[ht][e]), s);
    return s;
}

// Finishes the head sums of four key tiles at once: p_i is a lane's partial for tile
// i, and lane row g returns the sum of p_g over the four lane rows, added as
// (rows 0+1) + (rows 2+3).  Three lane-row swaps and three adds replace eight of
// each, and lane row g ends up holding exactly the tile it stores.
__device__ __forceinline__ float rowsum_scatter4(float p0, float p1, float p2, float p3) {
    // swap16(x, y): x' = rows (x0, y0, x2, y2), y' = rows (x1, y1, x3, y3)
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const u32x2 b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
    const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    // swap32(x, y): x' = rows (x0, x1, y0, y1), y' = rows (x2, x3, y2, y3)
    const u32x2 c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Linear-term operand of one wave's two queries: the head-weighted query
// qt = sum_j w_j q_I[j, :] (fp32) as LIN_NP e4m3 parts.  Part p of query q is MFMA
// row 4*(p/2) + 2*q + p%2, so lane row g finds parts 2g, 2g+1 of query 0 in
// accumulator elements 0, 1 and those of query 1 in elements 2, 3.
//
// Scale blocks.  The scaled MFMA numbers K so that bytes 0-15 of the four lane
// rows come first and bytes 16-31 second; its 32-element block b is therefore
// bytes 0-15 (b = 0, 1) or 16-31 (b = 2, 3) of lane rows 2(b%2) and 2(b%2)+1, and
// lane row b supplies that block's scale.  With lane row g holding channels
// 32g..32g+31 (as the k_I fragments do), channel c falls in block
// (c >= 64) + 2 * (c % 32 >= 16).
constexpr int LIN_NP = 8;
struct LinScratch {
    uint8_t part[16][128];   // [row][channel] e4m3 bytes
    uint8_t scale[16][4];    // [row][scale block] E8M0
};

template <int D_I, int HT>
__device__ void build_lin_rows(LinScratch& ls, const uint8_t* __restrict__ qI, const float* __restrict__ w,
                               const int64_t (&qrow)[2], const bool (&valid)[2], int H_I, int lane) {
    const int c = 2 * lane;                                   // this lane's channels c, c+1
    const int blk = (lane >= 32) + 2 * ((lane & 15) >= 8);    // their scale block; its lanes differ in bits 0-2, 4
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        float r0 = 0.f, r1 = 0.f;
        if (valid[q] && c < D_I) {
            // every head's two channels in flight at once (one memory round trip), then the
            // head-weighted sum in head order
            const uint8_t* base = qI + qrow[q] * D_I + c;
            const float* wq = w + qrow[q];
            unsigned short v[16 * HT];
            float wj[16 * HT];
#pragma unroll
            for (int j = 0; j < 16 * HT; ++j) {
                v[j] = j < H_I ? *reinterpret_cast<const unsigned short*>(base + (int64_t)j * D_I) : (unsigned short)0;
                wj[j] = j < H_I ? wq[j] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 16 * HT; ++j) {
                const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(v[j], false);
                if (j < H_I) {
                    r0 = fmaf(wj[j], f[0], r0);
                    r1 = fmaf(wj[j], f[1], r1);
                }
            }
        }
#pragma unroll
        for (int p = 0; p < LIN_NP; ++p) {
            // Block scale: the block's largest |residual| maps into [128, 256), far from
            // e4m3's 448 limit; the byte also carries the 1/2 of the |y| split.
            float m = fmaxf(fabsf(r0), fabsf(r1));
            m = fmaxf(m, __shfl_xor(m, 1));
            m = fmaxf(m, __shfl_xor(m, 2));
            m = fmaxf(m, __shfl_xor(m, 4));
            m = fmaxf(m, __shfl_xor(m, 16));
            const int e = __builtin_amdgcn_frexp_expf(m) - 8;
            const bool ok = e + 126 >= 0;                     // residuals below 2^-118 are dropped
            const float v0 = ok ? ldexpf(r0, -e) : 0.f;
            const float v1 = ok ? ldexpf(r1, -e) : 0.f;
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false) & 0xffff;
            const f32x2 back = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
            r0 -= ldexpf(back[0], e);
            r1 -= ldexpf(back[1], e);
            const int row = 4 * (p >> 1) + 2 * q + (p & 1);
            *reinterpret_cast<unsigned short*>(&ls.part[row][c]) = (unsigned short)pk;
            if ((lane & 23) == 0) ls.scale[row][blk] = (uint8_t)(ok ? e + 126 : 0);   // lanes 0, 8, 32, 40
        }
    }
}

// Head weights of this lane (heads 16*ht + 4g + e) for one query row (NULL -> zeros).
template <int HT>
__device__ __forceinline__ void load_w(float (&wr)[HT][4], const float* wrow, int H_I, int g, float f = 1.f) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = 16 * ht + 4 * g + e;
            wr[ht][e] = (wrow != nullptr && hh < H_I) ? f * wrow[hh] : 0.f;
        }
}

// ---------------------------------------------------------------------------
// Prefill: workgroup = QW*NW consecutive queries of a chunk, all their keys.
// ---------------------------------------------------------------------------
// Two waves per SIMD is the occupancy either workgroup size runs at; saying so keeps the
// compiler from parking MFMA accumulators in AGPRs (each VALU read would then cost a copy).
template <bool FP8, int D_I, int HT, int QW, int NW, int KB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void indexer_prefill_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI_,
    float* __restrict__ scores_, int64_t row_stride, int q_begin_, int nq_, int pos_begin_, int H_I, int seg_blocks,
    const int32_t* __restrict__ run_if, const ic_seq_group grp, int64_t k_seq_bytes, int q_step) {
    if (run_if != nullptr && *run_if == 0) return;            // a refresh that was not needed
    using G = IdxGeom<FP8, D_I>;
    static_assert(KB % 64 == 0, "a key block is stored 64 keys per instruction");
    constexpr int QB = QW * NW;
    constexpr int NT = NW * 64;
    constexpr int NKT = KB / 16;                              // 16-key tiles per block
    constexpr int CHUNKS = KB * G::ROWB / 16;                 // 16-byte pieces per key block
    constexpr int CPT = (CHUNKS + NT - 1) / NT;               // pieces per thread
    constexpr int CPR = G::ROWB / 16;                         // pieces per key row
    constexpr bool LIN = FP8 && QW == 2;                      // |y| epilogue + linear-term MFMA row
    __shared__ __attribute__((aligned(32))) uint8_t lds[2][KB * G::LSTR];
    __shared__ __attribute__((aligned(32))) LinScratch lin_lds[LIN ? NW : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // Late (long) query blocks first.  In a grouped launch the block belongs to one sequence
    // of the group: its rows, positions and keys are that sequence's.
    int blk, nq = nq_, pos_begin = pos_begin_, q_begin = q_begin_;
    const uint8_t* kI = kI_;
    float* scores = scores_;
    if (grp.n > 0) {
        const int gb = grp.blk0[grp.n] - 1 - (int)blockIdx.x;
        const int i = group_find(grp.blk0, grp.n, gb);
        blk = gb - grp.blk0[i];
        nq = grp.row0[i + 1] - grp.row0[i];
        pos_begin = grp.pos0[i];
        q_begin = q_begin_ + grp.row0[i];
        kI = kI_ + (int64_t)grp.seq[i] * k_seq_bytes;
        scores = scores_ + (int64_t)grp.row0[i] * row_stride;
    } else {
        blk = (nq + QB - 1) / QB - 1 - (int)blockIdx.x;
    }
    const int t0 = blk * QB;
    const int t_last = min(t0 + QB, nq) - 1;
    const int nkeys = pos_begin + t_last * q_step + 1;        // keys visible to the block
    const int nkb = (nkeys + KB - 1) / KB;
    // Work item: this query block's key blocks [kb_begin, kb_end).  Scores need no sum
    // across keys, so splitting long rows into segments only balances the load.
    const int kb_begin = (int)blockIdx.y * seg_blocks;
    if (kb_begin >= nkb) return;                              // past the causal edge (whole workgroup)
    const int kb_end = min(nkb, kb_begin + seg_blocks);

    // This wave's queries: A fragments (q_I slabs) and head weights, kept in VGPRs.
    Frag<FP8, D_I> A[QW][HT];
    float wr[QW][HT][4];
    int pq[QW];                                               // absolute position, -1 if no query
    float* srow[QW];
    int64_t qrows[QW];
    bool qvalid[QW];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int t = t0 + wv * QW + q;
        const bool valid = t < nq;
        qvalid[q] = valid;
        pq[q] = valid ? pos_begin + t * q_step : -1;
        srow[q] = scores + (int64_t)(valid ? t : 0) * row_stride + 16 * g + r;
        const int64_t qrow = (int64_t)(q_begin + (valid ? t : 0) * q_step) * H_I;
        qrows[q] = qrow;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + r;
            load_frag<FP8, D_I>(A[q][ht], (valid && h < H_I) ? qI + (qrow + h) * G::ROWB : nullptr, g);
        }
        load_w<HT>(wr[q], valid ? w + qrow : nullptr, H_I, g, LIN ? 0.5f : 1.f);
    }
    i32x8 Alin = {0, 0, 0, 0, 0, 0, 0, 0};
    int sAlin = 0;
    if constexpr (LIN) {
        build_lin_rows<D_I, HT>(lin_lds[wv], qI, w, qrows, qvalid, H_I, lane);
        __syncthreads();
        Alin = *reinterpret_cast<const i32x8*>(&lin_lds[wv].part[r][32 * g]);
        sAlin = lin_lds[wv].scale[r][g];
    }

    // Cooperative k_I block load: piece c -> key c / CPR, byte offset (c % CPR) * 16.
    i32x4 stage[CPT];
    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            // Keys past the block's last visible key re-read that key: their score
            // columns are never stored, and the load needs no branch.
            const int key = min(kb * KB + c / CPR, nkeys - 1);
            if (c < CHUNKS)
                stage[i] = *reinterpret_cast<const i32x4*>(kI + (int64_t)key * G::ROWB + (c % CPR) * 16);
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

    gload(kb_begin);
    lstore(0);
    // Drain every load issued so far (q_I, w, block 0) on all paths, so the loop's only
    // outstanding load is the next k_I block, waited for just before its LDS store.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kb = kb_begin; kb < kb_end; ++kb) {
        const int buf = (kb - kb_begin) & 1;
        if (kb + 1 < kb_end) gload(kb + 1);
        // Software pipeline over the block's tiles: the MFMAs of tile kt are issued before
        // the ReLU / head-sum epilogue of tile kt-1, so matrix and vector units overlap.  The
        // key fragment of tile kt+1 is read from LDS one stage ahead, so no stage waits on
        // LDS before its MFMAs (the scheduler would otherwise run the epilogue first and
        // leave the matrix pipe idle behind it).
        float val[QW][NKT];
        f32x4 acc[2][QW][HT];
        f32x4 lin[2];
        Frag<FP8, D_I> Bcur;
        load_frag_lds<FP8, D_I>(Bcur, &lds[buf][r * G::LSTR], g);
#pragma unroll
        for (int kt = 0; kt <= NKT; ++kt) {
            Frag<FP8, D_I> Bnxt;
            if (kt + 1 < NKT) load_frag_lds<FP8, D_I>(Bnxt, &lds[buf][((kt + 1) * 16 + r) * G::LSTR], g);
            if (kt < NKT) {
#pragma unroll
                for (int q = 0; q < QW; ++q)
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) acc[kt & 1][q][ht] = tile_mma<FP8, D_I>(A[q][ht], Bcur);
                if constexpr (LIN) {
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    lin[kt & 1] = mfma_fp8_k128_scale_a(Alin, sAlin, Bcur.f8, z);
                }
            }
            if (kt > 0) {
                if constexpr (LIN) {
                    const f32x4& l = lin[(kt - 1) & 1];
                    val[0][kt - 1] = head_partial_abs<HT>(acc[(kt - 1) & 1][0], wr[0], l[0] + l[1]);
                    val[1][kt - 1] = head_partial_abs<HT>(acc[(kt - 1) & 1][1], wr[1], l[2] + l[3]);
                } else {
#pragma unroll
                    for (int q = 0; q < QW; ++q) val[q][kt - 1] = head_partial<HT>(acc[(kt - 1) & 1][q], wr[q]);
                }
            }
            if constexpr (LIN && HT == 4) {
                // Interleave within the stage: the next fragment's LDS reads first, then each
                // MFMA followed by four of the epilogue's vector ops.
                if (kt + 1 < NKT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                if (kt > 0 && kt < NKT) {
#pragma unroll
                    for (int i = 0; i < 9; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    }
                }
            }
            // One pipeline stage per scheduling region.  The partials are consumed by an
            // empty asm so their VALU work stays in this stage: otherwise it sinks to the
            // stores, every tile's MFMAs issue first and the live accumulators spill.
            if (kt > 0) {
#pragma unroll
                for (int q = 0; q < QW; ++q) asm volatile("" : "+v"(val[q][kt - 1]));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < NKT) Bcur = Bnxt;
        }
        // Stage the next block first: its wait then covers only that load, not the stores.
        if (kb + 1 < kb_end) lstore(buf ^ 1);
        // Lane row g stores tile 4*grp + g: 64 consecutive keys per query per instruction.
#pragma unroll
        for (int grp = 0; grp < NKT / 4; ++grp) {
            const int s = kb * KB + 64 * grp + 16 * g + r;
#pragma unroll
            for (int q = 0; q < QW; ++q) {
                const float v = rowsum_scatter4(val[q][4 * grp], val[q][4 * grp + 1], val[q][4 * grp + 2],
                                                val[q][4 * grp + 3]);
                if (s <= pq[q]) srow[q][kb * KB + 64 * grp] = v;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Decode: one query per sequence; workgroup = (key range, sequence).  Keys
// stream straight from HBM into B fragments (no reuse to stage in LDS).  A wave
// sweeps DEC_CHUNKS chunks of DEC_TILES 16-key tiles and loads the next chunk
// while it scores the current one, so its q_I slab is loaded once per 256 keys.
// ---------------------------------------------------------------------------
constexpr int DEC_TILES = 4;                                 // 16-key tiles per chunk
constexpr int DEC_CHUNKS = 4;                                // chunks per wave
constexpr int DEC_NW = 4;
constexpr int DEC_KEYS_PER_WAVE = DEC_CHUNKS * DEC_TILES * 16;
constexpr int DEC_KEYS_PER_WG = DEC_NW * DEC_KEYS_PER_WAVE;

template <bool FP8, int D_I, int HT>
__global__ __launch_bounds__(DEC_NW * 64) __attribute__((amdgpu_waves_per_eu(FP8 ? 3 : 2, FP8 ? 3 : 2))) void indexer_decode_kernel(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const int32_t* __restrict__ seq_len, float* __restrict__ scores, int64_t score_stride, int Lk, int H_I) {
    using G = IdxGeom<FP8, D_I>;
    const int b = blockIdx.y;
    const int n = max(1, min(seq_len[b], Lk));              // visible keys (clamped to the cache)
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int key0 = blockIdx.x * DEC_KEYS_PER_WG + wv * DEC_KEYS_PER_WAVE;
    if (key0 >= n) return;

    const uint8_t* kbase = kI + (int64_t)b * Lk * G::ROWB;
    Frag<FP8, D_I> Bf[2][DEC_TILES];
    auto load_chunk = [&](Frag<FP8, D_I> (&B)[DEC_TILES], int c) {
#pragma unroll
        for (int i = 0; i < DEC_TILES; ++i) {
            // keys past the last visible one re-read it: their scores are never stored
            const int s = min(key0 + (c * DEC_TILES + i) * 16 + r, n - 1);
            load_frag_lds<FP8, D_I>(B[i], kbase + (int64_t)s * G::ROWB, g);
        }
    };
    load_chunk(Bf[0], 0);
    Frag<FP8, D_I> A[HT];
    float wr[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = 16 * ht + r;
        load_frag<FP8, D_I>(A[ht], h < H_I ? qI + ((int64_t)b * H_I + h) * G::ROWB : nullptr, g);
    }
    load_w<HT>(wr, w + (int64_t)b * H_I, H_I, g);
    float* srow = scores + (int64_t)b * score_stride;
#pragma unroll
    for (int c = 0; c < DEC_CHUNKS; ++c) {
        const int kc = key0 + c * DEC_TILES * 16;
        if (kc >= n) break;
        if (c + 1 < DEC_CHUNKS) load_chunk(Bf[(c + 1) & 1], c + 1);
        float val[DEC_TILES];
#pragma unroll
        for (int i = 0; i < DEC_TILES; ++i) {
            f32x4 acc[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) acc[ht] = tile_mma<FP8, D_I>(A[ht], Bf[c & 1][i]);
            val[i] = head_partial<HT>(acc, wr);
        }
#pragma unroll
        for (int grp = 0; grp < DEC_TILES / 4; ++grp) {
            const int s = kc + 64 * grp + 16 * g + r;
            const float v = rowsum_scatter4(val[4 * grp], val[4 * grp + 1], val[4 * grp + 2], val[4 * grp + 3]);
            if (s < n) srow[s] = v;
        }
    }
}

constexpr int PREFILL_KB = 128;                              // keys per LDS block

// Key blocks per work item: the longest query block splits into two pieces, or more when
// the launch has few query blocks (at least 512 work items for the longest rows, two per
// CU), and no piece is shorter than 1024 keys, which keeps the per-item set-up (q_I slab,
// linear-term rows) small next to its key sweep.  Measured on the stack32k stack
// (alternating runs, identical indices): two pieces 37.3 ms per step, one 37.3-37.9,
// three 38.4, four 37.8, eight 39.1.
inline int prefill_max_keys(const ic_indexer_args& a);
inline int prefill_seg_blocks(const ic_indexer_args& a, int nblk) {
    const int nkb_max = (prefill_max_keys(a) + PREFILL_KB - 1) / PREFILL_KB;
    const int pieces = std::max(2, (512 + nblk - 1) / std::max(nblk, 1));
    return std::max(1024 / PREFILL_KB, (nkb_max + pieces - 1) / pieces);
}

// Keys visible to the launch's longest row.
inline int prefill_max_keys(const ic_indexer_args& a) {
    if (!a.grp) return a.pos_begin + (a.nq - 1) * a.q_step + 1;
    int m = 1;
    for (int i = 0; i < a.grp->n; ++i) m = std::max(m, a.grp->pos0[i] + a.grp->row0[i + 1] - a.grp->row0[i]);
    return m;
}

template <bool FP8, int D_I, int HT, int NW>
hipError_t prefill_launch(const ic_indexer_args& a, hipStream_t st) {
    constexpr int QW = FP8 ? 2 : 1;
    constexpr int QB = QW * NW;
    ic_seq_group grp{};
    int nblk = (a.nq + QB - 1) / QB;
    if (a.grp) {                                        // query blocks of each sequence, in order
        grp = *a.grp;
        grp.blk0[0] = 0;
        for (int i = 0; i < grp.n; ++i) grp.blk0[i + 1] = grp.blk0[i] + (grp.row0[i + 1] - grp.row0[i] + QB - 1) / QB;
        nblk = grp.blk0[grp.n];
    }
    const int nkb_max = (prefill_max_keys(a) + PREFILL_KB - 1) / PREFILL_KB;
    const int seg_blocks = prefill_seg_blocks(a, nblk);
    const dim3 grid(nblk, (nkb_max + seg_blocks - 1) / seg_blocks);
    hipLaunchKernelGGL((indexer_prefill_kernel<FP8, D_I, HT, QW, NW, PREFILL_KB>), grid, dim3(NW * 64), 0, st,
                       (const uint8_t*)a.q_I, a.w, (const uint8_t*)a.k_I, a.scores, a.row_stride,
                       a.q_begin, a.nq, a.pos_begin, a.H_I, seg_blocks, a.run_if, grp, a.k_seq_bytes,
                       a.grp ? 1 : a.q_step);
    return hipGetLastError();
}

// 4-wave workgroups, two per CU (one wave of each on every SIMD): while one workgroup
// waits at its per-block barrier, the other's MFMAs keep the SIMD's matrix pipe busy,
// and the finer workgroups share CUs better with the top-k and attention launches that
// run beside the indexer in the stack.  Measured on stack32k (alternating runs, identical
// indices): one 32K-query launch 3.33 ms against 3.43 with 8-wave workgroups (one per CU,
// both waves of a SIMD stopping at the same barrier); the 16-layer stack 37.5 ms against
// 39.0.  2-wave workgroups (three per CU, LDS-bound) took 4.2 ms and 42.0 ms.
template <bool FP8, int D_I, int HT>
hipError_t prefill_dispatch(const ic_indexer_args& a, hipStream_t st) {
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
