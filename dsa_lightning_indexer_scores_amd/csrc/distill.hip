// Multi-layer distillation loss, forward only, on gfx950.
//
// "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
// (arXiv abstract): training-aware IndexCache trains each retained indexer
// against the averaged attention distributions of all the layers it serves
// (gist.science summary, "Methodologie": an F layer predicts the attention of
// itself and of the S layers after it, through a KL divergence to their
// average).  Per query t, over its selected entries S_t (the F layer's top-k):
//     p_t[s] = mean over served layers j and heads h of softmax_s(q_j[t,h] . K_j[s] / sqrt(d))
//     r_t[s] = softmax_s(I[t, s])              (the F layer's indexer scores)
//     loss_t = KL(p_t || r_t) = sum_s p_t[s] (ln p_t[s] - ln r_t[s])
// An entry of -1, or one outside the keys the query sees, is not part of S_t.
//
// One workgroup per query; its four waves split the entries.  For every served
// layer and group of 16 heads: a first sweep gathers the entries' K rows
// (coalesced whole-row loads through the wave's LDS tile, as in the sparse
// attention) and keeps each head's running max and exp-sum; the waves merge
// those; a second sweep recomputes the logits and adds each entry's
// probability, summed over the 16 heads with DPP row adds, into a per-entry
// LDS accumulator.  Then the indexer scores at the entries (read from the score
// tile the indexer kernel wrote) give log r, and the workgroup sums p (log p -
// log r).  Everything runs in the exp2/log2 domain (v_exp_f32, v_log_f32);
// every sum is taken in a fixed order, so the result is deterministic.
#include "common.h"

using namespace ic;

namespace {

constexpr int DW = 4;                   // waves per workgroup
constexpr int DKT = 32;                 // entries per step

template <int D>
struct DGeom {
    static constexpr int NDC = D / 32;  // K=32 chunks of the contraction
    static constexpr int RB = 4 * D;    // bytes per [K | V] row
    static constexpr int KB = 2 * D;    // bytes of its K part
    static constexpr int PPR = KB / 16; // 16-byte pieces of a K part
    static constexpr int RPI = 64 / PPR;    // K parts per load instruction
    static constexpr int NI = DKT / RPI;    // load instructions per step
    static constexpr int STR = KB + 16;     // LDS bytes per staged K part (16-byte skew)
    static_assert(NI % 4 == 0, "row offsets are read four at a time");
};

__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Sum over the 16 lanes of each lane row (DPP), result in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    return x;
}

// Merge two (max, exp2-sum) pairs of the same head; m = -inf marks "nothing seen".
__device__ __forceinline__ void merge_stat(float& m, float& z, float m2, float z2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) { m = M; z = 0.f; return; }
    z = z * __builtin_amdgcn_exp2f(m - M) + z2 * __builtin_amdgcn_exp2f(m2 - M);
    m = M;
}

template <int D>
__global__ __launch_bounds__(DW * 64) void distill_kl_kernel(ic_distill_args a, float scale_log2) {
    using G = DGeom<D>;
    __shared__ __attribute__((aligned(16))) uint8_t ktile_all[DW][DKT * G::STR];
    __shared__ __attribute__((aligned(16))) uint32_t ioff_all[DW][DKT];
    __shared__ float p_lds[IC_DISTILL_MAX_K];
    __shared__ float wstat[DW][16][2];
    __shared__ float wred[DW];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int r = blockIdx.x;                                 // row of the score tile
    const int t = a.q_begin + r;                              // query
    const int vis = min(a.pos0 + t + 1, a.Lk);                // keys the query sees
    const int k = a.k;
    const int32_t* irow = a.idx + (int64_t)t * k;
    const float* srow = a.scores + (int64_t)r * a.score_stride;
    uint8_t* ktile = ktile_all[wv];
    uint32_t* ioff = ioff_all[wv];
    const int per = ((k + DW - 1) / DW + DKT - 1) / DKT * DKT;
    const int e_begin = wv * per, e_end = min(k, e_begin + per);
    const int nsteps = e_end > e_begin ? (e_end - e_begin + DKT - 1) / DKT : 0;
    const int HG = (a.H + 15) / 16;
    const float inv_cnt = 1.f / (float)(a.nserved * a.H);

    for (int e = e_begin + lane; e < e_end; e += 64) p_lds[e] = 0.f;   // the wave's own entries
    // emask[e]: all ones in the lanes with n % 4 == e (kept opaque so the selection by it
    // stays bitwise and is not turned into an indexed scratch access)
    uint32_t emask[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        emask[e] = ((n & 3) == e) ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(emask[e]));
    }

    struct Tile {
        i32x4 raw[G::NI];                                     // the step's K parts, as loaded
        uint32_t valid;                                       // bit e: entry e of the step is in S_t
    };
    auto load_entry = [&](int e0) -> int {                    // raw idx of entry e0 + lane (lanes < 32)
        const int e = e0 + (lane & 31);
        const int v = irow[min(e, e_end - 1)];                // unconditional load: no branch around it
        return (e < e_end && lane < 32) ? v : -1;
    };
    auto issue = [&](Tile& T, int raw, const uint8_t* kvb) {
        __builtin_amdgcn_sched_barrier(0);
        const bool ok = (uint32_t)raw < (uint32_t)vis;
        T.valid = (uint32_t)__ballot(ok);
        const uint32_t row = ok ? (uint32_t)raw : 0u;          // a real row, masked later
        // row offsets through the wave's LDS words, de-interleaved: entry RPI*i + q -> slot q*NI + i
        if (lane < DKT) ioff[(lane % G::RPI) * G::NI + lane / G::RPI] = row * (uint32_t)G::RB;
        lds_wave_sync();
        uint32_t roff[G::NI];
#pragma unroll
        for (int i = 0; i < G::NI; i += 4) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(ioff + (lane / G::PPR) * G::NI + i);
            roff[i] = v[0]; roff[i + 1] = v[1]; roff[i + 2] = v[2]; roff[i + 3] = v[3];
        }
        const uint32_t piece = (lane % G::PPR) * 16;
#pragma unroll
        for (int i = 0; i < G::NI; ++i) T.raw[i] = *reinterpret_cast<const i32x4*>(kvb + (roff[i] + piece));
    };
    // S^T of a step: lane (n, g) gets head n of the group, entries 16*kt + 4g + e (log2 units,
    // -inf for entries outside S_t).
    auto logits = [&](const Tile& T, const i32x4* qf, float x[8]) {
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
            *reinterpret_cast<i32x4*>(ktile + (G::RPI * i + lane / G::PPR) * G::STR + (lane % G::PPR) * 16) = T.raw[i];
        lds_wave_sync();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < G::NDC; ++dc) {
                const i32x4 kf = *reinterpret_cast<const i32x4*>(ktile + (16 * kt + n) * G::STR + 64 * dc + 16 * g);
                acc = mfma_bf16_k32(kf, qf[dc], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[4 * kt + e] = ((T.valid >> (16 * kt + 4 * g + e)) & 1u) ? acc[e] * scale_log2 : -INFINITY;
        }
        lds_wave_sync();                                      // the tile is rewritten by the next step
    };
    // One sweep over the wave's entries; f(x, step_begin) sees each step's logits.
    auto sweep = [&](const uint8_t* kvb, const i32x4* qf, auto&& f) {
        if (nsteps == 0) return;
        Tile TA, TB;
        int iA = load_entry(e_begin), iB = load_entry(e_begin + DKT);
        issue(TA, iA, kvb);
        float x[8];
        int s = 0;
        for (; s + 2 < nsteps; s += 2) {
            iA = load_entry(e_begin + (s + 2) * DKT);
            issue(TB, iB, kvb);
            logits(TA, qf, x);
            f(x, e_begin + s * DKT);
            iB = load_entry(e_begin + (s + 3) * DKT);
            issue(TA, iA, kvb);
            logits(TB, qf, x);
            f(x, e_begin + (s + 1) * DKT);
        }
        if (s + 1 < nsteps) {
            issue(TB, iB, kvb);
            logits(TA, qf, x);
            f(x, e_begin + s * DKT);
            logits(TB, qf, x);
            f(x, e_begin + (s + 1) * DKT);
        } else {
            logits(TA, qf, x);
            f(x, e_begin + s * DKT);
        }
    };

    for (int j = 0; j < a.nserved; ++j) {
        const uint8_t* kvb = static_cast<const uint8_t*>(a.kv[j]);
        const uint16_t* qj = static_cast<const uint16_t*>(a.q[j]);
        for (int hg = 0; hg < HG; ++hg) {
            const int head = 16 * hg + n;
            i32x4 qf[G::NDC];                                 // Q^T fragments: head n, d = 32*dc + 8g .. +7
#pragma unroll
            for (int dc = 0; dc < G::NDC; ++dc) {
                i32x4 v = {0, 0, 0, 0};
                if (head < a.H) v = *reinterpret_cast<const i32x4*>(qj + ((int64_t)t * a.H + head) * D + 32 * dc + 8 * g);
                qf[dc] = v;
            }
            // Sweep 1: each head's max and exp2-sum over S_t.
            float m = -INFINITY, z = 0.f;
            sweep(kvb, qf, [&](const float x[8], int) {
                float mx = x[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) mx = fmax_nan(mx, x[e]);
                if (mx > m) {
                    z *= __builtin_amdgcn_exp2f(m - mx);
                    m = mx;
                }
                if (m != -INFINITY) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) z += __builtin_amdgcn_exp2f(x[e] - m);
                }
            });
            {
                // The four lanes of a head (g = 0..3): each swap hands a lane its own value and
                // its partner's (lane rows 0<->1, 2<->3, then halves), in the same order for m
                // and z; the merge is symmetric, so both lanes get the same result.
                u32x2 mm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                u32x2 zz = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
                m = __uint_as_float(mm[0]); z = __uint_as_float(zz[0]);
                merge_stat(m, z, __uint_as_float(mm[1]), __uint_as_float(zz[1]));
                mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                zz = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
                m = __uint_as_float(mm[0]); z = __uint_as_float(zz[0]);
                merge_stat(m, z, __uint_as_float(mm[1]), __uint_as_float(zz[1]));
            }
            if (g == 0) { wstat[wv][n][0] = m; wstat[wv][n][1] = z; }
            __syncthreads();
            float M = -INFINITY, Z = 0.f;
#pragma unroll
            for (int w = 0; w < DW; ++w) merge_stat(M, Z, wstat[w][n][0], wstat[w][n][1]);
            __syncthreads();                                  // wstat is rewritten by the next group
            // Sweep 2: add every entry's probability, summed over the group's heads.
            const float w_head = (head < a.H && Z > 0.f) ? inv_cnt / Z : 0.f;
            sweep(kvb, qf, [&](const float x[8], int e0) {
                float c[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) c[e] = row16_sum(__builtin_amdgcn_exp2f(x[e] - M) * w_head);
                // lane (n < 4, g) adds entries 16*kt + 4g + n
                if (n < 4) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        uint32_t vb = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) vb |= __float_as_uint(c[4 * kt + e]) & emask[e];
                        const float v = __uint_as_float(vb);
                        const int e = e0 + 16 * kt + 4 * g + n;
                        if (e < e_end) p_lds[e] += v;
                    }
                }
            });
        }
    }

    // The indexer's distribution over S_t: log2 r = I*log2(e) - log2 sum exp2(I*log2(e)).
    // Entries go eight per lane at a time, with unconditional (clamped) loads, so each
    // block costs one memory round trip.
    constexpr float LOG2E = 1.4426950408889634f;
    auto for_entries = [&](auto&& f) {                        // f(entry, score*log2e) for the wave's entries in S_t
        for (int eb = e_begin; eb < e_end; eb += 64 * 8) {
            int sv[8];
            float iv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) sv[u] = irow[min(eb + 64 * u + lane, e_end - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) iv[u] = srow[min((uint32_t)sv[u], (uint32_t)(vis - 1))] * LOG2E;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = eb + 64 * u + lane;
                if (e < e_end && (uint32_t)sv[u] < (uint32_t)vis) f(e, iv[u]);
            }
        }
    };
    float imax = -INFINITY;
    for_entries([&](int, float v) { imax = fmaxf(imax, v); });
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) imax = fmaxf(imax, __shfl_xor(imax, sh));
    if (lane == 0) wred[wv] = imax;
    __syncthreads();
    float GM = -INFINITY;
#pragma unroll
    for (int w = 0; w < DW; ++w) GM = fmaxf(GM, wred[w]);
    __syncthreads();
    float isum = 0.f;
    for_entries([&](int, float v) { isum += __builtin_amdgcn_exp2f(v - GM); });
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) isum += __shfl_xor(isum, sh);
    if (lane == 0) wred[wv] = isum;
    __syncthreads();
    float IZ = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) IZ += wred[w];
    __syncthreads();
    const float lse2 = GM + __builtin_amdgcn_logf(IZ);         // v_log_f32 is log2
    float part = 0.f;
    for_entries([&](int e, float v) {
        const float p = p_lds[e];
        if (p > 0.f) part += p * (__builtin_amdgcn_logf(p) - (v - lse2));
    });
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) part += __shfl_xor(part, sh);
    if (lane == 0) wred[wv] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
        float kl = 0.f;
#pragma unroll
        for (int w = 0; w < DW; ++w) kl += wred[w];
        a.kl[t] = kl * 0.6931471805599453f;                   // log2 units -> nats
    }
}

// Mean of n values in a fixed order: one workgroup, per-thread strided sums, then a tree.
__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int64_t n, float* __restrict__ out) {
    __shared__ double part[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)x[i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = (float)(part[0] / (double)n);
}

}  // namespace

hipError_t launch_distill(const ic_distill_args& a, hipStream_t st) {
    if (a.nrows <= 0) return hipSuccess;
    if (a.k < 1 || a.k > IC_DISTILL_MAX_K || a.nserved < 1 || a.nserved > IC_DISTILL_MAX_SERVED)
        return hipErrorInvalidValue;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)a.d));
    if (a.d == 128)
        hipLaunchKernelGGL((distill_kl_kernel<128>), dim3((unsigned)a.nrows), dim3(DW * 64), 0, st, a, scale_log2);
    else if (a.d == 64)
        hipLaunchKernelGGL((distill_kl_kernel<64>), dim3((unsigned)a.nrows), dim3(DW * 64), 0, st, a, scale_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t st) {
    if (n <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, st, x, n, out);
    return hipGetLastError();
}
