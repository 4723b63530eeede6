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
// One workgroup per query; its eight waves split the entries.  For every served
// layer and group of 16 heads: a first sweep gathers the entries' K halves
// straight into the wave's LDS stage (global_load_lds_dwordx4, as in the sparse
// attention; the next step's halves fly while a step's statistics are computed)
// and keeps each head's running max and exp-sum; the waves merge those; a second
// sweep recomputes the logits and adds each entry's probability, summed over the
// 16 heads with DPP row adds, into a per-entry LDS accumulator.  Each wave's row
// offsets are read from the idx row once, into LDS, for all of its sweeps.  Then the indexer scores at the entries (read from the score
// tile the indexer kernel wrote) give log r, and the workgroup sums p (log p -
// log r).  Everything runs in the exp2/log2 domain (v_exp_f32, v_log_f32);
// every sum is taken in a fixed order, so the result is deterministic.
#include "common.h"

using namespace ic;

namespace {

// Waves per workgroup (one query): each keeps one step in flight, so more waves per CU
// hide more of the gather latency.  Eight (80 KB of LDS per workgroup at k = 2048, two
// workgroups per CU) measured faster than four or two.
constexpr int DW = 8;
constexpr int DKT = 32;                 // entries per step

template <int D>
struct DGeom {
    static constexpr int NDC = D / 32;  // K=32 chunks of the contraction
    static constexpr int RB = 4 * D;    // bytes per [K | V] row
    static constexpr int KB = 2 * D;    // bytes of its K part
    static constexpr int NCH = KB / 16; // 16-byte chunks of a K part
    static constexpr int RPI = 1024 / KB;   // K parts per DMA instruction (64 lanes x 16 bytes)
    static constexpr int NI = DKT / RPI;    // DMA instructions per step
    static constexpr int SB = DKT * KB;     // bytes of a staged step
    static_assert(NI % 4 == 0, "row offsets are read four at a time");
};
constexpr uint32_t NO_ROW = 0xFFFFFFFFu;   // an entry outside S_t

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
__global__ __launch_bounds__(DW * 64) void distill_kl_kernel(ic_distill_args a, float scale_log2, int per) {
    using G = DGeom<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t ktile_all[DW][G::SB];
    __shared__ float wstat[DW][16][2];
    __shared__ float wred[DW];
    // dynamic: p [round_up(k, 4)] floats, then each wave's row offsets [DW][per]
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int r = blockIdx.x;                                 // row of the score tile
    const int t = a.q_begin + r;                              // query
    const int vis = min(a.pos0 + t + 1, a.Lk);                // keys the query sees
    const int k = a.k;
    const int32_t* irow = a.idx + (int64_t)t * k;
    const float* srow = a.scores + (int64_t)r * a.score_stride;
    float* p_lds = reinterpret_cast<float*>(dyn_lds);
    uint32_t* offs = dyn_lds + ((k + 3) & ~3) + wv * per;    // this wave's entries' row offsets
    const uint8_t* ktile = ktile_all[wv];
    const uint32_t k_lds = lds_addr(ktile);
    const int e_begin = wv * per, e_end = min(k, e_begin + per);
    const int nsteps = e_end > e_begin ? (e_end - e_begin + DKT - 1) / DKT : 0;
    const int HG = (a.H + 15) / 16;
    const float inv_cnt = 1.f / (float)(a.nserved * a.H);

    for (int e = e_begin + lane; e < e_end; e += 64) p_lds[e] = 0.f;   // the wave's own entries
    // Row byte offsets of the wave's entries (NO_ROW outside S_t), step by step and
    // de-interleaved so that a lane reads its DMA addresses as one vector: entry RPI*i + q
    // of a step -> slot q*NI + i.  Eight unconditional (clamped) loads per lane per block.
    for (int xb = 0; xb < nsteps * DKT; xb += 64 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = irow[min(e_begin + xb + 64 * u + lane, e_end - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int x = xb + 64 * u + lane, j = x % DKT;
            const bool ok = e_begin + x < e_end && (uint32_t)v[u] < (uint32_t)vis;
            if (x < nsteps * DKT)
                offs[x - j + (j % G::RPI) * G::NI + j / G::RPI] = ok ? (uint32_t)v[u] * (uint32_t)G::RB : NO_ROW;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");       // the wave reads only its own offsets
    // emask[e]: all ones in the lanes with n % 4 == e (kept opaque so the selection by it
    // stays bitwise and is not turned into an indexed scratch access)
    uint32_t emask[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        emask[e] = ((n & 3) == e) ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(emask[e]));
    }
    // Lane l of DMA instruction i fetches chunk (l % NCH) ^ swz(row) of staged row RPI*i + l / NCH.
    uint32_t cof[G::NI];
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
        cof[i] = ((uint32_t)(lane % G::NCH) ^ dma_swz<G::NCH>(G::RPI * i + lane / G::NCH)) * 16u;
    const uint32_t swz_k = dma_swz<G::NCH>(n);
    // Step s's K halves -> the wave's stage (entries outside S_t fetch row 0); returns the
    // step's valid entries as a wave-uniform mask.
    auto issue = [&](const uint8_t* kvb, int s) -> uint32_t {
        const uint32_t* so = offs + s * DKT;
        const uint32_t ev = so[(lane % G::RPI) * G::NI + (lane & 31) / G::RPI];   // entry lane % 32
        const uint32_t valid = (uint32_t)__ballot(ev != NO_ROW);
        uint32_t roff[G::NI];
#pragma unroll
        for (int i = 0; i < G::NI; i += 4) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(so + (lane / G::NCH) * G::NI + i);
            roff[i] = w[0]; roff[i + 1] = w[1]; roff[i + 2] = w[2]; roff[i + 3] = w[3];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the stage's previous reads are done
#pragma unroll
        for (int i = 0; i < G::NI; ++i) dma_b128(kvb, (roff[i] == NO_ROW ? 0u : roff[i]) + cof[i], k_lds + 1024u * i);
        return __builtin_amdgcn_readfirstlane(valid);
    };
    // One sweep over the wave's entries; f(x, step_begin) sees each step's logits: lane (n, g)
    // gets head n of the group, entries 16*kt + 4g + e (log2 units, -inf outside S_t).
    // Step s+1's halves are issued as soon as step s's are read, and land while f runs.
    auto sweep = [&](const uint8_t* kvb, const i32x4* qf, auto&& f) {
        if (nsteps == 0) return;
        uint32_t valid = issue(kvb, 0);
        for (int s = 0; s < nsteps; ++s) {
            wait_vm<0>();                                    // step s landed
            float x[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dc = 0; dc < G::NDC; ++dc) {
                    const i32x4 kf = *reinterpret_cast<const i32x4*>(ktile + (16 * kt + n) * G::KB +
                                                                     (((uint32_t)(4 * dc + g) ^ swz_k) * 16u));
                    acc = mfma_bf16_k32(kf, qf[dc], acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[4 * kt + e] = ((valid >> (16 * kt + 4 * g + e)) & 1u) ? acc[e] * scale_log2 : -INFINITY;
            }
            const uint32_t valid_next = s + 1 < nsteps ? issue(kvb, s + 1) : 0u;
            f(x, e_begin + s * DKT);
            valid = valid_next;
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
    const int per = ((a.k + DW - 1) / DW + DKT - 1) / DKT * DKT;              // entries per wave
    const size_t dyn = (size_t)(((a.k + 3) & ~3) + DW * per) * sizeof(uint32_t);
    if (a.d == 128)
        hipLaunchKernelGGL((distill_kl_kernel<128>), dim3((unsigned)a.nrows), dim3(DW * 64), dyn, st, a, scale_log2, per);
    else if (a.d == 64)
        hipLaunchKernelGGL((distill_kl_kernel<64>), dim3((unsigned)a.nrows), dim3(DW * 64), dyn, st, a, scale_log2, per);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t st) {
    if (n <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, st, x, n, out);
    return hipGetLastError();
}
