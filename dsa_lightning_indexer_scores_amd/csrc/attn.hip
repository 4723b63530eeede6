// Sparse gather attention over the top-k rows, on gfx950 MFMA.
//
// "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
// (arXiv abstract): with the indexer's top-k, core attention runs over k
// tokens instead of L.  Per query and head,
//     out = sum_s softmax_s(q . K[s] / sqrt(d)) V[s],   s over idx (-1 skipped),
// with one KV head shared by all query heads; a token's row is [K | V].
//
// One wave owns one (query, group of 16 heads[, key split]).
//   prefill: the selected rows go straight from memory into the wave's LDS with
//       global_load_lds_dwordx4 (64 lanes x 16 bytes: four 256-byte K or V halves
//       per instruction, fully coalesced), with no VGPR round trip and no LDS write
//       instructions; the idx row reaches LDS the same way.  Few registers and
//       18 KB of LDS per wave (one K and one V stage of 32 half rows, two idx
//       chunks) give eight waves per CU, and the CU's LDS holds the bytes in flight;
//   split-K decode, latency-bound with one or two steps per wave, gathers K
//       straight into fragments and stages only V;
//   S^T (32 keys x 16 heads) = K Q^T;
//   online softmax in fp32 (exp2 domain) on S^T, whose lane layout (head =
//       lane % 16) is also the layout of O^T below, so the running max and
//       rescale never leave the lane.  The reference max moves only when a
//       step's max passes it by more than 2^8, so most steps skip the O rescale;
//   O^T (d x 16 heads) += V^T P^T : V read back transposed with
//       ds_read_b64_tr_b16; P^T is the S^T accumulator packed to bf16 (its
//       k order matches the transposed read, so no shuffle is needed);
//   l += ones^T P^T, one more MFMA, so the denominator sums the same bf16 P
//       as the numerator and costs no VALU.
// Steps past a query's last real idx entry are not run; a query whose idx row has
// no valid entry at all gets a zero output vector.
// Decode splits a query's rows over several waves (split-K): the 4 waves of a
// workgroup merge their partial (max, sum, O) in LDS, and a small kernel merges
// the workgroups' partials in split order, so results are deterministic.  (A
// fused last-workgroup merge needs device-scope ordering, which on this part
// costs L2 write-back / invalidation or serialised coherent loads: slower.)
#include "common.h"

using namespace ic;

namespace {

constexpr int ATT_NW = 4;
constexpr int KT = 32;                  // selected rows per step
// Prefill: four waves (queries) per workgroup with one K and one V stage each (18 KB of
// LDS per wave, eight waves per CU).  Measured on a 32K layer: a second V stage (six waves
// per CU) and two- or eight-wave workgroups were all slower.
constexpr int DMA_NW = 4;
// The running max of a head is moved (and O, l rescaled) only when a step's max
// exceeds it by more than this many powers of two, so most steps skip the rescale;
// the probabilities stay <= 2^RESCALE_LOG2, far inside fp32 and bf16 range.  Any
// reference value gives the same softmax once O is divided by l.
constexpr float RESCALE_LOG2 = 8.f;

template <int D>
struct AttGeom {                        // split-K decode
    static constexpr int NDC = D / 32;  // K=32 chunks of the QK^T contraction
    static constexpr int NDT = D / 16;  // 16-wide d tiles of the output
    static constexpr int RB = 4 * D;    // bytes per KV row: K[d] then V[d], bf16
    static constexpr int STR = 2 * D + 16;            // LDS bytes per V row (padded)
    static constexpr int VPPR = D * 2 / 16;           // 16-byte pieces per V row
    static constexpr int VPL = KT * VPPR / 64;        // V pieces per lane
};

__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Split-K decode: wave (query, head group, split) runs its slice of the idx row and the
// workgroup's four splits merge into one partial.
template <int D>
__global__ __launch_bounds__(ATT_NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    float* __restrict__ part, int64_t kv_seq_stride, int Lk, int nq, int q_per_seq,
    int H, int k, int nsplit, float scale_log2) {
    using G = AttGeom<D>;
    static_assert(ATT_NW * 16 * D * 4 + ATT_NW * 16 * 8 <= ATT_NW * KT * G::STR,
                  "the LDS merge reuses the row tiles");
    __shared__ __attribute__((aligned(16))) uint8_t vlds_all[ATT_NW][KT * G::STR];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps addressing scalar
    const int n = lane & 15, g = lane >> 4;
    const int HG = (H + 15) / 16;
    const int64_t item = (int64_t)blockIdx.x * ATT_NW + wv;
    const int sp = (int)(item % nsplit);
    const int hg = (int)((item / nsplit) % HG);
    const int64_t qi = item / ((int64_t)nsplit * HG);
    if (qi >= nq) return;
    uint8_t* vlds = vlds_all[wv];

    const int seq = (int)(qi / q_per_seq);
    const uint16_t* kvs = kv + (int64_t)seq * kv_seq_stride;
    // byte view of this sequence's rows, addressed with 32-bit offsets (a sequence's
    // KV rows span < 4 GiB), so loads use a scalar base plus one VGPR offset
    const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kvs);
    const int32_t* irow = idx + qi * k;
    const int head = 16 * hg + n;

    // Q^T fragments (B operand): lane (n, g) holds head n, d = 32*dc + 8g .. +7.
    i32x4 qf[G::NDC];
#pragma unroll
    for (int dc = 0; dc < G::NDC; ++dc) {
        i32x4 v = {0, 0, 0, 0};
        if (head < H) v = *reinterpret_cast<const i32x4*>(q + (qi * H + head) * D + 32 * dc + 8 * g);
        qf[dc] = v;
    }

    // This split's slice of the idx row, in steps of KT.
    const int per = ((k + nsplit - 1) / nsplit + KT - 1) / KT * KT;
    const int j_begin = sp * per;
    const int j_end = min(k, j_begin + per);
    // A step's idx entries, raw: they are first used at that step's issue.  Loads
    // complete in order, so each step's entries are fetched before the row loads of the
    // step issued just ahead of it; its issue then never waits for those rows.
    auto load_idx = [&](int j0) -> int {
        const int jl = j0 + (lane & 31);
        const int v = irow[min(jl, j_end - 1)];           // unconditional load: no branch around it
        return (jl < j_end && lane < 32) ? v : -1;
    };
    int idxA = load_idx(j_begin), idxB = load_idx(j_begin + KT);   // in flight with the scan below
    // Only the steps up to the last entry that names a row are run (an idx row padded
    // with -1 because fewer than k keys are visible costs only its real steps).
    int j_last = -1;
    for (int jb = j_begin; jb < j_end; jb += 64 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {                    // unconditional (clamped) loads: one wait for all eight
            const int j = jb + 64 * u + lane;
            v[u] = irow[min(j, j_end - 1)];
            v[u] = j < j_end ? v[u] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if ((uint32_t)v[u] < (uint32_t)Lk) j_last = max(j_last, jb + 64 * u + lane);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) j_last = max(j_last, __shfl_xor(j_last, sh));
    const int nsteps = __builtin_amdgcn_readfirstlane(j_last < 0 ? 0 : (j_last - j_begin) / KT + 1);
    // Ends with a wait for every load so far: the step loop below starts from a clean count.
    __builtin_amdgcn_s_waitcnt(0);

    f32x4 o[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Reference max of the head (log2 units).  Finite from the start, so a step whose
    // entries are all -1 gives exp2(-inf) = 0 rather than exp2(-inf + inf).
    float m_run = -1e30f;
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};                   // softmax denominator (every slot)
    const i32x4 ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};   // bf16 1.0 pairs

    // One step of KT selected rows.  Loads of step t+1 are issued before step t is
    // computed (two register sets, A and B, both possibly in flight), and the idx
    // entries of a step are fetched two steps ahead.  Every step issues its loads and is computed (entries
    // of -1 read a real row and are masked), so no branch separates a load from its
    // use and the compiler's in-order load counting stays exact.
    struct Tile {
        i32x4 kf[2][G::NDC];                                 // K fragments, keys 16*kt + m
        i32x4 vst[G::VPL];                                   // V rows, staged for LDS
        uint32_t valid;                                      // bit e: entry e of the step is a row
    };
    auto issue = [&](Tile& T, int raw_idx) {
        // Nothing of an issue may be scheduled into the previous compute: its first use of
        // raw_idx waits for every load before it, including the tile that compute overlaps.
        __builtin_amdgcn_sched_barrier(0);
        const bool ok = (uint32_t)raw_idx < (uint32_t)Lk;   // -1 or past the KV rows: no row
        T.valid = (uint32_t)__ballot(ok);
        const int safe_idx = ok ? raw_idx : 0;               // a real row, masked later
#pragma unroll
        for (int i = 0; i < G::VPL; ++i) {                   // V piece c -> row c / VPPR, byte (c % VPPR) * 16
            const int c = lane + 64 * i;
            const int r = __shfl(safe_idx, c / G::VPPR);
            const uint32_t off = (uint32_t)r * G::RB + 2 * D + (c % G::VPPR) * 16;
            T.vst[i] = *reinterpret_cast<const i32x4*>(kvb + off);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {                     // lane (m, g): key 16*kt + m, d = 32*dc + 8g
            const int r = __shfl(safe_idx, 16 * kt + n);
            const uint32_t off = (uint32_t)r * G::RB + 16 * g;
#pragma unroll
            for (int dc = 0; dc < G::NDC; ++dc)
                T.kf[kt][dc] = *reinterpret_cast<const i32x4*>(kvb + off + 64 * dc);
        }
    };
    auto compute = [&](const Tile& T) {
        const uint32_t valid = T.valid;
#pragma unroll
        for (int i = 0; i < G::VPL; ++i) {
            const int c = lane + 64 * i;
            *reinterpret_cast<i32x4*>(vlds + (c / G::VPPR) * G::STR + (c % G::VPPR) * 16) = T.vst[i];
        }
        // S^T = K Q^T: lane (n, g) gets head n, keys 16*kt + 4g + e.  K fragment: key 16*kt + n,
        // d = 32*dc + 8g .. +7.
        f32x4 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < G::NDC; ++dc) acc = mfma_bf16_k32(T.kf[kt][dc], qf[dc], acc);
            s[kt] = acc;
        }
        float x[8];                                          // raw scores; -inf for -1 entries
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * kt + e] = s[kt][e];
        if (valid != 0xFFFFFFFFu) {                          // wave-uniform: only ragged steps mask
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!((valid >> (16 * kt + 4 * g + e)) & 1u)) x[4 * kt + e] = -INFINITY;
        }
        float tmax = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmax_nan(tmax, x[e]);
        tmax = max_xor32(max_xor16(tmax)) * scale_log2;      // finite: the step has a row
        if (__ballot(tmax > m_run + RESCALE_LOG2)) {         // some head's max grew a lot (always at the first step)
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < G::NDT; ++dt) o[dt] *= alpha;
            lsum *= alpha;
            m_run = m_new;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], scale_log2, -m_run));
        // P^T fragment: slots 0..3 = keys 4g+e, slots 4..7 = keys 16+4g+e.
        i32x4 pf;
        pf[0] = (int)pack_bf16x2(x[0], x[1]);
        pf[1] = (int)pack_bf16x2(x[2], x[3]);
        pf[2] = (int)pack_bf16x2(x[4], x[5]);
        pf[3] = (int)pack_bf16x2(x[6], x[7]);

        // O^T += V^T P^T.  Transposed LDS reads: within each 16-lane row g, lane src
        // points at V[4g + src/4 (+16)][16dt + 4*(src%4)], and receives V[keys][d = 16dt + src].
        const int src = n;
        lds_wave_sync();
        const uint8_t* vr0 = vlds + (4 * g + (src >> 2)) * G::STR + (4 * (src & 3)) * 2;
        const uint8_t* vr1 = vr0 + 16 * G::STR;
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt) {
            const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr0 + 32 * dt));
            const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr1 + 32 * dt));
            const u32x2 w0 = __builtin_bit_cast(u32x2, a0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, a1);
            const i32x4 vf = {(int)w0[0], (int)w0[1], (int)w1[0], (int)w1[1]};
            o[dt] = mfma_bf16_k32(vf, pf, o[dt]);
        }
        // l += sum over the step's keys of P (as rounded to bf16, like the numerator):
        // every d row of ones^T P^T is that sum, so each lane gets its head's l.
        lsum = mfma_bf16_k32(ones, pf, lsum);
        lds_wave_sync();
    };

    Tile TA, TB;
    if (nsteps > 0) {
        issue(TA, idxA);
        int t = 0;
        for (; t + 2 < nsteps; t += 2) {                     // both issues unconditional
            idxA = load_idx(j_begin + (t + 2) * KT);
            issue(TB, idxB);                                 // TA's rows may still be in flight
            compute(TA);
            idxB = load_idx(j_begin + (t + 3) * KT);
            issue(TA, idxA);                                 // TB's rows may still be in flight
            compute(TB);
        }
        if (t + 1 < nsteps) {                                // last two steps
            issue(TB, idxB);
            compute(TA);
            compute(TB);
        } else {                                             // last step
            compute(TA);
        }
    }

    const float l_run = lsum[0];
    if (l_run == 0.f) m_run = -INFINITY;                 // no selected row: an empty partial
    {
        // Split-K: the workgroup's 4 waves hold 4 consecutive splits of one (query, head
        // group).  Merge them through LDS (the V tiles are no longer needed) and write
        // one partial: unnormalised O^T [16 heads][D] and (max, sum) per head.
        float* mo = reinterpret_cast<float*>(vlds_all[0]);   // [4 waves][16 heads][D]
        float* ml = mo + ATT_NW * 16 * D;                     // [4 waves][16 heads][2]
        __syncthreads();                                      // every wave is done with its V tile
        float4* dst = reinterpret_cast<float4*>(mo + (wv * 16 + n) * D + 4 * g);
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt) dst[4 * dt] = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
        if (g == 0) {
            ml[(wv * 16 + n) * 2] = m_run;
            ml[(wv * 16 + n) * 2 + 1] = l_run;
        }
        __syncthreads();
        float* po = part + (item / ATT_NW) * (16 * D + 32);   // ((qi*HG + hg)*nsplit/4 + sp/4)
        for (int e = threadIdx.x; e < 16 * D; e += ATT_NW * 64) {
            const int hn = e / D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < ATT_NW; ++w) M = fmaxf(M, ml[(w * 16 + hn) * 2]);
            float num = 0.f, den = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < ATT_NW; ++w) {
                    const float c = exp2f(ml[(w * 16 + hn) * 2] - M);   // 0 for an empty split
                    num += c * mo[(w * 16) * D + e];
                    den += c * ml[(w * 16 + hn) * 2 + 1];
                }
            }
            po[e] = num;
            if (e % D == 0) {
                po[16 * D + 2 * hn] = M;
                po[16 * D + 2 * hn + 1] = den;
            }
        }
    }
}

// Prefill with the gather going straight into LDS (global_load_lds_dwordx4): a wave's
// selected rows travel memory -> LDS with no VGPR round trip and no LDS write
// instructions, so the wave needs few registers and the CU's LDS holds the bytes in
// flight.  Per wave: one K stage and one V stage of 32 half rows each, and a ring of two
// 256-entry chunks of its idx row, all filled by DMA.  Step s (32 keys):
//   wait K(s); S^T = K Q^T; issue K(s+1); online softmax;
//   wait V(s); O^T += V^T P^T, l += ones^T P^T; issue V(s+1)
// so each half has about half a step of compute to land in, and eight waves per CU
// overlap one another's waits.  The waits are explicit vmcnt counts: the compiler does
// not see these loads.
//
// Half-row layout in LDS: 16-byte slot j of staged row r holds the half's chunk
// j ^ swz(r), so that the K-fragment reads (16 rows, one chunk each) and the transposed
// V reads (8 rows, two adjacent chunks each) fall on distinct banks.
template <int D>
struct DmaGeom {
    static constexpr int NDC = D / 32;       // K=32 chunks of the QK^T contraction
    static constexpr int NDT = D / 16;       // 16-wide d tiles of the output
    static constexpr int RB = 4 * D;         // bytes per KV row: K[d] then V[d], bf16
    static constexpr int HB = 2 * D;         // bytes per half row
    static constexpr int NCH = HB / 16;      // 16-byte chunks per half row
    static constexpr int RPI = 1024 / HB;    // half rows per DMA instruction (64 lanes x 16 bytes)
    static constexpr int NI = KT / RPI;      // DMA instructions per half step
    static constexpr int SB = KT * HB;       // bytes per stage
    static constexpr int ICH = 256;          // idx entries per ring chunk
    static constexpr int SPC = ICH / KT;     // steps per chunk
    static_assert((NCH == 16 || NCH == 8) && KT % RPI == 0, "half row must be 256 or 128 bytes");
    __device__ static uint32_t swz(int r) { return dma_swz<NCH>(r); }
};

template <int D>
__global__ __launch_bounds__(DMA_NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, int64_t kv_seq_stride, int Lk, int nq, int q_per_seq, int H, int k,
    float scale_log2, const ic_seq_group grp) {
    using G = DmaGeom<D>;
    constexpr int CI = G::ICH / 64;                      // DMA instructions per idx chunk
    // the in-flight counts waited for below (NI, CI and their sum) must be exact vmcnt values
    static_assert(G::NI % 4 == 0 && CI % 4 == 0 && G::NI + CI <= 28, "wait_vm_n takes multiples of 4 below 32");
    __shared__ __attribute__((aligned(1024))) uint8_t stage_all[DMA_NW][2][G::SB];   // K, V
    __shared__ __attribute__((aligned(16))) int32_t ring_all[DMA_NW][2 * G::ICH];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int HG = (H + 15) / 16;
    const int64_t item = (int64_t)blockIdx.x * DMA_NW + wv;
    const int hg = (int)(item % HG);
    const int64_t qi = item / HG;
    if (qi >= nq) return;
    const uint8_t* kst = stage_all[wv][0];
    const uint8_t* vst = stage_all[wv][1];
    const int32_t* ring = ring_all[wv];
    const uint32_t k_lds = lds_addr(kst), v_lds = lds_addr(vst), ring_lds = lds_addr(ring);
    // the query's sequence: a group entry's cache slot in a grouped launch, else qi / q_per_seq
    const int seq = grp.n > 0 ? grp.seq[group_find(grp.row0, grp.n, (int)qi)] : (int)(qi / q_per_seq);
    const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv + (int64_t)seq * kv_seq_stride);
    const int32_t* irow = idx + qi * k;
    const int head = 16 * hg + n;

    i32x4 qf[G::NDC];                                    // Q^T fragments: head n, d = 32*dc + 8g .. +7
#pragma unroll
    for (int dc = 0; dc < G::NDC; ++dc) {
        i32x4 v = {0, 0, 0, 0};
        if (head < H) v = *reinterpret_cast<const i32x4*>(q + (qi * H + head) * D + 32 * dc + 8 * g);
        qf[dc] = v;
    }
    int j_last = -1;                                      // steps after the last real entry are not run
    for (int jb = 0; jb < k; jb += 64 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {                    // unconditional (clamped) loads: one wait for all eight
            const int j = jb + 64 * u + lane;
            v[u] = irow[min(j, k - 1)];
            v[u] = j < k ? v[u] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if ((uint32_t)v[u] < (uint32_t)Lk) j_last = max(j_last, jb + 64 * u + lane);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) j_last = max(j_last, __shfl_xor(j_last, sh));
    const int nsteps = __builtin_amdgcn_readfirstlane(j_last < 0 ? 0 : j_last / KT + 1);
    __builtin_amdgcn_s_waitcnt(0);

    // chunk c of the idx row -> ring slot c % 2 (entries past the row repeat its last entry;
    // the valid mask drops them by position)
    auto issue_chunk = [&](int c) {
        const uint32_t dst = ring_lds + (uint32_t)(c & 1) * (G::ICH * 4);
#pragma unroll
        for (int w = 0; w < CI; ++w)
            dma_b32(irow, (uint32_t)min(c * G::ICH + 64 * w + lane, k - 1) * 4u, dst + 256u * w);
    };
    // Lane l of instruction i fetches chunk (l % NCH) ^ swz(r) of half row r = RPI*i + l / NCH.
    uint32_t cof[G::NI];
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
        cof[i] = ((uint32_t)(lane % G::NCH) ^ G::swz(G::RPI * i + lane / G::NCH)) * 16u;
    uint32_t roff[G::NI];                                // row offsets of the step being fetched
    // Row offsets of step s from the ring and its valid keys as a wave-uniform 32-bit mask
    // (entry in [0, Lk) and inside the idx row).  Entries outside [0, Lk) fetch row 0, a key
    // every query sees: a masked entry's probability is 0, and 0 times its V row must stay
    // 0, which rows past the context (capacity that may hold anything) would not guarantee.
    auto offsets = [&](int s) -> uint32_t {
        const int32_t* ir = ring + ((s / G::SPC) & 1) * G::ICH + (s % G::SPC) * KT;
        const int ev = ir[lane & 31];
        const uint32_t vm = (uint32_t)__ballot((uint32_t)ev < (uint32_t)Lk && s * KT + (lane & 31) < k);
#pragma unroll
        for (int i = 0; i < G::NI; ++i) {
            const uint32_t v = (uint32_t)ir[G::RPI * i + lane / G::NCH];
            roff[i] = (v < (uint32_t)Lk ? v : 0u) * (uint32_t)G::RB + cof[i];
        }
        return __builtin_amdgcn_readfirstlane(vm);
    };
    auto issue_half = [&](uint32_t dst, uint32_t half_off) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of the stage being refilled are done
#pragma unroll
        for (int i = 0; i < G::NI; ++i) dma_b128(kvb, roff[i] + half_off, dst + 1024u * i);
    };

    f32x4 o[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -1e30f;                                // reference max of the head (log2 units)
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
    const i32x4 ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
    const uint32_t swz_k = G::swz(n);
    const int vrow = 4 * g + (n >> 2);                    // transposed V reads: rows vrow and vrow + 16
    const uint32_t swz_v = G::swz(vrow);

    uint32_t vmask = 0;
    if (nsteps > 0) {
        issue_chunk(0);
        issue_chunk(1);
        wait_vm<CI>();                                   // chunk 0 landed
        vmask = offsets(0);
        issue_half(k_lds, 0);
        issue_half(v_lds, G::HB);
    }
    // DMA instructions issued after V(s) that may still be in flight when K(s) or V(s) is
    // waited for.  chunk(s): an idx chunk went out right after V(s).
    auto chunk_after = [&](int t) -> bool { return t > 0 && t % G::SPC == 0; };
    for (int s = 0; s < nsteps; ++s) {
        const bool more = s + 1 < nsteps;
        const int cs = chunk_after(s) ? CI : 0;
        wait_vm_n(G::NI + cs);                           // K(s) landed (V(s) and its chunk may fly)
        // S^T = K Q^T: lane (n, g) gets head n, keys 16*kt + 4g + e
        f32x4 sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < G::NDC; ++dc) {
                const i32x4 kf = *reinterpret_cast<const i32x4*>(kst + (16 * kt + n) * G::HB +
                                                                 (((uint32_t)(4 * dc + g) ^ swz_k) * 16u));
                acc = mfma_bf16_k32(kf, qf[dc], acc);
            }
            sc[kt] = acc;
        }
        uint32_t vmask_next = 0;
        if (more) {
            vmask_next = offsets(s + 1);
            issue_half(k_lds, 0);                        // K(s+1)
        }
        float x[8];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * kt + e] = sc[kt][e];
        if (vmask != 0xFFFFFFFFu) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!((vmask >> (16 * kt + 4 * g + e)) & 1u)) x[4 * kt + e] = -INFINITY;
        }
        float tmax = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmax_nan(tmax, x[e]);
        tmax = max_xor32(max_xor16(tmax)) * scale_log2;
        if (__ballot(tmax > m_run + RESCALE_LOG2)) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < G::NDT; ++dt) o[dt] *= alpha;
            lsum *= alpha;
            m_run = m_new;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], scale_log2, -m_run));
        i32x4 pf;
        pf[0] = (int)pack_bf16x2(x[0], x[1]);
        pf[1] = (int)pack_bf16x2(x[2], x[3]);
        pf[2] = (int)pack_bf16x2(x[4], x[5]);
        pf[3] = (int)pack_bf16x2(x[6], x[7]);
        // V(s) landed: still in flight may be the chunk issued after it and K(s+1)
        wait_vm_n(cs + (more ? G::NI : 0));
        // O^T += V^T P^T: lane (n, g) reads 8 bytes of rows vrow and vrow + 16, d = 16*dt + 4*(n%4) .. +3
        const uint8_t* vr0 = vst + vrow * G::HB + 8 * (n & 1);
        const uint8_t* vr1 = vr0 + 16 * G::HB;
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt) {
            const uint32_t c = ((uint32_t)(2 * dt + ((n >> 1) & 1)) ^ swz_v) * 16u;
            const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr0 + c));
            const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vr1 + c));
            const u32x2 w0 = __builtin_bit_cast(u32x2, a0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, a1);
            const i32x4 vf = {(int)w0[0], (int)w0[1], (int)w1[0], (int)w1[1]};
            o[dt] = mfma_bf16_k32(vf, pf, o[dt]);
        }
        lsum = mfma_bf16_k32(ones, pf, lsum);
        if (more) {
            issue_half(v_lds, G::HB);                    // V(s+1)
            if (chunk_after(s + 1)) issue_chunk((s + 1) / G::SPC + 1);
        }
        vmask = vmask_next;
    }
    __builtin_amdgcn_s_waitcnt(0);                       // an idx chunk may still be in flight
    if (head < H) {
        // a row without a single valid entry has nothing to attend to: its output is zero
        const float inv = lsum[0] > 0.f ? 1.f / lsum[0] : 0.f;
        uint16_t* op = out + (qi * H + head) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt) {
            uint2 v;
            v.x = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
            v.y = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
            *reinterpret_cast<uint2*>(op + 16 * dt) = v;
        }
    }
}

// Merge the workgroups' partials of each (query, head) in split order: one
// workgroup per (query, head), one thread per channel.
constexpr int COMBINE_FAST = 16;        // partials merged from registers after one round of loads
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                        int H, int nparts) {
    const int HG = (H + 15) / 16;
    const int64_t qi = blockIdx.x / H;
    const int head = blockIdx.x % H;
    const int hg = head / 16, hn = head % 16;
    const float* base = part + (qi * HG + hg) * nparts * (16 * D + 32);
    const int dd = threadIdx.x;
    float M = -INFINITY, num = 0.f, den = 0.f;
    if (nparts <= COMBINE_FAST) {
        // Every load issued before any use: one memory round trip for the whole merge.
        float mm[COMBINE_FAST], ll[COMBINE_FAST], oo[COMBINE_FAST];
#pragma unroll
        for (int p = 0; p < COMBINE_FAST; ++p) {
            mm[p] = -INFINITY;
            ll[p] = 0.f;
            oo[p] = 0.f;
            if (p < nparts) {
                const float* ps = base + p * (16 * D + 32);
                mm[p] = ps[16 * D + 2 * hn];
                ll[p] = ps[16 * D + 2 * hn + 1];
                oo[p] = ps[hn * D + dd];
            }
        }
#pragma unroll
        for (int p = 0; p < COMBINE_FAST; ++p) M = fmaxf(M, mm[p]);
#pragma unroll
        for (int p = 0; p < COMBINE_FAST; ++p) {
            const float c = (mm[p] == -INFINITY) ? 0.f : exp2f(mm[p] - M);   // empty split adds nothing
            num += c * oo[p];
            den += c * ll[p];
        }
    } else {
        for (int p = 0; p < nparts; ++p) M = fmaxf(M, base[p * (16 * D + 32) + 16 * D + 2 * hn]);
        for (int p = 0; p < nparts; ++p) {
            const float* ps = base + p * (16 * D + 32);
            const float m = ps[16 * D + 2 * hn];
            const float c = (m == -INFINITY) ? 0.f : exp2f(m - M);   // a split with no selected rows adds nothing
            num += c * ps[hn * D + dd];
            den += c * ps[16 * D + 2 * hn + 1];
        }
    }
    const float v = den > 0.f ? num / den : 0.f;             // no valid entry in any split: zero
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[(qi * H + head) * D + dd] = (uint16_t)(u >> 16);
}

template <int D>
hipError_t attn_launch(const ic_attn_args& a, hipStream_t st) {
    const int HG = (a.H + 15) / 16;
    const int64_t items = (int64_t)a.nq * HG * a.nsplit;
    const int64_t blocks = (items + ATT_NW - 1) / ATT_NW;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (a.nsplit == 1) {                                // prefill: one wave per (query, head group)
        if ((int64_t)a.Lk * DmaGeom<D>::RB > (int64_t)UINT32_MAX) return hipErrorInvalidValue;   // 32-bit row offsets
        const int64_t dblocks = (items + DMA_NW - 1) / DMA_NW;
        ic_seq_group grp{};
        if (a.grp) grp = *a.grp;
        hipLaunchKernelGGL((sparse_attn_dma_kernel<D>), dim3((unsigned)dblocks), dim3(DMA_NW * 64), 0, st,
                           (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (uint16_t*)a.out,
                           a.kv_seq_stride, a.Lk, a.nq, a.q_per_seq, a.H, a.k, scale_log2, grp);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((sparse_attn_split_kernel<D>), dim3((unsigned)blocks), dim3(ATT_NW * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, a.ws,
                       a.kv_seq_stride, a.Lk, a.nq, a.q_per_seq, a.H, a.k, a.nsplit, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((int64_t)a.nq * a.H)), dim3(D), 0, st,
                       a.ws, (uint16_t*)a.out, a.H, a.nsplit / ATT_NW);
    return hipGetLastError();
}

}  // namespace

size_t sparse_attn_ws_bytes(int32_t nq, int32_t H, int32_t d, int32_t nsplit) {
    if (nsplit <= 1) return 0;
    const int64_t HG = (H + 15) / 16;
    return (size_t)nq * HG * (nsplit / ATT_NW) * (16 * d + 32) * sizeof(float);
}

hipError_t launch_sparse_attn(const ic_attn_args& a, hipStream_t st) {
    if (a.nq <= 0) return hipSuccess;
    if (a.nsplit > 1 && (a.nsplit % ATT_NW != 0 || a.ws == nullptr))
        return hipErrorInvalidValue;                        // splits merge 4 per workgroup, then in a combine kernel
    if (a.d == 128) return attn_launch<128>(a, st);
    if (a.d == 64) return attn_launch<64>(a, st);
    return hipErrorInvalidValue;
}
