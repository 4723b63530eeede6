// Per-query top-k over the indexer scores: exact radix select on gfx950.
//
// The indexer "selects the top-k most relevant tokens per query" ("IndexCache:
// Accelerating Sparse Attention via Cross-Layer Index Reuse", arXiv abstract);
// the agent skill page (Step 1) shapes the result (batch, seq_len, k).  Rule
// implemented here: the k largest visible scores of a row; among equal scores
// the lower key index wins; the row is written in ascending key order and
// padded with -1 when fewer than k keys are visible.
//
// One workgroup per row.  Scores become order-preserving u32 keys (-0.0 folded
// onto +0.0).  The bits shared by the row's smallest and largest key are
// skipped; the rest are resolved most-significant digit first with 11-bit LDS
// histograms until the k-th key's prefix is exact or its bin is taken whole.
// A final pass walks the row in index order and compacts the selected
// positions with wave ballots and a workgroup prefix sum, so the output is
// sorted for free and ties resolve to the lowest indices.  Rows of up to
// LDS_ROW_CAP keys are staged once in LDS; longer rows are re-read from
// global memory (L2 / MALL) at every pass.
#include "common.h"

using namespace ic;

namespace {

constexpr int HIST_BITS = 11;
constexpr int HIST_BINS = 1 << HIST_BITS;
constexpr int LDS_ROW_CAP = 36864;   // keys staged in LDS (144 KiB)
constexpr int EPT = 8;               // elements per thread per emit segment

template <int NT>
struct TopkShared {
    uint32_t hist[HIST_BINS];
    uint32_t wtot[NT / 64];
    uint32_t wtot2[NT / 64];
    uint32_t kmin, kmax;
    uint32_t found_bin, found_above;
};

// Exclusive prefix sum of x over the workgroup (thread order). Returns it; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wtot, uint32_t* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint32_t v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) wtot[wv] = v;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint32_t t = wtot[i];
        before += (i < wv) ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return before + v - x;
}

template <int NT, bool IN_LDS>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                  int first_len, const int32_t* __restrict__ seq_len, int k,
                                                  int32_t* __restrict__ idx, int max_len) {
    extern __shared__ uint32_t keys_lds[];
    __shared__ TopkShared<NT> sh;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    // visible length, clamped to the staged / allocated row (a bad seq_len cannot overrun)
    const int n = max(1, min(seq_len ? seq_len[row] : first_len + row, max_len));
    int32_t* out = idx + (int64_t)row * k;
    const float* src = scores + (int64_t)row * row_stride;

    if (n <= k) {                                   // every visible key is selected
        for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
        return;
    }

    auto key_at = [&](int i) -> uint32_t {
        if constexpr (IN_LDS) return keys_lds[i];
        else return score_key(src[i]);
    };

    // Stage (or scan) the row: smallest and largest key.
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int i = tid; i < n; i += NT) {
        const uint32_t kk = score_key(src[i]);
        if constexpr (IN_LDS) keys_lds[i] = kk;
        lo = min(lo, kk);
        hi = max(hi, kk);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor(lo, o));
        hi = max(hi, (uint32_t)__shfl_xor(hi, o));
    }
    if (tid == 0) { sh.kmin = 0xFFFFFFFFu; sh.kmax = 0u; }
    __syncthreads();
    if (lane == 0) { atomicMin(&sh.kmin, lo); atomicMax(&sh.kmax, hi); }
    __syncthreads();
    const uint32_t kmin = sh.kmin, kmax = sh.kmax;

    // Radix select state: candidates are keys with (key >> shift) == prefix.
    int shift = (kmin == kmax) ? 0 : 32 - __clz(kmin ^ kmax);
    uint32_t prefix = shift >= 32 ? 0u : (kmax >> shift);
    uint32_t k_rem = (uint32_t)k;                   // still to take among the candidates

    while (shift > 0) {
        const int width = min(HIST_BITS, shift);
        const int sh_lo = shift - width;
        const uint32_t mask = (1u << width) - 1u;
        const int nb = 1 << width;
        for (int b = tid; b < nb; b += NT) sh.hist[b] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint32_t kk = key_at(i);
            const uint32_t hi_bits = shift >= 32 ? 0u : (kk >> shift);
            if (hi_bits == prefix) atomicAdd(&sh.hist[(kk >> sh_lo) & mask], 1u);
        }
        __syncthreads();
        // Find bin b with above(b) < k_rem <= above(b) + hist[b], above = count in higher bins.
        constexpr int BPT = (HIST_BINS + NT - 1) / NT;
        uint32_t local = 0;
        uint32_t hv[BPT];
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = tid * BPT + j;
            hv[j] = b < nb ? sh.hist[b] : 0u;
            local += hv[j];
        }
        // suffix sum over threads: count in bins owned by higher threads
        uint32_t suf = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t y = __shfl_down(suf, o);
            if (lane + o < 64) suf += y;
        }
        if (lane == 0) sh.wtot[wv] = suf;
        __syncthreads();
        uint32_t above = suf - local;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) above += (i > wv) ? sh.wtot[i] : 0u;
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
            const int b = tid * BPT + j;
            if (b < nb && above < k_rem && k_rem <= above + hv[j]) {
                sh.found_bin = (uint32_t)b;
                sh.found_above = above;
            }
            above += hv[j];
        }
        __syncthreads();
        const uint32_t fb = sh.found_bin;
        const uint32_t fa = sh.found_above;
        const uint32_t in_bin = sh.hist[fb];
        prefix = (shift >= 32 ? 0u : (prefix << width)) | fb;
        k_rem -= fa;
        shift = sh_lo;
        __syncthreads();                             // hist / found_* reused next pass
        if (in_bin == k_rem) break;                  // the whole bin is taken: no ties to cut
    }

    // Emit in index order: key prefix above -> selected; equal -> the first k_rem of them.
    uint32_t eq_run = 0, sel_run = 0;
    for (int base = 0; base < n; base += NT * EPT) {
        uint32_t kk[EPT];
        bool gt[EPT], eq[EPT];
        uint32_t eqc = 0;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = base + tid * EPT + j;
            gt[j] = eq[j] = false;
            if (i < n) {
                kk[j] = key_at(i);
                const uint32_t dgt = shift >= 32 ? 0u : (kk[j] >> shift);
                gt[j] = dgt > prefix;
                eq[j] = dgt == prefix;
                eqc += eq[j];
            }
        }
        uint32_t eq_tot;
        uint32_t eq_rank = eq_run + block_excl_scan<NT>(eqc, sh.wtot, &eq_tot);
        bool sel[EPT];
        uint32_t selc = 0;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            sel[j] = gt[j] || (eq[j] && eq_rank < k_rem);
            eq_rank += eq[j];
            selc += sel[j];
        }
        uint32_t sel_tot;
        uint32_t pos = sel_run + block_excl_scan<NT>(selc, sh.wtot2, &sel_tot);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (sel[j] && pos < (uint32_t)k) out[pos++] = base + tid * EPT + j;
        }
        eq_run += eq_tot;
        sel_run += sel_tot;
    }
}

template <int NT, bool IN_LDS>
hipError_t topk_launch(const ic_topk_args& a, hipStream_t st) {
    size_t lds = IN_LDS ? (size_t)a.max_len * 4 : 0;
    static bool attr_set = false;
    if (IN_LDS && !attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<NT, IN_LDS>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           LDS_ROW_CAP * 4);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((topk_kernel<NT, IN_LDS>), dim3(a.rows), dim3(NT), lds, st, a.scores, a.row_stride,
                       a.first_len, a.seq_len, a.k, a.idx, a.max_len);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const ic_topk_args& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    if (a.max_len <= LDS_ROW_CAP) {
        if (a.max_len <= 4096) return topk_launch<256, true>(a, st);
        if (a.max_len <= 16384) return topk_launch<512, true>(a, st);
        return topk_launch<1024, true>(a, st);
    }
    return topk_launch<1024, false>(a, st);
}
