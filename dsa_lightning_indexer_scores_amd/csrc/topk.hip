// Per-query top-k over the indexer scores: exact radix select on gfx950.
//
// In DSA the lightning indexer keeps, for every query, the k keys with the
// highest scores ("IndexCache: Accelerating Sparse Attention via Cross-Layer
// Index Reuse", arXiv abstract); the agent skill page (Step 1) gives the
// result the shape (batch, seq_len, k).  Rule implemented here: the k largest
// visible scores of a row; among equal scores the lower key index wins; the
// row is written in ascending key order and padded with -1 when fewer than k
// keys are visible.
//
// One workgroup per row.  Scores become order-preserving u32 keys (-0.0 folded
// onto +0.0).  The bits shared by the row's smallest and largest key are
// skipped; the rest are resolved most-significant digit first with 11-bit LDS
// histograms (for long rows one copy per wave, summed at the scan) until the
// k-th key's prefix is exact or its bin is taken whole.
// Once the bin holding the k-th key has at most CAND_CAP keys (after the first
// pass, for smooth score distributions), one pass gathers that bin's keys and
// positions into LDS and ranks them exactly, giving the threshold pair (key,
// position); when no other key shares the threshold value a plain key test
// selects.  A final pass walks the row in index order and ranks the selected
// positions with wave ballots (mbcnt prefix counts) and a prefix sum over the
// waves, so the output is sorted for free and ties resolve to the lowest
// indices; the ranked positions are staged in LDS (the histograms' space) and
// written out with coalesced stores.  Rounds of a wave that lie past the row's
// end are skipped in every pass.
//
// Few long rows (decode: one row per sequence) would leave most CUs idle, so
// they run in two launches.  First every (row, segment of SEG keys) takes its
// own top-k with the register-resident select, writing each pick's global
// position and key; the row's top-k lies inside the union of those.  Then one
// workgroup per row selects from that candidate list (coalesced key loads, no
// score gather).  Candidates are in ascending position order, so the
// index-order compaction still gives ascending output and ties still go to the
// lower position.
//
// The row is cut into blocks of NT*EPT keys.  In a block, wave w owns the
// contiguous span [w*64*EPT, (w+1)*64*EPT) and lane l holds its keys
// 256*j + 4*l + e (j < EPT/4, e < 4): loads are coalesced 16-byte vectors and
// every pass works out of VGPRs.  Rows of one block (<= 32768 keys with 1024
// threads) are read from HBM exactly once; longer rows stream their blocks
// again at every pass (re-reads hit L2 / MALL).
#include "common.h"

using namespace ic;

namespace {

constexpr int HIST_BITS = 11;
constexpr int HIST_BINS = 1 << HIST_BITS;
constexpr int CAND_CAP = 256;       // threshold-bin keys resolved by exact ranking in LDS

// acc + the number of lanes below this one whose bit is set in m (mbcnt adds its accumulator
// operand for free, so running prefixes chain through it)
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t acc = 0u) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, acc));
}

// Wave-wide sum / min / max, result in every lane: DPP pairs inside each 16-lane row
// (quad swaps, half-row and row mirrors), then the two lane-row swaps.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
    const u32x2 a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(a[0], a[1]);
    const u32x2 b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return op(b[0], b[1]);
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) { return wave_reduce(x, OpAdd()); }

// Inclusive prefix sum over the 64 lanes in lane order: shifts within each 16-lane row,
// then the row broadcasts of lane 15 (into rows 1, 3) and lane 31 (into rows 2, 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix over waves of a wave-uniform value; *total gets the sum over all waves.
// Ends with a barrier, so `wtot` may be reused right after.
template <int NT>
__device__ __forceinline__ uint32_t waves_scan(uint32_t wave_total, uint32_t* wtot, uint32_t* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) wtot[wv] = wave_total;
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
    return before;
}

// Row sources: a score row; a segment of one (TOPK_SEGS: launch row = row * nseg +
// segment; also writes the picks' keys to ckeys); or a row's candidates (TOPK_GATHER:
// keys from ckeys, positions from cand).
enum { TOPK_ROWS = 0, TOPK_SEGS = 1, TOPK_GATHER = 2 };
constexpr int TOPK_MANY_ROWS = 1024;     // launches of this many rows use the several-rows-per-CU shapes

// A workgroup ranks one row through a chain of short phases separated by barriers, so a
// CU is kept busy by several rows at once: one row's barriers and waits hide behind the
// others' work.  Many-row launches therefore use shapes held to 64 VGPRs (two 1024-thread
// or four 512-thread workgroups per CU) or 512 x 64 at 128 (two per CU).  Measured on the
// stack's eight 4096-row launches over a 32K layer (ms per launch, largest rows last):
// 1024 x 24 and 1024 x 32 at one row per CU 0.19-0.26; 512 x 32 / 1024 x 24 (capped) /
// 512 x 64 at two to four rows per CU 0.083-0.19, 0.92 ms in all against 1.19.  (At the
// cap 1024 x 24 spills five registers and still beats 768 x 32 and 512 x 48; 1024 x 32
// capped spills more and loses to 512 x 64.)  The few-row shapes (decode) keep their
// registers: with one row per CU, a row's latency is what counts.  Streamed 512 x 32 rows
// read with scalar (unaligned) loads need more than 64 VGPRs and run two per CU instead.
constexpr int topk_waves_per_eu(int NT, int EPT, bool VEC, bool STREAM, int MODE) {
    return MODE != TOPK_ROWS ? 1
         : (NT == 512 && EPT == 32 && STREAM && !VEC) ? 4
         : ((NT == 1024 && EPT <= 16) || (NT == 512 && EPT <= 32) || (NT == 1024 && EPT == 24)) ? 8
         : (NT == 512 && EPT == 64) ? 4 : 1;
}

template <int NT, int EPT, bool VEC, bool STREAM, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(topk_waves_per_eu(NT, EPT, VEC, STREAM, MODE)))) void topk_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                  int first_len, const int32_t* __restrict__ seq_len, int k,
                                                  int32_t* __restrict__ idx, int max_len, int seg, int nseg,
                                                  const int32_t* __restrict__ cand, int cand_len,
                                                  uint32_t* __restrict__ ckeys, int len_step,
                                                  const int32_t* __restrict__ run_if, const ic_seq_group grp) {
    if (run_if != nullptr && *run_if == 0) return;            // a refresh that was not needed
    constexpr int NR = EPT / 4;                      // rounds of 4 consecutive keys per lane
    constexpr int BLOCK = NT * EPT;                  // keys per block
    // Long rows keep one histogram per wave: a concentrated score distribution puts
    // most keys in a few bins, and per-wave copies keep the LDS atomics of different
    // waves apart.  Short rows share one copy (a cheaper scan wins there).
    constexpr int NH = (NT * EPT > 32768) ? NT / 64 : 1;
    // One-copy histograms alternate between two buffers: a pass zeroes the next pass's
    // buffer while scanning its own, so zeroing costs no barrier.
    constexpr int NHB = NH == 1 ? 2 : 1;
    static_assert(NHB * NH * HIST_BINS >= 4096, "the output staging reuses the histograms (k <= 4096)");
    __shared__ uint32_t hist[NHB * NH][HIST_BINS];
    __shared__ uint32_t wtot[NT / 64];
    __shared__ uint32_t kminmax[2], found[3];
    __shared__ __attribute__((aligned(16))) uint32_t cand_key[CAND_CAP];
    __shared__ __attribute__((aligned(16))) int32_t cand_idx[CAND_CAP];
    __shared__ uint32_t ncand, thr_key, thr_ties;
    __shared__ int32_t thr_idx;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    int32_t* out = idx + (int64_t)row * k;
    const int srow = MODE == TOPK_SEGS ? row / nseg : row;   // score row
    // visible length of the score row, clamped to the allocated row (a bad seq_len cannot overrun)
    int vis;
    if (grp.n > 0) {                                 // grouped rows: the row's own sequence and position
        const int i = group_find(grp.row0, grp.n, srow);
        vis = grp.pos0[i] + srow - grp.row0[i] + 1;
    } else {
        vis = seq_len ? seq_len[srow] : first_len + srow * len_step;
    }
    const int len = max(1, min(vis, (STREAM || MODE != TOPK_ROWS) ? max_len : min(max_len, BLOCK)));
    int n = len, off = 0;                            // keys this workgroup ranks; position offset
    uint32_t* okey = ckeys + (int64_t)row * k;       // TOPK_SEGS: keys of the picks
    if constexpr (MODE == TOPK_SEGS) {
        off = (row % nseg) * seg;
        n = min(seg, len - off);
        if (n <= 0) {                                // segment past the row's end
            for (int i = tid; i < k; i += NT) { out[i] = -1; okey[i] = 0u; }
            return;
        }
    }
    const float* src = scores + (int64_t)srow * row_stride + off;
    if (MODE == TOPK_GATHER ? len <= k : n <= k) {   // every visible key is selected
        for (int i = tid; i < k; i += NT) {
            out[i] = i < n ? off + i : -1;
            if (MODE == TOPK_SEGS) okey[i] = i < n ? score_key(src[i]) : 0u;
        }
        return;
    }
    const int32_t* crow = cand + (int64_t)row * (MODE == TOPK_GATHER ? cand_len : 0);
    const uint32_t* ckrow = ckeys + (int64_t)row * (MODE == TOPK_GATHER ? cand_len : 0);
    if constexpr (MODE == TOPK_GATHER) n = cand_len;  // candidate slots (key 0 = none)
    // output value of the key at position p of what this workgroup ranks
    auto out_pos = [&](int p) -> int32_t { return MODE == TOPK_GATHER ? crow[p] : off + p; };
    const int lane_base = wv * 64 * EPT + 4 * lane;  // element of (round 0, slot 0) within a block
    const int nblocks = STREAM ? (n + BLOCK - 1) / BLOCK : 1;

    uint32_t key[EPT];
    // Round j of a wave covers positions [w0 + 256 j, w0 + 256 (j + 1)) of its block; when
    // that lies inside the row (wave-uniform test) its keys need no bounds checks.
    auto round_full = [&](int blk, int j) -> bool {
        return blk * BLOCK + wv * 64 * EPT + 256 * (j + 1) <= n;
    };
    // ... and when it starts past the row end it holds only key-0 padding: skipped.
    auto round_live = [&](int blk, int j) -> bool {
        return MODE == TOPK_GATHER || blk * BLOCK + wv * 64 * EPT + 256 * j < n;
    };
    auto load_block = [&](int blk) {
        const int b0 = blk * BLOCK + lane_base;
        if constexpr (MODE == TOPK_GATHER) {         // the candidates' keys, as the segments wrote them
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                const int i0 = b0 + 256 * j;
                if (VEC) {
                    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
                    if (i0 < n) kv = *reinterpret_cast<const uint4*>(ckrow + i0);
                    key[4 * j] = kv.x; key[4 * j + 1] = kv.y; key[4 * j + 2] = kv.z; key[4 * j + 3] = kv.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) key[4 * j + e] = (i0 + e < n) ? ckrow[i0 + e] : 0u;
                }
            }
            return;
        }
        float v[EPT];
#pragma unroll
        for (int j = 0; j < NR; ++j) {               // every load first (one wait for all of them)
            const int i0 = b0 + 256 * j;
            if (VEC) {
                // a lane past the row reads the row's first 16 B instead (its keys are zeroed
                // below); 16 B from i0 < n stay inside the row since row_stride % 4 == 0
                const float4 f = *reinterpret_cast<const float4*>(src + (i0 < n ? i0 : 0));
                v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * j + e] = (i0 + e < n) ? src[i0 + e] : 0.f;
            }
        }
        // Positions past the row get key 0, which no score maps to (a real key is
        // >= 0x007FFFFF): it sorts below every real key, lands in histogram bin 0 of the
        // first pass (subtracted there) and comes after every real key in index order,
        // so it is never selected.
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int i0 = b0 + 256 * j;
            if (round_full(blk, j)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) key[4 * j + e] = score_key(v[4 * j + e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) key[4 * j + e] = (i0 + e < n) ? score_key(v[4 * j + e]) : 0u;
            }
        }
    };
    // Smallest and largest real key of the row.
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int blk = 0; blk < nblocks; ++blk) {
        load_block(blk);
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (!round_live(blk, j)) continue;
            if (MODE != TOPK_GATHER && round_full(blk, j)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo = min(lo, key[4 * j + e]);
                    hi = max(hi, key[4 * j + e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kk = key[4 * j + e];
                    lo = min(lo, kk ? kk : 0xFFFFFFFFu);
                    hi = max(hi, kk);
                }
            }
        }
    }
    lo = wave_reduce(lo, OpMin());
    hi = wave_reduce(hi, OpMax());
    if (tid == 0) { kminmax[0] = 0xFFFFFFFFu; kminmax[1] = 0u; ncand = 0u; }
    // the first pass's histogram starts zeroed (both buffers when they alternate); the
    // candidate list starts as padding (key 0, below and unequal to every real key), so a
    // ranking over it rounded up to 16 entries needs no padding step of its own
    for (int b = tid; b < NHB * NH * HIST_BINS; b += NT) (&hist[0][0])[b] = 0u;
    for (int c = tid; c < CAND_CAP; c += NT) { cand_key[c] = 0u; cand_idx[c] = INT32_MAX; }
    __syncthreads();
    if (lane == 0) {
        atomicMin(&kminmax[0], lo);
        atomicMax(&kminmax[1], hi);
    }
    __syncthreads();
    const uint32_t kmin = kminmax[0], kmax = kminmax[1];

    // Radix select: candidates are the keys with (key >> shift) == prefix.  Every real key
    // shares the first pass's prefix (the bits common to kmin and kmax), so that pass
    // histograms the rounds inside the row without a test.
    int shift = (kmin == kmax) ? 0 : 32 - __clz(kmin ^ kmax);
    uint32_t prefix = shift >= 32 ? 0u : (kmax >> shift);
    uint32_t k_rem = (uint32_t)k;                    // still to take among the candidates
    bool ranked = false;                             // threshold bin resolved by ranking its keys
    bool whole = false;                              // the k-th key's bin is taken whole
    bool first = true;
    int hb = 0;                                      // histogram buffer of this pass
    while (shift > 0) {
        const int width = min(HIST_BITS, shift);
        const int sh_lo = shift - width;
        const uint32_t mask = (1u << width) - 1u;
        const int nb = 1 << width;
        uint32_t (*H)[HIST_BINS] = &hist[hb * NH];
        if (NHB == 1 && !first) {                    // one buffer: zero it now
            for (int b = tid; b < nb * NH; b += NT) H[b / nb][b % nb] = 0u;
            __syncthreads();
        }
        for (int blk = 0; blk < nblocks; ++blk) {
            if (STREAM) load_block(blk);
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if (!round_live(blk, j)) continue;
                uint32_t* Hw = &H[NH > 1 ? wv : 0][0];
                if (first && MODE != TOPK_GATHER && round_full(blk, j)) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) atomicAdd(&Hw[(key[4 * j + e] >> sh_lo) & mask], 1u);
                } else {
                    // key-0 slots are never counted (they would all hit one bin)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t kk = key[4 * j + e];
                        if (kk != 0u && (first || (kk >> shift) == prefix)) atomicAdd(&Hw[(kk >> sh_lo) & mask], 1u);
                    }
                }
            }
        }
        __syncthreads();
        if (NHB == 2) {                              // the next pass's buffer (last read two passes ago)
            uint32_t* nxt = &hist[(hb ^ 1) * NH][0];
            for (int b = tid; b < HIST_BINS; b += NT) nxt[b] = 0u;
        }
        // Bin b with above(b) < k_rem <= above(b) + count(b), above = count in higher bins.
        // Thread t holds bins 2047 - (BPT*t + j) (descending), so above is a prefix sum.
        constexpr int BPT = (HIST_BINS + NT - 1) / NT;

        uint32_t local = 0, hv[BPT];
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = HIST_BINS - 1 - (tid * BPT + j);
            uint32_t c = 0;
            if (b >= 0 && b < nb) {
#pragma unroll
                for (int w = 0; w < NH; ++w) c += H[w][b];
            }
            hv[j] = c;
            local += c;
        }
        const uint32_t incl = wave_incl_scan(local);
        if (lane == 63) wtot[wv] = incl;
        __syncthreads();
        uint32_t above = incl - local;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) above += (i < wv) ? wtot[i] : 0u;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = HIST_BINS - 1 - (tid * BPT + j);
            if (b >= 0 && b < nb && above < k_rem && k_rem <= above + hv[j]) {
                found[0] = (uint32_t)b;
                found[1] = above;
                found[2] = hv[j];
            }
            above += hv[j];
        }
        __syncthreads();
        // found, wtot and this buffer are next written only after the next pass's first barrier
        const uint32_t fb = found[0], fa = found[1];
        const uint32_t in_bin = found[2];
        prefix = (shift >= 32 ? 0u : (prefix << width)) | fb;
        k_rem -= fa;
        shift = sh_lo;
        hb ^= NHB - 1;
        first = false;
        if (in_bin == k_rem) {                       // the whole bin is taken: no ties to cut
            whole = true;
            break;
        }
        if (in_bin <= (uint32_t)CAND_CAP) {          // few keys share the k-th key's bin: rank them
            ranked = true;
            break;
        }
    }

    // The selected positions are ranked into LDS (the histograms are no longer needed)
    // and written out with coalesced stores at the end.
    int32_t* ostage = reinterpret_cast<int32_t*>(&hist[0][0]);
    uint32_t pos_run = 0;
    // Emit in index order the keys that sel(key, position) picks: per block, wave counts
    // from ballots, a prefix over the waves, then ranks within the wave from ballots.
    // With `counted` (a row held in registers), wtot already holds every wave's number of
    // selected keys, and the counting sweep is skipped.
    auto emit = [&](auto&& sel_fn, bool counted) {
        for (int blk = 0; blk < nblocks; ++blk) {
            if (STREAM) load_block(blk);
            // positions are recomputed from an opaque base in every pass, so that no
            // per-round position registers stay live through the whole kernel (spills)
            int b0 = blk * BLOCK + lane_base;
            asm volatile("" : "+v"(b0));
            uint32_t sel_tot = 0, pos = 0;
            if (!STREAM && counted) {
#pragma unroll
                for (int i = 0; i < NT / 64; ++i) pos += (i < wv) ? wtot[i] : 0u;
            } else {
                uint32_t wcount = 0;
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (!round_live(blk, j)) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wcount += (uint32_t)__popcll(__ballot(sel_fn(key[4 * j + e], b0 + 256 * j + e)));
                }
                pos = pos_run + waves_scan<NT>(wcount, wtot, &sel_tot);
            }
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if (!round_live(blk, j)) continue;
                bool sel[4];
                uint32_t r = pos, tot = 0;                   // r: this lane's first output slot
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sel[e] = sel_fn(key[4 * j + e], b0 + 256 * j + e);
                    const uint64_t b = __ballot(sel[e]);
                    r = lanes_below(b, r);
                    tot += (uint32_t)__popcll(b);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (sel[e]) {
                        if (r < (uint32_t)k) {
                            ostage[r] = out_pos(b0 + 256 * j + e);
                            if (MODE == TOPK_SEGS) okey[r] = key[4 * j + e];
                        }
                        ++r;
                    }
                }
                pos += tot;
            }
            pos_run += sel_tot;
        }
    };

    if (ranked) {
        // Gather the bin's keys (with their positions) into LDS and find the k_rem-th of
        // them in (key descending, position ascending) order: the exact threshold pair,
        // and how many keys share its value.  (ncand and the padded list were set up
        // before the first pass.)  A row held in registers also counts, per wave, the keys
        // above the bin (all selected); the ranking adds each wave's selected bin keys, so
        // the emit knows every wave's output offset without a counting sweep.
        uint32_t n_above = 0;
        for (int blk = 0; blk < nblocks; ++blk) {
            if (STREAM) load_block(blk);
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if (!round_live(blk, j)) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kk = key[4 * j + e];
                    if (!STREAM) n_above += (kk >> shift) > prefix ? 1u : 0u;   // key 0 is never above
                    if (kk != 0u && (kk >> shift) == prefix) {
                        const uint32_t at = atomicAdd(&ncand, 1u);
                        if (at < (uint32_t)CAND_CAP) {
                            cand_key[at] = kk;
                            int p0 = blk * BLOCK + lane_base;
                            asm volatile("" : "+v"(p0));
                            cand_idx[at] = p0 + 256 * j + e;
                        }
                    }
                }
            }
        }
        if (!STREAM) {                               // wtot was last read before the pass's final barrier
            const uint32_t wa = wave_sum(n_above);
            if (lane == 0) wtot[wv] = wa;
        }
        __syncthreads();
        const int nc = (int)min(ncand, (uint32_t)CAND_CAP);
        // the ranking reads 16 candidates per step with vector LDS loads; the slots past nc
        // still hold the padding written before the first pass
        const int ncp = (nc + 15) & ~15;
        for (int c = tid; c < nc; c += NT) {
            const uint32_t ck = cand_key[c];
            const int32_t ci = cand_idx[c];
            uint32_t rank = 0, same = 0;
            constexpr int RU = EPT >= 32 ? 2 : 4;       // 16-byte reads per list per step (registers)
            for (int o = 0; o < ncp; o += 4 * RU) {
                uint4 ok[RU];
                int4 oi[RU];
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    ok[u] = *reinterpret_cast<const uint4*>(&cand_key[o + 4 * u]);
                    oi[u] = *reinterpret_cast<const int4*>(&cand_idx[o + 4 * u]);
                }
#pragma unroll
                for (int u = 0; u < RU; ++u) {
                    const uint32_t kq[4] = {ok[u].x, ok[u].y, ok[u].z, ok[u].w};
                    const int32_t iq[4] = {oi[u].x, oi[u].y, oi[u].z, oi[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rank += (kq[e] > ck) || (kq[e] == ck && iq[e] < ci);
                        same += kq[e] == ck;
                    }
                }
            }
            if (rank == k_rem - 1u) { thr_key = ck; thr_idx = ci; thr_ties = same; }
            if (!STREAM && rank < k_rem) atomicAdd(&wtot[ci / (64 * EPT)], 1u);   // selected: its wave's count
        }
        __syncthreads();
        const uint32_t tk = thr_key;
        const int32_t ti = thr_idx;
        if (thr_ties == 1u)                          // the threshold value is unique: a key test suffices
            emit([&](uint32_t kk, int) { return kk >= tk; }, true);
        else
            emit([&](uint32_t kk, int p) { return (kk > tk) || (kk == tk && p <= ti); }, true);
    } else {
        // Digit above the prefix -> selected; equal -> the first k_rem of them in index
        // order (all of them when the bin is taken whole).  Empty candidate slots (key 0)
        // sit anywhere in a candidate list, so they never count as equal (key 0 is never
        // above the prefix either).
        auto digit = [&](uint32_t kk) -> uint32_t { return shift >= 32 ? 0u : (kk >> shift); };
        auto is_eq = [&](uint32_t kk) -> bool { return digit(kk) == prefix && (MODE != TOPK_GATHER || kk != 0u); };
        if (whole) {
            emit([&](uint32_t kk, int) { return digit(kk) > prefix || is_eq(kk); }, false);
        } else {
            // the k_rem-th equal key in index order is the last one taken: find its position
            // (per block: wave counts of equal keys, a prefix over the waves, ballot ranks)
            if (tid == 0) thr_idx = INT32_MAX;
            uint32_t eq_run = 0;
            for (int blk = 0; blk < nblocks; ++blk) {
                if (STREAM) load_block(blk);
                int b0 = blk * BLOCK + lane_base;
                asm volatile("" : "+v"(b0));
                uint32_t wcount = 0;
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (!round_live(blk, j)) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) wcount += (uint32_t)__popcll(__ballot(is_eq(key[4 * j + e])));
                }
                uint32_t eq_tot;
                uint32_t r = eq_run + waves_scan<NT>(wcount, wtot, &eq_tot);
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    if (!round_live(blk, j)) continue;
                    bool eq[4];
                    uint32_t q = r, tot = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        eq[e] = is_eq(key[4 * j + e]);
                        const uint64_t b = __ballot(eq[e]);
                        q = lanes_below(b, q);
                        tot += (uint32_t)__popcll(b);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (eq[e]) {
                            if (q == k_rem - 1u) thr_idx = b0 + 256 * j + e;
                            ++q;
                        }
                    }
                    r += tot;
                }
                eq_run += eq_tot;
            }
            __syncthreads();
            const int32_t ti = thr_idx;
            emit([&](uint32_t kk, int p) { return digit(kk) > prefix || (is_eq(kk) && p <= ti); }, false);
        }
    }
    __syncthreads();
    for (int i = tid; i < k; i += NT) out[i] = ostage[i];
}

// One launch of `rows` workgroups; `len` bounds what one workgroup ranks (the row, a
// segment, or a candidate list) and picks the block shape.
template <int MODE>
hipError_t topk_launch(const ic_topk_args& a, int rows, int len, int seg, int nseg, const int32_t* cand,
                       uint32_t* ckeys, int32_t* out, bool vec, hipStream_t st) {
    ic_seq_group grp{};
    if (a.grp && MODE == TOPK_ROWS) grp = *a.grp;
#define IC_TOPK_GO(NT, EPT, STREAM)                                                                          \
    do {                                                                                                    \
        if (vec)                                                                                            \
            hipLaunchKernelGGL((topk_kernel<NT, EPT, true, STREAM, MODE>), dim3(rows), dim3(NT), 0, st,      \
                               a.scores, a.row_stride, a.first_len, a.seq_len, a.k, out, a.max_len, seg,    \
                               nseg, cand, len, ckeys, a.len_step, a.run_if, grp);                          \
        else                                                                                                \
            hipLaunchKernelGGL((topk_kernel<NT, EPT, false, STREAM, MODE>), dim3(rows), dim3(NT), 0, st,     \
                               a.scores, a.row_stride, a.first_len, a.seq_len, a.k, out, a.max_len, seg,    \
                               nseg, cand, len, ckeys, a.len_step, a.run_if, grp);                          \
        return hipGetLastError();                                                                           \
    } while (0)
    if (len <= 2048) IC_TOPK_GO(256, 8, false);
    if (len <= 4096) IC_TOPK_GO(256, 16, false);
    if constexpr (MODE == TOPK_ROWS) {
        if (len <= 8192) IC_TOPK_GO(512, 16, false);
        if (rows >= TOPK_MANY_ROWS) {                 // several rows per CU
            if (len <= 16384) IC_TOPK_GO(512, 32, false);
            if (len <= 24576) IC_TOPK_GO(1024, 24, false);
            if (len <= 32768) IC_TOPK_GO(512, 64, false);
            // streamed, four rows per CU: faster than one 1024-thread row per CU up to about
            // 64K keys (0.33 against 0.45 ms for 4096 rows of 33K-37K keys); longer rows keep
            // the per-wave histograms of 1024 x 32 (1.13 against 1.29 ms at 127K-131K)
            if (len <= 65536) IC_TOPK_GO(512, 32, true);
        } else {                                      // about one row per CU: all threads on a row
            if (len <= 16384) IC_TOPK_GO(1024, 16, false);
            if (len <= 32768) IC_TOPK_GO(1024, 32, false);
        }
        IC_TOPK_GO(1024, 32, true);
    } else {
        // a segment, or a candidate list of at most TOPK_GATHER_MAX keys: one register-resident
        // block of 1024 x 16 (32 keys per thread spill in these modes)
        if (len <= 16384) IC_TOPK_GO(1024, 16, false);
        return hipErrorInvalidValue;
    }
#undef IC_TOPK_GO
}

}  // namespace

int topk_segments(const ic_topk_args& a) {
    if (a.max_len <= 32768 || a.rows > TOPK_SEG_MAX_ROWS) return 0;
    const int64_t nseg = ((int64_t)a.max_len + TOPK_SEG - 1) / TOPK_SEG;
    // the candidate list must fit one register-resident 1024 x 16 block
    return nseg * a.k <= TOPK_GATHER_MAX ? (int)nseg : 0;
}

size_t topk_ws_bytes(const ic_topk_args& a) {
    const int nseg = topk_segments(a);
    return nseg ? 2 * (size_t)a.rows * nseg * a.k * sizeof(int32_t) : 0;   // positions, then keys
}

hipError_t launch_topk(const ic_topk_args& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    const bool vec = (a.row_stride % 4 == 0) && (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0);
    const int nseg = topk_segments(a);
    if (nseg && a.cand != nullptr) {
        // segments of TOPK_SEG keys -> candidates [rows][nseg * k] (positions, keys), then one select per row
        const int clen = nseg * a.k;
        uint32_t* ckeys = reinterpret_cast<uint32_t*>(a.cand + (size_t)a.rows * clen);
        hipError_t e = topk_launch<TOPK_SEGS>(a, a.rows * nseg, TOPK_SEG, TOPK_SEG, nseg, nullptr, ckeys, a.cand,
                                              vec && TOPK_SEG % 4 == 0, st);
        if (e != hipSuccess) return e;
        return topk_launch<TOPK_GATHER>(a, a.rows, clen, 0, 1, a.cand, ckeys, a.idx, clen % 4 == 0, st);
    }
    return topk_launch<TOPK_ROWS>(a, a.rows, a.max_len, 0, 1, nullptr, nullptr, a.idx, vec, st);
}
