// Shared device-side helpers for the gfx950 (CDNA4) kernels: vector types,
// MFMA wrappers, cross-lane reductions and the launch interface between the
// C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ic {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---- MFMA tiles (16 x 16 output; lane l holds column l%16, rows 4*(l/16)+0..3) ----
// A operand: lane l holds row l%16 and a 1/4 slice of K selected by l/16;
// B operand: lane l holds column l%16 and the same K slice.  Any consistent
// lane->K assignment for A and B gives the same contraction.

__device__ __forceinline__ f32x4 mfma_bf16_k32(const i32x4& a, const i32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp8 e4m3 x fp8 e4m3, K = 128 (32 bytes per lane); unit block scales.
__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same contraction with an E8M0 scale on A: lane l's byte scales row l%16 over K block
// l/16 (32 elements) by 2^(byte - 127).  B is unscaled.
__device__ __forceinline__ f32x4 mfma_fp8_k128_scale_a(const i32x8& a, int scale_a, const i32x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}

// ---- cross-lane sums over the four 16-lane rows of a wave ----
// x + x from the row 16 lanes away (rows 0<->1, 2<->3).
__device__ __forceinline__ float sum_xor16(float x) {
    u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + x from the lane 32 away.
__device__ __forceinline__ float sum_xor32(float x) {
    u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// IEEE 754-2019 maximum (NaN-propagating): v_maximum3_f32 needs no input canonicalisation,
// unlike fmaxf on values the compiler cannot prove canonical (MFMA results).
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_xor16(float x) {
    u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- memory -> LDS DMA (global_load_lds), waited for by explicit vmcnt counts ----
// The loads are inline asm with M0 as an operand, so the compiler neither counts them nor
// inserts its own waits for LDS reads behind them: every wait is the caller's.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 16 bytes per lane from base + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma_b128(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
// 4 bytes per lane from base + voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma_b32(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// vmcnt(n) for a wave-uniform n that is a multiple of 4 below 32; any other n waits for
// every load (always safe: it only waits longer than asked).
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
    case 0: wait_vm<0>(); break;
    case 4: wait_vm<4>(); break;
    case 8: wait_vm<8>(); break;
    case 12: wait_vm<12>(); break;
    case 16: wait_vm<16>(); break;
    case 20: wait_vm<20>(); break;
    case 24: wait_vm<24>(); break;
    case 28: wait_vm<28>(); break;
    default: wait_vm<0>(); break;
    }
}
// Slot permutation of a staged K or V half row r (only r % 16 matters): 16-byte slot j holds
// the half's chunk j ^ dma_swz(r).  For 256-byte halves (16 chunks), r ^ (r << 1) was the
// fastest of a dozen candidates for both read patterns (K fragments with ds_read_b128,
// transposed V with ds_read_b64_tr_b16) in an LDS microbenchmark; for 128-byte halves the
// 8 even (odd) rows of a K tile get distinct slots and the rows of a transposed V read
// distinct chunk pairs.
template <int NCH>
__device__ __forceinline__ uint32_t dma_swz(int r) {
    static_assert(NCH == 16 || NCH == 8, "half row must be 256 or 128 bytes");
    return NCH == 16 ? (uint32_t)((r ^ (r << 1)) & 15) : (uint32_t)((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}

// Order-preserving map of an fp32 score to u32 (larger float -> larger key).
// -0.0 is folded onto +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    // negative: all bits flipped; otherwise the sign bit set (three VALU ops)
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}


// Two fp32 -> bf16 with round-to-nearest-even, packed (lo in bits 0-15): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace ic

// ---- host-side launchers implemented in the .hip files ----

// A group of consecutive sequences of a ragged batch served by one launch.  Sequence i of
// the group owns the launch's packed query rows [row0[i], row0[i+1]); its row r sits at
// position pos0[i] + r - row0[i] and sees that sequence's own keys, cache slot seq[i] of the
// k_I / kv arrays.  For the indexer, its query blocks are [blk0[i], blk0[i+1]).  Passed to the
// kernels by value (about 1 KB of kernel arguments), so a launch needs no table in memory.
constexpr int IC_GROUP_MAX = 64;
struct ic_seq_group {
    int32_t n;                          // sequences in the group; 0: the launch is not grouped
    int32_t row0[IC_GROUP_MAX + 1];
    int32_t pos0[IC_GROUP_MAX];
    int32_t seq[IC_GROUP_MAX];
    int32_t blk0[IC_GROUP_MAX + 1];
};

namespace ic {
// The group entry i with start[i] <= x < start[i + 1] (start ascending, start[0] <= x).
__device__ __forceinline__ int group_find(const int32_t* start, int n, int x) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}
}  // namespace ic

struct ic_indexer_args {
    const void* q_I;      // [Lq_total, H_I, d_I] of this sequence, row 0 = first query of the call
    const float* w;       // [Lq_total, H_I]
    const void* k_I;      // [Lk, d_I]
    float* scores;        // tile rows: [nq, row_stride]
    int64_t row_stride;
    int32_t q_begin;      // first query (index into q_I / w) of this tile
    int32_t nq;           // queries in this tile
    int32_t pos_begin;    // absolute position of query q_begin
    int32_t H_I, d_I;
    int32_t fp8;
    int32_t q_step = 1;   // query t of the tile is q_I row q_begin + t * q_step at position
                          // pos_begin + t * q_step (strided probe rows); score row t stays dense
    const int32_t* run_if = nullptr;   // optional device flag: the launch does nothing while it is 0
    // Grouped launch (several sequences): q_I / w rows, score rows and row counts follow the
    // group's packed rows (q_begin, nq and pos_begin are then unused); sequence i's keys start
    // at k_I + grp->seq[i] * k_seq_bytes.
    const ic_seq_group* grp = nullptr;
    int64_t k_seq_bytes = 0;
};
hipError_t launch_indexer_prefill(const ic_indexer_args& a, hipStream_t st);

struct ic_indexer_decode_args {
    const void* q_I;      // [B, H_I, d_I]: one query per sequence
    const float* w;       // [B, H_I]
    const void* k_I;      // [B, Lk, d_I]
    const int32_t* seq_len;  // [B] device: row b sees seq_len[b] keys
    float* scores;        // [B, score_stride]
    int64_t score_stride; // >= Lk
    int32_t B, Lk, H_I, d_I, fp8;
};
hipError_t launch_indexer_decode(const ic_indexer_decode_args& a, hipStream_t st);

struct ic_topk_args {
    const float* scores;  // [rows, row_stride]
    int64_t row_stride;
    int32_t rows;
    int32_t first_len;    // visible entries of row 0; row r has first_len + r (when seq_len == NULL)
    const int32_t* seq_len;  // optional device [rows]: row r has seq_len[r] visible entries
    int32_t k;
    int32_t* idx;         // [rows, k]
    int32_t max_len;      // upper bound of any row's visible length (host-known)
    int32_t* cand;        // optional workspace of topk_ws_bytes(): few long rows run segmented
    int32_t len_step = 1; // without seq_len, row r has first_len + r * len_step visible entries
    const int32_t* run_if = nullptr;   // optional device flag: the launch does nothing while it is 0
    const ic_seq_group* grp = nullptr; // grouped rows: row r of sequence i has pos0[i] + r - row0[i] + 1 entries
};
// Few long rows (decode) are ranked in TOPK_SEG-key segments first, then over the
// segments' candidates; that needs topk_ws_bytes() of workspace (0 otherwise).
constexpr int TOPK_SEG = 16384;                 // keys per segment (one register-resident block)
constexpr int TOPK_SEG_MAX_ROWS = 1024;
constexpr int TOPK_GATHER_MAX = 16384;          // candidates per row the second launch ranks
int topk_segments(const ic_topk_args& a);
size_t topk_ws_bytes(const ic_topk_args& a);
hipError_t launch_topk(const ic_topk_args& a, hipStream_t st);

struct ic_attn_args {
    const void* q;        // [nq, H, d] bf16
    const void* kv;       // per sequence [Lk, 2, d] bf16; sequence of query i = i / q_per_seq
    const int32_t* idx;   // [nq, k]
    void* out;            // [nq, H, d] bf16
    int64_t kv_seq_stride;   // elements between sequences in kv
    int32_t Lk;              // KV rows per sequence (idx entries >= Lk are ignored)
    int32_t nq, q_per_seq, H, d, k;
    // split-K (decode): nsplit > 1 (a multiple of 4) writes partials to ws and a
    // combine kernel merges them
    int32_t nsplit;
    float* ws;
    const ic_seq_group* grp = nullptr; // grouped queries: query r belongs to cache slot seq[i] (prefill only)
};
hipError_t launch_sparse_attn(const ic_attn_args& a, hipStream_t st);

// Multi-layer distillation loss (forward) of the queries of one score tile.
constexpr int IC_DISTILL_MAX_K = 4096;
constexpr int IC_DISTILL_MAX_SERVED = 16;
struct ic_distill_args {
    const float* scores;      // indexer score tile [nrows, score_stride]; row r = query q_begin + r, keys 0..pos
    int64_t score_stride;
    const int32_t* idx;       // [Lq, k] of this sequence: the entries the loss is taken over
    const void* q[IC_DISTILL_MAX_SERVED];    // served layer j: [Lq, H, d] bf16 of this sequence
    const void* kv[IC_DISTILL_MAX_SERVED];   // served layer j: [Lk, 2, d] bf16 of this sequence
    float* kl;                // [Lq] of this sequence, nats
    int32_t q_begin, nrows, pos0, Lk, nserved, H, d, k;
};
hipError_t launch_distill(const ic_distill_args& a, hipStream_t st);
// Mean of n floats, summed in a fixed order (one workgroup).
hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t st);

// Per-row overlap of two index caches [rows, k] (rows ascending, -1 padded); means may be NULL.
// Row r of A is at ia + r * a_row_step * k (a_row_step = 1: contiguous).
hipError_t launch_overlap(const int32_t* ia, const int32_t* ib, int64_t rows, int k, int32_t* inter, float* jac,
                          float* rec, float* means, hipStream_t st, int64_t a_row_step = 1);
// Drift decision of one probe: hit = sum of inter[0..P), refresh iff hit < tau * own;
// writes flag[0] (1 = refresh), refreshed[0] and recall[0] = hit / own.
hipError_t launch_drift_decision(const int32_t* inter, int P, int64_t own, double tau, int32_t* flag,
                                 int32_t* refreshed, float* recall, hipStream_t st);
size_t sparse_attn_ws_bytes(int32_t nq, int32_t H, int32_t d, int32_t nsplit);
