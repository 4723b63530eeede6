// Sustained rates of this GPU, measured so that the kernels' roofline fractions can
// be read against what the hardware actually sustains: fp8 MFMA throughput, the
// HBM read bandwidth of a plain streaming kernel, and the rate of a pure row gather
// over a given index list (the sparse attention's address stream without its math).
//
// Each wave runs a stream of independent v_mfma_f32_16x16x128_f8f6f4 over 8 A
// slabs and 2 B slabs (the shape of an indexer tile loop).  With random=0 the
// operands are constant e4m3 ones; with random=1 they are random e4m3 bytes and
// B changes every iteration, as it does when an indexer sweeps its keys.  Data
// that toggles draws more power, and the part clocks down to hold its power
// limit, so the random stream sustains markedly less than the constant one.
//
// A third stream has the indexer's own operand pattern: fixed random q_I slabs, a fresh
// random key tile from LDS every step and the scaled linear-term MFMA; a fourth adds the
// indexer's vector epilogue to it.
//
// This is measurement support only (built into libicprobe.so, loaded by the
// benchmark); nothing on the indexer path uses it.
#include "common.h"

using namespace ic;

namespace {

__device__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Four finite e4m3 codes with |value| <= 2 (exponent field <= 8), from a hash.
__device__ int random_e4m3x4(uint32_t seed) {
    const uint32_t h = mix(seed);
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = (h >> (8 * i)) & 0xffu;
        r |= ((b & 0x80u) | ((b & 0x7fu) % 0x40u)) << (8 * i);
    }
    return (int)r;
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_stream_kernel(float* __restrict__ out, int iters) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    i32x8 A[8], B[2];
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 8; ++i) A[j][i] = RANDOM ? random_e4m3x4(t * 131u + j * 17u + i) : 0x38383838;
    for (int j = 0; j < 2; ++j)
        for (int i = 0; i < 8; ++i) B[j][i] = RANDOM ? random_e4m3x4(t * 977u + j * 29u + i + 7u) : 0x38383838;
    f32x4 c[8];
    for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
        const int bi = it & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[j], B[bi], c[j], 0, 0, 0, 0, 0, 0);
        if (RANDOM) {
#pragma unroll
            for (int i = 0; i < 8; ++i) B[bi][i] ^= 0x01010101 << (it & 3);   // keeps the operand bits moving
        }
    }
    float s = 0.f;
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[t] = s;                                      // keeps the stream live
}

// The indexer's operand pattern with none of its vector work: per 16-key tile, a B
// fragment of fresh random e4m3 keys read from LDS (a 64-key table per wave, as the
// indexer stages its keys), 8 score MFMAs against 8 fixed random A slabs (two queries x
// four head tiles of q_I) and one scaled MFMA (the head-weighted linear term).  So it
// draws the power the indexer's matrix work draws, and its rate is the ceiling the
// indexer's MFMA stream can sustain on this GPU.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_indexer_operands_kernel(
    float* __restrict__ out, int iters) {
    constexpr int TABLE = 64 * 1024;                 // bytes of random keys per workgroup (16 KB per wave)
    __shared__ __attribute__((aligned(32))) uint8_t keys[TABLE];
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    for (int i = threadIdx.x; i < TABLE / 4; i += 256)
        reinterpret_cast<int*>(keys)[i] = random_e4m3x4(blockIdx.x * 65537u + (uint32_t)i * 3u + 11u);
    i32x8 A[8], L;
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 8; ++i) A[j][i] = random_e4m3x4(t * 131u + j * 17u + i);
    for (int i = 0; i < 8; ++i) L[i] = random_e4m3x4(t * 313u + i + 5u);
    const int scale = 120 + (int)(mix(t) & 7u);
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint8_t* base = keys + wv * (TABLE / 4) + (lane & 15) * 160 + (lane >> 4) * 32;   // skewed rows
    f32x4 c[8], cl = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 16 keys x 128 bytes per tile; 6 tiles of distinct rows fit a wave's 16 KB.  The next
    // tile is read while this one's MFMAs run, as the indexer's pipeline does.
    i32x8 B = *reinterpret_cast<const i32x8*>(base);
    for (int it = 0; it < iters; ++it) {
        i32x8 Bn = *reinterpret_cast<const i32x8*>(base + ((it + 1) % 6) * 2560);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[j], B, c[j], 0, 0, 0, 0, 0, 0);
        cl = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(L, B, cl, 0, 0, 0, scale, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" : "+v"(Bn));                 // the next tile stays a register value read ahead
        B = Bn;
    }
    float s = cl[0] + cl[1] + cl[2] + cl[3];
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[t] = s;                                      // keeps the stream live
}

// Lane row g of the result holds the sum of p_g over the four lane rows (three swaps, three
// adds): four key tiles' head sums finished at once.
__device__ __forceinline__ float lane_rows_sum4(float p0, float p1, float p2, float p3) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const u32x2 b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
    const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    const u32x2 c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The indexer's whole arithmetic with none of its memory traffic, per-block key loads or
// barriers: the operand stream above (8 score MFMAs and the scaled linear-term MFMA per
// 16-key tile, each tile's keys read from LDS one tile ahead) plus its vector epilogue,
// pipelined the way the indexer runs it.  In stage t the MFMAs of tile t issue beside the
// epilogue of tile t-1, each MFMA followed by four vector ops: per query the two linear-term
// parts added, then one fma per head with |y| as a free input modifier (16 heads per lane).
// After each block of 8 tiles the lane-row sums finish four tiles per query at once, and
// their results are added into a register where the indexer stores its scores.  Its rate is
// what the indexer's instruction mix sustains on this GPU.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_indexer_compute_kernel(
    float* __restrict__ out, int nblocks) {
    constexpr int TABLE = 64 * 1024;
    constexpr int NKT = 8;                           // tiles per block, as the indexer's 128-key blocks
    __shared__ __attribute__((aligned(32))) uint8_t keys[TABLE];
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    for (int i = threadIdx.x; i < TABLE / 4; i += 256)
        reinterpret_cast<int*>(keys)[i] = random_e4m3x4(blockIdx.x * 65537u + (uint32_t)i * 3u + 11u);
    i32x8 A[8], L;
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 8; ++i) A[j][i] = random_e4m3x4(t * 131u + j * 17u + i);
    for (int i = 0; i < 8; ++i) L[i] = random_e4m3x4(t * 313u + i + 5u);
    float wr[2][16];                                 // head weights of the wave's two queries
    for (int q = 0; q < 2; ++q)
        for (int i = 0; i < 16; ++i) wr[q][i] = (float)(mix(t * 7u + q * 97u + i) & 0xffu) * (1.f / 512.f);
    const int scale = 120 + (int)(mix(t) & 7u);
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint8_t* base = keys + wv * (TABLE / 4) + (lane & 15) * 160 + (lane >> 4) * 32;   // skewed rows
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    float sink = 0.f;
    for (int b = 0; b < nblocks; ++b) {
        f32x4 acc[2][8];
        f32x4 lin[2];
        float val[2][NKT];
        i32x8 Bcur = *reinterpret_cast<const i32x8*>(base + (b % 6) * 2560);
#pragma unroll
        for (int kt = 0; kt <= NKT; ++kt) {
            i32x8 Bnxt;
            if (kt + 1 < NKT) Bnxt = *reinterpret_cast<const i32x8*>(base + ((b + kt + 1) % 6) * 2560);
            if (kt < NKT) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[kt & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[j], Bcur, z, 0, 0, 0, 0, 0, 0);
                lin[kt & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(L, Bcur, z, 0, 0, 0, scale, 0, 127);
            }
            if (kt > 0) {
                const f32x4& l = lin[(kt - 1) & 1];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float v = l[2 * q] + l[2 * q + 1];
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                        for (int e = 0; e < 4; ++e) v = fmaf(wr[q][4 * ht + e], fabsf(acc[(kt - 1) & 1][4 * q + ht][e]), v);
                    val[q][kt - 1] = v;
                }
            }
            if (kt + 1 < NKT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if (kt > 0 && kt < NKT) {
#pragma unroll
                for (int i = 0; i < 9; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            }
            if (kt > 0) {
#pragma unroll
                for (int q = 0; q < 2; ++q) asm volatile("" : "+v"(val[q][kt - 1]));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < NKT) Bcur = Bnxt;
        }
#pragma unroll
        for (int grp = 0; grp < NKT / 4; ++grp)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                sink += lane_rows_sum4(val[q][4 * grp], val[q][4 * grp + 1], val[q][4 * grp + 2], val[q][4 * grp + 3]);
    }
    out[t] = sink;                                   // keeps the stream live
}

// Grid-stride 16-byte reads of n16 vectors; one word per thread keeps the loads live.
__global__ __launch_bounds__(256) void stream_read_kernel(const int4* __restrict__ p, size_t n16, int* __restrict__ out) {
    size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 1024;
    int acc = 0;
    for (; i < n16; i += stride) {
        int4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (i + 256 * u < n16) ? p[i + 256 * u] : make_int4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// The sparse attention's data movement with no math: one wave per query row of idx
// [nq, k], four waves per workgroup; per step of 32 entries the K halves and then the V
// halves of the named rows (row_bytes = 2 * HB) go straight into a K and a V stage of
// the wave's LDS (global_load_lds_dwordx4, 64 lanes x 16 bytes), K(s+1) issued once K(s)
// has landed and V(s+1) once V(s) has, and the idx row reaches LDS through a ring of two
// 256-entry chunks the same way.  Entries outside [0, Lk) read row 0; steps past the
// row's last real entry are not run.  One LDS word per lane is written to out at the end.
template <int HB>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ kv, const int32_t* __restrict__ idx,
                                                          int nq, int k, int Lk, int* __restrict__ out) {
    constexpr int KT = 32, NCH = HB / 16, RPI = 1024 / HB, NI = KT / RPI, SB = KT * HB, ICH = 256, SPC = ICH / KT;
    __shared__ __attribute__((aligned(1024))) uint8_t stage_all[4][2][SB];
    __shared__ __attribute__((aligned(16))) int32_t ring_all[4][2 * ICH];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qi = blockIdx.x * 4 + wv;
    if (qi >= nq) return;
    const int32_t* irow = idx + (int64_t)qi * k;
    const int32_t* ring = ring_all[wv];
    const uint32_t k_lds = lds_addr(stage_all[wv][0]), v_lds = lds_addr(stage_all[wv][1]), ring_lds = lds_addr(ring);
    int j_last = -1;                                     // as the attention: steps past the last real entry are not run
    for (int jb = 0; jb < k; jb += 64 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
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
    if (nsteps == 0) return;
    auto issue_chunk = [&](int c) {
        const uint32_t dst = ring_lds + (uint32_t)(c & 1) * (ICH * 4);
#pragma unroll
        for (int w = 0; w < ICH / 64; ++w)
            dma_b32(irow, (uint32_t)min(c * ICH + 64 * w + lane, k - 1) * 4u, dst + 256u * w);
    };
    uint32_t roff[NI];
    auto offsets = [&](int s) {
        const int32_t* ir = ring + ((s / SPC) & 1) * ICH + (s % SPC) * KT;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t v = (uint32_t)ir[RPI * i + lane / NCH];
            roff[i] = (v < (uint32_t)Lk ? v : 0u) * (uint32_t)(2 * HB) + (uint32_t)(lane % NCH) * 16u;
        }
    };
    auto issue_half = [&](uint32_t dst, uint32_t half_off) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < NI; ++i) dma_b128(kv, roff[i] + half_off, dst + 1024u * i);
    };
    issue_chunk(0);
    issue_chunk(1);
    wait_vm<ICH / 64>();
    offsets(0);
    issue_half(k_lds, 0);
    issue_half(v_lds, HB);
    for (int s = 0; s < nsteps; ++s) {
        const bool more = s + 1 < nsteps;
        const bool cs = s > 0 && s % SPC == 0;           // an idx chunk went out after V(s)
        if (cs) wait_vm<NI + ICH / 64>(); else wait_vm<NI>();                    // K(s) landed
        if (more) {
            offsets(s + 1);
            issue_half(k_lds, 0);
        }
        if (more) {                                                              // V(s) landed
            if (cs) wait_vm<NI + ICH / 64>(); else wait_vm<NI>();
        } else {
            wait_vm<0>();
        }
        if (more) {
            issue_half(v_lds, HB);
            if ((s + 1) % SPC == 0) issue_chunk((s + 1) / SPC + 1);
        }
    }
    wait_vm<0>();
    out[(int64_t)qi * 64 + lane] = reinterpret_cast<const int*>(stage_all[wv][1])[lane];
}

}  // namespace

// Pure gather of the rows idx [nq, k] names from kv (row_bytes 256 or 512 per row, Lk
// rows); out needs nq * 64 ints.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int icp_gather_rows(const void* kv, const int32_t* idx, int nq, int k,
                                                                     int Lk, int row_bytes, int* out, void* stream) {
    if (kv == nullptr || idx == nullptr || out == nullptr || nq < 1 || k < 1 || Lk < 1) return (int)hipErrorInvalidValue;
    const dim3 grid((nq + 3) / 4);
    if (row_bytes == 512)
        hipLaunchKernelGGL(gather_rows_kernel<256>, grid, dim3(256), 0, (hipStream_t)stream,
                           static_cast<const uint8_t*>(kv), idx, nq, k, Lk, out);
    else if (row_bytes == 256)
        hipLaunchKernelGGL(gather_rows_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream,
                           static_cast<const uint8_t*>(kv), idx, nq, k, Lk, out);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from `src` with `blocks` workgroups of 256 threads;
// out needs blocks * 256 ints.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int icp_stream_read(const void* src, size_t bytes, int blocks,
                                                                     int* out, void* stream) {
    if (src == nullptr || out == nullptr || blocks < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const int4*>(src), bytes / 16, out);
    return (int)hipGetLastError();
}

// Launches `blocks` workgroups of 4 waves, each wave issuing 8 * iters fp8 MFMAs of
// 16x16x128 (65536 flop each), or 9 * iters with random = 2 (the indexer's operand
// pattern: 8 score MFMAs plus the linear-term one per key tile) or random = 3 (the same
// with the indexer's vector epilogue; iters a multiple of 8); out needs blocks * 256
// floats.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int icp_mfma_stream(int random, int blocks, int iters, float* out,
                                                                     void* stream) {
    if (blocks < 1 || iters < 1 || out == nullptr) return (int)hipErrorInvalidValue;
    if (random == 3) {
        if (iters % 8 != 0) return (int)hipErrorInvalidValue;
        hipLaunchKernelGGL(mfma_indexer_compute_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters / 8);
    } else if (random == 2)
        hipLaunchKernelGGL(mfma_indexer_operands_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    else if (random)
        hipLaunchKernelGGL(mfma_stream_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    else
        hipLaunchKernelGGL(mfma_stream_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}
