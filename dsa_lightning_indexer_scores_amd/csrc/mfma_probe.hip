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
// This is measurement support only (built into libicprobe.so, loaded by the
// benchmark); nothing on the indexer path uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// One wave per query row of idx [nq, k]: every 32 entries, the rows' bytes are read with
// coalesced 16-byte loads (64 lanes cover 64 * 16 / row_bytes rows per instruction; row
// offsets de-interleaved through LDS as in the attention kernel), two steps in flight,
// and folded into an XOR that keeps the loads live.  Entries < 0 or >= Lk read row 0.
template <int ROWB>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ kv, const int32_t* __restrict__ idx,
                                                          int nq, int k, int Lk, int* __restrict__ out) {
    constexpr int KTG = 32, PPR = ROWB / 16, RPI = 64 / PPR, NI = KTG / RPI;
    __shared__ __attribute__((aligned(16))) uint32_t ioff_all[4][KTG];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qi = blockIdx.x * 4 + wv;
    if (qi >= nq) return;
    const int32_t* irow = idx + (int64_t)qi * k;
    uint32_t* ioff = ioff_all[wv];
    const uint32_t piece = (lane % PPR) * 16;
    const int nsteps = __builtin_amdgcn_readfirstlane((k + KTG - 1) / KTG);
    int4 acc = make_int4(0, 0, 0, 0);
    int4 raw[2][NI];
    auto issue = [&](int s, int slot) {
        __builtin_amdgcn_sched_barrier(0);
        const int j = s * KTG + (lane & 31);
        const int v = irow[min(j, k - 1)];
        const bool ok = j < k && lane < 32 && (uint32_t)v < (uint32_t)Lk;
        if (lane < KTG) ioff[(lane % RPI) * NI + lane / RPI] = (ok ? (uint32_t)v : 0u) * (uint32_t)ROWB;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        uint32_t roff[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) roff[i] = ioff[(lane / PPR) * NI + i];
#pragma unroll
        for (int i = 0; i < NI; ++i) raw[slot][i] = *reinterpret_cast<const int4*>(kv + (roff[i] + piece));
    };
    auto fold = [&](int slot) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            acc.x ^= raw[slot][i].x; acc.y ^= raw[slot][i].y; acc.z ^= raw[slot][i].z; acc.w ^= raw[slot][i].w;
        }
    };
    issue(0, 0);
    for (int s = 0; s < nsteps; s += 2) {
        issue(min(s + 1, nsteps - 1), 1);
        fold(0);
        issue(min(s + 2, nsteps - 1), 0);
        if (s + 1 < nsteps) fold(1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    out[(int64_t)qi * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// Pure gather of the rows idx [nq, k] names from kv (row_bytes 256 or 512 per row, Lk
// rows); out needs nq * 64 ints.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int icp_gather_rows(const void* kv, const int32_t* idx, int nq, int k,
                                                                     int Lk, int row_bytes, int* out, void* stream) {
    if (kv == nullptr || idx == nullptr || out == nullptr || nq < 1 || k < 1 || Lk < 1) return (int)hipErrorInvalidValue;
    const dim3 grid((nq + 3) / 4);
    if (row_bytes == 512)
        hipLaunchKernelGGL(gather_rows_kernel<512>, grid, dim3(256), 0, (hipStream_t)stream,
                           static_cast<const uint8_t*>(kv), idx, nq, k, Lk, out);
    else if (row_bytes == 256)
        hipLaunchKernelGGL(gather_rows_kernel<256>, grid, dim3(256), 0, (hipStream_t)stream,
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
// 16x16x128 (65536 flop each); out needs blocks * 256 floats.  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int icp_mfma_stream(int random, int blocks, int iters, float* out,
                                                                     void* stream) {
    if (blocks < 1 || iters < 1 || out == nullptr) return (int)hipErrorInvalidValue;
    if (random)
        hipLaunchKernelGGL(mfma_stream_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    else
        hipLaunchKernelGGL(mfma_stream_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}
