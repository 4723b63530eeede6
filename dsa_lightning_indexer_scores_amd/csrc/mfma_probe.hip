// Sustained rates of this GPU, measured so that the kernels' roofline fractions can
// be read against what the hardware actually sustains: fp8 MFMA throughput, and the
// HBM read bandwidth of a plain streaming kernel.
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

}  // namespace

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
