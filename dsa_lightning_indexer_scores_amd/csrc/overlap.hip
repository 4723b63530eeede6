// Cross-layer overlap of two index caches.
//
// The agent skill page ("Indexcache Sparse Attention Acceleration", Step 1)
// decides which layers may share indices by the per-position Jaccard similarity
// of their top-k sets; the arXiv abstract reports that adjacent layers' sets
// overlap strongly.  Per row r of idx_a, idx_b [rows, k] (each row ascending,
// then -1 padding, as the top-k writes it):
//     inter[r]   = |A & B|
//     jaccard[r] = inter / (|A | B| + 1e-8)
//     recall[r]  = inter / |B|  (0 when B is empty)
// and, optionally, means = (mean_r jaccard[r], mean_r recall[r]), summed in a
// fixed order so that they are deterministic.
//
// One workgroup per row: B's entries go to LDS, each thread takes a slice of A
// and binary-searches it there (both rows are sorted), and the counts are summed
// with wave reductions.
#include "common.h"

using namespace ic;

namespace {

constexpr int OV_NT = 256;
constexpr int OV_MAXK = 4096;

__device__ __forceinline__ int wave_isum(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ __launch_bounds__(OV_NT) void overlap_kernel(const int32_t* __restrict__ ia, const int32_t* __restrict__ ib,
                                                         int k, int32_t* __restrict__ inter,
                                                         float* __restrict__ jac, float* __restrict__ rec,
                                                         int64_t a_row_step) {
    __shared__ int32_t bl[OV_MAXK];
    __shared__ int part[3][OV_NT / 64];
    const int64_t row = blockIdx.x;
    const int32_t* a = ia + row * a_row_step * k;
    const int32_t* b = ib + row * k;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int na = 0, nb = 0;
    for (int i = tid; i < k; i += OV_NT) {
        const int32_t vb = b[i];
        bl[i] = vb;
        nb += vb >= 0;
        na += a[i] >= 0;
    }
    __syncthreads();
    // |B|: the -1 padding is a suffix, so B's valid entries are bl[0 .. nbt)
    na = wave_isum(na);
    nb = wave_isum(nb);
    if (lane == 0) { part[0][wv] = na; part[1][wv] = nb; }
    __syncthreads();
    int nat = 0, nbt = 0;
#pragma unroll
    for (int w = 0; w < OV_NT / 64; ++w) { nat += part[0][w]; nbt += part[1][w]; }
    int hit = 0;
    for (int i = tid; i < nat; i += OV_NT) {
        const int32_t x = a[i];
        int lo = 0, hi = nbt;                          // first position with bl[pos] >= x
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (bl[mid] < x) lo = mid + 1; else hi = mid;
        }
        hit += (lo < nbt && bl[lo] == x);
    }
    hit = wave_isum(hit);
    if (lane == 0) part[2][wv] = hit;
    __syncthreads();
    if (tid == 0) {
        int it = 0;
#pragma unroll
        for (int w = 0; w < OV_NT / 64; ++w) it += part[2][w];
        const int un = nat + nbt - it;
        if (inter) inter[row] = it;
        if (jac) jac[row] = (float)it / ((float)un + 1e-8f);
        if (rec) rec[row] = nbt > 0 ? (float)it / (float)nbt : 0.f;
    }
}

// means[0] = mean of jac, means[1] = mean of rec: one workgroup, fixed per-thread strides and
// a fixed tree, so the result does not depend on timing.
__global__ __launch_bounds__(1024) void overlap_mean_kernel(const float* __restrict__ jac, const float* __restrict__ rec,
                                                            int64_t rows, float* __restrict__ means) {
    __shared__ float sj[1024], sr[1024];
    const int tid = threadIdx.x;
    float j = 0.f, r = 0.f;
    for (int64_t i = tid; i < rows; i += 1024) {
        j += jac[i];
        r += rec[i];
    }
    sj[tid] = j;
    sr[tid] = r;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (tid < s) {
            sj[tid] += sj[tid + s];
            sr[tid] += sr[tid + s];
        }
        __syncthreads();
    }
    if (tid == 0) {
        means[0] = sj[0] / (float)rows;
        means[1] = sr[0] / (float)rows;
    }
}

}  // namespace

hipError_t launch_overlap(const int32_t* ia, const int32_t* ib, int64_t rows, int k, int32_t* inter, float* jac,
                          float* rec, float* means, hipStream_t st, int64_t a_row_step) {
    if (rows <= 0) return hipSuccess;
    if (k < 1 || k > OV_MAXK) return hipErrorInvalidValue;
    hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)rows), dim3(OV_NT), 0, st, ia, ib, k, inter, jac, rec,
                       a_row_step);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || means == nullptr) return e;
    hipLaunchKernelGGL(overlap_mean_kernel, dim3(1), dim3(1024), 0, st, jac, rec, rows, means);
    return hipGetLastError();
}

namespace {

// Drift decision of a probe: the pooled recall's numerator summed exactly (int64, one
// workgroup, fixed order), the comparison taken in double.
__global__ __launch_bounds__(256) void drift_decision_kernel(const int32_t* __restrict__ inter, int P, int64_t own,
                                                             double tau, int32_t* __restrict__ flag,
                                                             int32_t* __restrict__ refreshed,
                                                             float* __restrict__ recall) {
    __shared__ long long part[256];
    long long s = 0;
    for (int i = threadIdx.x; i < P; i += 256) s += inter[i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const long long hit = part[0];
        const int32_t go = (double)hit < tau * (double)own ? 1 : 0;
        flag[0] = go;
        if (refreshed) refreshed[0] = go;
        if (recall) recall[0] = own > 0 ? (float)((double)hit / (double)own) : 0.f;
    }
}

}  // namespace

hipError_t launch_drift_decision(const int32_t* inter, int P, int64_t own, double tau, int32_t* flag,
                                 int32_t* refreshed, float* recall, hipStream_t st) {
    if (P <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(drift_decision_kernel, dim3(1), dim3(256), 0, st, inter, P, own, tau, flag, refreshed, recall);
    return hipGetLastError();
}
