// The first rung of the kernel ladder ("Bare Metal Bard", page 1, first
// paragraph): one thread per output element, each thread walking a row of A
// and a column of B straight from global memory.  Kept as the debug / parity
// reference family inside the library; the dispatch table never picks it for
// performance.  On a wave64 machine the 64 lanes of a wave take 64
// consecutive columns of one row, so B and C accesses are coalesced and the A
// access is a broadcast.
//
// Also here: the K == 0 case (C = 0, the empty sum), written by a plain fill
// kernel rather than a memset so that it is safe inside captured graphs.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

__device__ __forceinline__ float ld_elem(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t *p, int64_t i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float ld_elem(const F16Bits *p, int64_t i)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, p[i].v));
}

constexpr int kCols = 64;   // one wave spans 64 columns
constexpr int kRows = 4;    // four waves per block, one row each

template <typename T>
__global__ __launch_bounds__(256) void naive_kernel(int64_t M, int64_t N, int64_t K,
                                                    const T *__restrict__ A, int64_t lda,
                                                    const T *__restrict__ B, int64_t ldb,
                                                    float *__restrict__ C, int64_t ldc,
                                                    int64_t col_blocks)
{
    const int64_t blk = blockIdx.x;
    const int64_t j = (blk % col_blocks) * kCols + (threadIdx.x % kCols);
    const int64_t i = (blk / col_blocks) * kRows + (threadIdx.x / kCols);
    if (i >= M || j >= N) return;
    const T *a = A + i * lda;
    const T *b = B + j;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = fmaf(ld_elem(a, k), ld_elem(b, k * ldb), acc);
    C[i * ldc + j] = acc;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int64_t M, int64_t N, float *__restrict__ C,
                                                        int64_t ldc, int64_t col_blocks)
{
    const int64_t blk = blockIdx.x;
    const int64_t j = (blk % col_blocks) * kCols + (threadIdx.x % kCols);
    const int64_t i = (blk / col_blocks) * kRows + (threadIdx.x / kCols);
    if (i < M && j < N) C[i * ldc + j] = 0.0f;
}

template <typename T>
hipError_t launch_naive(const Problem &p, hipStream_t s)
{
    const int64_t cb = (p.N + kCols - 1) / kCols;
    const int64_t rb = (p.M + kRows - 1) / kRows;
    if (cb * rb > kMaxBlocks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(naive_kernel<T>, dim3(static_cast<uint32_t>(cb * rb)), dim3(256), 0, s,
                       p.M, p.N, p.K, static_cast<const T *>(p.A), p.lda,
                       static_cast<const T *>(p.B), p.ldb, p.C, p.ldc, cb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_naive_f32(const Problem &p, hipStream_t s) { return launch_naive<float>(p, s); }
hipError_t launch_naive_bf16(const Problem &p, hipStream_t s) { return launch_naive<uint16_t>(p, s); }
hipError_t launch_naive_f16(const Problem &p, hipStream_t s) { return launch_naive<F16Bits>(p, s); }

hipError_t launch_fill_zero(const Problem &p, hipStream_t s)
{
    const int64_t cb = (p.N + kCols - 1) / kCols;
    const int64_t rb = (p.M + kRows - 1) / kRows;
    if (cb * rb > kMaxBlocks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<uint32_t>(cb * rb)), dim3(256), 0, s,
                       p.M, p.N, p.C, p.ldc, cb);
    return hipGetLastError();
}

}  // namespace mi355gemm
