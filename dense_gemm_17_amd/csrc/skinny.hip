// Bandwidth family for products with few rows (M <= 16): C (M x N) = A B
// where B (K x N) is streamed from HBM exactly once.
//
// These shapes sit far below the ridge point (one or a few flops per byte of
// B), so their time is the time to read B.  The devpost write-up ("What we
// built") routes such bandwidth-bound shapes to their own kernel family;
// vidyal.ai Part 2 ("The CUDA Programming Model") is the first kernel that
// hits the memory-bandwidth limit, and vidyal.ai Part 8 ("Reductions") is the
// in-block sum used here to combine the K split.
//
//   * a work-group owns a strip of C's columns: 8 lanes x 16 bytes = 32 fp32
//     or 64 bf16 columns, one 128-byte line of each B row (narrower strips
//     were measured slower: neighbouring half-lines land on different XCDs);
//   * its threads form K-groups of 8 lanes; each K-group takes one contiguous
//     range of K and keeps 16 B rows of its strip in flight per thread (128-bit
//     loads), so that the chip holds the ~20 MB in flight that HBM needs at
//     full rate (bytes in flight = bandwidth x latency); strips are few when
//     N is small, so then a work-group has 512 threads instead of 256;
//   * A is tiny (M x K) and read by every work-group: it is loaded straight
//     from the caches, four k at a time per row;
//   * the partial sums of the K-groups are added in a fixed order (lane
//     shuffles inside a wave, then LDS across waves), so the result is
//     deterministic; no atomics, no workspace;
//   * ragged N and unaligned B or A fall back to element loads with masks.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kLanes = 8;                     // lanes per K-group (one 128-byte line)
constexpr int kMaxM = 16;

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerLoad = 4;        // columns per 16-byte load
    typedef f32x4 Raw;
    __device__ static float to_f(float x) { return x; }
    __device__ static float get(const Raw &r, int e) { return r[e]; }
};
template <> struct Elem<uint16_t> {
    static constexpr int kPerLoad = 8;
    typedef u16x8 Raw;
    __device__ static float to_f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
    __device__ static float get(const Raw &r, int e) { return to_f(r[e]); }
};

// B rows in flight per thread: fewer when there are more accumulators
// (output rows x columns per lane), to stay within the register file.
template <int kAcc> constexpr int unroll_for() { return kAcc <= 32 ? 16 : kAcc <= 64 ? 8 : 4; }

// The kPerLoad columns of B row k starting at column n, raw (zero where
// the row or a column is out of range).
template <typename T, bool kVec>
__device__ __forceinline__ typename Elem<T>::Raw load_b(const T *__restrict__ B, int64_t ldb,
                                                        int64_t k, int64_t n, int64_t N, bool krow)
{
    constexpr int P = Elem<T>::kPerLoad;
    typename Elem<T>::Raw v = {};
    if (!krow) return v;
    const T *p = B + k * ldb + n;
    if (kVec && n + P <= N) return *reinterpret_cast<const typename Elem<T>::Raw *>(p);
#pragma unroll
    for (int e = 0; e < P; ++e)
        if (n + e < N) v[e] = p[e];
    return v;
}

// A[m][k .. k+3] as fp32 (zero past K), vector load when aligned.
template <typename T, bool kVec>
__device__ __forceinline__ f32x4 load_a4(const T *__restrict__ A, int64_t lda, int m, int64_t k,
                                         int64_t K)
{
    const T *p = A + m * lda + k;
    if (kVec && k + 4 <= K) {
        if constexpr (Elem<T>::kPerLoad == 4) {
            return *reinterpret_cast<const f32x4 *>(p);
        } else {
            const u16x4 x = *reinterpret_cast<const u16x4 *>(p);
            return f32x4{Elem<T>::to_f(x[0]), Elem<T>::to_f(x[1]), Elem<T>::to_f(x[2]),
                         Elem<T>::to_f(x[3])};
        }
    }
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (k + e < K) ? Elem<T>::to_f(p[e]) : 0.f;
    return v;
}

template <typename T, int kM, bool kVec, int kThreads>
__global__ __launch_bounds__(kThreads) void skinny_kernel(int64_t M, int64_t N, int64_t K,
                                                          const T *__restrict__ A, int64_t lda,
                                                          const T *__restrict__ B, int64_t ldb,
                                                          float *__restrict__ C, int64_t ldc,
                                                          int64_t kg_len)
{
    constexpr int P = Elem<T>::kPerLoad;
    constexpr int kCols = kLanes * P;                       // strip width
    constexpr int kWaves = kThreads / 64;
    __shared__ float red[kWaves * kM * kCols];              // per-wave partial sums

    const int tid = threadIdx.x;
    const int lane = tid % kLanes, grp = tid / kLanes;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kCols;
    const int64_t n = n0 + lane * P;
    const int64_t kb = grp * kg_len;                        // this K-group's range
    const int64_t ke = (kb + kg_len < K) ? kb + kg_len : K;

    float acc[kM][P];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) acc[m][e] = 0.f;

    constexpr int kUnroll = unroll_for<kM * P>();
    if (n < N) {
        for (int64_t k = kb; k < ke; k += kUnroll) {
            typename Elem<T>::Raw b[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) b[u] = load_b<T, kVec>(B, ldb, k + u, n, N, k + u < ke);
#pragma unroll
            for (int u4 = 0; u4 < kUnroll; u4 += 4) {
#pragma unroll
                for (int m = 0; m < kM; ++m) {
                    // Rows past M read row 0 (in bounds); their sums are not stored.
                    const f32x4 a = load_a4<T, kVec>(A, lda, m < M ? m : 0, k + u4, ke);
#pragma unroll
                    for (int uu = 0; uu < 4; ++uu)
#pragma unroll
                        for (int e = 0; e < P; ++e)
                            acc[m][e] = fmaf(a[uu], Elem<T>::get(b[u4 + uu], e), acc[m][e]);
                }
            }
        }
    }

    // Fixed-order reduction: the eight K-groups of a wave by lane shuffles
    // (xor 8, 16, 32), then the waves through LDS.
    static_assert(kLanes == 8, "shuffle pattern assumes 8 lanes per K-group");
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) {
            float v = acc[m][e];
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[m][e] = v;
        }
    const int wave = tid / 64;
    if ((tid % 64) < kLanes) {
#pragma unroll
        for (int m = 0; m < kM; ++m)
#pragma unroll
            for (int e = 0; e < P; ++e) red[(wave * kM + m) * kCols + lane * P + e] = acc[m][e];
    }
    __syncthreads();
    for (int o = tid; o < kM * kCols; o += kThreads) {
        const int m = o / kCols, col = o % kCols;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) sum += red[(w * kM + m) * kCols + col];
        if (m < M && n0 + col < N) C[m * ldc + n0 + col] = sum;
    }
}

template <typename T, int kM, int kThreads>
hipError_t launch_m(const Problem &p, hipStream_t s, bool vec)
{
    constexpr int kCols = kLanes * Elem<T>::kPerLoad;
    constexpr int kGroups = kThreads / kLanes;
    const int64_t blocks = (p.N + kCols - 1) / kCols;
    if (blocks > kMaxBlocks) return hipErrorInvalidValue;
    // K range per group: a multiple of 4 (aligned A quads), at least one row.
    int64_t kg = (p.K + kGroups - 1) / kGroups;
    kg = (kg + 3) & ~int64_t(3);
    const T *A = static_cast<const T *>(p.A);
    const T *B = static_cast<const T *>(p.B);
    if (vec)
        hipLaunchKernelGGL((skinny_kernel<T, kM, true, kThreads>),
                           dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p.M, p.N,
                           p.K, A, p.lda, B, p.ldb, p.C, p.ldc, kg);
    else
        hipLaunchKernelGGL((skinny_kernel<T, kM, false, kThreads>),
                           dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p.M, p.N,
                           p.K, A, p.lda, B, p.ldb, p.C, p.ldc, kg);
    return hipGetLastError();
}

template <typename T, int kM>
hipError_t launch_threads(const Problem &p, hipStream_t s, bool vec)
{
    constexpr int kCols = kLanes * Elem<T>::kPerLoad;
    // Fewer strips than CUs: bigger work-groups keep enough bytes in flight
    // (not with the largest accumulator sets, which need the registers of
    // a 256-thread work-group).
    if constexpr (kM * Elem<T>::kPerLoad <= 64) {
        if ((p.N + kCols - 1) / kCols < 256) return launch_m<T, kM, 512>(p, s, vec);
    }
    return launch_m<T, kM, 256>(p, s, vec);
}

// Row counts are rounded up to one of a few compiled sizes.
template <typename T>
hipError_t launch_skinny(const Problem &p, hipStream_t s)
{
    if (p.M < 1 || p.M > kMaxM) return hipErrorInvalidValue;
    const bool vec = (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 &&
                     p.ldb % Elem<T>::kPerLoad == 0 &&
                     (reinterpret_cast<uintptr_t>(p.A) & (4 * sizeof(T) - 1)) == 0 && p.lda % 4 == 0;
    if (p.M <= 1) return launch_threads<T, 1>(p, s, vec);
    if (p.M <= 2) return launch_threads<T, 2>(p, s, vec);
    if (p.M <= 4) return launch_threads<T, 4>(p, s, vec);
    if (p.M <= 8) return launch_threads<T, 8>(p, s, vec);
    return launch_threads<T, 16>(p, s, vec);
}

}  // namespace

static_assert(kMaxM == kSkinnyMaxM, "skinny row limit");

hipError_t launch_skinny_f32(const Problem &p, hipStream_t s) { return launch_skinny<float>(p, s); }
hipError_t launch_skinny_bf16(const Problem &p, hipStream_t s) { return launch_skinny<uint16_t>(p, s); }

}  // namespace mi355gemm
