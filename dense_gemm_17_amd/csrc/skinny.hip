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
//   * a work-group owns a strip of C's columns; its threads form K-groups of
//     kL lanes, each lane loading 16 bytes of a B row, so a K-group reads kL
//     x 16 contiguous bytes of every row it visits (256 or 128 bytes,
//     whichever puts fewer bytes of a row through the busiest CU; 64 bytes
//     only for very narrow B);
//   * K is dealt to the K-groups in blocks of four rows, round robin (group g
//     takes blocks g, g + G, g + 2G, ...): at any moment the groups of all
//     work-groups read one contiguous band of B rows, which measured 1.3-1.4x
//     faster than giving each group one long contiguous range of rows, and
//     four consecutive k let A be read as one 16-byte load per row of A;
//   * several blocks per thread are loaded before any is used (the bytes in
//     flight that hide HBM latency); the work-group size and that depth
//     follow from the accumulator count (output rows x columns per lane);
//   * A is tiny (M x K) and read by every work-group from the caches, but
//     from the caches a lane loads 16 bytes of every row of A per four rows
//     of B; where that is the larger share of the load instructions (the
//     row-split pairs and work-groups of 9-16 rows) and A's rows fit in 64
//     KiB, the work-group first copies them into LDS (7 x 4096 x 4096:
//     21.4 -> 20.2 us; 12 x 8960 x 1536: 32.1 -> 27.8);
//   * when strips are fewer than CUs and there are more than 4 rows, each
//     strip is split by rows between two work-groups whose ids land on the
//     same XCD back to back, so all CUs stream B and the second read of each
//     B line hits that XCD's L2 (1.26x at 7 x 4096 x 4096);
//   * the partial sums of the K-groups are added in a fixed order (lane
//     shuffles inside a wave, then LDS across waves), so the result is
//     deterministic; no atomics, no workspace;
//   * ragged N and unaligned B or A fall back to element loads with masks.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxM = 16;

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerLoad = 4;        // columns per 16-byte load
    typedef f32x4 Raw;
    __device__ static float to_f(float x) { return x; }
    __device__ static float raw(float x) { return x; }
    __device__ static float get(const Raw &r, int e) { return r[e]; }
};
template <> struct Elem<uint16_t> {            // bf16 patterns
    static constexpr int kPerLoad = 8;
    typedef u16x8 Raw;
    __device__ static float to_f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
    __device__ static uint16_t raw(uint16_t x) { return x; }
    __device__ static float get(const Raw &r, int e) { return to_f(r[e]); }
};
template <> struct Elem<F16Bits> {             // IEEE binary16 patterns
    static constexpr int kPerLoad = 8;
    typedef u16x8 Raw;
    __device__ static float to_f(uint16_t x) { return static_cast<float>(__builtin_bit_cast(_Float16, x)); }
    __device__ static float to_f(F16Bits x) { return to_f(x.v); }
    __device__ static uint16_t raw(F16Bits x) { return x.v; }
    __device__ static float get(const Raw &r, int e) { return to_f(r[e]); }
};

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
        if (n + e < N) v[e] = Elem<T>::raw(p[e]);
    return v;
}

// A[m][k .. k+3] as fp32 (zero past K), one vector load when aligned.
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

// A[m][k .. k+3] as fp32 from the LDS copy of A's rows (row stride K
// elements; k a multiple of 4 and k + 4 <= K).
template <typename T>
__device__ __forceinline__ f32x4 lds_a4(const uint8_t *a_lds, int64_t K, int m, int64_t k)
{
    const int64_t at = (m * K + k) * static_cast<int64_t>(sizeof(T));
    if constexpr (Elem<T>::kPerLoad == 4) {
        return *reinterpret_cast<const f32x4 *>(a_lds + at);
    } else {
        const u16x4 x = *reinterpret_cast<const u16x4 *>(a_lds + at);
        return f32x4{Elem<T>::to_f(x[0]), Elem<T>::to_f(x[1]), Elem<T>::to_f(x[2]),
                     Elem<T>::to_f(x[3])};
    }
}

// Bytes of LDS that hold A's rows (the kLdsA kernels).
constexpr int kLdsABytes = 64 * 1024;

// Work-group -> columns and rows of C:
//   kStrips:   work-group s owns columns s kCols .. s kCols + kCols - 1;
//   kRowSplit: rows split between two work-groups (ids 16 q + 8 h + x hold
//              strip 8 q + x, rows kM h .. kM h + kM - 1; ids differing by
//              8 share an XCD);
//   kBalanced: exactly one work-group per CU, the columns dealt out evenly
//              in kPerLoad-column units (at most kL of them each), so every
//              CU streams about the same share of B; consecutive shares go
//              to one XCD, so a cache line split between two shares is read
//              from HBM once and hit in that XCD's L2 the second time.
constexpr int kStrips = 1, kRowSplit = 2, kBalanced = 3;

// First (next = 0) or one-past-last (next = 1) column of this work-group's
// share under kBalanced: shares are consecutive on one XCD (work-group ids
// x, x + 8, x + 16, .. run on XCD x).
template <int P>
__device__ __forceinline__ int64_t balanced_edge(int64_t N, int next)
{
    const int64_t W = gridDim.x, units = (N + P - 1) / P;
    const int64_t share = (blockIdx.x % kNumXcd) * (W / kNumXcd) + blockIdx.x / kNumXcd + next;
    const int64_t edge = P * (share * units / W);
    return edge < N ? edge : N;
}

// kL lanes per K-group, kU rows (kU / 4 blocks) in flight per thread;
// kLdsA: A's rows copied into LDS first (16-byte aligned rows, K a multiple
// of 16 bytes, at most kLdsABytes).
template <typename T, int kM, int kL, int kThreads, int kU, bool kVec, int kMode, bool kLdsA>
__global__ __launch_bounds__(kThreads) void skinny_kernel(int64_t M, int64_t N, int64_t K,
                                                          const T *__restrict__ A, int64_t lda,
                                                          const T *__restrict__ B, int64_t ldb,
                                                          float *__restrict__ C, int64_t ldc)
{
    constexpr int P = Elem<T>::kPerLoad;
    constexpr int kCols = kL * P;                           // strip width
    constexpr int kGroups = kThreads / kL;
    constexpr int kWaves = kThreads / 64;
    constexpr int kBlocks = kU / 4;
    static_assert(kU % 4 == 0 && kL <= 64 && 64 % kL == 0, "shape of the K split");
    __shared__ float red[kWaves * kM * kCols];              // per-wave partial sums
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[kLdsA ? kLdsABytes : 16];

    const int tid = threadIdx.x;
    const int lane = tid % kL, grp = tid / kL;
    int64_t strip = blockIdx.x;
    if constexpr (kMode == kRowSplit) {
        const int64_t id = blockIdx.x;
        const int64_t half = (id >> 3) & 1;
        strip = (id >> 4) * 8 + (id & 7);
        A += half * kM * lda;
        C += half * kM * ldc;
        M -= half * kM;
        if (M <= 0 || strip * kCols >= N) return;   // whole work-group
    }
    // This work-group's columns [n0, n1).
    const int64_t n0 = kMode == kBalanced ? balanced_edge<P>(N, 0) : strip * kCols;
    const int64_t n1 = kMode == kBalanced ? balanced_edge<P>(N, 1) : N;
    const int64_t n = n0 + lane * P;

    if constexpr (kLdsA) {
        // this work-group's rows of A (at most kM), 16 bytes per copy
        const int rows = M < kM ? static_cast<int>(M) : kM;
        const int chunks = static_cast<int>(K * static_cast<int64_t>(sizeof(T)) / 16);
        for (int i = tid; i < rows * chunks; i += kThreads) {
            const int m = i / chunks, c = i - m * chunks;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                reinterpret_cast<const uint8_t *>(A + m * lda) + c * 16);
            *reinterpret_cast<f32x4 *>(a_lds + (static_cast<int64_t>(m) * chunks + c) * 16) = v;
        }
        __syncthreads();
    }

    float acc[kM][P];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) acc[m][e] = 0.f;

    if (n < n1) {
        const int64_t nblk = (K + 3) / 4;
        for (int64_t b0 = grp; b0 < nblk; b0 += int64_t(kGroups) * kBlocks) {
            typename Elem<T>::Raw b[kU];
#pragma unroll
            for (int v = 0; v < kBlocks; ++v)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t k = 4 * (b0 + int64_t(kGroups) * v) + r;
                    b[4 * v + r] = load_b<T, kVec>(B, ldb, k, n, n1, k < K);
                }
#pragma unroll
            for (int v = 0; v < kBlocks; ++v) {
                const int64_t k4 = 4 * (b0 + int64_t(kGroups) * v);
                if (k4 >= K) continue;
#pragma unroll
                for (int m = 0; m < kM; ++m) {
                    // Rows past M read row 0 (in bounds); their sums are not stored.
                    const f32x4 a = kLdsA ? lds_a4<T>(a_lds, K, m < M ? m : 0, k4)
                                          : load_a4<T, kVec>(A, lda, m < M ? m : 0, k4, K);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int e = 0; e < P; ++e)
                            acc[m][e] = fmaf(a[r], Elem<T>::get(b[4 * v + r], e), acc[m][e]);
                }
            }
        }
    }

    // Fixed-order reduction: the K-groups of a wave by lane shuffles over
    // the lane bits above kL, then the waves through LDS.
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) {
            float v = acc[m][e];
#pragma unroll
            for (int off = kL; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            acc[m][e] = v;
        }
    const int wave = tid / 64;
    if ((tid % 64) < kL) {
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
        if (m < M && n0 + col < n1) C[m * ldc + n0 + col] = sum;
    }
}

template <typename T, int kM, int kL, int kThreads, int kU, int kMode>
hipError_t launch_cfg(const Problem &p, hipStream_t s, bool vec)
{
    constexpr int kCols = kL * Elem<T>::kPerLoad;
    const int64_t strips = (p.N + kCols - 1) / kCols;
    const int64_t blocks = kMode == kRowSplit ? 16 * ((strips + 7) / 8)
                           : kMode == kBalanced ? kCUs : strips;
    if (blocks > kMaxBlocks) return hipErrorInvalidValue;
    const T *A = static_cast<const T *>(p.A);
    const T *B = static_cast<const T *>(p.B);
    const dim3 grid(static_cast<uint32_t>(blocks));
    if constexpr (kMode == kRowSplit || kM == 16) {
        // A's rows whole in LDS: 16-byte rows and copies, within kLdsABytes
        const int64_t es = sizeof(T);
        if (vec && (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 && (p.lda * es) % 16 == 0 &&
            (p.K * es) % 16 == 0 && kM * p.K * es <= kLdsABytes) {
            hipLaunchKernelGGL((skinny_kernel<T, kM, kL, kThreads, kU, true, kMode, true>), grid,
                               dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc);
            return hipGetLastError();
        }
    }
    if (vec)
        hipLaunchKernelGGL((skinny_kernel<T, kM, kL, kThreads, kU, true, kMode, false>), grid,
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc);
    else
        hipLaunchKernelGGL((skinny_kernel<T, kM, kL, kThreads, kU, false, kMode, false>), grid,
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc);
    return hipGetLastError();
}

// Work-group size and rows in flight per thread by accumulator count
// (measured: 512 x 8 rows for M = 1, 1024 x 4 rows for M = 7 fp32).  Larger
// sets take smaller work-groups so that each thread has the registers
// without spilling (1024 threads allow 128 VGPRs, 512 allow 256).
// (kM is the rows per work-group; measured for split work-groups of 4
// fp32 rows: 1024 x 4 beats 512 x 8.)
template <typename T, int kM, int kL, int kMode>
hipError_t launch_lanes(const Problem &p, hipStream_t s, bool vec)
{
    constexpr int kAcc = kM * Elem<T>::kPerLoad;
    if constexpr (kAcc <= 16 && kMode == kStrips) return launch_cfg<T, kM, kL, 512, 8, kMode>(p, s, vec);
    else if constexpr (kAcc <= 32) return launch_cfg<T, kM, kL, 1024, 4, kMode>(p, s, vec);
    else if constexpr (kAcc <= 64) return launch_cfg<T, kM, kL, 512, 4, kMode>(p, s, vec);
    else return launch_cfg<T, kM, kL, 256, 4, kMode>(p, s, vec);
}

// Strip width in lanes: 16 (256 bytes of a B row) when those strips occupy
// more than half the CUs, else 8 (128 bytes), else 4 (64 bytes) when even
// 8-lane strips number fewer than 128.  Wider strips read longer runs of
// each row; narrower ones put more CUs to work.  Measured: 1 x 8960 x 1536
// 15.2 us with 140 strips of 256 bytes (17.8 with 280 of 128); 4 x 8192 x
// 2048 18.1 us with 256 strips of 128 bytes (22.1 with 128 of 256);
// 1 x 19200 x 1536 28.7 us with 300 of 256 (29.5 with 600 of 128); 1 x 4096
// x 4096 22.4 us with 128 of 128 (25.3 with 256 of 64).
template <typename T>
int lanes_of(const Problem &p)
{
    constexpr int P = Elem<T>::kPerLoad;
    if ((p.N + 16 * P - 1) / (16 * P) > kCUs / 2) return 16;
    if ((p.N + 8 * P - 1) / (8 * P) >= 128) return 8;
    return 4;
}

template <typename T, int kM, int kMode>
hipError_t launch_m(const Problem &p, hipStream_t s, bool vec)
{
    const int lanes = lanes_of<T>(p);
    if (lanes == 16) return launch_lanes<T, kM, 16, kMode>(p, s, vec);
    if (lanes == 8) return launch_lanes<T, kM, 8, kMode>(p, s, vec);
    return launch_lanes<T, kM, 4, kMode>(p, s, vec);
}

// Strips of the width launch_m picks (one per work-group without a split).
template <typename T>
int64_t strips_of(const Problem &p)
{
    const int64_t cols = static_cast<int64_t>(lanes_of<T>(p)) * Elem<T>::kPerLoad;
    return (p.N + cols - 1) / cols;
}

// Row counts are rounded up to one of a few compiled sizes.  With fewer
// strips than CUs, up to 4 rows take the balanced split (one work-group per
// CU, 1024 threads with 4 rows in flight each: 1 x 8960 x 1536 in 13.8
// instead of 15.1 us, 1 x 4096 x 4096 in 20.4 instead of 22.4, 3 x 12288 x
// 1024 in 13.0 instead of 14.4, with 140, 128 and 192 strips), and more
// rows are split between two work-groups (for 7 and 8 rows that beats the
// balanced split, 22.5 vs 36.9 us at 7 x 4096 x 4096: it reads each B line
// twice, once per half, but keeps half the accumulators per thread).  The
// balanced split is used for fp32 with at most 3/4 as many strips as CUs
// (with 224 strips of 2 x 14336 x 4096 the strips already stream at 5.1
// TB/s and the balanced split is slower, 51.0 vs 46.5 us) and where 8-lane
// strips number at least 128 (where it was measured).  For bf16 a share
// holds half as many bytes per lane and it measured slower on every shape
// but one (1 x 8960 x 1536: 10.9 vs 10.3 us; 4 x 8192 x 2048: 24.1 vs 19.0).
template <typename T>
hipError_t launch_skinny(const Problem &p, hipStream_t s)
{
    constexpr int P = Elem<T>::kPerLoad;
    if (p.M < 1 || p.M > kMaxM) return hipErrorInvalidValue;
    const bool vec = (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && p.ldb % P == 0 &&
                     (reinterpret_cast<uintptr_t>(p.A) & (4 * sizeof(T) - 1)) == 0 && p.lda % 4 == 0;
    const int64_t strips = strips_of<T>(p);
    const bool few = strips < kCUs;
    if (P == 4 && p.M <= 4 && 4 * strips <= 3 * kCUs && (p.N + 8 * P - 1) / (8 * P) >= 128) {
        if (p.M <= 1) return launch_cfg<T, 1, 16, 1024, 4, kBalanced>(p, s, vec);
        if (p.M <= 2) return launch_cfg<T, 2, 16, 1024, 4, kBalanced>(p, s, vec);
        return launch_cfg<T, 4, 16, 1024, 4, kBalanced>(p, s, vec);
    }
    if (p.M <= 1) return launch_m<T, 1, kStrips>(p, s, vec);
    if (p.M <= 2) return launch_m<T, 2, kStrips>(p, s, vec);
    if (p.M <= 4) return launch_m<T, 4, kStrips>(p, s, vec);
    if (p.M <= 8) return few ? launch_m<T, 4, kRowSplit>(p, s, vec) : launch_m<T, 8, kStrips>(p, s, vec);
    return few ? launch_m<T, 8, kRowSplit>(p, s, vec) : launch_m<T, 16, kStrips>(p, s, vec);
}

}  // namespace

static_assert(kMaxM == kSkinnyMaxM, "skinny row limit");

hipError_t launch_skinny_f32(const Problem &p, hipStream_t s) { return launch_skinny<float>(p, s); }
hipError_t launch_skinny_bf16(const Problem &p, hipStream_t s) { return launch_skinny<uint16_t>(p, s); }
hipError_t launch_skinny_f16(const Problem &p, hipStream_t s) { return launch_skinny<F16Bits>(p, s); }

}  // namespace mi355gemm
