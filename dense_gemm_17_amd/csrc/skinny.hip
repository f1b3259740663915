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
//   * fp32 with 96-255 strips of 128 bytes (48-95 from K = 8192) and a long
//     K splits each strip's
//     K range between two work-groups (skinny_ksplit_kernel below), so every
//     CU streams distinct bytes of B; the two halves add into C filled with
//     -0.0 (two addends: the same bits whichever lands first);
//   * otherwise, when strips are fewer than CUs and there are more than 4
//     rows, each strip is split by rows between two work-groups whose ids
//     land on the same XCD back to back, so all CUs stream B and the second
//     read of each B line hits that XCD's L2 (1.26x at 7 x 4096 x 4096);
//   * the partial sums of the K-groups are added in a fixed order (lane
//     shuffles inside a wave, then LDS across waves), so the result is
//     deterministic; no workspace;
//   * ragged N and unaligned B or A fall back to element loads with masks.
#include <type_traits>

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

// ---------------------------------------------------------------------------
// K split over two work-groups (fp32, 1-16 rows, 96-255 strips of 128 bytes).
//
// With fewer strips than CUs, one work-group per strip leaves CUs idle, and
// one CU pulls only about 25-30 GB/s from HBM however many loads it keeps in
// flight, so the strips' CUs cannot reach the chip's bandwidth.  Here each
// strip's K range is split in two halves, each streamed by its own
// work-group (ids 16 q + x and 16 q + 8 + x: the same XCD), so every CU
// streams distinct bytes of B.  The two partial strips are added into C,
// which is first filled with -0.0: with exactly two addends the sum does
// not depend on which arrives first (-0.0 + x = x, and x + y = y + x), so
// the result is bitwise repeatable.
//
//   * a lane loads 16 bytes (4 columns) of 4 consecutive rows per step and,
//     in the same step, the 16 bytes of A it needs for those rows; the next
//     step's loads are issued before the current step's arithmetic, so every
//     wave keeps a step of B in flight while it computes;
//   * with 4 or more rows the arithmetic runs on the matrix cores:
//     v_mfma_f32_4x4x1_16b_f32 forms sixteen independent 4 x 4 outer
//     products per wave; lane l supplies the A value of row l % 4 and the B
//     value of column l % 4 of block l / 4, and receives that column's four
//     rows.  The four lanes of a block are half a K-group (same B row), so
//     each lane's four columns (one per element of its 16-byte load) give
//     four products, one per column offset, for each group of four rows;
//   * one row uses plain FMAs (four per loaded element pair);
//   * the wave and work-group sums use the fixed-order reduction of the
//     kernels above.
template <int kM, int kThreads, bool kAVec>
__global__ __launch_bounds__(kThreads) void skinny_ksplit_kernel(int64_t M, int64_t N, int64_t K,
                                                                 int64_t khalf,
                                                                 const float *__restrict__ A, int64_t lda,
                                                                 const float *__restrict__ B, int64_t ldb,
                                                                 float *__restrict__ C, int64_t ldc)
{
    constexpr int kL = 8, P = 4, kCols = kL * P, kGroups = kThreads / kL, kWaves = kThreads / 64;
    constexpr bool kMfma = kM >= 4;
    constexpr int kH = kMfma ? kM / 4 : 1;      // groups of four rows (A loads per step)
    constexpr int kStep = 4 + kH;                // 16-byte loads per step: 4 of B, kH of A
    static_assert(kM == 1 || kM == 4 || kM == 8 || kM == 16, "compiled row counts");
    __shared__ float red[kWaves * kM * kCols];

    const int tid = threadIdx.x, lane = tid % kL, grp = tid / kL;
    const int64_t id = blockIdx.x;
    const int64_t part = (id >> 3) & 1;
    const int64_t n0 = ((id >> 4) * 8 + (id & 7)) * kCols;
    if (n0 >= N) return;                          // whole work-group
    const int64_t k0 = part * khalf, k1 = part ? K : khalf;
    const int64_t n = n0 + lane * P;
    const int64_t nl = n < N ? n : N - P;         // past N: a valid column, sums dropped

    // This lane's rows of A (rows past M read row 0; their sums are dropped).
    int64_t arow[kH];
#pragma unroll
    for (int h = 0; h < kH; ++h) {
        const int r = kMfma ? 4 * h + (tid & 3) : 0;
        arow[h] = (r < M ? r : 0) * lda;
    }
    // Byte offsets of this lane's B loads from the step's first row (32-bit:
    // the launcher keeps 4 kGroups rows of B within 2^31 bytes).
    uint32_t boff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) boff[r] = static_cast<uint32_t>(((4 * grp + r) * ldb + nl) * 4);

    // Step j covers rows k0 + 4 (j kGroups + grp) .. + 3 of this lane.
    auto load = [&](f32x4 *x, int64_t row0) {
        const char *bb = reinterpret_cast<const char *>(B + row0 * ldb);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = *reinterpret_cast<const f32x4 *>(bb + boff[r]);
        const float *aa = A + row0 + 4 * grp;
#pragma unroll
        for (int h = 0; h < kH; ++h) {
            if constexpr (kAVec) {
                x[4 + h] = *reinterpret_cast<const f32x4 *>(aa + arow[h]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[4 + h][r] = aa[arow[h] + r];
            }
        }
    };

    f32x4 macc[P][kH];
    float facc[P];
#pragma unroll
    for (int e = 0; e < P; ++e) {
        facc[e] = 0.f;
#pragma unroll
        for (int h = 0; h < kH; ++h) macc[e][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto compute = [&](const f32x4 *x) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < P; ++e) {
                if constexpr (kMfma) {
#pragma unroll
                    for (int h = 0; h < kH; ++h)
                        macc[e][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(x[4 + h][r], x[r][e], macc[e][h], 0, 0, 0);
                } else {
                    facc[e] = fmaf(x[4][r], x[r][e], facc[e]);
                }
            }
    };

    // Whole steps (every lane's four rows inside [k0, k1)), two register
    // sets in turn so that no copy waits on a load in flight.
    constexpr int64_t kRows = 4 * int64_t(kGroups);
    const int64_t full = (k1 - k0) / kRows;
    int64_t row0 = k0;
    f32x4 xa[kStep], xb[kStep];
    if (full > 0) {
        load(xa, row0);
        int64_t j = 1;
        for (; j + 1 < full; j += 2) {
            load(xb, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xa);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
            load(xa, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xb);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
        }
        if (j < full) {
            load(xb, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xa);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
            compute(xb);
        } else {
            compute(xa);
        }
        row0 += kRows;
    }
    // The rest of the half: this lane's rows past k1 (and the A values of
    // columns of A past k1) are zero.  Every lane takes part (the matrix
    // instruction works on the whole wave).
    for (; row0 < k1; row0 += kRows) {
        const int64_t k4 = row0 + 4 * grp;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            xa[r] = k4 + r < k1 ? *reinterpret_cast<const f32x4 *>(B + (k4 + r) * ldb + nl)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < kH; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) xa[4 + h][r] = k4 + r < k1 ? A[arow[h] + k4 + r] : 0.f;
        compute(xa);
    }

    // This lane's sums: rows m, columns n + e.
    float acc[kM][P];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) acc[m][e] = kMfma ? macc[e][m / 4][m % 4] : facc[e];
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
        if (m < M && n0 + col < N) unsafeAtomicAdd(C + m * ldc + n0 + col, sum);
    }
}

constexpr int kSplitThreads = 512;
constexpr int kSplitThreads16 = 512;

// Whether the K split takes this fp32 product: aligned 16-byte loads of B
// (A's rows may be unaligned: then read one element at a time), N a
// multiple of 4, at most 16 rows, 96-255 strips of 128 bytes (192-510
// work-groups; with as many strips as CUs one work-group per strip wins:
// 7 x 8192 x 4096 29.6 vs 32.0 us) or 48-95 from K = 8192 (half the CUs or
// more: 4 x 2560 x 16384 78.1 -> 47.5 us, 12 x 3000 x 8192 59.7 -> 32.5; at
// 7 x 2048 x 4096 no gain) and K long enough to amortise the fill
// (measured against the row split: 8 x 3072 x 1500 10.7 vs 17.4 us, 7 x
// 4096 x 4096 18.1 vs 20.1, 16 x 4096 x 4096 20.4 vs 24.9, 7 x 6144 x 4096
// 29.5 vs 38.2, 7 x 5120 x 8192 52.0 vs 74.7, but 12 x 4096 x 1536 13.1
// vs 12.7, so 9-16 rows need K >= 2048).
bool ksplit_fits(const Problem &p)
{
    const int64_t strips = (p.N + 31) / 32;
    const bool vec_b = (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && p.ldb % 4 == 0;
    return vec_b && p.N % 4 == 0 && p.M <= kMaxM && p.K >= (p.M <= 8 ? 1024 : 2048) &&
           (8 * strips >= 3 * kCUs || (16 * strips >= 3 * kCUs && p.K >= 8192)) && strips < kCUs &&
           p.ldb <= (int64_t(1) << 31) / (4 * 4 * (kSplitThreads / 8));
}

template <int kM>
hipError_t launch_ksplit_m(const Problem &p, hipStream_t s, dim3 grid, dim3 block, int64_t khalf, bool vec_a)
{
    const float *A = static_cast<const float *>(p.A), *B = static_cast<const float *>(p.B);
    if (vec_a)
        hipLaunchKernelGGL((skinny_ksplit_kernel<kM, kSplitThreads, true>), grid, block, 0, s, p.M, p.N, p.K,
                           khalf, A, p.lda, B, p.ldb, p.C, p.ldc);
    else
        hipLaunchKernelGGL((skinny_ksplit_kernel<kM, kSplitThreads, false>), grid, block, 0, s, p.M, p.N, p.K,
                           khalf, A, p.lda, B, p.ldb, p.C, p.ldc);
    return hipGetLastError();
}

hipError_t launch_ksplit(const Problem &p, hipStream_t s)
{
    const int64_t strips = (p.N + 31) / 32;
    const int64_t khalf = ((p.K + 1) / 2 + 3) / 4 * 4;     // a multiple of 4 below K
    const hipError_t e = launch_fill(p, -0.0f, s);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<uint32_t>(16 * ((strips + 7) / 8))), block(kSplitThreads);
    const bool vec_a = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 && p.lda % 4 == 0;
    if (p.M <= 1) return launch_ksplit_m<1>(p, s, grid, block, khalf, vec_a);
    if (p.M <= 4) return launch_ksplit_m<4>(p, s, grid, block, khalf, vec_a);
    if (p.M <= 8) return launch_ksplit_m<8>(p, s, grid, block, khalf, vec_a);
    return launch_ksplit_m<16>(p, s, grid, block, khalf, vec_a);
}

// The same K split for 16-bit operands (bf16 or fp16 bits), products on
// v_mfma_f32_4x4x4_16b_bf16 / _f16: sixteen independent 4 x 4 blocks, each
// summing over 4 k, lane l supplying row l % 4 of A and column l % 4 of B
// of block l / 4 (4 consecutive k each) and receiving that column's four
// rows.  A lane's four B rows give one 16-byte load per row (8 columns);
// column e's four values are gathered into the lane's B operand, so a step
// is one instruction per column and group of four rows.  kL = 8 lanes per
// K-group: strips of 128 bytes.
template <typename T, int kM, int kL, bool kAVec>
__global__ __launch_bounds__(kSplitThreads16) void skinny_ksplit16_kernel(
    int64_t M, int64_t N, int64_t K, int64_t khalf, const T *__restrict__ A, int64_t lda,
    const T *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
    constexpr int kThreads = kSplitThreads16;
    constexpr int P = 8, kCols = kL * P, kGroups = kThreads / kL, kWaves = kThreads / 64;
    constexpr int kH = kM / 4;
    constexpr bool kF16 = !std::is_same<T, uint16_t>::value;
    static_assert(kM == 4 || kM == 8, "compiled row counts");
    __shared__ float red[kWaves * kM * kCols];

    const int tid = threadIdx.x, lane = tid % kL, grp = tid / kL;
    const int64_t id = blockIdx.x;
    const int64_t part = (id >> 3) & 1;
    const int64_t n0 = ((id >> 4) * 8 + (id & 7)) * kCols;
    if (n0 >= N) return;                          // whole work-group
    const int64_t k0 = part * khalf, k1 = part ? K : khalf;
    const int64_t n = n0 + lane * P;
    const int64_t nl = n < N ? n : N - P;         // past N: a valid column, sums dropped
    const uint16_t *A16 = reinterpret_cast<const uint16_t *>(A);
    const uint16_t *B16 = reinterpret_cast<const uint16_t *>(B);

    int64_t arow[kH];
#pragma unroll
    for (int h = 0; h < kH; ++h) {
        const int r = 4 * h + (tid & 3);
        arow[h] = (r < M ? r : 0) * lda;
    }
    uint32_t boff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) boff[r] = static_cast<uint32_t>(((4 * grp + r) * ldb + nl) * 2);

    struct Step {
        u16x8 b[4];
        u16x4 a[kH];
    };
    auto load = [&](Step &x, int64_t row0) {
        const char *bb = reinterpret_cast<const char *>(B16 + row0 * ldb);
#pragma unroll
        for (int r = 0; r < 4; ++r) x.b[r] = *reinterpret_cast<const u16x8 *>(bb + boff[r]);
        const uint16_t *aa = A16 + row0 + 4 * grp;
#pragma unroll
        for (int h = 0; h < kH; ++h) {
            if constexpr (kAVec) {
                x.a[h] = *reinterpret_cast<const u16x4 *>(aa + arow[h]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) x.a[h][r] = aa[arow[h] + r];
            }
        }
    };
    f32x4 macc[P][kH];
#pragma unroll
    for (int e = 0; e < P; ++e)
#pragma unroll
        for (int h = 0; h < kH; ++h) macc[e][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Step &x) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const u16x4 bcol = {x.b[0][e], x.b[1][e], x.b[2][e], x.b[3][e]};
#pragma unroll
            for (int h = 0; h < kH; ++h) {
                if constexpr (kF16)
                    macc[e][h] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h16x4, x.a[h]),
                                                                    __builtin_bit_cast(h16x4, bcol),
                                                                    macc[e][h], 0, 0, 0);
                else
                    macc[e][h] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, x.a[h]),
                                                                       __builtin_bit_cast(s16x4, bcol),
                                                                       macc[e][h], 0, 0, 0);
            }
        }
    };

    constexpr int64_t kRows = 4 * int64_t(kGroups);
    const int64_t full = (k1 - k0) / kRows;
    int64_t row0 = k0;
    Step xa, xb;
    if (full > 0) {
        load(xa, row0);
        int64_t j = 1;
        for (; j + 1 < full; j += 2) {
            load(xb, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xa);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
            load(xa, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xb);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
        }
        if (j < full) {
            load(xb, row0 + kRows);
            __builtin_amdgcn_sched_barrier(0);
            compute(xa);
            __builtin_amdgcn_sched_barrier(0);
            row0 += kRows;
            compute(xb);
        } else {
            compute(xa);
        }
        row0 += kRows;
    }
    // the rest of the half: rows past k1 and A's columns past k1 are zero;
    // every lane takes part (the matrix instruction works on the whole wave)
    for (; row0 < k1; row0 += kRows) {
        const int64_t k4 = row0 + 4 * grp;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            xa.b[r] = k4 + r < k1 ? *reinterpret_cast<const u16x8 *>(B16 + (k4 + r) * ldb + nl)
                                  : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < kH; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) xa.a[h][r] = k4 + r < k1 ? A16[arow[h] + k4 + r] : uint16_t(0);
        compute(xa);
    }

    // this lane's sums: rows m, columns n + e; then the K-groups of a wave
    // by lane shuffles, the waves through LDS, in a fixed order
    float acc[kM][P];
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < P; ++e) {
            float v = macc[e][m / 4][m % 4];
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
        if (m < M && n0 + col < N) unsafeAtomicAdd(C + m * ldc + n0 + col, sum);
    }
}

// 16-bit K split: strips of 128 bytes (64 columns), at most 8 rows (16
// rows' 32 accumulator blocks spill at two waves per SIMD), the 32-bit B
// offsets as for fp32.  96-128 strips (192-256 work-groups) from K = 1024
// (4 x 8192 x 8192: 52.8 -> 37.1 us); 48-95 strips (half the CUs or more)
// only from K = 8192, where each work-group's half is long enough (8 x 4096
// x 14336: 68.0 -> 48.7 us; at K = 4096 the row split stays ahead, 1 x 4096
// x 4096 19.7 vs 20.9).  64-byte strips (two work-groups sharing each line)
// measured slower in both cases (25.3 and 50.5 us).
bool ksplit16_fits(const Problem &p)
{
    const int64_t strips = (p.N + 63) / 64;
    const bool vec_b = (reinterpret_cast<uintptr_t>(p.B) & 15) == 0 && p.ldb % 8 == 0;
    const bool many = 8 * strips >= 3 * kCUs, half = 16 * strips >= 3 * kCUs && p.K >= 8192;
    return vec_b && p.N % 8 == 0 && p.M <= 8 && p.K >= 1024 && (many || half) && 2 * strips <= kCUs &&
           p.ldb <= (int64_t(1) << 31) / (2 * 4 * (kSplitThreads16 / 8));
}

template <typename T, int kM, int kL>
hipError_t launch_ksplit16_m(const Problem &p, hipStream_t s, dim3 grid, int64_t khalf, bool vec_a)
{
    const T *A = static_cast<const T *>(p.A), *B = static_cast<const T *>(p.B);
    if (vec_a)
        hipLaunchKernelGGL((skinny_ksplit16_kernel<T, kM, kL, true>), grid, dim3(kSplitThreads16), 0, s, p.M,
                           p.N, p.K, khalf, A, p.lda, B, p.ldb, p.C, p.ldc);
    else
        hipLaunchKernelGGL((skinny_ksplit16_kernel<T, kM, kL, false>), grid, dim3(kSplitThreads16), 0, s, p.M,
                           p.N, p.K, khalf, A, p.lda, B, p.ldb, p.C, p.ldc);
    return hipGetLastError();
}

template <typename T, int kL>
hipError_t launch_ksplit16(const Problem &p, hipStream_t s)
{
    const int64_t strips = (p.N + kL * 8 - 1) / (kL * 8);
    const int64_t khalf = ((p.K + 1) / 2 + 3) / 4 * 4;     // a multiple of 4 below K
    const hipError_t e = launch_fill(p, -0.0f, s);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<uint32_t>(16 * ((strips + 7) / 8)));
    const bool vec_a = (reinterpret_cast<uintptr_t>(p.A) & 7) == 0 && p.lda % 4 == 0;
    if (p.M <= 4) return launch_ksplit16_m<T, 4, kL>(p, s, grid, khalf, vec_a);
    return launch_ksplit16_m<T, 8, kL>(p, s, grid, khalf, vec_a);
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
    if constexpr (P == 4) {
        if (ksplit_fits(p)) return launch_ksplit(p, s);
    } else {
        if (ksplit16_fits(p)) return launch_ksplit16<T, 8>(p, s);
    }
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
