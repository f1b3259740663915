// fp32 family for products too small to fill the chip with tiles: one 32 x
// 32 tile of C per work-group, its K range shared by the work-group's four
// waves.
//
// A 64 x 64 tile gives each of its waves one 32 x 32 block and the whole K
// range: K / 2 dependent v_mfma_f32_32x32x2_f32 per wave (64 cycles each),
// so a 256^3 product (16 such tiles) takes 8192 cycles on 16 CUs however idle
// the other 240 are.  Here the waves of a work-group take the 8-wide K groups
// round robin (wave w: groups w, w + 4, ...), each accumulating its own
// partial 32 x 32 block, and the four partial blocks are added in LDS in a
// fixed order (deterministic, no atomics, no workspace); with 32 x 32 tiles
// there are four times as many work-groups and each runs a quarter of the K
// chain.  Grid size as the first lever for small problems is the subject of
// vidyal.ai Part 2 ("The CUDA Programming Model").
//
//   * operands go straight from global memory (L2-resident at these sizes) to
//     registers: lane (h, c) reads k = 8g + 4h .. 8g + 4h + 3 of A row c as
//     one 16-byte load (when A's rows are 16-byte aligned and K % 4 == 0) and the same four
//     rows of B at column c (coalesced across the half-wave); MFMA j of the
//     group then multiplies k = 8g + 4h + j on both sides, so every k meets
//     its own B row;
//   * kU groups per wave make one step, and each step's operands are loaded
//     while the previous step's MFMAs run;
//   * rows past M, columns past N and k past K are loaded as zeros;
//   * C is written once per element, as a streaming store.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // four waves
constexpr int kU = 8;           // K groups per step (per wave)
constexpr int kPad = 33;        // LDS row stride of a partial block (floats)

// x where keep is all ones, +0 where it is zero (a bitwise select: the load
// of x stays unconditional, and an Inf or NaN out of range cannot leak in).
__device__ __forceinline__ float masked(float x, uint32_t keep)
{
    return __uint_as_float(__float_as_uint(x) & keep);
}

template <bool kVecA>
__global__ __launch_bounds__(kThreads) void mfma_f32_splitk_kernel(
    int64_t M, int64_t N, int64_t K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc, int64_t tiles_m,
    int64_t tiles_n)
{
    __shared__ float red[4 * 32 * kPad];   // the four waves' partial blocks

    const TileCoord t = map_tile(tiles_m, tiles_n, 4);
    const int64_t m0 = t.tm * 32, n0 = t.tn * 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, c = lane & 31;
    const int64_t row = m0 + c, col = n0 + c;
    const bool row_ok = row < M, col_ok = col < N;
    const float *arow = A + (row_ok ? row : 0) * lda;
    const float *bcol = B + (col_ok ? col : 0);

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    // kU groups per step; the next step's operands are loaded before this
    // step's MFMAs are issued (two register sets), so the loads of one step
    // overlap the MFMAs of the previous one.
    const int64_t groups = (K + 7) / 8;
    // Every load is issued unconditionally at a clamped, in-bounds address and
    // the values out of range are zeroed afterwards: no branches between the
    // loads, so they all go out before the first wait.
    auto load = [&](int64_t g0, f32x4 (&a)[kU], float (&b)[kU][4]) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t k = 8 * (g0 + 4 * u) + 4 * h;
            if constexpr (kVecA) {
                // K % 4 == 0 here, so the four k are all in range or all out.
                const f32x4 v = *reinterpret_cast<const f32x4 *>(arow + (k < K ? k : K - 4));
                const uint32_t keep = (row_ok && k < K) ? ~0u : 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[u][e] = masked(v[e], keep);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = arow[k + e < K ? k + e : K - 1];
                    a[u][e] = masked(v, (row_ok && k + e < K) ? ~0u : 0u);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = bcol[(k + j < K ? k + j : K - 1) * ldb];
                b[u][j] = masked(v, (col_ok && k + j < K) ? ~0u : 0u);
            }
        }
    };
    auto mfmas = [&](const f32x4 (&a)[kU], const float (&b)[kU][4]) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][j], b[u][j], acc, 0, 0, 0);
    };
    f32x4 a0[kU], a1[kU];
    float b0[kU][4], b1[kU][4];
    int64_t g0 = wave;
    if (g0 < groups) load(g0, a0, b0);
    while (g0 < groups) {
        const int64_t g1 = g0 + 4 * kU;
        if (g1 < groups) load(g1, a1, b1);
        mfmas(a0, b0);
        if (g1 >= groups) break;
        const int64_t g2 = g1 + 4 * kU;
        if (g2 < groups) load(g2, a0, b0);
        mfmas(a1, b1);
        g0 = g2;
    }

    // Register r of lane (h, c) is row 8 (r / 4) + 4 h + r % 4, column c of
    // this wave's partial block.
#pragma unroll
    for (int r = 0; r < 16; ++r)
        red[(wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * kPad + c] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 32; e += kThreads) {
        const int rr = e >> 5, cc = e & 31;
        float v = red[rr * kPad + cc];
#pragma unroll
        for (int w = 1; w < 4; ++w) v += red[(w * 32 + rr) * kPad + cc];
        if (m0 + rr < M && n0 + cc < N) store_c_stream(C + (m0 + rr) * ldc + n0 + cc, v);
    }
}

}  // namespace

hipError_t launch_mfma_f32_splitk(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + 31) / 32, tn = (p.N + 31) / 32;
    if (tm * tn > kMaxBlocks) return hipErrorInvalidValue;
    const auto *A = static_cast<const float *>(p.A);
    const auto *B = static_cast<const float *>(p.B);
    const bool vec = (reinterpret_cast<uintptr_t>(p.A) & 15) == 0 && p.lda % 4 == 0 && p.K % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(mfma_f32_splitk_kernel<true>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc,
                           tm, tn);
    else
        hipLaunchKernelGGL(mfma_f32_splitk_kernel<false>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc,
                           tm, tn);
    return hipGetLastError();
}

}  // namespace mi355gemm
