// fp32 vector-ALU family: the shared-memory / register-tiled rungs of the
// kernel ladder ("Bare Metal Bard", page 1, first paragraph: coalescing,
// shared-memory tiling, register tiling, float4 loads, warp-level blocking,
// double buffering; vidyal.ai Part 5, "Writing a Fast Matmul in CUDA, Step
// by Step"), written for wave64 and LDS:
//
//   * block tile 128 x 128, K step 16, 256 threads in a 16 x 16 grid; each
//     lane accumulates an 8 x 8 register tile made of 2 x 2 sub-tiles of
//     4 x 4 placed 64 rows / 64 columns apart, so the 16 lanes of a row read
//     one contiguous 256-byte run of a B row (no bank conflicts) and the
//     four rows of lanes in a wave read four A addresses (broadcasts);
//   * per k: four 128-bit LDS reads feed 64 fp32 FMAs (scalar v_fma_f32;
//     packed fp32 is not used);
//   * A is stored k-major in LDS (transposed on the way in, rows padded by 4
//     floats) so a lane's 4 consecutive rows are one 128-bit read; B keeps
//     its row-major layout;
//   * global -> registers (128-bit where aligned), registers -> LDS after the
//     current step's math, two LDS stages, one barrier per step;
//   * ragged edges load zeros and are masked at the store.
// The dispatch table does not pick this family (the matrix-core families are
// faster on every measured shape); it is kept as the vector-ALU rung of the
// ladder and as an independent cross-check in the parity tests.  A 128 x 256
// tile with 8 x 16 per lane (fewer LDS reads per FMA) measured 89.5 instead
// of 78.8 TFLOP/s at 4096^3 but 85.4 instead of 87.4 at 8192^3 and slower on
// shapes with fewer tiles, so the 8 x 8 lane tile stays.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int kThreads = 256;
constexpr int kPadA = 4;                     // As row pitch = BM + 4 floats
constexpr int kGroup = 8;

template <bool kVec>
__device__ __forceinline__ f32x4 load4(const float *__restrict__ base, int64_t ld, int64_t row,
                                       int64_t col, int64_t rows, int64_t cols, bool full)
{
    if (kVec && full) return *reinterpret_cast<const f32x4 *>(base + row * ld + col);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < rows) {
        const float *p = base + row * ld;
        if (col + 0 < cols) v.x = p[col + 0];
        if (col + 1 < cols) v.y = p[col + 1];
        if (col + 2 < cols) v.z = p[col + 2];
        if (col + 3 < cols) v.w = p[col + 3];
    }
    return v;
}

struct Stage {
    f32x4 a[2];   // A: 128 rows x 16 k = 512 float4, two per thread
    f32x4 b[2];   // B: 16 k x 128 cols = 512 float4, two per thread
};

template <bool kVec>
__device__ __forceinline__ void load_stage(Stage &st, const float *__restrict__ A, int64_t lda,
                                           const float *__restrict__ B, int64_t ldb, int64_t M,
                                           int64_t N, int64_t K, int64_t m0, int64_t n0,
                                           int64_t k0, bool a_full, bool b_full)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + kThreads * i;            // A float4 index: row p / 4, k quad p % 4
        st.a[i] = load4<kVec>(A, lda, m0 + (p >> 2), k0 + 4 * (p & 3), M, K, a_full);
        const int q = tid + kThreads * i;            // B float4 index: row q / 32, col quad q % 32
        st.b[i] = load4<kVec>(B, ldb, k0 + (q >> 5), n0 + 4 * (q & 31), K, N, b_full);
    }
}

__device__ __forceinline__ void store_stage(const Stage &st, float *As, float *Bs)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 2, kq = p & 3;
        As[(4 * kq + 0) * (BM + kPadA) + row] = st.a[i].x;
        As[(4 * kq + 1) * (BM + kPadA) + row] = st.a[i].y;
        As[(4 * kq + 2) * (BM + kPadA) + row] = st.a[i].z;
        As[(4 * kq + 3) * (BM + kPadA) + row] = st.a[i].w;
        const int q = tid + kThreads * i;
        *reinterpret_cast<f32x4 *>(Bs + (q >> 5) * BN + 4 * (q & 31)) = st.b[i];
    }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void valu_f32_kernel(int64_t M, int64_t N, int64_t K, const float *__restrict__ A, int64_t lda,
                     const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
                     int64_t tiles_m, int64_t tiles_n, int cvec)
{
    __shared__ __attribute__((aligned(16))) float As[2][BK * (BM + kPadA)];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BN];

    const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const bool a_rows_full = m0 + BM <= M;
    const bool b_cols_full = n0 + BN <= N;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    const int64_t ktiles = (K + BK - 1) / BK;
    Stage st;
    load_stage<kVec>(st, A, lda, B, ldb, M, N, K, m0, n0, 0, a_rows_full && BK <= K,
                     b_cols_full && BK <= K);
    store_stage(st, As[0], Bs[0]);
    __syncthreads();

    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < ktiles;
        if (more) {
            const int64_t k0 = (kt + 1) * BK;
            const bool kfull = k0 + BK <= K;
            load_stage<kVec>(st, A, lda, B, ldb, M, N, K, m0, n0, k0, a_rows_full && kfull,
                             b_cols_full && kfull);
        }
        const float *as = As[cur];
        const float *bs = Bs[cur];
        // Partial unroll: a full one lets the compiler hoist every LDS read
        // of the step into registers at once and spill.
#pragma unroll 2
        for (int k = 0; k < BK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(as + k * (BM + kPadA) + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(as + k * (BM + kPadA) + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bs + k * BN + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bs + k * BN + 64 + 4 * tx);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) store_stage(st, As[cur ^ 1], Bs[cur ^ 1]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
        if (row >= M) continue;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t col = n0 + half * 64 + 4 * tx;
            float *p = C + row * ldc + col;
            const f32x4 v = {acc[i][4 * half + 0], acc[i][4 * half + 1], acc[i][4 * half + 2],
                             acc[i][4 * half + 3]};
            if (cvec && col + 3 < N) {
                store_c_stream(reinterpret_cast<f32x4 *>(p), v);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < N) store_c_stream(p + e, static_cast<float>(v[e]));
            }
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_valu_f32(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn > kMaxBlocks) return hipErrorInvalidValue;
    const bool vec = aligned16(p.A) && aligned16(p.B) && p.lda % 4 == 0 && p.ldb % 4 == 0;
    const int cvec = aligned16(p.C) && p.ldc % 4 == 0;
    const auto *A = static_cast<const float *>(p.A);
    const auto *B = static_cast<const float *>(p.B);
    if (vec)
        hipLaunchKernelGGL(valu_f32_kernel<true>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn, cvec);
    else
        hipLaunchKernelGGL(valu_f32_kernel<false>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn, cvec);
    return hipGetLastError();
}

}  // namespace mi355gemm
