// Bandwidth kernels for 8-bit float products with few rows (M <= 16):
// C (M x N) = A B with B given transposed (Bt, N x K, each row running
// along K), the shape of a decode step through FP8 weights (vidyal.ai tag
// page, Part 11: low-precision matmuls are bandwidth-bound at small batch).
// Such products sit far below the ridge point, so their time is the time
// to stream Bt once.  Without block scales the products run on the matrix
// cores (skinny_fp8_mfma_kernel below); with MX scales on the vector ALUs:
//
//   * each wave owns four rows of Bt (four columns of C); its 64 lanes
//     take consecutive 16-byte chunks of each row, so every load
//     instruction reads 1 KiB contiguous per row;
//   * A (at most 16 rows) is read from the caches by every wave;
//   * the 8-bit values are widened to fp32 with the hardware conversion
//     (v_cvt_pk_f32_fp8 / _bf8) and multiplied and added in fp32 (exact
//     products);
//   * each lane's partial sums are added over the wave by an xor butterfly,
//     which leaves the same total in every lane (a fixed order: the result
//     is repeatable bit for bit);
//   * with MX block scales (kMX: one E8M0 scale per 32 elements of K of each
//     row of A and of Bt, block kb of row i at x[kb * ld + i]) a chunk's
//     16 products are summed on their own and added times 2^(sa + sb - 254)
//     (v_ldexp_f32: the exact power-of-two scaling, rounded once); the four
//     Bt rows' scales of a block are one 4-byte load, A's come from the
//     caches; a NaN scale (255) makes the chunk's contribution NaN.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 4;    // rows of Bt per wave
constexpr int kWaves = 4;   // waves per work-group

// Sixteen 8-bit values (format 0 e4m3, 1 e5m2) as fp32.  A and B are
// widened by the same code, so any order of the values within the chunk
// pairs each k with its partner.
template <int kFmt>
__device__ __forceinline__ void widen16(const u32x4 &v, float (&out)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int w = static_cast<int>(v[q]);
        f32x2 lo, hi;
        if constexpr (kFmt == 0) {
            lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        } else {
            lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
            hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
        }
        out[4 * q] = lo[0];
        out[4 * q + 1] = lo[1];
        out[4 * q + 2] = hi[0];
        out[4 * q + 3] = hi[1];
    }
}

// kMR >= M accumulator rows; K a multiple of 16, rows 16-byte aligned
// (with kMX: K a multiple of 32, ldxb a multiple of 4, xb 4-byte aligned).
template <int kMR, int kFA, int kFB, bool kMX = false>
__global__ __launch_bounds__(64 * kWaves) void skinny_fp8_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ A, int64_t lda,
    const uint8_t *__restrict__ Bt, int64_t ldb, float *__restrict__ C, int64_t ldc,
    const uint8_t *__restrict__ xa = nullptr, int64_t ldxa = 0,
    const uint8_t *__restrict__ xb = nullptr, int64_t ldxb = 0)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * kRows;
    if (j0 >= N) return;   // wave-uniform
    float acc[kMR][kRows];
#pragma unroll
    for (int i = 0; i < kMR; ++i)
#pragma unroll
        for (int r = 0; r < kRows; ++r) acc[i][r] = 0.f;
    const int64_t chunks = K / 16;
#pragma unroll 2
    for (int64_t c = lane; c < chunks; c += 64) {
        u32x4 b[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r)
            b[r] = (j0 + r < N) ? *reinterpret_cast<const u32x4 *>(Bt + (j0 + r) * ldb + 16 * c)
                                : u32x4{0u, 0u, 0u, 0u};
        float bf[kRows][16];
#pragma unroll
        for (int r = 0; r < kRows; ++r) widen16<kFB>(b[r], bf[r]);
        uint32_t xbw = 0;   // the four Bt rows' scales of this chunk's block
        if constexpr (kMX) {
            // j0 is a multiple of 4 and ldxb >= N a multiple of 4: the word is
            // inside the block's row of scales
            xbw = *reinterpret_cast<const uint32_t *>(xb + (c >> 1) * ldxb + j0);
        }
#pragma unroll
        for (int i = 0; i < kMR; ++i) {
            if (i >= M) break;
            const u32x4 a = *reinterpret_cast<const u32x4 *>(A + i * lda + 16 * c);
            float af[16];
            widen16<kFA>(a, af);
            if constexpr (kMX) {
                const int ea = xa[(c >> 1) * ldxa + i];
#pragma unroll
                for (int r = 0; r < kRows; ++r) {
                    float t = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) t = __builtin_fmaf(af[e], bf[r][e], t);
                    const int eb = (xbw >> (8 * r)) & 255;
                    const float v = (ea == 255 || eb == 255) ? __builtin_nanf("")
                                                             : __builtin_ldexpf(t, ea + eb - 254);
                    acc[i][r] += v;
                }
            } else {
#pragma unroll
                for (int r = 0; r < kRows; ++r)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[i][r] = __builtin_fmaf(af[e], bf[r][e], acc[i][r]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kMR; ++i)
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            float v = acc[i][r];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            acc[i][r] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kMR; ++i)
#pragma unroll
            for (int r = 0; r < kRows; ++r)
                if (i < M && j0 + r < N) store_c_stream(C + i * ldc + j0 + r, acc[i][r]);
    }
}

// ---------------------------------------------------------------------------
// Without block scales, up to 16 rows: the products on the matrix cores.
//
// The widening and fp32 FMAs above cost about 4 vector operations per byte
// of Bt at 4 rows (16 at 16 rows), more than the stream leaves time for.
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) takes both operands in
// exactly the stored layout: lane l supplies 32 bytes of K of row l % 16 of
// A and of row l % 16 of Bt, and the instruction sums over the 128 bytes of
// K that the four lane groups hold.  Which 32 bytes a lane group holds does
// not matter for an unscaled product as long as A and Bt use the same
// assignment (each k still meets its partner), so lane group g takes bytes
// 32 g .. 32 g + 31 of each 128-byte block, two 16-byte loads per operand.
//
//   * a work-group owns 16 rows of Bt (16 columns of C), its four waves
//     take the 128-byte K blocks round robin (wave w: blocks w, w + 4, ..);
//     rows of A past M and of Bt past N re-read the last valid row (their
//     sums are dropped);
//   * each wave loads kU blocks per step and issues the next step's loads
//     before the current step's products (two register sets in turn); two
//     accumulators alternate so that consecutive products are independent;
//   * the 16 x 16 sums land with lane l holding rows 4 (l / 16) .. + 3 of
//     column l % 16; the four waves' sums are added through LDS in wave
//     order (the same bits every run);
//   * a last block that K does not fill is loaded with zeros past K.
template <int kFA, int kFB>
__global__ __launch_bounds__(256) void skinny_fp8_mfma_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ A, int64_t lda,
    const uint8_t *__restrict__ Bt, int64_t ldb, float *__restrict__ C, int64_t ldc)
{
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kU = 4;                        // 128-byte blocks per step
    __shared__ f32x4 red[4][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t ar = i < M ? i : M - 1, br = j0 + i < N ? j0 + i : N - 1;
    const uint8_t *pa = A + ar * lda + 32 * g;
    const uint8_t *pb = Bt + br * ldb + 32 * g;

    const int64_t nfull = K / 128;               // whole blocks
    // this wave's whole blocks: w, w + 4, ... below nfull
    const int64_t mine = nfull > wave ? (nfull - wave + 3) / 4 : 0;
    const int64_t steps = mine / kU;

    auto load = [&](i32x8 (&xa)[kU], i32x8 (&xb)[kU], int64_t t0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t off = (wave + 4 * (t0 + u)) * 128;
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(pa + off);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(pa + off + 16);
            const u32x4 b0 = *reinterpret_cast<const u32x4 *>(pb + off);
            const u32x4 b1 = *reinterpret_cast<const u32x4 *>(pb + off + 16);
            xa[u] = i32x8{int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]),
                          int(a1[0]), int(a1[1]), int(a1[2]), int(a1[3])};
            xb[u] = i32x8{int(b0[0]), int(b0[1]), int(b0[2]), int(b0[3]),
                          int(b1[0]), int(b1[1]), int(b1[2]), int(b1[3])};
        }
    };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    auto compute = [&](const i32x8 (&xa)[kU], const i32x8 (&xb)[kU]) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
            acc[u & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[u], xb[u], acc[u & 1], kFA,
                                                                          kFB, 0, 127, 0, 127);
    };

    int64_t t = 0;
    if (steps > 0) {
        i32x8 a0[kU], b0[kU], a1[kU], b1[kU];
        load(a0, b0, 0);
        int64_t s = 1;
        for (; s + 1 < steps; s += 2) {
            load(a1, b1, kU * s);
            __builtin_amdgcn_sched_barrier(0);
            compute(a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            load(a0, b0, kU * (s + 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(a1, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < steps) {
            load(a1, b1, kU * s);
            __builtin_amdgcn_sched_barrier(0);
            compute(a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            compute(a1, b1);
        } else {
            compute(a0, b0);
        }
        t = kU * steps;
    }
    // the rest of this wave's blocks one at a time, the last partial block
    // (K not a multiple of 128) with zeros past K
    for (;; ++t) {
        const int64_t kb = wave + 4 * t;
        if (kb * 128 >= K) break;
        const int64_t off = kb * 128;
        const bool in0 = off + 32 * g < K, in1 = off + 32 * g + 16 < K;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a0 = in0 ? *reinterpret_cast<const u32x4 *>(pa + off) : z;
        const u32x4 a1 = in1 ? *reinterpret_cast<const u32x4 *>(pa + off + 16) : z;
        const u32x4 b0 = in0 ? *reinterpret_cast<const u32x4 *>(pb + off) : z;
        const u32x4 b1 = in1 ? *reinterpret_cast<const u32x4 *>(pb + off + 16) : z;
        const i32x8 xa = {int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]),
                          int(a1[0]), int(a1[1]), int(a1[2]), int(a1[3])};
        const i32x8 xb = {int(b0[0]), int(b0[1]), int(b0[2]), int(b0[3]),
                          int(b1[0]), int(b1[1]), int(b1[2]), int(b1[3])};
        acc[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, xb, acc[t & 1], kFA, kFB, 0,
                                                                       127, 0, 127);
    }

    red[wave][lane] = acc[0] + acc[1];
    __syncthreads();
    // thread q: lane q % 64's element q / 64 (row 4 (l / 16) + r, column l % 16)
    const int q = threadIdx.x, l = q & 63, r = q >> 6;
    const float v = ((red[0][l][r] + red[1][l][r]) + red[2][l][r]) + red[3][l][r];
    const int64_t row = 4 * (l >> 4) + r, col = j0 + (l & 15);
    if (row < M && col < N) store_c_stream(C + row * ldc + col, v);
}

template <int kMR, bool kMX>
void launch_rows(const Problem &p, dim3 grid, hipStream_t s)
{
    const auto *A = static_cast<const uint8_t *>(p.A);
    const auto *B = static_cast<const uint8_t *>(p.B);
#define MI355_SKINNY_FP8(FA, FB)                                                                 \
    hipLaunchKernelGGL((skinny_fp8_kernel<kMR, FA, FB, kMX>), grid, dim3(64 * kWaves), 0, s,   \
                       p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, p.xa, p.ldxa, p.xb, p.ldxb)
    switch (2 * p.fa + p.fb) {
    case 0: MI355_SKINNY_FP8(0, 0); break;
    case 1: MI355_SKINNY_FP8(0, 1); break;
    case 2: MI355_SKINNY_FP8(1, 0); break;
    default: MI355_SKINNY_FP8(1, 1); break;
    }
#undef MI355_SKINNY_FP8
}

}  // namespace

bool supports_skinny_fp8(const Problem &p)
{
    return supports_fp8(p) && p.batch == 1 && p.M <= (p.xa ? 8 : kSkinnyMaxM);
}

hipError_t launch_skinny_fp8(const Problem &p, hipStream_t s)
{
    if (!supports_skinny_fp8(p)) return hipErrorInvalidValue;
    if (!p.xa) {
        const int64_t wgs = (p.N + 15) / 16;
        if (wgs > kMaxBlocks) return hipErrorInvalidValue;
        const auto *A = static_cast<const uint8_t *>(p.A);
        const auto *B = static_cast<const uint8_t *>(p.B);
#define MI355_SKINNY_FP8_MFMA(FA, FB)                                                                  \
    hipLaunchKernelGGL((skinny_fp8_mfma_kernel<FA, FB>), dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, s, \
                       p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc)
        switch (2 * p.fa + p.fb) {
        case 0: MI355_SKINNY_FP8_MFMA(0, 0); break;
        case 1: MI355_SKINNY_FP8_MFMA(0, 1); break;
        case 2: MI355_SKINNY_FP8_MFMA(1, 0); break;
        default: MI355_SKINNY_FP8_MFMA(1, 1); break;
        }
#undef MI355_SKINNY_FP8_MFMA
        return hipGetLastError();
    }
    const int64_t per_block = kWaves * kRows;
    const int64_t blocks = (p.N + per_block - 1) / per_block;
    if (blocks > kMaxBlocks) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(blocks));
    if (p.xa) {   // MX scales: at most 8 rows (16 would leave one wave per SIMD)
        if (p.M <= 1) launch_rows<1, true>(p, grid, s);
        else if (p.M <= 2) launch_rows<2, true>(p, grid, s);
        else if (p.M <= 4) launch_rows<4, true>(p, grid, s);
        else launch_rows<8, true>(p, grid, s);
    } else {
        if (p.M <= 1) launch_rows<1, false>(p, grid, s);
        else if (p.M <= 2) launch_rows<2, false>(p, grid, s);
        else if (p.M <= 4) launch_rows<4, false>(p, grid, s);
        else if (p.M <= 8) launch_rows<8, false>(p, grid, s);
        else launch_rows<16, false>(p, grid, s);
    }
    return hipGetLastError();
}

}  // namespace mi355gemm
