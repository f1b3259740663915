// Bandwidth kernel for 8-bit float products with few rows (M <= 16):
// C (M x N) = A B with B given transposed (Bt, N x K, each row running
// along K), the shape of a decode step through FP8 weights (vidyal.ai tag
// page, Part 11: low-precision matmuls are bandwidth-bound at small batch).
// Such products sit far below the ridge point, so their time is the time
// to stream Bt once.
//
// Widening the 8-bit values and multiplying in fp32 on the vector ALUs
// costs about 4 vector operations per byte of Bt at 4 rows (16 at 16 rows),
// more than the stream leaves time for, so the products run on the matrix
// cores: v_mfma_scale_f32_16x16x128_f8f6f4 takes both operands in their
// stored layout (rows of A and of Bt both run along K).  Lane (i, g) (i =
// l % 16, g = l / 16) supplies 32 bytes of row i of A and of row i of Bt;
// measured on the GPU, the instruction takes them as bytes 16 g .. 16 g +
// 15 and 64 + 16 g .. 64 + 16 g + 15 of its 128 bytes of K, and applies the
// scale operand of lane (i, g) to the 32-element block g (bytes 32 g .. 32
// g + 31) of row i -- so a lane loads those two 16-byte pieces and passes
// the E8M0 scale of block g of its row (OCP microscaling: one scale per 32
// elements; 127 = 2^0 without scales; 255, NaN, gives NaN).
//
//   * a work-group owns 16 rows of Bt (16 columns of C); its kW waves (4,
//     or 8 when the work-groups number at most the CUs: 1 x 4096 x 16384
//     17.3 -> 15.9 us) take the 128-byte K blocks round robin (wave w:
//     blocks w, w + kW, ..);
//     rows of A past M and of Bt past N re-read the last valid row (their
//     sums are dropped);
//   * each wave loads kU blocks per step and issues the next step's loads
//     before the current step's products (two register sets in turn); two
//     accumulators alternate so that consecutive products are independent;
//   * the 16 x 16 sums land with lane l holding rows 4 (l / 16) .. + 3 of
//     column l % 16; the waves' sums are added through LDS in wave order
//     (the same bits every run);
//   * the blocks left after the whole steps (and a last block that K does
//     not fill) form one more step with zeros past K and the scales of
//     blocks past K read as 127, so short K keeps its loads in flight
//     together.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kU = 4;   // 128-byte K blocks per step

__device__ __forceinline__ i32x8 join(const u32x4 &lo, const u32x4 &hi)
{
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

// K a multiple of 16 (of 32 with kMX), rows 16-byte aligned.
template <int kFA, int kFB, bool kMX, int kW>
__global__ __launch_bounds__(64 * kW) void skinny_fp8_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ A, int64_t lda,
    const uint8_t *__restrict__ Bt, int64_t ldb, float *__restrict__ C, int64_t ldc,
    const uint8_t *__restrict__ xa, int64_t ldxa, const uint8_t *__restrict__ xb, int64_t ldxb)
{
    __shared__ f32x4 red[kW][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t ar = i < M ? i : M - 1, br = j0 + i < N ? j0 + i : N - 1;
    const uint8_t *pa = A + ar * lda + 16 * g;
    const uint8_t *pb = Bt + br * ldb + 16 * g;
    // this lane's scales: block 4 kb + g of row ar (A) and br (Bt)
    const uint8_t *qa = kMX ? xa + g * ldxa + ar : nullptr;
    const uint8_t *qb = kMX ? xb + g * ldxb + br : nullptr;

    const int64_t nfull = K / 128;               // whole blocks
    // this wave's whole blocks: w, w + kW, ... below nfull
    const int64_t mine = nfull > wave ? (nfull - wave + kW - 1) / kW : 0;
    const int64_t steps = mine / kU;

    struct Step {
        i32x8 a[kU], b[kU];
        int sa[kU], sb[kU];
    };
    auto load = [&](Step &x, int64_t t0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t kb = wave + kW * (t0 + u), off = kb * 128;
            x.a[u] = join(*reinterpret_cast<const u32x4 *>(pa + off),
                          *reinterpret_cast<const u32x4 *>(pa + off + 64));
            x.b[u] = join(*reinterpret_cast<const u32x4 *>(pb + off),
                          *reinterpret_cast<const u32x4 *>(pb + off + 64));
            if constexpr (kMX) {
                x.sa[u] = qa[4 * kb * ldxa];
                x.sb[u] = qb[4 * kb * ldxb];
            } else {
                x.sa[u] = x.sb[u] = 127;
            }
        }
    };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    auto compute = [&](const Step &x) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
            acc[u & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x.a[u], x.b[u], acc[u & 1], kFA, kFB,
                                                                          0, x.sa[u], 0, x.sb[u]);
    };

    int64_t t = 0;
    if (steps > 0) {
        Step x0, x1;
        load(x0, 0);
        int64_t s = 1;
        for (; s + 1 < steps; s += 2) {
            load(x1, kU * s);
            __builtin_amdgcn_sched_barrier(0);
            compute(x0);
            __builtin_amdgcn_sched_barrier(0);
            load(x0, kU * (s + 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(x1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < steps) {
            load(x1, kU * s);
            __builtin_amdgcn_sched_barrier(0);
            compute(x0);
            __builtin_amdgcn_sched_barrier(0);
            compute(x1);
        } else {
            compute(x0);
        }
        t = kU * steps;
    }
    // The rest of this wave's blocks (fewer than kU whole ones, and the last
    // partial block if it is this wave's) as one more step, every load
    // issued before the first product: blocks past K and bytes past K are
    // zeros (their scales 127), which add nothing.
    if (wave + kW * t < (K + 127) / 128) {   // wave-uniform
        Step x;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t kb = wave + kW * (t + u), off = kb * 128;
            const bool in0 = off + 16 * g < K, in1 = off + 64 + 16 * g < K;
            const u32x4 z = {0u, 0u, 0u, 0u};
            x.a[u] = join(in0 ? *reinterpret_cast<const u32x4 *>(pa + off) : z,
                          in1 ? *reinterpret_cast<const u32x4 *>(pa + off + 64) : z);
            x.b[u] = join(in0 ? *reinterpret_cast<const u32x4 *>(pb + off) : z,
                          in1 ? *reinterpret_cast<const u32x4 *>(pb + off + 64) : z);
            x.sa[u] = x.sb[u] = 127;
            if constexpr (kMX) {
                if (off + 32 * g < K) {
                    x.sa[u] = qa[4 * kb * ldxa];
                    x.sb[u] = qb[4 * kb * ldxb];
                }
            }
        }
        compute(x);
    }

    red[wave][lane] = acc[0] + acc[1];
    __syncthreads();
    // thread q < 256: lane q % 64's element q / 64 (row 4 (l / 16) + r,
    // column l % 16), the waves added in order
    const int q = threadIdx.x, l = q & 63, r = (q >> 6) & 3;
    if (q < 256) {
        float v = red[0][l][r];
#pragma unroll
        for (int w = 1; w < kW; ++w) v += red[w][l][r];
        const int64_t row = 4 * (l >> 4) + r, col = j0 + (l & 15);
        if (row < M && col < N) store_c_stream(C + row * ldc + col, v);
    }
}

template <bool kMX, int kW>
void launch_formats(const Problem &p, dim3 grid, hipStream_t s)
{
    const auto *A = static_cast<const uint8_t *>(p.A);
    const auto *B = static_cast<const uint8_t *>(p.B);
#define MI355_SKINNY_FP8(FA, FB)                                                                     \
    hipLaunchKernelGGL((skinny_fp8_kernel<FA, FB, kMX, kW>), grid, dim3(64 * kW), 0, s, p.M, p.N, p.K, A, \
                       p.lda, B, p.ldb, p.C, p.ldc, p.xa, p.ldxa, p.xb, p.ldxb)
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
    return supports_fp8(p) && p.batch == 1 && p.M <= kSkinnyMaxM;
}

hipError_t launch_skinny_fp8(const Problem &p, hipStream_t s)
{
    if (!supports_skinny_fp8(p)) return hipErrorInvalidValue;
    const int64_t wgs = (p.N + 15) / 16;
    if (wgs > kMaxBlocks) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(wgs));
    // with at most one work-group per CU, eight waves per work-group keep
    // twice the loads in flight
    const bool eight = wgs <= kCUs;
    if (p.xa) eight ? launch_formats<true, 8>(p, grid, s) : launch_formats<true, 4>(p, grid, s);
    else eight ? launch_formats<false, 8>(p, grid, s) : launch_formats<false, 4>(p, grid, s);
    return hipGetLastError();
}

}  // namespace mi355gemm
