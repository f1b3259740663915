// fp32 matrix-core family: v_mfma_f32_32x32x2_f32 (full fp32 products, fp32
// accumulation; gfx950 has no reduced-precision "TF32" matrix instruction, so
// fp32 inputs are never rounded down here).
//
// This is the matrix-instruction rung of the kernel ladder ("Bare Metal
// Bard", page 1, first paragraph: the tensor-core kernel that follows
// coalescing, shared-memory tiling, register tiling, float4 loads,
// warp-level blocking and double buffering; vidyal.ai Part 6, "Tensor
// Cores": what one instruction computes and how to feed it from shared
// memory without bank conflicts), redone for CDNA4:
//
//   * block tile 256 x 256 (large shapes) or 128 x 128 (shapes whose 256 x
//     256 tiles would leave CUs idle), K step 32; 256 threads = 4 wave64s in a
//     2 x 2 grid, each wave owning a quarter of the tile as 32 x 32 MFMA
//     blocks (4 x 4 blocks and 256 accumulators per lane for the large tile,
//     2 x 2 and 64 for the small one, which then runs two work-groups per CU);
//   * global -> registers with 128-bit loads (coalesced along A rows and B
//     rows), registers -> LDS after the current tile's math, two LDS stages
//     (double buffering), one barrier per K step;
//   * A in LDS: 256 rows of 32 floats, the eight 16-byte chunks of each row
//     XOR-permuted by a row hash so that the 32 rows one MFMA operand read
//     touches fall in distinct banks;
//   * B in LDS: 32 rows of BN floats, read as vectors: lane c of a half-wave
//     takes NB consecutive columns, one for each of the wave's NB 32-column
//     MFMA blocks (block q owns columns NB*c + q).  The accumulators of those
//     blocks then hold NB consecutive columns of C per lane, which the
//     epilogue writes as one vector store;
//   * K reordering inside a 128-bit A read: lanes 0-31 carry k = 8g..8g+3 and
//     lanes 32-63 carry k = 8g+4..8g+7 of each group g of eight; the B rows
//     are read with the same pairing, so every k is multiplied with its own
//     B row;
//   * ragged edges: rows of A past M, columns of B past N and k past K are
//     loaded as zeros; rows and columns of C past M, N are not stored.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32;
constexpr int kThreads = 256;
constexpr int kGroup = 4;                          // tile-rows per group in the tile order

// Chunk permutation of an A row in LDS (8 chunks of 4 floats per row).  For
// any 16 consecutive rows read at one logical chunk, the physical 16-byte
// slots modulo 256 bytes are all different, and so are any 8 consecutive
// rows modulo 128 bytes.
__device__ __forceinline__ int a_swz(int row) { return (row + (row >> 3)) & 7; }

template <int NB> struct VecN;
template <> struct VecN<1> { typedef float T; };
template <> struct VecN<2> { typedef f32x2 T; };
template <> struct VecN<4> { typedef f32x4 T; };

template <int BM, int BN>
struct Tile {
    static constexpr int kWM = BM / 2, kWN = BN / 2;       // wave tile
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;   // MFMA blocks per wave
    static constexpr int kAChunks = BM * BK / 4 / kThreads;
    static constexpr int kBChunks = BK * BN / 4 / kThreads;
    static constexpr int kBChunksPerRow = BN / 4;
    static_assert(kNB == 1 || kNB == 2 || kNB == 4, "B read width");
};

template <int BM, int BN>
struct Frag {
    f32x4 a[Tile<BM, BN>::kAChunks];
    f32x4 b[Tile<BM, BN>::kBChunks];
};

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

template <int BM, int BN, bool kVec>
__device__ __forceinline__ void load_tile(Frag<BM, BN> &f, const float *__restrict__ A, int64_t lda,
                                          const float *__restrict__ B, int64_t ldb, int64_t M,
                                          int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                          bool a_full, bool b_full)
{
    using T = Tile<BM, BN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < T::kAChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 3, c = p & 7;
        f.a[i] = load4<kVec>(A, lda, m0 + row, k0 + 4 * c, M, K, a_full);
    }
#pragma unroll
    for (int i = 0; i < T::kBChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p / T::kBChunksPerRow, c = p % T::kBChunksPerRow;
        f.b[i] = load4<kVec>(B, ldb, k0 + row, n0 + 4 * c, K, N, b_full);
    }
}

template <int BM, int BN>
__device__ __forceinline__ void store_tile(const Frag<BM, BN> &f, float *As, float *Bs)
{
    using T = Tile<BM, BN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < T::kAChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 3, c = p & 7;
        *reinterpret_cast<f32x4 *>(As + row * BK + ((c ^ a_swz(row)) << 2)) = f.a[i];
    }
#pragma unroll
    for (int i = 0; i < T::kBChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p / T::kBChunksPerRow, c = p % T::kBChunksPerRow;
        *reinterpret_cast<f32x4 *>(Bs + row * BN + (c << 2)) = f.b[i];
    }
}

template <int BM, int BN, int MB, int NB>
__device__ __forceinline__ void compute_tile(f32x16 (&acc)[MB][NB], const float *As,
                                             const float *Bs, int wm, int wn, int lane)
{
    using T = Tile<BM, BN>;
    static_assert(MB == T::kMB && NB == T::kNB, "accumulator shape");
    using BV = typename VecN<T::kNB>::T;
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
        f32x4 a[T::kMB];
        float b[4][T::kNB];
#pragma unroll
        for (int mb = 0; mb < T::kMB; ++mb) {
            const int row = wm * T::kWM + mb * 32 + c;
            a[mb] = *reinterpret_cast<const f32x4 *>(As + row * BK + (((2 * g + h) ^ a_swz(row)) << 2));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const BV v = *reinterpret_cast<const BV *>(Bs + (8 * g + 4 * h + j) * BN + wn * T::kWN +
                                                       T::kNB * c);
            if constexpr (T::kNB == 1) {
                b[j][0] = v;
            } else {
#pragma unroll
                for (int q = 0; q < T::kNB; ++q) b[j][q] = v[q];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < T::kMB; ++mb)
#pragma unroll
                for (int nb = 0; nb < T::kNB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][j], b[j][nb],
                                                                        acc[mb][nb], 0, 0, 0);
    }
}

template <int BM, int BN, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, BM == 256 ? 1 : 2)))
void mfma_f32_kernel(int64_t M, int64_t N, int64_t K, const float *__restrict__ A, int64_t lda,
                     const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
                     int64_t tiles_m, int64_t tiles_n, int cvec)
{
    using T = Tile<BM, BN>;
    __shared__ float As[2][BM * BK];
    __shared__ float Bs[2][BK * BN];

    const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool a_rows_full = m0 + BM <= M;
    const bool b_cols_full = n0 + BN <= N;

    f32x16 acc[T::kMB][T::kNB];
#pragma unroll
    for (int i = 0; i < T::kMB; ++i)
#pragma unroll
        for (int j = 0; j < T::kNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = (K + BK - 1) / BK;
    Frag<BM, BN> f;
    load_tile<BM, BN, kVec>(f, A, lda, B, ldb, M, N, K, m0, n0, 0, a_rows_full && BK <= K,
                            b_cols_full && BK <= K);
    store_tile<BM, BN>(f, As[0], Bs[0]);
    __syncthreads();

    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < ktiles;
        if (more) {
            const int64_t k0 = (kt + 1) * BK;
            const bool kfull = k0 + BK <= K;
            load_tile<BM, BN, kVec>(f, A, lda, B, ldb, M, N, K, m0, n0, k0, a_rows_full && kfull,
                                    b_cols_full && kfull);
        }
        compute_tile<BM, BN>(acc, As[cur], Bs[cur], wm, wn, lane);
        if (more) store_tile<BM, BN>(f, As[cur ^ 1], Bs[cur ^ 1]);
        __syncthreads();
    }

    // Epilogue: lane (h, c) of block (mb, nb) holds C rows
    // 8*(r/4) + 4*h + r%4 and column NB*c + nb of the wave's piece.
    using BV = typename VecN<T::kNB>::T;
    const int h = lane >> 5, c = lane & 31;
    const int64_t col = n0 + wn * T::kWN + T::kNB * c;
#pragma unroll
    for (int mb = 0; mb < T::kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * T::kWM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row >= M) continue;
            float *p = C + row * ldc + col;
            if (cvec && col + T::kNB <= N) {
                BV v;
                if constexpr (T::kNB == 1) {
                    v = acc[mb][0][r];
                } else {
#pragma unroll
                    for (int nb = 0; nb < T::kNB; ++nb) v[nb] = acc[mb][nb][r];
                }
                *reinterpret_cast<BV *>(p) = v;
            } else {
#pragma unroll
                for (int nb = 0; nb < T::kNB; ++nb)
                    if (col + nb < N) p[nb] = acc[mb][nb][r];
            }
        }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int BM, int BN>
hipError_t launch_tiles(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn > kMaxBlocks) return hipErrorInvalidValue;
    const bool vec = aligned16(p.A) && aligned16(p.B) && p.lda % 4 == 0 && p.ldb % 4 == 0;
    const int cvec = aligned16(p.C) && p.ldc % 4 == 0;
    const auto *A = static_cast<const float *>(p.A);
    const auto *B = static_cast<const float *>(p.B);
    if (vec)
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, true>), dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn, cvec);
    else
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, false>), dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn, cvec);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_f32(const Problem &p, hipStream_t s) { return launch_tiles<256, 256>(p, s); }
hipError_t launch_mfma_f32_128(const Problem &p, hipStream_t s) { return launch_tiles<128, 128>(p, s); }

}  // namespace mi355gemm
