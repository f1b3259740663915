// Transposed-factor and strided-batched products on the matrix cores:
//
//     C_b = op(A_b) * op(B_b)      for b < batch,
//
// op(A_b) the M x K matrix at A + b*stride_a, stored as written (row i at
// A + i*lda) or transposed (stored K x M, element (i, k) at A[k*lda + i]);
// op(B_b) the K x N matrix at B + b*stride_b, stored K x N or N x K; C_b at
// C + b*stride_c, row-major.  These are the layouts of a training step's
// backward pass (the GPT of "Bare Metal Bard", page 1, second paragraph,
// trained on the same kernels: the input gradient multiplies by a weight
// stored transposed, the weight gradient by activations stored transposed)
// and of per-head attention products (same page, third paragraph).
//
// One template serves every layout.  An operand tile is staged in LDS in
// the orientation it has in memory, so the global loads stay 128-bit and
// coalesced whichever way a factor is stored; what changes with the layout
// is how a lane reads its MFMA fragment back out of LDS:
//
//   * a tile whose rows run along K (A as written, B transposed) is kept as
//     rows of BK elements with their 16-byte chunks XOR-permuted by a row
//     hash, and a lane reads its fragment as one 16-byte read of one row;
//   * a tile whose rows run along M or N (A transposed, B as written) is
//     kept as BK rows of BM or BN elements.  fp32 lanes then read 4-byte
//     values of consecutive columns (a vector of MB or NB of them, one per
//     32 x 32 block, the blocks interleaved over the columns); bf16 lanes
//     use gfx950's transposing LDS read (ds_read_b64_tr_b16), which hands
//     each lane one column of four consecutive rows.
//
// Tiles are 256 x 256 (one work-group per CU, 256 accumulators per lane) or
// 128 x 128 (two per CU); K step 32 (fp32) or 64 (bf16); 256 threads = four
// wave64s in a 2 x 2 grid; global -> registers -> LDS with two LDS stages
// and one barrier per K step.  The work-groups of all products form one
// grid: the work-group id is spread over the XCDs as for a single product,
// so each XCD runs a contiguous range of (product, tile) pairs and the tiles
// of one product share that XCD's L2.  Ragged edges load zeros (rows past
// M or N, k past K) and are masked on store.  K = 0 writes C_b = 0.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// One 32 x 32 x 16 MFMA on 16-bit patterns: bf16, or IEEE fp16 when kF16
// (the kernels stage, read and lay out the same bits either way).
template <bool kF16>
__device__ __forceinline__ f32x16 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef unsigned short u16x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Operand kinds of the 16-bit-staged kernels: 0 bf16, 1 fp16, and the OCP
// 8-bit floats staged two to a 16-bit slot, kFp8Op + 2 * fa + fb with
// fa, fb the formats of A and B (0 e4m3, 1 e5m2).
constexpr int kFp8Op = 2;

// One 32 x 32 x 64 MFMA on 8-bit floats; sa and sb are lane (b, c)'s E8M0
// scales of block b (of 32 elements of K) of row c of A and of B (127 is
// 2^0).  Each operand is the lane's 32 bytes of K: the two 16-byte halves
// given, which the instruction takes as K positions 16 h .. 16 h + 15 and
// 32 + 16 h .. 47 + 16 h of its 64 (block 0 is the first half of both
// half-waves, block 1 the second).  A and B take the same bytes of K from
// their halves, so every k meets its partner.
template <int kOp>
__device__ __forceinline__ f32x16 mfma8(const bf16x8 &a0, const bf16x8 &a1, const bf16x8 &b0,
                                        const bf16x8 &b1, const f32x16 &c, int sa = 127,
                                        int sb = 127)
{
    constexpr int fa = (kOp - kFp8Op) >> 1, fb = (kOp - kFp8Op) & 1;
    const i32x8 a = __builtin_bit_cast(
        i32x8, __builtin_shufflevector(__builtin_bit_cast(u16x8, a0), __builtin_bit_cast(u16x8, a1),
                                       0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
    const i32x8 b = __builtin_bit_cast(
        i32x8, __builtin_shufflevector(__builtin_bit_cast(u16x8, b0), __builtin_bit_cast(u16x8, b1),
                                       0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, fa, fb, 0, sa, 0, sb);
}

constexpr int kThreads = 256;
constexpr int kGroup = 4;   // tile-rows per group in the tile order

template <int W> struct VecF;
template <> struct VecF<2> { typedef f32x2 T; };
template <> struct VecF<4> { typedef f32x4 T; };

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32.  Within each 8-wide K group g, lanes 0-31
// carry k = 8g .. 8g+3 and lanes 32-63 carry k = 8g+4 .. 8g+7 (MFMA j of the
// group takes the j-th of each), for A and B alike, so every k meets its own
// partner whichever way the fragments were read.

namespace f32 {

constexpr int BK = 32;

// Chunk permutation of a row of 32 floats (8 chunks of 16 bytes) in a
// K-contiguous tile: chunk c of row r is stored at c ^ swz(r).
__device__ __forceinline__ int swz(int row) { return (row + (row >> 3)) & 7; }

template <int BM, int BN>
struct Shape {
    static constexpr int kWM = BM / 2, kWN = BN / 2;       // wave tile
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;   // 32 x 32 blocks per wave
    static constexpr int kAChunks = BM * BK / 4 / kThreads;
    static constexpr int kBChunks = BK * BN / 4 / kThreads;
    static_assert(kMB == 2 || kMB == 4, "A read width");
    static_assert(kNB == 2 || kNB == 4, "B read width");
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

// Chunk i of a thread's share of an operand tile spanning R rows or columns
// of the product (R = BM for A, BN for B) and BK values of k.  kKRows: the
// operand's stored rows run along K, so the tile is R stored rows of BK
// (8 chunks per row); otherwise it is BK stored rows of R.
template <int R, bool kKRows>
__device__ __forceinline__ void chunk_pos(int i, int &srow, int &schunk)
{
    const int p = threadIdx.x + kThreads * i;
    if constexpr (kKRows) {
        srow = p >> 3;
        schunk = p & 7;
    } else {
        srow = p / (R / 4);
        schunk = p % (R / 4);
    }
}

template <int R, int kChunks, bool kKRows, bool kVec>
__device__ __forceinline__ void load_operand(f32x4 (&v)[kChunks], const float *__restrict__ X,
                                             int64_t ld, int64_t r0, int64_t rows, int64_t k0,
                                             int64_t K, bool full)
{
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        int sr, sc;
        chunk_pos<R, kKRows>(i, sr, sc);
        if constexpr (kKRows) v[i] = load4<kVec>(X, ld, r0 + sr, k0 + 4 * sc, rows, K, full);
        else v[i] = load4<kVec>(X, ld, k0 + sr, r0 + 4 * sc, K, rows, full);
    }
}

// Stored row of a K-contiguous B tile in LDS: row n = wn*WN + NB*c + nb (the
// column lane c reads for block nb) goes to slot nb*(BN/NB) + n/NB, so the
// 32 rows one fragment read touches are 32 consecutive slots.
template <int BN, int NB>
__device__ __forceinline__ int b_slot(int n) { return (n % NB) * (BN / NB) + n / NB; }

template <int BM, int BN, bool TA, bool TB, int NA, int NBC>
__device__ __forceinline__ void store_operands(const f32x4 (&va)[NA], const f32x4 (&vb)[NBC],
                                               float *As, float *Bs)
{
    using S = Shape<BM, BN>;
    static_assert(NA == S::kAChunks && NBC == S::kBChunks, "chunk counts");
#pragma unroll
    for (int i = 0; i < S::kAChunks; ++i) {
        int sr, sc;
        chunk_pos<BM, !TA>(i, sr, sc);
        float *p = TA ? As + sr * BM + 4 * sc : As + sr * BK + ((sc ^ swz(sr)) << 2);
        *reinterpret_cast<f32x4 *>(p) = va[i];
    }
#pragma unroll
    for (int i = 0; i < S::kBChunks; ++i) {
        int sr, sc;
        chunk_pos<BN, TB>(i, sr, sc);
        float *p;
        if constexpr (TB) {
            const int s = b_slot<BN, S::kNB>(sr);
            p = Bs + s * BK + ((sc ^ swz(s)) << 2);
        } else {
            p = Bs + sr * BN + 4 * sc;
        }
        *reinterpret_cast<f32x4 *>(p) = vb[i];
    }
}

template <int BM, int BN, bool TA, bool TB, int MB, int NB>
__device__ __forceinline__ void compute(f32x16 (&acc)[MB][NB], const float *As, const float *Bs,
                                        int wm, int wn, int lane)
{
    using S = Shape<BM, BN>;
    static_assert(MB == S::kMB && NB == S::kNB, "accumulator shape");
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
        float a[MB][4], b[4][NB];
        if constexpr (TA) {
            // A-lane c of block mb is row MB*c + mb of the wave's piece.
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const auto v = *reinterpret_cast<const typename VecF<MB>::T *>(
                    As + (8 * g + 4 * h + j) * BM + wm * S::kWM + MB * c);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) a[mb][j] = v[mb];
            }
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * S::kWM + mb * 32 + c;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(
                    As + row * BK + (((2 * g + h) ^ swz(row)) << 2));
#pragma unroll
                for (int j = 0; j < 4; ++j) a[mb][j] = v[j];
            }
        }
        if constexpr (TB) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int s = nb * (BN / NB) + wn * 32 + c;   // b_slot(wn*WN + NB*c + nb)
                const f32x4 v = *reinterpret_cast<const f32x4 *>(
                    Bs + s * BK + (((2 * g + h) ^ swz(s)) << 2));
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j][nb] = v[j];
            }
        } else {
            // B-lane c of block nb is column NB*c + nb of the wave's piece.
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const auto v = *reinterpret_cast<const typename VecF<NB>::T *>(
                    Bs + (8 * g + 4 * h + j) * BN + wn * S::kWN + NB * c);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) b[j][nb] = v[nb];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][j], b[j][nb],
                                                                        acc[mb][nb], 0, 0, 0);
    }
}

template <int BM, int BN, bool TA, bool TB, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, BM == 256 ? 1 : 2)))
void batched_kernel(int64_t M, int64_t N, int64_t K, const float *__restrict__ A, int64_t lda,
                    int64_t sa, const float *__restrict__ B, int64_t ldb, int64_t sb,
                    float *__restrict__ C, int64_t ldc, int64_t sc, int64_t batch,
                    int64_t tiles_m, int64_t tiles_n, int cvec)
{
    using S = Shape<BM, BN>;
    constexpr int MB = S::kMB, NB = S::kNB;
    __shared__ __attribute__((aligned(16))) float As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BN];

    const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
    A += t.b * sa;
    B += t.b * sb;
    C += t.b * sc;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool a_full = m0 + BM <= M, b_full = n0 + BN <= N;

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = (K + BK - 1) / BK;
    if (ktiles > 0) {
        f32x4 va[S::kAChunks], vb[S::kBChunks];
        load_operand<BM, S::kAChunks, !TA, kVec>(va, A, lda, m0, M, 0, K, a_full && BK <= K);
        load_operand<BN, S::kBChunks, TB, kVec>(vb, B, ldb, n0, N, 0, K, b_full && BK <= K);
        store_operands<BM, BN, TA, TB, S::kAChunks, S::kBChunks>(va, vb, As[0], Bs[0]);
        __syncthreads();
        for (int64_t kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < ktiles;
            if (more) {
                const int64_t k0 = (kt + 1) * BK;
                const bool kfull = k0 + BK <= K;
                load_operand<BM, S::kAChunks, !TA, kVec>(va, A, lda, m0, M, k0, K, a_full && kfull);
                load_operand<BN, S::kBChunks, TB, kVec>(vb, B, ldb, n0, N, k0, K, b_full && kfull);
            }
            compute<BM, BN, TA, TB, MB, NB>(acc, As[cur], Bs[cur], wm, wn, lane);
            if (more) store_operands<BM, BN, TA, TB, S::kAChunks, S::kBChunks>(va, vb, As[cur ^ 1], Bs[cur ^ 1]);
            __syncthreads();
        }
    }

    // Register r of block (mb, nb) in lane (h, c) is the MFMA output row
    // i = 8*(r/4) + 4*h + r%4 (an A-lane index) and column c (a B-lane
    // index); the NB columns of a lane are consecutive, so they go out as
    // one vector store.
    using BV = typename VecF<NB>::T;
    const int h = lane >> 5, c = lane & 31;
    const int64_t col = n0 + wn * S::kWN + NB * c;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * h + (r & 3);
            const int64_t row = m0 + wm * S::kWM + (TA ? MB * i + mb : mb * 32 + i);
            if (row >= M) continue;
            float *p = C + row * ldc + col;
            if (cvec && col + NB <= N) {
                BV v;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) v[nb] = acc[mb][nb][r];
                store_c_stream(reinterpret_cast<BV *>(p), v);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    if (col + nb < N) store_c_stream(p + nb, acc[mb][nb][r]);
            }
        }
}

}  // namespace f32

// ---------------------------------------------------------------------------
// bf16: v_mfma_f32_32x32x16_bf16.  Lane (h, c) supplies row (A) or column
// (B) c of a 32-wide block and the eight k = 16s + 8h .. 16s + 8h + 7 of
// K slice s.

namespace bf {

constexpr int BK = 64;

// K-contiguous tile rows (64 bf16 = 8 chunks): chunk c of row r at
// c ^ ((r >> 1) & 7), so the 32 consecutive rows of one fragment read fall
// in distinct banks.
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }

// Rows of an M- or N-contiguous tile (16 or 32 chunks): chunk c of row r at
// c ^ mask(r mod 4), masks {0, 4, 10, 14}, so the four rows one transposing
// read touches fall in distinct banks.
__device__ __forceinline__ int rswz(int row)
{
    const int r = row & 3;
    return ((r >> 1) << 1) | ((r & 1) << 2) | ((r >> 1) << 3);
}

template <int BM, int BN>
struct Shape {
    static constexpr int kWM = BM / 2, kWN = BN / 2;
    static constexpr int kMB = kWM / 32, kNB = kWN / 32;
    static constexpr int kAChunks = BM * BK / 8 / kThreads;
    static constexpr int kBChunks = BK * BN / 8 / kThreads;
    static_assert(BM / 8 >= 16 && BN / 8 >= 16, "row swizzle needs 16 chunks");
};

template <bool kVec>
__device__ __forceinline__ u16x8 load8(const uint16_t *__restrict__ base, int64_t ld, int64_t row,
                                       int64_t col, int64_t rows, int64_t cols, bool full)
{
    if (kVec && full) return *reinterpret_cast<const u16x8 *>(base + row * ld + col);
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row < rows) {
        const uint16_t *p = base + row * ld;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < cols) v[e] = p[col + e];
    }
    return v;
}

template <int R, bool kKRows>
__device__ __forceinline__ void chunk_pos(int i, int &srow, int &schunk)
{
    const int p = threadIdx.x + kThreads * i;
    if constexpr (kKRows) {
        srow = p >> 3;
        schunk = p & 7;
    } else {
        srow = p / (R / 8);
        schunk = p % (R / 8);
    }
}

template <int R, int kChunks, bool kKRows, bool kVec>
__device__ __forceinline__ void load_operand(u16x8 (&v)[kChunks], const uint16_t *__restrict__ X,
                                             int64_t ld, int64_t r0, int64_t rows, int64_t k0,
                                             int64_t K, bool full)
{
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        int sr, sc;
        chunk_pos<R, kKRows>(i, sr, sc);
        if constexpr (kKRows) v[i] = load8<kVec>(X, ld, r0 + sr, k0 + 8 * sc, rows, K, full);
        else v[i] = load8<kVec>(X, ld, k0 + sr, r0 + 8 * sc, K, rows, full);
    }
}

template <int R, int kChunks, bool kKRows>
__device__ __forceinline__ void store_operand(const u16x8 (&v)[kChunks], uint16_t *Xs)
{
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        int sr, sc;
        chunk_pos<R, kKRows>(i, sr, sc);
        uint16_t *p = kKRows ? Xs + sr * BK + ((sc ^ kswz(sr)) << 3)
                             : Xs + sr * R + ((sc ^ rswz(sr)) << 3);
        *reinterpret_cast<u16x8 *>(p) = v[i];
    }
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 read_tr(const uint16_t *lds_elem)
{
    auto p = (lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)(lds_elem));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

// Fragment of 32-wide block `base` (first row or column of the block inside
// the tile) for K slice s.  kKRows: 16-byte read of stored row base + c.
// Otherwise (stored rows along K, R wide): in each group of 16 lanes, lane i
// points at 4 consecutive columns of row k_lo = 16s + 8h + i/4 and the
// transposing read returns, to lane i, column i of those four rows; a second
// read 4 rows down gives the other four k.
template <int R, bool kKRows>
__device__ __forceinline__ bf16x8 fragment(const uint16_t *Xs, int base, int s, int lane)
{
    const int h = lane >> 5;
    if constexpr (kKRows) {
        const int row = base + (lane & 31);
        const u16x8 v = *reinterpret_cast<const u16x8 *>(
            Xs + row * BK + (((2 * s + h) ^ kswz(row)) << 3));
        return __builtin_bit_cast(bf16x8, v);
    } else {
        const int i = lane & 15, half = (lane >> 4) & 1;
        const int k_lo = 16 * s + 8 * h + (i >> 2);
        const int col = base + half * 16 + 4 * (i & 3);
        const uint16_t *p0 = Xs + k_lo * R + (((col >> 3) ^ rswz(k_lo)) << 3) + (col & 7);
        const bf16x4 lo = read_tr(p0), hi = read_tr(p0 + 4 * R);   // rswz(k_lo + 4) == rswz(k_lo)
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// kOp: bf16 (0), fp16 (1) or 8-bit floats (kFp8Op and up; A as written and
// B transposed only, every dimension and leading dimension in 16-bit slots,
// i.e. halved).  An 8-bit K tile is 128 bytes: two 64-byte MFMA steps, each
// made of the lane's 16-byte reads of slices 2t and 2t + 1 (bytes 16 h ..
// 16 h + 15 and 32 + 16 h .. 47 + 16 h of the step, the instruction's own
// K positions).  kMX (8-bit only, a single product): MX block scales, the
// scale of 32-byte block kb of row i of A at xa[kb * ldxa + i] and of row j
// of B at xb[kb * ldxb + j]; lane (h, c) passes the scale of block
// 4 kt + 2 t + h of its row, and the next tile's scale bytes are loaded
// with its operands (127 past the last block of K, where the operands are
// zero-filled).
template <int BM, int BN, bool TA, bool TB, bool kVec, int kOp, bool kMX = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, BM == 256 ? 1 : 2)))
void batched_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A, int64_t lda,
                    int64_t sa, const uint16_t *__restrict__ B, int64_t ldb, int64_t sb,
                    float *__restrict__ C, int64_t ldc, int64_t sc, int64_t batch,
                    int64_t tiles_m, int64_t tiles_n, const uint8_t *__restrict__ xa = nullptr,
                    int64_t ldxa = 0, const uint8_t *__restrict__ xb = nullptr, int64_t ldxb = 0)
{
    using S = Shape<BM, BN>;
    constexpr int MB = S::kMB, NB = S::kNB;
    static_assert(kOp < kFp8Op || (!TA && TB), "8-bit operands: A as written, B transposed");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BK * BN];

    const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
    A += t.b * sa;
    B += t.b * sb;
    C += t.b * sc;
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool a_full = m0 + BM <= M, b_full = n0 + BN <= N;

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = (K + BK - 1) / BK;
    // MX scales of the lane's blocks for the two steps of a tile (this tile
    // and the next, loaded with its operands)
    int xs_a[2][MB], xs_b[2][NB], xn_a[2][MB], xn_b[2][NB];
    const int xh = lane >> 5, xc = lane & 31;
    auto load_scales = [&](int64_t kt, int (&ya)[2][MB], int (&yb)[2][NB]) {
        const int64_t nblk = K / 16;   // 32-byte blocks of K (K in 16-bit slots)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t kb = 4 * kt + 2 * t + xh;
            const bool in = kb < nblk;
            const int64_t kbc = in ? kb : 0;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t r = m0 + wm * S::kWM + mb * 32 + xc;
                const int v = xa[kbc * ldxa + (r < ldxa ? r : ldxa - 1)];
                ya[t][mb] = in ? v : 127;
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int64_t r = n0 + wn * S::kWN + nb * 32 + xc;
                const int v = xb[kbc * ldxb + (r < ldxb ? r : ldxb - 1)];
                yb[t][nb] = in ? v : 127;
            }
        }
    };
    if (ktiles > 0) {
        u16x8 va[S::kAChunks], vb[S::kBChunks];
        load_operand<BM, S::kAChunks, !TA, kVec>(va, A, lda, m0, M, 0, K, a_full && BK <= K);
        load_operand<BN, S::kBChunks, TB, kVec>(vb, B, ldb, n0, N, 0, K, b_full && BK <= K);
        if constexpr (kMX) load_scales(0, xs_a, xs_b);
        store_operand<BM, S::kAChunks, !TA>(va, As[0]);
        store_operand<BN, S::kBChunks, TB>(vb, Bs[0]);
        __syncthreads();
        for (int64_t kt = 0; kt < ktiles; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < ktiles;
            if (more) {
                const int64_t k0 = (kt + 1) * BK;
                const bool kfull = k0 + BK <= K;
                load_operand<BM, S::kAChunks, !TA, kVec>(va, A, lda, m0, M, k0, K, a_full && kfull);
                load_operand<BN, S::kBChunks, TB, kVec>(vb, B, ldb, n0, N, k0, K, b_full && kfull);
                if constexpr (kMX) load_scales(kt + 1, xn_a, xn_b);
            }
            if constexpr (kMX) {
#pragma unroll
                for (int t = 0; t < BK / 32; ++t) {
                    bf16x8 a0[MB], a1[MB], b0[NB], b1[NB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        a0[mb] = fragment<BM, true>(As[cur], wm * S::kWM + mb * 32, 2 * t, lane);
                        a1[mb] = fragment<BM, true>(As[cur], wm * S::kWM + mb * 32, 2 * t + 1, lane);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        b0[nb] = fragment<BN, true>(Bs[cur], wn * S::kWN + nb * 32, 2 * t, lane);
                        b1[nb] = fragment<BN, true>(Bs[cur], wn * S::kWN + nb * 32, 2 * t + 1, lane);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = mfma8<kOp>(a0[mb], a1[mb], b0[nb], b1[nb], acc[mb][nb],
                                                     xs_a[t][mb], xs_b[t][nb]);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) xs_a[t][mb] = xn_a[t][mb];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) xs_b[t][nb] = xn_b[t][nb];
                }
            } else if constexpr (kOp >= kFp8Op) {
#pragma unroll
                for (int t = 0; t < BK / 32; ++t) {
                    bf16x8 a0[MB], a1[MB], b0[NB], b1[NB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        a0[mb] = fragment<BM, true>(As[cur], wm * S::kWM + mb * 32, 2 * t, lane);
                        a1[mb] = fragment<BM, true>(As[cur], wm * S::kWM + mb * 32, 2 * t + 1, lane);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        b0[nb] = fragment<BN, true>(Bs[cur], wn * S::kWN + nb * 32, 2 * t, lane);
                        b1[nb] = fragment<BN, true>(Bs[cur], wn * S::kWN + nb * 32, 2 * t + 1, lane);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = mfma8<kOp>(a0[mb], a1[mb], b0[nb], b1[nb], acc[mb][nb]);
                }
            } else {
#pragma unroll
                for (int s = 0; s < BK / 16; ++s) {
                    bf16x8 a[MB], b[NB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        a[mb] = fragment<BM, !TA>(As[cur], wm * S::kWM + mb * 32, s, lane);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        b[nb] = fragment<BN, TB>(Bs[cur], wn * S::kWN + nb * 32, s, lane);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[mb][nb] = mfma16<kOp == 1>(a[mb], b[nb], acc[mb][nb]);
                }
            }
            if (more) {
                store_operand<BM, S::kAChunks, !TA>(va, As[cur ^ 1]);
                store_operand<BN, S::kBChunks, TB>(vb, Bs[cur ^ 1]);
            }
            __syncthreads();
        }
    }

    // Register r of block (mb, nb) in lane (h, c): row 8*(r/4) + 4*h + r%4
    // and column c of that 32 x 32 block.
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t col = n0 + wn * S::kWN + nb * 32 + c;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * S::kWM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) store_c_stream(C + row * ldc + col, acc[mb][nb][r]);
            }
        }
}

}  // namespace bf

// ---------------------------------------------------------------------------
// fp32 split-K for products whose output is too small to fill the chip with
// tiles but whose K is long: the weight gradient X^T dY of a layer is a
// d_in x d_out output summed over every token of the batch (16384 for the
// GPT above).  One 32 x 32 tile of C per work-group; its four waves take the
// K groups round robin, each accumulating its own partial 32 x 32 block,
// and the four partial blocks are added in LDS in a fixed order
// (deterministic, no atomics, no workspace).  Operands go straight from
// global memory (L2) to registers, kU groups per step, the next step's
// loads in flight while this step's MFMAs run.  Every load is issued at a
// clamped, in-bounds address and values out of range are zeroed with a
// bitwise mask, so no branch sits between the loads.
//
// Lane (h, c) supplies row c of the tile's A block and column c of its B
// block.  Along a stored row of K (A as written, B transposed) a lane's
// values are one 16-byte load when the rows allow it; across stored rows
// (A transposed, B as written) they are 4-byte loads that are coalesced
// over the 32 lanes of a half-wave.

namespace sk {

constexpr int kPad = 33;   // LDS row stride of a partial block (floats)

__device__ __forceinline__ float masked(float x, uint32_t keep)
{
    return __uint_as_float(__float_as_uint(x) & keep);
}

__device__ __forceinline__ int64_t clampk(int64_t k, int64_t K) { return k < K ? k : K - 1; }

// The kW partial blocks of a work-group's waves, added in wave order, to C.
template <int kW = 4>
__device__ __forceinline__ void reduce_store(float *red, const f32x16 &acc, int wave, int lane,
                                             float *__restrict__ C, int64_t ldc, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0)
{
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        red[(wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * kPad + c] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 32; e += 64 * kW) {
        const int rr = e >> 5, cc = e & 31;
        float v = red[rr * kPad + cc];
#pragma unroll
        for (int w = 1; w < kW; ++w) v += red[(w * 32 + rr) * kPad + cc];
        if (m0 + rr < M && n0 + cc < N) store_c_stream(C + (m0 + rr) * ldc + n0 + cc, v);
    }
}

// Waves per work-group of the fp32 split-K kernel and K groups each loads
// per step.  Measured on the GPT QKV weight gradient (384 x 1152 x 16384,
// A transposed): 4 waves x 8 groups 49.4 TFLOP/s (two waves per SIMD);
// 8 waves x 4 groups 20.0, although it runs four waves per SIMD.
constexpr int kSkWaves = 4, kSkU = 8;

// fp32 (v_mfma_f32_32x32x2_f32): group g is k = 8g .. 8g+7, lane half h
// carries k = 8g + 4h + j for MFMA j.
template <bool TA, bool TB, bool kVecA, bool kVecB>
__global__ __launch_bounds__(64 * kSkWaves) void f32_kernel(
    int64_t M, int64_t N, int64_t K, const float *__restrict__ A, int64_t lda, int64_t sa,
    const float *__restrict__ B, int64_t ldb, int64_t sb, float *__restrict__ C, int64_t ldc,
    int64_t sc, int64_t batch, int64_t tiles_m, int64_t tiles_n)
{
    constexpr int kU = kSkU, kW = kSkWaves;
    __shared__ float red[kW * 32 * kPad];
    const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
    A += t.b * sa;
    B += t.b * sb;
    C += t.b * sc;
    const int64_t m0 = t.tm * 32, n0 = t.tn * 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, c = lane & 31;
    const bool row_ok = m0 + c < M, col_ok = n0 + c < N;
    const int64_t row = row_ok ? m0 + c : 0, col = col_ok ? n0 + c : 0;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    const int64_t groups = (K + 7) / 8;
    auto load = [&](int64_t g0, float (&a)[kU][4], float (&b)[kU][4]) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t k = 8 * (g0 + kW * u) + 4 * h;
            if constexpr (!TA && kVecA) {
                // K % 4 == 0 here, so the four k are all in range or all out
                const f32x4 v = *reinterpret_cast<const f32x4 *>(A + row * lda + (k < K ? k : K - 4));
                const uint32_t keep = (row_ok && k < K) ? ~0u : 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[u][e] = masked(v[e], keep);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t kk = clampk(k + e, K);
                    const float v = TA ? A[kk * lda + row] : A[row * lda + kk];
                    a[u][e] = masked(v, (row_ok && k + e < K) ? ~0u : 0u);
                }
            }
            if constexpr (TB && kVecB) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(B + col * ldb + (k < K ? k : K - 4));
                const uint32_t keep = (col_ok && k < K) ? ~0u : 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) b[u][j] = masked(v[j], keep);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t kk = clampk(k + j, K);
                    const float v = TB ? B[col * ldb + kk] : B[kk * ldb + col];
                    b[u][j] = masked(v, (col_ok && k + j < K) ? ~0u : 0u);
                }
            }
        }
    };
    auto mfmas = [&](const float (&a)[kU][4], const float (&b)[kU][4]) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][j], b[u][j], acc, 0, 0, 0);
    };
    float a0[kU][4], a1[kU][4], b0[kU][4], b1[kU][4];
    int64_t g0 = wave;
    if (g0 < groups) load(g0, a0, b0);
    while (g0 < groups) {
        const int64_t g1 = g0 + kW * kU;
        if (g1 < groups) load(g1, a1, b1);
        mfmas(a0, b0);
        if (g1 >= groups) break;
        const int64_t g2 = g1 + kW * kU;
        if (g2 < groups) load(g2, a0, b0);
        mfmas(a1, b1);
        g0 = g2;
    }
    reduce_store<kW>(red, acc, wave, lane, C, ldc, M, N, m0, n0);
}

}  // namespace sk

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int BM, int BN, bool TA, bool TB>
void launch_f32_layout(const Problem &p, bool vec, int cvec, uint32_t blocks, int64_t tm,
                       int64_t tn, hipStream_t s)
{
    const auto *A = static_cast<const float *>(p.A);
    const auto *B = static_cast<const float *>(p.B);
    if (vec)
        hipLaunchKernelGGL((f32::batched_kernel<BM, BN, TA, TB, true>), dim3(blocks),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb, p.sb,
                           p.C, p.ldc, p.sc, p.batch, tm, tn, cvec);
    else
        hipLaunchKernelGGL((f32::batched_kernel<BM, BN, TA, TB, false>), dim3(blocks),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb, p.sb,
                           p.C, p.ldc, p.sc, p.batch, tm, tn, cvec);
}

template <int BM, int BN>
hipError_t launch_f32(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn * p.batch > kMaxBlocks) return hipErrorInvalidValue;
    const uint32_t blocks = static_cast<uint32_t>(tm * tn * p.batch);
    const bool vec = aligned16(p.A) && aligned16(p.B) && p.lda % 4 == 0 && p.ldb % 4 == 0 &&
                     p.sa % 4 == 0 && p.sb % 4 == 0;
    const int cvec = aligned16(p.C) && p.ldc % 4 == 0 && p.sc % 4 == 0;
    if (p.ta && p.tb) launch_f32_layout<BM, BN, true, true>(p, vec, cvec, blocks, tm, tn, s);
    else if (p.ta) launch_f32_layout<BM, BN, true, false>(p, vec, cvec, blocks, tm, tn, s);
    else if (p.tb) launch_f32_layout<BM, BN, false, true>(p, vec, cvec, blocks, tm, tn, s);
    else launch_f32_layout<BM, BN, false, false>(p, vec, cvec, blocks, tm, tn, s);
    return hipGetLastError();
}

template <int BM, int BN, bool TA, bool TB, int kOp>
void launch_bf16_layout(const Problem &p, bool vec, uint32_t blocks, int64_t tm, int64_t tn,
                        hipStream_t s)
{
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
    // MX block scales: the 128 x 128 tile only (the 256 x 256 one runs out of
    // registers with the scale bytes); the 8-bit operands are always
    // vector-aligned
    if constexpr (kOp >= kFp8Op && !TA && TB && BM == 128) {
        if (p.xa) {
            hipLaunchKernelGGL((bf::batched_kernel<BM, BN, TA, TB, true, kOp, true>), dim3(blocks),
                               dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb,
                               p.sb, p.C, p.ldc, p.sc, p.batch, tm, tn, p.xa, p.ldxa, p.xb,
                               p.ldxb);
            return;
        }
    }
    if (vec)
        hipLaunchKernelGGL((bf::batched_kernel<BM, BN, TA, TB, true, kOp>), dim3(blocks),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb, p.sb,
                           p.C, p.ldc, p.sc, p.batch, tm, tn);
    else
        hipLaunchKernelGGL((bf::batched_kernel<BM, BN, TA, TB, false, kOp>), dim3(blocks),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb, p.sb,
                           p.C, p.ldc, p.sc, p.batch, tm, tn);
}

template <int BM, int BN, bool kF16 = false>
hipError_t launch_bf16(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn * p.batch > kMaxBlocks) return hipErrorInvalidValue;
    const uint32_t blocks = static_cast<uint32_t>(tm * tn * p.batch);
    const bool vec = aligned16(p.A) && aligned16(p.B) && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
                     p.sa % 8 == 0 && p.sb % 8 == 0;
    constexpr int op = kF16 ? 1 : 0;
    if (p.ta && p.tb) launch_bf16_layout<BM, BN, true, true, op>(p, vec, blocks, tm, tn, s);
    else if (p.ta) launch_bf16_layout<BM, BN, true, false, op>(p, vec, blocks, tm, tn, s);
    else if (p.tb) launch_bf16_layout<BM, BN, false, true, op>(p, vec, blocks, tm, tn, s);
    else launch_bf16_layout<BM, BN, false, false, op>(p, vec, blocks, tm, tn, s);
    return hipGetLastError();
}

// 8-bit operands (A as written, B transposed; K, lda, ldb, stride_a and
// stride_b multiples of 16 bytes and A, B 16-byte aligned, as validated):
// the 16-bit kernel on the same bytes seen as 16-bit slots.
template <int BM, int BN>
hipError_t launch_fp8(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn * p.batch > kMaxBlocks || !supports_fp8(p)) return hipErrorInvalidValue;
    if (p.xa && (BM != 128 || p.batch != 1)) return hipErrorInvalidValue;
    const uint32_t blocks = static_cast<uint32_t>(tm * tn * p.batch);
    Problem q = p;
    q.K = p.K / 2;
    q.lda = p.lda / 2;
    q.ldb = p.ldb / 2;
    q.sa = p.sa / 2;
    q.sb = p.sb / 2;
    switch (2 * p.fa + p.fb) {
    case 0: launch_bf16_layout<BM, BN, false, true, kFp8Op + 0>(q, true, blocks, tm, tn, s); break;
    case 1: launch_bf16_layout<BM, BN, false, true, kFp8Op + 1>(q, true, blocks, tm, tn, s); break;
    case 2: launch_bf16_layout<BM, BN, false, true, kFp8Op + 2>(q, true, blocks, tm, tn, s); break;
    default: launch_bf16_layout<BM, BN, false, true, kFp8Op + 3>(q, true, blocks, tm, tn, s); break;
    }
    return hipGetLastError();
}

template <typename T, bool TA, bool TB, bool VA, bool VB>
void launch_sk_layout(const Problem &p, uint32_t blocks, int64_t tm, int64_t tn, hipStream_t s)
{
    const auto *A = static_cast<const T *>(p.A);
    const auto *B = static_cast<const T *>(p.B);
    hipLaunchKernelGGL((sk::f32_kernel<TA, TB, VA, VB>), dim3(blocks), dim3(64 * sk::kSkWaves), 0, s,
                       p.M, p.N, p.K, A, p.lda, p.sa, B, p.ldb, p.sb, p.C, p.ldc, p.sc, p.batch,
                       tm, tn);
}

// The vector load exists only along a stored row of K (A as written, B
// transposed); it needs 16-byte aligned rows and K a multiple of the vector.
template <typename T>
hipError_t launch_splitk(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + 31) / 32, tn = (p.N + 31) / 32;
    if (tm * tn * p.batch > kMaxBlocks) return hipErrorInvalidValue;
    const uint32_t blocks = static_cast<uint32_t>(tm * tn * p.batch);
    constexpr int64_t v = 16 / sizeof(T);
    const bool kv = p.K % v == 0;
    const bool va = !p.ta && kv && aligned16(p.A) && p.lda % v == 0 && p.sa % v == 0;
    const bool vb = p.tb && kv && aligned16(p.B) && p.ldb % v == 0 && p.sb % v == 0;
    if (p.ta && p.tb) {
        if (vb) launch_sk_layout<T, true, true, false, true>(p, blocks, tm, tn, s);
        else launch_sk_layout<T, true, true, false, false>(p, blocks, tm, tn, s);
    } else if (p.ta) {
        launch_sk_layout<T, true, false, false, false>(p, blocks, tm, tn, s);
    } else if (p.tb) {
        if (va && vb) launch_sk_layout<T, false, true, true, true>(p, blocks, tm, tn, s);
        else if (va) launch_sk_layout<T, false, true, true, false>(p, blocks, tm, tn, s);
        else if (vb) launch_sk_layout<T, false, true, false, true>(p, blocks, tm, tn, s);
        else launch_sk_layout<T, false, true, false, false>(p, blocks, tm, tn, s);
    } else {
        if (va) launch_sk_layout<T, false, false, true, false>(p, blocks, tm, tn, s);
        else launch_sk_layout<T, false, false, false, false>(p, blocks, tm, tn, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_f32_batched_splitk(const Problem &p, hipStream_t s)
{
    return launch_splitk<float>(p, s);
}

hipError_t launch_mfma_f16_batched(const Problem &p, hipStream_t s)
{
    return launch_bf16<256, 256, true>(p, s);
}

hipError_t launch_mfma_f16_batched128(const Problem &p, hipStream_t s)
{
    return launch_bf16<128, 128, true>(p, s);
}

hipError_t launch_mfma_f32_batched(const Problem &p, hipStream_t s)
{
    return launch_f32<256, 256>(p, s);
}

hipError_t launch_mfma_f32_batched128(const Problem &p, hipStream_t s)
{
    return launch_f32<128, 128>(p, s);
}

hipError_t launch_mfma_bf16_batched(const Problem &p, hipStream_t s)
{
    return launch_bf16<256, 256>(p, s);
}

hipError_t launch_mfma_bf16_batched128(const Problem &p, hipStream_t s)
{
    return launch_bf16<128, 128>(p, s);
}

hipError_t launch_mfma_fp8_batched(const Problem &p, hipStream_t s)
{
    return launch_fp8<256, 256>(p, s);
}

hipError_t launch_mfma_fp8_batched128(const Problem &p, hipStream_t s)
{
    return launch_fp8<128, 128>(p, s);
}

}  // namespace mi355gemm
