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
//   * A in LDS: BM rows of 32 floats, the eight 16-byte chunks of each row
//     XOR-permuted by a row hash that spreads the 32 rows one MFMA operand
//     read touches over the banks (the hash was chosen by timing on gfx950);
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
//
// Those are the register-staged kernels (mfma_f32, mfma_f32_128).  The
// LDS-direct kernels further down (mfma_f32_direct with 256 x 256 tiles,
// mfma_f32_direct128 with 128 x 128, mfma_f32_direct128x64 with 128 x 64,
// mfma_f32_direct64 with 64 x 64, and the narrow ones with 4-byte loads for
// any layout) are one template: global -> LDS without registers, a
// four-stage LDS ring, fragments read one K group ahead, one barrier per
// tile; they also take a factor stored transposed and strided batches, and
// they are what the dispatch table runs wherever they apply.
#include <type_traits>

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

// Chunk permutation of an A row in LDS (8 chunks of 4 floats = 128 bytes
// per row): chunk c of row r is stored at c ^ ((r + r/8) mod 8).  Chosen by
// measurement on gfx950: (r >> 1) mod 8 makes the operand reads free of bank
// conflicts (SQ_LDS_BANK_CONFLICT = 0, against about 1.3 conflict cycles per
// LDS instruction with this hash), yet an A/B run on one board timed this
// register-staged kernel 13% faster with (r + r/8) mod 8 at 8192^3 (111.1
// vs 96.5 TFLOP/s) and 8% at 4096^3, so the faster one is kept here.
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
                store_c_stream(reinterpret_cast<BV *>(p), v);
            } else {
#pragma unroll
                for (int nb = 0; nb < T::kNB; ++nb)
                    if (col + nb < N) store_c_stream(p + nb, acc[mb][nb][r]);
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

// ---------------------------------------------------------------------------
// Direct variants (BM x BN tile of 256 x 256 or 128 x 128, K step 16, four
// LDS stages): global -> LDS with LDS-direct 128-bit loads (no register
// staging, no LDS write instructions) so the loads for tile t + 3 are in
// flight while tile t is multiplied; operand fragments are read one 8-wide K
// group ahead, across the tile boundary, each read and each load slotted
// between MFMAs; one barrier per tile.  Four waves in a 2 x 2 grid, each
// owning (BM/2) x (BN/2) of C as MB x NB blocks of 32 x 32.  Same layouts as
// the staged kernel (A rows of 16 floats = 4 chunks, chunk-swizzled; B rows
// of BN floats; B read NB columns at a time, interleaved over the blocks).
// The 256 tile runs one work-group per CU (256 accumulators per lane); the
// 128 tile (64 accumulators, 64 KB of LDS) runs two, so that one
// work-group's MFMAs cover the other's barrier, and it leaves fewer CUs idle
// on shapes whose 256-tile count is a poor multiple of 256.
//
// Instruction economy matters here: with one wave per SIMD every non-MFMA
// instruction sits between two MFMAs.  So the loads use the scalar-base
// form (a wave-uniform 64-bit base advanced once per tile plus a fixed
// 32-bit lane offset: no vector address arithmetic), the reads use one
// lane base per stage plus immediate offsets (the A-row swizzle of the rows
// a lane reads depends only on the lane), and the loads past the last tile
// re-fetch the last tile into a stage nobody reads again instead of being
// branched around.
//
// Shapes: K a multiple of 16 (and K > 0), 16-byte aligned A and B with lda
// and ldb multiples of 4, and lane offsets within 32 bits.  A factor stored
// with rows of K (A as written, B transposed) has its lane offsets within a
// panel of up to 256 stored rows; one stored with rows of M or N (A
// transposed, B as written) within 16 stored rows, and that dimension a
// multiple of 4.  Rows of A past M and columns of B past N are fetched from
// the last valid row / chunk (their products land only in rows and columns
// of C that are not stored).  With batch > 1 the grid covers the tiles of
// every product (the 4- and 16-byte narrow and direct tiles alike; the
// narrow ones take untransposed factors only).

constexpr int DBK = 16;           // K step of the direct variants
constexpr int DSTAGES = 4;

typedef float f32x1 __attribute__((ext_vector_type(1)));
template <int NB> struct DVec;
template <> struct DVec<1> { typedef f32x1 T; };
template <> struct DVec<2> { typedef f32x2 T; };
template <> struct DVec<4> { typedef f32x4 T; };

// kW: bytes per lane of one LDS-direct load (16 for the aligned kernels, 4
// for the narrow one); one wave's load fills 64 kW bytes of LDS.
//
// TA / TB: A stored K x M (a transposed factor) / B stored N x K.  A factor
// is staged in LDS in its stored orientation: rows of K (A as written, B
// transposed) as 16-float rows read 16 bytes per lane, rows of M or N (A
// transposed, B as written) as 16 rows read 4 bytes per lane, a vector of
// one value per 32 x 32 block (the blocks interleaved over the columns).
template <int BM, int BN, int kW, bool TA = false, bool TB = false>
struct DTile {
    static_assert(kW == 16 || (!TA && !TB), "transposed factors take the 16-byte loads");
    static constexpr int kMB = BM / 64, kNB = BN / 64;          // blocks per wave
    static constexpr int kAInst = BM * DBK * 4 / (64 * kW) / 4; // LDS-direct loads per wave per tile (A)
    static constexpr int kBInst = DBK * BN * 4 / (64 * kW) / 4; // ... (B)
    static constexpr int kPerTile = kAInst + kBInst;
    static constexpr int kStageFloats = BM * DBK + DBK * BN;
    static constexpr int kBChunksPerRow = BN / 4;
    static constexpr int kQ = 4 * kMB * kNB;                    // MFMAs per 8-wide K group
    static constexpr int kReads = (TA ? 4 : kMB) + (TB ? kNB : 4);   // fragment reads per group
    // The reads of the next group go out after MFMAs 0, 2, 4, .. (after
    // every MFMA when there are fewer than two per read); the loads of a
    // later tile after MFMAs kLoadQ0, kLoadQ0 + kLoadStep, ...
    static constexpr bool kReadEveryOther = 2 * kReads <= kQ;
    // When the loads outnumber the MFMAs of a group (the narrow 128 x 64
    // tile: 12 loads, 8 MFMAs), load l goes after MFMA l * kQ / kPerTile.
    // With one block per wave (64 x 64) the reads outnumber the MFMAs too
    // (5 reads, 4 MFMAs): reads and loads are then both spread that way.
    static constexpr bool kSpreadReads = kReads > kQ;
    static constexpr bool kSpreadLoads = kPerTile > kQ || kSpreadReads;
    static constexpr int kLoadQ0 =
        BM == 256 ? 20 : kSpreadLoads ? 0 : kNB == 1 ? kQ - kPerTile : (kW == 16 ? 1 : 0);
    static constexpr int kLoadStep = kW == 16 && kNB > 1 ? 4 : 1;
    // Work-groups per CU the LDS ring allows (and the occupancy asked of the
    // compiler): 1 for 256 x 256, 2 for 128 x 128, 3 for 128 x 64.
    static constexpr int kPerCU = 160 * 1024 / (DSTAGES * kStageFloats * 4);
    // With one 32-column block per wave, B is read 4 bytes per lane and the
    // two half-waves read rows 4 apart: 16-byte chunks of B rows are
    // XOR-permuted by 8 * bit 2 of the row so those rows use different banks.
    static constexpr bool kBSwz = !TB && kNB == 1;
    // The same for a transposed A read 4 bytes per lane (one block per wave).
    static constexpr bool kASwz = TA && kMB == 1;
    static_assert((kReads <= kQ || kSpreadLoads) &&
                      (kSpreadLoads || kLoadQ0 + kLoadStep * (kPerTile - 1) < kQ),
                  "slots");
    static_assert((DSTAGES - 2) * kPerTile <= 63, "vmcnt is six bits");
    static_assert(kNB == 1 || kNB == 2 || kNB == 4, "B read width");
};

__device__ __forceinline__ int b_swz8(int row) { return ((row >> 2) & 1) << 3; }

// A rows of 4 chunks (64 bytes): chunk c of row r is stored at c ^ ((r >> 2) & 3).
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT, one-pattern microbenchmark):
// the operand read (32 lanes = 32 consecutive rows at one logical chunk per
// half-wave) is conflict-free with this permutation, while the unswizzled
// layout is 4-way and a (r>>1)^(r>>3) hash 2-way conflicted.
__device__ __forceinline__ int a_swz4(int row) { return (row >> 2) & 3; }

// One LDS-direct 128-bit load as inline assembly, scalar-base form: lane i
// reads 16 bytes at sbase + voff and they land at LDS byte M0 + 16 i.  The
// compiler's wait-count pass does not see these loads (it would otherwise
// drain them before every LDS read); the kernel counts them itself.  M0 is
// declared clobbered (nothing else in these kernels keeps a value in it);
// the s_nop covers the M0-write hazard.
__device__ __forceinline__ void lds_direct_load16(uint32_t voff, const void *sbase, uint32_t m0v)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

// The same with 4 bytes per lane (lane i's dword lands at M0 + 4 i); any
// fp32 element address qualifies.
__device__ __forceinline__ void lds_direct_load4(uint32_t voff, const void *sbase, uint32_t m0v)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) void *)(p)));
}

// This wave's LDS reads complete, its LDS-direct loads down to kCntVm in
// flight, then the barrier; inline assembly so the LDS part is not weakened
// by the compiler (it guarantees no wave still reads a stage being refilled).
template <int kCntVm>
__device__ __forceinline__ void wait_lds_vm_barrier()
{
    static_assert(kCntVm >= 0 && kCntVm <= 63, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(kCntVm) : "memory");
}

// Everything a wave needs to address its loads and reads.
template <int BM, int BN, int kW, bool TA = false, bool TB = false>
struct DCtx {
    using T = DTile<BM, BN, kW, TA, TB>;
    uint32_t a_voff[T::kAInst], b_voff[T::kBInst];   // lane offsets (bytes) of each load
    const char *abase, *bbase;                       // tile (k = 0) bases, wave-uniform
    int64_t a_kstride, b_kstride;                    // bytes per K step
    uint32_t lds0;                                   // LDS byte address of stage 0
    int wave;
    uint32_t rdA0, rdA1, rdB, rdB1;                  // lane parts of the read offsets in a stage
};

// The scalar-base loads need their base in scalar registers; where the
// compiler cannot prove a base wave-uniform (after the row epilogue below
// was added it stopped proving it for these kernels) the two readfirstlanes
// put it there.  They cost nothing where the base already is scalar (the
// kernels' code is unchanged by them).
__device__ __forceinline__ const void *uniform_ptr(const void *p)
{
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void *>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int kW>
__device__ __forceinline__ void lds_direct_load(uint32_t voff, const void *sbase, uint32_t m0v)
{
    sbase = uniform_ptr(sbase);
    if constexpr (kW == 16) lds_direct_load16(voff, sbase, m0v);
    else lds_direct_load4(voff, sbase, m0v);
}

template <int BM, int BN, int kW, bool TA, bool TB>
__device__ __forceinline__ void load_one(const DCtx<BM, BN, kW, TA, TB> &x, uint32_t stage_lds,
                                         int64_t kt, int l)
{
    using T = DTile<BM, BN, kW, TA, TB>;
    if (l < T::kAInst)
        lds_direct_load<kW>(x.a_voff[l], x.abase + kt * x.a_kstride,
                            stage_lds + (x.wave * T::kAInst + l) * 64 * kW);
    else
        lds_direct_load<kW>(x.b_voff[l - T::kAInst], x.bbase + kt * x.b_kstride,
                            stage_lds + BM * DBK * 4 + (x.wave * T::kBInst + l - T::kAInst) * 64 * kW);
}

// Fragments of one 8-wide K group for a wave's MB x NB blocks.  A as
// written: a[mb] holds k = 4h .. 4h+3 of row c of block mb; transposed: a[j]
// holds, for k-step j, the MB rows MB c .. MB c + MB - 1 (one per block).  B
// as written: b[j] holds, for k-step j, the NB columns NB c .. NB c + NB - 1
// (one per block nb); transposed: b[nb] holds k = 4h .. 4h+3 of column c of
// block nb.
template <int BM, int BN, bool TA = false, bool TB = false>
struct FragG {
    static constexpr int kMB = BM / 64, kNB = BN / 64;
    using AV = typename DVec<kMB>::T;
    using BV = typename DVec<kNB>::T;
    std::conditional_t<TA, AV, f32x4> a[TA ? 4 : kMB];
    std::conditional_t<TB, f32x4, BV> b[TB ? kNB : 4];
    __device__ __forceinline__ float av(int mb, int j) const
    {
        if constexpr (TA) return a[j][mb];
        else return a[mb][j];
    }
    __device__ __forceinline__ float bv(int j, int nb) const
    {
        if constexpr (TB) return b[nb][j];
        else return b[j][nb];
    }
};

template <int BM, int BN, int kW, bool TA, bool TB>
__device__ __forceinline__ void read_one(FragG<BM, BN, TA, TB> &f, const float *stage,
                                         const DCtx<BM, BN, kW, TA, TB> &x, int g, int idx)
{
    using F = FragG<BM, BN, TA, TB>;
    constexpr int nA = TA ? 4 : F::kMB;
    const char *st = reinterpret_cast<const char *>(stage);
    if (idx < nA) {
        if constexpr (TA)
            f.a[idx] = *reinterpret_cast<const typename F::AV *>(st + x.rdA0 + (8 * g + idx) * (BM * 4));
        else
            f.a[idx] = *reinterpret_cast<const f32x4 *>(st + (g ? x.rdA1 : x.rdA0) + idx * 2048);
    } else {
        const int i = idx - nA;
        if constexpr (TB)
            f.b[i] = *reinterpret_cast<const f32x4 *>(st + (g ? x.rdB1 : x.rdB) + i * 2048);
        else
            f.b[i] = *reinterpret_cast<const typename F::BV *>(st + x.rdB + (8 * g + i) * (BN * 4));
    }
}

// The MFMAs of group `cur`: the reads of `nxt` go out after MFMAs 0, 2, ..
// (well ahead of their use), and (if loads) this wave's LDS-direct loads
// of a later tile after the load slots.  sched_barrier(0) pins that order.
// 64 x 64 tiles (one 32 x 32 block per wave): odd K steps accumulate into
// acc_odd, so consecutive MFMAs are independent instead of one dependent
// chain (added to acc after the K loop); other tiles leave acc_odd unused.
template <int BM, int BN, int kW, bool TA, bool TB>
__device__ __forceinline__ void mfma_phase_f32(f32x16 (&acc)[BM / 64][BN / 64], f32x16 &acc_odd,
                                               const FragG<BM, BN, TA, TB> &cur,
                                               FragG<BM, BN, TA, TB> &nxt, const float *rstage,
                                               const DCtx<BM, BN, kW, TA, TB> &x, int g_next,
                                               uint32_t lstage, int64_t kload, bool loads)
{
    using T = DTile<BM, BN, kW, TA, TB>;
#pragma unroll
    for (int q = 0; q < T::kQ; ++q) {
        const int j = q / (T::kMB * T::kNB), mb = (q / T::kNB) % T::kMB, nb = q % T::kNB;
        if constexpr (BM == 64 && BN == 64) {
            f32x16 &a = (q & 1) ? acc_odd : acc[0][0];
            a = __builtin_amdgcn_mfma_f32_32x32x2f32(cur.av(0, j), cur.bv(j, 0), a, 0, 0, 0);
        } else {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur.av(mb, j), cur.bv(j, nb),
                                                                acc[mb][nb], 0, 0, 0);
        }
        const bool rd = T::kReadEveryOther ? (q < 2 * T::kReads && (q & 1) == 0) : q < T::kReads;
        if constexpr (T::kSpreadLoads) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (T::kSpreadReads) {
#pragma unroll
                for (int r = 0; r < T::kReads; ++r)
                    if (r * T::kQ / T::kReads == q) read_one(nxt, rstage, x, g_next, r);
            } else {
                if (rd) read_one(nxt, rstage, x, g_next, q);
            }
            if (loads) {
#pragma unroll
                for (int l = 0; l < T::kPerTile; ++l)
                    if (l * T::kQ / T::kPerTile == q) load_one(x, lstage, kload, l);
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            const bool ld = loads && q >= T::kLoadQ0 &&
                            q < T::kLoadQ0 + T::kLoadStep * T::kPerTile &&
                            (q - T::kLoadQ0) % T::kLoadStep == 0;
            if (rd || ld) {
                __builtin_amdgcn_sched_barrier(0);
                if (rd) read_one(nxt, rstage, x, g_next, T::kReadEveryOther ? q >> 1 : q);
                if (ld) load_one(x, lstage, kload, (q - T::kLoadQ0) / T::kLoadStep);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Row epilogue of the 128-row tiles: the accumulators go into the idle LDS
// ring as rows (16-byte chunks XOR-permuted by bit 2 of the row so the two
// half-waves' rows 4 apart use different banks), then the work-group writes
// C as 16-byte streaming stores of whole rows, one pass (the ring holds the
// tile).  In the library, on the table's choices: GPT QKV (128 x 64) 112.8
// -> 111.4 us, MLP-up (128 x 128) 145.8 -> 144.2, MLP-down unchanged; the
// 128 x 128 tile on QKV 125.6 -> 118.6.  The 256 x 256 tile, whose lanes
// already hold four consecutive columns, keeps its direct 16-byte stores
// (the staging cost it 1.3%).  Needs C 16-byte aligned with ldc and N
// multiples of 4.
template <int BM, int BN, int kW, bool TA = false, bool TB = false>
__device__ __forceinline__ void store_c_rows_f32(const f32x16 (&acc)[BM / 64][BN / 64],
                                                 float *lf, float *__restrict__ C, int64_t ldc,
                                                 int64_t M, int64_t N, int64_t m0, int64_t n0,
                                                 int wm, int wn, int lane)
{
    using T = DTile<BM, BN, kW>;
    constexpr int MB = T::kMB, NB = T::kNB, WN = BN / 2;
    constexpr int kHalf = MB * 32;           // rows per wave
    constexpr int kChunks = BN / 4;          // 16-byte chunks per row
    static_assert(BM * BN <= DSTAGES * T::kStageFloats, "the ring holds the tile");
    static_assert(BM * kChunks % kThreads == 0, "whole chunks per thread");
    const int h = lane >> 5, c = lane & 31;
    // every wave's loads landed and reads done: the ring is free
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = TB ? wn * WN + nb * 32 + c : wn * WN + NB * c + nb;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * h + (r & 3);
                const int lrow = wm * kHalf + (TA ? MB * i + mb : mb * 32 + i);
                const int swz = kChunks >= 16 ? (((lrow >> 2) & 1) << 3) : 0;
                lf[lrow * BN + (((col >> 2) ^ swz) << 2) + (col & 3)] = acc[mb][nb][r];
            }
        }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < BM * kChunks / kThreads; ++i) {
        const int q = threadIdx.x + kThreads * i;
        const int lrow = q / kChunks, chunk = q % kChunks;
        const int swz = kChunks >= 16 ? (((lrow >> 2) & 1) << 3) : 0;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(lf + lrow * BN + ((chunk ^ swz) << 2));
        const int64_t row = m0 + lrow, col = n0 + 4 * chunk;
        if (row < M && col < N) store_c_stream(reinterpret_cast<f32x4 *>(C + row * ldc + col), v);
    }
}

// kBatch: a batch of products (stride_a, stride_b, stride_c elements apart)
// runs as one grid of (product, tile) work-groups.  A single product keeps
// the plain tile map (no division by the tile count, no pointer offsets).
// kSplit2 (a single product, kW == 16): two work-groups per tile, the first
// and the second half of the K tiles, each adding its sums into C (set to
// -0.0 beforehand) with one atomic add per element: p0 + p1 rounded once in
// either order, so the result repeats exactly from run to run.
template <int BM, int BN, int kW, bool kRowsC = false, bool TA = false, bool TB = false,
          bool kBatch = false, bool kSplit2 = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DTile<BM, BN, kW>::kPerCU, DTile<BM, BN, kW>::kPerCU)))
void mfma_f32_direct_kernel(int64_t M, int64_t N, int64_t K, const float *__restrict__ A,
                            int64_t lda, const float *__restrict__ B, int64_t ldb,
                            float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n,
                            int cvec, int64_t sa, int64_t sb, int64_t sc, int64_t batch)
{
    using T = DTile<BM, BN, kW, TA, TB>;
    constexpr int MB = T::kMB, NB = T::kNB, WM = BM / 2, WN = BN / 2;
    static_assert(!kSplit2 || (kW == 16 && !kBatch && !kRowsC), "two-way K split: aligned K, one product");
    __shared__ __attribute__((aligned(1024))) float lds[DSTAGES * T::kStageFloats];

    int64_t m0, n0, kt0 = 0, kt_count = K / DBK;   // this work-group's K tiles
    if constexpr (kSplit2) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, 2, kGroup);
        m0 = t.tm * BM;
        n0 = t.tn * BN;
        const int64_t mid = (kt_count + 1) / 2;
        kt0 = t.b ? mid : 0;
        kt_count = t.b ? kt_count - mid : mid;
    } else if constexpr (kBatch) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
        A += t.b * sa;
        B += t.b * sb;
        C += t.b * sc;
        m0 = t.tm * BM;
        n0 = t.tn * BN;
    } else {
        const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
        m0 = t.tm * BM;
        n0 = t.tn * BN;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, c = lane & 31;

    DCtx<BM, BN, kW, TA, TB> x;
    x.wave = wave;
    x.lds0 = lds_offset(lds);
    // Rows of K start at the tile's first row and step 16 floats per tile;
    // rows of M or N start at the tile's first column and step 16 rows.
    x.abase = reinterpret_cast<const char *>(TA ? A + m0 : A + m0 * lda);
    x.bbase = reinterpret_cast<const char *>(TB ? B + n0 * ldb : B + n0);
    x.a_kstride = TA ? DBK * lda * 4 : DBK * 4;
    x.b_kstride = TB ? DBK * 4 : DBK * ldb * 4;
    // Stated wave-uniform here, so that the per-tile load bases stay in
    // scalar registers (without it the compiler computed them with vector
    // instructions and a readfirstlane per load group: 151.4 -> 148.8
    // TFLOP/s at 8192^3).
    if constexpr (kSplit2) {   // tile kt of this work-group is tile kt0 + kt of the product
        x.abase += kt0 * x.a_kstride;
        x.bbase += kt0 * x.b_kstride;
    }
    x.abase = static_cast<const char *>(uniform_ptr(x.abase));
    x.bbase = static_cast<const char *>(uniform_ptr(x.bbase));
    x.a_kstride = uniform_i64(x.a_kstride);
    x.b_kstride = uniform_i64(x.b_kstride);
    // p: the kW-byte unit of the stage's A (or B) region this lane fills;
    // the element(s) it holds follow from the layout.
#pragma unroll
    for (int i = 0; i < T::kAInst; ++i) {
        const int p = (wave * T::kAInst + i) * 64 + lane;
        if constexpr (TA) {
            // 16 rows of BM floats: row k, chunk slot p % (BM / 4); columns
            // past M re-fetch the last full chunk (M % 4 == 0 here)
            const int row = p / (BM / 4), slot = p % (BM / 4);
            const int lc = T::kASwz ? slot ^ b_swz8(row) : slot;
            const int64_t col = (m0 + 4 * lc < M) ? 4 * lc : M - 4 - m0;
            x.a_voff[i] = static_cast<uint32_t>((row * lda + col) * 4);
            continue;
        }
        int row, kk;
        if constexpr (kW == 16) {
            row = p >> 2;
            kk = 4 * ((p & 3) ^ a_swz4(row));
        } else {
            row = p >> 4;
            kk = 4 * (((p >> 2) & 3) ^ a_swz4(row)) + (p & 3);
        }
        const int64_t r = (m0 + row < M) ? row : M - 1 - m0;
        x.a_voff[i] = static_cast<uint32_t>((r * lda + kk) * 4);
    }
#pragma unroll
    for (int i = 0; i < T::kBInst; ++i) {
        const int p = (wave * T::kBInst + i) * 64 + lane;
        if constexpr (TB) {
            // BN rows of 16 floats, laid out as A's: row n, chunk slot p & 3
            const int row = p >> 2;
            const int kk = 4 * ((p & 3) ^ a_swz4(row));
            const int64_t r = (n0 + row < N) ? row : N - 1 - n0;
            x.b_voff[i] = static_cast<uint32_t>((r * ldb + kk) * 4);
            continue;
        }
        int64_t row, col;
        if constexpr (kW == 16) {
            row = p / T::kBChunksPerRow;
            const int slot = p % T::kBChunksPerRow;
            const int lc = T::kBSwz ? slot ^ b_swz8(static_cast<int>(row)) : slot;
            col = (n0 + 4 * lc < N) ? 4 * lc : N - 4 - n0;
        } else {
            row = p / BN;
            int cl = p % BN;
            if constexpr (T::kBSwz) cl = 4 * ((cl >> 2) ^ b_swz8(static_cast<int>(row))) + (cl & 3);
            col = (n0 + cl < N) ? cl : N - 1 - n0;
        }
        x.b_voff[i] = static_cast<uint32_t>((row * ldb + col) * 4);
    }
    // Rows this lane reads are wm*WM + 32*idx + c: their swizzle is a_swz4(c).
    const int swz = a_swz4(c);
    if constexpr (TA) {
        // k rows 4h + 8g + j, columns MB c .. MB c + MB - 1 of the wave's rows
        if constexpr (T::kASwz) {
            const int m = wm * WM + c;
            x.rdA0 = 4 * h * (BM * 4) + ((((m >> 2) ^ (h << 3)) << 2) + (m & 3)) * 4;
        } else {
            x.rdA0 = 4 * h * (BM * 4) + (wm * WM + MB * c) * 4;
        }
        x.rdA1 = x.rdA0;
    } else {
        x.rdA0 = (wm * WM + c) * DBK * 4 + (((0 + h) ^ swz) << 4);
        x.rdA1 = (wm * WM + c) * DBK * 4 + (((2 + h) ^ swz) << 4);
    }
    if constexpr (TB) {
        // rows wn*WN + 32*idx + c of the stage's B region, as for A
        x.rdB = BM * DBK * 4 + (wn * WN + c) * DBK * 4 + (((0 + h) ^ swz) << 4);
        x.rdB1 = BM * DBK * 4 + (wn * WN + c) * DBK * 4 + (((2 + h) ^ swz) << 4);
    } else if constexpr (T::kBSwz) {
        // rows this lane reads are 4h + 8g + j: bit 2 is h
        const int n = wn * WN + c;
        x.rdB = BM * DBK * 4 + 4 * h * (BN * 4) + ((((n >> 2) ^ (h << 3)) << 2) + (n & 3)) * 4;
    } else {
        x.rdB = BM * DBK * 4 + 4 * h * (BN * 4) + (wn * WN + NB * c) * 4;
    }

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    f32x16 acc_odd;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_odd[r] = 0.f;

    const int64_t ktiles = kt_count;
    auto stage = [&](int64_t kt) { return lds + (kt % DSTAGES) * T::kStageFloats; };
    auto lstage = [&](int64_t kt) {
        return x.lds0 + static_cast<uint32_t>(kt % DSTAGES) * T::kStageFloats * 4;
    };
    auto kclamp = [&](int64_t kt) { return kt < ktiles ? kt : ktiles - 1; };

    FragG<BM, BN, TA, TB> f0, f1;
    // The aligned kernels take K % 16 == 0 and K > 0 only; the narrow one
    // may have no full tile (K < 16), then only the tail below runs.
    if (kW == 16 || ktiles > 0) {
        // Prologue: tiles 0..2 in flight (re-fetching the last tile past
        // the end), wait for tile 0, read its first group.
#pragma unroll
        for (int s = 0; s < DSTAGES - 1; ++s)
#pragma unroll
            for (int l = 0; l < T::kPerTile; ++l) load_one(x, lstage(s), kclamp(s), l);
        wait_lds_vm_barrier<(DSTAGES - 2) * T::kPerTile>();

#pragma unroll
        for (int i = 0; i < T::kReads; ++i) read_one(f0, stage(0), x, 0, i);

        // Tile kt: MFMAs on group 0 with group 1's reads and the loads of
        // tile kt + 3 slotted in (its stage was last read in tile kt - 1,
        // finished by every wave before the previous barrier) | wait for tile
        // kt + 1 and for this wave's reads, barrier | MFMAs on group 1 with
        // the reads of group 0 of tile kt + 1 (in the last tile: reads of a
        // landed stage, unused).
        for (int64_t kt = 0; kt < ktiles; ++kt) {
            const int64_t nxt = kt + DSTAGES - 1;
            mfma_phase_f32(acc, acc_odd, f0, f1, stage(kt), x, 1, lstage(nxt), kclamp(nxt), true);
            wait_lds_vm_barrier<(DSTAGES - 2) * T::kPerTile>();
            mfma_phase_f32(acc, acc_odd, f1, f0, stage(kt + 1), x, 0, 0, 0, false);
        }
        // No LDS-direct load may still be writing LDS when the work-group
        // ends or stage 0 is refilled below.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (kW == 4) {
        // K tail (K % 16 columns of A, rows of B): written into stage 0 by
        // ordinary loads and LDS stores, zero past K, in the same layout;
        // rows of A past M and columns of B past N repeat the last valid
        // one as in the loads above.
        const int64_t k0 = ktiles * DBK;
        if (k0 < K) {
            wait_lds_vm_barrier<0>();        // every wave done with every stage
            for (int p = threadIdx.x; p < BM * DBK; p += kThreads) {
                const int row = p >> 4;
                const int64_t k = k0 + 4 * (((p >> 2) & 3) ^ a_swz4(row)) + (p & 3);
                const int64_t r = (m0 + row < M) ? m0 + row : M - 1;
                lds[p] = (k < K) ? A[r * lda + k] : 0.f;
            }
            for (int p = threadIdx.x; p < DBK * BN; p += kThreads) {
                const int row = p / BN;
                int c4 = p % BN;
                if constexpr (T::kBSwz) c4 = 4 * ((c4 >> 2) ^ b_swz8(row)) + (c4 & 3);
                const int64_t k = k0 + row;
                const int64_t cl = n0 + c4;
                lds[BM * DBK + p] = (k < K) ? B[k * ldb + (cl < N ? cl : N - 1)] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < T::kReads; ++i) read_one(f0, stage(0), x, 0, i);
            mfma_phase_f32(acc, acc_odd, f0, f1, stage(0), x, 1, 0, 0, false);
            mfma_phase_f32(acc, acc_odd, f1, f0, stage(0), x, 0, 0, 0, false);
        }
    }

    if constexpr (BM == 64 && BN == 64) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][0][r] += acc_odd[r];
    }
    if constexpr (kRowsC) {
        store_c_rows_f32<BM, BN, kW, TA, TB>(acc, lds, C, ldc, M, N, m0, n0, wm, wn, lane);
        return;
    }
    if constexpr (kSplit2) {
        // the epilogue's mapping below, one atomic add per element
        const int64_t col0 = n0 + wn * WN + (TB ? c : NB * c);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * h + (r & 3);
                const int64_t row = m0 + wm * WM + (TA ? MB * i + mb : mb * 32 + i);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int64_t col = col0 + (TB ? 32 * nb : nb);
                    if (row < M && col < N) unsafeAtomicAdd(C + row * ldc + col, acc[mb][nb][r]);
                }
            }
        return;
    }
    // Epilogue: register r of block (mb, nb) in lane (h, c) is the MFMA
    // output row i = 8*(r/4) + 4*h + r%4, which is row 32*mb + i of the
    // wave's piece (MB*i + mb with a transposed A), and column NB*c + nb
    // (32*nb + c with a transposed B).
    const int64_t col = n0 + wn * WN + (TB ? c : NB * c);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * h + (r & 3);
            const int64_t row = m0 + wm * WM + (TA ? MB * i + mb : mb * 32 + i);
            if (row >= M) continue;
            float *p = C + row * ldc + col;
            if constexpr (TB) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    if (col + 32 * nb < N) store_c_stream(p + 32 * nb, acc[mb][nb][r]);
                continue;
            }
            typename DVec<NB>::T v;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) v[nb] = acc[mb][nb][r];
            if (cvec && col + NB <= N) {
                store_c_stream(reinterpret_cast<typename DVec<NB>::T *>(p), v);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    if (col + nb < N) store_c_stream(p + nb, static_cast<float>(v[nb]));
            }
        }
}

}  // namespace

hipError_t launch_mfma_f32(const Problem &p, hipStream_t s) { return launch_tiles<256, 256>(p, s); }
hipError_t launch_mfma_f32_128(const Problem &p, hipStream_t s) { return launch_tiles<128, 128>(p, s); }

}  // namespace mi355gemm

namespace mi355gemm {

bool supports_mfma_f32_direct(const Problem &p)
{
    const auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    // Lane offsets of the scalar-base loads are 32-bit byte offsets within a
    // panel of up to 256 rows of K (A as written, B transposed) or 16 rows
    // of M or N (A transposed, B as written).  A factor stored with rows of
    // M or N has its last chunk re-fetched past the edge, so that dimension
    // is a multiple of 4.
    const int64_t krows = int64_t(1) << 22, mnrows = int64_t(1) << 26;
    const bool a_ok = p.ta ? p.M % 4 == 0 && p.lda < mnrows : p.lda < krows;
    const bool b_ok = p.tb ? p.ldb < krows : p.N % 4 == 0 && p.ldb < mnrows;
    // K > 0: the prologue loads the first tiles unconditionally (K = 0 is
    // written by the fill kernel, or by another general kernel).
    return p.K > 0 && p.K % 16 == 0 && p.lda % 4 == 0 && p.ldb % 4 == 0 && p.sa % 4 == 0 &&
           p.sb % 4 == 0 && al(p.A) && al(p.B) && a_ok && b_ok;
}

// The narrow variant takes any fp32 layout of untransposed factors: 4-byte
// loads need only element alignment, and the K tail is zero-filled.  Lane
// offsets are 32-bit byte offsets within a 128-row panel of A and a 16-row
// panel of B.
bool supports_mfma_f32_narrow(const Problem &p)
{
    return !p.ta && !p.tb && p.lda < (int64_t(1) << 23) && p.ldb < (int64_t(1) << 26);
}

namespace {

template <int BM, int BN, int kW, bool TA, bool TB, bool kBatch = true>
hipError_t launch_direct_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    const int cvec =
        (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && p.ldc % 4 == 0 && p.sc % 4 == 0;
    const auto *A = static_cast<const float *>(p.A);
    const auto *B = static_cast<const float *>(p.B);
    const dim3 grid(static_cast<uint32_t>(tm * tn * p.batch));
    if constexpr (BM == 128) {
        if (cvec && p.N % 4 == 0) {
            hipLaunchKernelGGL((mfma_f32_direct_kernel<BM, BN, kW, true, TA, TB, kBatch>), grid,
                               dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C,
                               p.ldc, tm, tn, cvec, p.sa, p.sb, p.sc, p.batch);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((mfma_f32_direct_kernel<BM, BN, kW, false, TA, TB, kBatch>), grid, dim3(kThreads),
                       0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm, tn, cvec, p.sa,
                       p.sb, p.sc, p.batch);
    return hipGetLastError();
}

template <int BM, int BN, int kW>
hipError_t launch_direct(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    const bool ok = kW == 16 ? supports_mfma_f32_direct(p) : supports_mfma_f32_narrow(p);
    if (tm * tn * p.batch > kMaxBlocks || !ok) return hipErrorInvalidValue;
    if constexpr (kW == 16) {
        if (p.ta && p.tb) return launch_direct_layout<BM, BN, kW, true, true>(p, s, tm, tn);
        if (p.ta) return launch_direct_layout<BM, BN, kW, true, false>(p, s, tm, tn);
        if (p.tb) return launch_direct_layout<BM, BN, kW, false, true>(p, s, tm, tn);
    }
    if (p.batch != 1) return launch_direct_layout<BM, BN, kW, false, false>(p, s, tm, tn);
    return launch_direct_layout<BM, BN, kW, false, false, false>(p, s, tm, tn);
}

}  // namespace

hipError_t launch_mfma_f32_direct(const Problem &p, hipStream_t s) { return launch_direct<256, 256, 16>(p, s); }
hipError_t launch_mfma_f32_direct128(const Problem &p, hipStream_t s) { return launch_direct<128, 128, 16>(p, s); }
hipError_t launch_mfma_f32_narrow128(const Problem &p, hipStream_t s) { return launch_direct<128, 128, 4>(p, s); }
hipError_t launch_mfma_f32_direct128x64(const Problem &p, hipStream_t s) { return launch_direct<128, 64, 16>(p, s); }
hipError_t launch_mfma_f32_narrow128x64(const Problem &p, hipStream_t s) { return launch_direct<128, 64, 4>(p, s); }
hipError_t launch_mfma_f32_direct64(const Problem &p, hipStream_t s) { return launch_direct<64, 64, 16>(p, s); }

namespace {

template <bool TA, bool TB>
void launch_direct64x2_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    hipLaunchKernelGGL((mfma_f32_direct_kernel<64, 64, 16, false, TA, TB, false, true>),
                       dim3(static_cast<uint32_t>(2 * tm * tn)), dim3(kThreads), 0, s, p.M, p.N, p.K,
                       static_cast<const float *>(p.A), p.lda, static_cast<const float *>(p.B),
                       p.ldb, p.C, p.ldc, tm, tn, 0, p.sa, p.sb, p.sc, p.batch);
}

}  // namespace

bool supports_mfma_f32_direct64x2(const Problem &p)
{
    return p.batch == 1 && p.K >= 2 * 16 && supports_mfma_f32_direct(p);
}

// The 64 x 64 LDS-direct tile with the K tiles split over two work-groups
// per tile (small outputs over a long K: every CU streams operands); C is
// first set to -0.0 by a fill kernel on the same stream.
hipError_t launch_mfma_f32_direct64x2(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + 63) / 64, tn = (p.N + 63) / 64;
    if (2 * tm * tn > kMaxBlocks || !supports_mfma_f32_direct64x2(p)) return hipErrorInvalidValue;
    const hipError_t e = launch_fill(p, -0.0f, s);   // the identity of fp32 addition
    if (e != hipSuccess) return e;
    if (p.ta && p.tb) launch_direct64x2_layout<true, true>(p, s, tm, tn);
    else if (p.ta) launch_direct64x2_layout<true, false>(p, s, tm, tn);
    else if (p.tb) launch_direct64x2_layout<false, true>(p, s, tm, tn);
    else launch_direct64x2_layout<false, false>(p, s, tm, tn);
    return hipGetLastError();
}
hipError_t launch_mfma_f32_narrow64(const Problem &p, hipStream_t s) { return launch_direct<64, 64, 4>(p, s); }

}  // namespace mi355gemm
