// bf16-in / fp32-accumulate matrix-core family: v_mfma_f32_32x32x16_bf16,
// and v_mfma_f32_16x16x32_bf16 on the 256 x 256 LDS-direct tile (further
// below); the 8-bit kernels share the staging.
//
// The matrix-instruction rung of the kernel ladder ("Bare Metal Bard", page
// 1, first paragraph) with bf16 operands (vidyal.ai Part 6, "Tensor Cores":
// what one instruction computes, feeding it from shared memory without bank
// conflicts, and what BF16 costs in accuracy).  A bf16 x bf16 product is
// exact in fp32, so the only rounding is the fp32 accumulation.
//
// The register-staged kernel (mfma_bf16_kernel, any layout the others
// refuse):
//   * block tile 256 x 256, K step 64; 4 wave64s in a 2 x 2 grid, each
//     owning 128 x 128 of C as 4 x 4 MFMA blocks of 32 x 32 (256 fp32
//     accumulators per lane);
//   * global -> registers with 128-bit loads (8 bf16), registers -> LDS
//     after the current tile's math, two LDS stages, one barrier per step;
//   * A operand: lane (h, c) needs row c of a 32-row block and k = 8h..8h+7
//     of a 16-wide K slice, which is one 16-byte chunk of a row-major A tile
//     (ds_read_b128).  The eight chunks of each LDS row are XOR-permuted by a
//     row hash so that the rows of one read land in distinct banks;
//   * B operand: lane (h, c) needs column c and the same eight k.  B is
//     row-major (columns contiguous), so it stays that way in LDS and is read
//     with gfx950's transposing LDS load (ds_read_b64_tr_b16): in each group
//     of 16 lanes, lane s points at 4 consecutive columns of row s/4 and the
//     hardware hands lane i the column i of those four rows.  Two such reads
//     give the eight k.  The 16-byte chunks of each B row are XOR-permuted by
//     (row mod 4) so the four rows of one read fall in distinct banks;
//   * ragged edges: rows past M, columns past N and k past K load as zeros;
//     C is stored with row and column masks.
#include "gemm_internal.h"
#include "tile_map.h"

namespace mi355gemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kAChunks = BM * BK / 8 / kThreads;   // 8
constexpr int kBChunks = BK * BN / 8 / kThreads;   // 8
constexpr int kGroup = 4;

// Chunk permutation of an A row in LDS: chunk c of row r is stored at
// c ^ a_swz(r).  Rows of 8 chunks (128 bytes, K step 64): (r >> 1) & 7;
// rows of 4 chunks (64 bytes, K step 32): (r >> 2) & 3.  Both were measured
// conflict-free on gfx950 for the operand read (32 consecutive rows at one
// logical chunk per half-wave) with a one-pattern microbenchmark
// (SQ_LDS_BANK_CONFLICT); e.g. (r + r/8) mod 8 and (r>>1)^(r>>3) are 2-way
// conflicted, unswizzled layouts 4- to 8-way.
template <int kChunks>
__device__ __forceinline__ int a_swz(int row)
{
    if constexpr (kChunks == 8) return (row >> 1) & 7;
    else return (row >> 2) & 3;
}

// B rows hold 32 chunks.  A transposing read by 16 lanes touches two
// adjacent chunks of four consecutive rows; a half-wave touches four
// adjacent chunks of the same rows.  XOR masks {0, 4, 10, 14} for row mod 4
// put both sets in distinct bank slots (8 slots of 16 bytes and 16 slots of
// 16 bytes respectively).
__device__ __forceinline__ int b_swz(int row)
{
    const int r = row & 3;
    return ((r >> 1) << 1) | ((r & 1) << 2) | ((r >> 1) << 3);
}

// The same for rows of kCh 16-byte chunks in the LDS-direct tiles: 16 or
// more chunks take b_swz; rows of 8 chunks (128 bytes, a 64-wide tile) put
// rows r and r + 1 in different halves of the 256-byte bank window already,
// so only rows two apart collide, and XOR mask 4 for rows 2 and 3 (mod 4)
// separates both the 16-lane pairs of chunks and the half-wave's four.
template <int kCh>
__device__ __forceinline__ int b_swzc(int row)
{
    if constexpr (kCh == 8) return ((row >> 1) & 1) << 2;
    else return b_swz(row);
}

struct Frag {
    u16x8 a[kAChunks];
    u16x8 b[kBChunks];
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

template <bool kVec>
__device__ __forceinline__ void load_tile(Frag &f, const uint16_t *__restrict__ A, int64_t lda,
                                          const uint16_t *__restrict__ B, int64_t ldb, int64_t M,
                                          int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                          bool a_full, bool b_full)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 3, c = p & 7;
        f.a[i] = load8<kVec>(A, lda, m0 + row, k0 + 8 * c, M, K, a_full);
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 5, c = p & 31;
        f.b[i] = load8<kVec>(B, ldb, k0 + row, n0 + 8 * c, K, N, b_full);
    }
}

__device__ __forceinline__ void store_tile(const Frag &f, uint16_t *As, uint16_t *Bs)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 3, c = p & 7;
        *reinterpret_cast<u16x8 *>(As + row * BK + ((c ^ a_swz<8>(row)) << 3)) = f.a[i];
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 5, c = p & 31;
        *reinterpret_cast<u16x8 *>(Bs + row * BN + ((c ^ b_swz(row)) << 3)) = f.b[i];
    }
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 read_tr(const uint16_t *lds_elem)
{
    auto p = (lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)(lds_elem));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

template <int kBK>
__device__ __forceinline__ void compute_tile(f32x16 (&acc)[4][4], const uint16_t *As,
                                             const uint16_t *Bs, int wm, int wn, int lane)
{
    const int h = lane >> 5, c = lane & 31;
    const int i = lane & 15, nhalf = (lane >> 4) & 1;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int row = wm * 128 + mb * 32 + c;
            const u16x8 v = *reinterpret_cast<const u16x8 *>(
                As + row * kBK + (((2 * s + h) ^ a_swz<kBK / 8>(row)) << 3));
            a[mb] = __builtin_bit_cast(bf16x8, v);
        }
        const int k_lo = 16 * s + 8 * h + (i >> 2);   // row of the first read; +4 for the second
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = wn * 128 + nb * 32 + nhalf * 16 + 4 * (i & 3);
            const int chunk = n >> 3, within = n & 7;
            const int sw = b_swz(k_lo);                  // same for k_lo + 4
            const uint16_t *p0 = Bs + k_lo * BN + ((chunk ^ sw) << 3) + within;
            const uint16_t *p1 = p0 + 4 * BN;
            const bf16x4 lo = read_tr(p0), hi = read_tr(p1);
            b[nb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb],
                                                                       0, 0, 0);
    }
}

// Epilogue for a wave owning MB x NB blocks (a 32 MB x 32 NB piece of the
// tile at wave position (wm, wn)): register r of block (mb, nb) in lane
// (h, c) is C row 8*(r/4) + 4*h + r%4, column c of that 32 x 32 block.
template <int MB, int NB>
__device__ __forceinline__ void store_c(const f32x16 (&acc)[MB][NB], float *__restrict__ C,
                                        int64_t ldc, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                        int wm, int wn, int lane)
{
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t col = n0 + wn * 32 * NB + nb * 32 + c;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 32 * MB + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) store_c_stream(C + row * ldc + col, acc[mb][nb][r]);
            }
        }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_bf16_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A, int64_t lda,
                      const uint16_t *__restrict__ B, int64_t ldb, float *__restrict__ C,
                      int64_t ldc, int64_t tiles_m, int64_t tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BK * BN];

    const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool a_rows_full = m0 + BM <= M;
    const bool b_cols_full = n0 + BN <= N;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = (K + BK - 1) / BK;
    Frag f;
    load_tile<kVec>(f, A, lda, B, ldb, M, N, K, m0, n0, 0, a_rows_full && BK <= K,
                    b_cols_full && BK <= K);
    store_tile(f, As[0], Bs[0]);
    __syncthreads();

    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < ktiles;
        if (more) {
            const int64_t k0 = (kt + 1) * BK;
            const bool kfull = k0 + BK <= K;
            load_tile<kVec>(f, A, lda, B, ldb, M, N, K, m0, n0, k0, a_rows_full && kfull,
                            b_cols_full && kfull);
        }
        compute_tile<BK>(acc, As[cur], Bs[cur], wm, wn, lane);
        if (more) store_tile(f, As[cur ^ 1], Bs[cur ^ 1]);
        __syncthreads();
    }

    store_c(acc, C, ldc, M, N, m0, n0, wm, wn, lane);
}


// ---------------------------------------------------------------------------
// Direct variants (128 x 128 tile, two work-groups per CU, and 64 x 64 here;
// the 256 x 256 tile, one work-group per CU, shares this staging but runs
// the 16 x 16 x 32 instruction, further below): global -> LDS
// with gfx950's LDS-direct 128-bit loads (global_load_lds_dwordx4), no
// register staging and no LDS write instructions, into a ring of four
// 32-wide K stages so that the loads for tile t + 3 are in flight while tile
// t is multiplied.  One such load per wave writes 1 KiB of LDS at
// consecutive 16-byte slots in lane order; choosing which global chunk each
// lane fetches realises the same swizzled layouts as above.  Operand
// fragments are read one 16-wide K slice ahead (across the tile boundary),
// each read and each load slotted between MFMAs; one barrier per tile.  Four
// waves in a 2 x 2 grid, each owning (TM/2) x (TN/2) of C as MB x NB blocks
// of 32 x 32.
//
// Instruction economy: the loads use the scalar-base form (wave-uniform base
// advanced once per tile + a fixed 32-bit lane offset), the reads use a few
// lane bases plus immediate offsets (the swizzles of the rows a lane reads
// depend only on the lane), and the loads past the last tile re-fetch the
// last tile into a stage nobody reads again instead of being branched
// around.
//
// Shapes: K a multiple of 32 (and K > 0), 16-byte aligned A and B with lda
// and ldb multiples of 8, lane offsets within 32 bits: a factor stored with
// rows of K (A as written, B transposed) within 256 stored rows, one stored
// with rows of M or N (A transposed, B as written) within 32 stored rows,
// and that dimension a multiple of 8.  Rows of A past M and columns of B
// past N are fetched from the last valid row / chunk (their products land
// only in rows and columns of C that are not stored).  The same kernels run
// fp16 operands with the fp16 instruction, and strided batches as one grid.

constexpr int DBK = 32;
constexpr int DSTAGES = 4;

// TA / TB: A stored K x M / B stored N x K.  Each factor is staged in its
// stored orientation: rows of K (A as written, B transposed) are read with
// 16-byte reads, rows of M or N (A transposed, B as written) with the
// transposing reads (two per 32-wide block and slice).
template <int TM, int TN, bool TA = false, bool TB = false>
struct DTile {
    static constexpr int kMB = TM / 64, kNB = TN / 64;         // blocks per wave
    static constexpr int kAInst = TM * DBK * 2 / 1024 / 4;     // LDS-direct loads per wave per tile (A)
    static constexpr int kBInst = DBK * TN * 2 / 1024 / 4;     // ... (B)
    static constexpr int kPerTile = kAInst + kBInst;
    static constexpr int kStageElems = TM * DBK + DBK * TN;    // bf16 elements per stage
    static constexpr int kBChunks = TN / 8;                    // 16-byte chunks per B row
    static constexpr int kQ = kMB * kNB;                       // MFMAs per 16-wide K slice
    static constexpr int kReads = (TA ? 2 * kMB : kMB) + (TB ? kNB : 2 * kNB);   // reads per slice
    // Work-groups per CU the LDS ring allows: 1 (256 x 256), 2 (128 x 128).
    static constexpr int kPerCU = 160 * 1024 / (DSTAGES * kStageElems * 2);
    static_assert((DSTAGES - 2) * kPerTile <= 63, "vmcnt is six bits");
};

// One LDS-direct 128-bit load as inline assembly, scalar-base form: lane i
// reads 16 bytes at sbase + voff and they land at LDS byte M0 + 16 i.  The
// compiler's wait-count pass does not see these loads (it would drain them
// before every LDS read); the kernel waits for them itself with exact
// counts.  M0 is declared clobbered (nothing else in these kernels keeps a
// value in it); the s_nop covers the M0-write hazard.
__device__ __forceinline__ void lds_direct_load16(uint32_t voff, const void *sbase, uint32_t m0v)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) void *)(p)));
}

// Everything a wave needs to address its loads and reads.
// kF16: the 16-bit patterns are IEEE binary16 (v_mfma_f32_32x32x16_f16)
// rather than bf16; staging, reads and layouts are the same bits either way.
template <int TM, int TN, bool TA = false, bool TB = false, bool kF16 = false>
struct DCtx {
    using T = DTile<TM, TN, TA, TB>;
    uint32_t a_voff[T::kAInst], b_voff[T::kBInst];   // lane offsets (bytes) of each load
    const char *abase, *bbase;                       // tile (k = 0) bases, wave-uniform
    int64_t a_kstride, b_kstride;                    // bytes per K step
    uint32_t lds0;                                   // LDS byte address of stage 0
    int wave;
    uint32_t rdA[TA ? T::kMB : 2];                   // lane read offsets: A, per K slice (per block)
    uint32_t rdB[TB ? 2 : T::kNB];                   // lane read offsets: B, per block (per K slice)
};

template <int TM, int TN, bool TA, bool TB, bool kF16>
__device__ __forceinline__ void load_one(const DCtx<TM, TN, TA, TB, kF16> &x, uint32_t stage_lds,
                                         int64_t kt, int l)
{
    using T = DTile<TM, TN, TA, TB>;
    if (l < T::kAInst)
        lds_direct_load16(x.a_voff[l], x.abase + kt * x.a_kstride,
                          stage_lds + (x.wave * T::kAInst + l) * 1024);
    else
        lds_direct_load16(x.b_voff[l - T::kAInst], x.bbase + kt * x.b_kstride,
                          stage_lds + TM * DBK * 2 + (x.wave * T::kBInst + l - T::kAInst) * 1024);
}

// Operand fragments of one 16-wide K slice for a wave's MB x NB MFMA blocks:
// A as one 8-element register quad per 32-row block, B as two 4-element
// halves (k 0-3 and 4-7 of the lane's eight) per 32-column block.
template <int TM, int TN, bool TA = false, bool TB = false>
struct Frag16 {
    static constexpr int kMB = TM / 64, kNB = TN / 64;
    // a (A as written) or alo / ahi (transposed); blo / bhi (B as written)
    // or b (transposed).  The members a layout does not use are never
    // touched and take no registers.
    bf16x8 a[kMB];
    bf16x4 alo[kMB], ahi[kMB];
    bf16x4 blo[kNB], bhi[kNB];
    bf16x8 b[kNB];
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ bf16x4 read_tr4(const char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t *)((__attribute__((address_space(3))) char *)(p)));
}

// Read j of slice s from the stage at `stage`.  A as written: j < MB is A
// block j (one 16-byte read); transposed: j < 2 MB is A block j / 2, lower /
// upper four k (transposing reads).  Then B: as written, block (j - nA) / 2,
// lower / upper four k; transposed, block j - nA (one 16-byte read).
template <int TM, int TN, bool TA, bool TB, bool kF16>
__device__ __forceinline__ void read_one(Frag16<TM, TN, TA, TB> &f, const uint16_t *stage,
                                         const DCtx<TM, TN, TA, TB, kF16> &x, int s, int j)
{
    using T = DTile<TM, TN, TA, TB>;
    constexpr int nA = TA ? 2 * T::kMB : T::kMB;
    const char *st = reinterpret_cast<const char *>(stage);
    if (j < nA) {
        if constexpr (TA) {
            const int mb = j >> 1, upper = j & 1;
            const bf16x4 v = read_tr4(st + x.rdA[mb] + s * (16 * TM * 2) + upper * (4 * TM * 2));
            if (upper) f.ahi[mb] = v;
            else f.alo[mb] = v;
        } else {
            const u16x8 v = *reinterpret_cast<const u16x8 *>(st + x.rdA[s] + j * 2048);
            f.a[j] = __builtin_bit_cast(bf16x8, v);
        }
    } else if constexpr (TB) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(st + x.rdB[s] + (j - nA) * 2048);
        f.b[j - nA] = __builtin_bit_cast(bf16x8, v);
    } else {
        const int nb = (j - nA) >> 1, upper = (j - nA) & 1;
        const bf16x4 v = read_tr4(st + x.rdB[nb] + s * (16 * TN * 2) + upper * (4 * TN * 2));
        if (upper) f.bhi[nb] = v;
        else f.blo[nb] = v;
    }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// One 32 x 32 x 16 MFMA on 16-bit patterns: bf16, or fp16 when kF16.
template <bool kF16>
__device__ __forceinline__ f32x16 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool kF16, int TM, int TN, bool TA, bool TB>
__device__ __forceinline__ void mfma_one(f32x16 (&acc)[TM / 64][TN / 64],
                                         const Frag16<TM, TN, TA, TB> &f, int q)
{
    constexpr int NB = TN / 64;
    const int mb = q / NB, nb = q % NB;
    bf16x8 a, b;
    if constexpr (TA) a = __builtin_shufflevector(f.alo[mb], f.ahi[mb], 0, 1, 2, 3, 4, 5, 6, 7);
    else a = f.a[mb];
    if constexpr (TB) b = f.b[nb];
    else b = __builtin_shufflevector(f.blo[nb], f.bhi[nb], 0, 1, 2, 3, 4, 5, 6, 7);
    acc[mb][nb] = mfma16<kF16>(a, b, acc[mb][nb]);
}

// The MFMAs of one slice with the reads of the next slice and (if loads)
// this wave's LDS-direct loads of a later tile slotted in: one read after
// each of the first MFMAs and a load after every other MFMA when there are
// enough MFMAs (256 x 256), spread evenly otherwise (128 x 128: 4 MFMAs, 6
// reads, 4 loads).  sched_barrier(0) pins that order so the matrix unit
// keeps running while reads and loads are in flight.
template <int TM, int TN, bool TA, bool TB, bool kF16>
__device__ __forceinline__ void mfma_phase(f32x16 (&acc)[TM / 64][TN / 64],
                                           const Frag16<TM, TN, TA, TB> &cur,
                                           Frag16<TM, TN, TA, TB> &nxt, const uint16_t *rstage,
                                           const DCtx<TM, TN, TA, TB, kF16> &x, int s_next,
                                           uint32_t lstage, int64_t kload, bool loads)
{
    using T = DTile<TM, TN, TA, TB>;
#pragma unroll
    for (int q = 0; q < T::kQ; ++q) {
        mfma_one<kF16>(acc, cur, q);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (T::kReads <= T::kQ) {
            if (q < T::kReads) read_one(nxt, rstage, x, s_next, q);
        } else {
#pragma unroll
            for (int r = 0; r < T::kReads; ++r)
                if (r * T::kQ / T::kReads == q) read_one(nxt, rstage, x, s_next, r);
        }
        if (loads) {
            if constexpr (2 * T::kPerTile <= T::kQ) {
                if (q & 1) load_one(x, lstage, kload, q >> 1);
            } else {
#pragma unroll
                for (int l = 0; l < T::kPerTile; ++l)
                    if (l * T::kQ / T::kPerTile == q) load_one(x, lstage, kload, l);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// This wave's LDS reads complete (lgkmcnt 0) and its LDS-direct loads down
// to kCntVm in flight, then the work-group barrier.  Inline assembly so that
// the compiler's wait-count pass cannot weaken the LDS part: it is what
// guarantees that no wave still reads a stage another wave refills after
// the barrier.
template <int kCntVm>
__device__ __forceinline__ void wait_lds_vm_barrier()
{
    static_assert(kCntVm >= 0 && kCntVm <= 63, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(kCntVm) : "memory");
}

// Epilogue of the direct kernels through the idle LDS ring: every wave
// writes its accumulators into LDS rows (16-byte chunks XOR-permuted by bit
// 2 of the row, so the two half-waves' rows 4 apart use different banks),
// then the work-group writes C as 16-byte chunks of whole rows (a 256-wide
// row is one 1 KiB store instruction), in as many passes as the ring holds
// rows (two for 256 x 256, one for 128 x 128).  Against the direct stores
// from the MFMA layout (two 128-byte row pieces per instruction), with
// streaming stores on both sides: 8192^3 bf16 865 -> 858 us, 16384 x 1152 x
// 384 (128 x 128 tiles) 29.4 -> 27.1 us.  Needs C 16-byte aligned with ldc
// and N multiples of 4.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int TM, int TN>
__device__ __forceinline__ void store_c_rows(const f32x16 (&acc)[TM / 64][TN / 64], float *lf,
                                             float *__restrict__ C, int64_t ldc, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane)
{
    constexpr int MB = TM / 64, NB = TN / 64;
    constexpr int kRingFloats = DSTAGES * DTile<TM, TN>::kStageElems / 2;
    constexpr int kRingRows = kRingFloats / TN;   // whole rows the ring holds ...
    constexpr int kPow2Rows = kRingRows >= 256 ? 256 : kRingRows >= 128 ? 128 : 64;   // ... as 2^n
    constexpr int kPassRows = kPow2Rows < TM ? kPow2Rows : TM;
    constexpr int kPasses = TM / kPassRows;
    constexpr int kMBP = MB / kPasses;       // 32-row blocks per wave per pass
    constexpr int kHalf = kMBP * 32;         // rows per wave per pass
    constexpr int kChunks = TN / 4;          // 16-byte chunks per row
    static_assert(kPasses * kPassRows == TM && kMBP * kPasses == MB, "passes");
    const int h = lane >> 5, c = lane & 31;
    // every wave's loads landed and reads done: the ring is free
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        if (pass) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int mbl = 0; mbl < kMBP; ++mbl)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int col = wn * (TN / 2) + nb * 32 + c;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lrow = wm * kHalf + mbl * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int pcol = ((col >> 2) ^ (((lrow >> 2) & 1) << 3)) * 4 + (col & 3);
                    lf[lrow * TN + pcol] = acc[pass * kMBP + mbl][nb][r];
                }
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int i = 0; i < kPassRows * kChunks / kThreads; ++i) {
            const int q = threadIdx.x + kThreads * i;
            const int lrow = q / kChunks, chunk = q % kChunks;
            const int pchunk = chunk ^ (((lrow >> 2) & 1) << 3);
            const f32x4 v = *reinterpret_cast<const f32x4 *>(lf + lrow * TN + pchunk * 4);
            const int64_t row = m0 + (lrow / kHalf) * (TM / 2) + pass * kHalf + lrow % kHalf;
            const int64_t col = n0 + 4 * chunk;
            if (row < M && col < N) store_c_stream(reinterpret_cast<f32x4 *>(C + row * ldc + col), v);
        }
    }
}

__device__ __forceinline__ const void *uniform_ptr(const void *p)
{
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void *>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    return static_cast<int64_t>(reinterpret_cast<uintptr_t>(
        uniform_ptr(reinterpret_cast<const void *>(static_cast<uintptr_t>(v)))));
}

// kBatch: a batch of products (stride_a, stride_b, stride_c elements apart)
// as one grid of (product, tile) work-groups; a single product keeps the
// plain tile map.
template <int TM, int TN, bool kRowsC, bool TA = false, bool TB = false, bool kBatch = false,
          bool kF16 = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DTile<TM, TN>::kPerCU, DTile<TM, TN>::kPerCU)))
void mfma_bf16_direct_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A,
                             int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
                             float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n,
                             int64_t sa, int64_t sb, int64_t sc, int64_t batch)
{
    using T = DTile<TM, TN, TA, TB>;
    constexpr int MB = T::kMB, NB = T::kNB, WM = TM / 2, WN = TN / 2;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[DSTAGES * T::kStageElems];

    int64_t m0, n0;
    if constexpr (kBatch) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
        A += t.b * sa;
        B += t.b * sb;
        C += t.b * sc;
        m0 = t.tm * TM;
        n0 = t.tn * TN;
    } else {
        const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
        m0 = t.tm * TM;
        n0 = t.tn * TN;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, c = lane & 31;
    const int i16 = lane & 15, nhalf = (lane >> 4) & 1;

    DCtx<TM, TN, TA, TB, kF16> x;
    x.wave = wave;
    x.lds0 = lds_offset(lds);
    // Rows of K start at the tile's first row and step 32 elements per
    // tile; rows of M or N start at the tile's first column and step 32
    // rows.  Stated wave-uniform so the per-tile bases stay scalar.
    x.abase = static_cast<const char *>(uniform_ptr(TA ? A + m0 : A + m0 * lda));
    x.bbase = static_cast<const char *>(uniform_ptr(TB ? B + n0 * ldb : B + n0));
    x.a_kstride = uniform_i64(TA ? DBK * lda * 2 : DBK * 2);
    x.b_kstride = uniform_i64(TB ? DBK * 2 : DBK * ldb * 2);
#pragma unroll
    for (int i = 0; i < T::kAInst; ++i) {
        const int p = (wave * T::kAInst + i) * 64 + lane;   // LDS chunk this lane fills
        if constexpr (TA) {
            // 32 rows of TM elements, laid out as B's; columns past M
            // re-fetch the last full chunk (M % 8 == 0 here)
            const int row = p / (TM / 8), slot = p % (TM / 8);
            const int cc = slot ^ b_swzc<TM / 8>(row);
            const int64_t col = (m0 + 8 * cc < M) ? 8 * cc : M - 8 - m0;
            x.a_voff[i] = static_cast<uint32_t>((row * lda + col) * 2);
            continue;
        }
        const int row = p >> 2, slot = p & 3;
        const int cc = slot ^ a_swz<4>(row);
        const int64_t r = (m0 + row < M) ? row : M - 1 - m0;
        x.a_voff[i] = static_cast<uint32_t>((r * lda + 8 * cc) * 2);
    }
#pragma unroll
    for (int i = 0; i < T::kBInst; ++i) {
        const int p = (wave * T::kBInst + i) * 64 + lane;
        if constexpr (TB) {
            // TN rows of 32 elements, laid out as A's
            const int row = p >> 2, slot = p & 3;
            const int cc = slot ^ a_swz<4>(row);
            const int64_t r = (n0 + row < N) ? row : N - 1 - n0;
            x.b_voff[i] = static_cast<uint32_t>((r * ldb + 8 * cc) * 2);
            continue;
        }
        const int row = p / T::kBChunks, slot = p % T::kBChunks;
        const int cc = slot ^ b_swzc<TN / 8>(row);
        const int64_t col = (n0 + 8 * cc < N) ? 8 * cc : N - 8 - n0;
        x.b_voff[i] = static_cast<uint32_t>((row * ldb + col) * 2);
    }
    // A rows this lane reads are wm*WM + 32*j + c: their swizzle is a_swz<4>(c)
    // (it depends on bits 2-3 of the row only).
    const int aswz = a_swz<4>(c);
    // Rows of M or N this lane points at are 16s + 8h + i16/4 (+4): swizzle
    // b_swzc(i16/4) for the row width of A (TM) or B (TN).
    const int bswz = b_swzc<TN / 8>(i16 >> 2);
    if constexpr (TA) {
        const int aswz_t = b_swzc<TM / 8>(i16 >> 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = wm * WM + mb * 32 + nhalf * 16 + 4 * (i16 & 3);
            x.rdA[mb] = (8 * h + (i16 >> 2)) * TM * 2 + (((m >> 3) ^ aswz_t) << 4) + (m & 7) * 2;
        }
    } else {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            x.rdA[s] = (wm * WM + c) * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
    }
    if constexpr (TB) {
        // rows wn*WN + 32*nb + c of the B region, as for A
#pragma unroll
        for (int s = 0; s < 2; ++s)
            x.rdB[s] = TM * DBK * 2 + (wn * WN + c) * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = wn * WN + nb * 32 + nhalf * 16 + 4 * (i16 & 3);
            x.rdB[nb] = TM * DBK * 2 + (8 * h + (i16 >> 2)) * TN * 2 + (((n >> 3) ^ bswz) << 4) +
                        (n & 7) * 2;
        }
    }

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = K / DBK;
    auto stage = [&](int64_t kt) { return lds + (kt % DSTAGES) * T::kStageElems; };
    auto lstage = [&](int64_t kt) {
        return x.lds0 + static_cast<uint32_t>(kt % DSTAGES) * T::kStageElems * 2;
    };
    auto kclamp = [&](int64_t kt) { return kt < ktiles ? kt : ktiles - 1; };

    // Prologue: tiles 0..2 in flight (re-fetching the last tile past the
    // end), wait for tile 0, read its first slice.
#pragma unroll
    for (int st = 0; st < DSTAGES - 1; ++st)
#pragma unroll
        for (int l = 0; l < T::kPerTile; ++l) load_one(x, lstage(st), kclamp(st), l);
    wait_lds_vm_barrier<(DSTAGES - 2) * T::kPerTile>();

    Frag16<TM, TN, TA, TB> f0, f1;
#pragma unroll
    for (int j = 0; j < T::kReads; ++j) read_one(f0, stage(0), x, 0, j);

    // Tile kt:  MFMAs on slice 0 with the reads of slice 1 and the loads of
    // tile kt + 3 slotted in (that stage was last read in tile kt - 1, which
    // every wave finished before the previous barrier) | wait until tile
    // kt + 1 has landed everywhere and this wave's reads are done, barrier |
    // MFMAs on slice 1 with the reads of slice 0 of tile kt + 1 (in the last
    // tile: reads of a landed stage, unused).
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int64_t nxt = kt + DSTAGES - 1;
        mfma_phase(acc, f0, f1, stage(kt), x, 1, lstage(nxt), kclamp(nxt), true);
        wait_lds_vm_barrier<(DSTAGES - 2) * T::kPerTile>();
        mfma_phase(acc, f1, f0, stage(kt + 1), x, 0, 0, 0, false);
    }
    // No LDS-direct load may still be writing LDS when the work-group ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (kRowsC)
        store_c_rows<TM, TN>(acc, reinterpret_cast<float *>(lds), C, ldc, M, N, m0, n0, wm, wn,
                             lane);
    else
        store_c(acc, C, ldc, M, N, m0, n0, wm, wn, lane);
}

// ---- 256 x 256 tiles on the 16 x 16 x 32 instruction ------------------------
// The same LDS-direct ring, loads and layouts as above, but each wave's
// 128 x 128 piece of C is 8 x 8 blocks of 16 x 16 on v_mfma_f32_16x16x32_bf16
// (or _f16): one MFMA consumes a whole 32-deep stage.  Per flop this moves
// half as many accumulator bytes through the register file as the 32 x 32 x
// 16 instruction; under the board's power limit a loop of nothing but these
// MFMAs on random bf16 operands sustains 0.72 of the nominal peak against
// 0.69 for the 32 x 32 shape, and this tile runs 3-5% faster than the 32 x 32
// tile at 4096^3 and 8192^3 (vidyal.ai Part 6 on feeding the matrix
// instructions; the smaller instruction is the gfx950 variant, not the
// pages').  Operand layout: lane (i, g) = (lane mod 16, lane / 16) supplies
// row (A) or column (B) i of a block and k = 8g .. 8g + 7; it holds C rows
// 4g .. 4g + 3 of column i.
//
// Schedule of one stage (one barrier): the 64 MFMAs in column-block-major
// order (q = 8 nb + mb).  B fragments are re-read from the next stage in
// place, each half right after the last MFMA that uses it; A fragments go to
// the second of two register sets, one block every eighth MFMA; this wave's
// loads of the tile three stages ahead follow every eighth MFMA from the
// second.  Measured against the other placements tried (reads and loads
// bunched at the start of the stage, every second or fourth MFMA): 2-5%
// faster at 8192^3.  The first stage's MFMAs start from zero instead of
// zeroed accumulators: with 256 zero-initialised registers live into the
// loop the register allocator split them between register files and spilled.
//
// A 16-lane transposing read touches rows 8 apart within a half-wave (the
// groups g and g + 1 want k = 8g .. and 8g + 8 ..), so rows of M or N get the
// b_swz masks with bit 1 flipped when bit 3 of the row is set: both 16-byte
// slot sets of a half-wave are then distinct.
namespace d16 {

constexpr int kTile = 256;
constexpr int kBlocks = 8;                                  // 16-wide blocks per wave, each way
constexpr int kInst = kTile * DBK * 2 / 1024 / 4;           // LDS-direct loads per wave per factor
constexpr int kPerTile = 2 * kInst;
constexpr int kStage = 2 * kTile * DBK;                     // bf16 elements per stage
constexpr int kRegion = kTile * DBK * 2;                    // bytes of one factor per stage

__device__ __forceinline__ int swz_mn(int row) { return b_swz(row) ^ (((row >> 3) & 1) << 1); }

// Rows of 4 chunks (a factor stored along K): 16 consecutive rows at one
// logical chunk per 16 lanes.  (row >> 2) & 3, the 32 x 32 tile's mask,
// measured 3.9 conflict cycles per read in this pattern (SQ_LDS_BANK_CONFLICT),
// row & 3 and (row ^ row >> 2) & 3 the same; (row >> 1) & 3 measured none.
__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 3; }

// One factor's operand fragments.  Stored along K (A as written, B
// transposed): one 16-byte read per block into w; stored along M or N: two
// transposing reads per block into lo / hi.  Unused members take no registers.
struct Frag {
    bf16x8 w[kBlocks];
    bf16x4 lo[kBlocks], hi[kBlocks];
};

struct Ctx {
    uint32_t a_voff[kInst], b_voff[kInst];
    const char *abase, *bbase;
    int64_t a_kstride, b_kstride;
    uint32_t lds0;
    int wave;
    uint32_t rdA[kBlocks], rdB[kBlocks];   // lane read offsets (bytes) of each block
};

__device__ __forceinline__ void load_one(const Ctx &x, uint32_t stage_lds, int64_t kt, int l)
{
    if (l < kInst)
        lds_direct_load16(x.a_voff[l], x.abase + kt * x.a_kstride, stage_lds + (x.wave * kInst + l) * 1024);
    else
        lds_direct_load16(x.b_voff[l - kInst], x.bbase + kt * x.b_kstride,
                          stage_lds + kRegion + (x.wave * kInst + l - kInst) * 1024);
}

template <bool kAlongK>
__device__ __forceinline__ void read_block(Frag &f, const char *stage, uint32_t off, int j)
{
    if constexpr (kAlongK) {
        f.w[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(stage + off));
    } else {
        f.lo[j] = read_tr4(stage + off);
        f.hi[j] = read_tr4(stage + off + 4 * kTile * 2);
    }
}

template <bool kAlongK>
__device__ __forceinline__ bf16x8 operand(const Frag &f, int j)
{
    if constexpr (kAlongK) return f.w[j];
    else return __builtin_shufflevector(f.lo[j], f.hi[j], 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool kF16>
__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One stage: MFMAs on (cur, fb) with the next stage's reads (A into nxt, B
// in place) and this wave's loads of tile kload slotted in.  kFirst: the
// accumulators start at zero.
template <bool kFirst, bool kF16, bool TA, bool TB>
__device__ __forceinline__ void phase(f32x4 (&acc)[kBlocks][kBlocks], const Frag &cur, Frag &nxt,
                                      Frag &fb, const uint16_t *rstage, const Ctx &x,
                                      uint32_t lstage, int64_t kload)
{
    const char *st = reinterpret_cast<const char *>(rstage);
#pragma unroll
    for (int q = 0; q < kBlocks * kBlocks; ++q) {
        const int nb = q / kBlocks, mb = q % kBlocks;
        acc[mb][nb] = mfma<kF16>(operand<!TA>(cur, mb), operand<TB>(fb, nb),
                                 kFirst ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TB) {
            if (mb == kBlocks - 1) read_block<true>(fb, st, x.rdB[nb], nb);
        } else {
            if (mb == kBlocks - 1) fb.lo[nb] = read_tr4(st + x.rdB[nb]);
            if (mb == 3 && nb > 0) fb.hi[nb - 1] = read_tr4(st + x.rdB[nb - 1] + 4 * kTile * 2);
            if (q == kBlocks * kBlocks - 1)
                fb.hi[kBlocks - 1] = read_tr4(st + x.rdB[kBlocks - 1] + 4 * kTile * 2);
        }
        if (q % 8 == 4) read_block<!TA>(nxt, st, x.rdA[q / 8], q / 8);
        if (q % 8 == 1) load_one(x, lstage, kload, q / 8);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// C through the idle ring in two passes of 128 rows (64 per wave row): each
// lane writes its four rows of each block (16-byte chunks XOR-permuted by
// rows / 4 mod 4, so the four row groups of one write hit distinct banks),
// then the work-group writes whole 16-byte row chunks.
__device__ __forceinline__ void store_rows(const f32x4 (&acc)[kBlocks][kBlocks], float *lf,
                                           float *__restrict__ C, int64_t ldc, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int wm, int wn,
                                           int lane)
{
    const int i16 = lane & 15, g = lane >> 4;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        if (pass) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int mbl = 0; mbl < 4; ++mbl)
#pragma unroll
            for (int nb = 0; nb < kBlocks; ++nb) {
                const int col = wn * 128 + nb * 16 + i16;
                const f32x4 v = acc[pass * 4 + mbl][nb];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lrow = wm * 64 + mbl * 16 + 4 * g + r;
                    const int pcol = ((col >> 2) ^ (((lrow >> 2) & 3) << 2)) * 4 + (col & 3);
                    lf[lrow * kTile + pcol] = v[r];
                }
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int i = 0; i < 128 * (kTile / 4) / kThreads; ++i) {
            const int q = threadIdx.x + kThreads * i;
            const int lrow = q / (kTile / 4), chunk = q % (kTile / 4);
            const int pchunk = chunk ^ (((lrow >> 2) & 3) << 2);
            const f32x4 v = *reinterpret_cast<const f32x4 *>(lf + lrow * kTile + pchunk * 4);
            const int64_t row = m0 + (lrow / 64) * 128 + pass * 64 + lrow % 64;
            const int64_t col = n0 + 4 * chunk;
            if (row < M && col < N) store_c_stream(reinterpret_cast<f32x4 *>(C + row * ldc + col), v);
        }
    }
}

// C straight from the MFMA layout (any C alignment).
__device__ __forceinline__ void store_direct(const f32x4 (&acc)[kBlocks][kBlocks],
                                             float *__restrict__ C, int64_t ldc, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane)
{
    const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < kBlocks; ++mb)
#pragma unroll
        for (int nb = 0; nb < kBlocks; ++nb) {
            const int64_t col = n0 + wn * 128 + nb * 16 + i16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 128 + mb * 16 + 4 * g + r;
                if (row < M && col < N) store_c_stream(C + row * ldc + col, acc[mb][nb][r]);
            }
        }
}

}  // namespace d16

template <bool kRowsC, bool TA, bool TB, bool kBatch, bool kF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_bf16_d16_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A,
                          int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
                          float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n,
                          int64_t sa, int64_t sb, int64_t sc, int64_t batch)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[DSTAGES * d16::kStage];

    int64_t m0, n0;
    if constexpr (kBatch) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
        A += t.b * sa;
        B += t.b * sb;
        C += t.b * sc;
        m0 = t.tm * d16::kTile;
        n0 = t.tn * d16::kTile;
    } else {
        const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
        m0 = t.tm * d16::kTile;
        n0 = t.tn * d16::kTile;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int i16 = lane & 15, g = lane >> 4;

    d16::Ctx x;
    x.wave = wave;
    x.lds0 = lds_offset(lds);
    x.abase = static_cast<const char *>(uniform_ptr(TA ? A + m0 : A + m0 * lda));
    x.bbase = static_cast<const char *>(uniform_ptr(TB ? B + n0 * ldb : B + n0));
    x.a_kstride = uniform_i64(TA ? DBK * lda * 2 : DBK * 2);
    x.b_kstride = uniform_i64(TB ? DBK * 2 : DBK * ldb * 2);
    // Load lane offsets.  Along K: 256 rows of 4 chunks, chunk c of row r at
    // slot c ^ swz_k(r), rows past the edge re-read the last one.  Along
    // M or N: 32 rows of 32 chunks at slot c ^ swz_mn(r), chunks past the
    // edge re-read the last whole one (that dimension is a multiple of 8).
    const auto along_k = [&](int p, int64_t base, int64_t extent, int64_t ld) {
        const int row = p >> 2, slot = p & 3;
        const int cc = slot ^ d16::swz_k(row);
        const int64_t r = (base + row < extent) ? row : extent - 1 - base;
        return static_cast<uint32_t>((r * ld + 8 * cc) * 2);
    };
    const auto along_mn = [&](int p, int64_t base, int64_t extent, int64_t ld) {
        const int row = p / (d16::kTile / 8), slot = p % (d16::kTile / 8);
        const int cc = slot ^ d16::swz_mn(row);
        const int64_t col = (base + 8 * cc < extent) ? 8 * cc : extent - 8 - base;
        return static_cast<uint32_t>((row * ld + col) * 2);
    };
#pragma unroll
    for (int i = 0; i < d16::kInst; ++i) {
        const int p = (wave * d16::kInst + i) * 64 + lane;
        x.a_voff[i] = TA ? along_mn(p, m0, M, lda) : along_k(p, m0, M, lda);
        x.b_voff[i] = TB ? along_k(p, n0, N, ldb) : along_mn(p, n0, N, ldb);
    }
    // Read offsets.  Along K: block j's rows base + 16 j + i16, chunk g; the
    // swizzle (rows / 2 mod 4) depends on the lane only.  Along M or N: rows
    // 8g + i16 / 4 (+4 for the upper half), 4 columns from base + 16 j +
    // 4 (i16 mod 4); the swizzle touches chunk bits 1-3, so per block.
#pragma unroll
    for (int j = 0; j < d16::kBlocks; ++j) {
        const int rk = (wm * 128 + 16 * j + i16) * DBK * 2 + ((g ^ d16::swz_k(i16)) << 4);
        const int row = 8 * g + (i16 >> 2);
        const int ma = wm * 128 + 16 * j + 4 * (i16 & 3);
        x.rdA[j] = TA ? row * d16::kTile * 2 + (((ma >> 3) ^ d16::swz_mn(row)) << 4) + (ma & 7) * 2 : rk;
        const int rkb = d16::kRegion + (wn * 128 + 16 * j + i16) * DBK * 2 + ((g ^ d16::swz_k(i16)) << 4);
        const int nb_ = wn * 128 + 16 * j + 4 * (i16 & 3);
        x.rdB[j] = TB ? rkb : d16::kRegion + row * d16::kTile * 2 + (((nb_ >> 3) ^ d16::swz_mn(row)) << 4) + (nb_ & 7) * 2;
    }

    const int64_t ktiles = K / DBK;
    auto stage = [&](int64_t kt) { return lds + (kt % DSTAGES) * d16::kStage; };
    auto lstage = [&](int64_t kt) {
        return x.lds0 + static_cast<uint32_t>(kt % DSTAGES) * d16::kStage * 2;
    };
    auto kclamp = [&](int64_t kt) { return kt < ktiles ? kt : ktiles - 1; };

    // Prologue: tiles 0..2 in flight (past the end re-fetching the last),
    // wait for tile 0, read all of its fragments.
#pragma unroll
    for (int st = 0; st < DSTAGES - 1; ++st)
#pragma unroll
        for (int l = 0; l < d16::kPerTile; ++l) d16::load_one(x, lstage(st), kclamp(st), l);
    wait_lds_vm_barrier<(DSTAGES - 2) * d16::kPerTile>();
    d16::Frag a0, a1, fb;
    {
        const char *st0 = reinterpret_cast<const char *>(stage(0));
#pragma unroll
        for (int j = 0; j < d16::kBlocks; ++j) {
            d16::read_block<!TA>(a0, st0, x.rdA[j], j);
            d16::read_block<TB>(fb, st0, x.rdB[j], j);
        }
    }
    // Stage kt: wait until tile kt + 1 has landed everywhere and every
    // wave's reads of tile kt are done, barrier, then the MFMAs of tile kt
    // with the reads of tile kt + 1 and the loads of tile kt + 3 (whose
    // stage was last read in stage kt - 2).  A sets alternate a0, a1.
    f32x4 acc[d16::kBlocks][d16::kBlocks];   // written by stage 0's MFMAs
    wait_lds_vm_barrier<d16::kPerTile>();
    d16::phase<true, kF16, TA, TB>(acc, a0, a1, fb, stage(1), x, lstage(3), kclamp(3));
    int64_t kt = 1;
    for (; kt + 1 < ktiles; kt += 2) {
        wait_lds_vm_barrier<d16::kPerTile>();
        d16::phase<false, kF16, TA, TB>(acc, a1, a0, fb, stage(kt + 1), x, lstage(kt + 3), kclamp(kt + 3));
        wait_lds_vm_barrier<d16::kPerTile>();
        d16::phase<false, kF16, TA, TB>(acc, a0, a1, fb, stage(kt + 2), x, lstage(kt + 4), kclamp(kt + 4));
    }
    if (kt < ktiles) {   // an even number of tiles: the last one on a1
        wait_lds_vm_barrier<d16::kPerTile>();
        d16::phase<false, kF16, TA, TB>(acc, a1, a0, fb, stage(kt + 1), x, lstage(kt + 3), kclamp(kt + 3));
    }
    // No LDS-direct load may still be writing LDS when the work-group ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (kRowsC)
        d16::store_rows(acc, reinterpret_cast<float *>(lds), C, ldc, M, N, m0, n0, wm, wn, lane);
    else
        d16::store_direct(acc, C, ldc, M, N, m0, n0, wm, wn, lane);
}

// ---- 8-bit floats on the same staging ---------------------------------------
// The OCP e4m3 / e5m2 operands of v_mfma_scale_f32_32x32x64_f8f6f4, A as
// written and B transposed: both factors then have rows along K, and two
// 8-bit values sit in each 16-bit slot of the bf16 kernel's staging, so a K
// tile of DBK slots is 64 bytes of K, exactly one MFMA deep.  Lane (h, c)'s
// 32 bytes per operand are bytes 16 h .. 16 h + 15 and 32 + 16 h .. 47 + 16 h
// of the tile (two 16-byte reads), which is where the instruction takes K
// positions from: its 32-element block 0 is the first 16 bytes of both
// half-waves, block 1 the second 16, and the scale of block b of row
// (column) c is the scale operand of lane (b, c) (measured: lanes holding
// bytes 32 h .. 32 h + 31 with the scale of block h give exactly the sums
// of that mapping).  MX block scales (vidyal.ai tag page, Part 11, names
// them; OCP microscaling fixes the block at 32 elements and the scale
// format at E8M0) so need no other operand layout.  Without them every
// scale is 127 (2^0); with them (kMX) each stage also holds the tile's
// scales -- two blocks of K for each row of A and each column of B,
// 2 TM + 2 TN bytes, loaded by one more 4-byte LDS-direct load per wave --
// and lane (h, c) reads the byte of block h of its row (column) beside its
// fragments.  Per MFMA the matrix unit is busy twice as long as
// for bf16 while the bytes staged per MFMA are the same, so one tile's
// MFMAs cover the loads of a tile and the reads of the next: one phase per
// tile, with the next tile's reads and the loads of the tile four ahead
// slotted between the MFMAs.  128 x 128 tiles (two work-groups per CU) or
// 256 x 128 (one): at 256 x 256 the two fragment sets (128 registers)
// beside 256 accumulators made the compiler spill (about 600 registers to
// scratch), so that size is not built.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// A wave's 8-bit operands for one tile: per 32-row (A) or 32-column (B)
// block the lane's 32 bytes, filled a 16-byte half (one slice) at a time
// straight into the register tuple the MFMA takes.
template <int TM, int TN>
struct Frag8 {
    i32x8 a[TM / 64], b[TN / 64];
    int sa[TM / 64], sb[TN / 64];   // MX scales (E8M0 in the low byte) of the lane's blocks
};

// MX scale staging of one wave: its 4-byte LDS-direct load of the tile's
// scale bytes (scalar base, advanced by kstride bytes per tile, lane offset
// voff, landing at byte lds_off of each stage) and the stage byte offsets
// of the lane's scales of its A and B blocks.
template <int TM, int TN>
struct MXCtx {
    const char *base;
    int64_t kstride;
    uint32_t voff, lds_off;
    uint32_t rdA[TM / 64], rdB[TN / 64];
};

// One LDS-direct 4-byte load, scalar-base form: lane i's 4 bytes land at
// LDS byte M0 + 4 i (counted like the 16-byte loads).
__device__ __forceinline__ void lds_direct_load4(uint32_t voff, const void *sbase, uint32_t m0v)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

template <int TM, int TN>
__device__ __forceinline__ void read_scales(Frag8<TM, TN> &f, const uint16_t *stage,
                                            const MXCtx<TM, TN> &mx)
{
    const uint8_t *st = reinterpret_cast<const uint8_t *>(stage);
#pragma unroll
    for (int j = 0; j < TM / 64; ++j) f.sa[j] = st[mx.rdA[j]];
#pragma unroll
    for (int j = 0; j < TN / 64; ++j) f.sb[j] = st[mx.rdB[j]];
}

template <int kHalf>
__device__ __forceinline__ void set_half(i32x8 &v, const u16x8 &x)
{
    const i32x4 w = __builtin_bit_cast(i32x4, x);
    const i32x8 ww = __builtin_shufflevector(w, w, 0, 1, 2, 3, 0, 1, 2, 3);
    if constexpr (kHalf == 0) v = __builtin_shufflevector(v, ww, 8, 9, 10, 11, 4, 5, 6, 7);
    else v = __builtin_shufflevector(v, ww, 0, 1, 2, 3, 12, 13, 14, 15);
}

// Read r of a tile: r < 2 kMB: A block r / 2, slice r % 2; then B likewise.
template <int TM, int TN>
__device__ __forceinline__ void read8(Frag8<TM, TN> &f, const uint16_t *stage,
                                      const DCtx<TM, TN, false, true> &x, int r)
{
    constexpr int nA = 2 * (TM / 64);
    const char *st = reinterpret_cast<const char *>(stage);
    const bool isA = r < nA;
    const int j = (isA ? r : r - nA) >> 1, s = r & 1;
    const u16x8 v = *reinterpret_cast<const u16x8 *>(st + (isA ? x.rdA[s] : x.rdB[s]) + j * 2048);
    if (isA) {
        if (s) set_half<1>(f.a[j], v);
        else set_half<0>(f.a[j], v);
    } else {
        if (s) set_half<1>(f.b[j], v);
        else set_half<0>(f.b[j], v);
    }
}

// fp8 operation codes: 2 * fa + fb, fa and fb the formats (0 e4m3, 1 e5m2);
// sa and sb the E8M0 scales of the lane's blocks (127: 2^0).
template <int kFmt>
__device__ __forceinline__ f32x16 mfma8(const i32x8 &a, const i32x8 &b, const f32x16 &c,
                                        int sa = 127, int sb = 127)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFmt >> 1, kFmt & 1, 0, sa,
                                                           0, sb);
}

// MFMAs of one tile (fragments cur) with the reads of the next tile into
// nxt and this wave's loads of tile `kload` into stage `lstage` slotted in,
// spread evenly (256 x 256: one read after each MFMA, a load after every
// other).
// Load l of a tile: the A and B chunks, then (kMX) the scale load.
template <bool kMX, int TM, int TN>
__device__ __forceinline__ void load8_one(const DCtx<TM, TN, false, true> &x,
                                          const MXCtx<TM, TN> &mx, uint32_t stage_lds, int64_t kt,
                                          int l)
{
    if (kMX && l == DTile<TM, TN, false, true>::kPerTile)
        lds_direct_load4(mx.voff, mx.base + kt * mx.kstride, stage_lds + mx.lds_off);
    else
        load_one(x, stage_lds, kt, l);
}

template <int kFmt, bool kMX, bool kFirst, int TM, int TN>
__device__ __forceinline__ void mfma_phase8(f32x16 (&acc)[TM / 64][TN / 64],
                                            const Frag8<TM, TN> &cur, Frag8<TM, TN> &nxt,
                                            const uint16_t *rstage,
                                            const DCtx<TM, TN, false, true> &x,
                                            const MXCtx<TM, TN> &mx, uint32_t lstage,
                                            int64_t kload)
{
    using T = DTile<TM, TN, false, true>;
    constexpr int NB = T::kNB, R = 2 * T::kReads, Q = T::kQ, P = T::kPerTile + (kMX ? 1 : 0);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int mb = q / NB, nb = q % NB;
        const f32x16 c0 = kFirst ? f32x16{} : acc[mb][nb];
        if constexpr (kMX)
            acc[mb][nb] = mfma8<kFmt>(cur.a[mb], cur.b[nb], c0, cur.sa[mb], cur.sb[nb]);
        else
            acc[mb][nb] = mfma8<kFmt>(cur.a[mb], cur.b[nb], c0);
        __builtin_amdgcn_sched_barrier(0);
        if (kMX && q == 0) read_scales(nxt, rstage, mx);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r * Q / R == q) read8(nxt, rstage, x, r);
#pragma unroll
        for (int l = 0; l < P; ++l)
            if (l * Q / P == q) load8_one<kMX>(x, mx, lstage, kload, l);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// M, N, K, lda, ldb, stride_a and stride_b in 16-bit slots (bytes / 2).
// kMX: xa / xb are the MX scales (E8M0), the scale of 32-element block kb of
// row i of A at xa[kb * ldxa + i], of row j of B (column j of the product)
// at xb[kb * ldxb + j]; ldxa and ldxb multiples of 4, xa and xb 4-byte
// aligned (a single product).
template <int TM, int TN, bool kRowsC, bool kBatch, int kFmt, bool kMX = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DTile<TM, TN>::kPerCU, DTile<TM, TN>::kPerCU)))
void mfma_fp8_direct_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A,
                            int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
                            float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n,
                            int64_t sa, int64_t sb, int64_t sc, int64_t batch,
                            const uint8_t *__restrict__ xa = nullptr, int64_t ldxa = 0,
                            const uint8_t *__restrict__ xb = nullptr, int64_t ldxb = 0)
{
    using T = DTile<TM, TN, false, true>;
    constexpr int MB = T::kMB, NB = T::kNB, WM = TM / 2, WN = TN / 2;
    constexpr int P = T::kPerTile + (kMX ? 1 : 0);
    // a stage: the A and B tiles, then (kMX) 1 KiB for the scales, one
    // 256-byte slot per wave's scale load
    constexpr int SE = T::kStageElems + (kMX ? 512 : 0);
    static_assert((DSTAGES - 1) * P <= 63, "vmcnt is six bits");
    static_assert(!kMX || (2 * TM % 256 == 0 && 2 * TM + 2 * TN <= 1024), "scale slots");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[DSTAGES * SE];

    int64_t m0, n0;
    if constexpr (kBatch) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, batch, kGroup);
        A += t.b * sa;
        B += t.b * sb;
        C += t.b * sc;
        m0 = t.tm * TM;
        n0 = t.tn * TN;
    } else {
        const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
        m0 = t.tm * TM;
        n0 = t.tn * TN;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, c = lane & 31;

    // Both factors as the bf16 kernel's A: rows of K, DBK slots per tile,
    // rows past M or N re-fetch the last row.
    DCtx<TM, TN, false, true> x;
    x.wave = wave;
    x.lds0 = lds_offset(lds);
    x.abase = static_cast<const char *>(uniform_ptr(A + m0 * lda));
    x.bbase = static_cast<const char *>(uniform_ptr(B + n0 * ldb));
    x.a_kstride = DBK * 2;
    x.b_kstride = DBK * 2;
#pragma unroll
    for (int i = 0; i < T::kAInst; ++i) {
        const int p = (wave * T::kAInst + i) * 64 + lane;
        const int row = p >> 2, cc = (p & 3) ^ a_swz<4>(p >> 2);
        const int64_t r = (m0 + row < M) ? row : M - 1 - m0;
        x.a_voff[i] = static_cast<uint32_t>((r * lda + 8 * cc) * 2);
    }
#pragma unroll
    for (int i = 0; i < T::kBInst; ++i) {
        const int p = (wave * T::kBInst + i) * 64 + lane;
        const int row = p >> 2, cc = (p & 3) ^ a_swz<4>(p >> 2);
        const int64_t r = (n0 + row < N) ? row : N - 1 - n0;
        x.b_voff[i] = static_cast<uint32_t>((r * ldb + 8 * cc) * 2);
    }
    const int aswz = a_swz<4>(c);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        x.rdA[s] = (wm * WM + c) * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
        x.rdB[s] = TM * DBK * 2 + (wn * WN + c) * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
    }

    // Scale staging: the stage's scale bytes are [A block 2kt][A block
    // 2kt+1][B block 2kt][B block 2kt+1] (TM, TM, TN, TN bytes); wave w loads
    // bytes 256 w .. 256 w + 255 of it, waves past the end repeat the last
    // load into their own (unread) slot.  A row past M (column past N) reads
    // a byte of the row's padding, clamped to the last 4-byte word of the
    // row, which is in bounds (its product rows are never stored).
    MXCtx<TM, TN> mx{};
    if constexpr (kMX) {
        constexpr int kLoadsX = (2 * TM + 2 * TN) / 256;
        const int src = wave < kLoadsX ? wave : kLoadsX - 1;
        const int pos = 256 * src + 4 * lane;
        if (256 * src < 2 * TM) {
            const int kbo = pos / TM, row = pos % TM;
            const int64_t r = (m0 + row <= ldxa - 4) ? m0 + row : ldxa - 4;
            mx.base = reinterpret_cast<const char *>(uniform_ptr(xa + m0));
            mx.voff = static_cast<uint32_t>(kbo * ldxa + (r - m0));
            mx.kstride = 2 * ldxa;
        } else {
            const int q = pos - 2 * TM, kbo = q / TN, col = q % TN;
            const int64_t r = (n0 + col <= ldxb - 4) ? n0 + col : ldxb - 4;
            mx.base = reinterpret_cast<const char *>(uniform_ptr(xb + n0));
            mx.voff = static_cast<uint32_t>(kbo * ldxb + (r - n0));
            mx.kstride = 2 * ldxb;
        }
        mx.lds_off = T::kStageElems * 2 + 256 * wave;
#pragma unroll
        for (int j = 0; j < MB; ++j) mx.rdA[j] = T::kStageElems * 2 + h * TM + wm * WM + 32 * j + c;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            mx.rdB[j] = T::kStageElems * 2 + 2 * TM + h * TN + wn * WN + 32 * j + c;
    }

    f32x16 acc[MB][NB];   // written by tile 0's MFMAs (kFirst)

    const int64_t ktiles = K / DBK;
    auto stage = [&](int64_t kt) { return lds + (kt % DSTAGES) * SE; };
    auto lstage = [&](int64_t kt) {
        return x.lds0 + static_cast<uint32_t>(kt % DSTAGES) * SE * 2;
    };
    auto kclamp = [&](int64_t kt) { return kt < ktiles ? kt : ktiles - 1; };

    // Prologue: tiles 0..3 in flight (re-fetching the last tile past the
    // end); read tile 0 once it has landed; then wait for tile 1 (and every
    // wave's reads of tile 0, whose stage the first phase refills).
#pragma unroll
    for (int st = 0; st < DSTAGES; ++st)
#pragma unroll
        for (int l = 0; l < P; ++l) load8_one<kMX>(x, mx, lstage(st), kclamp(st), l);
    wait_lds_vm_barrier<(DSTAGES - 1) * P>();
    Frag8<TM, TN> f, g;
#pragma unroll
    for (int r = 0; r < 2 * T::kReads; ++r) read8(f, stage(0), x, r);
    if constexpr (kMX) read_scales(f, stage(0), mx);
    wait_lds_vm_barrier<(DSTAGES - 2) * P>();

    // Tile kt: MFMAs on its fragments (in registers) with the reads of tile
    // kt + 1 and the loads of tile kt + 4 into tile kt's stage (read in the
    // previous phase, which every wave finished before the last barrier) |
    // wait until tile kt + 2 has landed everywhere and this wave's reads are
    // done, barrier.  Two tiles per trip so the fragment sets alternate
    // without copies; reads past the last tile hit landed re-fetches.  Tile
    // 0's MFMAs start from zero instead of zeroed accumulators (which, live
    // into the loop, made the register allocator spill).
    mfma_phase8<kFmt, kMX, true>(acc, f, g, stage(1), x, mx, lstage(0), kclamp(DSTAGES));
    wait_lds_vm_barrier<(DSTAGES - 2) * P>();
    int64_t kt = 1;
    for (; kt + 1 < ktiles; kt += 2) {
        mfma_phase8<kFmt, kMX, false>(acc, g, f, stage(kt + 1), x, mx, lstage(kt),
                                      kclamp(kt + DSTAGES));
        wait_lds_vm_barrier<(DSTAGES - 2) * P>();
        mfma_phase8<kFmt, kMX, false>(acc, f, g, stage(kt + 2), x, mx, lstage(kt + 1),
                                      kclamp(kt + 1 + DSTAGES));
        wait_lds_vm_barrier<(DSTAGES - 2) * P>();
    }
    if (kt < ktiles) {
        mfma_phase8<kFmt, kMX, false>(acc, g, f, stage(kt + 1), x, mx, lstage(kt),
                                      kclamp(kt + DSTAGES));
        wait_lds_vm_barrier<(DSTAGES - 2) * P>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (kRowsC)
        store_c_rows<TM, TN>(acc, reinterpret_cast<float *>(lds), C, ldc, M, N, m0, n0, wm, wn,
                             lane);
    else
        store_c(acc, C, ldc, M, N, m0, n0, wm, wn, lane);
}

// ---- small outputs over a long K: the K range split over the waves -----------
// A weight gradient (a d_in x d_out output summed over every token of a
// training step) has few output tiles and a long K; with one 32 x 32 block
// per wave the 64 x 64 tile above does one MFMA per slice between its
// reads, loads and barrier.  Here each wave of a 64 x 64 work-group
// computes the whole tile (2 x 2 blocks, four MFMAs per slice) over every
// fourth 32-deep K tile, through a 4-stage LDS ring of its own (8 KiB per
// stage, filled by its own LDS-direct loads): the waves never wait for each
// other until the end, where waves 1-3 leave their partial tiles in LDS
// and wave 0 adds them in the order 0, 1, 2, 3 (deterministic) and writes
// C.  Staging, swizzles and reads per factor layout as in the tiles above
// (rows of K: 4 chunks per row, a_swz; rows of 64 M or N: 8 chunks,
// b_swzc<8>, transposing reads).
constexpr int WS_STAGE = 8192;                      // bytes per stage: A then B, 4 KiB each
constexpr int WS_RING = DSTAGES * WS_STAGE;         // bytes per wave

template <bool TA, bool TB>
struct WsCtx {
    uint32_t a_voff[4], b_voff[4];
    const char *abase, *bbase;
    int64_t a_kstride, b_kstride;
    uint32_t ring;                                  // LDS byte address of this wave's ring
    uint32_t rdA[TA ? 2 : 2], rdB[2];               // A: per block (TA) or slice; B: per block (!TB) or slice
};

template <bool TA, bool TB>
__device__ __forceinline__ void ws_loads(const WsCtx<TA, TB> &x, int stage, int64_t kt, int l)
{
    const uint32_t st = x.ring + stage * WS_STAGE;
    if (l < 4) lds_direct_load16(x.a_voff[l], x.abase + kt * x.a_kstride, st + l * 1024);
    else lds_direct_load16(x.b_voff[l - 4], x.bbase + kt * x.b_kstride, st + 4096 + (l - 4) * 1024);
}

// Read j of slice s from stage `st` (a byte pointer into this wave's ring).
// A: j < nA (one 16-byte read per block, or two transposing reads); then B.
template <bool TA, bool TB>
__device__ __forceinline__ void ws_read(Frag16<128, 128, TA, TB> &f, const char *st,
                                        const WsCtx<TA, TB> &x, int s, int j)
{
    constexpr int nA = TA ? 4 : 2;
    if (j < nA) {
        if constexpr (TA) {
            const int mb = j >> 1, upper = j & 1;
            const bf16x4 v = read_tr4(st + x.rdA[mb] + s * (16 * 64 * 2) + upper * (4 * 64 * 2));
            if (upper) f.ahi[mb] = v;
            else f.alo[mb] = v;
        } else {
            const u16x8 v = *reinterpret_cast<const u16x8 *>(st + x.rdA[s] + j * 2048);
            f.a[j] = __builtin_bit_cast(bf16x8, v);
        }
    } else if constexpr (TB) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(st + 4096 + x.rdB[s] + (j - nA) * 2048);
        f.b[j - nA] = __builtin_bit_cast(bf16x8, v);
    } else {
        const int nb = (j - nA) >> 1, upper = (j - nA) & 1;
        const bf16x4 v = read_tr4(st + 4096 + x.rdB[nb] + s * (16 * 64 * 2) + upper * (4 * 64 * 2));
        if (upper) f.bhi[nb] = v;
        else f.blo[nb] = v;
    }
}

template <bool kF16, bool TA, bool TB>
__device__ __forceinline__ void ws_phase(f32x16 (&acc)[2][2], const Frag16<128, 128, TA, TB> &cur,
                                         Frag16<128, 128, TA, TB> &nxt, const char *rst,
                                         const WsCtx<TA, TB> &x, int s_next, int lstage,
                                         int64_t kload, bool loads)
{
    constexpr int R = (TA ? 4 : 2) + (TB ? 2 : 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int mb = q >> 1, nb = q & 1;
        bf16x8 a, b;
        if constexpr (TA) a = __builtin_shufflevector(cur.alo[mb], cur.ahi[mb], 0, 1, 2, 3, 4, 5, 6, 7);
        else a = cur.a[mb];
        if constexpr (TB) b = cur.b[nb];
        else b = __builtin_shufflevector(cur.blo[nb], cur.bhi[nb], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[mb][nb] = mfma16<kF16>(a, b, acc[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r * 4 / R == q) ws_read(nxt, rst, x, s_next, r);
        if (loads) {
            ws_loads(x, lstage, kload, 2 * q);
            ws_loads(x, lstage, kload, 2 * q + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// kSplit2: two work-groups per tile, the first and the second half of the
// K tiles, each adding its sums into C (set to -0.0 beforehand) with one
// atomic add per element.  Two addends onto -0.0 give p0 + p1 rounded once
// in either order (fp32 addition commutes), so the result is the same on
// every run and equals a fixed-order two-way reduction; it needs no memory
// beyond C.
template <bool TA, bool TB, bool kF16, bool kSplit2 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_bf16_wsplit_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A,
                             int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
                             float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * WS_RING];

    int64_t m0, n0, kt0 = 0, kt1 = K / DBK;   // this work-group's K tiles [kt0, kt1)
    if constexpr (kSplit2) {
        const BatchTile t = map_batch_tile(tiles_m, tiles_n, 2, kGroup);
        m0 = t.tm * 64;
        n0 = t.tn * 64;
        const int64_t mid = (kt1 + 1) / 2;
        if (t.b == 0) kt1 = mid;
        else kt0 = mid;
    } else {
        const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
        m0 = t.tm * 64;
        n0 = t.tn * 64;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, c = lane & 31, i16 = lane & 15, nhalf = (lane >> 4) & 1;

    WsCtx<TA, TB> x;
    x.ring = lds_offset(lds) + wave * WS_RING;
    x.abase = static_cast<const char *>(uniform_ptr(TA ? A + m0 : A + m0 * lda));
    x.bbase = static_cast<const char *>(uniform_ptr(TB ? B + n0 * ldb : B + n0));
    x.a_kstride = uniform_i64(TA ? DBK * lda * 2 : DBK * 2);
    x.b_kstride = uniform_i64(TB ? DBK * 2 : DBK * ldb * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = i * 64 + lane;   // 16-byte LDS slot this lane fills (of 256 per factor)
        if constexpr (TA) {
            // 32 rows of K, 64 elements of M each (8 chunks); columns past M
            // re-fetch the last full chunk (M % 8 == 0 here)
            const int row = p >> 3, slot = p & 7;
            const int cc = slot ^ b_swzc<8>(row);
            const int64_t col = (m0 + 8 * cc < M) ? 8 * cc : M - 8 - m0;
            x.a_voff[i] = static_cast<uint32_t>((row * lda + col) * 2);
        } else {
            const int row = p >> 2, slot = p & 3;
            const int cc = slot ^ a_swz<4>(row);
            const int64_t r = (m0 + row < M) ? row : M - 1 - m0;
            x.a_voff[i] = static_cast<uint32_t>((r * lda + 8 * cc) * 2);
        }
        if constexpr (TB) {
            const int row = p >> 2, slot = p & 3;
            const int cc = slot ^ a_swz<4>(row);
            const int64_t r = (n0 + row < N) ? row : N - 1 - n0;
            x.b_voff[i] = static_cast<uint32_t>((r * ldb + 8 * cc) * 2);
        } else {
            const int row = p >> 3, slot = p & 7;
            const int cc = slot ^ b_swzc<8>(row);
            const int64_t col = (n0 + 8 * cc < N) ? 8 * cc : N - 8 - n0;
            x.b_voff[i] = static_cast<uint32_t>((row * ldb + col) * 2);
        }
    }
    const int aswz = a_swz<4>(c);
    const int tswz = b_swzc<8>(i16 >> 2);
    if constexpr (TA) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int m = mb * 32 + nhalf * 16 + 4 * (i16 & 3);
            x.rdA[mb] = (8 * h + (i16 >> 2)) * 64 * 2 + (((m >> 3) ^ tswz) << 4) + (m & 7) * 2;
        }
    } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) x.rdA[s] = c * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
    }
    if constexpr (TB) {
#pragma unroll
        for (int s = 0; s < 2; ++s) x.rdB[s] = c * DBK * 2 + (((2 * s + h) ^ aswz) << 4);
    } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int n = nb * 32 + nhalf * 16 + 4 * (i16 & 3);
            x.rdB[nb] = (8 * h + (i16 >> 2)) * 64 * 2 + (((n >> 3) ^ tswz) << 4) + (n & 7) * 2;
        }
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // This wave's K tiles: kt0 + wave, kt0 + wave + 4, ... below kt1; past
    // the last, the last one is re-fetched (landed, never used).
    const int64_t ktiles = kt1 - kt0;
    const int64_t nj = ktiles > wave ? (ktiles - wave + 3) / 4 : 0;
    auto ktile = [&](int64_t j) {
        const int64_t kt = wave + 4 * j;
        return kt0 + (kt < ktiles ? kt : ktiles - 1);
    };
    auto stage_ptr = [&](int64_t j) {
        return reinterpret_cast<const char *>(lds) + wave * WS_RING + (j % DSTAGES) * WS_STAGE;
    };
    constexpr int P = 8;                 // loads per tile
    constexpr int R = (TA ? 4 : 2) + (TB ? 2 : 4);
    if (nj > 0) {
#pragma unroll
        for (int st = 0; st < DSTAGES - 1; ++st)
#pragma unroll
            for (int l = 0; l < P; ++l) ws_loads(x, st, ktile(st), l);
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"((DSTAGES - 2) * P) : "memory");
        Frag16<128, 128, TA, TB> f0, f1;
#pragma unroll
        for (int r = 0; r < R; ++r) ws_read(f0, stage_ptr(0), x, 0, r);
        for (int64_t j = 0; j < nj; ++j) {
            const int64_t jn = j + DSTAGES - 1;
            ws_phase<kF16>(acc, f0, f1, stage_ptr(j), x, 1, static_cast<int>(jn % DSTAGES),
                           ktile(jn), true);
            asm volatile("s_waitcnt vmcnt(%0)" : : "n"((DSTAGES - 2) * P) : "memory");
            ws_phase<kF16>(acc, f1, f0, stage_ptr(j + 1), x, 0, 0, 0, false);
        }
    }
    // Every wave's loads landed and LDS reads done: the rings are free.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float *part = reinterpret_cast<float *>(lds);   // waves 1-3: [w - 1][block][reg][lane]
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                part[(((wave - 1) * 4 + b) * 16 + r) * 64 + lane] = acc[b >> 1][b & 1][r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wave != 0) return;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = acc[b >> 1][b & 1][r];
#pragma unroll
            for (int w = 0; w < 3; ++w) v += part[((w * 4 + b) * 16 + r) * 64 + lane];
            acc[b >> 1][b & 1][r] = v;
        }
    if constexpr (kSplit2) {
        // register r of block b in lane (h, c): row 8 (r / 4) + 4 h + r % 4,
        // column c of that 32 x 32 block (as store_c)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t col = n0 + (b & 1) * 32 + c;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + (b >> 1) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M && col < N) unsafeAtomicAdd(C + row * ldc + col, acc[b >> 1][b & 1][r]);
            }
        }
    } else {
        store_c(acc, C, ldc, M, N, m0, n0, 0, 0, lane);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_mfma_bf16(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn > kMaxBlocks) return hipErrorInvalidValue;
    const bool vec = aligned16(p.A) && aligned16(p.B) && p.lda % 8 == 0 && p.ldb % 8 == 0;
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
    if (vec)
        hipLaunchKernelGGL(mfma_bf16_kernel<true>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn);
    else
        hipLaunchKernelGGL(mfma_bf16_kernel<false>, dim3(static_cast<uint32_t>(tm * tn)),
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm,
                           tn);
    return hipGetLastError();
}

}  // namespace mi355gemm

namespace mi355gemm {

// Shapes the LDS-direct variant takes (see its description above).
bool supports_mfma_bf16_direct(const Problem &p)
{
    const auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    // Lane offsets of the scalar-base loads are 32-bit byte offsets within a
    // panel of up to 256 rows of K (A as written, B transposed) or 32 rows
    // of M or N (A transposed, B as written).  A factor stored with rows of
    // M or N re-fetches its last chunk past the edge, so that dimension is a
    // multiple of 8.  K > 0: the prologue loads the first tiles
    // unconditionally.
    const int64_t krows = int64_t(1) << 23, mnrows = int64_t(1) << 26;
    const bool a_ok = p.ta ? p.M % 8 == 0 && p.lda < mnrows : p.lda < krows;
    const bool b_ok = p.tb ? p.ldb < krows : p.N % 8 == 0 && p.ldb < mnrows;
    return p.K > 0 && p.K % 32 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 && p.sa % 8 == 0 &&
           p.sb % 8 == 0 && al(p.A) && al(p.B) && a_ok && b_ok;
}

namespace {

template <int TM, int TN, bool kF16, bool TA, bool TB, bool kBatch = true>
hipError_t launch_direct_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
    const dim3 grid(static_cast<uint32_t>(tm * tn * p.batch));
    // whole 16-byte chunks of C rows: C aligned, ldc, N and stride_c multiples of 4
    const bool rows_c = (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && p.ldc % 4 == 0 &&
                        p.N % 4 == 0 && p.sc % 4 == 0;
    if (rows_c)
        hipLaunchKernelGGL((mfma_bf16_direct_kernel<TM, TN, true, TA, TB, kBatch, kF16>), grid,
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc,
                           tm, tn, p.sa, p.sb, p.sc, p.batch);
    else
        hipLaunchKernelGGL((mfma_bf16_direct_kernel<TM, TN, false, TA, TB, kBatch, kF16>), grid,
                           dim3(kThreads), 0, s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc,
                           tm, tn, p.sa, p.sb, p.sc, p.batch);
    return hipGetLastError();
}

template <bool kF16, bool TA, bool TB, bool kBatch = true>
hipError_t launch_d16_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
    const dim3 grid(static_cast<uint32_t>(tm * tn * p.batch));
    const bool rows_c = (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && p.ldc % 4 == 0 &&
                        p.N % 4 == 0 && p.sc % 4 == 0;
    if (rows_c)
        hipLaunchKernelGGL((mfma_bf16_d16_kernel<true, TA, TB, kBatch, kF16>), grid, dim3(kThreads), 0,
                           s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm, tn, p.sa, p.sb,
                           p.sc, p.batch);
    else
        hipLaunchKernelGGL((mfma_bf16_d16_kernel<false, TA, TB, kBatch, kF16>), grid, dim3(kThreads), 0,
                           s, p.M, p.N, p.K, A, p.lda, B, p.ldb, p.C, p.ldc, tm, tn, p.sa, p.sb,
                           p.sc, p.batch);
    return hipGetLastError();
}

// The 256 x 256 tile runs on the 16 x 16 x 32 instruction, the smaller
// tiles on the 32 x 32 x 16 one.
template <int TM, int TN, bool kF16 = false>
hipError_t launch_direct(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + TM - 1) / TM, tn = (p.N + TN - 1) / TN;
    if (tm * tn * p.batch > kMaxBlocks || !supports_mfma_bf16_direct(p)) return hipErrorInvalidValue;
    if constexpr (TM == 256 && TN == 256) {
        if (p.ta && p.tb) return launch_d16_layout<kF16, true, true>(p, s, tm, tn);
        if (p.ta) return launch_d16_layout<kF16, true, false>(p, s, tm, tn);
        if (p.tb) return launch_d16_layout<kF16, false, true>(p, s, tm, tn);
        if (p.batch != 1) return launch_d16_layout<kF16, false, false>(p, s, tm, tn);
        return launch_d16_layout<kF16, false, false, false>(p, s, tm, tn);
    } else {
        if (p.ta && p.tb) return launch_direct_layout<TM, TN, kF16, true, true>(p, s, tm, tn);
        if (p.ta) return launch_direct_layout<TM, TN, kF16, true, false>(p, s, tm, tn);
        if (p.tb) return launch_direct_layout<TM, TN, kF16, false, true>(p, s, tm, tn);
        if (p.batch != 1) return launch_direct_layout<TM, TN, kF16, false, false>(p, s, tm, tn);
        return launch_direct_layout<TM, TN, kF16, false, false, false>(p, s, tm, tn);
    }
}

}  // namespace

hipError_t launch_mfma_bf16_direct(const Problem &p, hipStream_t s) { return launch_direct<256, 256>(p, s); }
hipError_t launch_mfma_bf16_direct128(const Problem &p, hipStream_t s) { return launch_direct<128, 128>(p, s); }
hipError_t launch_mfma_bf16_direct64(const Problem &p, hipStream_t s) { return launch_direct<64, 64>(p, s); }

// The K-split-over-waves 64 x 64 tile: the LDS-direct layout conditions, a
// single product.
bool supports_mfma_bf16_wsplit(const Problem &p)
{
    return p.batch == 1 && supports_mfma_bf16_direct(p);
}

bool supports_mfma_bf16_wsplit2(const Problem &p)
{
    return supports_mfma_bf16_wsplit(p) && p.K >= 2 * DBK;
}

namespace {
template <bool TA, bool TB>
void launch_wsplit_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    hipLaunchKernelGGL((mfma_bf16_wsplit_kernel<TA, TB, false>), dim3(static_cast<uint32_t>(tm * tn)),
                       dim3(kThreads), 0, s, p.M, p.N, p.K, static_cast<const uint16_t *>(p.A),
                       p.lda, static_cast<const uint16_t *>(p.B), p.ldb, p.C, p.ldc, tm, tn);
}
}  // namespace

hipError_t launch_mfma_bf16_wsplit(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + 63) / 64, tn = (p.N + 63) / 64;
    if (tm * tn > kMaxBlocks || !supports_mfma_bf16_wsplit(p)) return hipErrorInvalidValue;
    if (p.ta && p.tb) launch_wsplit_layout<true, true>(p, s, tm, tn);
    else if (p.ta) launch_wsplit_layout<true, false>(p, s, tm, tn);
    else if (p.tb) launch_wsplit_layout<false, true>(p, s, tm, tn);
    else launch_wsplit_layout<false, false>(p, s, tm, tn);
    return hipGetLastError();
}

namespace {
template <bool TA, bool TB>
void launch_wsplit2_layout(const Problem &p, hipStream_t s, int64_t tm, int64_t tn)
{
    hipLaunchKernelGGL((mfma_bf16_wsplit_kernel<TA, TB, false, true>),
                       dim3(static_cast<uint32_t>(2 * tm * tn)), dim3(kThreads), 0, s, p.M, p.N,
                       p.K, static_cast<const uint16_t *>(p.A), p.lda,
                       static_cast<const uint16_t *>(p.B), p.ldb, p.C, p.ldc, tm, tn);
}
}  // namespace

// The same tiles with the K range split over two work-groups per tile (twice
// the CUs streaming operands); C is first set to -0.0 by a fill kernel on
// the same stream.  K of at least two 32-wide tiles.
hipError_t launch_mfma_bf16_wsplit2(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + 63) / 64, tn = (p.N + 63) / 64;
    if (2 * tm * tn > kMaxBlocks || !supports_mfma_bf16_wsplit2(p)) return hipErrorInvalidValue;
    // -0.0 is the identity of fp32 addition: -0 + x is x for every x
    const hipError_t e = launch_fill(p, -0.0f, s);
    if (e != hipSuccess) return e;
    if (p.ta && p.tb) launch_wsplit2_layout<true, true>(p, s, tm, tn);
    else if (p.ta) launch_wsplit2_layout<true, false>(p, s, tm, tn);
    else if (p.tb) launch_wsplit2_layout<false, true>(p, s, tm, tn);
    else launch_wsplit2_layout<false, false>(p, s, tm, tn);
    return hipGetLastError();
}

hipError_t launch_mfma_f16_direct(const Problem &p, hipStream_t s) { return launch_direct<256, 256, true>(p, s); }

// 8-bit operands: K a multiple of 64 bytes (one tile), the general 8-bit
// layout conditions, and lane offsets within 32 bits over the 256 rows of
// a panel.
bool supports_mfma_fp8_direct(const Problem &p)
{
    const int64_t krows = int64_t(1) << 24;   // bytes per row
    return supports_fp8(p) && p.K > 0 && p.K % 64 == 0 && p.lda < krows && p.ldb < krows;
}

namespace {

template <int TM, int TN, bool kRowsC, bool kBatch, bool kMX = false>
void launch_fp8_fmt(const Problem &p, const dim3 &grid, int64_t tm, int64_t tn, hipStream_t s)
{
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
#define MI355_FP8_LAUNCH(F)                                                                        \
    hipLaunchKernelGGL((mfma_fp8_direct_kernel<TM, TN, kRowsC, kBatch, F, kMX>), grid,            \
                       dim3(kThreads), 0, s, p.M, p.N, p.K / 2, A, p.lda / 2, B, p.ldb / 2, p.C,  \
                       p.ldc, tm, tn, p.sa / 2, p.sb / 2, p.sc, p.batch, p.xa, p.ldxa, p.xb,      \
                       p.ldxb)
    switch (2 * p.fa + p.fb) {
    case 0: MI355_FP8_LAUNCH(0); break;
    case 1: MI355_FP8_LAUNCH(1); break;
    case 2: MI355_FP8_LAUNCH(2); break;
    default: MI355_FP8_LAUNCH(3); break;
    }
#undef MI355_FP8_LAUNCH
}

template <int TM, int TN>
hipError_t launch_fp8_direct(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + TM - 1) / TM, tn = (p.N + TN - 1) / TN;
    if (tm * tn * p.batch > kMaxBlocks || !supports_mfma_fp8_direct(p)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(tm * tn * p.batch));
    const bool rows_c = (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && p.ldc % 4 == 0 &&
                        p.N % 4 == 0 && p.sc % 4 == 0;
    if (p.xa) {   // MX block scales: a single product
        if (p.batch != 1) return hipErrorInvalidValue;
        if (rows_c) launch_fp8_fmt<TM, TN, true, false, true>(p, grid, tm, tn, s);
        else launch_fp8_fmt<TM, TN, false, false, true>(p, grid, tm, tn, s);
    } else if (p.batch != 1) {
        if (rows_c) launch_fp8_fmt<TM, TN, true, true>(p, grid, tm, tn, s);
        else launch_fp8_fmt<TM, TN, false, true>(p, grid, tm, tn, s);
    } else {
        if (rows_c) launch_fp8_fmt<TM, TN, true, false>(p, grid, tm, tn, s);
        else launch_fp8_fmt<TM, TN, false, false>(p, grid, tm, tn, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_fp8_direct128(const Problem &p, hipStream_t s) { return launch_fp8_direct<128, 128>(p, s); }
hipError_t launch_mfma_fp8_direct256x128(const Problem &p, hipStream_t s) { return launch_fp8_direct<256, 128>(p, s); }
hipError_t launch_mfma_fp8_direct256(const Problem &p, hipStream_t s) { return launch_fp8_direct<256, 256>(p, s); }
hipError_t launch_mfma_f16_direct128(const Problem &p, hipStream_t s) { return launch_direct<128, 128, true>(p, s); }

}  // namespace mi355gemm
