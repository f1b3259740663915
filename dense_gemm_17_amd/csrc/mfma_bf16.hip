// bf16-in / fp32-accumulate matrix-core family: v_mfma_f32_32x32x16_bf16.
//
// The matrix-instruction rung of the kernel ladder ("Bare Metal Bard", page
// 1, first paragraph) with bf16 operands (vidyal.ai Part 6, "Tensor Cores":
// what one instruction computes, feeding it from shared memory without bank
// conflicts, and what BF16 costs in accuracy).  A bf16 x bf16 product is
// exact in fp32, so the only rounding is the fp32 accumulation.
//
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

// Chunk permutation of an A row in LDS.  With 8 chunks per row (K step 64)
// any 16 consecutive rows read at one logical chunk occupy distinct 16-byte
// slots modulo 256 bytes, and any 8 consecutive rows distinct slots modulo
// 128 bytes; with 4 chunks per row (K step 32) the same holds for the
// 64-byte rows.
template <int kChunks>
__device__ __forceinline__ int a_swz(int row)
{
    if constexpr (kChunks == 8) return (row + (row >> 3)) & 7;
    else return ((row >> 1) ^ (row >> 3)) & 3;
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

// Epilogue: register r of block (mb, nb) in lane (h, c) is C row
// 8*(r/4) + 4*h + r%4, column c of that 32 x 32 block.
__device__ __forceinline__ void store_c(const f32x16 (&acc)[4][4], float *__restrict__ C,
                                        int64_t ldc, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                        int wm, int wn, int lane)
{
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int64_t col = n0 + wn * 128 + nb * 32 + c;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) C[row * ldc + col] = acc[mb][nb][r];
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
// Direct variant: global -> LDS with gfx950's LDS-direct 128-bit loads
// (global_load_lds_dwordx4), no register staging and no LDS write
// instructions, into a ring of kStages LDS stages so that the loads for tile
// t + kStages - 1 are in flight while tile t is multiplied.  One such load
// per wave writes 1 KiB of LDS at consecutive 16-byte slots in lane order;
// choosing which global chunk each lane fetches realises the same swizzled
// layouts as above.  Shapes: K a multiple of the K step, N a multiple of 8,
// 16-byte aligned A and B with lda and ldb multiples of 8 (the dispatch table
// checks this).  Rows of A past M and columns of B past N are fetched from
// the last valid row / chunk instead (their products land only in rows and
// columns of C that are not stored).

template <int kBK>
struct DirectShape {
    static constexpr int kAInst = BM * kBK * 2 / 1024 / 4;   // LDS-direct loads per wave for A
    static constexpr int kBInst = kBK * BN * 2 / 1024 / 4;   // ... for B
    static constexpr int kPerTile = kAInst + kBInst;
    static constexpr int kStageElems = BM * kBK + kBK * BN;  // bf16 elements per stage
};

// One LDS-direct 128-bit load: M0 holds the wave's LDS destination, each lane
// fetches 16 bytes from `src` and the hardware writes them to M0 + 16 * lane.
// Written as inline assembly on purpose: the compiler's wait-count pass does
// not see these loads, so it does not drain them before every LDS read; the
// kernel waits for them itself (wait_all_lds_and_vm_then_barrier) with exact
// counts.
// M0 is declared clobbered.  The s_nop covers the M0-write hazard.
__device__ __forceinline__ void lds_direct_load16(const void *src, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) void *)(p)));
}

template <int kBK>
__device__ __forceinline__ void issue_tile(uint16_t *stage, const uint16_t *const (&asrc)[DirectShape<kBK>::kAInst],
                                           const uint16_t *const (&bsrc)[DirectShape<kBK>::kBInst],
                                           int64_t k0, int64_t ldb, int wave)
{
    using S = DirectShape<kBK>;
    const uint32_t a_dst = lds_offset(stage) + wave * S::kAInst * 1024;
    const uint32_t b_dst = lds_offset(stage + BM * kBK) + wave * S::kBInst * 1024;
#pragma unroll
    for (int i = 0; i < S::kAInst; ++i)
        lds_direct_load16(asrc[i] + k0, __builtin_amdgcn_readfirstlane(a_dst + i * 1024));
#pragma unroll
    for (int i = 0; i < S::kBInst; ++i)
        lds_direct_load16(bsrc[i] + k0 * ldb, __builtin_amdgcn_readfirstlane(b_dst + i * 1024));
}

// Operand fragments of one 16-wide K slice for a wave's 4 x 4 MFMA blocks:
// A as one 8-element register quad per 32-row block, B as two 4-element
// halves (k 0-3 and 4-7 of the lane's eight) per 32-column block.
struct Frag16 {
    bf16x8 a[4];
    bf16x4 blo[4], bhi[4];
};

// Slice reads are issued one at a time (12 per slice: 4 A reads, 8 B
// transposing reads) so they can be slotted between MFMAs.
template <int kBK>
struct SliceReader {
    const uint16_t *As, *Bs;
    int s, wm, wn, lane;

    __device__ __forceinline__ void read(Frag16 &f, int j) const
    {
        const int h = lane >> 5, c = lane & 31;
        const int i = lane & 15, nhalf = (lane >> 4) & 1;
        if (j < 4) {
            const int row = wm * 128 + j * 32 + c;
            const u16x8 v = *reinterpret_cast<const u16x8 *>(
                As + row * kBK + (((2 * s + h) ^ a_swz<kBK / 8>(row)) << 3));
            f.a[j] = __builtin_bit_cast(bf16x8, v);
        } else {
            const int nb = (j - 4) >> 1, upper = (j - 4) & 1;
            const int k_lo = 16 * s + 8 * h + (i >> 2);
            const int n = wn * 128 + nb * 32 + nhalf * 16 + 4 * (i & 3);
            const uint16_t *p0 = Bs + k_lo * BN + (((n >> 3) ^ b_swz(k_lo)) << 3) + (n & 7);
            if (upper) f.bhi[nb] = read_tr(p0 + 4 * BN);
            else f.blo[nb] = read_tr(p0);
        }
    }
};

__device__ __forceinline__ void mfma_one(f32x16 (&acc)[4][4], const Frag16 &f, int q)
{
    const int mb = q >> 2, nb = q & 3;
    const bf16x8 b = __builtin_shufflevector(f.blo[nb], f.bhi[nb], 0, 1, 2, 3, 4, 5, 6, 7);
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mb], b, acc[mb][nb], 0, 0, 0);
}

// The 16 MFMAs of slice `cur`, with the 12 reads of slice `nxt` slotted
// after MFMAs 0..11 and (if do_loads) this wave's LDS-direct loads of a later
// tile after every other MFMA.  sched_barrier(0) pins that order so that the
// matrix unit keeps running while reads and loads are in flight; the first
// MFMA waits only for `cur`, whose reads went out a whole slice earlier.
template <int kBK>
__device__ __forceinline__ void mfma_phase(
    f32x16 (&acc)[4][4], const Frag16 &cur, Frag16 &nxt, const SliceReader<kBK> &rd,
    uint16_t *stage, const uint16_t *const (&asrc)[DirectShape<kBK>::kAInst],
    const uint16_t *const (&bsrc)[DirectShape<kBK>::kBInst], int64_t k0, int64_t ldb, int wave,
    bool do_loads)
{
    using S = DirectShape<kBK>;
    constexpr int kLoads = S::kAInst + S::kBInst;
    static_assert(16 % kLoads == 0, "loads must divide the MFMA count");
    constexpr int kEvery = 16 / kLoads;
    const uint32_t a_dst = lds_offset(stage) + wave * S::kAInst * 1024;
    const uint32_t b_dst = lds_offset(stage + BM * kBK) + wave * S::kBInst * 1024;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        mfma_one(acc, cur, q);
        __builtin_amdgcn_sched_barrier(0);
        if (q < 12) rd.read(nxt, q);
        if (q % kEvery == kEvery - 1 && do_loads) {
            const int l = q / kEvery;
            if (l < S::kAInst)
                lds_direct_load16(asrc[l] + k0, __builtin_amdgcn_readfirstlane(a_dst + l * 1024));
            else
                lds_direct_load16(bsrc[l - S::kAInst] + k0 * ldb,
                                  __builtin_amdgcn_readfirstlane(b_dst + (l - S::kAInst) * 1024));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int kCntVm>
__device__ __forceinline__ void wait_all_lds_and_vm_then_barrier()
{
    // This wave's LDS reads complete (lgkmcnt 0) and its LDS-direct loads
    // down to kCntVm in flight, then the work-group barrier.  Inline assembly
    // so that the compiler's wait-count pass cannot weaken the LDS part: it
    // is what guarantees that no wave still reads a stage another wave
    // refills after the barrier.
    static_assert(kCntVm >= 0 && kCntVm <= 63, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(kCntVm) : "memory");
}

template <int kBK, int kStages>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_bf16_direct_kernel(int64_t M, int64_t N, int64_t K, const uint16_t *__restrict__ A,
                             int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
                             float *__restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n)
{
    using S = DirectShape<kBK>;
    static_assert(kBK == 32, "two 16-wide K slices per tile");
    static_assert(kStages >= 3, "the ring needs a stage being filled, one in flight, one read");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages * S::kStageElems];

    const TileCoord t = map_tile(tiles_m, tiles_n, kGroup);
    const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Per-lane source of every LDS-direct load of this wave, at k = 0.
    constexpr int kAChunksPerRow = kBK / 8;
    const uint16_t *asrc[S::kAInst];
    const uint16_t *bsrc[S::kBInst];
#pragma unroll
    for (int i = 0; i < S::kAInst; ++i) {
        const int p = (wave * S::kAInst + i) * 64 + lane;    // LDS chunk this lane fills
        const int row = p / kAChunksPerRow, slot = p % kAChunksPerRow;
        const int c = slot ^ a_swz<kAChunksPerRow>(row);
        const int64_t r = (m0 + row < M) ? m0 + row : M - 1;
        asrc[i] = A + r * lda + 8 * c;
    }
#pragma unroll
    for (int i = 0; i < S::kBInst; ++i) {
        const int p = (wave * S::kBInst + i) * 64 + lane;
        const int row = p >> 5, slot = p & 31;
        const int c = slot ^ b_swz(row);
        const int64_t col = (n0 + 8 * c < N) ? n0 + 8 * c : N - 8;
        bsrc[i] = B + row * ldb + col;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t ktiles = K / kBK;
    auto stage = [&](int64_t kt) { return lds + (kt % kStages) * S::kStageElems; };

    // Prologue: tiles 0 .. kStages-2 in flight, wait for tile 0, read its
    // first slice.
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < ktiles) issue_tile<kBK>(stage(s), asrc, bsrc, s * kBK, ldb, wave);
    if (ktiles >= kStages - 1) wait_all_lds_and_vm_then_barrier<(kStages - 2) * S::kPerTile>();
    else wait_all_lds_and_vm_then_barrier<0>();

    Frag16 f0, f1;
    {
        const SliceReader<kBK> rd{stage(0), stage(0) + BM * kBK, 0, wm, wn, lane};
#pragma unroll
        for (int j = 0; j < 12; ++j) rd.read(f0, j);
    }

    // Tile kt:  MFMAs on slice 0 with the reads of slice 1 and the loads of
    // tile kt + kStages - 1 slotted in (that stage was last read in tile
    // kt - 1, which every wave finished before the previous barrier) | wait
    // until tile kt + 1 has landed everywhere and this wave's reads are done,
    // barrier | MFMAs on slice 1 with the reads of slice 0 of tile kt + 1 (in
    // the last tile, a harmless re-read of the current stage).
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        uint16_t *cur = stage(kt);
        const int64_t nxt = kt + kStages - 1;
        const SliceReader<kBK> rd1{cur, cur + BM * kBK, 1, wm, wn, lane};
        mfma_phase<kBK>(acc, f0, f1, rd1, stage(nxt), asrc, bsrc, nxt * kBK, ldb, wave,
                        nxt < ktiles);
        // In flight after this: tiles kt + 2 .. min(nxt, ktiles - 1).
        if (nxt < ktiles) wait_all_lds_and_vm_then_barrier<(kStages - 2) * S::kPerTile>();
        else wait_all_lds_and_vm_then_barrier<0>();
        uint16_t *n1 = stage(kt + 1 < ktiles ? kt + 1 : kt);
        const SliceReader<kBK> rd0{n1, n1 + BM * kBK, 0, wm, wn, lane};
        mfma_phase<kBK>(acc, f1, f0, rd0, n1, asrc, bsrc, 0, ldb, wave, false);
    }

    store_c(acc, C, ldc, M, N, m0, n0, wm, wn, lane);
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
    return p.K % 32 == 0 && p.N % 8 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 && al(p.A) && al(p.B);
}

hipError_t launch_mfma_bf16_direct(const Problem &p, hipStream_t s)
{
    const int64_t tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
    if (tm * tn > kMaxBlocks || !supports_mfma_bf16_direct(p)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mfma_bf16_direct_kernel<32, 4>), dim3(static_cast<uint32_t>(tm * tn)),
                       dim3(kThreads), 0, s, p.M, p.N, p.K, static_cast<const uint16_t *>(p.A),
                       p.lda, static_cast<const uint16_t *>(p.B), p.ldb, p.C, p.ldc, tm, tn);
    return hipGetLastError();
}

}  // namespace mi355gemm
