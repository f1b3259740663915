// Internal declarations shared by the kernel files and the C-ABI layer.
// Not installed; the public interface is include/mi355gemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355gemm {

enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2, kFp8 = 3 };

// Storage type of an IEEE binary16 operand in the kernels templated on the
// element type (bf16 operands are plain uint16_t patterns there).
struct F16Bits {
    uint16_t v;
};

// Arguments of one product after validation.  Pointers are device pointers;
// A and B are `const void*` so one signature serves both element types.
// The last fields describe the general form C_b = op(A_b) op(B_b), b < batch:
// ta / tb mark a factor stored transposed (A as K x M, B as N x K) and
// sa, sb, sc are the element distances between consecutive products.  A
// plain product has ta = tb = 0 and batch = 1; only the kernels registered
// as general read these fields.  8-bit float operands (dtype kFp8) come as
// A as written and B transposed only (ta = 0, tb = 1), with fa and fb the
// formats of A and B (0 e4m3, 1 e5m2); their sizes and strides are bytes.
// xa / xb, when not null, are MX block scales of such a product (one E8M0
// byte per 32 elements of K: block kb of row i of A at xa[kb * ldxa + i],
// of row j of Bt at xb[kb * ldxb + j]); a single product only.
struct Problem {
    int64_t M, N, K;
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    float *C; int64_t ldc;
    int dtype;
    int ta = 0, tb = 0;
    int64_t batch = 1, sa = 0, sb = 0, sc = 0;
    int fa = 0, fb = 0;
    const uint8_t *xa = nullptr, *xb = nullptr;
    int64_t ldxa = 0, ldxb = 0;
};

// True when only a general (transposed / batched) kernel can take p.
inline bool is_general(const Problem &p) { return p.ta || p.tb || p.batch != 1; }

// Arguments of the fused attention forward after validation: Q, K, V, O are
// (B, H, S, D) with unit stride along D and element strides per sequence,
// head and position; lse is null or B*H*S packed floats.  scale_log2 is the
// caller's score scale times log2(e); nqb is set by the launcher.
struct AttnArgs {
    const float *Q, *K, *V;
    float *O, *lse;
    int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss, o_sb, o_sh, o_ss;
    int64_t B, H, S;
    int causal;
    float scale_log2;
    int64_t nqb;
};
// Attention kernels: 0 = 128 queries per work-group, key tiles through LDS;
// 1 = 32 queries per work-group, key tiles split over its waves (head width
// 64); 2 = kernel 0 with 32-key tiles (head width 64).  attention_variant
// picks one (forced >= 0 overrides where it can).
int attention_variant(int64_t B, int64_t H, int64_t S, int64_t D, int forced);
hipError_t launch_attention_fwd(const AttnArgs &a, int64_t D, int variant, hipStream_t s);

// A launcher enqueues its kernel(s) for `p` on `stream` and returns the
// launch status.  It may assume p passed validation and its `supports` test.
using LaunchFn = hipError_t (*)(const Problem &p, hipStream_t stream);
using SupportsFn = bool (*)(const Problem &p);

struct KernelInfo {
    const char *name;
    int dtype;
    LaunchFn launch;
    SupportsFn supports;   // shapes / alignments this kernel can take
    bool general = false;  // also takes transposed factors and batches
};

// ---- per-family launchers (defined in the kernel files) -------------------
hipError_t launch_naive_f32(const Problem &p, hipStream_t s);
hipError_t launch_naive_bf16(const Problem &p, hipStream_t s);
hipError_t launch_fill_zero(const Problem &p, hipStream_t s);
// C (p.M x p.N, row stride p.ldc) set to `value` (the K-split kernels that
// add two halves into C start it at -0.0, the identity of fp32 addition).
hipError_t launch_fill(const Problem &p, float value, hipStream_t s);
hipError_t launch_null(hipStream_t s);
hipError_t launch_valu_f32(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_direct(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_direct128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_narrow128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_narrow128x64(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_direct64(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_narrow64(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_splitk(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_direct128x64(const Problem &p, hipStream_t s);
bool supports_mfma_f32_narrow(const Problem &p);
bool supports_mfma_f32_direct(const Problem &p);
hipError_t launch_mfma_bf16(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_direct(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_direct128(const Problem &p, hipStream_t s);
bool supports_mfma_bf16_direct(const Problem &p);
hipError_t launch_mfma_f32_batched(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_batched128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_batched(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_batched128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_batched_splitk(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f16_direct(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f16_direct128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f16_batched(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f16_batched128(const Problem &p, hipStream_t s);
hipError_t launch_skinny_f16(const Problem &p, hipStream_t s);
hipError_t launch_mfma_fp8_batched(const Problem &p, hipStream_t s);
hipError_t launch_mfma_fp8_batched128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_fp8_direct128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_fp8_direct256x128(const Problem &p, hipStream_t s);
hipError_t launch_mfma_fp8_direct256(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_direct64(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_wsplit(const Problem &p, hipStream_t s);
hipError_t launch_mfma_bf16_wsplit2(const Problem &p, hipStream_t s);
hipError_t launch_mfma_f32_direct64x2(const Problem &p, hipStream_t s);
bool supports_mfma_f32_direct64x2(const Problem &p);
bool supports_mfma_bf16_wsplit(const Problem &p);
bool supports_mfma_bf16_wsplit2(const Problem &p);
bool supports_mfma_fp8_direct(const Problem &p);
hipError_t launch_skinny_fp8(const Problem &p, hipStream_t s);
bool supports_skinny_fp8(const Problem &p);

// Layout every 8-bit kernel needs: A as written and B transposed, K, lda,
// ldb, stride_a and stride_b multiples of 16 (bytes), A and B 16-byte
// aligned, formats 0 or 1.
inline bool supports_fp8(const Problem &p)
{
    const auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    return p.dtype == kFp8 && p.ta == 0 && p.tb == 1 && (p.fa == 0 || p.fa == 1) &&
           (p.fb == 0 || p.fb == 1) && p.K % 16 == 0 && p.lda % 16 == 0 && p.ldb % 16 == 0 &&
           p.sa % 16 == 0 && p.sb % 16 == 0 && al(p.A) && al(p.B);
}
// The 256 x 256 register-staged 8-bit tile takes no MX scales.
inline bool supports_fp8_unscaled(const Problem &p) { return supports_fp8(p) && !p.xa; }
hipError_t launch_naive_f16(const Problem &p, hipStream_t s);
hipError_t launch_sum_partials(const float *W, int64_t S, int64_t M, int64_t N, float *C,
                               int64_t ldc, hipStream_t s);
hipError_t launch_skinny_f32(const Problem &p, hipStream_t s);
hipError_t launch_skinny_bf16(const Problem &p, hipStream_t s);

// Largest M the skinny (bandwidth) family takes.
constexpr int64_t kSkinnyMaxM = 16;

// Compute units of an MI355X (8 XCDs of 32); the dispatch table and the
// skinny family size their grids against it.
constexpr int64_t kCUs = 256;

// Every kernel writes each element of C once and never reads it back, so C
// goes out with the nontemporal (streaming) hint: the output stream then
// does not displace operand lines from the L2 and the last-level cache.
// Measured on bf16 products whose fp32 output dominates: 16384 x 1152 x 384
// from 38.8 to 29.0 us, 8192 x 8192 x 1024 from 182 to 158 us.
template <typename V>
__device__ __forceinline__ void store_c_stream(V *p, V v)
{
    __builtin_nontemporal_store(v, p);
}

// 1-D grids only: gridDim.x is the sole dimension with a 2^31 - 1 limit.
constexpr int64_t kMaxBlocks = 2147483647LL;

}  // namespace mi355gemm
