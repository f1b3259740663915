// Matrix-core ceiling probe (measurement only, not part of the GEMM path).
//
// A loop of nothing but independent MFMAs, operands held in registers, no
// memory traffic: the most any kernel built on the same instruction can
// reach on this board.  The ceiling depends on the data: MI355X runs the
// bf16 matrix cores at its power limit, and the power drawn depends on the
// operand bits, so the probe multiplies operands like the benchmark's
// (random normal-range bf16 values, random fp32 values) or, for contrast,
// zeros.  Each lane's operands come from a hash of its global index and are
// fixed for the whole loop; two operand sets alternate so consecutive MFMAs
// see different bits.
//
// Built into its own library (libmi355probe.so) by dense_gemm_17_amd/build.py;
// only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Eight bf16 values with random sign, exponent in [2^-7, 2^6] and mantissa
// (xorshift32 steps from one hashed seed).
__device__ __forceinline__ bf16x8 bf16_operand(uint32_t seed)
{
    uint32_t x = mix(seed) | 1u;
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        v[e] = static_cast<unsigned short>((x & 0x8000u) | ((120u + (x >> 16) % 14u) << 7) |
                                           (x & 0x7fu));
    }
    return __builtin_bit_cast(bf16x8, v);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 e4m3 values with random sign, exponent field in [4, 10] (2^-3 .. 2^3)
// and mantissa: never the NaN pattern.
__device__ __forceinline__ i32x8 fp8_operand(uint32_t seed)
{
    uint32_t x = mix(seed) | 1u;
    i32x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t w = 0;
#pragma unroll
        for (int byte = 0; byte < 4; ++byte) {
            x ^= x << 13;
            x ^= x >> 17;
            x ^= x << 5;
            w |= ((x & 0x80u) | ((4u + (x >> 16) % 7u) << 3) | ((x >> 8) & 7u)) << (8 * byte);
        }
        v[e] = static_cast<int>(w);
    }
    return v;
}

__device__ __forceinline__ float f32_operand(uint32_t seed)
{
    const uint32_t h = mix(seed);
    return __uint_as_float((h & 0x807fffffu) | ((120u + (h >> 23) % 14u) << 23));
}

// 4 x 4 independent 32x32 accumulators per wave (one wave per SIMD, as the
// GEMM kernels run), 2 operand sets, `iters` rounds of 16 MFMAs.
template <bool kZero>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bf16_loop(float *out, int iters)
{
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    bf16x8 a[2][4], b[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[s][i] = kZero ? bf16x8{} : bf16_operand(t * 16u + s * 8u + i);
            b[s][i] = kZero ? bf16x8{} : bf16_operand(t * 16u + s * 8u + 4u + i);
        }
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][i], b[s][j], acc[i][j],
                                                                         0, 0, 0);
    }
    // One element of each accumulator keeps every MFMA live.
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += acc[i][j][0];
    out[t] = sum;
}

template <bool kZero>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fp8_loop(float *out, int iters)
{
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    i32x8 a[2][4], b[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[s][i] = kZero ? i32x8{} : fp8_operand(t * 16u + s * 8u + i);
            b[s][i] = kZero ? i32x8{} : fp8_operand(t * 16u + s * 8u + 4u + i);
        }
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[s][i], b[s][j], acc[i][j], 0, 0, 0, 127, 0, 127);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += acc[i][j][0];
    out[t] = sum;
}

template <bool kZero>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void f32_loop(float *out, int iters)
{
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    float a[2][4], b[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[s][i] = kZero ? 0.f : f32_operand(t * 16u + s * 8u + i);
            b[s][i] = kZero ? 0.f : f32_operand(t * 16u + s * 8u + 4u + i);
        }
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s][i], b[s][j], acc[i][j],
                                                                      0, 0, 0);
    }
    // One element of each accumulator keeps every MFMA live.
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += acc[i][j][0];
    out[t] = sum;
}

// Vector-ALU counterpart: 16 independent fp32 FMA chains per lane
// (acc = acc * a + b, |a| < 1 so the values stay bounded), no memory
// traffic, several waves per SIMD to cover the FMA latency.  The ceiling of
// the scalar (non-packed) fp32 FMA issue rate, which the vector-ALU GEMM
// kernel is built on.
template <bool kZero>
__global__ __launch_bounds__(256) void valu_loop(float *out, int iters)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = kZero ? 0.f : f32_operand(t * 16u + j);
    // a in [0.5, 0.99): 0.49 * (a float in [1, 2) with a hashed mantissa) + 0.01
    const float a = kZero ? 0.f : 0.49f * __uint_as_float(0x3f800000u | (mix(t ^ 0x9e3779b9u) >> 9)) + 0.01f;
    const float b = kZero ? 0.f : f32_operand(t * 16u + 15u) * 0.01f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_fmaf(acc[j], a, b);
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += acc[j];
    out[t] = sum;
}

}  // namespace

// dtype 0 = fp32 (v_mfma_f32_32x32x2_f32), 1 = bf16 (v_mfma_f32_32x32x16_bf16),
// 2 = fp32 vector FMA (valu_loop: blocks * 256 * iters * 16 FMAs of 2 flops),
// 3 = e4m3 (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales; 2*32*32*64 flops).
// One launch: `blocks` work-groups of 256 threads, each wave doing `iters`
// (even) rounds of 16 MFMAs, i.e. blocks * 4 * iters * 16 MFMAs of
// 2*32*32*2 (fp32) or 2*32*32*16 (bf16) flops.  `out` holds blocks * 256
// floats (device memory owned by the caller).  Returns a hipError_t value.
extern "C" int probe_mfma_loop(int dtype, int blocks, int iters, int zero, float *out,
                               hipStream_t stream)
{
    if (blocks <= 0 || iters <= 0 || (iters & 1) || !out || dtype < 0 || dtype > 3)
        return hipErrorInvalidValue;
    const dim3 g(blocks), b(256);
    if (dtype == 1 && zero) hipLaunchKernelGGL(bf16_loop<true>, g, b, 0, stream, out, iters);
    if (dtype == 1 && !zero) hipLaunchKernelGGL(bf16_loop<false>, g, b, 0, stream, out, iters);
    if (dtype == 0 && zero) hipLaunchKernelGGL(f32_loop<true>, g, b, 0, stream, out, iters);
    if (dtype == 0 && !zero) hipLaunchKernelGGL(f32_loop<false>, g, b, 0, stream, out, iters);
    if (dtype == 2 && zero) hipLaunchKernelGGL(valu_loop<true>, g, b, 0, stream, out, iters);
    if (dtype == 2 && !zero) hipLaunchKernelGGL(valu_loop<false>, g, b, 0, stream, out, iters);
    if (dtype == 3 && zero) hipLaunchKernelGGL(fp8_loop<true>, g, b, 0, stream, out, iters);
    if (dtype == 3 && !zero) hipLaunchKernelGGL(fp8_loop<false>, g, b, 0, stream, out, iters);
    return hipGetLastError();
}
