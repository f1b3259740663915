// Fused attention forward in fp32 ("Bare Metal Bard", page 1, third
// paragraph: a FlashAttention-style kernel that never writes the score matrix
// to memory, keeps each score tile in registers and carries a running maximum
// and sum from one tile of keys to the next).
//
// For one (sequence, head) the work-group takes 128 queries, 32 per wave,
// and walks the keys in tiles of BN (64, or 32 for sequences of up to 256
// tokens, where the smaller LDS stages and register set let three
// work-groups share a CU); each tile of K and V goes through LDS once and
// serves all four waves.  Per tile, a wave
//   1. computes the scores of its 32 queries against the tile's keys on the
//      fp32 matrix cores, transposed (S^T = K Q^T): in the 32 x 32 MFMA
//      accumulator a lane owns one column, so here a lane owns one query and
//      16 of the tile's keys, and the row statistics of the softmax are a
//      lane's own registers plus one exchange with the lane 32 away (the
//      other 16 keys of the same query);
//   2. scales the scores into the base-2 domain (scale * log2 e), masks keys
//      past the sequence or after the query (causal), raises the running
//      maximum, rescales the running sum and the output accumulators by
//      2^(m_old - m_new) and exponentiates;
//   3. multiplies the probabilities straight out of the score registers into
//      the output, again transposed (O^T += V^T P^T): a probability register
//      of lane (h, c) is exactly the B operand the MFMA wants for query c
//      and the key that register holds, so P never leaves registers; the
//      values come from LDS, one 4-byte read per MFMA.
// At the end each lane divides its query's output by the sum and writes it
// (16-byte stores), and the log-sum-exp of the query if asked for.
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x2_f32): lane (h, c),
// h = lane / 32, c = lane % 32, supplies A[c][h] and B[h][c]; accumulator
// register r of the lane is element (8 (r / 4) + 4 h + r % 4, c).  The
// contraction index of one MFMA is h, so any pairing of the two half-waves'
// terms is a valid order of the sum as long as A and B agree on it: for the
// scores the half-wave h covers head dimensions h*D/2 .. h*D/2 + D/2 - 1 (a
// lane's share of a K row is contiguous: 16-byte LDS reads, and its query's
// share of Q sits in registers for the whole kernel); for P V the terms are
// the keys exactly where the score accumulator left them.
//
// Staging: the next tile of K and V is loaded into registers (16-byte global
// loads, coalesced along the head dimension) while the current tile is
// computed, written to the other LDS buffer after it, and one barrier per
// tile separates the two.  LDS rows are padded (K: D + 4 floats, V: D + 8)
// so that the 16-byte K reads of 16 consecutive rows and the 4-byte V reads
// of two rows four apart fall in different banks.
//
// Under the causal mask a work-group visits only the key tiles up to its
// last query and a wave skips the 32-key halves past its own last query;
// work-groups with the most keys are launched first.
#include "gemm_internal.h"

namespace mi355gemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttnThreads = 256;   // four waves
constexpr int kQW = 32;             // queries per wave
constexpr int kBM = 4 * kQW;        // queries per work-group

template <int D, int BN>
struct AttnCfg {
    static_assert(D % 32 == 0 && BN % 32 == 0, "tiles of 32");
    static constexpr int DH = D / 2;                       // head dims per half-wave
    static constexpr int KS = D + 4;                       // LDS row stride of K (floats)
    static constexpr int VS = D + 8;                       // LDS row stride of V (floats)
    static constexpr int kStage = BN * (KS + VS);          // floats per LDS stage
    static constexpr int kLoads = BN * D / 4 / kAttnThreads;   // 16-byte loads per thread per tensor
    static_assert(kLoads * 4 * kAttnThreads == BN * D, "whole tiles per pass");
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// x where keep is all ones, +0 where it is zero (a bitwise select, so the
// load of x stays unconditional).
__device__ __forceinline__ float masked(float x, uint32_t keep)
{
    return __uint_as_float(__float_as_uint(x) & keep);
}

template <int D, int BN>
__global__ __launch_bounds__(kAttnThreads, (D == 64 && BN == 32) ? 3 : 2) void attention_fwd_kernel(AttnArgs a)
{
    using C = AttnCfg<D, BN>;
    __shared__ __attribute__((aligned(16))) float lds[2 * C::kStage];

    const int64_t BH = a.B * a.H;
    const int64_t blk = blockIdx.x;
    // Under the causal mask the last query tiles have the most keys: they go
    // first, so the short ones fill in behind them.
    const int64_t qb = a.causal ? a.nqb - 1 - blk / BH : blk / BH;
    const int64_t bh = blk % BH;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, c = lane & 31;

    const int64_t S = a.S;
    const int64_t q0 = qb * kBM;                 // first query of the work-group
    const int64_t qw = q0 + wave * kQW;          // first query of this wave
    const int64_t qi = qw + c;                   // this lane's query
    const bool q_ok = qi < S;

    const float *Qp = a.Q + bi * a.q_sb + hi * a.q_sh;
    const float *Kp = a.K + bi * a.k_sb + hi * a.k_sh;
    const float *Vp = a.V + bi * a.v_sb + hi * a.v_sh;

    // This lane's share of its query: head dimensions h*DH .. h*DH + DH - 1.
    float qf[C::DH];
    {
        const float *src = Qp + (q_ok ? qi : 0) * a.q_ss + h * C::DH;
#pragma unroll
        for (int t = 0; t < C::DH / 4; ++t) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 4 * t);
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[4 * t + e] = q_ok ? v[e] : 0.f;
        }
    }

    // Keys the work-group visits, and the keys this wave can see.
    const int64_t kend = a.causal ? (S < q0 + kBM ? S : q0 + kBM) : S;
    const int64_t ntiles = (kend + BN - 1) / BN;
    const int64_t wend = qw >= S ? 0 : (a.causal ? (S < qw + kQW ? S : qw + kQW) : S);

    f32x16 o[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float m = neg_inf();     // running maximum (base-2 domain), shared by the lane pair
    float l = 0.f;           // this lane's part of the running sum

    // Tile t's rows of K and V: loaded raw into registers (rows past S read
    // row 0), zeroed past S only when written to LDS, so nothing uses the
    // loaded values before then and the loads stay in flight through the
    // tile computed meanwhile.
    f32x4 kreg[C::kLoads], vreg[C::kLoads];
    auto gload = [&](int64_t t) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int f = threadIdx.x + kAttnThreads * i;
            const int row = f / (D / 4), col = (f % (D / 4)) * 4;
            const int64_t key = t * BN + row;
            const int64_t kk = key < S ? key : 0;
            kreg[i] = *reinterpret_cast<const f32x4 *>(Kp + kk * a.k_ss + col);
            vreg[i] = *reinterpret_cast<const f32x4 *>(Vp + kk * a.v_ss + col);
        }
    };
    auto lstore = [&](int buf, int64_t t) {
        float *Ks = lds + buf * C::kStage;
        float *Vs = Ks + BN * C::KS;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) {
            const int f = threadIdx.x + kAttnThreads * i;
            const int row = f / (D / 4), col = (f % (D / 4)) * 4;
            const uint32_t keep = t * BN + row < S ? ~0u : 0u;
            f32x4 kv, vv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kv[e] = masked(kreg[i][e], keep);
                vv[e] = masked(vreg[i][e], keep);
            }
            *reinterpret_cast<f32x4 *>(Ks + row * C::KS + col) = kv;
            *reinterpret_cast<f32x4 *>(Vs + row * C::VS + col) = vv;
        }
    };

    if (ntiles > 0) {
        gload(0);
        lstore(0, 0);
        if (ntiles > 1) gload(1);
    }
    __syncthreads();

    const float sl2 = a.scale_log2;
    for (int64_t t = 0; t < ntiles; ++t) {
        const float *Ks = lds + (t & 1) * C::kStage;
        const float *Vs = Ks + BN * C::KS;
        const int64_t k0 = t * BN;
        if (k0 < wend) {
            // 1. scores, transposed: s[sb] holds keys k0 + 32 sb + (8 (r/4) + 4 h + r%4)
            //    for query c of this wave.  The 32-key halves the wave sees
            //    (both but on its diagonal tile) run as independent MFMA
            //    chains, interleaved.
            f32x16 s[BN / 32];
#pragma unroll
            for (int sb = 0; sb < BN / 32; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
            const bool all_halves = k0 + BN <= wend;
#pragma unroll
            for (int u = 0; u < C::DH / 4; ++u) {
                f32x4 kv[BN / 32];
#pragma unroll
                for (int sb = 0; sb < BN / 32; ++sb)
                    if (sb == 0 || all_halves)
                        kv[sb] = *reinterpret_cast<const f32x4 *>(Ks + (32 * sb + c) * C::KS +
                                                                  h * C::DH + 4 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int sb = 0; sb < BN / 32; ++sb)
                        if (sb == 0 || all_halves)
                            s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[sb][e], qf[4 * u + e],
                                                                          s[sb], 0, 0, 0);
            }
            if (!all_halves) {
                // the diagonal tile's later halves, each only if the wave sees it
#pragma unroll
                for (int sb = 1; sb < BN / 32; ++sb) {
                    if (k0 + 32 * sb >= wend) break;
                    const float *krow = Ks + (32 * sb + c) * C::KS + h * C::DH;
#pragma unroll
                    for (int u = 0; u < C::DH / 4; ++u) {
                        const f32x4 kv = *reinterpret_cast<const f32x4 *>(krow + 4 * u);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[4 * u + e],
                                                                          s[sb], 0, 0, 0);
                    }
                }
            }
            // 2. mask (only where a key can be past the sequence or after a
            //    query of this wave), scale, running maximum and sum
            float mx = neg_inf();
            const bool masked = k0 + BN > S || (a.causal && k0 + BN - 1 > qw);
            if (masked) {
                const int kl = static_cast<int>(k0) + 4 * h;   // keys and queries fit in 32 bits
                const int lim = a.causal ? (qi < S ? static_cast<int>(qi) : static_cast<int>(S) - 1)
                                         : static_cast<int>(S) - 1;
#pragma unroll
                for (int sb = 0; sb < BN / 32; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kl + 32 * sb + 8 * (r >> 2) + (r & 3);
                        const float x = key <= lim ? s[sb][r] * sl2 : neg_inf();
                        s[sb][r] = x;
                        mx = fmaxf(mx, x);
                    }
            } else {
#pragma unroll
                for (int sb = 0; sb < BN / 32; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = s[sb][r] * sl2;
                        s[sb][r] = x;
                        mx = fmaxf(mx, x);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, mx);
            const float m_use = m_new == neg_inf() ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m - m_use);
            float psum = 0.f;
#pragma unroll
            for (int sb = 0; sb < BN / 32; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(s[sb][r] - m_use);
                    s[sb][r] = p;
                    psum += p;
                }
            l = l * alpha + psum;
            m = m_new;
#pragma unroll
            for (int d = 0; d < D / 32; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
            // 3. O^T += V^T P^T, the probabilities straight from the score registers
#pragma unroll
            for (int sb = 0; sb < BN / 32; ++sb) {
                if (k0 + 32 * sb < wend) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float *vrow = Vs + (32 * sb + 8 * (r >> 2) + 4 * h + (r & 3)) * C::VS + c;
#pragma unroll
                        for (int d = 0; d < D / 32; ++d)
                            o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * d], s[sb][r],
                                                                         o[d], 0, 0, 0);
                    }
                }
            }
        }
        if (t + 1 < ntiles) lstore((t + 1) & 1, t + 1);
        if (t + 2 < ntiles) gload(t + 2);
        __syncthreads();
    }

    if (!q_ok) return;
    const float lt = l + __shfl_xor(l, 32);
    const float inv = 1.f / lt;
    float *Op = a.O + bi * a.o_sb + hi * a.o_sh + qi * a.o_ss;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = o[d][4 * g + j] * inv;
            *reinterpret_cast<f32x4 *>(Op + 32 * d + 8 * g + 4 * h) = v;
        }
    if (a.lse && h == 0)
        a.lse[bh * S + qi] = (m + __builtin_amdgcn_logf(lt)) * 0.693147180559945309f;
}

// ---- few sequences and heads: the keys split over the waves ------------------
// With few (sequence, head) pairs the kernel above runs on a handful of
// CUs, each walking every key tile of its 128 queries alone (a single GPT
// sequence: 6 heads x 2 query tiles = 12 work-groups).  Here a work-group
// takes 32 queries and its four waves split the key tiles between them
// (wave w takes tiles w, w + 4, ...), each with its own running maximum,
// sum and output in registers; at the end the four partial softmaxes are
// merged through LDS (the maximum of the maxima m, each part's sum and
// output scaled by 2^(m_w - m), output over summed weights).  Each wave
// reads its K and V tiles straight from memory into the MFMA operand
// layout (a lane's 16-byte pieces of its key's row of K; 4-byte values of
// V, 32 lanes on one row), the next tile's while the current one is
// computed (two register sets, one wave per SIMD so that both fit; a single
// GPT sequence, causal: 11.4 -> 11.0 us).  Head width 64.
constexpr int kSplitQ = 32;   // queries per work-group
constexpr int kSplitBN = 32;  // keys per tile

__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_fwd_split_kernel(AttnArgs a)
{
    constexpr int D = 64, DH = D / 2;
    __shared__ float mrg_o[3][D / 32][16][64];   // waves 1..3: output registers by lane
    __shared__ float mrg_ml[3][2][64];           // waves 1..3: maximum and sum by lane

    const int64_t BH = a.B * a.H;
    const int64_t blk = blockIdx.x;
    const int64_t nq = (a.S + kSplitQ - 1) / kSplitQ;
    const int64_t qb = a.causal ? nq - 1 - blk / BH : blk / BH;
    const int64_t bh = blk % BH;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, c = lane & 31;
    const int S = static_cast<int>(a.S);
    const int q0 = static_cast<int>(qb) * kSplitQ;
    const int qi = q0 + c;
    const bool q_ok = qi < S;

    const float *Qp = a.Q + bi * a.q_sb + hi * a.q_sh;
    const float *Kp = a.K + bi * a.k_sb + hi * a.k_sh;
    const float *Vp = a.V + bi * a.v_sb + hi * a.v_sh;

    float qf[DH];
    {
        const float *src = Qp + static_cast<int64_t>(q_ok ? qi : 0) * a.q_ss + h * DH;
#pragma unroll
        for (int t = 0; t < DH / 4; ++t) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 4 * t);
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[4 * t + e] = q_ok ? v[e] : 0.f;
        }
    }
    const int kend = a.causal ? (S < q0 + kSplitQ ? S : q0 + kSplitQ) : S;
    const int ntiles = (kend + kSplitBN - 1) / kSplitBN;
    const int lim = a.causal ? (q_ok ? qi : S - 1) : S - 1;   // last key this lane sees

    f32x16 o[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float m = neg_inf(), l = 0.f;

    // tile t's operands: K row (key t*32 + c), this half's 32 dims; V at
    // keys t*32 + 8 (r/4) + 4 h + r%4, dims 32 d + c (zero past S)
    auto load = [&](f32x4 (&kf)[DH / 4], float (&vf)[16][D / 32], int t) {
        const int key = t * kSplitBN + c;
        const bool ok = key < S;
        const uint32_t kkeep = ok ? ~0u : 0u;
        const float *kr = Kp + static_cast<int64_t>(ok ? key : 0) * a.k_ss + h * DH;
#pragma unroll
        for (int u = 0; u < DH / 4; ++u) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(kr + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) kf[u][e] = masked(v[e], kkeep);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int vk = t * kSplitBN + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool vok = vk < S;
            const uint32_t vkeep = vok ? ~0u : 0u;
            const float *vr = Vp + static_cast<int64_t>(vok ? vk : 0) * a.v_ss + c;
#pragma unroll
            for (int d = 0; d < D / 32; ++d) vf[r][d] = masked(vr[32 * d], vkeep);
        }
    };

    const float sl2 = a.scale_log2;
    auto tile = [&](const f32x4 (&kc)[DH / 4], const float (&vc)[16][D / 32], int t) {
        f32x16 sc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
        for (int u = 0; u < DH / 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sc = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[u][e], qf[4 * u + e], sc, 0, 0, 0);
        float mx = neg_inf();
        const int kl = t * kSplitBN + 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kl + 8 * (r >> 2) + (r & 3);
            const float x = key <= lim ? sc[r] * sl2 : neg_inf();
            sc[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == neg_inf() ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(sc[r] - m_use);
            sc[r] = pr;
            psum += pr;
        }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int d = 0; d < D / 32; ++d)
                o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vc[r][d], sc[r], o[d], 0, 0, 0);
    };

    // Two register sets: the next tile's operands are loaded into one while
    // the current tile is computed from the other.  Every load is issued at
    // a clamped, in-bounds address and zeroed with a bitwise mask, and a
    // tile index past the end is clamped rather than the load skipped: with
    // no branch around a load the compiler can count the loads in flight and
    // leaves the next tile's in flight through this tile's MFMAs.
    f32x4 k0[DH / 4], k1[DH / 4];
    float v0[16][D / 32], v1[16][D / 32];
    auto clampt = [&](int t) { return t < ntiles ? t : ntiles - 1; };   // ntiles >= 1
    int t = wave;
    load(k0, v0, clampt(t));
    for (; t < ntiles; t += 8) {
        load(k1, v1, clampt(t + 4));
        __builtin_amdgcn_sched_barrier(0);
        tile(k0, v0, t);
        if (t + 4 >= ntiles) break;
        load(k0, v0, clampt(t + 8));
        __builtin_amdgcn_sched_barrier(0);
        tile(k1, v1, t + 4);
    }
    l += __shfl_xor(l, 32);

    // merge the four waves' partial softmaxes (every lane takes part; a wave
    // that saw no key has m = -inf and weight 0)
    if (wave > 0) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) mrg_o[wave - 1][d][r][lane] = o[d][r];
        mrg_ml[wave - 1][0][lane] = m;
        mrg_ml[wave - 1][1][lane] = l;
    }
    __syncthreads();
    if (wave != 0 || !q_ok) return;
    float mw[3], lw[3];
    float mt = m;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        mw[w] = mrg_ml[w][0][lane];
        lw[w] = mrg_ml[w][1][lane];
        mt = fmaxf(mt, mw[w]);
    }
    const float f0 = __builtin_amdgcn_exp2f(m - mt);
    float fw[3];
    float lt = l * f0;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        fw[w] = __builtin_amdgcn_exp2f(mw[w] - mt);
        lt += lw[w] * fw[w];
    }
    const float inv = 1.f / lt;
    float *Op = a.O + bi * a.o_sb + hi * a.o_sh + static_cast<int64_t>(qi) * a.o_ss;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g + j;
                float acc = o[d][r] * f0;
#pragma unroll
                for (int w = 0; w < 3; ++w) acc += mrg_o[w][d][r][lane] * fw[w];
                v[j] = acc * inv;
            }
            *reinterpret_cast<f32x4 *>(Op + 32 * d + 8 * g + 4 * h) = v;
        }
    if (a.lse && h == 0)
        a.lse[bh * a.S + qi] = (mt + __builtin_amdgcn_logf(lt)) * 0.693147180559945309f;
}

}  // namespace

int attention_variant(int64_t B, int64_t H, int64_t S, int64_t D, int forced)
{
    const int64_t blocks = (S + kBM - 1) / kBM * B * H;
    if (D != 64) return 0;
    if (forced >= 0 && forced <= 2) return forced;
    // Fewer 128-query work-groups than CUs: split the keys over the waves of
    // 32-query work-groups instead.  Up to 256 tokens, 32-key tiles (half the
    // LDS and 146 instead of 202 registers: three work-groups per CU) beat
    // 64-key tiles (GPT 64 x 6 x 256 causal 60.5 -> 53.2 us, full 68.6 ->
    // 66.8, 128 tokens causal 41.9 -> 38.8); from 384 tokens on the longer
    // tiles win (384 causal 53.3 vs 56.7, 2048 causal 266 vs 284).
    if (blocks < kCUs) return 1;
    return S <= 256 ? 2 : 0;
}

hipError_t launch_attention_fwd(const AttnArgs &args, int64_t D, int variant, hipStream_t s)
{
    AttnArgs a = args;
    a.nqb = (a.S + kBM - 1) / kBM;
    const int64_t blocks = a.nqb * a.B * a.H;
    if (blocks == 0) return hipSuccess;
    if (blocks > kMaxBlocks) return hipErrorInvalidValue;
    if (variant == 1) {
        if (D != 64) return hipErrorInvalidValue;
        const int64_t split = (a.S + kSplitQ - 1) / kSplitQ * a.B * a.H;
        if (split > kMaxBlocks) return hipErrorInvalidValue;
        hipLaunchKernelGGL(attention_fwd_split_kernel, dim3(static_cast<uint32_t>(split)),
                           dim3(kAttnThreads), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<uint32_t>(blocks));
    if (D == 64 && variant == 2)
        hipLaunchKernelGGL((attention_fwd_kernel<64, 32>), grid, dim3(kAttnThreads), 0, s, a);
    else if (D == 64)
        hipLaunchKernelGGL((attention_fwd_kernel<64, 64>), grid, dim3(kAttnThreads), 0, s, a);
    else if (D == 128)
        hipLaunchKernelGGL((attention_fwd_kernel<128, 32>), grid, dim3(kAttnThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mi355gemm
