// Masked attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, per (batch, head), O = softmax(scale·Q·Kᵀ + pad)·V and the
// natural-log LSE of every query row without ever forming the Tq x Tk score
// matrix: the score tile of 64 keys lives in registers, is reduced with an
// online softmax and immediately multiplied into the output accumulator.
// Padding is the additive -inf on padded keys that the MultiheadAttention
// fast-path page describes for the SDPA replacement (molayo1419.me, section
// "CPU에서 양을 측정하기"); the per-row LSE is the quantity the ring-attention
// merge needs (sglang PR 49078 analysis, section "1. aiter.py").
//
// Work decomposition
//   workgroup = 4 wavefronts of one (batch, head); each wave owns NB*32
//   queries (NB column blocks of the MFMA, NB = 2 -> 256 queries per
//   workgroup).  K/V are walked in tiles of BN keys (64 at D = 64, 32 at
//   D = 128 so that the register budget holds) staged in LDS (double
//   buffered, one barrier per tile); the next tile's global loads are in
//   flight while the current tile is computed.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, operands 8 bf16 per lane,
// accumulator 16 fp32 per lane; lane l holds column l%32 of the result and
// rows (i/4)*8 + (l/32)*4 + i%4 for accumulator element i):
//   Sᵀ[key, query] = K·Qᵀ  (A = K rows from LDS, B = Q rows from registers)
//     so each lane owns ONE query and 16 of its keys: row max and row sum are
//     in-lane plus one exchange with lane l^32.
//   Oᵀ[d, query] += Vᵀ·Pᵀ (A = Vᵀ from LDS, B = P from registers)
//     so the rescale of a query's output is in-lane too.
//   The K rows fed to the first product are permuted (bits 2 and 3 of the row
//   index swapped) so that the eight P values a lane needs as one B operand of
//   the second product are exactly eight consecutive accumulator elements.
//
// Online softmax with lazy rescaling: the running max m of a row is only
// moved (and O, l rescaled) when a tile raises the max by more than TAU in
// log2 units; otherwise the stale max is kept, which bounds every weight by
// 2^TAU.  Final O = acc / l and LSE = (m·c + log2 l)·ln 2 are exact for any
// reference max, so this changes rounding only.
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NWAVE = 4;
constexpr int NT = 64 * NWAVE;  // threads per workgroup
constexpr int PAD = 8;          // bf16 elements of row padding in LDS
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units

// Tile shape per head dimension: BN keys per tile, NB 32-query blocks per wave.
template <int D> struct Shape;
template <> struct Shape<64> { static constexpr int BN = 64, NB = 2; };
template <> struct Shape<128> { static constexpr int BN = 32, NB = 2; };

template <int D, int BN>
struct Lds {
    static constexpr int KS = D + PAD;    // K tile row stride (elements), [key][d]
    static constexpr int VS = BN + PAD;   // Vᵀ tile row stride (elements), [d][key]
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int BYTES = 2 * BUF * (int)sizeof(bf16);
};

__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D, bool WRITE_LSE>
__global__ __launch_bounds__(NT, 1)
void fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const uint8_t* __restrict__ mask,
                     bf16* __restrict__ o, float* __restrict__ lse,
                     int H, int Tq, int Tk, float c, int n_qt, int total) {
    constexpr int BN = Shape<D>::BN;      // keys per tile
    constexpr int NB = Shape<D>::NB;      // 32-query column blocks per wave
    constexpr int MB = BN / 32;           // 32-key row blocks per tile
    constexpr int QW = NB * 32;           // queries per wave
    constexpr int BM = QW * NWAVE;        // queries per workgroup
    constexpr int KSTEPS = D / 16;        // MFMA k-steps of Q·Kᵀ
    constexpr int PSTEPS = BN / 16;       // MFMA k-steps of P·V
    constexpr int DB = D / 32;            // 32-row blocks of Oᵀ
    using L = Lds<D, BN>;
    constexpr uint64_t TILE_BITS = BN == 64 ? ~0ull : ((1ull << BN) - 1);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
    if (logical >= total) return;
    const int bh = logical / n_qt;
    const int qt = logical - bh * n_qt;
    const int b = bh / H;
    const bf16* qp = q + (size_t)bh * Tq * D;
    const bf16* kp = k + (size_t)bh * Tk * D;
    const bf16* vp = v + (size_t)bh * Tk * D;
    const uint8_t* mp = mask ? mask + (size_t)b * Tk : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = qt * BM + wave * QW;

    // Q as the B operand of Sᵀ = K·Qᵀ: lane holds query (l%32) and d = kk*16 + hl*8 + 0..7.
    // Rows past Tq are clamped to a valid row; their results are never stored.
    bf16x8 qreg[NB][KSTEPS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = min(q0 + nb * 32 + l32, Tq - 1);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qreg[nb][kk] = as_bf16x8(ldg128(qp + (size_t)row * D + kk * 16 + hl * 8));
    }

    // Cooperative tile loads: K as 16-byte row chunks; V as key pairs so that
    // the transposed LDS tile is written one 32-bit (two-key) word at a time.
    // Keys past Tk load as zeros (finite, and masked below).
    constexpr int KCH = D / 8;
    constexpr int K_LOADS = BN * KCH / NT;
    constexpr int V_TASKS = (BN / 2) * KCH / NT;
    static_assert(K_LOADS * NT == BN * KCH && V_TASKS * NT == (BN / 2) * KCH, "tile split");
    u32x4 kr[K_LOADS];
    u32x4 vr[V_TASKS][2];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    auto gload = [&](int kt) {
        const int base = kt * BN;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int cidx = tid + i * NT;
            const int row = cidx / KCH, col = cidx % KCH;
            const int key = base + row;
            kr[i] = key < Tk ? ldg128(kp + (size_t)key * D + col * 8) : zero4;
        }
#pragma unroll
        for (int i = 0; i < V_TASKS; ++i) {
            const int cidx = tid + i * NT;
            const int kpair = cidx % (BN / 2), col = cidx / (BN / 2);
            const int key = base + 2 * kpair;
            vr[i][0] = key < Tk ? ldg128(vp + (size_t)key * D + col * 8) : zero4;
            vr[i][1] = key + 1 < Tk ? ldg128(vp + (size_t)(key + 1) * D + col * 8) : zero4;
        }
    };
    auto sstore = [&](int buf) {
        bf16* ks = smem + buf * L::BUF;
        bf16* vs = ks + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int cidx = tid + i * NT;
            const int row = cidx / KCH, col = cidx % KCH;
            *reinterpret_cast<u32x4*>(ks + row * L::KS + col * 8) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < V_TASKS; ++i) {
            const int cidx = tid + i * NT;
            const int kpair = cidx % (BN / 2), col = cidx / (BN / 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t a = vr[i][0][j], bb = vr[i][1][j];
                const uint32_t w0 = (a & 0xffffu) | (bb << 16);          // d = col*8+2j
                const uint32_t w1 = (a >> 16) | (bb & 0xffff0000u);      // d = col*8+2j+1
                *reinterpret_cast<uint32_t*>(vs + (col * 8 + 2 * j) * L::VS + 2 * kpair) = w0;
                *reinterpret_cast<uint32_t*>(vs + (col * 8 + 2 * j + 1) * L::VS + 2 * kpair) = w1;
            }
        }
    };
    // Lane j reports whether key kt*BN + j is padded or past Tk (lanes >= BN unused).
    auto pad_flag = [&](int kt) -> int {
        const int key = kt * BN + lane;
        if (lane >= BN || key >= Tk) return 1;
        return mp ? (int)(mp[key] != 0) : 0;
    };

    f32x16 oacc[DB][NB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][nb][i] = 0.f;
    float mrun[NB], mc[NB], lsum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { mrun[nb] = kNegInf; mc[nb] = 0.f; lsum[nb] = 0.f; }

    const int ntiles = (Tk + BN - 1) / BN;
    int padf = pad_flag(0);
    gload(0);
    sstore(0);
    __syncthreads();

    const int krow = swap_bits23(l32);

    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        const uint64_t pm = __ballot(padf) & TILE_BITS;   // bit j: key kt*BN+j is padded
        if (kt + 1 < ntiles) {
            padf = pad_flag(kt + 1);
            gload(kt + 1);
        }
        if (pm != TILE_BITS) {          // workgroup-uniform: skip tiles with no unpadded key
            const bf16* ks = smem + buf * L::BUF;
            const bf16* vs = ks + L::K_ELEMS;

            // ---- Sᵀ = K·Qᵀ for BN keys x QW queries
            f32x16 s[MB][NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[mb][nb][i] = 0.f;
                const bf16* krp = ks + (mb * 32 + krow) * L::KS + hl * 8;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(krp + kk * 16);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][kk], s[mb][nb], 0, 0, 0);
                }
            }

            // ---- key padding: element i of block mb holds key mb*32 + (i/8)*16 + hl*8 + i%8
            if (pm != 0ull) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kl = mb * 32 + (i >> 3) * 16 + hl * 8 + (i & 7);
                        if ((pm >> kl) & 1ull) {
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) s[mb][nb][i] = kNegInf;
                        }
                    }
            }

            // ---- online softmax statistics (lazy rescale)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float mx = s[0][nb][0];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mb][nb][i]);
                mx = fmaxf(mx, xor32(mx));
                const float mnew = fmaxf(mrun[nb], mx);
                const bool need = (mnew - mrun[nb]) * c > TAU;
                if (__ballot(need)) {
                    const float alpha = __builtin_amdgcn_exp2f((mrun[nb] - mnew) * c);
                    mrun[nb] = mnew;
                    mc[nb] = mnew * c;
                    lsum[nb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][nb][i] *= alpha;
                }
            }

            // ---- P = exp2(S·c - m·c), packed to bf16 as the B operand of Oᵀ += Vᵀ·Pᵀ
            u32x4 pw[NB][PSTEPS];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][nb][i], c, -mc[nb]));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][nb][i + 1], c, -mc[nb]));
                        lsum[nb] += p0;
                        lsum[nb] += p1;
                        pw[nb][2 * mb + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(p0, p1);
                    }

            // ---- Oᵀ += Vᵀ·Pᵀ
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16* vrp = vs + (db * 32 + l32) * L::VS + hl * 8;
#pragma unroll
                for (int k2 = 0; k2 < PSTEPS; ++k2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrp + k2 * 16);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pw[nb][k2]), oacc[db][nb], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < ntiles) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = (m·c + log2 l)·ln 2
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float lt = lsum[nb] + xor32(lsum[nb]);
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        const int qi = q0 + nb * 32 + l32;
        if (qi < Tq) {
            bf16* orow = o + ((size_t)bh * Tq + qi) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[db][nb][4 * g] * inv, oacc[db][nb][4 * g + 1] * inv);
                    w[1] = pack_bf16x2(oacc[db][nb][4 * g + 2] * inv, oacc[db][nb][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(orow + db * 32 + g * 8 + hl * 4) = w;
                }
            if (WRITE_LSE && hl == 0)
                lse[(size_t)bh * Tq + qi] = lt > 0.f ? (mc[nb] + __log2f(lt)) * kLn2 : kNegInf;
        }
    }
}

template <int D, bool WRITE_LSE>
hipError_t launch_one(const FwdArgs& a) {
    constexpr int BN = Shape<D>::BN;
    constexpr int BM = Shape<D>::NB * 32 * NWAVE;
    using L = Lds<D, BN>;
    auto kern = fwd_bf16_kernel<D, WRITE_LSE>;
    // LDS above 64 KiB must be opted into once per kernel (thread-safe static init).
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    if (attr != hipSuccess) return attr;
    const int n_qt = (a.Tq + BM - 1) / BM;
    const int total = a.B * a.H * n_qt;
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), L::BYTES, (hipStream_t)a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.mask,
                       (bf16*)a.o, a.lse, a.H, a.Tq, a.Tk, c, n_qt, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.D == 64) return a.lse ? launch_one<64, true>(a) : launch_one<64, false>(a);
    return a.lse ? launch_one<128, true>(a) : launch_one<128, false>(a);
}

}  // namespace mattn
