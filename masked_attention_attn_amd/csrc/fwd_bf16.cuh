// Masked attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, per (batch, head), O = softmax(scale·Q·Kᵀ + pad)·V and the
// natural-log LSE of every query row without ever forming the Tq x Tk score
// matrix: a 32-key block of scores lives in registers, is reduced with an
// online softmax and immediately multiplied into the output accumulator.
// Padding is the additive -inf on padded keys that the MultiheadAttention
// fast-path page describes for the SDPA replacement (molayo1419.me, section
// "CPU에서 양을 측정하기"); the per-row LSE is the quantity the ring-attention
// merge needs (sglang PR 49078 analysis, section "1. aiter.py").
//
// Work decomposition
//   workgroup = 4 wavefronts (one per SIMD) of one (batch, head); each wave
//   owns 64 queries (two 32-column blocks of the MFMA), so a workgroup covers
//   256 queries.  K/V are staged in LDS in tiles of TK keys (64 at D = 64,
//   32 at D = 128); the compute steps over blocks of 32 keys.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, operands 8 bf16 per lane,
// accumulator 16 fp32 per lane; lane l holds column l%32 of the result and
// rows (i/4)*8 + (l/32)*4 + i%4 for accumulator element i):
//   Sᵀ[key, query] = K·Qᵀ  (A = K rows from LDS, B = Q rows from registers)
//     so each lane owns ONE query and 16 of its keys: row max and row sum are
//     in-lane plus one exchange with lane l^32.
//   Oᵀ[d, query] += Vᵀ·Pᵀ (A = Vᵀ from LDS, B = P from registers)
//     so the rescale of a query's output is in-lane too.
//   K rows are stored in LDS with bits 2 and 3 of the row index swapped, so
//   the eight P values a lane needs as one B operand of the second product
//   are eight consecutive accumulator elements of the first.
//
// Software pipeline.  Step u holds the raw scores S_u of key block u in
// registers (computed by step u-1) and, in one straight block of code whose
// issue order is fixed slot by slot, turns S_u into P_u while issuing the
// matrix-core work S_{u+1} = K_{u+1}·Qᵀ and O += V_uᵀ·P_u: the exp / convert
// / sum vector work of one block overlaps the MFMAs of two.  K tiles live in
// a ring of three LDS buffers (the pipeline reads tile T+1 while tile T+2 is
// being stored), V tiles in a ring of three (a deferred PV reads the previous
// tile); global loads go through buffer
// resources whose range check returns zeros past Tk, so no lane branches.
// Padding (a rare, workgroup-uniform case) and the lazy rescale are handled
// before the fixed block, so the common path has no per-element masking.
// Leading and trailing fully padded key blocks are never visited: the
// workgroup first finds its sequence's first and last unpadded keys.
//
// Online softmax with lazy rescaling: the running max m of a row is only
// moved (and O, l rescaled) when a block raises the max by more than TAU in
// log2 units; otherwise the stale max is kept, which bounds every weight by
// 2^TAU.  Final O = acc / l and LSE = (m·c + log2 l)·ln 2 are exact for any
// reference max, so this changes rounding only.
#pragma once

#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace fwdk {

constexpr int NWAVE = 4;
constexpr int NT = 64 * NWAVE;  // threads per workgroup
constexpr int PAD = 8;          // bf16 elements of row padding in LDS
constexpr int CK = 32;          // keys per compute step
constexpr int NB = 2;           // 32-query column blocks per wave
constexpr int QW = NB * 32;     // queries per wave
constexpr int BM = QW * NWAVE;  // queries per workgroup
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units

template <int D> struct Tile;
template <> struct Tile<64> { static constexpr int TK = 64; };
template <> struct Tile<128> { static constexpr int TK = 32; };

template <int D>
struct Lds {
    static constexpr int TK = Tile<D>::TK;
    static constexpr int KS = D + PAD;    // K tile row stride (elements), [key][d]
    static constexpr int VS = TK + PAD;   // Vᵀ tile row stride (elements), [d][key]
    static constexpr int K_TILE = TK * KS;
    static constexpr int V_TILE = D * VS;
    static constexpr int K_RING = 3, V_RING = 3;
    static constexpr int ELEMS = K_RING * K_TILE + V_RING * V_TILE;
    static constexpr int BYTES = ELEMS * (int)sizeof(bf16);
};

__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max / sum of x over lanes l and l^32 (v_permlane32_swap exchanges the two
// wave halves; the pair of results holds both halves' values in every lane).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer over `bytes` bytes at p: loads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int D, bool WRITE_LSE>
__global__ __launch_bounds__(NT, 1)
void fwd_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const uint8_t* __restrict__ mask,
                     bf16* __restrict__ o, float* __restrict__ lse,
                     int H, int Tq, int Tk, float c, int n_qt, int total) {
    using L = Lds<D>;
    constexpr int TK = L::TK;             // keys per LDS tile
    constexpr int HALVES = TK / CK;       // compute steps per tile
    constexpr int KSTEPS = D / 16;        // MFMA k-steps of K·Qᵀ
    constexpr int PSTEPS = CK / 16;       // MFMA k-steps of Vᵀ·Pᵀ per step (2)
    constexpr int DB = D / 32;            // 32-row blocks of Oᵀ
    constexpr uint64_t TILE_BITS = TK == 64 ? ~0ull : ((1ull << TK) - 1);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);
    __shared__ int red_s[NWAVE];

    const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
    if (logical >= total) return;
    const int bh = logical / n_qt;
    const int qt = logical - bh * n_qt;
    const int b = bh / H;
    const bf16* qp = q + (size_t)bh * Tq * D;
    const uint8_t* mp = mask ? mask + (size_t)b * Tk : nullptr;
    const uint32_t kv_bytes = (uint32_t)Tk * D * (uint32_t)sizeof(bf16);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bh * Tk * D, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (size_t)bh * Tk * D, kv_bytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = qt * BM + wave * QW;

    // ---- first and last unpadded key of this sequence (workgroup-wide scans)
    int first = 0, last = Tk - 1;
    if (mp) {
        last = -1;
        for (int base = Tk - 1; base >= 0; base -= NT) {       // backwards, NT keys per round
            const int key = base - tid;
            const uint64_t bal = __ballot(key >= 0 && mp[key] == 0);
            if (lane == 0) red_s[wave] = bal ? base - (wave * 64 + __builtin_ctzll(bal)) : -1;
            __syncthreads();
            last = max(max(red_s[0], red_s[1]), max(red_s[2], red_s[3]));
            __syncthreads();
            if (last >= 0) break;
        }
        first = last + 1;
        for (int base = 0; base <= last; base += NT) {           // forwards
            const int key = base + tid;
            const uint64_t bal = __ballot(key <= last && mp[key] == 0);
            if (lane == 0) red_s[wave] = bal ? base + wave * 64 + __builtin_ctzll(bal) : 0x7fffffff;
            __syncthreads();
            first = min(min(red_s[0], red_s[1]), min(red_s[2], red_s[3]));
            __syncthreads();
            if (first <= last) break;
        }
    }
    // Visited key blocks: [u_first, u_last] in units of CK keys; LDS tiles of TK keys.
    const int t_first = first / TK;
    const int u_first = t_first * HALVES;                  // steps start on a tile boundary
    const int u_last = last >= 0 ? last / CK : -1;
    const int nsteps = last >= first ? u_last - u_first + 1 : 0;
    const int t_last = last >= 0 ? last / TK : -1;

    // ---- Q as the B operand of Sᵀ = K·Qᵀ: lane holds query (l%32), d = kk*16 + hl*8 + 0..7.
    // Rows past Tq are clamped to a valid row; their results are never stored.
    bf16x8 qreg[NB][KSTEPS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = min(q0 + nb * 32 + l32, Tq - 1);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qreg[nb][kk] = as_bf16x8(ldg128(qp + (size_t)row * D + kk * 16 + hl * 8));
    }

    // ---- cooperative tile loads: K as 16-byte row chunks; V as key pairs so the
    // transposed LDS tile is written one 32-bit (two-key) word at a time.  Keys
    // past Tk read as zeros (buffer range check; they are masked).
    constexpr int KCH = D / 8;
    constexpr int K_LOADS = TK * KCH / NT;
    constexpr int V_TASKS_ALL = (TK / 2) * KCH;
    constexpr int V_TASKS = (V_TASKS_ALL + NT - 1) / NT;
    static_assert(K_LOADS * NT == TK * KCH, "tile split");
    u32x4 kr[K_LOADS];
    u32x4 vr[V_TASKS][2];
    uint32_t k_voff[K_LOADS], v_voff[V_TASKS];
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
        const int cidx = tid + i * NT;
        k_voff[i] = (uint32_t)((cidx / KCH) * D + (cidx % KCH) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < V_TASKS; ++i) {
        const int cidx = tid + i * NT;
        v_voff[i] = (uint32_t)((2 * (cidx % (TK / 2))) * D + (cidx / (TK / 2)) * 8) * 2u;
    }
    auto gload = [&](int tk, int tv) {
        const uint32_t ks_off = (uint32_t)tk * TK * D * 2u, vs_off = (uint32_t)tv * TK * D * 2u;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) kr[i] = bload128(krs, k_voff[i], ks_off);
#pragma unroll
        for (int i = 0; i < V_TASKS; ++i) {
            if (V_TASKS * NT == V_TASKS_ALL || tid + i * NT < V_TASKS_ALL) {
                vr[i][0] = bload128(vrs, v_voff[i], vs_off);
                vr[i][1] = bload128(vrs, v_voff[i] + D * 2u, vs_off);
            }
        }
    };
    auto kslot = [&](int t) -> bf16* { return smem + (t % L::K_RING) * L::K_TILE; };
    auto vslot = [&](int t) -> bf16* { return smem + L::K_RING * L::K_TILE + (t % L::V_RING) * L::V_TILE; };
    // K row r of a 32-row block goes to LDS row swap23(r) (an involution), so
    // lane l reading LDS row l%32 receives key swap23(l%32) on conflict-free rows.
    auto sstore = [&](bf16* ks, bf16* vs) {
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int cidx = tid + i * NT;
            const int row = cidx / KCH;
            const int lrow = (row & ~31) | swap_bits23(row & 31);
            *reinterpret_cast<u32x4*>(ks + lrow * L::KS + (cidx % KCH) * 8) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < V_TASKS; ++i) {
            const int cidx = tid + i * NT;
            if (V_TASKS * NT == V_TASKS_ALL || cidx < V_TASKS_ALL) {
                const int kpair = cidx % (TK / 2), col = cidx / (TK / 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t a = vr[i][0][j], bb = vr[i][1][j];
                    *reinterpret_cast<uint32_t*>(vs + (col * 8 + 2 * j) * L::VS + 2 * kpair) =
                        __builtin_amdgcn_perm(bb, a, 0x05040100u);            // d = col*8+2j
                    *reinterpret_cast<uint32_t*>(vs + (col * 8 + 2 * j + 1) * L::VS + 2 * kpair) =
                        __builtin_amdgcn_perm(bb, a, 0x07060302u);            // d = col*8+2j+1
                }
            }
        }
    };
    // Lane j reports whether key t*TK + j is padded or past Tk (lanes >= TK report 1).
    auto pad_flag = [&](int t) -> int {
        const int key = t * TK + lane;
        if (lane >= TK || key >= Tk) return 1;
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

    // Sᵀ = K·Qᵀ for one key block (u) from a tile in LDS: element i of lane l
    // holds key (i/8)*16 + (l/32)*8 + i%8 of the block.
    auto kblock = [&](int u) -> const bf16* {
        return kslot(u / HALVES) + ((u % HALVES) * 32 + l32) * L::KS + hl * 8;
    };
    auto qk_full = [&](int u, f32x16 (&S)[NB], float (&mx)[NB]) {
        const bf16* kp_ = kblock(u);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp_ + kk * 16);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (kk == 0) {
                    const f32x16 z = {};
                    S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][0], z, 0, 0, 0);
                } else {
                    S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][kk], S[nb], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float m = S[nb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) m = fmaxf(m, S[nb][i]);
            mx[nb] = m;
        }
    };

    uint64_t pm_tile = 0;
    int padf = 0;
    // Running-max threshold per query block: a block whose scores stay at or
    // below mthr needs no rescale (every weight stays <= 2^TAU).
    float mthr[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mthr[nb] = kNegInf;

    // The second PV k-step of block u is issued at the start of step u+1 (so
    // the MFMA stream never idles); pw_pend / va_pend carry its operands.
    u32x4 pw_pend[NB];
    const bf16* vp_pend = vslot(t_first) + l32 * L::VS + hl * 8;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pw_pend[nb] = u32x4{0u, 0u, 0u, 0u};
    auto pv_pend = [&](int db, int nb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vp_pend + db * 32 * L::VS + 16);
        oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pw_pend[nb]), oacc[db][nb], 0, 0, 0);
    };

    // One pipeline step for key block u = u_first + j: S holds its raw scores and
    // mx their in-lane row max; Sn / mxn receive block u+1's.  hf (the step's
    // half within its LDS tile) is a constant at each call site.
    auto step = [&](int j, const int hf, f32x16 (&S)[NB], float (&mx)[NB], f32x16 (&Sn)[NB],
                    float (&mxn)[NB]) {
        const int u = u_first + j;
        const int T = u / HALVES;
        if (hf == 0) pm_tile = __ballot(padf) & TILE_BITS;
        const uint32_t pm = (uint32_t)(pm_tile >> (hf * 32));   // bit i: key u*32+i padded
        if (pm != 0u) {             // workgroup-uniform, rare: mask and redo the row max
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kl = (i >> 3) * 16 + hl * 8 + (i & 7);
                if ((pm >> kl) & 1u) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) S[nb][i] = kNegInf;
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float m = S[nb][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) m = fmaxf(m, S[nb][i]);
                mx[nb] = m;
            }
        }
        bool need = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) need |= mx[nb] > mthr[nb];
        if (__ballot(need)) {       // lazy rescale: rare once the running max settles
            // finish block u-1 under the old scale, then rescale O and l
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) pv_pend(db, nb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                pw_pend[nb] = u32x4{0u, 0u, 0u, 0u};
                const float mnew = fmaxf(mrun[nb], pair_max(mx[nb]));
                const float alpha = __builtin_amdgcn_exp2f((mrun[nb] - mnew) * c);
                mrun[nb] = mnew;
                mc[nb] = mnew * c;
                mthr[nb] = mnew + TAU / c;
                lsum[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][nb][i] *= alpha;
            }
        }

        // ---- fixed block, issued slot by slot: the MFMA stream is
        //   PV(u-1, k-step 1) | QK(u+1) | PV(u, k-step 0)
        // and each slot also carries one stage of a three-stage softmax pipeline
        // (A: x = S·c - m·c, B: p = 2^x, C: l += p, pack to bf16), so every slot
        // has independent vector work; LDS operands are read a few slots ahead.
        const bf16* kp_ = kblock(u + 1);
        const bf16* vp_ = vslot(T) + l32 * L::VS + hf * 32 + hl * 8;
        bf16x8 ka[KSTEPS];
        bf16x8 va[DB];
        u32x4 pw[NB][PSTEPS];
        float xs[16][2], ps[16][2];
        auto rd_k = [&](int kk) { ka[kk] = *reinterpret_cast<const bf16x8*>(kp_ + kk * 16); };
        auto rd_v = [&](int db) { va[db] = *reinterpret_cast<const bf16x8*>(vp_ + db * 32 * L::VS); };
        // pair pp: chunk k2 = pp / (4*NB), query block nb, elements i, i+1
        auto pair_nb = [&](int pp) { return (pp / 4) % NB; };
        auto pair_i = [&](int pp) { return (pp / (4 * NB)) * 8 + (pp % 4) * 2; };
        auto stA = [&](int pp) {
            const int nb = pair_nb(pp), i = pair_i(pp);
            xs[pp][0] = __builtin_fmaf(S[nb][i], c, -mc[nb]);
            xs[pp][1] = __builtin_fmaf(S[nb][i + 1], c, -mc[nb]);
        };
        auto stB = [&](int pp) {
            ps[pp][0] = __builtin_amdgcn_exp2f(xs[pp][0]);
            ps[pp][1] = __builtin_amdgcn_exp2f(xs[pp][1]);
        };
        auto stC = [&](int pp) {
            const int nb = pair_nb(pp);
            lsum[nb] += ps[pp][0];
            lsum[nb] += ps[pp][1];
            pw[nb][pp / (4 * NB)][pp % 4] = pack_bf16x2(ps[pp][0], ps[pp][1]);
        };
        auto softmax_slot = [&](int sl) {     // stages for slot sl of 18
            if (sl >= 1 && sl <= 16) stB(sl - 1);
            if (sl < 16) stA(sl);
            if (sl >= 2 && sl <= 17) stC(sl - 2);
        };
        auto qk_one = [&](int qi) {     // qi = kk*NB + nb
            const int nb = qi % NB, kk = qi / NB;
            if (kk == 0) {
                const f32x16 z = {};
                Sn[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qreg[nb][0], z, 0, 0, 0);
            } else {
                Sn[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qreg[nb][kk], Sn[nb], 0, 0, 0);
            }
        };
        auto pv0_one = [&](int pi) {    // PV(u, k-step 0): pi = db*NB + nb
            const int nb = pi % NB, db = pi / NB;
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], as_bf16x8(pw[nb][0]), oacc[db][nb], 0, 0, 0);
        };
        auto max_part = [&](int nb, int i0, int n) {   // running in-lane max of Sn[nb][i0 .. i0+n)
            float m = Sn[nb][i0];
#pragma unroll
            for (int i = i0 + 1; i < i0 + n; ++i) m = fmaxf(m, Sn[nb][i]);
            mxn[nb] = i0 == 0 ? m : fmaxf(mxn[nb], m);
        };
        auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };

        if constexpr (D == 64) {
            // 16 MFMA slots + 2 drain slots:
            //   0-3 PV(u-1,1)   4-11 QK(u+1)   12-15 PV(u,0)   16-17 softmax drain
            // row max of S_{u+1}: 4 max3 per slot in 14-17 (QK done by slot 11).
            rd_k(0); rd_k(1);
            fence();
#pragma unroll
            for (int sl = 0; sl < 18; ++sl) {
                if (sl == 0) { rd_k(2); rd_k(3); }
                if (sl == 6) { rd_v(0); rd_v(1); }
                if (sl < 4) pv_pend(sl / NB, sl % NB);
                else if (sl < 12) qk_one(sl - 4);
                else if (sl < 16) pv0_one(sl - 12);
                softmax_slot(sl);
                if (sl >= 14) max_part((sl - 14) >> 1, ((sl - 14) & 1) * 8, 8);
                fence();
            }
        } else {
            // D=128: 32 MFMA slots:
            //   0-7 PV(u-1,1)   8-23 QK(u+1)   24-31 PV(u,0)
            // softmax pipeline in slots 0-17 (chunk 0 packed by slot 9), row max in 26-31.
            rd_k(0); rd_k(1);
            fence();
#pragma unroll
            for (int sl = 0; sl < 32; ++sl) {
                if (sl == 0) { rd_k(2); rd_k(3); }
                if (sl == 8) { rd_k(4); rd_k(5); }
                if (sl == 12) { rd_k(6); rd_k(7); }
                if (sl == 18) { rd_v(0); rd_v(1); }
                if (sl == 20) { rd_v(2); rd_v(3); }
                if (sl < 8) pv_pend(sl / NB, sl % NB);
                else if (sl < 24) qk_one(sl - 8);
                else pv0_one(sl - 24);
                if (sl < 18) softmax_slot(sl);
                if (sl >= 26 && sl < 30) max_part((sl - 26) >> 1, ((sl - 26) & 1) * 8, 8);
                fence();
            }
        }
        // hand block u's second k-step to step u+1
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) pw_pend[nb] = pw[nb][1];
        vp_pend = vp_;

        // ---- end of an LDS tile: store the tile loaded during this one, then
        // start loading the next (K tile T+3 and V tile T+2 land by T+1's end).
        // V tile T is still read by the pending PV of the next step, and tile
        // T-1 by this tile's first step: a ring of three V slots keeps both
        // while slot T+1 is written here.
        if (hf == HALVES - 1) {
            sstore(kslot(T + 2), vslot(T + 1));
            __syncthreads();
            gload(min(T + 3, t_last), min(T + 2, t_last));
            padf = pad_flag(min(T + 1, t_last));
        }
    };

    if (nsteps > 0) {
        f32x16 sA[NB], sB[NB];
        float mxA[NB], mxB[NB];
        padf = pad_flag(t_first);
        gload(t_first, t_first);
        sstore(kslot(t_first), vslot(t_first));
        gload(min(t_first + 1, t_last), t_first);
        sstore(kslot(t_first + 1), vslot(t_first + 1));
        __syncthreads();
        gload(min(t_first + 2, t_last), min(t_first + 1, t_last));   // stored by tile t_first's end
        qk_full(u_first, sA, mxA);
        for (int j = 0; j < nsteps; j += 2) {
            step(j, 0, sA, mxA, sB, mxB);
            if (j + 1 < nsteps) step(j + 1, HALVES - 1, sB, mxB, sA, mxA);
        }
        // flush the pending second k-step of the last block
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) pv_pend(db, nb);
    }

    // ---- epilogue: O = acc / l, LSE = (m·c + log2 l)·ln 2
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float lt = pair_sum(lsum[nb]);
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
    using L = Lds<D>;
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

}  // namespace fwdk
}  // namespace mattn
