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
//   workgroup = 256 queries of one (batch, head): at D = 64 four wavefronts of
//   64 queries (two 32-column blocks of the MFMA), at D = 128 eight
//   wavefronts of 32 queries.  K/V are staged in LDS in tiles of TK = 64 keys
//   shared by the workgroup; the compute steps over blocks of 32 keys (two per
//   tile).
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
// LDS tiles are filled by direct global->LDS buffer loads (no staging
// registers): lane i of a load writes bytes [16i, 16i+16) of a 1 KiB chunk,
// so each lane picks the global 16 bytes that belong there.  Both tiles are
// unpadded with an XOR swizzle of the 16-byte chunk index (k_swz / v_swz,
// chosen so that no read has bank conflicts); V keeps its natural [key][d]
// layout and the Vᵀ operand is read with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j%4
// of the 8-byte rows addressed by lanes j/4 + 4k).
//
// Software pipeline.  Step u holds the raw scores S_u of key block u in
// registers (computed by step u-1) and, in one straight block of code whose
// issue order is fixed slot by slot, turns S_u into P_u while issuing the
// matrix-core work S_{u+1} = K_{u+1}·Qᵀ and O += V_uᵀ·P_u: the exp / convert
// / sum vector work of one block overlaps the MFMAs of two.  The K operands
// of S_{u+1} are read from LDS during step u-1.  bf16: K tiles live in a ring
// of five LDS buffers and V tiles in a ring of four, loaded three tiles ahead
// (tile T+1 is readable during tile T while tiles T+2 .. T+4 are being
// stored); E4M3: three K buffers of codes and two V buffers, one tile ahead.
// The buffer resources' range check returns zeros past Tk, so no lane branches.
// Padding (a rare, workgroup-uniform case) is applied before the fixed block,
// so the common path has no per-element masking.  One pass over the mask
// finds the sequence's first and last unpadded keys and whether any padded
// key lies between them: leading and trailing fully padded key blocks are
// never visited, and without interior holes the mask of every visited block
// follows from the two indices, with no mask reads in the loop.
//
// Online softmax with a lazily raised reference: weights are 2^(S·c - mc)
// with mc set once from the exact row max of the first block that holds an
// unpadded key.  The common path computes no row max at all: after each
// 16-key chunk is exponentiated, its per-lane weight sum is compared with
// 2^TAU, and only if some lane exceeds it (the scores rose well above the
// reference) is mc raised to the chunk's row max, O and l scaled by
// 2^(old - new) and the chunk redone.  Every weight used is therefore at most
// 2^TAU.  Final O = acc / l and LSE = (mc + log2 l)·ln 2 are exact for any
// reference, so this changes rounding only.
//
// FP8 variant (FP8 = true): Q, K and V arrive as E4M3 codes with one float32
// scale per (sequence, head) (K and V: per KV head); the result is the
// attention of the dequantised tensors, O in bf16 plus the LSE, which the
// FP8 prefill the aiter ring-attention analysis describes does not return
// (sglang PR 49078 analysis, section "1. aiter.py").  Sᵀ = K·Qᵀ runs on the
// E4M3 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales:
// exact products, fp32 sums) straight from the codes, K tiles staged in LDS as
// codes (half the bytes); the Q and K scales fold into the softmax constant c.
// V is converted to bf16 on its way into LDS (every E4M3 value is a bf16
// value), so the P·V product, the softmax and the rescale logic are those of
// the bf16 kernel; the V scale multiplies O in the epilogue.  The weights stay
// bf16: E4M3 weights would cost more accuracy than the output tolerance.
#pragma once

#include "common.cuh"
#include "launch.h"
#include "mfma_lds.cuh"

namespace mattn {
namespace fwdk {
using namespace mattn::mfma;

constexpr int CK = 32;          // keys per compute step
// Wavefronts per workgroup and 32-query column blocks per wavefront.  D = 64:
// four waves of 64 queries (the K operand of a key block serves two query
// blocks).  D = 128: eight waves of 32 queries, which keeps a wave's live
// state (output 4x16, scores 2x16, Q 8x4, operands) within the 256 VGPRs of
// two waves per SIMD; a workgroup covers 256 queries either way.  WG_PER_CU is
// the launch bound's resident workgroups per CU: two at D = 64 make the compiler
// fit a wave in 256 registers (two waves per SIMD) instead of spreading it over
// 304 with accumulation registers (one wave per SIMD).
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int NWAVE = 4, NB = 2, WG_PER_CU = 2; };
template <> struct Cfg<128> { static constexpr int NWAVE = 8, NB = 1, WG_PER_CU = 1; };
template <int D> constexpr int kBM = Cfg<D>::NWAVE * Cfg<D>::NB * 32;   // queries per workgroup
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units
constexpr float kRescaleSum = 256.0f;   // 2^TAU: a lane's chunk sum above this forces a rescale

template <int D> struct Tile;
template <> struct Tile<64> { static constexpr int TK = 64; };
template <> struct Tile<128> { static constexpr int TK = 64; };

template <int D, bool FP8>
struct Lds {
    static constexpr int TK = Tile<D>::TK;
    static constexpr int RBK = FP8 ? D : D * 2;   // bytes per K row (E4M3 codes or bf16; unpadded, swizzled)
    static constexpr int RBV = D * 2;             // bytes per V row (bf16 either way)
    static constexpr int K_TILE = TK * RBK;       // bytes
    static constexpr int V_TILE = TK * RBV;
    // bf16: tiles are loaded three tiles ahead (K one tile earlier still, for the operand reads
    // one step ahead), so a ring of five K and four V tiles (72 KiB at D = 64, two workgroups
    // per CU; 144 KiB at D = 128); E4M3 (V through registers): one tile ahead, three K and two V.
    static constexpr int AHEAD = FP8 ? 1 : 3;     // tiles a load is issued ahead of its first use
    static constexpr int K_RING = AHEAD + 2, V_RING = AHEAD + 1;
    static constexpr int BYTES = K_RING * K_TILE + V_RING * V_TILE;
};

// Element type of Q, K and V in HBM.
template <bool FP8> struct ElemT { typedef bf16 type; };
template <> struct ElemT<true> { typedef uint8_t type; };
template <bool FP8> using Elem = typename ElemT<FP8>::type;

typedef int i32x8 __attribute__((ext_vector_type(8)));
// E4M3 x E4M3 32x32x64 product (format codes 0) with unit block scales (exponent 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 acc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// VARLEN = false: q/o [B, H, Tq, D], k/v [B, H_kv, Tk, D], mask [B, Tk] (or
// none), lse [B, H, Tq].
// VARLEN = true: packed q/o [total_q, H, D], k/v [total_k, H_kv, D] holding the
// sequences back to back at the offsets cu_q / cu_k (B+1 entries, clamped to
// [0, total]); lse [H, total_q]; no mask; Tq = the longest sequence (grid).
// Query head h reads KV head h / (H / H_kv).
// FP8: q, k, v are E4M3 codes (either layout); qsc [B, H], ksc and vsc [B, H_kv] (b = sequence).
// CAUSAL: query i of a sequence sees keys j <= i + (Tk - Tq) only.  A workgroup's
// key range ends at its last query's limit, the per-query limit is applied on
// the key blocks that cross a wave's diagonal, and q-tiles run last-first
// (the longest first, for the balance of the grid).
template <int D, bool WRITE_LSE, bool VARLEN, bool CAUSAL, bool FP8>
__global__ __launch_bounds__(64 * Cfg<D>::NWAVE, Cfg<D>::WG_PER_CU)
void fwd_bf16_kernel(const Elem<FP8>* __restrict__ q, const Elem<FP8>* __restrict__ k,
                     const Elem<FP8>* __restrict__ v, const uint8_t* __restrict__ mask,
                     bf16* __restrict__ o, float* __restrict__ lse,
                     int H, int H_kv, int Tq, int Tk, float c_in, int n_qt, int total, int nparts, int tpp,
                     const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                     int total_q, int total_k, const float* __restrict__ qsc,
                     const float* __restrict__ ksc, const float* __restrict__ vsc) {
    using L = Lds<D, FP8>;
    using ET = Elem<FP8>;
    constexpr int ES = (int)sizeof(ET);   // bytes per Q/K/V element in HBM
    constexpr int NWAVE = Cfg<D>::NWAVE;
    constexpr int NT = 64 * NWAVE;        // threads per workgroup
    constexpr int NB = Cfg<D>::NB;        // 32-query column blocks per wave
    constexpr int QW = NB * 32;           // queries per wave
    constexpr int BM = QW * NWAVE;        // queries per workgroup
    constexpr int NPP = 8 * NB;           // score pairs per lane and step
    constexpr int CP = 4 * NB;            // pairs per 16-key chunk
    constexpr int TK = L::TK;             // keys per LDS tile
    constexpr int HALVES = TK / CK;       // compute steps per tile
    constexpr int KSTEPS = D / 16;        // MFMA k-steps of K·Qᵀ (bf16)
    constexpr int KS8 = D / 64;           // MFMA k-steps of K·Qᵀ (E4M3)
    constexpr int PSTEPS = CK / 16;       // MFMA k-steps of Vᵀ·Pᵀ per step (2)
    constexpr int DB = D / 32;            // 32-row blocks of Oᵀ
    constexpr uint64_t TILE_BITS = TK == 64 ? ~0ull : ((1ull << TK) - 1);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    __shared__ int red_s[3 * NWAVE];

    // Workgroup -> (b, h, q-tile).  Workgroup i runs on XCD i % 8.
    int b, h, qt;
    if constexpr (!VARLEN) {
        // Equal work per (b, h): XCD x takes the x-th eighth of the (b, h, q-tile) order, so a
        // head's q-tiles share one L2.
        const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
        if (logical >= total) return;
        const int bh = logical / n_qt;
        const int r = logical - bh * n_qt;
        qt = CAUSAL ? n_qt - 1 - r : r;
        b = bh / H;
        h = bh - b * H;
    } else {
        // Sequences differ in length, so eighths of the grid would not balance.  The tiles of a
        // (sequence, KV head) group (its G query heads x n_qt q-tiles, q-tile-major, last q-tile
        // first when causal) form a chunk; each chunk is cut into nparts parts that take every
        // nparts-th tile (so each part mixes long and short causal tiles), and the parts are
        // dealt to the XCDs in turn: XCD x runs parts x, x+8, ..., one after the other, tpp
        // workgroup slots each.  The G heads of a group share the group's K/V in that L2.
        const int G = H / H_kv;
        const int x = blockIdx.x % kNumXcd, k = blockIdx.x / kNumXcd;
        const int part = (k / tpp) * kNumXcd + x;
        const int chunk = part / nparts;
        const int r = part - chunk * nparts + nparts * (k % tpp);
        if (chunk >= total / (G * n_qt) || r >= G * n_qt) return;
        const int qr = r / G;
        qt = CAUSAL ? n_qt - 1 - qr : qr;
        b = chunk / H_kv;
        h = (chunk - b * H_kv) * G + (r - qr * G);
    }
    const int bh = b * H + h;
    const int hk = h / (H / H_kv);        // KV head
    // This (b, h)'s rows: lengths, first rows and row strides (elements).
    int Tq_, Tk_, rsq, rsk;               // rows of Q/O and K/V, their row strides
    size_t q_row0, k_row0, l_row0;        // element offset of row 0 (LSE: index of row 0)
    if constexpr (VARLEN) {
        const int sq = min(max(cu_q[b], 0), total_q), eq = min(max(cu_q[b + 1], sq), total_q);
        const int sk = min(max(cu_k[b], 0), total_k), ek = min(max(cu_k[b + 1], sk), total_k);
        Tq_ = __builtin_amdgcn_readfirstlane(eq - sq);
        Tk_ = __builtin_amdgcn_readfirstlane(ek - sk);
        rsq = H * D;
        rsk = H_kv * D;
        q_row0 = ((size_t)sq * H + h) * D;
        k_row0 = ((size_t)sk * H_kv + hk) * D;
        l_row0 = (size_t)h * total_q + sq;
    } else {
        Tq_ = Tq;
        Tk_ = Tk;
        rsq = D;
        rsk = D;
        q_row0 = (size_t)bh * Tq * D;
        k_row0 = ((size_t)b * H_kv + hk) * Tk * D;
        l_row0 = (size_t)bh * Tq;
    }
    if (qt * BM >= Tq_) return;           // whole workgroup: past this sequence's queries
    // Softmax constant (log2 units) and output factor: FP8 scores are those of the codes,
    // times the Q and K scales; O is times the V scale.
    float c = c_in, osc = 1.f;
    if constexpr (FP8) {
        c = c_in * qsc[bh] * ksc[b * H_kv + hk];
        osc = vsc[b * H_kv + hk];
    }
    const ET* qp = q + q_row0;
    const uint8_t* mp = VARLEN ? nullptr : mask ? mask + (size_t)b * Tk_ : nullptr;
    // K/V buffer range ends after the last row, so rows >= Tk_ read as zero.
    const uint32_t kv_bytes = Tk_ > 0 ? (uint32_t)((Tk_ - 1) * rsk + D) * (uint32_t)ES : 0u;
    const i32x4_sgpr krs = make_rsrc(k + k_row0, kv_bytes);
    const i32x4_sgpr vrs = make_rsrc(v + k_row0, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs8 = brsrc(v + k_row0, kv_bytes);    // FP8: V through registers

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = qt * BM + wave * QW;

    // ---- one pass over this sequence's mask: first and last unpadded key, and
    // whether a padded key lies strictly between them (an interior hole).  Without
    // holes the only padded keys a visited block can hold lie outside
    // [first, last], so the per-block masks follow from the two indices alone.
    int first = 0, last = Tk_ - 1, holes = 0;
    if (mp) {
        int f = 0x7fffffff, l = -1, n = 0;
        for (int base = tid * 16; base < Tk_; base += NT * 16) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = base + j;
                if (key < Tk_ && mp[key] == 0) {
                    f = min(f, key);
                    l = max(l, key);
                    ++n;
                }
            }
        }
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1) {
            f = min(f, __shfl_xor(f, sh));
            l = max(l, __shfl_xor(l, sh));
            n += __shfl_xor(n, sh);
        }
        if (lane == 0) {
            red_s[wave] = f;
            red_s[NWAVE + wave] = l;
            red_s[2 * NWAVE + wave] = n;
        }
        __syncthreads();
        f = red_s[0];
        l = red_s[NWAVE];
        n = red_s[2 * NWAVE];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w) {
            f = min(f, red_s[w]);
            l = max(l, red_s[NWAVE + w]);
            n += red_s[2 * NWAVE + w];
        }
        if (n == 0) {
            first = 0;
            last = -1;
        } else {
            first = f;
            last = l;
            holes = n != l - f + 1;
        }
        first = __builtin_amdgcn_readfirstlane(first);
        last = __builtin_amdgcn_readfirstlane(last);
        holes = __builtin_amdgcn_readfirstlane(holes);
    }
    // Causal: no query of this workgroup sees a key past its last query's limit.
    const int coff = Tk_ - Tq_;           // query i sees keys <= i + coff
    if constexpr (CAUSAL) last = min(last, min(Tq_ - 1, qt * BM + BM - 1) + coff);
    // Visited key blocks: [u_first, u_last] in units of CK keys; LDS tiles of TK keys.
    const int t_first = first / TK;
    const int u_first = t_first * HALVES;                  // steps start on a tile boundary
    const int u_last = last >= 0 ? last / CK : -1;
    const int nsteps = last >= first ? u_last - u_first + 1 : 0;
    const int t_last = last >= 0 ? last / TK : -1;

    // ---- Q as the B operand of Sᵀ = K·Qᵀ: lane holds query (l%32), d = kk*16 + hl*8 + 0..7.
    // Rows past Tq are clamped to a valid row; their results are never stored.
    // FP8: lane holds query (l%32), d = s*64 + hl*32 + 0..31 (E4M3 operand layout).
    bf16x8 qreg[NB][KSTEPS];
    i32x8 q8[NB][KS8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = min(q0 + nb * 32 + l32, Tq_ - 1);
        if constexpr (FP8) {
#pragma unroll
            for (int s = 0; s < KS8; ++s) {
                const ET* p = qp + (size_t)row * rsq + s * 64 + hl * 32;
                const u32x4 a = ldg128(p), a1 = ldg128(p + 16);
                q8[nb][s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                                  (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                qreg[nb][kk] = as_bf16x8(ldg128(qp + (size_t)row * rsq + kk * 16 + hl * 8));
        }
    }

    // ---- tile loads straight into LDS: a tile is 8 KiB = 8 chunks of 1 KiB, wave w
    // fills chunks CPW*w .. CPW*w + CPW-1.  For LDS byte o of a tile (row r = o / RB, chunk
    // position p), K takes key perm(r) (bits 2,3 swapped within 32-row blocks),
    // chunk p ^ k_swz(r); V takes key r, chunk p ^ v_swz(r).  Keys past Tk read
    // as zeros (the buffer range check covers the per-lane offset, which is why the
    // tile offset is added there and not to the scalar offset; they are masked).
    // FP8: K tiles are codes (k8_swz); V does not use these loads (see vload below).
    constexpr int CPW = L::K_TILE / 1024 / NWAVE;    // K chunks per wave and tile
    constexpr int CPWV = L::V_TILE / 1024 / NWAVE;   // V chunks per wave and tile
    static_assert(CPW * NWAVE * 1024 == L::K_TILE && CPWV * NWAVE * 1024 == L::V_TILE,
                  "whole chunks per wave");
    uint32_t k_voff[CPW], v_voff[CPWV];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int o = (CPW * wave + i) * 1024 + lane * 16;
        const int r = o / L::RBK, pch = (o % L::RBK) / 16;
        const int kr = (r & ~31) | swap_bits23(r & 31);
        if constexpr (FP8) k_voff[i] = (uint32_t)(kr * rsk + (pch ^ k8_swz<D>(r)) * 16);
        else k_voff[i] = (uint32_t)(kr * rsk + (pch ^ k_swz<D>(r)) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < CPWV; ++i) {
        const int o = (CPWV * wave + i) * 1024 + lane * 16;
        const int r = o / L::RBV, pch = (o % L::RBV) / 16;
        v_voff[i] = (uint32_t)(r * rsk + (pch ^ v_swz<D>(r)) * 8) * 2u;
    }
    // Ring slots are counted from the first visited tile: tile t sits in K slot
    // (t - t_first) % K_RING and V slot (t - t_first) % V_RING; kcur / vcur
    // track the slots of the current tile.
    auto kslot_b = [&](int sl) -> unsigned char* { return smem_raw + sl * L::K_TILE; };
    // the same slots as LDS byte addresses (for the DMA's M0; scalar arithmetic only)
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)smem_raw);
    auto kslot_a = [&](int sl) -> uint32_t { return lds0 + (uint32_t)(sl * L::K_TILE); };
    auto vslot_a = [&](int sl) -> uint32_t {
        return lds0 + (uint32_t)(L::K_RING * L::K_TILE + sl * L::V_TILE);
    };
    auto vslot_b = [&](int sl) -> unsigned char* { return smem_raw + L::K_RING * L::K_TILE + sl * L::V_TILE; };
    auto kslot = [&](int sl) -> const bf16* { return reinterpret_cast<const bf16*>(kslot_b(sl)); };
    auto dma_k = [&](int t, int sl) {
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            dma16(krs, kslot_a(sl) + (uint32_t)((CPW * wave + i) * 1024), k_voff[i] + (uint32_t)t * TK * rsk * (uint32_t)ES, 0u);
    };
    auto dma_v = [&](int t, int sl) {
#pragma unroll
        for (int i = 0; i < CPWV; ++i)
            dma16(vrs, vslot_a(sl) + (uint32_t)((CPWV * wave + i) * 1024), v_voff[i] + (uint32_t)t * TK * rsk * 2u, 0u);
    };
    // FP8 V: thread tid loads codes 16*vt_j .. +15 of tile row vt_r into registers a tile
    // ahead and stores them, as bf16, as chunks 2*vt_j and 2*vt_j + 1 of that row of a bf16
    // V tile (the layout dma_v gives), so the Vᵀ reads are those of the bf16 kernel.
    constexpr int VJ = D / 16;
    static_assert(!FP8 || NT == TK * VJ, "one 16-byte V load per thread and tile");
    const int vt_r = tid / VJ, vt_j = tid % VJ;
    const uint32_t v8_off = (uint32_t)(vt_r * rsk + vt_j * 16);
    const int vw0 = vt_r * L::RBV + ((2 * vt_j) ^ v_swz<D>(vt_r)) * 16;
    const int vw1 = vt_r * L::RBV + ((2 * vt_j + 1) ^ v_swz<D>(vt_r)) * 16;
    auto vload = [&](int t) -> u32x4 { return bload16(vrs8, v8_off + (uint32_t)t * TK * rsk); };
    auto vstore = [&](const u32x4& w, int sl) {
        const u32x2 a0 = e4m3x4_to_bf16(w[0]), a1 = e4m3x4_to_bf16(w[1]);
        const u32x2 a2 = e4m3x4_to_bf16(w[2]), a3 = e4m3x4_to_bf16(w[3]);
        *reinterpret_cast<u32x4*>(vslot_b(sl) + vw0) = u32x4{a0[0], a0[1], a1[0], a1[1]};
        *reinterpret_cast<u32x4*>(vslot_b(sl) + vw1) = u32x4{a2[0], a2[1], a3[0], a3[1]};
    };
    u32x4 vraw = {};     // FP8: codes of the V tile two ahead of the current one
    int kcur = 0, vcur = 0;
    static_assert(L::K_RING == L::AHEAD + 2 && L::V_RING == L::AHEAD + 1, "slot arithmetic below");
    // Per-lane LDS offsets of the operand reads.
    //  K (A of K·Qᵀ): row hf*32 + l%32, chunk (kk*2 + hl) ^ k_swz(l % 32).
    const int kx = hl ^ k_swz<D>(l32);
    //  Vᵀ (A of Vᵀ·Pᵀ, transposed read): lane 16g+m addresses key row
    //  (g/2)*8 + m/4 (+4 for the second half) and d = db*32 + 16(g%2) + 4(m%4).
    const int vg = lane >> 4, vm = lane & 15;
    const int vrow = (vg >> 1) * 8 + (vm >> 2);
    const int vfv = v_swz<D>(vrow);
    const int vc0 = 2 * (vg & 1) + ((vm & 3) >> 1);
    const int vin = (vm & 1) * 4;                    // element offset inside the 16-byte chunk
    auto v_off = [&](int db) { return vrow * D + (((db * 4 + vc0) ^ vfv) * 8) + vin; };
    // LDS byte address of this lane's row block db in the current V slot, moved on with the
    // slot at each tile end, so the reads of a step take their row offsets as immediates
    uint32_t vaddr[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) vaddr[db] = vslot_a(0) + (uint32_t)(v_off(db) * 2);

    // Lane j reports whether key t*TK + j is padded or past Tk (lanes >= TK report 1).
    auto pad_flag = [&](int t) -> int {
        const int key = t * TK + lane;
        if (lane >= TK || key >= Tk_) return 1;
        return mp ? (int)(mp[key] != 0) : 0;
    };

    f32x16 oacc[DB][NB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][nb][i] = 0.f;
    // mc: the reference the weights are taken against, 2^(S·c - mc), in log2
    // units; always finite.  Kept negated (nmc = -mc), the addend of the fma that
    // forms every exponent.  lsum: running sum of the weights.
    float nmc[NB], lsum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { nmc[nb] = 0.f; lsum[nb] = 0.f; }

    // Sᵀ = K·Qᵀ for one key block (u) from a tile in LDS: element i of lane l
    // holds key (i/8)*16 + (l/32)*8 + i%8 of the block.
    // K rows of key block h (0 .. HALVES-1) of the tile in slot sl
    auto kblock = [&](int sl, int h) -> const bf16* { return kslot(sl) + (h * 32 + l32) * D; };
    auto k_opnd = [&](const bf16* krow, int kk) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(krow + ((kk * 2) ^ kx) * 8);
    };
    // FP8: K operand of k-step s (d = s*64 + hl*32 + 0..31) of key block hb in slot sl
    const int kf8 = k8_swz<D>(l32);
    auto k8_opnd = [&](int sl, int hb, int s) -> i32x8 {
        const unsigned char* row = kslot_b(sl) + (hb * 32 + l32) * L::RBK;
        const u32x4 a = *reinterpret_cast<const u32x4*>(row + ((4 * s + 2 * hl) ^ kf8) * 16);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(row + ((4 * s + 2 * hl + 1) ^ kf8) * 16);
        return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    auto qk_full = [&](f32x16 (&S)[NB]) {     // first block of slot 0
        if constexpr (FP8) {
#pragma unroll
            for (int s = 0; s < KS8; ++s) {
                const i32x8 a = k8_opnd(0, 0, s);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) S[nb] = mfma_e4m3(a, q8[nb][s], s == 0 ? f32x16{} : S[nb]);
            }
            return;
        }
        const bf16* kp_ = kblock(0, 0);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const bf16x8 a = k_opnd(kp_, kk);
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
    };

    // Blocks u_in0 .. u_in0 + in_span lie wholly inside [first, last]; without interior
    // holes nothing there is padded, and one unsigned compare recognises them (the range
    // is empty when there are holes or no such block).
    const int ui0 = (first + CK - 1) / CK, ui1 = (last + 1) / CK - 1;
    const bool any_in = ui1 >= ui0 && !holes;
    const int u_in0 = any_in ? ui0 : (1 << 30);
    const uint32_t in_span = any_in ? (uint32_t)(ui1 - ui0) : 0u;
    // bit i set: key u*CK + i of block u lies outside [first, last]
    auto edge_bits = [&](int u) -> uint32_t {
        const int lo = first - u * CK, hi = last - u * CK;
        uint32_t m = 0u;
        if (lo > 0) m |= lo >= 32 ? ~0u : (1u << lo) - 1u;
        if (hi < 31) m |= hi < 0 ? ~0u : ~((2u << hi) - 1u);
        return m;
    };
    // With interior holes, lane j of padf_nxt flags key j of the tile after the current
    // one, loaded a tile ahead; at a tile end (after its wait for loads) the flags are
    // gathered into the wave-uniform mask pm_next, which the next tile takes as pm_tile.
    uint64_t pm_tile = 0, pm_next = 0;
    int padf_nxt = 0;
    // Vᵀ operand (8 keys x one d per lane) of k-step k2 of half hf of the current V tile
    auto v_opnd = [&](int hf, int k2, int db) -> u32x4 {
        const uint32_t a = vaddr[db] + (uint32_t)((hf * 32 + k2 * 16) * D * 2);
        const u32x2 lo = ds_read_tr_at(a);
        const u32x2 hi = ds_read_tr_at(a + 4 * D * 2);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // The reference mc is set from the exact row max of the first visited block
    // that holds an unpadded key (then every weight of that block is <= 1) and
    // raised only when a 16-key chunk's weights sum past 2^TAU in some lane.
    int mc_set = 0;                 // wave-uniform (an SGPR, tested with one scalar compare)

    // One pipeline step for key block u = u_first + j: S holds its raw scores;
    // Sn receives block u+1's.  hf (the step's half within its LDS tile) is a
    // constant at each call site.
    // ka holds the K operands of the next QK product (block u+1 at step u):
    // they are read from LDS during the step before, so no step starts by
    // waiting on LDS.
    bf16x8 ka[KSTEPS];
    i32x8 ka8[KS8];
    auto step = [&](int j, const int hf, f32x16 (&S)[NB], f32x16 (&Sn)[NB]) {
        const int u = u_first + j;
        const int T = (int)((uint32_t)u / HALVES);   // u >= 0
        uint32_t pm = 0u;                           // bit i: key u*32+i padded
        if (__builtin_expect((uint32_t)(u - u_in0) > in_span, 0)) {   // an edge block, or holes
            pm = edge_bits(u);
            if (holes) {
                if (hf == 0) pm_tile = pm_next;
                pm |= (uint32_t)(pm_tile >> (hf * 32));
            }
            // Inside the edge branch, so that a block wholly inside the unpadded range passes
            // both tests with one branch not taken.
            if (pm != 0u) {         // workgroup-uniform: padded keys get -inf
                // element i of this lane is key (i/8)*16 + hl*8 + i%8 of the block
                const uint32_t pl = ((pm >> (hl * 8)) & 0xFFu) | (((pm >> (16 + hl * 8)) & 0xFFu) << 8);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if ((pl >> i) & 1u) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) S[nb][i] = kNegInf;
                    }
                }
            }
        }
        if constexpr (CAUSAL) {
            // key e of the block is past the limit of this lane's query nb iff
            // e > lim0 + nb*32 + l32; wave-uniform test on the wave's first query
            const int lim0 = q0 + coff - u * CK;
            if (lim0 < CK - 1) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = lim0 + nb * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if ((i >> 3) * 16 + hl * 8 + (i & 7) > lim) S[nb][i] = kNegInf;
                }
            }
        }
        if (__builtin_expect(__builtin_amdgcn_readfirstlane(mc_set) == 0, 0) && pm != ~0u) {   // once: first block with an unpadded key
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float m = S[nb][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) m = fmaxf(m, S[nb][i]);
                // a causal row may have no key at all (then any finite reference serves)
                m = pair_max(m);
                nmc[nb] = m == kNegInf ? 0.f : -(m * c);
            }
            mc_set = 1;
        }

        // ---- fixed block, issued slot by slot: the MFMA stream is
        //   QK(u+1) | PV(u, k-step 0) | PV(u, k-step 1)
        // and each slot also carries one stage of a three-stage softmax pipeline
        // (A: x = S·c - mc, B: p = 2^x, C: chunk sum += p, pack to bf16), so every
        // slot has independent vector work; LDS operands are read a few slots
        // ahead.  After each 16-key chunk is packed and before its PV MFMAs, its
        // per-lane sums are checked against 2^TAU (see rescale below).
        // K rows of block u+2, read here for the next step: at D = 64 (two blocks
        // per tile) that block is in tile T+1, published since the end of tile
        // T-1; at D = 128 it is tile T+2, read after this step's tile-end barrier.
        const int knext = kcur == L::K_RING - 1 ? 0 : kcur + 1;
        u32x4 va[DB], va1[DB];
        u32x4 pw[NB][PSTEPS];
        float cs[NB][PSTEPS];
        float xs[16][2], ps[16][2];
        auto rd_k = [&](int kk) { ka[kk] = k_opnd(kblock(knext, hf), kk); };
        auto rd_k8 = [&](int s) { ka8[s] = k8_opnd(knext, hf, s); };
        auto rd_v = [&](int db) { va[db] = v_opnd(hf, 0, db); };
        auto rd_v1 = [&](int db) { va1[db] = v_opnd(hf, 1, db); };
        // pair pp: chunk k2 = pp / (4*NB), query block nb, elements i, i+1
        auto pair_nb = [&](int pp) { return (pp / 4) % NB; };
        auto pair_i = [&](int pp) { return (pp / (4 * NB)) * 8 + (pp % 4) * 2; };
        auto stA = [&](int pp) {
            const int nb = pair_nb(pp), i = pair_i(pp);
            xs[pp][0] = __builtin_fmaf(S[nb][i], c, nmc[nb]);
            xs[pp][1] = __builtin_fmaf(S[nb][i + 1], c, nmc[nb]);
        };
        auto stB = [&](int pp) {
            ps[pp][0] = __builtin_amdgcn_exp2f(xs[pp][0]);
            ps[pp][1] = __builtin_amdgcn_exp2f(xs[pp][1]);
        };
        auto stC = [&](int pp) {
            const int nb = pair_nb(pp), k2 = pp / (4 * NB);
            if (pp % 4 == 0) cs[nb][k2] = ps[pp][0] + ps[pp][1];
            else cs[nb][k2] += ps[pp][0] + ps[pp][1];
            pw[nb][k2][pp % 4] = pack_bf16x2(ps[pp][0], ps[pp][1]);
        };
        auto softmax_slot = [&](int sl) {     // stages for slot sl of NPP + 2
            if (sl >= 1 && sl <= NPP) stB(sl - 1);
            if (sl < NPP) stA(sl);
            if (sl >= 2 && sl <= NPP + 1) stC(sl - 2);
        };
        // Lazy rescale of chunk k2 (rare; the common path never computes a row
        // max): if some lane's weights of the chunk sum past 2^TAU, raise mc to
        // the chunk's exact row max where that is higher, scale l and O by
        // 2^(old - new), and redo the chunk's weights, plus the stages of the
        // next chunk already in flight (at the check after slot CP+1, chunk 1's
        // stage A of pairs CP, CP+1 and stage B of pair CP).  Final O = acc / l and
        // LSE = (mc + log2 l)·ln 2 hold for any reference, so only rounding
        // changes.  Order: check(0) comes before any PV of chunk 0, and check(1)
        // after all of them and before any PV of chunk 1, so the scaled O holds
        // exactly the weights taken against the old reference.
        auto check = [&](int k2) {
            bool over = false;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) over |= cs[nb][k2] > kRescaleSum;
            // The rescale is rare: laid out off the common path, which then falls through
            // instead of branching over it (bf16 0.6-1.0% faster, E4M3 0.2%).
            const bool rescale = __ballot(over) != 0;
            if (__builtin_expect(rescale, 0)) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    // (highest index first: no partial max shared with the first-block
                    // reference above, which the compiler would otherwise hoist into
                    // the common path)
                    float m = S[nb][k2 * 8 + 7];
#pragma unroll
                    for (int i = 6; i >= 0; --i) m = fmaxf(m, S[nb][k2 * 8 + i]);
                    const float mn = fmaxf(-nmc[nb], pair_max(m) * c);
                    const float alpha = __builtin_amdgcn_exp2f(-nmc[nb] - mn);
                    nmc[nb] = -mn;
                    lsum[nb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][nb][i] *= alpha;
                }
#pragma unroll
                for (int q = 0; q < 4 * NB; ++q) {
                    const int pp = k2 * 4 * NB + q;
                    stA(pp);
                    stB(pp);
                    stC(pp);
                }
                if (k2 == 0) {
                    stA(CP);
                    stA(CP + 1);
                    stB(CP);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) lsum[nb] += cs[nb][k2];
        };
        auto qk8_one = [&](int qi) {    // FP8: qi = s*NB + nb
            const int nb = qi % NB, s = qi / NB;
            Sn[nb] = mfma_e4m3(ka8[s], q8[nb][s], s == 0 ? f32x16{} : Sn[nb]);
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
        auto pv_one = [&](int k2, int pi) {    // PV(u, k-step k2): pi = db*NB + nb
            const int nb = pi % NB, db = pi / NB;
            const u32x4 a = k2 == 0 ? va[db] : va1[db];
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pw[nb][k2]),
                                                                    oacc[db][nb], 0, 0, 0);
        };
        // The slots are fenced off from each other except in the bf16 D = 64 step, where two
        // waves per SIMD run it and the compiler's own interleaving of the slots measured faster.
        auto fence = [&]() {
            if constexpr (FP8 || D != 64) __builtin_amdgcn_sched_barrier(0);
        };

        if constexpr (D == 64) {
            // unfenced (bf16): the compiler's small-GEMM interleave of LDS reads and MFMAs
            // measured ~0.6% faster than its default order at P = 11,616
            if constexpr (!FP8) __builtin_amdgcn_iglp_opt(0);
            // 22 slots: 0-7 QK(u+1), 10-13 PV(u,0) (chunk 0 packed by slot 9),
            // 18-21 PV(u,1) (chunk 1 packed by slot 17); softmax in 0-17.  FP8: QK(u+1)
            // is two E4M3 MFMAs, in slots 0 and 2.
#pragma unroll
            for (int sl = 0; sl < 22; ++sl) {
                if (sl == 4) { rd_v(0); rd_v(1); }
                if (sl == 12) { rd_v1(0); rd_v1(1); }
                if constexpr (FP8) {
                    if (sl == 14) rd_k8(0);
                    if (sl == 0 || sl == 2) qk8_one(sl / 2);
                } else {
                    if (sl == 14) { rd_k(0); rd_k(1); }      // QK(u+2) operands: after QK(u+1) issued
                    if (sl == 15) { rd_k(2); rd_k(3); }
                    if (sl < 8) qk_one(sl);
                }
                if (sl >= 10 && sl < 14) pv_one(0, sl - 10);
                else if (sl >= 18) pv_one(1, sl - 18);
                if (sl < NPP + 2) softmax_slot(sl);
                fence();
                if (sl == CP + 1) check(0);
                if (sl == NPP + 1) check(1);
            }
        } else {
            // D=128, one query block: 16 slots.  QK(u+1) is one chain of 8 MFMAs
            // (slots 0-5, 7, 9); PV(u,0) in 6, 8, 10, 11 once chunk 0 is packed
            // (slot 5); PV(u,1) in 12-15 once chunk 1 is packed (slot 9) and checked
            // (after slot 11, when every PV of chunk 0 has been issued); softmax in 0-9.  FP8: QK(u+1) is a chain of two E4M3 MFMAs (slots 0, 4).
#pragma unroll
            for (int sl = 0; sl < 16; ++sl) {
                if (sl == 1) { rd_v(0); rd_v(1); }
                if (sl == 2) { rd_v(2); rd_v(3); }
                if (sl == 7) { rd_v1(0); rd_v1(1); }
                if (sl == 8) { rd_v1(2); rd_v1(3); }
                if constexpr (FP8) {
                    static_assert(HALVES == 2, "K of block u+2 is in the next tile");
                    if (sl == 10) rd_k8(0);
                    if (sl == 11) rd_k8(1);
                    if (sl == 0 || sl == 4) qk8_one(sl / 4);
                } else {
                    if constexpr (HALVES == 2) {          // QK(u+2) operands, after QK(u+1) issued
                        if (sl == 10) { rd_k(0); rd_k(1); }
                        if (sl == 11) { rd_k(2); rd_k(3); }
                        if (sl == 12) { rd_k(4); rd_k(5); }
                        if (sl == 13) { rd_k(6); rd_k(7); }
                    }
                    if (sl < 6) qk_one(sl);
                    else if (sl == 7) qk_one(6);
                    else if (sl == 9) qk_one(7);
                }
                if (sl == 6) pv_one(0, 0);
                else if (sl == 8) pv_one(0, 1);
                else if (sl == 10) pv_one(0, 2);
                else if (sl == 11) pv_one(0, 3);
                else if (sl >= 12) pv_one(1, sl - 12);
                if (sl < NPP + 2) softmax_slot(sl);
                fence();
                if (sl == CP + 1) check(0);
                if (sl == 11) check(1);
            }
        }

        // ---- end of an LDS tile: publish the tiles loaded during the previous one, then
        // start loading the next batch.
        //  bf16: K tile T+5 and V tile T+4 (into the slots tile T leaves), always issued (a
        //  tile past the last reads zeros through the buffer range), so every batch is
        //  CPW + CPWV loads and waiting for at most two batches outstanding means the batches
        //  issued at the ends of tiles T-1 and T-2 may still be in flight while the one from
        //  T-3 (K_{T+2}, V_{T+1}: read during tile T+1) has landed.  The loads are asm with a
        //  memory clobber and so is the wait, so this count is a property of the source;
        //  any loads the compiler adds after a batch (the hole flags) only make it stricter.
        //  The look-ahead offsets of tiles past the last may exceed 32 bits and wrap; the
        //  wrapped offset is still range-checked by the buffer load and the slot is never read.
        //  E4M3: K tile T+3 and the V codes of T+3 (registers), one tile ahead, waiting for all.
        //  The hole flags are ordinary loads the compiler waits for with a full count, so they
        //  are gathered (and the next one issued) before the batch, not behind it.
        if (hf == HALVES - 1) {
            if constexpr (FP8) wait_vmem();     // this wave's part of K_{T+2} and V_{T+1} has landed
            else wait_vmem_le<(L::AHEAD - 1) * (CPW + CPWV)>();    // all but the two newest batches
            if (__builtin_expect(holes, 0)) {      // off the common path, which falls through
                pm_next = __ballot(padf_nxt) & TILE_BITS;
                padf_nxt = pad_flag(min(T + 2, t_last));
            }
            __syncthreads();
            if constexpr (FP8) {
                if (T + 3 <= t_last) dma_k(T + 3, kcur);     // into the slot tile T leaves
                if (T + 2 <= t_last) vstore(vraw, vcur);   // codes loaded during tile T-1
                if (T + 3 <= t_last) vraw = vload(T + 3);
            } else {
                dma_k(T + L::AHEAD + 2, kcur);
                dma_v(T + L::AHEAD + 1, vcur);
            }
            kcur = knext;
            const bool vwrap = vcur == L::V_RING - 1;
            vcur = vwrap ? 0 : vcur + 1;
            const uint32_t vstep = vwrap ? (uint32_t)(-(L::V_RING - 1) * L::V_TILE) : (uint32_t)L::V_TILE;
#pragma unroll
            for (int db = 0; db < DB; ++db) vaddr[db] += vstep;
            if constexpr (HALVES == 1 && !FP8) {    // K of block u+2 = tile T+2, just published
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) ka[kk] = k_opnd(kblock(kcur == L::K_RING - 1 ? 0 : kcur + 1, 0), kk);
            }
        }
    };

    if (nsteps > 0) {
        f32x16 sA[NB], sB[NB];
        u32x4 vraw1 = {};
        dma_k(t_first, 0);
        if constexpr (FP8) vraw = vload(t_first);
        else dma_v(t_first, 0);
        if (t_first + 1 <= t_last) {
            dma_k(t_first + 1, 1);
            if constexpr (FP8) vraw1 = vload(t_first + 1);
            else dma_v(t_first + 1, 1);
        }
        int padf0 = 0;
        if (holes) {
            padf0 = pad_flag(t_first);
            padf_nxt = pad_flag(min(t_first + 1, t_last));
        }
        wait_vmem();
        if (holes) pm_next = __ballot(padf0) & TILE_BITS;
        if constexpr (FP8) {
            vstore(vraw, 0);
            if (t_first + 1 <= t_last) vstore(vraw1, 1);
        }
        __syncthreads();
        if constexpr (FP8) {
            if (t_first + 2 <= t_last) {     // waited for at the end of tile t_first
                dma_k(t_first + 2, 2);
                vraw = vload(t_first + 2);
            }
        } else {
            // K_{t+2}, then the batches of "tiles t_first - 2 and t_first - 1" (K_{t+3}, V_{t+2};
            // K_{t+4}, V_{t+3}), in this order: the ring then holds K tiles t .. t+4 and V tiles
            // t .. t+3, and the first tile end's wait (two batches outstanding) covers K_{t+2}
            dma_k(t_first + 2, 2);
            dma_k(t_first + 3, 3);
            dma_v(t_first + 2, 2);
            dma_k(t_first + 4, 4);
            dma_v(t_first + 3, 3);
        }
        qk_full(sA);
        if constexpr (FP8) {
            static_assert(!FP8 || HALVES == 2, "K of block u_first + 1 is in slot 0");
#pragma unroll
            for (int s = 0; s < KS8; ++s) ka8[s] = k8_opnd(0, 1, s);
        } else {
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)     // K of block u_first + 1
                ka[kk] = HALVES == 1 ? k_opnd(kblock(1, 0), kk) : k_opnd(kblock(0, 1), kk);
        }
        int j = 0;
        for (; j + 1 < nsteps; j += 2) {
            step(j, 0, sA, sB);
            step(j + 1, HALVES - 1, sB, sA);
        }
        if (j < nsteps) step(j, 0, sA, sB);
    }

    // the look-ahead batches (tiles past the last) land before the workgroup can end
    wait_vmem();
    // ---- epilogue: O = acc / l, LSE = (m·c + log2 l)·ln 2
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float lt = pair_sum(lsum[nb]);
        const float inv = lt > 0.f ? osc / lt : 0.f;
        const int qi = q0 + nb * 32 + l32;
        if (qi < Tq_) {
            bf16* orow = o + q_row0 + (size_t)qi * rsq;
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
                lse[l_row0 + (size_t)qi] = lt > 0.f ? (__log2f(lt) - nmc[nb]) * kLn2 : kNegInf;
        }
    }
}

template <int D, bool WRITE_LSE, bool VARLEN, bool CAUSAL, bool FP8 = false>
hipError_t launch_one(const FwdArgs& a) {
    using L = Lds<D, FP8>;
    using ET = Elem<FP8>;
    auto kern = fwd_bf16_kernel<D, WRITE_LSE, VARLEN, CAUSAL, FP8>;
    constexpr int BM = kBM<D>;
    const int n_qt = (a.Tq + BM - 1) / BM;       // varlen: Tq = the longest sequence
    const int total = a.B * a.H * n_qt;
    int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    int nparts = 1, tpp = 0;
    const int H_kv = a.H_kv > 0 ? a.H_kv : a.H;
    if (VARLEN) {   // chunk parts dealt to the XCDs in turn (see the kernel)
        const int chunks = a.B * H_kv, S = (a.H / H_kv) * n_qt;
        int g = kNumXcd, x = chunks;
        while (x % g) g /= 2;                     // gcd(chunks, 8): 8 is a power of two
        nparts = kNumXcd / g;
        tpp = (S + nparts - 1) / nparts;
        grid = chunks * nparts * tpp;             // chunks * nparts is a multiple of 8
        ATTN_CHECK((long long)nparts * tpp >= S && chunks * nparts % kNumXcd == 0, "parts cover every tile");
    } else {
        ATTN_CHECK(grid % kNumXcd == 0 && grid >= total, "the XCD swizzle covers every tile");
    }
    ATTN_CHECK(L::BYTES <= kLdsBytesPerCu, "LDS tile rings fit a CU");
    ATTN_CHECK(n_qt >= 1 && (long long)n_qt * BM >= a.Tq, "q-tiles cover every query row");
    ATTN_CHECK(grid >= 1 && grid <= kMaxGrid, "grid size");
    ATTN_CHECK(H_kv >= 1 && a.H % H_kv == 0, "query heads group onto KV heads");
    // per-lane tile offsets are 32-bit: rows past the last one (up to a tile) times the row stride
    ATTN_CHECK(((VARLEN ? (long long)a.total_k : a.Tk) + L::TK) * (VARLEN ? (long long)H_kv * a.D : a.D) *
                       (long long)sizeof(ET) < (1ll << 32),
               "K/V tile offsets fit 32 bits");
    // LDS above 64 KiB must be opted into once per kernel (thread-safe static init).
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    if (attr != hipSuccess) return attr;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * Cfg<D>::NWAVE), L::BYTES, (hipStream_t)a.stream,
                       (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.mask,
                       (bf16*)a.o, a.lse, a.H, a.H_kv > 0 ? a.H_kv : a.H, a.Tq, a.Tk, c, n_qt, total, nparts, tpp,
                       a.cu_q, a.cu_k, a.total_q, a.total_k, a.q_scale, a.k_scale, a.v_scale);
    return hipGetLastError();
}

template <int D, bool WRITE_LSE>
hipError_t launch_lse(const FwdArgs& a) {
    if (a.varlen)
        return a.causal ? launch_one<D, WRITE_LSE, true, true>(a) : launch_one<D, WRITE_LSE, true, false>(a);
    return a.causal ? launch_one<D, WRITE_LSE, false, true>(a) : launch_one<D, WRITE_LSE, false, false>(a);
}

template <int D>
hipError_t launch(const FwdArgs& a) {
    return a.lse ? launch_lse<D, true>(a) : launch_lse<D, false>(a);
}

// E4M3 inputs, either layout (GQA, padding and causal as in the bf16 kernel).
template <int D, bool WRITE_LSE>
hipError_t launch_fp8_lse(const FwdArgs& a) {
    if (a.varlen)
        return a.causal ? launch_one<D, WRITE_LSE, true, true, true>(a) : launch_one<D, WRITE_LSE, true, false, true>(a);
    return a.causal ? launch_one<D, WRITE_LSE, false, true, true>(a) : launch_one<D, WRITE_LSE, false, false, true>(a);
}
template <int D>
hipError_t launch_fp8(const FwdArgs& a) {
    return a.lse ? launch_fp8_lse<D, true>(a) : launch_fp8_lse<D, false>(a);
}

}  // namespace fwdk
}  // namespace mattn
