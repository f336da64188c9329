// bf16 single-token decode against the KV cache (GQA): persistent
// matrix-core wavefronts streaming the cache.
//
// The current token's query attends over every cached K/V position of its
// sequence (agentlenshq.com, "nanoVLM에서 KV 캐시 구현", section "KV 캐싱이
// 추론을 최적화하는 방법"); the work is reading the cache, 2·H_kv·D·2 bytes
// per cached token (blog.ruahverce.com, LLM inference memory accounting 2/10,
// "10. KV Cache Byte 공식"), and the query heads that share a KV head (GQA,
// same page "11. 계산 예시: GQA Decoder") are served by one read.
//
// Work decomposition ("stream" split).  The cache is cut into blocks of 32
// tokens of one item = (sequence b, split s of kDecodeSplit tokens, KV head
// g, group hg of up to 32 of g's query heads), in the global order b, s,
// (g, hg), block.  Every wavefront derives the same order from the lengths
// on the device and takes one contiguous range of bpw blocks (bpw >= the
// blocks of a split, so an item is shared by at most two wavefronts).  A
// wavefront streams its range without draining at item boundaries and
// writes one unnormalised partial (O, reference, weight sum) per item it
// touches: part 0 from the wavefront that holds the item's first block,
// part 1 from the next one.  The combine kernel recomputes the same order
// to find the parts and merges them with the log-sum-exp rule of the chunk
// merge (sglang PR 49078 analysis, "1. aiter.py").
//
// Per block, on the matrix cores, with the query heads as the 32 columns:
//   Sᵀ[key, head] = K·Qᵀ   (A = 32 K rows from LDS, B = Q from registers)
//   Oᵀ[d, head]  += Vᵀ·Pᵀ  (A = Vᵀ via the transposing LDS read, B = P)
// (lane l owns head column l%32 and 16 of the block's keys; K rows are
// stored with bits 2 and 3 of the row index swapped so a lane's P values are
// consecutive accumulator elements).  K, V and each item's Q reach LDS by
// direct buffer->LDS loads issued R-1 blocks ahead; buffer ranges end at the
// item's last token, so look-ahead past it reads zeros without touching
// memory.  Softmax per head column: weights 2^(S·c - mc), mc from the exact
// max of the item's first block here, raised only when a 16-key chunk's
// per-lane sum passes 2^8 (then l and O are rescaled).
#include "common.cuh"
#include "launch.h"
#include "mfma_lds.cuh"

namespace mattn {
namespace {
using namespace mattn::mfma;

constexpr int CK = 32;                         // tokens per block
constexpr int SB = kDecodeSplit / CK;          // blocks of a full split
constexpr float kRescaleSum = 256.0f;          // 2^8
static_assert(kDecodeSplit % CK == 0, "splits are whole blocks");

template <int D> struct Geo {
    static constexpr int RB = D * 2;               // bytes per cache row
    static constexpr int BLK = CK * RB;            // bytes of one K (or V) block
    static constexpr int NCH = BLK / 1024;         // 1 KiB loads per block
    static constexpr int R = D == 64 ? 4 : 3;      // ring depth in blocks
    static constexpr int QCH = 32 * RB / 1024;     // 1 KiB loads of a full 32-head Q slot
    static constexpr int RING = R * 2 * BLK;       // LDS bytes of the K/V ring
};
// Q slot bytes: the group's heads (at most 32) rounded up to whole 1 KiB loads.
inline int q_slot_bytes(int G, int D) { return (min(G, 32) * D * 2 + 1023) / 1024 * 1024; }

__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int T_max) {
    return min(max(lens[b], 0), T_max);
}

// inclusive prefix sum over the 64 lanes of the wavefront
__device__ __forceinline__ int wave_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// N loads of 16 bytes per lane straight into LDS: load k writes LDS bytes
// [m[k] + 16*lane, +16) from buffer offset vo[k] (per lane).  One statement
// per block keeps the M0 save / restore to once per N loads.
__device__ __forceinline__ void dma_x4(i32x4_sgpr r, const uint32_t* m, const uint32_t* vo) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %5, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %6, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %7, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %4\n\tbuffer_load_dwordx4 %8, %9, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m[0]), "s"(m[1]), "s"(m[2]), "s"(m[3]), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(r)
        : "memory");
}
__device__ __forceinline__ void dma_x2(i32x4_sgpr r, const uint32_t* m, const uint32_t* vo) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m[0]), "s"(m[1]), "v"(vo[0]), "v"(vo[1]), "s"(r)
        : "memory");
}
template <int N>
__device__ __forceinline__ void dma_n(i32x4_sgpr r, uint32_t lds_addr, const uint32_t* vo) {
    static_assert(N % 2 == 0, "whole pairs");
#pragma unroll
    for (int k = 0; k + 4 <= N; k += 4) {
        const uint32_t m[4] = {lds_addr + (k + 0) * 1024u, lds_addr + (k + 1) * 1024u, lds_addr + (k + 2) * 1024u,
                               lds_addr + (k + 3) * 1024u};
        dma_x4(r, m, vo + k);
    }
    if constexpr (N % 4 == 2) {
        const uint32_t m[2] = {lds_addr + (N - 2) * 1024u, lds_addr + (N - 1) * 1024u};
        dma_x2(r, m, vo + N - 2);
    }
}

// Two dwords at byte offsets o0, o1 of a wavefront-uniform table (scalar loads: they
// count in lgkmcnt, not vmcnt, so the vector-load accounting of the look-ahead is not
// disturbed).  Both offsets must lie inside the table.
__device__ __forceinline__ void sload2(const int32_t* p, uint32_t o0, uint32_t o1, int& a, int& b) {
    asm volatile(
        "s_load_dword %0, %2, %3\n\t"
        "s_load_dword %1, %2, %4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(a), "=&s"(b)
        : "s"(p), "s"(o0), "s"(o1)
        : "memory");
}

// Stores written as inline assembly so that their number is exact: stores
// count in vmcnt like loads, and the waits of the look-ahead stream allow for
// the partial-result stores issued since a block's loads.  Every lane issues
// them (offsets past the buffer range are dropped); the trailing s_nop keeps
// the data registers unmodified for the cycle after the last store.
__device__ __forceinline__ void store_x4x4(i32x4_sgpr r, uint32_t o0, u32x4 a, uint32_t o1, u32x4 b,
                                           uint32_t o2, u32x4 c2, uint32_t o3, u32x4 d2) {
    asm volatile(
        "buffer_store_dwordx4 %0, %1, %8, 0 offen\n\t"
        "buffer_store_dwordx4 %2, %3, %8, 0 offen\n\t"
        "buffer_store_dwordx4 %4, %5, %8, 0 offen\n\t"
        "buffer_store_dwordx4 %6, %7, %8, 0 offen\n\t"
        "s_nop 1"
        :
        : "v"(a), "v"(o0), "v"(b), "v"(o1), "v"(c2), "v"(o2), "v"(d2), "v"(o3), "s"(r)
        : "memory");
}
__device__ __forceinline__ void store_x2(i32x4_sgpr r, uint32_t o, u32x2 v) {
    asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen\n\ts_nop 1" : : "v"(v), "v"(o), "s"(r) : "memory");
}

// Clamped sequence lengths as seen by one wavefront: with at most 64
// sequences lane b holds len_b in a register (read back with readlane, no
// memory round trip); beyond that they are read from memory.
struct Lens {
    const int32_t* p;
    int B, T_max, reg;
    __device__ int get(int b) const { return B <= 64 ? __builtin_amdgcn_readlane(reg, b) : seq_len(p, b, T_max); }
};
__device__ __forceinline__ Lens load_lens(const int32_t* lens, int B, int T_max) {
    const int lane = threadIdx.x & 63;
    Lens L;
    L.p = lens;
    L.B = B;
    L.T_max = T_max;
    L.reg = lane < B ? seq_len(lens, lane, T_max) : 0;
    return L;
}

struct Plan {
    int total;   // blocks over all items
    int bpw;     // blocks per wavefront
};

// The block order: the plan and the sequence holding global block w*bpw (b0,
// with `before` blocks ahead of it).  Identical in every wavefront.
__device__ void make_plan(const Lens& L, int HG, int nwaves, int w, Plan& P, int& b0, int& before) {
    const int lane = threadIdx.x & 63;
    auto nblocks = [&](int len) { return (len + CK - 1) / CK * HG; };
    if (L.B <= 64) {
        const int n = nblocks(L.reg);
        const int inc = wave_scan(n);
        P.total = __builtin_amdgcn_readlane(inc, 63);
        P.bpw = max(SB, (P.total + nwaves - 1) / nwaves);
        const int a = w * P.bpw;
        const uint64_t m = __ballot(lane < L.B && inc > a);
        b0 = m ? __builtin_ctzll(m) : L.B;
        before = m ? __builtin_amdgcn_readlane(inc - n, b0) : P.total;
        return;
    }
    int total = 0;
    for (int base = 0; base < L.B; base += 64) {
        const int b = base + lane;
        total += __builtin_amdgcn_readlane(wave_scan(b < L.B ? nblocks(seq_len(L.p, b, L.T_max)) : 0), 63);
    }
    P.total = total;
    P.bpw = max(SB, (total + nwaves - 1) / nwaves);
    const int a = w * P.bpw;
    int carry = 0;
    b0 = L.B;
    before = total;
    for (int base = 0; base < L.B; base += 64) {
        const int b = base + lane;
        const int n = b < L.B ? nblocks(seq_len(L.p, b, L.T_max)) : 0;
        const int inc = wave_scan(n) + carry;
        const uint64_t m = __ballot(b < L.B && inc > a);
        if (m) {
            const int f = __builtin_ctzll(m);
            b0 = base + f;
            before = __builtin_amdgcn_readlane(inc - n, f);
            return;
        }
        carry = __builtin_amdgcn_readlane(inc, 63);
    }
}

// Position in the global block order (all fields wavefront-uniform).
struct Cursor {
    int b, len, full, nsplit;   // sequence, its length, full splits, splits
    int s, it, i, nb, t_end;    // split, item within the split, block within the item, blocks, item end
    int g, hg;                  // KV head and query-head group of the item (it = g*n_hg + hg)
};

__device__ __forceinline__ void set_split(Cursor& c) {
    if (c.s < c.full) {
        c.nb = SB;
        c.t_end = (c.s + 1) * kDecodeSplit;
    } else {
        c.nb = (c.len - c.full * kDecodeSplit + CK - 1) / CK;
        c.t_end = c.len;
    }
}
__device__ __forceinline__ void set_seq(Cursor& c, int len) {
    c.len = len;
    c.full = len / kDecodeSplit;
    c.nsplit = (len + kDecodeSplit - 1) / kDecodeSplit;
}
// Cursor at local block lb of sequence b.
__device__ Cursor cursor_at(const Lens& L, int HG, int n_hg, int b, int lb) {
    Cursor c;
    c.b = b;
    set_seq(c, L.get(b));
    const int fb = c.full * HG * SB;
    if (lb < fb) {
        c.s = lb / (HG * SB);
        const int q = lb - c.s * HG * SB;
        c.it = q / SB;
        c.i = q - c.it * SB;
    } else {
        c.s = c.full;
        set_split(c);
        const int q = lb - fb;
        c.it = q / c.nb;
        c.i = q - c.it * c.nb;
    }
    set_split(c);
    c.g = c.it / n_hg;
    c.hg = c.it - c.g * n_hg;
    return c;
}
// Next block in the global order.
__device__ __forceinline__ void advance(Cursor& c, const Lens& L, int HG, int n_hg) {
    if (++c.i < c.nb) return;
    c.i = 0;
    if (++c.it < HG) {
        if (++c.hg == n_hg) {
            c.hg = 0;
            ++c.g;
        }
        return;
    }
    c.it = 0;
    c.g = 0;
    c.hg = 0;
    if (++c.s < c.nsplit) {
        set_split(c);
        return;
    }
    c.s = 0;
    int len = 0;
    do {
        ++c.b;
    } while (c.b < L.B && (len = L.get(c.b)) == 0);
    if (c.b < L.B) {
        set_seq(c, len);
        set_split(c);
    }
}

// PAGED: kc / vc are page pools [num_pages, H_kv, 2^lps, D]; token t of sequence b is
// row t mod 2^lps of page bt[b * max_pages + (t >> lps)] (entries clamped to
// [0, num_pages)), T_max = max_pages << lps.  A 32-token block is loaded as two
// 16-token halves, each inside one page, each through its own buffer range.
template <int D, bool PAGED>
__global__ __launch_bounds__(64)
void decode_stream_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                          const bf16* __restrict__ vc, const int32_t* __restrict__ lens,
                          float* __restrict__ ws_o, float* __restrict__ ws_ml,
                          int B, int H_q, int H_kv, int T_max, int G, int n_hg, int nsplit,
                          int nwaves, int qb, float c,
                          const int32_t* __restrict__ bt, int lps, int max_pages, int num_pages) {
    using Gm = Geo<D>;
    constexpr int RB = Gm::RB, BLK = Gm::BLK, NCH = Gm::NCH, R = Gm::R, QCH = Gm::QCH;
    constexpr int KSTEPS = D / 16;     // MFMA k-steps of K·Qᵀ
    constexpr int DB = D / 32;         // 32-row blocks of Oᵀ
    constexpr int NWAIT = (R - 1) * 2 * NCH;   // loads younger than a block's own
    constexpr int NST = 4 * DB + 1;            // stores of one partial result (per lane)
    static_assert(NWAIT + (R - 1) * QCH <= 63, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int HG = H_kv * n_hg;
    const Lens L = load_lens(lens, B, T_max);
    Plan P;
    int b0, before;
    const int w = blockIdx.x;
    make_plan(L, HG, nwaves, w, P, b0, before);
    const int a0 = w * P.bpw;
    if (a0 >= P.total) return;
    const int nblk = min(P.total, a0 + P.bpw) - a0;
    b0 = __builtin_amdgcn_readfirstlane(b0);
    before = __builtin_amdgcn_readfirstlane(before);

    const int lane = threadIdx.x;
    const int hl = lane >> 5, l32 = lane & 31;

    // LDS byte o of a block: row r = o / RB, chunk position p.  K row r holds
    // key swap_bits23(r), chunk p = global chunk p ^ k_swz(r); V row r holds key r,
    // chunk p = global chunk p ^ v_swz(r).  A Q slot holds the group's heads as
    // rows in order.
    uint32_t k_voff[NCH], v_voff[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int o = ch * 1024 + lane * 16;
        const int r = o / RB, p = (o % RB) / 16;
        k_voff[ch] = (uint32_t)(swap_bits23(r) * RB + (p ^ k_swz<D>(r)) * 16);
        v_voff[ch] = (uint32_t)(r * RB + (p ^ v_swz<D>(r)) * 16);
    }
    auto kblk = [&](int sl) { return lds + sl * 2 * BLK; };
    auto vblk = [&](int sl) { return lds + sl * 2 * BLK + BLK; };
    auto qslot = [&](int sl) { return lds + Gm::RING + sl * qb; };
    // LDS byte address of the dynamic area (a constant of the launch)
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)lds));

    // Issue side: K, V (and, at an item's first block, its Q) of the block at
    // cursor ic into ring slot sl; past the wavefront's range, zero-range loads
    // keep the count of loads per block fixed without touching memory.  The
    // buffer descriptors are rebuilt only when the cursor enters a new item.
    Cursor ic = cursor_at(L, HG, n_hg, b0, a0 - before);
    int qs_issue = 0;            // Q slot of the item the issue cursor is in
    const i32x4_sgpr zrs = make_rsrc(kc, 0u);
    i32x4_sgpr krs, vrs;
    auto set_item = [&]() {
        if constexpr (!PAGED) {
            const size_t head = ((size_t)ic.b * H_kv + ic.g) * (size_t)T_max * D;
            krs = make_rsrc(kc + head, (uint32_t)ic.t_end * RB);
            vrs = make_rsrc(vc + head, (uint32_t)ic.t_end * RB);
        }
    };
    set_item();
    // Paged: a 32-token block is two 16-token halves; LDS chunks [0, NCH/2) hold keys
    // 0..15 of the block and chunks [NCH/2, NCH) keys 16..31 (the K row permutation
    // swaps bits 2 and 3 only, so it stays inside each half).
    constexpr int HCH = NCH / 2;
    auto issue_paged = [&](bool live, int sl) {
        const int t0 = ic.s * kDecodeSplit + ic.i * CK;
        i32x4_sgpr kh[2] = {zrs, zrs}, vh[2] = {zrs, zrs};
        uint32_t roff[2] = {0u, 0u};
        if (live) {
            // table entries of the halves; a half past the item's end reuses the last
            // valid token's entry (it is then read through the zero range)
            const int last = ic.t_end - 1;
            const int pi0 = t0 >> lps, pi1 = min(t0 + 16, last) >> lps;
            const uint32_t rowb = (uint32_t)ic.b * (uint32_t)max_pages * 4u;
            int e0, e1;
            sload2(bt, __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi0 * 4u),
                   __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi1 * 4u), e0, e1);
            const int pe[2] = {e0, e1}, pidx[2] = {pi0, pi1};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int th = t0 + 16 * h;
                if (th < ic.t_end) {
                    const int page = min(max(pe[h], 0), num_pages - 1);
                    const int pstart = pidx[h] << lps;
                    const int rows = min(1 << lps, ic.t_end - pstart);
                    const size_t head = (((size_t)page * H_kv + ic.g) << lps) * D;
                    kh[h] = make_rsrc(kc + head, (uint32_t)rows * RB);
                    vh[h] = make_rsrc(vc + head, (uint32_t)rows * RB);
                    roff[h] = (uint32_t)(th - pstart) * RB;
                }
            }
        }
        uint32_t vo[NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) vo[ch] = roff[ch / HCH] + k_voff[ch] - (ch / HCH) * 16u * RB;
        dma_n<HCH>(kh[0], lds0 + sl * 2 * BLK, vo);
        dma_n<HCH>(kh[1], lds0 + sl * 2 * BLK + HCH * 1024, vo + HCH);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) vo[ch] = roff[ch / HCH] + v_voff[ch] - (ch / HCH) * 16u * RB;
        dma_n<HCH>(vh[0], lds0 + sl * 2 * BLK + BLK, vo);
        dma_n<HCH>(vh[1], lds0 + sl * 2 * BLK + BLK + HCH * 1024, vo + HCH);
    };
    auto issue = [&](bool live, bool first_of_item, int sl) {
        if constexpr (PAGED) {
            issue_paged(live, sl);
        } else {
            const uint32_t row0 = (uint32_t)(ic.s * kDecodeSplit + ic.i * CK) * RB;
            uint32_t vo[NCH];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) vo[ch] = row0 + k_voff[ch];
            dma_n<NCH>(live ? krs : zrs, lds0 + sl * 2 * BLK, vo);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) vo[ch] = row0 + v_voff[ch];
            dma_n<NCH>(live ? vrs : zrs, lds0 + sl * 2 * BLK + BLK, vo);
        }
        if (live && first_of_item) {
            const int ncols = min(32, G - ic.hg * 32);
            const i32x4_sgpr qrs = make_rsrc(q + ((size_t)ic.b * H_q + ic.g * G + ic.hg * 32) * D,
                                             (uint32_t)(ncols * RB));
#pragma unroll
            for (int ch = 0; ch < QCH; ++ch)
                if (ch * 1024 < ncols * RB)
                    dma16(qrs, qslot(qs_issue) + ch * 1024, (uint32_t)(ch * 1024 + lane * 16), 0u);
        }
    };
    // the issue cursor's step: the next block, a new descriptor pair on a new item
    auto issue_advance = [&]() {
        advance(ic, L, HG, n_hg);
        if (ic.i == 0) {
            qs_issue = qs_issue == R - 1 ? 0 : qs_issue + 1;
            set_item();
        }
    };
    // Q of the wavefront's first item (loaded at its first block even when the
    // range starts inside the item).
    int issued = 0;
#pragma unroll
    for (int j = 0; j < R - 1; ++j) {
        const bool live = issued < nblk;
        issue(live, live && (ic.i == 0 || issued == 0), j);
        if (live) {
            ++issued;
            issue_advance();
        }
    }

    // Compute side.
    Cursor cc = cursor_at(L, HG, n_hg, b0, a0 - before);
    int part = cc.i == 0 ? 0 : 1;
    int qs = 0;
    bf16x8 qreg[KSTEPS];
    bool need_q = true;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mc = 0.f, lsum = 0.f;
    bool mc_set = false;

    // Vᵀ operand reads (as in the prefill kernel)
    const int vg = lane >> 4, vm = lane & 15;
    const int vrow = (vg >> 1) * 8 + (vm >> 2);
    const int vfv = v_swz<D>(vrow);
    const int vc0 = 2 * (vg & 1) + ((vm & 3) >> 1);
    const int vin = (vm & 1) * 4;
    auto v_opnd = [&](int sl, int k2, int db) -> u32x4 {
        const bf16* base = reinterpret_cast<const bf16*>(vblk(sl)) + (k2 * 16 + vrow) * D +
                           (((db * 4 + vc0) ^ vfv) * 8) + vin;
        const u32x2 lo = ds_read_tr(base);
        const u32x2 hi = ds_read_tr(base + 4 * D);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    int sl = 0;
    unsigned st_hist = 0;        // bit k: partial stores issued at the end of iteration j-1-k
    for (int j = 0; j < nblk; ++j) {
        {
            const bool live = issued < nblk;
            issue(live, live && ic.i == 0, sl == 0 ? R - 1 : sl - 1);   // the slot block j-1 left
            if (live) {
                ++issued;
                issue_advance();
            }
        }
        // block j (and its item's Q) has landed: allow for the loads of the R-1
        // younger blocks and for the partial stores issued since block j's loads
        {
            const int k = __builtin_popcount(st_hist);
            if (k == 0) wait_vmem_le<NWAIT>();
            else if (k == 1) wait_vmem_le<(NWAIT + NST > 63 ? 63 : NWAIT + NST)>();
            else if (k == 2) wait_vmem_le<(NWAIT + 2 * NST > 63 ? 63 : NWAIT + 2 * NST)>();
            else wait_vmem_le<(NWAIT + 3 * NST > 63 ? 63 : NWAIT + 3 * NST)>();
        }
        const int g = cc.g, hg = cc.hg;
        const int col = hg * 32 + l32;
        const bool col_ok = col < G;
        if (need_q) {                    // first block of an item: Q from its LDS slot
            // rows past the group's heads are not in the slot: read row 0 there, then zero
            const bf16* qrow = reinterpret_cast<const bf16*>(qslot(qs)) + (col_ok ? l32 : 0) * D;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hl * 8);
                qreg[kk] = __builtin_bit_cast(bf16x8, col_ok ? v : u32x4{0u, 0u, 0u, 0u});
            }
            need_q = false;
        }
        const bf16* krow = reinterpret_cast<const bf16*>(kblk(sl)) + l32 * D;
        f32x16 S = {};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * kk + hl) ^ k_swz<D>(l32)) * 8));
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], S, 0, 0, 0);
        }
        const int nvalid = cc.t_end - (cc.s * kDecodeSplit + cc.i * CK);   // keys before the item's end
        if (nvalid < CK) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i >> 3) * 16 + hl * 8 + (i & 7) >= nvalid) S[i] = kNegInf;
        }
        if (!mc_set) {                   // reference from this item's first block here
            float m = S[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) m = fmaxf(m, S[i]);
            mc = pair_max(m) * c;
            mc_set = true;
        }
        u32x4 pw[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            float p[8];
            float cs = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[k2 * 8 + e], c, -mc));
                cs += p[e];
            }
            if (__ballot(cs > kRescaleSum)) {     // rare: raise the reference
                float m = S[k2 * 8];
#pragma unroll
                for (int e = 1; e < 8; ++e) m = fmaxf(m, S[k2 * 8 + e]);
                const float mn = fmaxf(mc, pair_max(m) * c);
                const float alpha = __builtin_amdgcn_exp2f(mc - mn);
                mc = mn;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
                cs = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[k2 * 8 + e], c, -mc));
                    cs += p[e];
                }
            }
            lsum += cs;
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[k2][e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, v_opnd(sl, k2, db)), __builtin_bit_cast(bf16x8, pw[k2]),
                    oacc[db], 0, 0, 0);
        sl = sl == R - 1 ? 0 : sl + 1;

        // end of this wavefront's part of the item: write the partial
        const bool item_end = cc.i == cc.nb - 1 || j == nblk - 1;
        st_hist = (st_hist << 1 | (item_end ? 1u : 0u)) & ((1u << (R - 1)) - 1u);
        if (item_end) {
            const float Lsum = pair_sum(lsum);
            // the group's (split, part) slots: head column col, slot (col*nsplit + s)*2 + part
            const int ncols = min(32, G - hg * 32);
            const size_t grp = ((size_t)cc.b * H_q + g * G + hg * 32) * nsplit * 2;
            const i32x4_sgpr ors = make_rsrc(ws_o + grp * D, (uint32_t)(ncols * nsplit * 2 * D * 4));
            const i32x4_sgpr mrs = make_rsrc(ws_ml + grp * 2, (uint32_t)(ncols * nsplit * 2 * 8));
            const uint32_t slot = (uint32_t)((l32 * nsplit + cc.s) * 2 + part);
            const uint32_t oob = 0xFFFFFFF0u;            // dropped by the range check
            auto ooff = [&](int db, int g4) -> uint32_t {
                return col_ok ? (slot * D + db * 32 + g4 * 8 + hl * 4) * 4u : oob;
            };
            auto o4 = [&](int db, int g4) -> u32x4 {
                return u32x4{__float_as_uint(oacc[db][4 * g4]), __float_as_uint(oacc[db][4 * g4 + 1]),
                             __float_as_uint(oacc[db][4 * g4 + 2]), __float_as_uint(oacc[db][4 * g4 + 3])};
            };
#pragma unroll
            for (int db = 0; db < DB; ++db)
                store_x4x4(ors, ooff(db, 0), o4(db, 0), ooff(db, 1), o4(db, 1), ooff(db, 2), o4(db, 2),
                           ooff(db, 3), o4(db, 3));
            // lanes of the first half store (reference, sum); lanes of the second half the
            // empty part 1 of an item finished by the wavefront that began it
            const bool mark = part == 0 && cc.i == cc.nb - 1;
            const uint32_t moff = !col_ok ? oob : hl == 0 ? slot * 8u : mark ? (slot + 1) * 8u : oob;
            const u32x2 mv = hl == 0 ? u32x2{__float_as_uint(mc), __float_as_uint(Lsum)}
                                     : u32x2{__float_as_uint(kNegInf), 0u};
            store_x2(mrs, moff, mv);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
            lsum = 0.f;
            mc_set = false;
            need_q = true;
            part = 0;
            qs = qs == R - 1 ? 0 : qs + 1;
        }
        advance(cc, L, HG, n_hg);
    }
    wait_vmem_le<0>();     // drain the zero-range look-ahead loads before exit
}

// Merge the parts of every split of (b, query head) and normalise: one
// wavefront per (b, query head), lane l holding elements l*E .. l*E+E-1 of the
// output row.  The (reference, sum) of the parts (lane k: part k) and the O rows
// of the first 16 parts are loaded in one round, so the merge costs one memory
// latency for caches up to 8 splits; parts beyond are merged 16 at a time with
// a running reference.  Every (split, part) slot was written by the split
// kernel; an absent part 1 carries reference -inf and weight sum 0, and its O
// slot (never written) is read but not used.
template <int D>
__global__ __launch_bounds__(256)
void decode_stream_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                           const int32_t* __restrict__ lens, bf16* __restrict__ o,
                           float* __restrict__ lse, int H_q, int T_max, int nsplit, int n_bh) {
    constexpr int E = D / 64;
    constexpr int PG = 16;                       // parts per load round
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bh >= n_bh) return;
    const int b = bh / H_q;
    const int len = seq_len(lens, b, T_max);
    const int np = (len + kDecodeSplit - 1) / kDecodeSplit * 2;    // (split, part) slots
    const size_t base = (size_t)bh * nsplit * 2;
    const float* orow_ws = ws_o + base * D + lane * E;
    float M = kNegInf, lsum = 0.f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int k0 = 0; k0 < np; k0 += PG) {
        // one round: (m, l) of parts k0 .. k0+PG-1 in lanes 0..PG-1, and their O elements
        const int k = k0 + lane;
        const bool mine = lane < PG && k < np;
        const float m = mine ? ws_ml[(base + k) * 2] : kNegInf;
        const float l = mine ? ws_ml[(base + k) * 2 + 1] : 0.f;
        float ov[PG][E];
#pragma unroll
        for (int i = 0; i < PG; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) ov[i][e] = k0 + i < np ? orow_ws[(size_t)(k0 + i) * D + e] : 0.f;
        float mg = m;
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) mg = fmaxf(mg, __shfl_xor(mg, sh));
        mg = __shfl(mg, 0);
        const float Mn = fmaxf(M, mg);
        if (Mn == kNegInf) continue;             // nothing present yet
        const float alpha = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        M = Mn;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= alpha;
        lsum *= alpha;
        const float w = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - M);
        float lw = w * l;
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) lw += __shfl_xor(lw, sh);
        lsum += __shfl(lw, 0);
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            const float wi = __shfl(w, i);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = wi != 0.f ? __builtin_fmaf(ov[i][e], wi, acc[e]) : acc[e];
        }
    }
    bf16* orow = o + (size_t)bh * D + lane * E;
    if (M == kNegInf) {                          // no cached token
#pragma unroll
        for (int e = 0; e < E; ++e) orow[e] = (bf16)0.f;
        if (lse && lane == 0) lse[bh] = kNegInf;
        return;
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = (bf16)(acc[e] * inv);
    if (lse && lane == 0) lse[bh] = (M + __log2f(lsum)) * kLn2;
}

// Wavefronts the split kernel runs at once (one round of the whole GPU) for
// a given dynamic LDS size; the last query is cached.
template <int D, bool PAGED>
int resident_waves(int lds_bytes) {
    static int cached_lds = -1, cached = 0;
    if (lds_bytes == cached_lds) return cached;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_stream_kernel<D, PAGED>, 64, lds_bytes) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return 256;
    cached = cus * per_cu;
    cached_lds = lds_bytes;
    return cached;
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a) {
    // the largest dynamic LDS any call uses: ring + R full 32-head Q slots
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)decode_stream_kernel<D, PAGED>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            Geo<D>::RING + Geo<D>::R * q_slot_bytes(32, D));
    if (attr != hipSuccess) return attr;
    const int G = a.H_q / a.H_kv;
    const int n_hg = (G + 31) / 32;
    const int nsplit = decode_nsplit(a.T_max);
    const int qb = q_slot_bytes(G, D);
    const int lds = Geo<D>::RING + Geo<D>::R * qb;
    const int nwaves = resident_waves<D, PAGED>(lds);
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = ws_o + (size_t)a.B * a.H_q * nsplit * 2 * D;
    const int lps = PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
    hipLaunchKernelGGL((decode_stream_kernel<D, PAGED>), dim3(nwaves), dim3(64), lds, (hipStream_t)a.stream,
                       (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens, ws_o, ws_ml,
                       a.B, a.H_q, a.H_kv, a.T_max, G, n_hg, nsplit, nwaves, qb, a.scale * kLog2e,
                       a.block_table, lps, a.max_pages, a.num_pages);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_bh = a.B * a.H_q;
    hipLaunchKernelGGL((decode_stream_combine<D>), dim3((n_bh + 3) / 4), dim3(256), 0, (hipStream_t)a.stream,
                       ws_o, ws_ml, a.lens, (bf16*)a.o, a.lse, a.H_q, a.T_max, nsplit, n_bh);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a) {
    if (a.block_table) return a.D == 64 ? launch<64, true>(a) : launch<128, true>(a);
    return a.D == 64 ? launch<64, false>(a) : launch<128, false>(a);
}

}  // namespace mattn
