// Shared machinery of the single-token decode kernels (bf16 and FP8 caches):
// the block order of the work split, cursors over it, the lengths, buffer
// descriptors for the load builtins, and the combine kernel.
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
#pragma once

#include <atomic>

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

// Q slot bytes: the group's heads (at most 32) rounded up to whole 1 KiB loads.
inline int q_slot_bytes(int G, int D) { return (min(G, 32) * D * 2 + 1023) / 1024 * 1024; }

__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int T_max) {
    return min(max(lens[b], 0), T_max);
}

// Partials of items that end inside a wavefront's range are held until the range ends and
// written then: O in an LDS stash slot, (reference, sum) and where they go in registers.
// The same partial stores issued while the wavefront still streams its range cost ~7% of
// the decode's time (measured against a timing copy without them).  A wavefront holds at
// most kStashSlots, as many as the LDS left over at the kernel's occupancy allows (the host
// picks the count, possibly 0); items past that store at once.
constexpr int kStashSlots = 2;
// Bytes of one stash slot: the O rows of a group's columns (at most 32), D floats each.
__host__ __device__ inline int stash_slot_bytes(int G, int D) { return min(G, 32) * D * 4; }

// A held partial: the workspace slot of its column 0 (column c at slot0 + c·2·nsplit), its
// column count, whether its empty part 1 must be marked, and this lane's (reference, sum).
// All four live in vector registers: the stream loop has no scalar registers to spare.
struct Held {
    uint32_t slot0, nc_mark;     // nc_mark = column count | mark << 8
    float m, l;
};
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
    return v;
}
__device__ __forceinline__ Held make_held(uint32_t slot0, int ncols, bool mark, float m, float l) {
    return Held{in_vgpr(slot0), in_vgpr((uint32_t)ncols | (mark ? 256u : 0u)), m, l};
}

// This lane's column of an item's O (the MFMA accumulator layout, times vs when SCALE) into a
// stash slot: column c's D floats at float offset c·D.
template <int D, bool SCALE>
__device__ __forceinline__ void stash_o(unsigned char* slot, const f32x16* o, float vs, bool col_ok, int l32,
                                        int hl) {
    if (!col_ok) return;
    float* row = reinterpret_cast<float*>(slot) + l32 * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 v{o[db][4 * g4], o[db][4 * g4 + 1], o[db][4 * g4 + 2], o[db][4 * g4 + 3]};
            if constexpr (SCALE) v = f32x4{v[0] * vs, v[1] * vs, v[2] * vs, v[3] * vs};
            *reinterpret_cast<f32x4*>(row + db * 32 + g4 * 8 + hl * 4) = v;
        }
}

// A held partial to the workspace: O rows from its stash slot (consecutive lanes, consecutive
// 16 bytes of a row), (reference, sum) from the first half's lanes of its columns, the empty
// marker of part 1 from the second half's.
template <int D>
__device__ __forceinline__ void stash_flush(const unsigned char* slot, const Held& h, int nsplit,
                                            float* __restrict__ ws_o, float* __restrict__ ws_ml) {
    constexpr int QPC = D / 4;       // 16-byte chunks per column
    const int lane = threadIdx.x & 63, l32 = lane & 31;
    const size_t cstep = (size_t)nsplit * 2;
    const int ncols = (int)(h.nc_mark & 255u);
    for (int c = lane; c < ncols * QPC; c += 64) {
        const int col = c / QPC, qc = c - col * QPC;
        const f32x4 v = *reinterpret_cast<const f32x4*>(slot + (size_t)(col * D + qc * 4) * 4);
        *reinterpret_cast<f32x4*>(ws_o + (h.slot0 + col * cstep) * D + qc * 4) = v;
    }
    if (l32 < ncols) {
        if (lane < 32) *reinterpret_cast<f32x2*>(ws_ml + (h.slot0 + l32 * cstep) * 2) = f32x2{h.m, h.l};
        else if (h.nc_mark & 256u)
            *reinterpret_cast<f32x2*>(ws_ml + (h.slot0 + 1 + l32 * cstep) * 2) = f32x2{kNegInf, 0.f};
    }
}

// Workgroups of one wavefront of KERNEL resident per CU at a dynamic LDS size (0 if the query
// fails), cached per kernel and size: each entry packs (size + 1, count) into one word, and a
// new size takes the first free entry (once all eight are taken, the one its size picks).
template <auto KERNEL>
int blocks_per_cu(int lds_bytes) {
    static std::atomic<uint64_t> tab[8];
    const uint64_t key = (uint64_t)(uint32_t)(lds_bytes + 1) << 32;
    for (auto& e : tab) {
        const uint64_t v = e.load(std::memory_order_relaxed);
        if ((v & ~0xffffffffull) == key) return (int)(uint32_t)v;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, 64, lds_bytes) != hipSuccess || per_cu < 0)
        return 0;
    const uint64_t entry = key | (uint32_t)per_cu;
    for (auto& e : tab) {
        uint64_t empty = 0;
        if (e.compare_exchange_strong(empty, entry, std::memory_order_relaxed)) return per_cu;
    }
    tab[((uint32_t)lds_bytes >> 10) % 8].store(entry, std::memory_order_relaxed);
    return per_cu;
}
// Compute units of the current device, read once per device.
inline int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
// Stash slots for a launch of KERNEL: the most (up to kStashSlots, within max_dyn bytes of
// dynamic LDS) that leave its resident workgroups per CU at per_cu.
template <auto KERNEL>
int stash_slots(int lds0, int slot_bytes, int max_dyn, int per_cu) {
    for (int n = kStashSlots; n >= 1; --n) {
        const int lds = lds0 + n * slot_bytes;
        if (lds <= max_dyn && blocks_per_cu<KERNEL>(lds) == per_cu) return n;
    }
    return 0;
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

// Clamped sequence lengths as seen by one wavefront: with at most 64
// sequences lane b holds len_b in a register (read back with readlane, no
// memory round trip); beyond that they are read from memory.
struct Lens {
    const int32_t* p;
    int B, T_max, reg;
    __device__ int get(int b) const {
        if (B <= 64) return __builtin_amdgcn_readlane(reg, b);
        int v, u;              // scalar load: no wait on the wavefront's vector loads
        sload2(p, __builtin_amdgcn_readfirstlane((uint32_t)b * 4u), __builtin_amdgcn_readfirstlane((uint32_t)b * 4u), v, u);
        return min(max(v, 0), T_max);
    }
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
// Next block in the global order.  LIKELY marks staying inside the item as the expected case,
// which lays the item change out off the common path (the INT8 decode measured 85 against
// 88 us with it; the bf16 and E4M3 decodes neutral or slower, so they keep the default).
template <bool LIKELY = false>
__device__ __forceinline__ void advance(Cursor& c, const Lens& L, int HG, int n_hg) {
    if constexpr (LIKELY) {
        if (__builtin_expect(++c.i < c.nb, 1)) return;
    } else {
        if (++c.i < c.nb) return;
    }
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

// One 1 KiB buffer->LDS load: lane i's 16 bytes at byte offset voff of the buffer land at
// lds_chunk + 16 i.  Asm statements, volatile, so they keep their order among themselves; the
// last load of a group also carries a memory clobber (dma16), so no load the compiler issues
// later in program order is moved in front of the group, and the slot waits (asm with a memory
// clobber too) keep every load of the program order before them: the loads between a group
// and a counted vmcnt wait are exactly those of the program order, which the decode kernels'
// slot waits count.
// last: the group's final load, which carries the memory clobber; the earlier ones of the group
// (last = false) are ordered by it and by their own volatility.  NT: the streaming cache policy
// (the KV cache, read once per call); Q slots keep the default.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(const i32x4_sgpr& r, const unsigned char* lds_chunk, uint32_t voff,
                                          bool last = true) {
    const uint32_t a =
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)lds_chunk);
    if constexpr (NT) {
        if (last) dma16_nt(r, a, voff);
        else dma16_nb_nt(r, a, voff);
    } else {
        if (last) dma16(r, a, voff, 0u);
        else dma16_nb(r, a, voff);
    }
}

// The transposing LDS reads of one V block's operands (2 k-steps x DB row blocks x
// lo/hi), written as one asm statement ending in lgkmcnt(0).  They are asm so
// that the compiler inserts no wait of its own for the block's LDS loads (it
// cannot tell the ring slots apart for these reads and would wait for the most
// recent one); the caller waits for the slot explicitly.  addr[db]: this lane's
// LDS byte address of row block db for k-step 0, lo half.
template <int D>
__device__ __forceinline__ void v_operands(const uint32_t* addr, u32x4 (&va)[2][D / 32]) {
    constexpr int K2 = 16 * D * 2;     // bytes between the k-steps (16 rows)
    constexpr int HI = 4 * D * 2;      // bytes between the lo and hi 4-row groups
    u32x2 r[2][D / 32][2];
    if constexpr (D == 128) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %16 offset:%20\n\t"
            "ds_read_b64_tr_b16 %2, %17\n\tds_read_b64_tr_b16 %3, %17 offset:%20\n\t"
            "ds_read_b64_tr_b16 %4, %18\n\tds_read_b64_tr_b16 %5, %18 offset:%20\n\t"
            "ds_read_b64_tr_b16 %6, %19\n\tds_read_b64_tr_b16 %7, %19 offset:%20\n\t"
            "ds_read_b64_tr_b16 %8, %16 offset:%21\n\tds_read_b64_tr_b16 %9, %16 offset:%22\n\t"
            "ds_read_b64_tr_b16 %10, %17 offset:%21\n\tds_read_b64_tr_b16 %11, %17 offset:%22\n\t"
            "ds_read_b64_tr_b16 %12, %18 offset:%21\n\tds_read_b64_tr_b16 %13, %18 offset:%22\n\t"
            "ds_read_b64_tr_b16 %14, %19 offset:%21\n\tds_read_b64_tr_b16 %15, %19 offset:%22\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0][0][0]), "=&v"(r[0][0][1]), "=&v"(r[0][1][0]), "=&v"(r[0][1][1]),
              "=&v"(r[0][2][0]), "=&v"(r[0][2][1]), "=&v"(r[0][3][0]), "=&v"(r[0][3][1]),
              "=&v"(r[1][0][0]), "=&v"(r[1][0][1]), "=&v"(r[1][1][0]), "=&v"(r[1][1][1]),
              "=&v"(r[1][2][0]), "=&v"(r[1][2][1]), "=&v"(r[1][3][0]), "=&v"(r[1][3][1])
            : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "n"(HI), "n"(K2), "n"(K2 + HI)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
            "ds_read_b64_tr_b16 %2, %9\n\tds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:%11\n\tds_read_b64_tr_b16 %5, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %6, %9 offset:%11\n\tds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0][0][0]), "=&v"(r[0][0][1]), "=&v"(r[0][1][0]), "=&v"(r[0][1][1]),
              "=&v"(r[1][0][0]), "=&v"(r[1][0][1]), "=&v"(r[1][1][0]), "=&v"(r[1][1][1])
            : "v"(addr[0]), "v"(addr[1]), "n"(HI), "n"(K2), "n"(K2 + HI)
            : "memory");
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            va[k2][db] = u32x4{r[k2][db][0][0], r[k2][db][0][1], r[k2][db][1][0], r[k2][db][1][1]};
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
    const size_t base = (size_t)bh * nsplit * 2;
    const float* orow_ws = ws_o + base * D + lane * E;
    // The first round's loads do not wait for the length: slots 0 .. min(PG, 2·nsplit) - 1 are
    // this (b, head)'s own, so they are loaded together with it and the slots past the
    // sequence's parts are masked once it has arrived (a slot never written is loaded, not used).
    const int cap0 = min(PG, 2 * nsplit);
    float m0 = kNegInf, l0 = 0.f, ov0[PG][E];
    if (lane < cap0) {
        m0 = ws_ml[(base + lane) * 2];
        l0 = ws_ml[(base + lane) * 2 + 1];
    }
#pragma unroll
    for (int i = 0; i < PG; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) ov0[i][e] = i < cap0 ? orow_ws[(size_t)i * D + e] : 0.f;
    const int len = seq_len(lens, b, T_max);
    const int np = (len + kDecodeSplit - 1) / kDecodeSplit * 2;    // (split, part) slots
    float M = kNegInf, lsum = 0.f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    // merge parts k0 .. k0+PG-1: (m, l) of part k0 + lane in lanes 0..PG-1, ov[i] = O elements of part k0 + i
    auto merge_round = [&](int k0, float m, float l, const float (&ov)[PG][E]) {
        if (!(lane < PG && k0 + lane < np)) {
            m = kNegInf;
            l = 0.f;
        }
        float mg = m;
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) mg = fmaxf(mg, __shfl_xor(mg, sh));
        mg = __shfl(mg, 0);
        const float Mn = fmaxf(M, mg);
        if (Mn == kNegInf) return;               // nothing present yet
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
    };
    if (np > 0) merge_round(0, m0, l0, ov0);
    for (int k0 = PG; k0 < np; k0 += PG) {
        const int k = k0 + lane;
        const bool mine = lane < PG && k < np;
        const float m = mine ? ws_ml[(base + k) * 2] : kNegInf;
        const float l = mine ? ws_ml[(base + k) * 2 + 1] : 0.f;
        float ov[PG][E];
#pragma unroll
        for (int i = 0; i < PG; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) ov[i][e] = k0 + i < np ? orow_ws[(size_t)(k0 + i) * D + e] : 0.f;
        merge_round(k0, m, l, ov);
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

}  // namespace
}  // namespace mattn
