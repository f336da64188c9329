// Single-token decode against an 8-bit key/value cache: FP8 (E4M3) codes, or
// symmetric INT8 codes when INT8.
//
// KV-cache quantisation stores each cached element in fewer bytes plus scale
// metadata, and the attention kernel dequantises on the fly (blog.ruahverce.com,
// LLM inference memory accounting 2/10, section
// "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").
// Here the cache holds OCP E4M3 codes (or INT8 integers) with one float32 scale
// per (sequence, KV head) for K and one for V: a cached element is code value x
// scale.  Every E4M3 value and every integer in [-128, 127] is exact in bf16, so
// codes are converted to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1, or a
// byte-to-float convert and a pack) and the bf16 decode's matrix-core block runs
// unchanged; the scales
// act outside the products: the K scale multiplies the score multiplier, the V
// scale the partial O of an item.  The work split, cursors and combine are
// those of the bf16 decode (decode_common.cuh); the cache bytes per token are
// half of bf16's.
//
// Look-ahead, all in registers: K of a block is loaded in the A-operand layout
// of K·Qᵀ (8 codes per lane and k-step: key perm(l % 32), d = 16·kk +
// 8·(l / 32)) LK blocks ahead; V rows (16 codes per lane and 1 KiB load) RV - 1
// blocks ahead.  At its block, V is converted and written to a bf16 LDS tile in
// the bf16 kernel's swizzled layout and read back with the transposing LDS
// read.  Every global load is a compiler builtin, so the compiler derives the
// waits; each item's Q (bf16) reaches an LDS slot by buffer->LDS loads.  V rows
// (whole lines, read once) use the non-temporal cache policy; the K operand loads,
// which read each line over several k-steps, keep the default.  The E4M3 instances hold
// the partials of items that end inside a range until it ends, as the bf16 kernel does.
#include "decode_common.cuh"

namespace mattn {
namespace {

template <int D, bool INT8> struct Geo8 {
    static constexpr int RB = D;                   // bytes per cache row (one byte per element)
    static constexpr int BLK = CK * RB;            // bytes of one K (or V) block
    static constexpr int NV = BLK / 1024;          // 1 KiB V loads per block (16 bytes per lane)
    // V register ring (look-ahead RV - 1 blocks) and K look-ahead in blocks.  E4M3 at D = 128:
    // rings of 3 and 2 blocks, so a wave fits 256 registers and two waves share a SIMD (one
    // hides the other's conversion and softmax work; the bytes in flight per SIMD stay about
    // those of one deep-ring wave).  INT8 at D = 128: its conversion needs more temporaries,
    // which the small rings would spill, so one wave per SIMD with rings of 7 and 4 (8 would
    // push the excess past the accumulation registers into memory).  D = 64: rings of 8 and 4.
    static constexpr bool TWO_WAVES = D == 128 && !INT8;
    static constexpr int RV = D == 128 ? (INT8 ? 7 : 3) : 8;
    static constexpr int LK = TWO_WAVES ? 2 : 4;
    static constexpr int WAVES_MIN = TWO_WAVES ? 2 : 1, WAVES_MAX = D == 128 ? WAVES_MIN : 8;
    static constexpr int QCH = 32 * D * 2 / 1024;  // 1 KiB loads of a full 32-head bf16 Q slot
};

__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}


// At D = 128 the INT8 instance's K and V register rings alone fill 256 registers: one
// wavefront per SIMD, with the accumulation registers as well (no spills).  The E4M3 instance's
// smaller rings fit 256 registers in all, for two wavefronts per SIMD (the contiguous one
// keeps two 8-byte values in scratch memory, stored before the block loop and reloaded twice
// per block in it; measured faster than one wavefront per SIMD all the same).
// PAGED: kc / vc are page pools [num_pages, H_kv, 2^lps, D] of codes; token t of sequence b is
// row t mod 2^lps of page bt[b * max_pages + (t >> lps)] (entries clamped to [0, num_pages)),
// T_max = max_pages << lps.  V of a 32-token block is loaded as two 16-token halves, each
// through the buffer range of its page; K by per-lane global loads from the page of each key.
template <int D, bool INT8, bool PAGED>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(Geo8<D, INT8>::WAVES_MIN, Geo8<D, INT8>::WAVES_MAX)))
void decode_q8_kernel(const bf16* __restrict__ q, const uint8_t* __restrict__ kc,
                       const uint8_t* __restrict__ vc, const float* __restrict__ kscale,
                       const float* __restrict__ vscale, const int32_t* __restrict__ lens,
                       float* __restrict__ ws_o, float* __restrict__ ws_ml,
                       int B, int H_q, int H_kv, int T_max, int G, int n_hg, int nsplit,
                       int nwaves, int qbn, float c, const int32_t* __restrict__ bt, int max_pages,
                       int num_pages, int lps) {
    using Gm = Geo8<D, INT8>;
    constexpr int RB = Gm::RB, NV = Gm::NV, QCH = Gm::QCH, RV = Gm::RV, LK = Gm::LK;
    constexpr int KSTEPS = D / 16;     // MFMA k-steps of K·Qᵀ
    constexpr int DB = D / 32;         // 32-row blocks of Oᵀ
    constexpr int RB16 = D * 2;        // bytes per row of the bf16 V tile
    static_assert(LK >= 1 && LK < RV, "ring geometry");
    __shared__ __attribute__((aligned(16))) unsigned char vtile[CK * RB16];
    // Partials of items that end inside the range are held until it ends (E4M3 only: the INT8
    // kernel measured slower with the stash, ~89 against ~87 us on the decode workload with
    // the caches flushed, its loop being bound by the code conversions rather than the stores).
    // qbn: the Q slot bytes (a multiple of 1 KiB), plus the stash slots in its low bits; one
    // argument, so the INT8 instances keep the argument list they had without a stash (with
    // two more arguments their register allocation, and time, moved).
    constexpr bool STASH = !INT8;
    const int qb = STASH ? qbn & ~1023 : qbn;
    const int ns = STASH ? qbn & 1023 : 0;
    const int sob = stash_slot_bytes(G, D);
    extern __shared__ __attribute__((aligned(16))) unsigned char qlds[];   // RV Q slots of qb bytes
    auto qslot = [&](int s) -> unsigned char* { return qlds + s * qb; };
    unsigned char* const stash = qlds + RV * qb;    // ns slots of sob bytes after the Q slots

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

    // K: byte offsets of the operand layout within a block.  V: load i of a lane holds
    // block bytes i*1024 + 16*lane .. +15 = row r, codes of columns col .. col+15, i.e.
    // bf16 chunks g0 = col/8 and g0+1 of row r, which sit at LDS chunk positions
    // g0 ^ v_swz(r) and the next one (v_swz is even).
    uint32_t k_off[KSTEPS], v_off[NV], v_dst[NV];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) k_off[kk] = (uint32_t)(swap_bits23(l32) * RB + kk * 16 + hl * 8);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int o = i * 1024 + lane * 16;
        const int r = o / RB, g0 = (o % RB) / 8;
        v_off[i] = (uint32_t)o;
        v_dst[i] = (uint32_t)(r * RB16 + (g0 ^ v_swz<D>(r)) * 16);
    }
    const __amdgpu_buffer_rsrc_t zrs = brsrc(kc, 0u);
    constexpr int HNV = NV / 2;           // V loads per 16-row half of a block
    static_assert(HNV * 2 == NV && HNV * 1024 == 16 * RB, "a V load lies inside one half");

    // Paged: the V buffer ranges of the two 16-token halves of block (cursor) x, each inside
    // one page (pages are powers of two >= 16 tokens, blocks start at multiples of 32), and
    // the row offset of each half within its range.
    auto page_halves = [&](const Cursor& x, __amdgpu_buffer_rsrc_t* vh, uint32_t* roff) {
        const int t0 = x.s * kDecodeSplit + x.i * CK;
        const int last = x.t_end - 1;
        const int pi0 = t0 >> lps, pi1 = min(t0 + 16, last) >> lps;
        const uint32_t rowb = (uint32_t)x.b * (uint32_t)max_pages * 4u;
        int e0, e1;
        sload2(bt, __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi0 * 4u),
               __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi1 * 4u), e0, e1);
        const int pe[2] = {e0, e1}, pidx[2] = {pi0, pi1};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            vh[h] = zrs;
            roff[h] = 0u;
            const int th = t0 + 16 * h;
            if (th < x.t_end) {
                const int page = min(max(pe[h], 0), num_pages - 1);
                const int pstart = pidx[h] << lps;
                const int rows = min(1 << lps, x.t_end - pstart);
                const size_t head = (((size_t)page * H_kv + x.g) << lps) * D;
                vh[h] = brsrc(vc + head, (uint32_t)rows * RB);
                roff[h] = (uint32_t)(th - pstart) * RB;
            }
        }
    };

    // ---- issue side: V (+ Q) cursor RV-1 blocks ahead of the compute, K cursor LK ahead
    Cursor icv = cursor_at(L, HG, n_hg, b0, a0 - before);
    Cursor ick = icv;
    int nv = 0, nk = 0, qs_issue = 0;
    auto item_rsrc = [&](const Cursor& x, const uint8_t* base) {
        const size_t head = ((size_t)x.b * H_kv + x.g) * (size_t)T_max * D;
        return brsrc(base + head, (uint32_t)x.t_end * RB);
    };
    __amdgpu_buffer_rsrc_t vrs = zrs, krs = zrs;
    if constexpr (!PAGED) {
        vrs = item_rsrc(icv, vc);
        krs = item_rsrc(ick, kc);
    }
    u32x4 vr[RV][NV];
    u32x2 kr[RV][KSTEPS];
    auto issue_v = [&](int s) {
        const bool live = nv < nblk;
        if constexpr (PAGED) {
            __amdgpu_buffer_rsrc_t vh[2] = {zrs, zrs};
            uint32_t roff[2] = {0u, 0u};
            if (live) page_halves(icv, vh, roff);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                vr[s][i] = bload16_nt(vh[i / HNV], roff[i / HNV] + v_off[i] - (uint32_t)(i / HNV) * 16u * RB);
        } else {
            const uint32_t row0 = (uint32_t)(icv.s * kDecodeSplit + icv.i * CK) * RB;
#pragma unroll
            for (int i = 0; i < NV; ++i) vr[s][i] = bload16_nt(live ? vrs : zrs, row0 + v_off[i]);
        }
        if (!live) return;
        if (icv.i == 0 || nv == 0) {     // the item's Q (also for a range that starts inside it)
            const int ncols = min(32, G - icv.hg * 32);
            const i32x4_sgpr qrs =
                make_rsrc(q + ((size_t)icv.b * H_q + icv.g * G + icv.hg * 32) * D, (uint32_t)(ncols * RB16));
#pragma unroll
            for (int ch = 0; ch < QCH; ++ch)
                if (ch * 1024 < ncols * RB16)
                    lds_dma16(qrs, qslot(qs_issue) + ch * 1024, (uint32_t)(ch * 1024 + lane * 16),
                              (ch + 1) * 1024 >= ncols * RB16);
        }
        ++nv;
        advance<INT8>(icv, L, HG, n_hg);
        if (icv.i == 0) {
            qs_issue = qs_issue == RV - 1 ? 0 : qs_issue + 1;
            if constexpr (!PAGED) vrs = item_rsrc(icv, vc);
        }
    };
    auto issue_k = [&](int s) {
        const bool live = nk < nblk;
        if constexpr (PAGED) {
            // one global load per k-step from a per-lane address: lane l reads key perm(l % 32)
            // of the block from the page of its half; a key past the item's end (its score is
            // masked) and a block past the wavefront's range read row 0 of a valid page
            const uint8_t* src = kc;
            if (live) {
                const int t0 = ick.s * kDecodeSplit + ick.i * CK;
                const int last = ick.t_end - 1;
                const int pi0 = t0 >> lps, pi1 = min(t0 + 16, last) >> lps;
                const uint32_t rowb = (uint32_t)ick.b * (uint32_t)max_pages * 4u;
                int e0, e1;
                sload2(bt, __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi0 * 4u),
                       __builtin_amdgcn_readfirstlane(rowb + (uint32_t)pi1 * 4u), e0, e1);
                const int key = swap_bits23(l32);
                const int t = t0 + key <= last ? t0 + key : t0;       // t0 <= last: a live block
                const bool h1 = t - t0 >= 16;
                const int page = min(max(h1 ? e1 : e0, 0), num_pages - 1);
                const int pstart = (h1 ? pi1 : pi0) << lps;
                src = kc + ((((size_t)page * H_kv + ick.g) << lps) + (size_t)(t - pstart)) * D;
            }
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                kr[s][kk] = *reinterpret_cast<const u32x2*>(src + kk * 16 + hl * 8);
        } else {
            const uint32_t row0 = (uint32_t)(ick.s * kDecodeSplit + ick.i * CK) * RB;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) kr[s][kk] = bload8(live ? krs : zrs, row0 + k_off[kk]);
        }
        if (!live) return;
        ++nk;
        advance<INT8>(ick, L, HG, n_hg);
        if constexpr (!PAGED)
            if (ick.i == 0) krs = item_rsrc(ick, kc);
    };
#pragma unroll
    for (int s = 0; s < RV - 1; ++s) issue_v(s);
#pragma unroll
    for (int s = 0; s < LK; ++s) issue_k(s);

    // ---- compute side
    Cursor cc = cursor_at(L, HG, n_hg, b0, a0 - before);
    int part = cc.i == 0 ? 0 : 1;
    int qs = 0;
    bf16x8 qreg[KSTEPS];
    bool need_q = true;
    float ci = c, vsc = 1.f;           // this item's score multiplier and V scale
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mc = 0.f, lsum = 0.f;
    bool mc_set = false;
    Held held0{}, held1{};        // the held partials
    int nheld = 0;

    const int vg = lane >> 4, vm = lane & 15;
    const int vrow = (vg >> 1) * 8 + (vm >> 2);
    const int vfv = v_swz<D>(vrow);
    const int vc0 = 2 * (vg & 1) + ((vm & 3) >> 1);
    const int vin = (vm & 1) * 4;
    uint32_t vaddr[DB];                // this lane's LDS byte address of row block db in the tile
    {
        const uint32_t tb = (uint32_t)reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) unsigned char*)vtile);
#pragma unroll
        for (int db = 0; db < DB; ++db)
            vaddr[db] = tb + (uint32_t)((vrow * D + (((db * 4 + vc0) ^ vfv) * 8) + vin) * 2);
    }

    // The Q slot wait.  Loop iteration i issues, in this program order: V of block
    // i + RV - 1 (NV register loads, then the QCH buffer->LDS loads of the item's Q if that
    // block starts an item), K of block i + LK (KSTEPS loads), then computes block i.  The Q
    // loads are asm statements with a memory clobber and so is the wait: the compiler moves
    // no load across them, and the count below is a property of this source.  Between an
    // item's Q loads and the wait in front of its first block come at least the V loads of
    // the RV - 1 blocks after it and the K loads of LK + 1 blocks (the fewest at the first
    // block of a range): Q_LOADS_AFTER.  Loads return in issue order, so at most that many
    // outstanding (capped at the counter's 63, which only waits longer) means Q has landed.
    constexpr int Q_LOADS_AFTER = (RV - 1) * NV + (LK + 1) * KSTEPS;
    static_assert(LK + 1 <= RV && NV == Gm::BLK / 1024 && KSTEPS == D / 16, "the counted geometry");
    constexpr int NQ = Q_LOADS_AFTER < 63 ? Q_LOADS_AFTER : 63;

    auto compute = [&](int j, int s) {
        const int g = cc.g, hg = cc.hg;
        const int col = hg * 32 + l32;
        const bool col_ok = col < G;
        if (need_q) {                    // first block of an item: Q and the scales
            wait_vmem_le<NQ>();          // the Q slot's buffer->LDS loads have landed
            const bf16* qrow = reinterpret_cast<const bf16*>(qslot(qs)) + (col_ok ? l32 : 0) * D;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hl * 8);
                qreg[kk] = __builtin_bit_cast(bf16x8, col_ok ? v : u32x4{0u, 0u, 0u, 0u});
            }
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(cc.b * H_kv + g) * 4u);
            int kb, vb;
            sload2(reinterpret_cast<const int32_t*>(kscale), so, so, kb, vb);
            ci = c * __int_as_float(kb);
            sload2(reinterpret_cast<const int32_t*>(vscale), so, so, vb, kb);
            vsc = __int_as_float(vb);
            need_q = false;
        }
        f32x16 S = {};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const u32x2 a0 = codes4_to_bf16<INT8>(kr[s][kk][0]), a1 = codes4_to_bf16<INT8>(kr[s][kk][1]);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]}),
                                                        qreg[kk], S, 0, 0, 0);
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
            mc = pair_max(m) * ci;
            mc_set = true;
        }
        // Weights of the block's 16 keys in this lane.  If their sum passes 2^8 (rare), the
        // reference is raised to the block's row max where that is higher, O and l are scaled
        // by 2^(old - new) and all 16 weights are redone, before any of them is packed: the
        // P operand of both k-steps then uses one reference, the one O and l are kept in.
        float p[16];
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], ci, -mc));
            cs += p[e];
        }
        if (__ballot(cs > kRescaleSum)) {
            float m = S[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) m = fmaxf(m, S[e]);
            const float mn = fmaxf(mc, pair_max(m) * ci);
            const float alpha = __builtin_amdgcn_exp2f(mc - mn);
            mc = mn;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            cs = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], ci, -mc));
                cs += p[e];
            }
        }
        lsum += cs;
        u32x4 pw[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[k2][e] = pack_bf16x2(p[k2 * 8 + 2 * e], p[k2 * 8 + 2 * e + 1]);
        // V of this block: codes -> bf16 tile -> transposing operand reads
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32x4 v = vr[s][i];
            const u32x2 c0 = codes4_to_bf16<INT8>(v[0]), c1 = codes4_to_bf16<INT8>(v[1]);
            const u32x2 c2 = codes4_to_bf16<INT8>(v[2]), c3 = codes4_to_bf16<INT8>(v[3]);
            *reinterpret_cast<u32x4*>(vtile + v_dst[i]) = u32x4{c0[0], c0[1], c1[0], c1[1]};
            *reinterpret_cast<u32x4*>(vtile + v_dst[i] + 16) = u32x4{c2[0], c2[1], c3[0], c3[1]};
        }
        u32x4 va[2][DB];
        v_operands<D>(vaddr, va);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va[k2][db]), __builtin_bit_cast(bf16x8, pw[k2]),
                    oacc[db], 0, 0, 0);

        // end of this wavefront's part of the item: write the partial (O times the V scale)
        if (cc.i == cc.nb - 1 || j == nblk - 1) {
            const float Lsum = pair_sum(lsum);
            if (STASH && j < nblk - 1 && nheld < ns) {
                // the item ends inside the range: hold its partial until the range ends
                stash_o<D, true>(stash + nheld * sob, oacc, vsc, col_ok, l32, hl);
                const Held h = make_held((uint32_t)(((cc.b * H_q + g * G + hg * 32) * nsplit + cc.s) * 2 + part),
                                         min(32, G - hg * 32), part == 0, mc, Lsum);
                if (nheld == 0) held0 = h;
                else held1 = h;
                ++nheld;
            } else if (col_ok) {
                const size_t slot = ((size_t)(cc.b * H_q + g * G + col) * nsplit + cc.s) * 2 + part;
                float* orow = ws_o + slot * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        *reinterpret_cast<f32x4*>(orow + db * 32 + g4 * 8 + hl * 4) =
                            f32x4{oacc[db][4 * g4] * vsc, oacc[db][4 * g4 + 1] * vsc,
                                  oacc[db][4 * g4 + 2] * vsc, oacc[db][4 * g4 + 3] * vsc};
                if (hl == 0) *reinterpret_cast<f32x2*>(ws_ml + slot * 2) = f32x2{mc, Lsum};
                else if (part == 0 && cc.i == cc.nb - 1)
                    *reinterpret_cast<f32x2*>(ws_ml + (slot + 1) * 2) = f32x2{kNegInf, 0.f};
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
            lsum = 0.f;
            mc_set = false;
            need_q = true;
            part = 0;
            qs = qs == RV - 1 ? 0 : qs + 1;
        }
        advance<INT8>(cc, L, HG, n_hg);
    };

    // block j sits in V slot j % RV and K slot j % RV; unrolled RV times so every slot
    // index is a constant
    for (int j0 = 0; j0 < nblk; j0 += RV) {
#pragma unroll
        for (int r = 0; r < RV; ++r) {
            // past the range the issues are zero-range loads and the compute is skipped;
            // the loop is never left mid-body (no register copies on extra exits)
            const int j = j0 + r;
            issue_v((r + RV - 1) % RV);       // block j + RV - 1, into the slot block j - 1 left
            issue_k((r + LK) % RV);           // block j + LK
            if (j < nblk) compute(j, r);
        }
    }
    wait_vmem_le<0>();     // the Q loads into LDS land before the wavefront ends
    static_assert(kStashSlots == 2, "held0, held1");
    if constexpr (STASH) {
        if (nheld > 0) stash_flush<D>(stash, held0, nsplit, ws_o, ws_ml);
        if (nheld > 1) stash_flush<D>(stash + sob, held1, nsplit, ws_o, ws_ml);
    }
}

template <int D, bool INT8, bool PAGED>
hipError_t launch8(const DecodeFp8Args& a) {
    const int G = a.H_q / a.H_kv;
    const int n_hg = (G + 31) / 32;
    const int nsplit = decode_nsplit(a.T_max);
    const int qb = q_slot_bytes(G, D);           // a multiple of 1 KiB: the stash count rides in its low bits
    const int lds0 = Geo8<D, INT8>::RV * qb;
    ATTN_CHECK(G >= 1 && G * a.H_kv == a.H_q, "query heads group onto KV heads");
    ATTN_CHECK(lds0 <= kLdsBytesPerCu, "Q slots fit a CU");
    ATTN_CHECK(nsplit >= 1 && (long long)nsplit * kDecodeSplit >= a.T_max, "splits cover the cache");
    ATTN_CHECK((size_t)a.B * a.H_q * nsplit * 2 * (D + 2) * sizeof(float) <=
                   decode_workspace_bytes(a.B, a.H_q, a.T_max, D),
               "partials and (reference, sum) pairs fit the workspace");
    ATTN_CHECK((long long)a.B * a.H_q * nsplit * 2 < (1ll << 31), "partial slot indices fit 31 bits (held partials)");
    ATTN_CHECK(PAGED || (long long)a.T_max * D < (1ll << 31), "a (sequence, KV head) fits a 32-bit range");
    ATTN_CHECK(!PAGED || (a.page_size >= 16 && (a.page_size & (a.page_size - 1)) == 0 &&
                          (long long)a.max_pages * a.page_size == a.T_max),
               "pages are powers of two of at least 16 tokens");
    // the largest dynamic LDS any call uses: RV full 32-head Q slots and the stash slots
    static const int max_dyn = Geo8<D, INT8>::RV * q_slot_bytes(32, D) + kStashSlots * stash_slot_bytes(32, D);
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)decode_q8_kernel<D, INT8, PAGED>, hipFuncAttributeMaxDynamicSharedMemorySize, max_dyn);
    if (attr != hipSuccess) return attr;
    // one round of the whole GPU: the wavefronts resident at the Q slots' LDS, and as many
    // stash slots as leave that count unchanged
    const int cus = cu_count(), per_cu = blocks_per_cu<decode_q8_kernel<D, INT8, PAGED>>(lds0);
    const int nwaves = cus > 0 && per_cu > 0 ? cus * per_cu : 256;
    const int sob = stash_slot_bytes(G, D);
    const int ns = !INT8 && per_cu > 0 ? stash_slots<decode_q8_kernel<D, INT8, PAGED>>(lds0, sob, max_dyn, per_cu) : 0;
    const int lds = lds0 + ns * sob;
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = ws_o + (size_t)a.B * a.H_q * nsplit * 2 * D;
    const int lps = PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
    hipLaunchKernelGGL((decode_q8_kernel<D, INT8, PAGED>), dim3(nwaves), dim3(64), lds, (hipStream_t)a.stream,
                       (const bf16*)a.q, (const uint8_t*)a.k_cache, (const uint8_t*)a.v_cache, a.k_scale,
                       a.v_scale, a.lens, ws_o, ws_ml, a.B, a.H_q, a.H_kv, a.T_max, G, n_hg, nsplit, nwaves, qb + ns,
                       a.scale * kLog2e, a.block_table, a.max_pages, a.num_pages, lps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_bh = a.B * a.H_q;
    hipLaunchKernelGGL((decode_stream_combine<D>), dim3((n_bh + 3) / 4), dim3(256), 0, (hipStream_t)a.stream,
                       ws_o, ws_ml, a.lens, (bf16*)a.o, a.lse, a.H_q, a.T_max, nsplit, n_bh);
    return hipGetLastError();
}

}  // namespace

template <bool PAGED>
hipError_t launch8_fmt(const DecodeFp8Args& a) {
    if (a.int8) return a.D == 64 ? launch8<64, true, PAGED>(a) : launch8<128, true, PAGED>(a);
    return a.D == 64 ? launch8<64, false, PAGED>(a) : launch8<128, false, PAGED>(a);
}

hipError_t launch_decode_fp8kv(const DecodeFp8Args& a) {
    return a.block_table ? launch8_fmt<true>(a) : launch8_fmt<false>(a);
}

}  // namespace mattn
