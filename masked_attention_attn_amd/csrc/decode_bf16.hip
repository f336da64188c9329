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
// Work split: the stream of 32-token blocks in decode_common.cuh.
//
// Per block, on the matrix cores, with the query heads as the 32 columns:
//   Sᵀ[key, head] = K·Qᵀ   (A = 32 K rows from registers, B = Q from registers)
//   Oᵀ[d, head]  += Vᵀ·Pᵀ  (A = Vᵀ via the transposing LDS read, B = P)
// (lane l owns head column l%32 and 16 of the block's keys; K rows are taken
// with bits 2 and 3 of the row index swapped so a lane's P values are
// consecutive accumulator elements).  The look-ahead lives in registers as
// well as LDS, so that it is not capped by the LDS size: K of a block is
// loaded straight into the A-operand layout two blocks ahead, V by
// buffer->LDS loads into a ring of four slots three blocks ahead (each slot
// its own LDS array), and each item's Q into an LDS slot with the V of its
// first block.  The loads are compiler builtins, so the compiler derives the
// waits for K and Q; only the V slot reads carry an explicit wait.  V arrives in
// 1 KiB loads of whole cache lines, each line read once, so it uses the
// non-temporal cache policy; the K operand loads read each line over four k-step
// loads and keep the default.  Buffer
// ranges end at the item's last token, so look-ahead past it reads zeros
// without touching memory.  Softmax per head column: weights 2^(S·c - mc),
// mc from the exact max of the item's first block here, raised only when a
// lane's weights of one 32-key block sum past 2^8 (then l and O are rescaled
// and the block's weights redone against the new reference).  At D = 128 the
// partials of items that end inside a wavefront's range are held (O in LDS left
// over at the kernel's occupancy) and written after the range's last block.
#include "decode_common.cuh"

namespace mattn {
namespace {

template <int D> struct Geo {
    static constexpr int RB = D * 2;               // bytes per cache row
    static constexpr int BLK = CK * RB;            // bytes of one K (or V) block
    static constexpr int NCH = BLK / 1024;         // 1 KiB loads per block
    static constexpr int RV = 4;                   // V ring slots (look-ahead RV - 1 blocks)
    static constexpr int LK = 2;                   // K look-ahead in blocks (in registers)
    static constexpr int QCH = 32 * RB / 1024;     // 1 KiB loads of a full 32-head Q slot
};
// One persistent wavefront per resident slot.  Every load is a compiler
// builtin, so the compiler derives each wait from the loads issued after the
// one a use needs: K of a block goes straight into registers in the layout of
// the A operand of K·Qᵀ (lane l: key perm(l % 32), 16 bytes at d = 16·kk +
// 8·(l / 32)), LK blocks ahead; V goes by buffer->LDS loads into a ring of RV
// slots, RV - 1 blocks ahead, each slot its own LDS array so that a read of
// one slot waits only for that slot's loads; an item's Q goes by buffer->LDS
// loads into one of RV Q slots together with the V of its first block.
// PAGED: kc / vc are page pools [num_pages, H_kv, 2^lps, D]; token t of sequence b is
// row t mod 2^lps of page bt[b * max_pages + (t >> lps)] (entries clamped to
// [0, num_pages)), T_max = max_pages << lps.  V of a 32-token block is loaded as two
// 16-token halves, each inside one page through its own buffer range; K by
// per-lane global loads from the page of each key.
template <int D, bool PAGED>
__global__ __launch_bounds__(64)
void decode_stream_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                          const bf16* __restrict__ vc, const int32_t* __restrict__ lens,
                          float* __restrict__ ws_o, float* __restrict__ ws_ml,
                          int B, int H_q, int H_kv, int T_max, int G, int n_hg, int nsplit,
                          int nwaves, int qb, int ns, int sob, float c,
                          const int32_t* __restrict__ bt, int lps, int max_pages, int num_pages) {
    using Gm = Geo<D>;
    constexpr int RB = Gm::RB, BLK = Gm::BLK, NCH = Gm::NCH, QCH = Gm::QCH;
    constexpr int RV = Gm::RV, LK = Gm::LK;
    constexpr int KSTEPS = D / 16;     // MFMA k-steps of K·Qᵀ
    constexpr int DB = D / 32;         // 32-row blocks of Oᵀ
    constexpr int HCH = NCH / 2;       // 1 KiB V loads per 16-token half
    static_assert(RV == 4 && LK >= 1 && LK < RV, "ring geometry");
    __shared__ __attribute__((aligned(16))) unsigned char vs0[BLK], vs1[BLK], vs2[BLK], vs3[BLK];
    extern __shared__ __attribute__((aligned(16))) unsigned char qlds[];   // RV Q slots of qb bytes
    auto vslot = [&](int s) -> unsigned char* { return s == 0 ? vs0 : s == 1 ? vs1 : s == 2 ? vs2 : vs3; };
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

    // K: lane offsets of the operand layout within a block (bytes).  V: LDS byte o =
    // 1 KiB load ch at lane*16 holds row r = o / RB, chunk position p = global chunk
    // p ^ v_swz(r) (conflict-free transposing reads).
    uint32_t k_off[KSTEPS], v_voff[NCH];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) k_off[kk] = (uint32_t)(swap_bits23(l32) * RB + (kk * 16 + hl * 8) * 2);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int o = ch * 1024 + lane * 16;
        const int r = o / RB, p = (o % RB) / 16;
        v_voff[ch] = (uint32_t)(r * RB + (p ^ v_swz<D>(r)) * 16);
    }
    const __amdgpu_buffer_rsrc_t zrs = brsrc(kc, 0u);
    const i32x4_sgpr z4 = make_rsrc(kc, 0u);    // the same empty range, for the buffer->LDS loads

    // Paged: the buffer ranges of the two 16-token halves of block (cursor) x, each
    // inside one page (pages are powers of two >= 16 tokens, blocks start at
    // multiples of 32): kh/vh and the row offset of the half within its range.
    auto page_halves = [&](const Cursor& x, __amdgpu_buffer_rsrc_t* kh, i32x4_sgpr* vh,
                           uint32_t* roff) {
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
            if (kh) kh[h] = zrs;
            if (vh) vh[h] = z4;
            roff[h] = 0u;
            const int th = t0 + 16 * h;
            if (th < x.t_end) {
                const int page = min(max(pe[h], 0), num_pages - 1);
                const int pstart = pidx[h] << lps;
                const int rows = min(1 << lps, x.t_end - pstart);
                const size_t head = (((size_t)page * H_kv + x.g) << lps) * D;
                if (kh) kh[h] = brsrc(kc + head, (uint32_t)rows * RB);
                if (vh) vh[h] = make_rsrc(vc + head, (uint32_t)rows * RB);
                roff[h] = (uint32_t)(th - pstart) * RB;
            }
        }
    };

    // ---- issue side: V (+ Q) cursor RV-1 blocks ahead of the compute, K cursor LK ahead
    Cursor icv = cursor_at(L, HG, n_hg, b0, a0 - before);
    Cursor ick = icv;
    int nv = 0, nk = 0, qs_issue = 0;
    __amdgpu_buffer_rsrc_t krs = zrs;
    i32x4_sgpr vrs = z4;
    auto item_rsrc = [&](const Cursor& x, const bf16* base) {
        const size_t head = ((size_t)x.b * H_kv + x.g) * (size_t)T_max * D;
        return brsrc(base + head, (uint32_t)x.t_end * RB);
    };
    auto item_rsrc4 = [&](const Cursor& x, const bf16* base) {
        const size_t head = ((size_t)x.b * H_kv + x.g) * (size_t)T_max * D;
        return make_rsrc(base + head, (uint32_t)x.t_end * RB);
    };
    if constexpr (!PAGED) {
        vrs = item_rsrc4(icv, vc);
        krs = item_rsrc(ick, kc);
    }
    auto issue_v = [&](int s) {
        const bool live = nv < nblk;
        unsigned char* dst = vslot(s);
        if constexpr (PAGED) {
            i32x4_sgpr vh[2] = {z4, z4};
            uint32_t roff[2] = {0u, 0u};
            if (live) page_halves(icv, nullptr, vh, roff);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
                lds_dma16<true>(vh[ch / HCH], dst + ch * 1024, roff[ch / HCH] + v_voff[ch] - (ch / HCH) * 16u * RB,
                          ch == NCH - 1);
        } else {
            const uint32_t row0 = (uint32_t)(icv.s * kDecodeSplit + icv.i * CK) * RB;
            const i32x4_sgpr r = live ? vrs : z4;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) lds_dma16<true>(r, dst + ch * 1024, row0 + v_voff[ch], ch == NCH - 1);
        }
        if (!live) return;
        if (icv.i == 0 || nv == 0) {     // the item's Q (also for a range that starts inside it)
            const int ncols = min(32, G - icv.hg * 32);
            const i32x4_sgpr qrs =
                make_rsrc(q + ((size_t)icv.b * H_q + icv.g * G + icv.hg * 32) * D, (uint32_t)(ncols * RB));
#pragma unroll
            for (int ch = 0; ch < QCH; ++ch)
                if (ch * 1024 < ncols * RB)
                    lds_dma16(qrs, qslot(qs_issue) + ch * 1024, (uint32_t)(ch * 1024 + lane * 16),
                              (ch + 1) * 1024 >= ncols * RB);
        }
        ++nv;
        advance(icv, L, HG, n_hg);
        if (icv.i == 0) {
            qs_issue = qs_issue == RV - 1 ? 0 : qs_issue + 1;
            if constexpr (!PAGED) vrs = item_rsrc4(icv, vc);
        }
    };
    u32x4 kr[RV][KSTEPS];
    auto issue_k = [&](int s) {
        const bool live = nk < nblk;
        if constexpr (PAGED) {
            // one global load per k-step from a per-lane address: lane l reads key perm(l % 32)
            // of the block from the page of its half; a key past the item's end (its score is
            // masked) and a block past the wavefront's range read row 0 of a valid page
            const bf16* src = kc;
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
                kr[s][kk] = *reinterpret_cast<const u32x4*>(src + kk * 16 + hl * 8);
        } else {
            const uint32_t row0 = (uint32_t)(ick.s * kDecodeSplit + ick.i * CK) * RB;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) kr[s][kk] = bload16(live ? krs : zrs, row0 + k_off[kk]);
        }
        if (!live) return;
        ++nk;
        advance(ick, L, HG, n_hg);
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
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mc = 0.f, lsum = 0.f;
    bool mc_set = false;
    // Partials of items that ended inside the range, held until it ends.  At D = 64 two
    // workgroups per SIMD fill the LDS with their V rings and Q slots, so no slot is ever
    // free for them and the stash is compiled out.
    constexpr bool STASH = D == 128;
    Held held0{}, held1{};
    int nheld = 0;

    // Vᵀ operand reads (as in the prefill kernel)
    const int vg = lane >> 4, vm = lane & 15;
    const int vrow = (vg >> 1) * 8 + (vm >> 2);
    const int vfv = v_swz<D>(vrow);
    const int vc0 = 2 * (vg & 1) + ((vm & 3) >> 1);
    const int vin = (vm & 1) * 4;
    uint32_t v_lane[DB];           // this lane's byte offset of row block db in a V slot
#pragma unroll
    for (int db = 0; db < DB; ++db) v_lane[db] = (uint32_t)((vrow * D + (((db * 4 + vc0) ^ vfv) * 8) + vin) * 2);
    // The slot waits.  Loop iteration i issues, in this program order: V of block
    // i + RV - 1 (NCH buffer->LDS loads, then the QCH loads of the item's Q if that block
    // starts an item), K of block i + LK (KSTEPS loads), then computes block i.  The
    // buffer->LDS loads are asm statements with a memory clobber and the waits too, so the
    // compiler moves no load across either: the count below is a property of this source.
    // Between the V (and Q) loads of block j and the wait in front of computing j come at
    // least the V loads of the RV - 1 blocks after j and the K loads of LK + 1 blocks (the
    // fewest at the first block of a range, where the prologue has issued K of blocks
    // 0 .. LK - 1 only): NV_AFTER loads, plus any Q loads and partial stores.  Loads return
    // in issue order, so while block j's V or Q is outstanding so are all the loads after
    // it, and at most NV_AFTER outstanding means they have landed.
    constexpr int V_LOADS_AFTER = (RV - 1) * NCH;       // V of blocks j+1 .. j+RV-1
    constexpr int K_LOADS_AFTER = (LK + 1) * KSTEPS;    // K of (at least) LK + 1 blocks
    constexpr int NV_AFTER = V_LOADS_AFTER + K_LOADS_AFTER;
    static_assert(RV == 4 && LK == 2 && NCH == BLK / 1024 && KSTEPS == D / 16, "the counted geometry");
    static_assert(LK + 1 <= RV, "K of LK + 1 blocks is issued before block j is computed");
    static_assert(NV_AFTER <= 63, "vmcnt range");

    auto compute = [&](int j, int s) {
        const int g = cc.g, hg = cc.hg;
        const int col = hg * 32 + l32;
        const bool col_ok = col < G;
        if (need_q) {                    // first block of an item: Q from its LDS slot
            wait_vmem_le<NV_AFTER>();    // the slot's buffer->LDS loads have landed
            // rows past the group's heads are not in the slot: read row 0 there, then zero
            const bf16* qrow = reinterpret_cast<const bf16*>(qslot(qs)) + (col_ok ? l32 : 0) * D;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hl * 8);
                qreg[kk] = __builtin_bit_cast(bf16x8, col_ok ? v : u32x4{0u, 0u, 0u, 0u});
            }
            need_q = false;
        }
        f32x16 S = {};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[s][kk]), qreg[kk], S, 0, 0, 0);
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
        // Weights of the block's 16 keys in this lane.  If their sum passes 2^8 (rare), the
        // reference is raised to the block's row max where that is higher, O and l are scaled
        // by 2^(old - new) and all 16 weights are redone, before any of them is packed: the
        // P operand of both k-steps then uses one reference, the one O and l are kept in.
        float p[16];
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c, -mc));
            cs += p[e];
        }
        if (__ballot(cs > kRescaleSum)) {
            float m = S[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) m = fmaxf(m, S[e]);
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
            for (int e = 0; e < 16; ++e) {
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], c, -mc));
                cs += p[e];
            }
        }
        lsum += cs;
        u32x4 pw[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[k2][e] = pack_bf16x2(p[k2 * 8 + 2 * e], p[k2 * 8 + 2 * e + 1]);
        u32x4 va[2][DB];
        {
            const uint32_t sb = (uint32_t)reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) unsigned char*)vslot(s));
            uint32_t addr[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) addr[db] = sb + v_lane[db];
            wait_vmem_le<NV_AFTER>();
            v_operands<D>(addr, va);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va[k2][db]), __builtin_bit_cast(bf16x8, pw[k2]),
                    oacc[db], 0, 0, 0);

        // end of this wavefront's part of the item: write the partial
        if (cc.i == cc.nb - 1 || j == nblk - 1) {
            const float Lsum = pair_sum(lsum);
            if (STASH && j < nblk - 1 && nheld < ns) {
                // the item ends inside the range: hold its partial until the range ends
                stash_o<D, false>(stash + nheld * sob, oacc, 1.f, col_ok, l32, hl);
                const Held h = make_held((uint32_t)(((cc.b * H_q + g * G + hg * 32) * nsplit + cc.s) * 2 + part),
                                         min(32, G - hg * 32), part == 0, mc, Lsum);
                if (nheld == 0) held0 = h;
                else held1 = h;
                ++nheld;
            } else if (col_ok) {
                // the group's (split, part) slots: head column col, slot (col*nsplit + s)*2 + part
                const size_t slot = ((size_t)(cc.b * H_q + g * G + col) * nsplit + cc.s) * 2 + part;
                float* orow = ws_o + slot * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        *reinterpret_cast<f32x4*>(orow + db * 32 + g4 * 8 + hl * 4) =
                            f32x4{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
                // lanes of the first half store (reference, sum); lanes of the second half
                // the empty part 1 of an item finished by the wavefront that began it
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
        advance(cc, L, HG, n_hg);
    };

    // block j sits in V slot j % RV and K slot j % RV; the loop is unrolled RV times so
    // every slot index is a constant
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
    wait_vmem_le<0>();     // the look-ahead's LDS loads land before the wavefront ends
    static_assert(kStashSlots == 2, "held0, held1");
    if constexpr (STASH) {
        if (nheld > 0) stash_flush<D>(stash, held0, nsplit, ws_o, ws_ml);
        if (nheld > 1) stash_flush<D>(stash + sob, held1, nsplit, ws_o, ws_ml);
    }
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a) {
    const int G = a.H_q / a.H_kv;
    const int n_hg = (G + 31) / 32;
    const int nsplit = decode_nsplit(a.T_max);
    const int qb = q_slot_bytes(G, D);
    const int lds0 = Geo<D>::RV * qb;
    ATTN_CHECK(G >= 1 && G * a.H_kv == a.H_q, "query heads group onto KV heads");
    ATTN_CHECK(lds0 + Geo<D>::RV * Geo<D>::BLK <= kLdsBytesPerCu, "V ring and Q slots fit a CU");
    ATTN_CHECK(nsplit >= 1 && (long long)nsplit * kDecodeSplit >= a.T_max, "splits cover the cache");
    ATTN_CHECK((size_t)a.B * a.H_q * nsplit * 2 * (D + 2) * sizeof(float) <=
                   decode_workspace_bytes(a.B, a.H_q, a.T_max, D),
               "partials and (reference, sum) pairs fit the workspace");
    ATTN_CHECK((long long)a.B * a.H_q * nsplit * 2 < (1ll << 31), "partial slot indices fit 31 bits (held partials)");
    ATTN_CHECK(PAGED || (long long)a.T_max * D * 2 < (1ll << 31), "a (sequence, KV head) fits a 32-bit range");
    ATTN_CHECK(!PAGED || (a.page_size >= 16 && (a.page_size & (a.page_size - 1)) == 0 &&
                          (long long)a.max_pages * a.page_size == a.T_max),
               "pages are powers of two of at least 16 tokens");
    ATTN_CHECK((long long)a.B * a.H_q / 4 + 1 <= kMaxGrid, "combine grid size");
    // the largest dynamic LDS any call uses: RV full 32-head Q slots and the stash slots
    static const int max_dyn = Geo<D>::RV * q_slot_bytes(32, D) + kStashSlots * stash_slot_bytes(32, D);
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)decode_stream_kernel<D, PAGED>, hipFuncAttributeMaxDynamicSharedMemorySize, max_dyn);
    if (attr != hipSuccess) return attr;
    // one round of the whole GPU: the wavefronts resident at the Q slots' LDS, and as many
    // stash slots as leave that count unchanged
    const int cus = cu_count(), per_cu = blocks_per_cu<decode_stream_kernel<D, PAGED>>(lds0);
    const int nwaves = cus > 0 && per_cu > 0 ? cus * per_cu : 256;
    const int sob = stash_slot_bytes(G, D);
    const int ns = D == 128 && per_cu > 0 ? stash_slots<decode_stream_kernel<D, PAGED>>(lds0, sob, max_dyn, per_cu) : 0;
    const int lds = lds0 + ns * sob;
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = ws_o + (size_t)a.B * a.H_q * nsplit * 2 * D;
    const int lps = PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
    hipLaunchKernelGGL((decode_stream_kernel<D, PAGED>), dim3(nwaves), dim3(64), lds, (hipStream_t)a.stream,
                       (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens, ws_o, ws_ml,
                       a.B, a.H_q, a.H_kv, a.T_max, G, n_hg, nsplit, nwaves, qb, ns, sob, a.scale * kLog2e,
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
