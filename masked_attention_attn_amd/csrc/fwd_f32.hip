// Masked attention forward for float32 inputs, float32 arithmetic throughout.
//
// Same operation as the bf16 path (scores scale·Q·Kᵀ, additive -inf on
// padded keys, online softmax, product with V, per-row LSE; molayo1419.me
// MultiheadAttention fast-path page, sections "소스의 현실" and
// "CPU에서 양을 측정하기"), for the fp32 case whose error budget rules out
// bf16 matrix-core inputs.  Both products run on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 sums) in the bf16 kernel's
// transposed mapping:
//   Sᵀ[key, query] = K·Qᵀ: k-step ks takes d = ks from lanes 0-31 and
//     d = D/2 + ks from lanes 32-63, so a lane's K and Q operands are D/2
//     consecutive floats of one row;
//   Oᵀ[d, query] += Vᵀ·Pᵀ: lane l owns query l%32 and 16 keys of a 32-key
//     block (rows (i/4)*8 + (l/32)*4 + i%4 of the score accumulator), and
//     its i-th weight is the B operand of k-step i, whose two keys are the
//     i-th keys of the two lane halves.
//
// Work decomposition: a workgroup of four wavefronts owns 32 queries of one
// (b, h); wavefront w takes key blocks w, w+4, w+8, ... with an online
// softmax of its own, and the four partial states (reference, weight sum,
// unnormalised O) are merged through LDS with the log-sum-exp rule at the
// end.  K and V operands are loaded from global memory (L2) straight into
// the operand layouts: V at the start of its block (it is first used after
// the block's K·Qᵀ and softmax), K a block ahead at D = 64.  D = 128 holds
// twice the operands and runs one workgroup per CU.
#include "common.cuh"
#include "launch.h"
#include "mfma_lds.cuh"

namespace mattn {
namespace {
using mfma::pair_max;
using mfma::pair_sum;

constexpr int NW = 4;            // wavefronts per workgroup
constexpr int QB = 32;           // queries per workgroup
constexpr int KB = 32;           // keys per block

template <int D> constexpr int merge_lds_bytes() { return NW * QB * (D + 1) * 4 + 2 * NW * QB * 4; }

template <int D> constexpr int wg_per_cu() { return D == 64 ? 2 : 1; }

template <int D, bool WRITE_LSE>
__global__ __launch_bounds__(64 * NW, wg_per_cu<D>())
void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, const uint8_t* __restrict__ mask,
                    float* __restrict__ o, float* __restrict__ lse,
                    int H, int Tq, int Tk, float c, int n_qt, int total) {
    constexpr int HK = D / 2;            // k-steps of K·Qᵀ (two d per step)
    constexpr int DB = D / 32;           // 32-row blocks of Oᵀ
    constexpr int DP = D + 1;            // LDS row pitch of the merge (conflict-free stores)
    constexpr bool AHEAD = D == 64;      // next block's K loaded during this one's products
    extern __shared__ float smem[];
    float* sm_o = smem;                          // [NW][QB][DP]
    float* sm_m = smem + NW * QB * DP;           // [NW][QB]
    float* sm_l = sm_m + NW * QB;                // [NW][QB]

    const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
    if (logical >= total) return;
    const int bh = logical / n_qt;
    const int qt = logical - bh * n_qt;
    const int b = bh / H;
    const float* qp = q + (size_t)bh * Tq * D;
    const float* kp = k + (size_t)bh * Tk * D;
    const float* vp = v + (size_t)bh * Tk * D;
    const uint8_t* mp = mask ? mask + (size_t)b * Tk : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hl = lane >> 5;
    const int q0 = qt * QB;

    // Q as the B operand of K·Qᵀ: query l32 (rows past Tq read the last row; never stored)
    float qv[HK];
    {
        const float* qrow = qp + (size_t)min(q0 + l32, Tq - 1) * D + hl * HK;
#pragma unroll
        for (int e = 0; e < HK; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(qrow + e);
            qv[e] = t[0]; qv[e + 1] = t[1]; qv[e + 2] = t[2]; qv[e + 3] = t[3];
        }
    }
    // operands of key block kb: K (A of K·Qᵀ, key row l32, d = hl*HK ..) and Vᵀ (A of
    // Vᵀ·Pᵀ: k-step i, row block db: key (i/4)*8 + hl*4 + i%4, d = db*32 + l32); keys past
    // Tk read the last row (their weights are zero)
    auto load_k = [&](int kb, float (&kr)[HK]) {
        const float* krow = kp + (size_t)min(kb * KB + l32, Tk - 1) * D + hl * HK;
#pragma unroll
        for (int e = 0; e < HK; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(krow + e);
            kr[e] = t[0]; kr[e + 1] = t[1]; kr[e + 2] = t[2]; kr[e + 3] = t[3];
        }
    };
    auto load_v = [&](int kb, float (&va)[16][DB]) {
        const int key0 = kb * KB;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* vrow = vp + (size_t)min(key0 + (i >> 2) * 8 + hl * 4 + (i & 3), Tk - 1) * D + l32;
#pragma unroll
            for (int db = 0; db < DB; ++db) va[i][db] = vrow[db * 32];
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m = kNegInf, lsum = 0.f;       // reference (log2 units) and this lane's weight sum
    const int nkb = (Tk + KB - 1) / KB;
    float kr[HK], va[16][DB];
    if (AHEAD && wave < nkb) load_k(wave, kr);
    for (int kb = wave; kb < nkb; kb += NW) {
        if constexpr (!AHEAD) load_k(kb, kr);
        load_v(kb, va);
        f32x16 s = {};
#pragma unroll
        for (int ks = 0; ks < HK; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[ks], qv[ks], s, 0, 0, 0);
        if (AHEAD && kb + NW < nkb) load_k(kb + NW, kr);
        // padded keys: lane j < 32 flags key key0 + j, gathered into one wave-uniform mask
        const int key0 = kb * KB;
        int padf = 1;
        if (lane < KB) {
            const int key = key0 + lane;
            padf = key >= Tk ? 1 : (mp ? (int)(mp[key] != 0) : 0);
        }
        const uint32_t pm = (uint32_t)__ballot(padf);
        if (pm == ~0u) continue;           // every key of the block padded (wave-uniform)
        float sv[16];
        float bm = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kj = (i >> 2) * 8 + hl * 4 + (i & 3);
            sv[i] = ((pm >> kj) & 1u) ? kNegInf : s[i] * c;
            bm = fmaxf(bm, sv[i]);
        }
        const float mn = fmaxf(m, pair_max(bm));     // finite: the block holds an unpadded key
        const float alpha = __builtin_amdgcn_exp2f(m - mn);    // m = -inf: 0
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sv[i] - m);          // padded: 0
            lsum += p[i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[i][db], p[i], oacc[db], 0, 0, 0);
    }

    // ---- merge of the four wavefronts' states: (m, l) per query and O in [query][d]
    const float lt = pair_sum(lsum);
    if (hl == 0) {
        sm_m[wave * QB + l32] = m;
        sm_l[wave * QB + l32] = lt;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sm_o[(wave * QB + l32) * DP + db * 32 + (i >> 2) * 8 + hl * 4 + (i & 3)] = oacc[db][i];
    __syncthreads();
    // thread t: query t/8, elements (t%8)*D/8 .. + D/8
    constexpr int EPT = D / 8;
    const int qq = tid >> 3, d0 = (tid & 7) * EPT;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * QB + qq]);
    const int qi = q0 + qq;
    if (qi >= Tq) return;
    float* orow = o + ((size_t)bh * Tq + qi) * D + d0;
    if (M == kNegInf) {                  // no unpadded key
#pragma unroll
        for (int e = 0; e < EPT; ++e) orow[e] = 0.f;
        if (WRITE_LSE && (tid & 7) == 0) lse[(size_t)bh * Tq + qi] = kNegInf;
        return;
    }
    float wt[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w * QB + qq];
        wt[w] = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += wt[w] * sm_l[w * QB + qq];
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
        f32x4 r;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) acc = __builtin_fmaf(wt[w], sm_o[(w * QB + qq) * DP + d0 + e + x], acc);
            r[x] = acc * inv;
        }
        *reinterpret_cast<f32x4*>(orow + e) = r;
    }
    if (WRITE_LSE && (tid & 7) == 0) lse[(size_t)bh * Tq + qi] = (M + __log2f(L)) * kLn2;
}

template <int D, bool WRITE_LSE>
hipError_t launch_one(const FwdArgs& a) {
    const int n_qt = (a.Tq + QB - 1) / QB;
    const long long total = (long long)a.B * a.H * n_qt;
    const long long grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    ATTN_CHECK(n_qt >= 1 && (long long)n_qt * QB >= a.Tq, "query blocks cover every row");
    ATTN_CHECK(grid >= total && grid <= kMaxGrid && grid % kNumXcd == 0, "grid size");
    constexpr int lds = merge_lds_bytes<D>();
    ATTN_CHECK(lds * wg_per_cu<D>() <= kLdsBytesPerCu, "the workgroups' merge areas fit a CU");
    // LDS above 64 KiB must be opted into once per kernel (thread-safe static init).
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)fwd_f32_kernel<D, WRITE_LSE>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((fwd_f32_kernel<D, WRITE_LSE>), dim3((unsigned)grid), dim3(64 * NW), lds,
                       (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, a.mask,
                       (float*)a.o, a.lse, a.H, a.Tq, a.Tk, a.scale * kLog2e, n_qt, (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
    if (a.D == 64) return a.lse ? launch_one<64, true>(a) : launch_one<64, false>(a);
    return a.lse ? launch_one<128, true>(a) : launch_one<128, false>(a);
}

}  // namespace mattn
