// Masked attention forward for float32 inputs, float32 arithmetic throughout.
//
// Same operation as the bf16 path (scores scale·Q·Kᵀ, additive -inf on
// padded keys, online softmax, product with V, per-row LSE; molayo1419.me
// MultiheadAttention fast-path page, sections "소스의 현실" and
// "CPU에서 양을 측정하기"), for the fp32 case whose error budget rules out
// bf16 matrix-core inputs.  Vector-ALU kernel: two threads own one query row
// (each holds half of the head dimension of q and of the output), K/V tiles
// of 32 keys are staged in LDS and read as broadcasts.
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NT = 256;          // threads per workgroup
constexpr int QPB = NT / 2;      // queries per workgroup
constexpr int TK = 32;           // keys per tile

template <int D, bool WRITE_LSE>
__global__ __launch_bounds__(NT)
void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, const uint8_t* __restrict__ mask,
                    float* __restrict__ o, float* __restrict__ lse,
                    int H, int Tq, int Tk, float c, int n_qt, int total) {
    constexpr int HD = D / 2;                 // head-dim elements owned by one thread
    __shared__ __attribute__((aligned(16))) float ks[TK][D];
    __shared__ __attribute__((aligned(16))) float vs[TK][D];
    __shared__ int pad_s[TK];

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
    const int half = tid & 1;
    const int qi = qt * QPB + (tid >> 1);
    const int qrow = min(qi, Tq - 1);
    const int d0 = half * HD;

    float qr[HD], acc[HD];
#pragma unroll
    for (int e = 0; e < HD; e += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(qp + (size_t)qrow * D + d0 + e);
        qr[e] = t[0]; qr[e + 1] = t[1]; qr[e + 2] = t[2]; qr[e + 3] = t[3];
        acc[e] = acc[e + 1] = acc[e + 2] = acc[e + 3] = 0.f;
    }
    float m = kNegInf, l = 0.f;

    const int ntiles = (Tk + TK - 1) / TK;
    for (int kt = 0; kt < ntiles; ++kt) {
        const int base = kt * TK;
        __syncthreads();
        for (int idx = tid; idx < TK * D / 4; idx += NT) {
            const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const int key = base + row;
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (key < Tk) {
                kk = *reinterpret_cast<const f32x4*>(kp + (size_t)key * D + col);
                vv = *reinterpret_cast<const f32x4*>(vp + (size_t)key * D + col);
            }
            *reinterpret_cast<f32x4*>(&ks[row][col]) = kk;
            *reinterpret_cast<f32x4*>(&vs[row][col]) = vv;
        }
        if (tid < TK) {
            const int key = base + tid;
            pad_s[tid] = key >= Tk ? 1 : (mp ? (int)(mp[key] != 0) : 0);
        }
        __syncthreads();

        // scores of this tile, already in log2 units (·scale·log2 e)
        float s[TK];
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < HD; ++e) part = __builtin_fmaf(qr[e], ks[j][d0 + e], part);
            const float full = part + __shfl_xor(part, 1, 64);
            s[j] = pad_s[j] ? kNegInf : full * c;
            tmax = fmaxf(tmax, s[j]);
        }
        if (tmax == kNegInf) continue;          // every key of the tile is padded
        const float mnew = fmaxf(m, tmax);
        const float alpha = exp2f(m - mnew);    // m = -inf -> 0
        l *= alpha;
#pragma unroll
        for (int e = 0; e < HD; ++e) acc[e] *= alpha;
        m = mnew;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            const float p = exp2f(s[j] - m);    // padded: exp2(-inf) = 0
            l += p;
#pragma unroll
            for (int e = 0; e < HD; ++e) acc[e] = __builtin_fmaf(p, vs[j][d0 + e], acc[e]);
        }
    }

    if (qi < Tq) {
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float* orow = o + ((size_t)bh * Tq + qi) * D + d0;
#pragma unroll
        for (int e = 0; e < HD; e += 4) {
            f32x4 t = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + e) = t;
        }
        if (WRITE_LSE && half == 0)
            lse[(size_t)bh * Tq + qi] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
    }
}

template <int D, bool WRITE_LSE>
hipError_t launch_one(const FwdArgs& a) {
    const int n_qt = (a.Tq + QPB - 1) / QPB;
    const int total = a.B * a.H * n_qt;
    const int grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
    ATTN_CHECK(n_qt >= 1 && (long long)n_qt * QPB >= a.Tq, "query blocks cover every row");
    ATTN_CHECK(grid >= total && grid <= kMaxGrid && grid % kNumXcd == 0, "grid size");
    hipLaunchKernelGGL((fwd_f32_kernel<D, WRITE_LSE>), dim3(grid), dim3(NT), 0, (hipStream_t)a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, a.mask,
                       (float*)a.o, a.lse, a.H, a.Tq, a.Tk, a.scale * kLog2e, n_qt, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
    if (a.D == 64) return a.lse ? launch_one<64, true>(a) : launch_one<64, false>(a);
    return a.lse ? launch_one<128, true>(a) : launch_one<128, false>(a);
}

}  // namespace mattn
