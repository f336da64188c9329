// Single-token decode against the KV cache, grouped-query attention.
//
// The current token's query attends over every cached K/V position of its
// sequence (agentlenshq.com, "nanoVLM에서 KV 캐시 구현", section "KV 캐싱이
// 추론을 최적화하는 방법").  The work is dominated by reading the cache:
// 2·H_kv·D·elem_bytes per cached token and layer (blog.ruahverce.com, LLM
// inference memory accounting 2/10, "10. KV Cache Byte 공식" and "13. KV는
// Token마다 자란다"), so the kernel is organised around reading every cache
// byte exactly once, coalesced: the query heads that share a KV head (GQA,
// same page "11. 계산 예시: GQA Decoder") are all served from one read.
//
// Split-K: workgroup (split, b, kv head, query-head group) streams tokens
// [split*S, min(len, (split+1)*S)) with S = kDecodeSplit.  A token's row of
// D elements is spread over LG lanes holding one 16-byte chunk each; the
// partial dot products are summed across those lanes.  Each token slot keeps
// its own online-softmax state (m, l, o); slots are merged in LDS and the
// split's unnormalised (m, l, o) goes to the workspace.  A second kernel
// merges the splits of every (b, query head) with the same log-sum-exp rule
// as the chunk merge (sglang PR 49078 analysis, "1. aiter.py") and
// normalises.  Lengths are read on the device; workgroups whose split starts
// past the length exit at once.
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr int UNROLL = 4;   // tokens per lane per batch of loads

template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
    static constexpr int EPC = 8;   // elements per 16-byte chunk
    static __device__ __forceinline__ void cvt(u32x4 w, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[2 * j] = bf16_lo(w[j]); x[2 * j + 1] = bf16_hi(w[j]); }
    }
};
template <> struct Chunk<float> {
    static constexpr int EPC = 4;
    static __device__ __forceinline__ void cvt(u32x4 w, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(w[j]);
    }
};

template <int LG>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = 1; off < LG; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <typename T, int D, int NG>
__global__ __launch_bounds__(NT)
void decode_split_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                         const T* __restrict__ vc, const int32_t* __restrict__ lens,
                         float* __restrict__ ws_o, float* __restrict__ ws_ml,
                         int H_q, int H_kv, int T_max, int G, int nsplit, float c) {
    constexpr int EPC = Chunk<T>::EPC;
    constexpr int LG = D / EPC;          // lanes per token
    constexpr int TPW = 64 / LG;         // token slots per wave
    constexpr int NSLOT = NWAVE * TPW;   // token slots per workgroup
    __shared__ float sm_o[NSLOT][D];
    __shared__ float sm_m[NSLOT][NG];
    __shared__ float sm_l[NSLOT][NG];

    const int split = blockIdx.y;
    const int ngrp = G / NG;
    const int bg = blockIdx.x / ngrp;
    const int grp = blockIdx.x - bg * ngrp;
    const int b = bg / H_kv;
    const int g = bg - b * H_kv;
    const int len = min(max(lens[b], 0), T_max);
    const int t_begin = split * kDecodeSplit;
    if (t_begin >= len) return;                  // whole workgroup: no barrier reached
    const int t_end = min(len, t_begin + kDecodeSplit);
    const int h0 = g * G + grp * NG;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ch = lane % LG;
    const int slot = wave * TPW + lane / LG;

    float qf[NG][EPC];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const u32x4 w = ldg128(q + ((size_t)b * H_q + h0 + j) * D + ch * EPC);
        Chunk<T>::cvt(w, qf[j]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) qf[j][e] *= c;
    }
    float m[NG], l[NG], acc[NG][EPC];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        m[j] = kNegInf; l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[j][e] = 0.f;
    }

    const size_t head_off = ((size_t)b * H_kv + g) * T_max * D + ch * EPC;
    const T* kb = kc + head_off;
    const T* vb = vc + head_off;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // Wave-uniform trip count so every lane takes part in the cross-lane sums.
    for (int t0 = t_begin + wave * TPW; t0 < t_end; t0 += NSLOT * UNROLL) {
        u32x4 kw[UNROLL], vw[UNROLL];
        bool valid[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int tt = t0 + lane / LG + u * NSLOT;
            valid[u] = tt < t_end;
            // whole token rows of consecutive slots, each cache line read once: streaming loads
            kw[u] = valid[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)tt * D)) : zero4;
            vw[u] = valid[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (size_t)tt * D)) : zero4;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            float kf[EPC], vf[EPC];
            Chunk<T>::cvt(kw[u], kf);
            Chunk<T>::cvt(vw[u], vf);
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) part = __builtin_fmaf(qf[j][e], kf[e], part);
                const float s = group_sum<LG>(part);       // score in log2 units
                if (valid[u]) {
                    const float mn = fmaxf(m[j], s);
                    const float alpha = __builtin_amdgcn_exp2f(m[j] - mn);   // -inf -> 0
                    const float p = __builtin_amdgcn_exp2f(s - mn);
                    l[j] = __builtin_fmaf(l[j], alpha, p);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[j][e] = __builtin_fmaf(acc[j][e], alpha, p * vf[e]);
                    m[j] = mn;
                }
            }
        }
    }

    // Merge the NSLOT token slots of this workgroup, one query head at a time
    // (fully unrolled so the per-head registers stay statically indexed).
#pragma unroll
    for (int j = 0; j < NG; ++j) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_o[slot][ch * EPC + e] = acc[j][e];
        if (ch == 0) { sm_m[slot][j] = m[j]; sm_l[slot][j] = l[j]; }
        __syncthreads();
        const size_t part = ((size_t)b * H_q + h0 + j) * nsplit + split;
        for (int d = tid; d < D; d += NT) {
            float M = kNegInf;
#pragma unroll
            for (int s = 0; s < NSLOT; ++s) M = fmaxf(M, sm_m[s][j]);
            float o = 0.f, L = 0.f;
#pragma unroll
            for (int s = 0; s < NSLOT; ++s) {
                const float w = __builtin_amdgcn_exp2f(sm_m[s][j] - M);     // empty slot -> 0
                o = __builtin_fmaf(sm_o[s][d], w, o);
                L = __builtin_fmaf(sm_l[s][j], w, L);
            }
            ws_o[part * D + d] = o;
            if (d == 0) { ws_ml[part * 2] = M; ws_ml[part * 2 + 1] = L; }
        }
        __syncthreads();
    }
}

template <typename T> struct Store;
template <> struct Store<bf16> {
    static __device__ __forceinline__ void one(bf16* p, float x) { *p = (bf16)x; }
};
template <> struct Store<float> {
    static __device__ __forceinline__ void one(float* p, float x) { *p = x; }
};

template <typename T, int D>
__global__ __launch_bounds__(D)
void decode_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                           const int32_t* __restrict__ lens, T* __restrict__ o,
                           float* __restrict__ lse, int H_q, int T_max, int nsplit) {
    const int bh = blockIdx.x;
    const int b = bh / H_q;
    const int len = min(max(lens[b], 0), T_max);
    const int ns = (len + kDecodeSplit - 1) / kDecodeSplit;
    const int d = threadIdx.x;
    const size_t base = (size_t)bh * nsplit;
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ws_ml[(base + s) * 2]);
    if (ns == 0 || M == kNegInf) {
        Store<T>::one(o + (size_t)bh * D + d, 0.f);
        if (lse && d == 0) lse[bh] = kNegInf;
        return;
    }
    float acc = 0.f, L = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = __builtin_amdgcn_exp2f(ws_ml[(base + s) * 2] - M);
        acc = __builtin_fmaf(ws_o[(base + s) * D + d], w, acc);
        L = __builtin_fmaf(ws_ml[(base + s) * 2 + 1], w, L);
    }
    Store<T>::one(o + (size_t)bh * D + d, acc / L);
    if (lse && d == 0) lse[bh] = (M + __log2f(L)) * kLn2;
}

template <typename T, int D, int NG>
void launch_split(const DecodeArgs& a, float* ws_o, float* ws_ml, int nsplit) {
    const int G = a.H_q / a.H_kv;
    dim3 grid(a.B * a.H_kv * (G / NG), nsplit);
    hipLaunchKernelGGL((decode_split_kernel<T, D, NG>), grid, dim3(NT), 0, (hipStream_t)a.stream,
                       (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache, a.lens,
                       ws_o, ws_ml, a.H_q, a.H_kv, a.T_max, G, nsplit, a.scale * kLog2e);
}

template <typename T, int D>
hipError_t launch(const DecodeArgs& a) {
    const int nsplit = decode_nsplit(a.T_max);
    const size_t parts = (size_t)a.B * a.H_q * nsplit;
    float* ws_o = static_cast<float*>(a.workspace);
    float* ws_ml = ws_o + parts * D;
    const int G = a.H_q / a.H_kv;
    ATTN_CHECK(G >= 1 && G * a.H_kv == a.H_q, "query heads group onto KV heads");
    ATTN_CHECK(parts * (D + 2) * sizeof(float) <= decode_workspace_bytes(a.B, a.H_q, a.T_max, D),
               "split partials fit the workspace");
    ATTN_CHECK((long long)a.B * a.H_kv * G <= kMaxGrid && (long long)a.B * a.H_q <= kMaxGrid, "grid size");
    if (G % 8 == 0) launch_split<T, D, 8>(a, ws_o, ws_ml, nsplit);
    else if (G % 4 == 0) launch_split<T, D, 4>(a, ws_o, ws_ml, nsplit);
    else if (G % 2 == 0) launch_split<T, D, 2>(a, ws_o, ws_ml, nsplit);
    else launch_split<T, D, 1>(a, ws_o, ws_ml, nsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.H_q), dim3(D), 0, (hipStream_t)a.stream,
                       ws_o, ws_ml, a.lens, (T*)a.o, a.lse, a.H_q, a.T_max, nsplit);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a) {
    return a.D == 64 ? launch<float, 64>(a) : launch<float, 128>(a);
}

}  // namespace mattn
