// LSE merge of attention results computed over disjoint KV chunks.
//
// For every row: lse = M + log sum_i exp(lse_i - M) with M = max_i lse_i,
// out = sum_i exp(lse_i - lse)·out_i — the online-softmax merge that ring
// attention applies to per-hop partial outputs (blog.secrett2633.cloud,
// sglang PR 49078 analysis, section "1. aiter.py — LSE 반환과 ring 지원
// 선언").  Rows where every chunk is empty (all lse_i = -inf) give out = 0
// and lse = -inf.
//
// Memory-bound: each thread owns 8 consecutive elements of one row, reads
// them once from every chunk with 16- or 32-byte vector loads and writes the
// merged 8 once; the per-row LSEs are tiny and cached.  For up to four chunks
// every load (LSEs and partial outputs) is issued before any is used, so a
// thread waits for memory once instead of once per chunk plus once for the
// LSEs; more chunks take a loop.  The partials are read
// and the result written with non-temporal accesses: each byte is touched
// once, and the output then does not linger in the caches for the next kernel
// to write back (a decode after the merge ran 8% faster with them).
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NT = 256;

struct ChunkPtrs {
    const void* outs[kMaxMergeChunks];
    const float* lses[kMaxMergeChunks];
};

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[2 * j] = bf16_lo(w[j]); x[2 * j + 1] = bf16_hi(w[j]); }
    }
    static __device__ __forceinline__ void store(void* p, const float* x) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
    }
    static __device__ __forceinline__ void store(void* p, const float* x) {
        f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p) + 1);
    }
};

// NF > 0: exactly NF chunks, all loads issued up front; NF = 0: any n, one chunk at a time.
template <typename T, int NF>
__global__ __launch_bounds__(NT)
void merge_kernel(ChunkPtrs ptrs, int n, T* __restrict__ out, float* __restrict__ lse_out,
                  int rows, int D) {
    const int per_row = D / 8;
    if constexpr (NF > 0) {
        // rows * per_row < 2^32 here (checked by the launcher): 32-bit index arithmetic
        const uint32_t idx = blockIdx.x * (uint32_t)NT + threadIdx.x;
        const uint32_t row = idx / (uint32_t)per_row;
        const uint32_t ch = idx - row * (uint32_t)per_row;
        if (row >= (uint32_t)rows) return;
        const size_t off = (size_t)row * D + (size_t)ch * 8;
        float l[NF], x[NF][8];
#pragma unroll
        for (int i = 0; i < NF; ++i) l[i] = ptrs.lses[i][row];
#pragma unroll
        for (int i = 0; i < NF; ++i) Vec8<T>::load(static_cast<const T*>(ptrs.outs[i]) + off, x[i]);
        // No branch on the LSEs (selects only), so the compiler cannot sink the output loads
        // behind the LSE loads.
        float M = l[0];
#pragma unroll
        for (int i = 1; i < NF; ++i) M = fmaxf(M, l[i]);
        const bool empty = M == kNegInf;          // every chunk empty: out = 0, lse = -inf
        const float Ms = empty ? 0.f : M;
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NF; ++i) tot += __expf(l[i] - Ms);
        const float lse = empty ? kNegInf : Ms + __logf(tot);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const float w = empty ? 0.f : __expf(l[i] - lse);   // empty chunk: exp(-inf) = 0
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(w, x[i][j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = empty ? 0.f : acc[j];
        Vec8<T>::store(out + off, acc);
        if (lse_out && ch == 0) lse_out[row] = lse;
        return;
    }
    const long idx = (long)blockIdx.x * NT + threadIdx.x;
    const long row = idx / per_row;
    const int ch = (int)(idx - row * per_row);
    if (row >= rows) return;

    float M = kNegInf;
    for (int i = 0; i < n; ++i) M = fmaxf(M, ptrs.lses[i][row]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const size_t off = (size_t)row * D + (size_t)ch * 8;
    if (M == kNegInf) {
        Vec8<T>::store(out + off, acc);
        if (lse_out && ch == 0) lse_out[row] = kNegInf;
        return;
    }
    float tot = 0.f;
    for (int i = 0; i < n; ++i) tot += __expf(ptrs.lses[i][row] - M);
    const float lse = M + __logf(tot);
    for (int i = 0; i < n; ++i) {
        const float w = __expf(ptrs.lses[i][row] - lse);   // empty chunk: exp(-inf) = 0
        float x[8];
        Vec8<T>::load(static_cast<const T*>(ptrs.outs[i]) + off, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(w, x[j], acc[j]);
    }
    Vec8<T>::store(out + off, acc);
    if (lse_out && ch == 0) lse_out[row] = lse;
}

template <typename T>
hipError_t launch(const MergeArgs& a) {
    ChunkPtrs p;
    for (int i = 0; i < kMaxMergeChunks; ++i) {
        p.outs[i] = i < a.n ? a.outs[i] : nullptr;
        p.lses[i] = i < a.n ? a.lses[i] : nullptr;
    }
    const long threads = (long)a.rows * (a.D / 8);
    const long grid = (threads + NT - 1) / NT;
    const bool idx32 = grid * (long)NT <= 0xFFFFFFFFL;
    ATTN_CHECK(a.n >= 1 && a.n <= kMaxMergeChunks && a.D % 8 == 0, "chunk count and row width");
    ATTN_CHECK(grid >= 1 && grid <= 0xFFFFFFFFL && grid * (long)NT >= threads, "grid covers every row");
    const auto kern = !idx32 || a.n > 4 ? merge_kernel<T, 0>
                    : a.n == 1 ? merge_kernel<T, 1> : a.n == 2 ? merge_kernel<T, 2>
                    : a.n == 3 ? merge_kernel<T, 3> : merge_kernel<T, 4>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), 0, (hipStream_t)a.stream,
                       p, a.n, (T*)a.out, a.lse_out, a.rows, a.D);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_bf16(const MergeArgs& a) { return launch<bf16>(a); }
hipError_t launch_merge_f32(const MergeArgs& a) { return launch<float>(a); }

}  // namespace mattn
