// Append one token per sequence to preallocated K/V caches.
//
// Decode computes K and V for the newest token only and adds them to the
// per-layer cache of shape (batch, heads, seq_len_cached, head_dim)
// (agentlenshq.com, "nanoVLM에서 KV 캐시 구현", sections "KV 캐싱이 추론을
// 최적화하는 방법" and "1. 어텐션 블록 업데이트").  With a cache of fixed
// capacity T_max, concatenation becomes a write at slot len_b followed by
// len_b += 1.
//
// One workgroup per sequence: every thread copies 16-byte chunks of the new
// K and V rows of all KV heads to slot len_b, then, after a barrier that
// orders every read of len_b before the write, thread 0 increments it.  A
// sequence whose length is outside [0, T_max) is left untouched.
//
// Paged cache (LLM inference memory accounting 2/10, section "15. Paged KV
// Cache가 해결하는 것": logical blocks of a sequence map to physical blocks of a
// shared pool through its block-table row): the pools are [num_pages, H_kv,
// page_size, D], slot t is row t % page_size of page block_table[b][t /
// page_size], and T_max = max_pages * page_size.  Table entries are clamped
// to [0, num_pages), so a bad entry writes a wrong page but never outside
// the pool.
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NT = 256;

template <bool PAGED>
__global__ __launch_bounds__(NT)
void kv_append_kernel(unsigned char* __restrict__ kc, unsigned char* __restrict__ vc,
                      int32_t* __restrict__ lens, const unsigned char* __restrict__ kn,
                      const unsigned char* __restrict__ vn, int H_kv, int T_max, int row_bytes,
                      const int32_t* __restrict__ block_table, int page_size, int max_pages,
                      int num_pages) {
    const int b = blockIdx.x;
    const int t = lens[b];
    const bool ok = t >= 0 && t < T_max;
    if (ok) {
        // element offset of slot t of head 0 and the stride between heads, in rows
        size_t row0, head_rows;
        if constexpr (PAGED) {
            const int e = block_table[(size_t)b * max_pages + t / page_size];
            const int page = min(max(e, 0), num_pages - 1);
            row0 = (size_t)page * H_kv * page_size + t % page_size;
            head_rows = (size_t)page_size;
        } else {
            row0 = (size_t)b * H_kv * T_max + t;
            head_rows = (size_t)T_max;
        }
        const int chunks = row_bytes / 16;            // per head
        const int total = 2 * H_kv * chunks;          // K then V
        for (int idx = threadIdx.x; idx < total; idx += NT) {
            const int which = idx / (H_kv * chunks);
            const int rem = idx - which * H_kv * chunks;
            const int g = rem / chunks, ch = rem - g * chunks;
            const size_t src = ((size_t)b * H_kv + g) * row_bytes + (size_t)ch * 16;
            const size_t dst = (row0 + g * head_rows) * row_bytes + (size_t)ch * 16;
            if (which == 0) stg128(kc + dst, ldg128(kn + src));
            else stg128(vc + dst, ldg128(vn + src));
        }
    }
    __syncthreads();
    if (ok && threadIdx.x == 0) lens[b] = t + 1;
}

// 8-bit caches: the new token's elements are quantised with the (b, KV head)
// scale, after an IEEE float32 division y = x / scale: E4M3 codes as
// E4M3(clamp(y, -448, 448)) (round to nearest, ties to even), INT8 codes as
// clamp(rint(y), -127, 127) (nearest integer, ties to even; symmetric INT8 is
// one of the cache formats of LLM inference memory accounting 2/10, section
// "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").  Four elements per thread become one
// dword of codes (element i in byte i).
// PAGED: the pools and slot mapping of kv_append_kernel's paged form.
template <bool INT8, bool PAGED>
__global__ __launch_bounds__(NT)
void kv_append_q8_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                          const float* __restrict__ ks, const float* __restrict__ vs,
                          int32_t* __restrict__ lens, const void* __restrict__ kn,
                          const void* __restrict__ vn, int new_bf16, int H_kv, int T_max, int D,
                          const int32_t* __restrict__ block_table, int page_size, int max_pages,
                          int num_pages) {
    const int b = blockIdx.x;
    const int t = lens[b];
    const bool ok = t >= 0 && t < T_max;
    if (ok) {
        size_t row0, head_rows;       // row of slot t in head 0, rows between heads
        if constexpr (PAGED) {
            const int e = block_table[(size_t)b * max_pages + t / page_size];
            const int page = min(max(e, 0), num_pages - 1);
            row0 = (size_t)page * H_kv * page_size + t % page_size;
            head_rows = (size_t)page_size;
        } else {
            row0 = (size_t)b * H_kv * T_max + t;
            head_rows = (size_t)T_max;
        }
        const int quads = D / 4;
        const int total = 2 * H_kv * quads;          // K then V
        for (int idx = threadIdx.x; idx < total; idx += NT) {
            const int which = idx / (H_kv * quads);
            const int rem = idx - which * H_kv * quads;
            const int g = rem / quads, qd = rem - g * quads;
            const float s = (which ? vs : ks)[b * H_kv + g];
            const size_t e0 = ((size_t)b * H_kv + g) * D + (size_t)qd * 4;
            const void* src = which ? vn : kn;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = new_bf16 ? (float)reinterpret_cast<const bf16*>(src)[e0 + e]
                                : reinterpret_cast<const float*>(src)[e0 + e];
            int wd;
            if constexpr (INT8) {       // nearest integer (ties to even), clamped to +-127
                uint32_t u = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = fminf(fmaxf(__builtin_rintf(__fdiv_rn(x[e], s)), -127.0f), 127.0f);
                    u |= ((uint32_t)(int)y & 0xFFu) << (8 * e);
                }
                wd = (int)u;
            } else {                    // clamped to +-448, nearest E4M3 value (ties to even)
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(__fdiv_rn(x[e], s), -448.0f), 448.0f);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wd, true);
            }
            uint8_t* dst = (which ? vc : kc) + (row0 + g * head_rows) * D + (size_t)qd * 4;
            *reinterpret_cast<uint32_t*>(dst) = (uint32_t)wd;
        }
    }
    __syncthreads();
    if (ok && threadIdx.x == 0) lens[b] = t + 1;
}

}  // namespace

hipError_t launch_kv_append_fp8(const AppendFp8Args& a) {
    ATTN_CHECK(a.B >= 1 && a.B <= kMaxGrid && a.D % 16 == 0, "one workgroup per sequence, whole 16-code rows");
    ATTN_CHECK(!a.block_table || (long long)a.max_pages * a.page_size == a.T_max, "paged capacity");
    auto kern = a.block_table ? (a.int8 ? kv_append_q8_kernel<true, true> : kv_append_q8_kernel<false, true>)
                              : (a.int8 ? kv_append_q8_kernel<true, false> : kv_append_q8_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3(a.B), dim3(NT), 0, (hipStream_t)a.stream,
                       (uint8_t*)a.k_cache, (uint8_t*)a.v_cache, a.k_scale, a.v_scale, a.lens, a.k_new,
                       a.v_new, a.new_bf16 ? 1 : 0, a.H_kv, a.T_max, a.D, a.block_table, a.page_size,
                       a.max_pages, a.num_pages);
    return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a) {
    const int row_bytes = a.D * a.elem_bytes;
    ATTN_CHECK(a.B >= 1 && a.B <= kMaxGrid && row_bytes % 16 == 0, "one workgroup per sequence, 16-byte rows");
    ATTN_CHECK(!a.block_table || (long long)a.max_pages * a.page_size == a.T_max, "paged capacity");
    if (a.block_table)
        hipLaunchKernelGGL(kv_append_kernel<true>, dim3(a.B), dim3(NT), 0, (hipStream_t)a.stream,
                           (unsigned char*)a.k_cache, (unsigned char*)a.v_cache, a.lens,
                           (const unsigned char*)a.k_new, (const unsigned char*)a.v_new,
                           a.H_kv, a.T_max, row_bytes, a.block_table, a.page_size, a.max_pages,
                           a.num_pages);
    else
        hipLaunchKernelGGL(kv_append_kernel<false>, dim3(a.B), dim3(NT), 0, (hipStream_t)a.stream,
                           (unsigned char*)a.k_cache, (unsigned char*)a.v_cache, a.lens,
                           (const unsigned char*)a.k_new, (const unsigned char*)a.v_new,
                           a.H_kv, a.T_max, row_bytes, nullptr, 0, 0, 0);
    return hipGetLastError();
}

}  // namespace mattn
