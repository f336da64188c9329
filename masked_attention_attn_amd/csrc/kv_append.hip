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
#include "common.cuh"
#include "launch.h"

namespace mattn {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT)
void kv_append_kernel(unsigned char* __restrict__ kc, unsigned char* __restrict__ vc,
                      int32_t* __restrict__ lens, const unsigned char* __restrict__ kn,
                      const unsigned char* __restrict__ vn, int H_kv, int T_max, int row_bytes) {
    const int b = blockIdx.x;
    const int t = lens[b];
    const bool ok = t >= 0 && t < T_max;
    if (ok) {
        const int chunks = row_bytes / 16;            // per head
        const int total = 2 * H_kv * chunks;          // K then V
        for (int idx = threadIdx.x; idx < total; idx += NT) {
            const int which = idx / (H_kv * chunks);
            const int rem = idx - which * H_kv * chunks;
            const int g = rem / chunks, ch = rem - g * chunks;
            const size_t src = ((size_t)b * H_kv + g) * row_bytes + (size_t)ch * 16;
            const size_t dst = (((size_t)b * H_kv + g) * T_max + t) * row_bytes + (size_t)ch * 16;
            if (which == 0) stg128(kc + dst, ldg128(kn + src));
            else stg128(vc + dst, ldg128(vn + src));
        }
    }
    __syncthreads();
    if (ok && threadIdx.x == 0) lens[b] = t + 1;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a) {
    const int row_bytes = a.D * a.elem_bytes;
    hipLaunchKernelGGL(kv_append_kernel, dim3(a.B), dim3(NT), 0, (hipStream_t)a.stream,
                       (unsigned char*)a.k_cache, (unsigned char*)a.v_cache, a.lens,
                       (const unsigned char*)a.k_new, (const unsigned char*)a.v_new,
                       a.H_kv, a.T_max, row_bytes);
    return hipGetLastError();
}

}  // namespace mattn
