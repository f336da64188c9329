// Internal launchers behind the C ABI.  Arguments are already validated by
// the API layer; each launcher enqueues its kernels on `stream` and returns
// hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "debug_checks.h"

namespace mattn {

struct FwdArgs {
    const void* q; const void* k; const void* v;
    const uint8_t* mask;
    void* o; float* lse;          // lse may be null
    int B, H, Tq, Tk, D;          // varlen: B sequences, Tq = the longest query sequence
    float scale;
    void* stream;
    // grouped-query attention: K/V have H_kv heads (0 = H); query head h reads h / (H / H_kv)
    int H_kv = 0;
    // causal: query i sees keys j <= i + (Tk - Tq) of its sequence (bf16 only)
    bool causal = false;
    // packed variable-length layout ([total, H, D], offsets in cu_q / cu_k)
    bool varlen = false;
    const int32_t* cu_q = nullptr;
    const int32_t* cu_k = nullptr;
    int total_q = 0, total_k = 0;
    // E4M3 inputs (launch_fwd_fp8_*): q, k, v are codes; q_scale [B, H], k_scale and
    // v_scale [B, H_kv] float32
    const float* q_scale = nullptr;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;
};

constexpr int kMaxMergeChunks = 32;

struct MergeArgs {
    int n;
    const void* outs[kMaxMergeChunks];
    const float* lses[kMaxMergeChunks];
    void* out; float* lse_out;    // lse_out may be null
    int rows, D;                  // rows = B*H*T
    void* stream;
};

struct AppendArgs {
    void* k_cache; void* v_cache; int32_t* lens;
    const void* k_new; const void* v_new;
    int B, H_kv, T_max, D, elem_bytes;
    void* stream;
    // paged cache: k_cache / v_cache are pools [num_pages, H_kv, page_size, D] and token t
    // of sequence b sits at row t % page_size of page block_table[b * max_pages + t / page_size]
    // (T_max = max_pages * page_size)
    const int32_t* block_table = nullptr;
    int page_size = 0, max_pages = 0, num_pages = 0;
};

struct DecodeArgs {
    const void* q; const void* k_cache; const void* v_cache;
    const int32_t* lens;
    void* o; float* lse;          // lse may be null
    int B, H_q, H_kv, T_max, D;
    float scale;
    void* workspace;
    void* stream;
    // paged cache, as in AppendArgs (page_size a power of two >= 16 here)
    const int32_t* block_table = nullptr;
    int page_size = 0, max_pages = 0, num_pages = 0;
};

// 8-bit cache: E4M3 codes (or INT8 when int8) [B, H_kv, T_max, D], one float32 scale per
// (b, KV head) for K and for V; q, o bf16.
struct DecodeFp8Args {
    const void* q; const void* k_cache; const void* v_cache;
    const float* k_scale; const float* v_scale;
    const int32_t* lens;
    void* o; float* lse;          // lse may be null
    int B, H_q, H_kv, T_max, D;
    float scale;
    void* workspace;
    void* stream;
    bool int8 = false;
    // paged pools, as in DecodeArgs
    const int32_t* block_table = nullptr;
    int page_size = 0, max_pages = 0, num_pages = 0;
};

struct AppendFp8Args {
    void* k_cache; void* v_cache;
    const float* k_scale; const float* v_scale;
    int32_t* lens;
    const void* k_new; const void* v_new;   // [B, H_kv, 1, D], bf16 or float32
    bool new_bf16;
    int B, H_kv, T_max, D;
    void* stream;
    bool int8 = false;            // symmetric INT8 codes instead of E4M3
    // paged pools, as in AppendArgs
    const int32_t* block_table = nullptr;
    int page_size = 0, max_pages = 0, num_pages = 0;
};

hipError_t launch_fwd_bf16_d64(const FwdArgs& a);
hipError_t launch_fwd_bf16_d128(const FwdArgs& a);
hipError_t launch_fwd_fp8_d64(const FwdArgs& a);
hipError_t launch_fwd_fp8_d128(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_merge_bf16(const MergeArgs& a);
hipError_t launch_merge_f32(const MergeArgs& a);
hipError_t launch_kv_append(const AppendArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a);
hipError_t launch_decode_f32(const DecodeArgs& a);
hipError_t launch_decode_fp8kv(const DecodeFp8Args& a);
hipError_t launch_kv_append_fp8(const AppendFp8Args& a);

// Split-K geometry of the decode path (shared by the workspace-size query
// and the launcher).
constexpr int kDecodeSplit = 1024;    // cached tokens per split
inline int decode_nsplit(int T_max) { return (T_max + kDecodeSplit - 1) / kDecodeSplit; }
// Two partial results per (sequence, query head, split): a split is shared by
// at most two wavefronts of the bf16 stream kernel.
inline size_t decode_workspace_bytes(int B, int H_q, int T_max, int D) {
    const size_t parts = (size_t)B * H_q * decode_nsplit(T_max) * 2;
    return parts * (size_t)D * sizeof(float) + parts * 2 * sizeof(float);
}

}  // namespace mattn
