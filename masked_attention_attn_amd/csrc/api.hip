// C ABI entry points: host-side argument checks, dtype / head-dim dispatch,
// launch on the caller's stream.  Nothing here allocates, synchronises or
// keeps a pointer; every check runs before the first HIP call, so a rejected
// call enqueues nothing.
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "attn.h"
#include "launch.h"

using namespace mattn;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool head_dim_ok(int D) { return D == 64 || D == 128; }
bool dtype_ok(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_BF16; }
int elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

// Work counts are kept in int on the device side; refuse sizes whose element
// counts would not fit comfortably in 63 bits or whose grids overflow.
bool fits(long long a, long long b, long long c, long long d) {
    const long long lim = 1ll << 46;
    if (a <= 0 || b <= 0 || c <= 0 || d <= 0) return false;
    long long x = a;
    if ((x *= b) > lim || (x *= c) > lim || (x *= d) > lim) return false;
    return true;
}

int finish(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// A tensor's byte range, for the aliasing rule: no output may share a byte with an input
// or with another output (a null pointer or an empty range overlaps nothing).
struct Span {
    const void* p;
    long long n;
};
bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.n <= 0 || b.n <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.n && b0 < a0 + (uintptr_t)a.n;
}
// true if some output overlaps an input or another output
bool aliased(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlap(*o, i)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return true;
    }
    return false;
}

int fwd_common(const void* q, const void* k, const void* v, const uint8_t* mask, void* o,
               float* lse, bool need_lse, int B, int H, int H_kv, int Tq, int Tk, int D,
               bool causal, float scale, int dtype, void* stream) {
    if (!q || !k || !v || !o || (need_lse && !lse)) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    // grouped-query and causal attention run in the bf16 kernel only
    if ((causal || H_kv != H) && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (H_kv < 1 || H < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H, Tq, D) || !fits(B, H_kv, Tk, D) || (long long)B * H > (1ll << 24) ||
        (long long)B * H * ((Tq + 127) / 128) > (1ll << 31) - 64)
        return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    {
        const long long es = elem_bytes(dtype);
        const Span sq{q, (long long)B * H * Tq * D * es}, sk{k, (long long)B * H_kv * Tk * D * es},
            sv{v, (long long)B * H_kv * Tk * D * es}, sm{mask, mask ? (long long)B * Tk : 0};
        if (aliased({Span{o, sq.n}, Span{lse, lse ? (long long)B * H * Tq * 4 : 0}}, {sq, sk, sv, sm}))
            return ATTN_ERR_ALIAS;
    }
    // the bf16 kernel addresses one head's K/V through a 32-bit buffer range
    if (dtype == ATTN_BF16 && (long long)Tk * D * 2 > (1ll << 31) - 1) return ATTN_ERR_SHAPE;
    FwdArgs a{q, k, v, mask, o, lse, B, H, Tq, Tk, D, scale, stream};
    a.H_kv = H_kv;
    a.causal = causal;
    if (dtype == ATTN_F32) return finish(launch_fwd_f32(a));
    return finish(D == 64 ? launch_fwd_bf16_d64(a) : launch_fwd_bf16_d128(a));
}

int varlen_common(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, void* o, float* lse, int B, int H, int H_kv,
                  int total_q, int total_k, int max_seqlen_q, int D, bool causal, float scale,
                  int dtype, void* stream) {
    // with no keys at all (total_k = 0) k and v are never read and may be null
    if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || (total_k > 0 && (!k || !v))) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || total_q < 0 || total_k < 0 ||
        max_seqlen_q < 0 || max_seqlen_q > total_q)
        return ATTN_ERR_SHAPE;
    // One packed row is H·D elements; tile offsets of 64 rows must fit the 32-bit buffer offset.
    if ((long long)H * D > (1ll << 22) || (long long)total_q * H * D > (1ll << 31) - 1 ||
        (long long)total_k * H_kv * D > (1ll << 30) - 1 ||
        (long long)B * H * ((max_seqlen_q + 127) / 128) > (1ll << 31) - 64)
        return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    {
        const Span sq{q, (long long)total_q * H * D * 2}, sk{k, (long long)total_k * H_kv * D * 2},
            sv{v, (long long)total_k * H_kv * D * 2}, scq{cu_seqlens_q, (long long)(B + 1) * 4},
            sck{cu_seqlens_k, (long long)(B + 1) * 4};
        if (aliased({Span{o, sq.n}, Span{lse, lse ? (long long)H * total_q * 4 : 0}}, {sq, sk, sv, scq, sck}))
            return ATTN_ERR_ALIAS;
    }
    if (total_q == 0 || max_seqlen_q == 0) return ATTN_OK;      // no query rows: nothing to write
    FwdArgs a{q, k, v, nullptr, o, lse, B, H, max_seqlen_q, 0, D, scale, stream};
    a.H_kv = H_kv;
    a.causal = causal;
    a.varlen = true;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.total_q = total_q;
    a.total_k = total_k;
    return finish(D == 64 ? launch_fwd_bf16_d64(a) : launch_fwd_bf16_d128(a));
}

// 8-bit caches (E4M3 codes, or INT8 codes when int8): shared checks of the append and decode calls.
int q8_append(void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
              int32_t* cache_seqlens, const void* k_new, const void* v_new, int B, int H_kv, int T_max,
              int D, int new_dtype, void* stream, bool int8) {
    if (!k_cache || !v_cache || !k_scale || !v_scale || !cache_seqlens || !k_new || !v_new) return ATTN_ERR_NULL;
    if (!dtype_ok(new_dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (!fits(B, H_kv, T_max, D) || B > (1 << 30)) return ATTN_ERR_SHAPE;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return ATTN_ERR_ALIGN;
    {
        const long long cb = (long long)B * H_kv * T_max * D, nb = (long long)B * H_kv * D * elem_bytes(new_dtype);
        const long long sb = (long long)B * H_kv * 4;
        if (aliased({Span{k_cache, cb}, Span{v_cache, cb}, Span{cache_seqlens, (long long)B * 4}},
                    {Span{k_new, nb}, Span{v_new, nb}, Span{k_scale, sb}, Span{v_scale, sb}}))
            return ATTN_ERR_ALIAS;
    }
    AppendFp8Args a{k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new,
                    new_dtype == ATTN_BF16, B, H_kv, T_max, D, stream};
    a.int8 = int8;
    return finish(launch_kv_append_fp8(a));
}

int q8_decode(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
              const float* v_scale, const int32_t* cache_seqlens, void* o, float* lse, int B,
              int H_q, int H_kv, int T_max, int D, float scale, void* workspace,
              size_t workspace_bytes, void* stream, bool int8) {
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !cache_seqlens || !o) return ATTN_ERR_NULL;
    if (!head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (H_kv <= 0 || H_q <= 0 || H_q % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H_kv, T_max, D) || !fits(B, H_q, 1, D) || (long long)B * H_q > (1 << 30))
        return ATTN_ERR_SHAPE;
    // one (sequence, KV head) of codes is addressed through a 32-bit buffer range
    if ((long long)T_max * D > (1ll << 31) - 1) return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!workspace || workspace_bytes < decode_workspace_bytes(B, H_q, T_max, D)) return ATTN_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(workspace))
        return ATTN_ERR_ALIGN;
    {
        const long long qb = (long long)B * H_q * D * 2, cb = (long long)B * H_kv * T_max * D;
        const long long sb = (long long)B * H_kv * 4;
        if (aliased({Span{o, qb}, Span{lse, lse ? (long long)B * H_q * 4 : 0},
                     Span{workspace, (long long)workspace_bytes}},
                    {Span{q, qb}, Span{k_cache, cb}, Span{v_cache, cb}, Span{k_scale, sb}, Span{v_scale, sb},
                     Span{cache_seqlens, (long long)B * 4}}))
            return ATTN_ERR_ALIAS;
    }
    DecodeFp8Args a{q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D,
                    scale, workspace, stream};
    a.int8 = int8;
    return finish(launch_decode_fp8kv(a));
}

}  // namespace

extern "C" {

int attn_fwd_masked(const void* q, const void* k, const void* v, const uint8_t* key_padding_mask,
                    void* o, int B, int H, int Tq, int Tk, int D, float scale, int dtype,
                    void* stream) {
    return fwd_common(q, k, v, key_padding_mask, o, nullptr, false, B, H, H, Tq, Tk, D, false, scale,
                      dtype, stream);
}

int attn_fwd_lse(const void* q, const void* k, const void* v, const uint8_t* key_padding_mask,
                 void* o, float* lse, int B, int H, int Tq, int Tk, int D, float scale, int dtype,
                 void* stream) {
    return fwd_common(q, k, v, key_padding_mask, o, lse, true, B, H, H, Tq, Tk, D, false, scale,
                      dtype, stream);
}

int attn_prefill(const void* q, const void* k, const void* v, const uint8_t* key_padding_mask,
                 void* o, float* lse, int B, int H_q, int H_kv, int Tq, int Tk, int D, int causal,
                 float scale, int dtype, void* stream) {
    return fwd_common(q, k, v, key_padding_mask, o, lse, false, B, H_q, H_kv, Tq, Tk, D,
                      causal != 0, scale, dtype, stream);
}

int attn_prefill_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, void* o, float* lse, int B, int H_q, int H_kv,
                        int total_q, int total_k, int max_seqlen_q, int D, int causal, float scale,
                        int dtype, void* stream) {
    return varlen_common(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, B, H_q, H_kv, total_q, total_k,
                         max_seqlen_q, D, causal != 0, scale, dtype, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, void* o, float* lse, int B, int H, int total_q,
                    int total_k, int max_seqlen_q, int D, float scale, int dtype, void* stream) {
    return varlen_common(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, B, H, H, total_q, total_k,
                         max_seqlen_q, D, false, scale, dtype, stream);
}

int attn_merge_lse(int n_chunks, const void* const* outs, const float* const* lses, void* out,
                   float* lse_out, int B, int H, int T, int D, int dtype, void* stream) {
    if (!outs || !lses || !out) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (n_chunks < 1) return ATTN_ERR_SHAPE;
    if (n_chunks > kMaxMergeChunks) return ATTN_ERR_UNSUPPORTED;
    if (!fits(B, H, T, D) || (long long)B * H * T > (1ll << 31) - 1) return ATTN_ERR_SHAPE;
    if (!aligned16(out)) return ATTN_ERR_ALIGN;
    MergeArgs a{};
    a.n = n_chunks;
    for (int i = 0; i < n_chunks; ++i) {
        if (!outs[i] || !lses[i]) return ATTN_ERR_NULL;
        if (!aligned16(outs[i])) return ATTN_ERR_ALIGN;
        const long long ob = (long long)B * H * T * D * elem_bytes(dtype), lb = (long long)B * H * T * 4;
        if (aliased({Span{out, ob}, Span{lse_out, lse_out ? lb : 0}}, {Span{outs[i], ob}, Span{lses[i], lb}}))
            return ATTN_ERR_ALIAS;
        a.outs[i] = outs[i];
        a.lses[i] = lses[i];
    }
    a.out = out;
    a.lse_out = lse_out;
    a.rows = B * H * T;
    a.D = D;
    a.stream = stream;
    return finish(dtype == ATTN_BF16 ? launch_merge_bf16(a) : launch_merge_f32(a));
}

int kv_append(void* k_cache, void* v_cache, int32_t* cache_seqlens, const void* k_new,
              const void* v_new, int B, int H_kv, int T_max, int D, int dtype, void* stream) {
    if (!k_cache || !v_cache || !cache_seqlens || !k_new || !v_new) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (!fits(B, H_kv, T_max, D) || B > (1 << 30)) return ATTN_ERR_SHAPE;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return ATTN_ERR_ALIGN;
    {
        const long long cb = (long long)B * H_kv * T_max * D * elem_bytes(dtype);
        const long long nb = (long long)B * H_kv * D * elem_bytes(dtype);
        if (aliased({Span{k_cache, cb}, Span{v_cache, cb}, Span{cache_seqlens, (long long)B * 4}},
                    {Span{k_new, nb}, Span{v_new, nb}}))
            return ATTN_ERR_ALIAS;
    }
    AppendArgs a{k_cache, v_cache, cache_seqlens, k_new, v_new, B, H_kv, T_max, D,
                 elem_bytes(dtype), stream};
    return finish(launch_kv_append(a));
}

// Shared checks of the paged pool geometry: page_size a power of two in [16, 2^20],
// capacity max_pages * page_size within the contiguous decode's limits, and the
// block table (B x max_pages int32) addressable with 32-bit byte offsets.
static int paged_geometry(int B, int H_kv, int num_pages, int page_size, int max_pages, int D,
                          int& T_max) {
    if (num_pages < 1 || max_pages < 1 || page_size < 16 || page_size > (1 << 20) ||
        (page_size & (page_size - 1)) != 0)
        return ATTN_ERR_SHAPE;
    const long long cap = (long long)max_pages * page_size;
    if (cap > (1ll << 30) || (long long)B * max_pages > (1ll << 29) ||
        !fits(num_pages, H_kv, page_size, D))
        return ATTN_ERR_SHAPE;
    T_max = (int)cap;
    return ATTN_OK;
}

// 8-bit paged pools: shared checks of the append and decode calls.
static int q8_append_paged(void* k_pages, void* v_pages, const float* k_scale, const float* v_scale,
                           const int32_t* block_table, int32_t* cache_seqlens, const void* k_new,
                           const void* v_new, int B, int H_kv, int num_pages, int page_size, int max_pages,
                           int D, int new_dtype, void* stream, bool int8) {
    if (!k_pages || !v_pages || !k_scale || !v_scale || !block_table || !cache_seqlens || !k_new || !v_new)
        return ATTN_ERR_NULL;
    if (!dtype_ok(new_dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (B < 1 || H_kv < 1 || B > (1 << 30)) return ATTN_ERR_SHAPE;
    int T_max = 0;
    if (const int st = paged_geometry(B, H_kv, num_pages, page_size, max_pages, D, T_max)) return st;
    if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_new) || !aligned16(v_new))
        return ATTN_ERR_ALIGN;
    {
        const long long pb = (long long)num_pages * H_kv * page_size * D;
        const long long nb = (long long)B * H_kv * D * elem_bytes(new_dtype), sb = (long long)B * H_kv * 4;
        if (aliased({Span{k_pages, pb}, Span{v_pages, pb}, Span{cache_seqlens, (long long)B * 4}},
                    {Span{k_new, nb}, Span{v_new, nb}, Span{k_scale, sb}, Span{v_scale, sb},
                     Span{block_table, (long long)B * max_pages * 4}}))
            return ATTN_ERR_ALIAS;
    }
    AppendFp8Args a{k_pages, v_pages, k_scale, v_scale, cache_seqlens, k_new, v_new,
                    new_dtype == ATTN_BF16, B, H_kv, T_max, D, stream};
    a.int8 = int8;
    a.block_table = block_table;
    a.page_size = page_size;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    return finish(launch_kv_append_fp8(a));
}

static int q8_decode_paged(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                           const float* v_scale, const int32_t* block_table, const int32_t* cache_seqlens,
                           void* o, float* lse, int B, int H_q, int H_kv, int num_pages, int page_size,
                           int max_pages, int D, float scale, void* workspace, size_t workspace_bytes,
                           void* stream, bool int8) {
    if (!q || !k_pages || !v_pages || !k_scale || !v_scale || !block_table || !cache_seqlens || !o)
        return ATTN_ERR_NULL;
    if (!head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (H_kv <= 0 || H_q <= 0 || H_q % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H_q, 1, D) || (long long)B * H_q > (1 << 30)) return ATTN_ERR_SHAPE;
    int T_max = 0;
    if (const int st = paged_geometry(B, H_kv, num_pages, page_size, max_pages, D, T_max)) return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!workspace || workspace_bytes < decode_workspace_bytes(B, H_q, T_max, D)) return ATTN_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(workspace))
        return ATTN_ERR_ALIGN;
    {
        const long long qb = (long long)B * H_q * D * 2, pb = (long long)num_pages * H_kv * page_size * D;
        const long long sb = (long long)B * H_kv * 4;
        if (aliased({Span{o, qb}, Span{lse, lse ? (long long)B * H_q * 4 : 0},
                     Span{workspace, (long long)workspace_bytes}},
                    {Span{q, qb}, Span{k_pages, pb}, Span{v_pages, pb}, Span{k_scale, sb}, Span{v_scale, sb},
                     Span{block_table, (long long)B * max_pages * 4}, Span{cache_seqlens, (long long)B * 4}}))
            return ATTN_ERR_ALIAS;
    }
    DecodeFp8Args a{q, k_pages, v_pages, k_scale, v_scale, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D,
                    scale, workspace, stream};
    a.int8 = int8;
    a.block_table = block_table;
    a.page_size = page_size;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    return finish(launch_decode_fp8kv(a));
}

int kv_append_paged(void* k_pages, void* v_pages, const int32_t* block_table, int32_t* cache_seqlens,
                    const void* k_new, const void* v_new, int B, int H_kv, int num_pages,
                    int page_size, int max_pages_per_seq, int D, int dtype, void* stream) {
    if (!k_pages || !v_pages || !block_table || !cache_seqlens || !k_new || !v_new) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    int T_max = 0;
    if (B < 1 || H_kv < 1 || B > (1 << 30)) return ATTN_ERR_SHAPE;
    if (const int st = paged_geometry(B, H_kv, num_pages, page_size, max_pages_per_seq, D, T_max))
        return st;
    if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_new) || !aligned16(v_new))
        return ATTN_ERR_ALIGN;
    {
        const long long pb = (long long)num_pages * H_kv * page_size * D * elem_bytes(dtype);
        const long long nb = (long long)B * H_kv * D * elem_bytes(dtype);
        if (aliased({Span{k_pages, pb}, Span{v_pages, pb}, Span{cache_seqlens, (long long)B * 4}},
                    {Span{k_new, nb}, Span{v_new, nb}, Span{block_table, (long long)B * max_pages_per_seq * 4}}))
            return ATTN_ERR_ALIAS;
    }
    AppendArgs a{k_pages, v_pages, cache_seqlens, k_new, v_new, B, H_kv, T_max, D,
                 elem_bytes(dtype), stream};
    a.block_table = block_table;
    a.page_size = page_size;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    return finish(launch_kv_append(a));
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* cache_seqlens, void* o, float* lse,
                      int B, int H_q, int H_kv, int num_pages, int page_size, int max_pages_per_seq,
                      int D, float scale, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
    if (!q || !k_pages || !v_pages || !block_table || !cache_seqlens || !o) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (H_kv <= 0 || H_q <= 0 || H_q % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H_q, 1, D) || (long long)B * H_q > (1 << 30)) return ATTN_ERR_SHAPE;
    int T_max = 0;
    if (const int st = paged_geometry(B, H_kv, num_pages, page_size, max_pages_per_seq, D, T_max))
        return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!workspace || workspace_bytes < decode_workspace_bytes(B, H_q, T_max, D))
        return ATTN_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
        !aligned16(workspace))
        return ATTN_ERR_ALIGN;
    {
        const long long qb = (long long)B * H_q * D * 2, pb = (long long)num_pages * H_kv * page_size * D * 2;
        if (aliased({Span{o, qb}, Span{lse, lse ? (long long)B * H_q * 4 : 0},
                     Span{workspace, (long long)workspace_bytes}},
                    {Span{q, qb}, Span{k_pages, pb}, Span{v_pages, pb},
                     Span{block_table, (long long)B * max_pages_per_seq * 4}, Span{cache_seqlens, (long long)B * 4}}))
            return ATTN_ERR_ALIAS;
    }
    DecodeArgs a{q, k_pages, v_pages, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                 workspace, stream};
    a.block_table = block_table;
    a.page_size = page_size;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    return finish(launch_decode_bf16(a));
}

int kv_append_fp8(void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                  int32_t* cache_seqlens, const void* k_new, const void* v_new, int B, int H_kv, int T_max,
                  int D, int new_dtype, void* stream) {
    return q8_append(k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new, B, H_kv, T_max, D,
                     new_dtype, stream, false);
}

int kv_append_int8(void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                   int32_t* cache_seqlens, const void* k_new, const void* v_new, int B, int H_kv, int T_max,
                   int D, int new_dtype, void* stream) {
    return q8_append(k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new, B, H_kv, T_max, D,
                     new_dtype, stream, true);
}

int attn_decode_fp8kv(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const int32_t* cache_seqlens, void* o, float* lse, int B,
                      int H_q, int H_kv, int T_max, int D, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return q8_decode(q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                     workspace, workspace_bytes, stream, false);
}

int attn_decode_int8kv(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                       const float* v_scale, const int32_t* cache_seqlens, void* o, float* lse, int B,
                       int H_q, int H_kv, int T_max, int D, float scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return q8_decode(q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                     workspace, workspace_bytes, stream, true);
}


int kv_append_fp8_paged(void* k_pages, void* v_pages, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t* cache_seqlens, const void* k_new, const void* v_new,
                        int B, int H_kv, int num_pages, int page_size, int max_pages_per_seq, int D,
                        int new_dtype, void* stream) {
    return q8_append_paged(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, k_new, v_new, B, H_kv,
                           num_pages, page_size, max_pages_per_seq, D, new_dtype, stream, false);
}

int kv_append_int8_paged(void* k_pages, void* v_pages, const float* k_scale, const float* v_scale,
                         const int32_t* block_table, int32_t* cache_seqlens, const void* k_new, const void* v_new,
                         int B, int H_kv, int num_pages, int page_size, int max_pages_per_seq, int D,
                         int new_dtype, void* stream) {
    return q8_append_paged(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, k_new, v_new, B, H_kv,
                           num_pages, page_size, max_pages_per_seq, D, new_dtype, stream, true);
}

int attn_decode_fp8kv_paged(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                            const float* v_scale, const int32_t* block_table, const int32_t* cache_seqlens,
                            void* o, float* lse, int B, int H_q, int H_kv, int num_pages, int page_size,
                            int max_pages_per_seq, int D, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return q8_decode_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, o, lse, B, H_q, H_kv,
                           num_pages, page_size, max_pages_per_seq, D, scale, workspace, workspace_bytes, stream,
                           false);
}

int attn_decode_int8kv_paged(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                             const float* v_scale, const int32_t* block_table, const int32_t* cache_seqlens,
                             void* o, float* lse, int B, int H_q, int H_kv, int num_pages, int page_size,
                             int max_pages_per_seq, int D, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return q8_decode_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, o, lse, B, H_q, H_kv,
                           num_pages, page_size, max_pages_per_seq, D, scale, workspace, workspace_bytes, stream,
                           true);
}

int attn_prefill_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                     const float* k_scale, const float* v_scale, const uint8_t* key_padding_mask, void* o,
                     float* lse, int B, int H_q, int H_kv, int Tq, int Tk, int D, int causal, float scale,
                     void* stream) {
    if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !o) return ATTN_ERR_NULL;
    if (!head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H_q, Tq, D) || !fits(B, H_kv, Tk, D) || (long long)B * H_q > (1ll << 24) ||
        (long long)B * H_q * ((Tq + 127) / 128) > (1ll << 31) - 64)
        return ATTN_ERR_SHAPE;
    // one (sequence, KV head) of codes is addressed through a 32-bit buffer range
    if ((long long)Tk * D > (1ll << 31) - 1) return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    {
        const long long qb = (long long)B * H_q * Tq * D, kb = (long long)B * H_kv * Tk * D;
        if (aliased({Span{o, qb * 2}, Span{lse, lse ? (long long)B * H_q * Tq * 4 : 0}},
                    {Span{q, qb}, Span{k, kb}, Span{v, kb}, Span{q_scale, (long long)B * H_q * 4},
                     Span{k_scale, (long long)B * H_kv * 4}, Span{v_scale, (long long)B * H_kv * 4},
                     Span{key_padding_mask, key_padding_mask ? (long long)B * Tk : 0}}))
            return ATTN_ERR_ALIAS;
    }
    FwdArgs a{q, k, v, key_padding_mask, o, lse, B, H_q, Tq, Tk, D, scale, stream};
    a.H_kv = H_kv;
    a.causal = causal != 0;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return finish(D == 64 ? launch_fwd_fp8_d64(a) : launch_fwd_fp8_d128(a));
}

int attn_prefill_varlen_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                            const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, void* o, float* lse, int B, int H_q, int H_kv,
                            int total_q, int total_k, int max_seqlen_q, int D, int causal, float scale,
                            void* stream) {
    // with no keys at all (total_k = 0) k and v are never read and may be null
    if (!q || !q_scale || !k_scale || !v_scale || !o || !cu_seqlens_q || !cu_seqlens_k ||
        (total_k > 0 && (!k || !v)))
        return ATTN_ERR_NULL;
    if (!head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 ||
        max_seqlen_q > total_q)
        return ATTN_ERR_SHAPE;
    // as the bf16 packed call: one packed row is H·D codes, and tile offsets of 64 rows fit the
    // 32-bit buffer offset (the O rows are bf16, so the same element bounds hold)
    if ((long long)H_q * D > (1ll << 22) || (long long)total_q * H_q * D > (1ll << 31) - 1 ||
        (long long)total_k * H_kv * D > (1ll << 30) - 1 ||
        (long long)B * H_q * ((max_seqlen_q + 127) / 128) > (1ll << 31) - 64)
        return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    {
        const long long qb = (long long)total_q * H_q * D, kb = (long long)total_k * H_kv * D;
        if (aliased({Span{o, qb * 2}, Span{lse, lse ? (long long)H_q * total_q * 4 : 0}},
                    {Span{q, qb}, Span{k, kb}, Span{v, kb}, Span{q_scale, (long long)B * H_q * 4},
                     Span{k_scale, (long long)B * H_kv * 4}, Span{v_scale, (long long)B * H_kv * 4},
                     Span{cu_seqlens_q, (long long)(B + 1) * 4}, Span{cu_seqlens_k, (long long)(B + 1) * 4}}))
            return ATTN_ERR_ALIAS;
    }
    if (total_q == 0 || max_seqlen_q == 0) return ATTN_OK;      // no query rows: nothing to write
    FwdArgs a{q, k, v, nullptr, o, lse, B, H_q, max_seqlen_q, 0, D, scale, stream};
    a.H_kv = H_kv;
    a.causal = causal != 0;
    a.varlen = true;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.total_q = total_q;
    a.total_k = total_k;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return finish(D == 64 ? launch_fwd_fp8_d64(a) : launch_fwd_fp8_d128(a));
}

size_t attn_decode_workspace_bytes(int B, int H_q, int H_kv, int T_max, int D) {
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || T_max <= 0 || !head_dim_ok(D) || H_q % H_kv != 0)
        return 0;
    return decode_workspace_bytes(B, H_q, T_max, D);
}

}  // extern "C"

namespace {

// The argument checks of attn_decode and attn_decode_noalloc.  caller_ws = false skips the
// workspace checks (the no-allocation call brings its own).
int decode_checks(const void* q, const void* k_cache, const void* v_cache, const int32_t* cache_seqlens,
                  void* o, float* lse, int B, int H_q, int H_kv, int T_max, int D, float scale, int dtype,
                  bool caller_ws, void* workspace, size_t workspace_bytes) {
    if (!q || !k_cache || !v_cache || !cache_seqlens || !o) return ATTN_ERR_NULL;
    if (!dtype_ok(dtype) || !head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
    if (H_kv <= 0 || H_q <= 0 || H_q % H_kv != 0) return ATTN_ERR_SHAPE;
    if (!fits(B, H_kv, T_max, D) || !fits(B, H_q, 1, D) || (long long)B * H_q > (1 << 30))
        return ATTN_ERR_SHAPE;
    if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_VALUE;
    if (caller_ws && (!workspace || workspace_bytes < decode_workspace_bytes(B, H_q, T_max, D)))
        return ATTN_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (workspace && !aligned16(workspace)))
        return ATTN_ERR_ALIGN;
    {
        const long long es = elem_bytes(dtype);
        const long long qb = (long long)B * H_q * D * es, cb = (long long)B * H_kv * T_max * D * es;
        if (aliased({Span{o, qb}, Span{lse, lse ? (long long)B * H_q * 4 : 0},
                     Span{workspace, (long long)workspace_bytes}},
                    {Span{q, qb}, Span{k_cache, cb}, Span{v_cache, cb}, Span{cache_seqlens, (long long)B * 4}}))
            return ATTN_ERR_ALIAS;
    }
    // the bf16 kernel addresses one (sequence, KV head) through a 32-bit buffer range
    if (dtype == ATTN_BF16 && (long long)T_max * D * 2 > (1ll << 31) - 1) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

// Scratch of attn_decode_noalloc: the decode's partial results (the workspace of attn_decode)
// in a file-scope device array, one copy per GPU that the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: each device's address
// comes from hipGetSymbolAddress, taken once with that device current.
constexpr size_t kNoallocScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_addr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// This device's address of `scratch`, or null (then *err says why).
void* scratch_on_current_device(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(scratch_once[dev], [dev] {
        void* p = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        scratch_addr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *err = scratch_err[dev];
    return scratch_addr[dev];
}

}  // namespace

extern "C" {

int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* cache_seqlens, void* o, float* lse, int B, int H_q, int H_kv,
                int T_max, int D, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (const int st = decode_checks(q, k_cache, v_cache, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                                     dtype, true, workspace, workspace_bytes))
        return st;
    DecodeArgs a{q, k_cache, v_cache, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                 workspace, stream};
    return finish(dtype == ATTN_BF16 ? launch_decode_bf16(a) : launch_decode_f32(a));
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_seqlens, void* o, float* lse, int B, int H_q, int H_kv,
                        int T_max, int D, float scale, int dtype, void* stream) {
    if (const int st = decode_checks(q, k_cache, v_cache, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale,
                                     dtype, false, nullptr, 0))
        return st;
    if (decode_workspace_bytes(B, H_q, T_max, D) > kNoallocScratchBytes) return ATTN_ERR_SCRATCH;
    hipError_t err;
    void* ws = scratch_on_current_device(&err);
    if (!ws) return ATTN_ERR_LAUNCH;
    DecodeArgs a{q, k_cache, v_cache, cache_seqlens, o, lse, B, H_q, H_kv, T_max, D, scale, ws, stream};
    return finish(dtype == ATTN_BF16 ? launch_decode_bf16(a) : launch_decode_f32(a));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "a size is out of range or inconsistent";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or chunk count";
        case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_VALUE: return "scale must be finite and > 0";
        case ATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_SCRATCH: return "the problem needs more scratch than the static no-allocation buffer holds";
        default: return "unknown status";
    }
}

}  // extern "C"
