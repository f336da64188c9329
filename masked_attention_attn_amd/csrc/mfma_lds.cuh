// Device helpers shared by the matrix-core attention kernels (prefill and
// decode): buffer descriptors, direct global->LDS tile loads, the gfx950
// transposing LDS read and lane-pair reductions of the 32x32 MFMA layout.
#pragma once

#include "common.cuh"

namespace mattn {
namespace mfma {

__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// XOR swizzles of the 16-byte chunk index in LDS rows of D bf16 (2D bytes; the
// LDS serves 64 banks of 4 bytes per pass).  Chunk c of row r sits at
// c ^ k_swz(r) in a K tile and at c ^ v_swz(r) in a V tile, which makes the
// K operand reads and the transposing Vᵀ reads (4 rows x 4 chunks per pass)
// free of bank conflicts at D = 128, where a row fills a 256-byte bank cycle;
// at D = 64 the K swizzle r & 7 measured faster than the shifted form a
// 64-bank model prefers.
template <int D> __device__ __forceinline__ int k_swz(int r) { return D == 64 ? (r & 7) : (r & 15); }
template <int D> __device__ __forceinline__ int v_swz(int r) { return D == 64 ? 2 * (r & 3) : 4 * (r & 3); }
// E4M3 K rows (D bytes, D/16 chunks): lane l reads chunks 4s + 2(l/32) and the next one of
// row l%32, two 16-byte reads per MFMA operand; chunk c of row r sits at c ^ k8_swz(r), which
// leaves both reads free of bank conflicts.
template <int D> __device__ __forceinline__ int k8_swz(int r) { return D == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max / sum of x over lanes l and l^32 (v_permlane32_swap exchanges the two
// wave halves; the pair of results holds both halves' values in every lane).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer descriptor over `bytes` bytes at p (gfx9 layout: base, stride 0,
// num_records = bytes, raw dword format): loads at offsets >= bytes return zero.
typedef int i32x4_sgpr __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_sgpr make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4_sgpr r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}
// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16*lane.
// Written as inline assembly on purpose: the compiler cannot tell these LDS
// writes apart from the operand reads of other ring slots and would put a
// wait for every outstanding global load in front of the next LDS read.  The
// calling kernel orders them itself (an explicit vmcnt wait, plus a barrier
// where other waves read the data); loads the compiler does not see only make
// its own vmcnt waits stricter, never too weak.
// lds_addr: LDS byte address of the 1 KiB destination (wave-uniform).
__device__ __forceinline__ void dma16(i32x4_sgpr r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    // M0 is declared clobbered, so the compiler sets it again wherever it needs it.  One
    // wait state separates the scalar write of M0 from the load that reads it as the LDS
    // address (a manual wait state of the CDNA ISA the compiler cannot insert into asm).
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}
// dma16 without the compiler memory barrier: the asm statement stays in order with the other
// asm statements (volatile), while the compiler may still move its own memory operations
// across it.  A group of these loads closed by one dma16 keeps every later load behind the
// whole group.
__device__ __forceinline__ void dma16_nb(i32x4_sgpr r, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "m0");
}
// Streaming forms of the two loads above: the non-temporal cache policy (nt) marks data read
// once, such as a decode's pass over the KV cache.  A probe streaming 576 MiB from HBM read
// 6.8-7.1 TB/s with it against 5.9-6.3 TB/s without, at any waves per CU or loads in flight.
// Only for loads whose lines no later load reads: the decode's K operand loads (each cache line
// read by four k-step loads) and the prefill's tiles (read by every q-tile of a head) measured
// much slower with it.
__device__ __forceinline__ void dma16_nt(i32x4_sgpr r, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_nb_nt(i32x4_sgpr r, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "m0");
}
// Cache-policy operand of the buffer-load builtins that selects nt on this target.
constexpr int kCachePolicyNT = 2;

// Buffer descriptor for the compiler's buffer-load builtins: `bytes` from p are
// addressable, offsets past them read as zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCachePolicyNT));
}

// Four E4M3 codes (one dword, element i in byte i) -> four bf16 (two dwords), exact: every
// E4M3 value is a bf16 value.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Four INT8 codes (one dword, element i in byte i) -> four bf16 (two dwords), exact: every
// integer in [-128, 127] is a bf16 value.
__device__ __forceinline__ u32x2 i8x4_to_bf16(uint32_t w) {
    const float f0 = (float)(int)(int8_t)(w & 0xFFu);
    const float f1 = (float)(int)(int8_t)((w >> 8) & 0xFFu);
    const float f2 = (float)(int)(int8_t)((w >> 16) & 0xFFu);
    const float f3 = (float)((int)w >> 24);
    return u32x2{pack_bf16x2(f0, f1), pack_bf16x2(f2, f3)};
}
// Four 8-bit cache codes (E4M3, or INT8 when INT8) -> four bf16, exact.
template <bool INT8>
__device__ __forceinline__ u32x2 codes4_to_bf16(uint32_t w) {
    if constexpr (INT8) return i8x4_to_bf16(w);
    else return e4m3x4_to_bf16(w);
}

// Wait for this wave's outstanding global loads (including LDS-direct ones).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// gfx950 transposing 8-byte LDS read (ds_read_b64_tr_b16): within each
// 16-lane group, lane j receives element j%4 of the 8-byte rows addressed by
// lanes j/4 + 4k (k = 0..3), i.e. a 4x4 transpose of 16-bit elements.
__device__ __forceinline__ u32x2 ds_read_tr(const bf16* p) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    const v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf*)(const_cast<bf16*>(p)));
    return __builtin_bit_cast(u32x2, r);
}

// The same read at LDS byte address a.
__device__ __forceinline__ u32x2 ds_read_tr_at(uint32_t a) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    const v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) v4bf*)(uintptr_t)a);
    return __builtin_bit_cast(u32x2, r);
}

// Wait until at most N of this wave's global loads (including LDS-direct ones)
// are outstanding; also a compiler barrier for memory operations, so no LDS
// read of the landed data is moved above it.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace mfma
}  // namespace mattn
