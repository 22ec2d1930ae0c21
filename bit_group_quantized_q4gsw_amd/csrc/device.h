// Device-side helpers shared by the q4gsw kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace q4gsw {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <typename T, typename F>
__device__ __forceinline__ T bitcast(F v) {
    static_assert(sizeof(T) == sizeof(F), "bitcast size");
    return __builtin_bit_cast(T, v);
}

// ---- scalar element loads widened to fp32 -------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)bitcast<_Float16>(b); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return bitcast<float>((uint32_t)b << 16); }

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
    if constexpr (DT == kF32) {
        return static_cast<const float*>(base)[i];
    } else if constexpr (DT == kF16) {
        return f16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    } else {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    }
}

__device__ __forceinline__ float load_scale(const void* base, int scale_f16, int64_t i) {
    return scale_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(base)[i])
                     : static_cast<const float*>(base)[i];
}

// ---- 4-bit code unpacking -----------------------------------------------------------------
// Pair s of a word: k-offsets (2s, 2s+1) of the word's octet in the low/high 16-bit halves.
// OR-ing 0x6400 builds the fp16 value 1024 + c exactly; subtracting 1032 gives c - 8 exactly.
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int s) { return (w >> (4 * s)) & 0x000F000Fu; }

__device__ __forceinline__ h2 codes_minus8_f16(uint32_t w, int s) {
    h2 v = bitcast<h2>(nib_pair(w, s) | 0x64006400u);
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    return v - off;
}

// Signed code value c - 8 of nibble position p, exactly, as an integer.  XOR-ing a word with
// 0x88888888 turns every nibble into the two's-complement 4-bit form of c - 8.
__device__ __forceinline__ int signed_code(uint32_t wx, int p) {
    // the builtin's C type is unsigned; the bits are the sign-extended field
    return (int)__builtin_amdgcn_sbfe((int)wx, 4 * p, 4);
}

// Exact (c - 8) pair s (k-offsets 2s, 2s+1) in bf16: small integers are exact in fp32 with
// a zero low half, so the bf16 value is the upper 16 bits.  wx = word ^ 0x88888888.
__device__ __forceinline__ uint32_t codes_minus8_bf16(uint32_t wx, int s) {
    const float lo = (float)signed_code(wx, s);
    const float hi = (float)signed_code(wx, s + 4);
    return __builtin_amdgcn_perm(bitcast<uint32_t>(hi), bitcast<uint32_t>(lo), 0x07060302u);
}

// The eight values c - 8 of a word as fp32, in k-offset order 0..7.
__device__ __forceinline__ void word_codes_minus8_f32(uint32_t w, float (&c)[8]) {
    const uint32_t wx = w ^ 0x88888888u;
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (float)signed_code(wx, nib_pos(j));
}

// ---- fp32 -> bf16 hi/lo split (round to nearest even both times) --------------------------
// a = hi + lo + e with |e| <= 2^-18 |a| (hi carries 8 significant bits, lo the next 8).
__device__ __forceinline__ void split_bf16(float a0, float a1, uint32_t& hi, uint32_t& lo) {
    b2 h = {(__bf16)a0, (__bf16)a1};
    uint32_t hb = bitcast<uint32_t>(h);
    float r0 = a0 - bitcast<float>(hb << 16);
    float r1 = a1 - bitcast<float>(hb & 0xFFFF0000u);
    b2 l = {(__bf16)r0, (__bf16)r1};
    hi = hb;
    lo = bitcast<uint32_t>(l);
}

// ---- MFMA (gfx950, 16x16x32, fp32 accumulate) ---------------------------------------------
// A fragment: lane l holds A[l%16][8*(l/16) + 0..7]; B fragment: B[8*(l/16) + 0..7][l%16];
// D: lane l, register r holds D[4*(l/16) + r][l%16].
__device__ __forceinline__ f4 mfma_f16(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<h8>(a), bitcast<h8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_bf16(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<b8>(a), bitcast<b8>(b), c, 0, 0, 0);
}

// gfx950 v_mfma_f32_32x32x16 (twice the issue rate of the 16x16x32 form on this chip):
// A fragment: lane l holds A[l%32][8*(l/32) + 0..7]; B fragment: B[8*(l/32) + 0..7][l%32];
// D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32_f16(u4 a, u4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<h8>(a), bitcast<h8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(u4 a, u4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<b8>(a), bitcast<b8>(b), c, 0, 0, 0);
}

// ---- global loads ---------------------------------------------------------------------------
__device__ __forceinline__ u4 ldg16(const void* p) { return *static_cast<const u4*>(p); }
__device__ __forceinline__ u4 ldg16_stream(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u4*>(p));
}
__device__ __forceinline__ u2 ldg8_stream(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u2*>(p));
}

// ---- LDS-DMA (global_load_lds) and explicit load/barrier ordering ----------------------------
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

// Each lane's bytes land at dst + size * lane; dst must be wave-uniform.
__device__ __forceinline__ void dma16(const void* src, lds_u8* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, lds_u8* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding and all of its LDS
// operations are done, then meet the other waves.  Vector loads (LDS-DMA included) retire in
// issue order, so this completes every load issued more than N loads ago.  The memory
// clobber keeps the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Sum of v over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one position of every 16-lane row), in
// every lane: gfx950's row swap and half swap, register to register.  Swapping a value with
// itself leaves row r's and row r ^ 1's copies in the two results (likewise the two halves).
__device__ __forceinline__ float wave_sum_rows(float v) {
    const uint32_t a = bitcast<uint32_t>(v);
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const float s = bitcast<float>(r[0]) + bitcast<float>(r[1]);
    const uint32_t b = bitcast<uint32_t>(s);
    const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return bitcast<float>(h[0]) + bitcast<float>(h[1]);
}

// Sum of v over the 32 lanes with the parity of this lane, in every lane: DPP inside each
// 16-lane row (quad_perm [2,3,0,1] pairs lane i with i ^ 2; rotations by 4 and 8 then cover
// the row's positions of that parity), then across the rows.
__device__ __forceinline__ float wave_sum_same_parity(float v) {
    v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x4E, 0xF, 0xF, false));
    v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x124, 0xF, 0xF, false));
    v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x128, 0xF, 0xF, false));
    return wave_sum_rows(v);
}

// p[i] when ok, else 0, from an unconditional load (index 0 stands in when !ok): no branch
// around the load, so a lane's loads can all be in flight before the first wait.
__device__ __forceinline__ float load_sel(const float* __restrict__ p, int64_t i, bool ok) {
    const float v = p[ok ? i : 0];
    return ok ? v : 0.0f;
}

// Sum of the partials P[s * stride + off], s = 0 .. count - 1 ascending (starting from 0 + P[0]),
// loads issued NB at a time.
template <int NB>
__device__ __forceinline__ float chunk_sum(const float* __restrict__ P, int64_t count, int64_t stride, int64_t off) {
    float v = 0.0f;
    for (int64_t s0 = 0; s0 < count; s0 += NB) {
        float p[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) p[k] = load_sel(P, (s0 + k) * stride + off, s0 + k < count);
#pragma unroll
        for (int k = 0; k < NB; ++k) v += p[k];       // past the last partial: + 0, exact
    }
    return v;
}

}  // namespace q4gsw
