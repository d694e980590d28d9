// attn_common.h -- gfx950 (CDNA4) device helpers shared by the attention
// kernels: vector types, buffer-resource loads with hardware range checks,
// LDS vector access and the MFMA wrappers.
//
// MFMA conventions used throughout (wave64, 32x32 output tiles):
//   A operand: lane l supplies row i = l % 32 of A and one contiguous run of
//              the contraction index chosen by its half h = l / 32;
//   B operand: lane l supplies column j = l % 32 of B and the same run of the
//              contraction index as A's lane half h (so any consistent
//              assignment of contraction indices to (h, slot) pairs gives the
//              same product);
//   C/D:       lane l, accumulator register r holds element
//              (row = 8*(r/4) + 4*h + r%4, col = l % 32).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Elt : int { ELT_F32 = 0, ELT_BF16 = 1, ELT_FP8 = 2 };

template <int E> struct EltInfo;
template <> struct EltInfo<ELT_F32> { static constexpr int bytes = 4; };
template <> struct EltInfo<ELT_BF16> { static constexpr int bytes = 2; };
template <> struct EltInfo<ELT_FP8> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// Buffer resources: loads beyond `nbytes` return zero in hardware, which is
// how every ragged tail (query rows >= Nq, key rows >= Nkv) is zero-filled.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  // dword3 = 0x00020000: raw (untyped) 32-bit data format for the gfx9 family.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS access (byte offsets into a __shared__ char array)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_store16(char* lds, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}
__device__ __forceinline__ void lds_store8(char* lds, uint32_t off, u32x2 v) {
  *reinterpret_cast<u32x2*>(lds + off) = v;
}
__device__ __forceinline__ u32x4 lds_load16(const char* lds, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(lds + off);
}
__device__ __forceinline__ float lds_loadf(const char* lds, uint32_t off) {
  return *reinterpret_cast<const float*>(lds + off);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (32x32 output tile, fp32 accumulate)
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// e4m3 x e4m3, K = 64 per instruction; unit scales (E8M0 code 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange a value with the lane 32 positions away (the other half-wave).
// Combine each lane's value with that of lane l ^ 32 (the other half of the
// wave).  v_permlane32_swap exchanges the upper half of one register with the
// lower half of another; applied to two copies of x it leaves x's lower half
// in both halves of one result and its upper half in both halves of the
// other, so one VALU instruction replaces an LDS permute and its wait.  (The
// two results are copied to scalars before the bit casts: a bit cast of an
// element of the returned vector read element 0 for both.)
__device__ __forceinline__ void wave_halves(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  wave_halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  wave_halves(x, a, b);
  return a + b;
}

// An empty volatile use of an MFMA result at this point of the program.  The
// optimiser otherwise sinks MFMAs (pure operations) towards their first use,
// past the branches and barriers that follow them, and the matrix work meant
// to overlap the code in between ends up after it.  The operand is an
// accumulation register: a VGPR operand would copy the result out after
// every MFMA and wait for it.
__device__ __forceinline__ void pin_acc(const f32x16& x) { asm volatile("" : : "a"(x)); }
// The same for a packed bf16 fragment computed by vector instructions.
__device__ __forceinline__ void pin_frag(const u32x4& x) { asm volatile("" : : "v"(x)); }

// f(integral_constant<int, I>) for I = B .. E-1, each call its own
// instantiation: loop bodies whose pieces depend on the index (if
// constexpr) stay small, and arrays indexed by it stay in registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// A float the whole wave reads from one address, through the scalar cache
// (a load from the constant address space; the data must not change while
// the kernel runs).
__device__ __forceinline__ float load_scalar(const float* ptr, int64_t i) {
  using cfloat = const __attribute__((address_space(4))) float;
  return ((cfloat*)(uintptr_t)ptr)[i];
}

// Round two floats to bf16 (RNE) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four consecutive output elements at element index idx: float32 when
// `f32` (partial results of a key range), otherwise bf16 (RNE).  idx is a
// multiple of 4, so both stores are naturally aligned.
__device__ __forceinline__ void store_o4(void* o, bool f32, int64_t idx, float a, float b, float c, float d) {
  if (f32) {
    *reinterpret_cast<f32x4*>((float*)o + idx) = f32x4{a, b, c, d};
  } else {
    const u32x2 pk = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>((__bf16*)o + idx) = pk;
  }
}

// Decode four e4m3 codes (one dword, byte 0 first) to bf16, exactly
// (every e4m3 value is representable in bf16).  Returns two packed dwords:
// .x = (byte0 | byte1 << 16), .y = (byte2 | byte3 << 16) as bf16 pairs.
// Uses the gfx950 scaled converts with a unit scale; the f32 route through
// v_cvt_pk_f32_fp8 plus bit packing is avoided because this compiler folds
// the high element of that builtin's result into the low one when both are
// bit-cast and repacked.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t codes) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Logical work-group id with the 8 XCDs of the chip each given one
// contiguous range of ids.  Work-groups are dispatched round-robin over the
// XCDs (id i runs on XCD i % 8), so this remap makes neighbouring logical
// ids -- neighbouring query tiles of one (batch, KV head) -- share one XCD's
// L2, where their common K/V tiles are re-read.  Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int i, int total) {
  constexpr int NXCD = 8;
  const int per = total / NXCD, rem = total % NXCD;
  const int xcd = i % NXCD, idx = i / NXCD;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace attn
