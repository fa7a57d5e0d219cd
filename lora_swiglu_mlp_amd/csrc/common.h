// Device-side building blocks shared by the gfx950 kernels of the LoRA SwiGLU
// MLP: element types, bf16 rounding, and the MFMA step on 16-byte operand
// chunks.
//
// Operand convention used by every matrix kernel here. A "chunk" is 16 bytes
// of one matrix row along the contraction axis: 8 bf16 or 4 fp32 values. One
// "k-step" feeds a 16x16 output tile from four consecutive chunks of 16 rows
// of each operand: lane l supplies row (l & 15), chunk (l >> 4). For bf16 this
// is exactly one v_mfma_f32_16x16x32_bf16. For fp32 it is four
// v_mfma_f32_16x16x4_f32, the j-th taking element j of each lane's chunk;
// together they contract the same 16 values, in a different order, which is
// fine because both operands use the same chunk layout.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace lmlp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

struct bf16_t { uint16_t bits; };

// ---------------------------------------------------------------------------
// scalar conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (NaN kept quiet). gfx950 lowers this pattern to
// its packed bf16 convert.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// The same rounding as pack_bf16x2 as one packed convert (gfx950
// v_cvt_pk_bf16_f32). Used where conversions dominate (the 4-bit decode in the
// GEMM K loop, the SwiGLU backward epilogue); elsewhere the two-convert form
// is kept because it leaves the GEMM K loops' register allocation as it is
// (with the packed form the compiler moved accumulators between AGPRs and
// VGPRs inside the plain, gate/up and dX K loops).
__device__ __forceinline__ uint32_t pack_bf16x2_pk(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------------------
// element traits: CH = elements per 16-byte chunk

template <typename T> struct elem;
template <> struct elem<bf16_t> {
  static constexpr int CH = 8;
  static constexpr int BYTES = 2;
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
  __device__ static void store(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }
  __device__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};
template <> struct elem<float> {
  static constexpr int CH = 4;
  static constexpr int BYTES = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static float round(float v) { return v; }
};

// Four consecutive outputs of one row, stored with one vector store.
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void load4(const bf16_t* p, float& a, float& b, float& c, float& d) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  a = __uint_as_float(v.x << 16);
  b = __uint_as_float(v.x & 0xFFFF0000u);
  c = __uint_as_float(v.y << 16);
  d = __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float& a, float& b, float& c, float& d) {
  float4 v = *reinterpret_cast<const float4*>(p);
  a = v.x; b = v.y; c = v.z; d = v.w;
}

// ---------------------------------------------------------------------------
// MFMA on chunks: acc[i] for the 16x16 tile D = SrcA * SrcB^T where lane l
// holds row (l & 15) of each source, k-chunk (l >> 4). Output layout: lane l
// holds D[4*(l>>4) + i][l & 15], i = 0..3 (rows of SrcA, columns of SrcB).

template <typename T> struct mma;
template <> struct mma<bf16_t> {
  __device__ static __forceinline__ f32x4_t step(const uint4& a, const uint4& b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct mma<float> {
  __device__ static __forceinline__ f32x4_t step(const uint4& a, const uint4& b, f32x4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    return acc;
  }
};

// ---------------------------------------------------------------------------
// SwiGLU pieces (fp32)

__device__ __forceinline__ float sigmoidf_fast(float g) {
  // 1 / (1 + e^-g) with the hardware reciprocal (v_rcp_f32, about 1 ulp).
  // The argument is >= 1, so no denormal input reaches it; e^-g overflows to
  // +inf for very negative g and rcp(+inf) is exactly 0, so no branch is
  // needed. A correctly rounded reciprocal costs a dozen instructions per
  // element here and pushed the GEMM epilogues into register spills.
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Unsigned 16-byte chunk helpers
__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// XOR swizzle of the 16-byte chunk position within a 128-byte LDS row, so
// that the 16 rows one MFMA operand read touches, and the rows a transposing
// store touches, fall in distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row ^ (row >> 3)) & 7);
}

// ---------------------------------------------------------------------------
// 4-bit block weights. A byte holds two two's-complement codes, the even
// element in the low nibble; the weight is bf16_rne(q * scale) with the
// product in fp32 (exact: an 11-bit fp16 significand times a 4-bit integer).
__device__ __forceinline__ uint32_t dq_pair(uint32_t byte2, float sc) {
  // byte2 holds two codes: low nibble = even element
  const int q0 = static_cast<int>(byte2 << 28) >> 28;
  const int q1 = static_cast<int>((byte2 >> 4) << 28) >> 28;
  return pack_bf16x2_pk(static_cast<float>(q0) * sc, static_cast<float>(q1) * sc);
}
__device__ __forceinline__ uint4 dq_chunk(uint32_t w, float sc) {
  // w = 4 bytes = 8 codes -> 8 bf16
  uint4 o;
  o.x = dq_pair(w & 0xFF, sc);
  o.y = dq_pair((w >> 8) & 0xFF, sc);
  o.z = dq_pair((w >> 16) & 0xFF, sc);
  o.w = dq_pair(w >> 24, sc);
  return o;
}
}  // namespace lmlp
