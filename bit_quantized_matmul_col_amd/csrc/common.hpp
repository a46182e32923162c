// Device helpers shared by the gfx950 kernels of the LLM.int8() linear layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmint8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Workspace regions are carved at this alignment.
constexpr size_t kAlign = 256;

// When the int8 GEMM runs on compacted operands (the K - |O| kept columns only).
// Compacting costs one pass over Wq plus writing the compacted copy, about
// (2K - |O|) * N bytes at HBM speed; it saves 2 * M * N * |O| int8 MFMA ops.
// With ~4 TB/s and ~2.5 POPS that pays off when M * |O| > 312.5 * (2K - |O|),
// which small-M (decode) calls never reach. The compacted row is staged in LDS,
// so K is also capped.
constexpr int kCompactMaxK = 32768;

__host__ __device__ inline bool use_compaction(int count, int64_t K, int64_t M) {
  return count > 0 && K <= kCompactMaxK && M * (int64_t)count * 16 > 5000 * (2 * K - count);
}

// Row count up to which the layer takes the small-M (decode) path, and the
// rows of one of its row groups (a GEMM block covers one group).
constexpr int kDecodeMaxM = 256;
constexpr int kDecodeGroupRows = 64;

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// fl32(127 / a) correctly rounded: the fp64 quotient of two fp32 values rounded
// once more to fp32 equals the correctly rounded fp32 quotient (53 >= 2*24 + 2).
__device__ inline float inv_scale(float a) { return (float)(127.0 / (double)a); }

// Symmetric int8 code of x for the scale inv = fl32(127 / absmax): one fp32
// multiply, round half to even, clamp to [-127, 127].
__device__ inline int quant_i8(float x, float inv) {
  float r = __builtin_rintf(x * inv);
  r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// The two 8-bit encodings of the layer. Each maps t = x * fl32(qmax / absmax)
// to a code byte: int8 rounds half to even and clamps to [-127, 127]; E4M3
// (the FP8 format of the "INT8 vs FP8 vs GPTQ" page, sections 2 and 4: 4
// exponent bits, 3 mantissa bits, largest value 448) takes the nearest value,
// ties to even, by the hardware conversion. |t| never exceeds qmax by more than the fp32
// rounding of the scale, which both encodings take to +-qmax.
struct CodecI8 {
  static constexpr double kQmax = 127.0;
  __device__ static uint32_t code(float t) {
    float r = __builtin_rintf(t);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(int)r & 0xffu;
  }
  // codes of t[0..3] packed little-endian
  __device__ static uint32_t code4(const float *t) {
    return code(t[0]) | code(t[1]) << 8 | code(t[2]) << 16 | code(t[3]) << 24;
  }
};

struct CodecE4M3 {
  static constexpr double kQmax = 448.0;
  __device__ static uint32_t code(float t) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xffu;
  }
  __device__ static uint32_t code4(const float *t) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
  }
};

// fl32(qmax / a) correctly rounded, as inv_scale.
template <class Codec>
__device__ inline float inv_scale_of(float a) { return (float)(Codec::kQmax / (double)a); }

// Absolute values of the 8 fp16 in a 16-byte chunk, folded into a running max.
__device__ inline void absmax8(const u32x4 &v, float *mx) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t w = v[e];
    mx[2 * e] = __builtin_fmaxf(mx[2 * e], __builtin_fabsf(h2f((uint16_t)(w & 0xffffu))));
    mx[2 * e + 1] = __builtin_fmaxf(mx[2 * e + 1], __builtin_fabsf(h2f((uint16_t)(w >> 16))));
  }
}

__device__ inline float fp16_lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ inline float fp16_hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// fl32(x * s) for the fp16 x in the low (fp16_lo_mul) or high (fp16_hi_mul)
// half of w: one v_fma_mix_f32 with a +0 addend does the conversion and the
// product with a single fp32 rounding, the same value as converting and then
// multiplying (only the sign of a zero product can differ).
__device__ inline float fp16_lo_mul(uint32_t w, float s) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(s));
  return r;
}
__device__ inline float fp16_hi_mul(uint32_t w, float s) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(s));
  return r;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace llmint8
