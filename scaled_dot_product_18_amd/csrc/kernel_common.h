// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa18 {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Parameters of one launch, passed by value. q/o are [B,Hq,Sq,D] and k/v
// [B,Hkv,Sk,D] with the byte strides below; lse is dense [B,Hq,Sq].
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, Sq, Sk;
  int group;          // Hq / Hkv: query heads per KV head
  int n_qtiles;       // ceil(Sq / BLOCK_M)
  float qk_scale_log2;  // scale * descale_q * descale_k * log2(e): scores enter exp2 directly
  float o_scale;        // descale_v (1 unless fp8 inputs)
  int xcd_remap;        // 1: order workgroups so each XCD owns whole KV heads ((B*Hkv) % 8 == 0)
  int causal_off;       // Sk - Sq: under the causal mask query i sees keys j <= i + causal_off
  // Byte strides of q, k, v, o between batches (sb), heads (sh) and sequence
  // positions (ss); the d elements of one position are contiguous. The dense
  // [B,H,S,d] layout has ss = d * element size, sh = S * ss, sb = H * sh; the
  // pages' (B,T,N,H) layout has ss = N * d * element size, sh = d * element size.
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_ss, k_ss, v_ss, o_ss;
  int p8_qtile = 0;  // fp8 d = 128 kernel: first q-tile whose P.V takes P rounded to e4m3
};

// First byte of head h of batch b of a strided [B,H,S,d] tensor.
__device__ __forceinline__ const unsigned char* head_ptr(const void* base, long long sb, long long sh, int b, int h) {
  return (const unsigned char*)base + (long long)b * sb + (long long)h * sh;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange a value between lane l and lane l^32 and combine: v_permlane32_swap
// swaps the upper half of one operand with the lower half of the other, so
// the two results hold {x[l], x[l^32]} in some order on every lane.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Swap bits 2 and 3 of a row index. Reading K row pi(i) into MFMA row i makes
// the score accumulator registers 0..7 of a lane hold 8 consecutive keys, which
// is the layout the P operand of the P.V product needs.
__device__ __forceinline__ int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// {a.lo16, b.lo16} and {a.hi16, b.hi16} as one 32-bit word (low half first).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 t;
  t[0] = (bf16_t)lo;
  t[1] = (bf16_t)hi;
  return __builtin_bit_cast(uint32_t, t);
}

}  // namespace sdpa18
