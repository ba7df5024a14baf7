// Matrix-core throughput microbenchmark for gfx950: the practical ceiling the
// attention kernels are measured against. Not part of the attention library;
// built into its own libmfmapeak.so and driven by `bench.py --mfma-peak`.
//
// Every wave issues a long stream of MFMAs on register operands into four
// independent accumulators (no memory traffic, no LDS, no VALU work in the
// loop), for the three instruction shapes the attention kernels use:
//   kind 0: v_mfma_f32_32x32x16_bf16          32768 FLOP per instruction
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4  131072 FLOP (e4m3 x e4m3, unit E8M0 scales)
//   kind 2: v_mfma_f32_32x32x2_f32              4096 FLOP
// A workgroup is four waves (one per SIMD of a CU); launching 256 * n
// workgroups puts n waves on every SIMD.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kUnroll = 8;  // MFMAs per loop iteration, over four accumulators
constexpr int kE8M0One = 127;

template <int KIND>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void mfma_peak_kernel(int iters, float* sink) {
  const int t = threadIdx.x;
  f32x16 c[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  if (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(1e-3f * (float)((t + e) & 7));
      b[e] = (__bf16)(1e-3f * (float)((t * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) c[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[u & 3], 0, 0, 0);
  } else if (KIND == 1) {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x20202020 + ((t + e) & 3);  // small e4m3 values
      b[e] = 0x18181818 + ((t * 3 + e) & 3);
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        c[u & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[u & 3], 0, 0, 0, kE8M0One, 0, kE8M0One);
  } else {
    const float a = 1e-3f * (float)(t & 7), b = 1e-3f * (float)((t * 3) & 7);
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) c[u & 3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c[u & 3], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += c[j][e];
  // The sums are never this value for the operands above; the compare keeps
  // every MFMA live without a store on the timed path.
  if (r == -1.0f) sink[blockIdx.x * 256 + t] = r;
}

}  // namespace

// Enqueue one launch of `blocks` workgroups of 256 threads, each wave running
// iters * 8 MFMAs of the given kind (0 bf16, 1 fp8, 2 fp32) on `stream`.
// sink: device buffer of blocks * 256 floats, written only in a case that does
// not occur. Returns 0, -1 for an unknown kind or bad sizes, -2 if the launch
// failed. FLOP per launch: blocks * 4 * iters * 8 * {32768, 131072, 4096}.
extern "C" int mfma_peak_launch(int kind, int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr) return -1;
  const void* fn = kind == 0   ? (const void*)&mfma_peak_kernel<0>
                   : kind == 1 ? (const void*)&mfma_peak_kernel<1>
                   : kind == 2 ? (const void*)&mfma_peak_kernel<2>
                               : nullptr;
  if (fn == nullptr) return -1;
  void* args[] = {&iters, &sink};
  return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, stream) == hipSuccess ? 0 : -2;
}
