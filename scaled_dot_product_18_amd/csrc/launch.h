// Host-side entry points of the kernel translation units (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_common.h"

namespace sdpa18 {

// Query rows per workgroup of each kernel family (the grid is
// ceil(Sq / block_m) x B x Hq workgroups).
int fp8_block_m(int d);
int fp8_pp_block_m();
int f32_block_m();
int bf16_block_m(int d);
int bf16_pp_block_m();

// bf16 inputs and output; d in {64, 128}.
hipError_t launch_attn_bf16(const AttnParams& p, int d, bool causal, hipStream_t stream);

// bf16, d = 128: eight waves in matrix-core / vector-unit ping-pong.
hipError_t launch_attn_bf16_pp(const AttnParams& p, bool causal, hipStream_t stream);

// fp8-e4m3fn inputs, bf16 output; d in {64, 128} (d = 128 runs the eight-wave
// ping-pong kernel).
hipError_t launch_attn_fp8(const AttnParams& p, int d, bool causal, hipStream_t stream);

// fp8-e4m3fn inputs, bf16 output, d = 128: eight waves in ping-pong.
hipError_t launch_attn_fp8_pp(const AttnParams& p, bool causal, hipStream_t stream);

// fp32 inputs and output; d in {64, 128}.
hipError_t launch_attn_f32(const AttnParams& p, int d, bool causal, hipStream_t stream);

// Split-KV forward: the keys of each KV head are cut into n_splits chunks of
// `chunk` keys (a multiple of 32), one workgroup per (column tile, batch, KV
// head, chunk); a column tile packs 32 (query head of the group, query) rows.
struct SplitParams {
  AttnParams a;     // n_qtiles and xcd_remap are unused
  float* part_o;    // [B*Hq*Sq][n_splits][d] normalised partial outputs (n_splits > 1)
  float* part_lse;  // [B*Hq*Sq][n_splits] base-2 log-sum-exp of the scaled scores of each chunk
  int n_splits;
  int chunk;
  int n_ctiles;     // ceil(group * Sq / 32)
};

// bf16 inputs and output, d in {64, 128}; with n_splits > 1 a second kernel
// merges the chunks into o and lse.
hipError_t launch_attn_splitkv_bf16(const SplitParams& sp, int d, bool causal, hipStream_t stream);

// Backward pass (attn_bwd.hip). q/o/dout/dq are [B,Hq,Sq,D], k/v/dk/dv
// [B,Hkv,Sk,D], lse, delta and lse2 [B,Hq,Sq]; all dense row-major, bf16
// except lse / delta / lse2 (fp32).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // forward log-sum-exp, natural log
  float* delta;      // workspace: rowsum(dO * O)
  float* lse2;       // workspace: lse * log2(e)
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Sq, Sk;
  int group;            // Hq / Hkv
  int causal_off;       // Sk - Sq under the causal mask, else 0
  float qk_scale_log2;  // multiplier of the dot products of the q, k arrays, times log2(e)
  // Factors that turn the arrays' values into the real ones (all 1 but the
  // dot-product scale unless q, k, v, dout are fp8 codes with descales):
  float delta_mul;      // delta = delta_mul * rowsum(dout * o), in the units of dout . v^T
  float dq_mul;         // dQ = dq_mul * sum dS K   (scale, times descales for fp8)
  float dk_mul;         // dK = dk_mul * sum dS^T Q
  float dv_mul;         // dV = dv_mul * sum P^T dout
  int n_qtiles;         // ceil(Sq / 128): dQ workgroups per (batch, query head)
  int n_ktiles;         // ceil(Sk / 128): dK/dV workgroups per (batch, KV head) and query-head subset
  int kv_split;         // query-head subsets per KV head in the dK/dV kernel (1: no partial sums)
  float* dkv_part;      // workspace, kv_split > 1 only: fp32 dK then dV partials [2][kv_split][B*Hkv*Sk][d]
};

// Query-head subsets per KV head for the dK/dV kernel: doubled while the grid
// is under two rounds of 256 workgroups and every subset keeps at least four
// query heads (MQA at long sequences would otherwise leave CUs idle).
inline int bwd_kv_split(int B, int Hkv, int Sk, int group) {
  const long long base = (long long)((Sk + 127) / 128) * B * Hkv;
  int ks = 1;
  while (base * ks < 512 && group % (2 * ks) == 0 && group / (2 * ks) >= 4) ks *= 2;
  return ks;
}

// bf16, d in {64, 128}: delta, then dQ, then dK and dV, on one stream.
hipError_t launch_attn_bwd_bf16(const BwdParams& bp, int d, bool causal, hipStream_t stream);

// fp8 inputs: q, k, v are e4m3fn codes and dout e5m2 codes (bp.q, bp.k,
// bp.v, bp.dout point at them), o is bf16. The codes are first widened to
// bf16 (exactly) into q16, k16, v16, do16 (each as many bf16 elements as the
// corresponding input), then the bf16 kernels run on the widened copies.
hipError_t launch_attn_bwd_fp8(const BwdParams& bp, void* q16, void* k16, void* v16, void* do16, int d, bool causal,
                               hipStream_t stream);

// fp32 inputs and outputs, d in {32, 64, 128}: delta, dQ, dK and dV on fp32
// matrix cores.
hipError_t launch_attn_bwd_f32(const BwdParams& bp, int d, bool causal, hipStream_t stream);

}  // namespace sdpa18
