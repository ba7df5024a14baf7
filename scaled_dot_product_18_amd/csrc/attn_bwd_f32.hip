// Attention backward pass for gfx950 on fp32 matrix cores: dQ, dK, dV from fp32
// Q, K, V, O, dO and the forward's log-sum-exp, fp32 products and
// accumulation, fp32 outputs. The full-precision member of the backward
// family, as attn_fwd_f32.hip is of the forward one.
//
// The gradients are the chain rule through the forward's three steps (codelab
// "Accelerate attention on GPU with cuDNN and TransformerEngine", section 4),
// with the attention weights recomputed tile by tile from the stored per-row
// statistic (article "Self-attention, CUDA kernels and FlashAttention",
// section 3):
//   P = exp(scale Q K^T - lse)         dV = P^T dO         dP = dO V^T
//   dS = P * (dP - delta), delta_i = sum_c dO_ic O_ic
//   dQ = scale dS K                    dK = scale dS^T Q
// Every product runs on v_mfma_f32_32x32x2_f32 (K depth 2), so no operand
// needs transposing: an MFMA step takes one element per lane, and the step
// that consumes a pair of keys (queries) takes them in the order the score
// registers hold them (key 8(r/4) + 4g + r%4 of register r on half-wave g).
// Tiles sit in LDS with rows padded by one float, so the column reads of the
// operands hit distinct banks.
//  * attn_bwd_f32_delta_kernel: delta and lse * log2(e) per query row;
//  * attn_bwd_f32_dq_kernel: one workgroup per 128 queries of one (batch,
//    query head), lane = query column; the Q fragment in registers, the
//    workgroup's dO rows and 32-key K/V tiles in LDS;
//  * attn_bwd_f32_dkdv_kernel: one workgroup per 64 keys of one (batch, KV
//    head), lane = key column; the workgroup's K and V rows in LDS, 32-query
//    tiles of Q and dO (with their lse and delta) streamed through LDS for
//    every query head of the KV head's group, so GQA/MQA sum over the group
//    inside the workgroup (no atomics, deterministic).
// Under the causal mask (query i sees keys j <= i + Sk - Sq) tiles that see
// nothing are skipped and edge tiles are masked.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {
namespace bwd32 {

// ---------------------------------------------------------------- delta
// delta[row] = delta_mul * sum_c dO[row, c] O[row, c]; lse2[row] = lse[row] * log2(e).
// D/4 lanes per row, 4 elements each.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_bwd_f32_delta_kernel(const BwdParams p) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const float4 a = *(const float4*)((const float*)p.o + row * D + 4 * part);
    const float4 b = *(const float4*)((const float*)p.dout + row * D + 4 * part);
    acc = (a.x * b.x + a.y * b.y) + (a.z * b.z + a.w * b.w);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && part == 0) {
    p.delta[row] = acc * p.delta_mul;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// Rows [r0, r0 + n) of a row-major [*, D] fp32 array -> LDS rows padded to
// D + 1 floats, by NT threads; rows at or past `limit` read as zeros.
template <int D, int NT>
__device__ __forceinline__ void load_rows(const float* src, int r0, int n, int limit, float* dst, int tid) {
  constexpr int LD = D + 1;
  for (int f = tid; f < n * (D / 4); f += NT) {
    const int row = f / (D / 4);
    const int c4 = f - row * (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + row < limit) x = *(const float4*)(src + (size_t)(r0 + row) * D + 4 * c4);
    float* d = dst + row * LD + 4 * c4;
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
  }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_bwd_f32_dq_kernel(const BwdParams p) {
  constexpr int BM = 128, BN = 32, LD = D + 1, DB = D / 32;
  __shared__ float ks[BN * LD];
  __shared__ float vs[BN * LD];
  __shared__ float dos[BM * LD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  const int BH = p.B * p.Hq;
  const int qt_seq = blockIdx.x / BH;
  const int rem = blockIdx.x - qt_seq * BH;
  const int b = rem / p.Hq;
  const int hq = rem - b * p.Hq;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - qt_seq) : qt_seq;  // heaviest first under the mask
  const int hk = hq / p.group;

  const int q0 = qt * BM;
  const int qw = q0 + 32 * wave;
  const int qi = qw + i32;
  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;
  const size_t kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Sk;
  const float* kbase = (const float*)p.k + kv_row0 * D;
  const float* vbase = (const float*)p.v + kv_row0 * D;

  const int kv_end = CAUSAL ? min(p.Sk, q0 + BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / BN + 1) : n_tiles);

  // Q fragment (B operand of S^T): step s, half g holds dim 2s + g of query qi.
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = qi < p.Sq ? ((const float*)p.q)[(qo_row0 + qi) * D + 2 * s + g] : 0.f;
  // Padding rows (qi >= Sq) have Q = dO = 0 and lse = delta = 0: every dS there is 0.
  const float lse2 = qi < p.Sq ? p.lse2[qo_row0 + qi] : 0.f;
  const float dlt = qi < p.Sq ? p.delta[qo_row0 + qi] : 0.f;
  load_rows<D, 256>((const float*)p.dout + qo_row0 * D, q0, BM, p.Sq, dos, tid);
  const float* dorow = dos + (32 * wave + i32) * LD;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  const float c = p.qk_scale_log2;

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int kv0 = kt * BN;
    __syncthreads();  // the previous tile is consumed (and the dO rows are in LDS)
    load_rows<D, 256>(kbase, kv0, BN, p.Sk, ks, tid);
    load_rows<D, 256>(vbase, kv0, BN, p.Sk, vs, tid);
    __syncthreads();
    if (kt >= wave_tiles) continue;
    // S^T = K Q^T and dP^T = V dO^T: row = key kv0 + i, column = this lane's query
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 2; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[i32 * LD + 2 * st + g], qf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[i32 * LD + 2 * st + g], dorow[2 * st + g], dp, 0, 0, 0);
    }
    // register r on half g: key kv0 + 8(r/4) + 4g + r%4
    const bool edge = (CAUSAL && kv0 + BN - 1 > qw + p.causal_off) || kv0 + BN > p.Sk;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(__builtin_fmaf(s[r], c, -lse2));
      if (edge) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < p.Sk && (!CAUSAL || key <= qi + p.causal_off);
        pr = ok ? pr : 0.f;
      }
      ds[r] = pr * (dp[r] - dlt);
    }
    // dQ^T += K^T dS^T, one pair of keys per MFMA in the registers' key order
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[key * LD + 32 * db + i32], ds[r], acc[db], 0, 0, 0);
      }
  }

  if (qi >= p.Sq) return;
  float* out = (float*)p.dq + (qo_row0 + qi) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      *(float4*)(out + d) = make_float4(acc[db][4 * q4] * p.dq_mul, acc[db][4 * q4 + 1] * p.dq_mul,
                                        acc[db][4 * q4 + 2] * p.dq_mul, acc[db][4 * q4 + 3] * p.dq_mul);
    }
}

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(128, 128)))
void attn_bwd_f32_dkdv_kernel(const BwdParams p) {
  constexpr int BK = 64, BT = 32, LD = D + 1, DB = D / 32;
  __shared__ float ks[BK * LD];
  __shared__ float vs[BK * LD];
  __shared__ float qs[BT * LD];
  __shared__ float os[BT * LD];  // dO
  __shared__ float st[2 * BT];   // lse2, then delta, of the tile's queries

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int kt = blockIdx.x / BH;
  const int rem = blockIdx.x - kt * BH;
  const int b = rem / p.Hkv;
  const int hk = rem - b * p.Hkv;

  const int k0 = kt * BK;
  const int kw = k0 + 32 * wave;
  const int kj = kw + i32;  // this lane's key
  const size_t kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Sk;
  load_rows<D, 128>((const float*)p.k + kv_row0 * D, k0, BK, p.Sk, ks, tid);
  load_rows<D, 128>((const float*)p.v + kv_row0 * D, k0, BK, p.Sk, vs, tid);
  const float* krow = ks + (32 * wave + i32) * LD;
  const float* vrow = vs + (32 * wave + i32) * LD;

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float c = p.qk_scale_log2;
  const int off = p.causal_off;
  // Queries that see a key of this workgroup: i >= k0 - off (all of them without the mask).
  const int t_first = CAUSAL ? max(0, k0 - off) / BT : 0;
  const int n_qt = (p.Sq + BT - 1) / BT;
  const bool wave_active = kw < p.Sk;

  for (int gq = 0; gq < p.group; ++gq) {
    const int hq = hk * p.group + gq;
    const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;
    for (int t = t_first; t < n_qt; ++t) {
      const int qb0 = t * BT;
      __syncthreads();  // the previous tile is consumed (and the K/V rows are in LDS)
      load_rows<D, 128>((const float*)p.q + qo_row0 * D, qb0, BT, p.Sq, qs, tid);
      load_rows<D, 128>((const float*)p.dout + qo_row0 * D, qb0, BT, p.Sq, os, tid);
      if (tid < 2 * BT) {
        const int qq = qb0 + (tid & (BT - 1));
        st[tid] = qq < p.Sq ? (tid < BT ? p.lse2 : p.delta)[qo_row0 + qq] : 0.f;
      }
      __syncthreads();
      if (!wave_active || (CAUSAL && qb0 + BT - 1 + off < kw)) continue;  // no query of the tile sees these keys
      // S = Q K^T, dP = dO V^T: row = query qb0 + i, column = this lane's key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int k2 = 0; k2 < D / 2; ++k2) {
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[i32 * LD + 2 * k2 + g], krow[2 * k2 + g], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x2f32(os[i32 * LD + 2 * k2 + g], vrow[2 * k2 + g], dp, 0, 0, 0);
      }
      // register r on half g: query qb0 + 8(r/4) + 4g + r%4
      const bool edge = (CAUSAL && kw + 31 > qb0 + off) || qb0 + BT > p.Sq || kw + 32 > p.Sk;
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * g + (r & 3);
        float x = exp2_fast(__builtin_fmaf(s[r], c, -st[qr]));
        if (edge) {
          const int qq = qb0 + qr;
          const bool ok = qq < p.Sq && kj < p.Sk && (!CAUSAL || kj <= qq + off);
          x = ok ? x : 0.f;
        }
        pr[r] = x;
        ds[r] = x * (dp[r] - st[BT + qr]);
      }
      // dV^T += dO^T P, dK^T += Q^T dS: one pair of queries per MFMA in the registers' query order
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 8 * (r >> 2) + 4 * g + (r & 3);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(os[qr * LD + 32 * db + i32], pr[r], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[qr * LD + 32 * db + i32], ds[r], dk[db], 0, 0, 0);
        }
    }
  }

  if (kj >= p.Sk) return;
  float* pk = (float*)p.dk + (kv_row0 + kj) * D;
  float* pv = (float*)p.dv + (kv_row0 + kj) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      *(float4*)(pk + d) = make_float4(dk[db][4 * q4] * p.dk_mul, dk[db][4 * q4 + 1] * p.dk_mul,
                                       dk[db][4 * q4 + 2] * p.dk_mul, dk[db][4 * q4 + 3] * p.dk_mul);
      *(float4*)(pv + d) = make_float4(dv[db][4 * q4] * p.dv_mul, dv[db][4 * q4 + 1] * p.dv_mul,
                                       dv[db][4 * q4 + 2] * p.dv_mul, dv[db][4 * q4 + 3] * p.dv_mul);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const BwdParams& bp, hipStream_t stream) {
  BwdParams arg = bp;
  void* args[] = {&arg};
  const size_t rows = (size_t)bp.B * bp.Hq * bp.Sq;
  constexpr int RPB = 256 / (D / 4);
  hipError_t e = hipLaunchKernel((const void*)&attn_bwd_f32_delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)),
                                 dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned n_q = (unsigned)((bp.Sq + 127) / 128);
  arg.n_qtiles = (int)n_q;
  e = hipLaunchKernel((const void*)&attn_bwd_f32_dq_kernel<D, CAUSAL>, dim3(n_q * (unsigned)bp.B * (unsigned)bp.Hq),
                      dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned n_k = (unsigned)((bp.Sk + 63) / 64);
  return hipLaunchKernel((const void*)&attn_bwd_f32_dkdv_kernel<D, CAUSAL>,
                         dim3(n_k * (unsigned)bp.B * (unsigned)bp.Hkv), dim3(128), args, 0, stream);
}

}  // namespace bwd32

hipError_t launch_attn_bwd_f32(const BwdParams& bp, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? bwd32::launch_d<128, true>(bp, stream) : bwd32::launch_d<128, false>(bp, stream);
  if (d == 32) return causal ? bwd32::launch_d<32, true>(bp, stream) : bwd32::launch_d<32, false>(bp, stream);
  return causal ? bwd32::launch_d<64, true>(bp, stream) : bwd32::launch_d<64, false>(bp, stream);
}

}  // namespace sdpa18
