// Fused scaled dot-product attention forward for gfx950 on fp32 matrix cores:
// fp32 inputs, fp32 products and accumulation, fp32 output. This is the
// full-precision member of the kernel family; it uses the same transposed
// formulation as the bf16/fp8 kernel (S^T = K . Q^T and O^T += V^T . P^T on
// v_mfma_f32_32x32x2_f32, one query column per lane, online softmax as in
// "Self-attention, CUDA kernels and FlashAttention", section 3) with P kept
// in fp32. With a K depth of 2 per MFMA no operand needs transposing: the
// A operand of P.V is one element of a V row per lane.
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); KV
// tiles of 32 keys go through one LDS buffer (K rows padded by one float so
// the column reads of the S^T operand hit distinct banks); at d = 128, and
// for grids up to 256 workgroups at d = 64, the next tile waits in registers
// meanwhile. Grids of up to 128 workgroups run the key-split kernel further
// down instead, one workgroup per 32 query rows.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {

template <int D, bool CAUSAL, bool PREFETCH>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_fwd_f32_kernel(const AttnParams p) {
  constexpr int BM = 128;
  constexpr int BN = 32;
  constexpr int KLD = D + 1;  // padded K row (floats)
  constexpr int DB = D / 32;
  constexpr int LOADS = BN * D / 4 / 256;  // float4 loads per thread per tensor per tile
  __shared__ float ks[BN * KLD];
  __shared__ __attribute__((aligned(16))) float vs[BN * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  const int BH = p.B * p.Hq;
  const int seq = blockIdx.x / BH;
  const int rem = blockIdx.x - seq * BH;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - seq) : seq;
  const int b = rem / p.Hq;
  const int hq = rem - b * p.Hq;
  const int hk = hq / p.group;

  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);

  const int kv_end = CAUSAL ? min(p.Sk, q0 + BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / BN + 1) : n_tiles);

  // Q fragment (B operand of S^T): step s, half g holds dim 2s + g.
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = (qi < p.Sq) ? ((const float*)(qbase + (size_t)qi * p.q_ss))[2 * s + g] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = p.qk_scale_log2;

  // PREFETCH: the next tile's K and V rows are loaded into registers while
  // the current tile is computed, and written to LDS after the barrier that
  // ends it. It costs 4 LOADS VGPRs: at d = 64 that lowers the resident waves
  // per SIMD from three to two, which large grids feel more than the hidden
  // load latency; without it each tile is loaded after the barrier.
  float4 kx[LOADS], vx[LOADS];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int f = tid + 256 * t;
      const int row = f / (D / 4);
      const int c4 = f - row * (D / 4);
      const int kr = kt * BN + row;
      kx[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      vx[t] = kx[t];
      if (kr < p.Sk) {
        kx[t] = *(const float4*)(kbase + (size_t)kr * p.k_ss + 16 * c4);
        vx[t] = *(const float4*)(vbase + (size_t)kr * p.v_ss + 16 * c4);
      }
    }
  };
  if (PREFETCH && n_tiles > 0) load_tile(0);
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int kv0 = kt * BN;
    __syncthreads();  // previous tile fully consumed
    if (!PREFETCH) load_tile(kt);
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int f = tid + 256 * t;
      const int row = f / (D / 4);
      const int c4 = f - row * (D / 4);
      float* kd = ks + row * KLD + 4 * c4;
      kd[0] = kx[t].x;
      kd[1] = kx[t].y;
      kd[2] = kx[t].z;
      kd[3] = kx[t].w;
      *(float4*)(vs + row * D + 4 * c4) = vx[t];
    }
    __syncthreads();
    if (PREFETCH && kt + 1 < n_tiles) load_tile(kt + 1);
    if (kt >= wave_tiles) continue;

    // S^T = K . Q^T: row i = key kv0 + i, column = query of this lane.
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 2; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[i32 * KLD + 2 * st + g], qf[st], s, 0, 0, 0);

    // register r on half g holds key kv0 + 8(r/4) + 4g + (r%4)
    const bool need_mask = (CAUSAL && kv0 + BN - 1 > qw + p.causal_off) || (kv0 + BN > p.Sk);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = (key < p.Sk) && (!CAUSAL || key <= qi + p.causal_off);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halfwave_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float pr[16];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = exp2_fast(__builtin_fmaf(s[r], c, -m_new));
      rs += pr[r];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;

    // O^T += V^T . P^T, one pair of keys per MFMA: step r takes key
    // 8(r/4) + 4g + (r%4) from half g, matching the score registers.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + 32 * db + i32], pr[r], acc[db], 0, 0, 0);
      }
  }

  if (!wave_active) return;
  const float l_tot = halfwave_sum(l_run);
  if (qi >= p.Sq) return;
  const float inv = 1.0f / l_tot;
  float* orow = (float*)((unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq) + (size_t)qi * p.o_ss);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      *(float4*)(orow + d) = make_float4(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv,
                                         acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv);
    }
  if (g == 0 && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// Small grids (up to 128 workgroups of 128 rows, e.g. one 128-token head): one
// workgroup per 32 query rows, so the work spreads over four times as many CUs, and its 4
// waves (one per SIMD) split the keys: keys arrive in super-tiles of 128 (one
// load round trip for four 32-key tiles) and wave s runs the online softmax
// over tiles s, s+4, s+8, ... The four partial states (running maximum,
// normaliser, accumulator) are merged through LDS by the identity the online
// softmax itself uses: O = sum_s 2^(m_s - m) acc_s / sum_s 2^(m_s - m) l_s.
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_fwd_f32_split_kernel(const AttnParams p) {
  constexpr int BM = 32;
  constexpr int BN = 32;
  constexpr int NS = 4;          // key splits, one per wave
  constexpr int SBN = NS * BN;   // keys per super-tile
  constexpr int KLD = D + 1;     // padded K row (floats)
  constexpr int DB = D / 32;
  constexpr int LOADS = SBN * D / 4 / 256;  // float4 loads per thread per tensor per super-tile
  constexpr int KV_FLOATS = SBN * KLD + SBN * D;
  constexpr int ST_FLOATS = DB * 16 * 64 + 2 * 64;  // one wave's state: accumulator, maximum, normaliser
  constexpr int MERGE_FLOATS = 2 * ST_FLOATS;
  static_assert((SBN * KLD) % 4 == 0, "V must start 16-byte aligned");
  __shared__ __attribute__((aligned(16))) float smem[KV_FLOATS > MERGE_FLOATS ? KV_FLOATS : MERGE_FLOATS];
  float* ks = smem;
  float* vs = smem + SBN * KLD;

  const int tid = threadIdx.x;
  const int sp = tid >> 6;  // key split = wave
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  const int BH = p.B * p.Hq;
  const int seq = blockIdx.x / BH;
  const int rem = blockIdx.x - seq * BH;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - seq) : seq;  // n_qtiles counts 32-row tiles here
  const int b = rem / p.Hq;
  const int hq = rem - b * p.Hq;
  const int hk = hq / p.group;

  const int qw = qt * BM;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);

  const int n_tiles = (CAUSAL ? min(p.Sk, qw + 31 + p.causal_off + 1) : p.Sk) + BN - 1;
  const int wave_tiles = n_tiles / BN;  // tiles these 32 rows need
  const int n_super = (wave_tiles + NS - 1) / NS;

  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = (qi < p.Sq) ? ((const float*)(qbase + (size_t)qi * p.q_ss))[2 * s + g] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = p.qk_scale_log2;

  for (int st = 0; st < n_super; ++st) {
    const int kv_s = st * SBN;
    __syncthreads();  // previous super-tile fully consumed
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int f = tid + 256 * t;
      const int row = f / (D / 4);
      const int c4 = f - row * (D / 4);
      const int kr = kv_s + row;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (kr < p.Sk) {
        kx = *(const float4*)(kbase + (size_t)kr * p.k_ss + 16 * c4);
        vx = *(const float4*)(vbase + (size_t)kr * p.v_ss + 16 * c4);
      }
      float* kd = ks + row * KLD + 4 * c4;
      kd[0] = kx.x;
      kd[1] = kx.y;
      kd[2] = kx.z;
      kd[3] = kx.w;
      *(float4*)(vs + row * D + 4 * c4) = vx;
    }
    __syncthreads();
    const int kt = st * NS + sp;
    if (qw >= p.Sq || kt >= wave_tiles) continue;
    const int kv0 = kt * BN;
    const float* kt_s = ks + sp * BN * KLD;
    const float* vt_s = vs + sp * BN * D;

    f32x16 s = f32x16{};
#pragma unroll
    for (int st2 = 0; st2 < D / 2; ++st2)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kt_s[i32 * KLD + 2 * st2 + g], qf[st2], s, 0, 0, 0);

    // register r on half g holds key kv0 + 8(r/4) + 4g + (r%4)
    const bool need_mask = (CAUSAL && kv0 + BN - 1 > qw + p.causal_off) || (kv0 + BN > p.Sk);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = (key < p.Sk) && (!CAUSAL || key <= qi + p.causal_off);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halfwave_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    // A split's first tile can hide every key from a row: keep the empty
    // state (maximum -inf, nothing accumulated) instead of exp2(-inf - -inf).
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    float pr[16];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = exp2_fast(__builtin_fmaf(s[r], c, -m_use));
      rs += pr[r];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt_s[key * D + 32 * db + i32], pr[r], acc[db], 0, 0, 0);
      }
  }

  // ---- merge of the four splits: (2 -> 0, 3 -> 1), then 1 -> 0 ------------
  auto put = [&](int slot) {
    float* d = smem + slot * ST_FLOATS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) d[(db * 16 + r) * 64 + lane] = acc[db][r];
    d[DB * 16 * 64 + lane] = m_run;
    d[DB * 16 * 64 + 64 + lane] = l_run;
  };
  auto take = [&](int slot) {
    const float* d = smem + slot * ST_FLOATS;
    const float m_o = d[DB * 16 * 64 + lane];
    const float l_o = d[DB * 16 * 64 + 64 + lane];
    const float m = fmaxf(m_run, m_o);
    const float a = m_run == -INFINITY ? 0.f : exp2_fast(m_run - m);
    const float bo = m_o == -INFINITY ? 0.f : exp2_fast(m_o - m);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = a * acc[db][r] + bo * d[(db * 16 + r) * 64 + lane];
    l_run = a * l_run + bo * l_o;
    m_run = m;
  };
  __syncthreads();  // the K/V super-tile is no longer read
  if (sp >= 2) put(sp - 2);
  __syncthreads();
  if (sp < 2) take(sp);
  __syncthreads();
  if (sp == 1) put(0);
  __syncthreads();
  if (sp != 0) return;
  take(0);

  if (qw >= p.Sq) return;
  const float l_tot = halfwave_sum(l_run);
  if (qi >= p.Sq) return;
  const float inv = 1.0f / l_tot;
  float* orow = (float*)((unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq) + (size_t)qi * p.o_ss);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      *(float4*)(orow + d) = make_float4(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv,
                                         acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv);
    }
  if (g == 0 && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
  // hipLaunchKernel reports the status of this launch alone.
  AttnParams arg = p;
  void* args[] = {&arg};
  // Small grids leave most matrix units idle: one workgroup per 32 query rows
  // instead, its four waves splitting the keys. Measured, the split is faster
  // up to 128 workgroups of 128 rows and slower from 192 (at d = 128 one split
  // workgroup fills a CU's LDS, so four times the grid takes several rounds).
  if (grid <= 128 && p.Sk > 32) {
    arg.n_qtiles = (p.Sq + 31) / 32;
    const unsigned grid32 = (unsigned)arg.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
    return hipLaunchKernel((const void*)&attn_fwd_f32_split_kernel<D, CAUSAL>, dim3(grid32), dim3(256), args, 0,
                           stream);
  }
  // Register prefetch of the next tile: always at d = 128 (one wave per SIMD
  // either way), at d = 64 up to 256 workgroups (measured faster there, slower
  // from 1024 up, where residency matters more).
  if (D == 128 || grid <= 256)
    return hipLaunchKernel((const void*)&attn_fwd_f32_kernel<D, CAUSAL, true>, dim3(grid), dim3(256), args, 0,
                           stream);
  return hipLaunchKernel((const void*)&attn_fwd_f32_kernel<D, CAUSAL, false>, dim3(grid), dim3(256), args, 0,
                         stream);
}

int f32_block_m() { return 128; }

hipError_t launch_attn_f32(const AttnParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
  if (d == 32) return causal ? launch_one<32, true>(p, stream) : launch_one<32, false>(p, stream);
  return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace sdpa18
