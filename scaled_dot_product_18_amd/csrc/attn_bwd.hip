// Attention backward pass for gfx950: dQ, dK, dV from Q, K, V, O, dO and the
// forward's log-sum-exp, bf16 in and out, fp32 accumulation.
//
// The gradients are the chain rule through the forward's three steps (codelab
// "Accelerate attention on GPU with cuDNN and TransformerEngine", section 4),
// and the attention weights are recomputed tile by tile from the stored
// per-row statistic instead of being kept (article "Self-attention, CUDA
// kernels and FlashAttention", section 3):
//   P = exp(scale Q K^T - lse)         dV = P^T dO         dP = dO V^T
//   dS = P * (dP - delta), delta_i = sum_c dO_ic O_ic    (= sum_j P_ij dP_ij)
//   dQ = scale dS K                    dK = scale dS^T Q
// Two kernels on one stream:
//  * attn_bwd_dq_kernel: one workgroup per 128 queries of one (batch, query
//    head); it first computes delta of its queries from their dO and O rows
//    and stores it (with lse * log2(e)) in the caller's workspace for the
//    second kernel. K/V tiles of 64 keys stream HBM -> LDS as in the forward. The
//    products are transposed as in the forward kernels (lane = query column):
//    S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16, the per-row
//    lse and delta are lane scalars, and dS^T rounded to bf16 is directly the
//    B operand of dQ^T += K^T dS^T, whose K^T operand is a transposing LDS read;
//  * attn_bwd_dkdv_kernel: one workgroup per 128 keys of one (batch, KV head),
//    lane = key column: the wave's 32 K and V rows sit in VGPRs as the B
//    operands of S = Q K^T and dP = dO V^T, Q and dO tiles of 64 queries stream
//    through LDS for every query head of the KV head's group (so GQA/MQA sums
//    over the group without atomics), and P, dS rounded to bf16 are the B
//    operands of dV^T += dO^T P and dK^T += Q^T dS.
// Under the causal mask (query i sees keys j <= i + Sk - Sq) tiles that see
// nothing are skipped and only edge blocks are masked.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {
namespace bwd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBufferConfig = 0x00020000;  // word 3 of a raw buffer resource: 32-bit data format

template <int D>
struct Cfg {
  static constexpr int RB = 2 * D;            // bytes per row
  static constexpr int CH = RB / 16;          // 16-byte chunks per row
  static constexpr int BT = 64;               // rows of a streamed tile
  static constexpr int TILE = BT * RB;        // bytes of one streamed tile
  static constexpr int DMA = TILE / 1024 / 4; // 1 KB wave-wide DMA loads per tile per wave
  static constexpr int QS = D / 16;           // MFMAs per 32x32 product over d
  static constexpr int DB = D / 32;           // 32-dim output blocks
  static_assert(DMA * 4 * 1024 == TILE, "4 waves cover a tile");
};

// Chunk swizzles. Tiles read only row-wise (16 lanes at 16 rows, one chunk)
// use row_swz. Tiles also read through the transposing read (lanes 0-31: 4
// consecutive rows, 64 bytes each) use dual_swz, which keeps both kinds free
// of bank conflicts: at d = 128 the row's two low bits pick the chunk's two
// high bits (4 consecutive rows cover the four 64-byte quarters of the banks)
// and its next two bits the chunk's low bits (16 consecutive rows cover all 16
// chunks); at d = 64, where two 128-byte rows share the banks, bit 1 of the
// row picks the chunk's high bit and bits 2-3 its low bits.
template <int D>
__device__ __forceinline__ int row_swz(int row) {
  return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int dual_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// A pointer the whole wave holds, moved into scalar registers: a buffer
// resource built from it then needs no per-lane loop around its loads.
__device__ __forceinline__ void* uniform_ptr(const void* ptr) {
  const unsigned long long a = (unsigned long long)ptr;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return (void*)(((unsigned long long)hi << 32) | lo);
}

// This wave's DMA loads of tile t of a row-major [rows, D] bf16 array, HBM ->
// LDS (lane l of load i fills dst + 1024 i + 16 l). Rows at or past the end
// fall outside the buffer's range and load as zeros.
template <int NLOAD>
__device__ __forceinline__ void dma_tile(const unsigned char* base, int tile_bytes, int t, int total_bytes,
                                         const unsigned* off, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(base + t * tile_bytes), (short)0, __builtin_amdgcn_readfirstlane(total_bytes - t * tile_bytes),
      kBufferConfig);
#pragma unroll
  for (int i = 0; i < NLOAD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * i), 16, off[i], 0, 0, 0);
}

// Offsets of the transposing reads that form a 32 (dim) x 16 (row) A operand
// from a row-major tile: in each 16-lane group lane J reads 4 dims
// [dbase + 4(J%4), +4) of row (row_base + J/4); the lo read (hi = 0) covers
// rows 16kc + 4g + J/4, the hi read (hi = 1) the same rows + 8, each with its
// own row's swizzle (row_base is a multiple of 16, which the swizzle ignores).
// Element e of the operand then pairs with row 16kc + 8(e/4) + 4g + e%4, the
// row order of the packed accumulator operands below.
template <int D>
__device__ __forceinline__ int tr_offset(int lane, int db, int hi) {
  const int J = lane & 15;
  const int g = lane >> 5;
  const int r = 4 * g + (J >> 2) + 8 * hi;
  const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
  return r * (2 * D) + 16 * ((d >> 3) ^ dual_swz<D>(r)) + 2 * (d & 7);
}

// 64 consecutive fp32 per-row statistics of tile t (one per query of the tile)
// HBM -> LDS, lane l filling dst + 4 l; rows past the end load as zeros.
__device__ __forceinline__ void dma_stat(const float* base, int t, int total_bytes, int lane, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(base + 64 * t), (short)0, __builtin_amdgcn_readfirstlane(total_bytes - 256 * t), kBufferConfig);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, 4 * lane, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* p, int lo_off, int hi_off) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + lo_off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi_off));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Stores a wave's 32-row output tile, scaled by sc and rounded to bf16. Lane
// (i32, g) holds dims 32 db + 8 q4 + 4 g + [0, 4) of tile row i32 in acc[db]
// registers 4 q4 .. 4 q4 + 3, so the wave first writes the tile to its 32 * RB
// bytes of LDS (16-byte chunks XOR-swizzled by row) and reads it back as whole
// rows: each global store then covers 1 KB of contiguous rows instead of 16
// bytes of 32 rows. Rows at or past n_rows are not stored; the stores carry
// the non-temporal hint.
template <int D>
__device__ __forceinline__ void store_tile(const f32x16* acc, float sc, unsigned char* stage, unsigned char* out,
                                           int n_rows, int lane) {
  constexpr int RB = 2 * D, CH = RB / 16;
  const int i32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int chunk = 4 * db + q4;
      *(u32x2*)(stage + i32 * RB + 16 * (chunk ^ (i32 & (CH - 1))) + 8 * g) =
          u32x2{pack_bf16x2(acc[db][4 * q4] * sc, acc[db][4 * q4 + 1] * sc),
                pack_bf16x2(acc[db][4 * q4 + 2] * sc, acc[db][4 * q4 + 3] * sc)};
    }
  const int pchunk = lane % CH;
#pragma unroll
  for (int t = 0; t < 32 * RB / 1024; ++t) {
    const int r = (1024 / RB) * t + lane / CH;
    const u32x4 val = *(const u32x4*)(stage + r * RB + 16 * pchunk);
    if (r < n_rows) __builtin_nontemporal_store(val, (u32x4*)(out + (size_t)r * RB + 16 * (pchunk ^ (r & (CH - 1)))));
  }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void attn_bwd_dq_kernel(const BwdParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[C::TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  const int q0 = qt * 128;
  const int qw = q0 + 32 * wave;
  const int qi = qw + i32;
  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;
  const size_t kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Sk;
  const unsigned char* kbase = (const unsigned char*)p.k + kv_row0 * C::RB;
  const unsigned char* vbase = (const unsigned char*)p.v + kv_row0 * C::RB;

  const int kv_end = CAUSAL ? min(p.Sk, q0 + 128 + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + C::BT - 1) / C::BT;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles =
      !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / C::BT + 1) : n_tiles);

  // DMA slot s = 64 (DMA w + i) + lane: row s / CH, physical chunk s % CH.
  unsigned kdma[C::DMA], vdma[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int r = (64 * (C::DMA * wave + i) + lane) / C::CH;
    const int pc = lane % C::CH;
    kdma[i] = r * C::RB + 16 * (pc ^ dual_swz<D>(r));   // K: row reads and transposing reads
    vdma[i] = r * C::RB + 16 * (pc ^ row_swz<D>(r));  // V: row reads
  }

  // Q and dO fragments (B operands): step s, half g holds dims [16s + 8g, +8) of query qi.
  u32x4 qf[C::QS], dof[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) {
    const bool ok = qi < p.Sq;
    qf[s] = ok ? *(const u32x4*)((const unsigned char*)p.q + (qo_row0 + qi) * C::RB + 32 * s + 16 * g)
               : u32x4{0, 0, 0, 0};
    dof[s] = ok ? *(const u32x4*)((const unsigned char*)p.dout + (qo_row0 + qi) * C::RB + 32 * s + 16 * g)
                : u32x4{0, 0, 0, 0};
  }
  // delta = delta_mul * sum_c dO_c O_c of query qi: each half g of the wave
  // holds half of the row's dims (the dO fragments above, the O fragments
  // read here), and the halves meet across lanes l and l ^ 32. Half 0 also
  // stores delta and lse2 = lse * log2(e) for the dK/dV kernel. Padding rows
  // (qi >= Sq) have Q = dO = 0, lse = delta = 0: every dS there is 0.
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < C::QS; ++s) {
    const u32x4 of = qi < p.Sq ? *(const u32x4*)((const unsigned char*)p.o + (qo_row0 + qi) * C::RB + 32 * s + 16 * g)
                               : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < 4; ++w) dsum += bf16_lo(dof[s][w]) * bf16_lo(of[w]) + bf16_hi(dof[s][w]) * bf16_hi(of[w]);
  }
  const float dlt = halfwave_sum(dsum) * p.delta_mul;
  const float lse2 = qi < p.Sq ? p.lse[qo_row0 + qi] * kLog2e : 0.f;
  if (g == 0 && qi < p.Sq) {
    p.delta[qo_row0 + qi] = dlt;
    p.lse2[qo_row0 + qi] = lse2;
  }

  int k_rd[C::QS], v_rd[C::QS], kt_lo[C::DB], kt_hi[C::DB];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) {
    k_rd[s] = i32 * C::RB + 16 * ((2 * s + g) ^ dual_swz<D>(i32));
    v_rd[s] = i32 * C::RB + 16 * ((2 * s + g) ^ row_swz<D>(i32));
  }
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    kt_lo[db] = tr_offset<D>(lane, db, 0);
    kt_hi[db] = tr_offset<D>(lane, db, 1);
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  const float c = p.qk_scale_log2;

  // Query qi sees keys [0, vis_end): the causal bound and the sequence end.
  const int vis_end = CAUSAL ? min(p.Sk, qi + 1 + p.causal_off) : p.Sk;
  constexpr int LA = 4;  // MFMAs whose LDS operand reads are in flight ahead

  // S^T and dP^T of key block kb (32 keys) of a tile: S and dP MFMAs
  // alternate, each A operand read LA MFMAs ahead of the matrix core.
  auto sdp = [&](const unsigned char* kl, const unsigned char* vl, int kb, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int st = 0; st < C::QS; ++st) {
      const u32x4 a = *(const u32x4*)(kl + kb * 32 * C::RB + k_rd[st]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]), s,
                                                  0, 0, 0);
      const u32x4 b = *(const u32x4*)(vl + kb * 32 * C::RB + v_rd[st]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, dof[st]),
                                                   dp, 0, 0, 0);
    }
    constexpr int N = 2 * C::QS;
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LA < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // dS^T of key block kb rounded to bf16: dsf[2kb + j], element e <-> key
  // 32kb + 16j + 8(e/4) + 4g + e%4 of the tile. In blocks that reach past a
  // lane's visible keys the masked entries are set to 0 (a select, so an
  // overflowing exp of a masked score cannot leak).
  auto dscore = [&](int kv0, int kb, const f32x16& s, const f32x16& dp, u32x4* dsf) {
    const int kb0 = kv0 + 32 * kb;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = exp2_fast(__builtin_fmaf(s[r], c, -lse2)) * (dp[r] - dlt);
    const bool edge = (CAUSAL && kb0 + 31 > qw + p.causal_off) || kb0 + 32 > p.Sk;
    if (edge) {
      const int rel = vis_end - kb0 - 4 * g;  // register r (key kb0 + 8(r/4) + 4g + r%4) is visible iff below
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = (8 * (r >> 2) + (r & 3) < rel) ? ds[r] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) dsf[2 * kb + j][e2] = pack_bf16x2(ds[8 * j + 2 * e2], ds[8 * j + 2 * e2 + 1]);
  };

  auto compute_tile = [&](int kt, const unsigned char* kl, const unsigned char* vl) {
    const int kv0 = kt * C::BT;
    u32x4 dsf[4];
    f32x16 s, dp;
    sdp(kl, vl, 0, s, dp);
    __builtin_amdgcn_sched_barrier(0);
    dscore(kv0, 0, s, dp, dsf);
    __builtin_amdgcn_sched_barrier(0);
    sdp(kl, vl, 1, s, dp);
    __builtin_amdgcn_sched_barrier(0);
    dscore(kv0, 1, s, dp, dsf);
    // dQ^T += K^T dS^T. Its own scheduling region: the two transposing reads
    // of each operand run LA MFMAs ahead of the matrix core.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kl + 16 * kc * C::RB, kt_lo[db], kt_hi[db]),
                                                          __builtin_bit_cast(bf16x8, dsf[kc]), acc[db], 0, 0, 0);
    constexpr int NUP = C::DB * 4;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
    for (int i = 0; i < NUP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LA < NUP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  const int kv_bytes = p.Sk * C::RB;
  unsigned char* const kd0 = k_lds0 + 1024 * C::DMA * wave;
  unsigned char* const vd0 = v_lds0 + 1024 * C::DMA * wave;
  unsigned char* const kd1 = k_lds1 + 1024 * C::DMA * wave;
  unsigned char* const vd1 = v_lds1 + 1024 * C::DMA * wave;
  if (n_tiles > 0) {
    dma_tile<C::DMA>(kbase, C::TILE, 0, kv_bytes, kdma, kd0);
    dma_tile<C::DMA>(vbase, C::TILE, 0, kv_bytes, vdma, vd0);
  }
  __syncthreads();
  for (int kt = 0; kt < n_tiles; kt += 2) {
    if (kt + 1 < n_tiles) {
      dma_tile<C::DMA>(kbase, C::TILE, kt + 1, kv_bytes, kdma, kd1);
      dma_tile<C::DMA>(vbase, C::TILE, kt + 1, kv_bytes, vdma, vd1);
    }
    if (kt < wave_tiles) compute_tile(kt, k_lds0, v_lds0);
    __syncthreads();
    if (kt + 1 >= n_tiles) break;
    if (kt + 2 < n_tiles) {
      dma_tile<C::DMA>(kbase, C::TILE, kt + 2, kv_bytes, kdma, kd0);
      dma_tile<C::DMA>(vbase, C::TILE, kt + 2, kv_bytes, vdma, vd0);
    }
    if (kt + 1 < wave_tiles) compute_tile(kt + 1, k_lds1, v_lds1);
    __syncthreads();
  }

  // dQ = dq_mul * acc. The K/V tiles are idle after the last barrier: wave w
  // stages its 32 rows in 32 * RB bytes of them.
  if (!wave_active) return;
  unsigned char* stage = (wave < 2 ? k_lds0 : v_lds0) + (wave & 1) * (32 * C::RB);
  store_tile<D>(acc, p.dq_mul, stage, (unsigned char*)p.dq + (qo_row0 + qw) * C::RB, p.Sq - qw, lane);
}

// ---------------------------------------------------------------- dK, dV
// One wave per SIMD (the wave's K and V rows and its dK, dV accumulators take
// most of the register file), so the wave overlaps its own vector and matrix
// work: query tiles are software-pipelined, and one step runs the P/dS
// arithmetic of tile t (VALU) beside the S/dP products of tile t+1 (matrix
// core), then the dV/dK products of tile t. Q, dO and their statistics go
// through three LDS buffers: t, t+1 and the load of t+2 in flight.
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1)))
void attn_bwd_dkdv_kernel(const BwdParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char o_lds0[C::TILE];  // dO
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char o_lds1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds2[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char o_lds2[C::TILE];
  // lse2 and delta of a tile's 64 queries, streamed with the tile
  __shared__ __attribute__((aligned(256))) float st_lds0[2 * C::BT];
  __shared__ __attribute__((aligned(256))) float st_lds1[2 * C::BT];
  __shared__ __attribute__((aligned(256))) float st_lds2[2 * C::BT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  // Work item (key tile, query-head subset, batch, KV head), key tiles
  // ascending: under the mask the first keys see the most queries.
  const int BH = p.B * p.Hkv;
  const int kt = blockIdx.x / (BH * p.kv_split);
  int rem = blockIdx.x - kt * BH * p.kv_split;
  const int sp = rem / BH;  // query-head subset
  rem -= sp * BH;
  const int b = rem / p.Hkv;
  const int hk = rem - b * p.Hkv;
  const int heads = p.group / p.kv_split;

  const int k0 = kt * 128;
  const int kw = k0 + 32 * wave;
  const int kj = kw + i32;  // this lane's key
  const bool wave_active = kw < p.Sk;
  const size_t kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Sk;

  // K and V rows of this lane's key (B operands): step s, half g holds dims [16s + 8g, +8).
  u32x4 kf[C::QS], vf[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) {
    const bool ok = kj < p.Sk;
    kf[s] = ok ? *(const u32x4*)((const unsigned char*)p.k + (kv_row0 + kj) * C::RB + 32 * s + 16 * g)
               : u32x4{0, 0, 0, 0};
    vf[s] = ok ? *(const u32x4*)((const unsigned char*)p.v + (kv_row0 + kj) * C::RB + 32 * s + 16 * g)
               : u32x4{0, 0, 0, 0};
  }

  unsigned qdma[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int r = (64 * (C::DMA * wave + i) + lane) / C::CH;
    qdma[i] = r * C::RB + 16 * ((lane % C::CH) ^ dual_swz<D>(r));  // Q and dO: row and transposing reads
  }
  int q_rd[C::QS], t_lo[C::DB], t_hi[C::DB];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) q_rd[s] = i32 * C::RB + 16 * ((2 * s + g) ^ dual_swz<D>(i32));
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    t_lo[db] = tr_offset<D>(lane, db, 0);
    t_hi[db] = tr_offset<D>(lane, db, 1);
  }

  f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float c = p.qk_scale_log2;
  const int off = p.causal_off;
  // Query tiles from the first one that sees a key of this workgroup (i >= k0 - off; all without the mask).
  const int t_first = CAUSAL ? max(0, k0 - off) / C::BT : 0;
  const int n_qt = (p.Sq + C::BT - 1) / C::BT;
  // Tiles from t_nomask on lie wholly below the diagonal for every key of the
  // workgroup (query 64 t sees key k0 + 127).
  const int t_nomask = CAUSAL ? (k0 + 127 - off + C::BT - 1) / C::BT : 0;

  // The work of one 64-query tile t for this wave's 32 keys, in two 32-query
  // blocks qb (lane = key kj; register r on half g <-> query 32qb + 8(r/4) + 4g + r%4):
  //   A(qb): S = Q K^T and dP = dO V^T, 2 D/16 MFMAs with a row read of Q or dO each;
  //   B(qb): P = exp2(c S - lse2) under the mask, dS = P (dP - delta), rounded
  //          to bf16 as B operands, four groups of 4 elements (VALU);
  //   C(qb): dV^T += dO^T P, dK^T += Q^T dS, 2 D/16 MFMAs with two transposing reads each.
  // One pipeline step for tile t runs four parts of 4-MFMA sub-chunks (four
  // per part at d = 128, two at d = 64), each sub-chunk beside its share of
  // vector work where there is one, with the next sub-chunk's operands read
  // ahead; fences keep the compiler from regrouping them:
  //    part 0  A(t, 1)   | B(t, 0)        part 2  A(t+1, 0) | -
  //    part 1  C(t, 0)   | B(t, 1)        part 3  C(t, 1)   | -
  // A(t+1, 0) reads tile t+1's buffers, so they are loaded one step ahead
  // (three buffer sets: t, t+1, and t+2 in flight). Past the last tile it
  // runs on a stale buffer and its results are never used.
  // Query rows past Sq need no mask: their Q, dO, lse2 and delta load as
  // zeros, so dS = 0 and they add nothing to dV = P^T dO; keys past Sk are
  // never stored, and each key's gradients stay in its own lane.
  constexpr int NB = 2;
  f32x16 s[NB], dp[NB];
  u32x4 pf[NB][2], dsf[NB][2];
  float pr[NB][16], ds[NB][16];
  // A MFMA i of block qb (0 <= i < NP): S for i < QS, dP after, over dims st = i % QS.
  constexpr int NP = 2 * C::QS;  // MFMAs of one stage for one block (A and C alike: 4 DB = 2 QS)
  static_assert(NP == 4 * C::DB && NP % 4 == 0, "stage sizes");
  auto a_operand = [&](int i, const unsigned char* ql, const unsigned char* ol, int qb) {
    return *(const u32x4*)((i >= C::QS ? ol : ql) + 32 * qb * C::RB + q_rd[i % C::QS]);
  };
  // The mask enters S through the first MFMA's accumulator: s_init[qb] holds
  // -inf where the query of a register cannot see this lane's key (so P =
  // exp2(-inf) = 0 exactly) and 0 elsewhere; it is all zeros once the tiles
  // are past the diagonal. Block 1 of the current tile and block 0 of the
  // next are the ones a step starts.
  f32x16 s_init[NB] = {f32x16{}, f32x16{}};
  auto mask_init = [&](int t, int qb) {
    const int vis = t * C::BT + off - kj + 4 * g;  // query 32qb+8m+4g+e sees kj iff vis + 32qb + 8m + e >= 0
    f32x16 r;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) r[4 * m + e] = (vis >= -(32 * qb + 8 * m + e)) ? 0.f : -__builtin_inff();
    return r;
  };
  auto a_mfma = [&](int i, int qb, u32x4 a) {
    const int st = i % C::QS;
    if (i < C::QS)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, kf[st]),
                                                      st == 0 ? (CAUSAL ? s_init[qb] : f32x16{}) : s[qb], 0, 0, 0);
    else
      dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, vf[st]),
                                                       st == 0 ? f32x16{} : dp[qb], 0, 0, 0);
  };
  // C MFMA i of block qb: db = i / 4, kc = (i / 2) % 2; even i: dV (dO^T), odd i: dK (Q^T)
  auto c_operand = [&](int i, const unsigned char* ql, const unsigned char* ol, int qb) {
    const int db = i >> 2, kc = (i >> 1) & 1;
    return tr_operand(((i & 1) ? ql : ol) + (32 * qb + 16 * kc) * C::RB, t_lo[db], t_hi[db]);
  };
  auto c_mfma = [&](int i, int qb, bf16x8 a) {
    const int db = i >> 2, kc = (i >> 1) & 1;
    if ((i & 1) == 0)
      dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[qb][kc]), dv[db], 0, 0, 0);
    else
      dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, dsf[qb][kc]), dk[db], 0, 0, 0);
  };
  // B group m of block qb with its statistics (lse2, delta of queries 32qb + 8m + 4g + 0..3).
  auto b_group = [&](int qb, int m, f32x4 l2, f32x4 dl) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * m + e;
      const float x = exp2_fast(__builtin_fmaf(s[qb][r], c, -l2[e]));
      pr[qb][r] = x;
      ds[qb][r] = x * (dp[qb][r] - dl[e]);
    }
    if (m & 1) {
      const int j = m >> 1;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        pf[qb][j][e2] = pack_bf16x2(pr[qb][8 * j + 2 * e2], pr[qb][8 * j + 2 * e2 + 1]);
        dsf[qb][j][e2] = pack_bf16x2(ds[qb][8 * j + 2 * e2], ds[qb][8 * j + 2 * e2 + 1]);
      }
    }
  };
  auto stat = [&](const float* stl, int qb, int m, int which) {
    return *(const f32x4*)(stl + which * C::BT + 32 * qb + 8 * m + 4 * g);
  };

  const int q_bytes = p.Sq * C::RB;
  const int st_bytes = p.Sq * 4;
  const int st_dst = wave == 0 ? 0 : 4 * C::BT;
  const unsigned char *qbase = nullptr, *obase = nullptr;
  const float* stat_src = nullptr;
  // Tile t's Q, dO and (waves 0 and 1: lse2, delta) statistics into one buffer set.
  auto load = [&](int t, unsigned char* ql, unsigned char* ol, float* stl) {
    dma_tile<C::DMA>(qbase, C::TILE, t, q_bytes, qdma, ql + 1024 * C::DMA * wave);
    dma_tile<C::DMA>(obase, C::TILE, t, q_bytes, qdma, ol + 1024 * C::DMA * wave);
    if (wave < 2) dma_stat(stat_src, t, st_bytes, lane, (unsigned char*)stl + st_dst);
  };

  // A step is 4 parts (0: A(t,1), 1: C(t,0), 2: A(t+1,0), 3: C(t,1)) of SUBS
  // sub-chunks of 4 MFMAs; the first two parts also run GPS of the 4 B groups
  // of their block per sub-chunk.
  constexpr int SUBS = NP / 4, GPS = 4 / SUBS, NSUB = 4 * SUBS;
  // Operands read ahead: A or C operands of the next sub-chunk, statistics of its B groups.
  u32x4 aop[4];
  bf16x8 cop[4];
  f32x4 nl2[GPS], ndl[GPS];
  auto fetch = [&](int k, const unsigned char* qc, const unsigned char* oc, const float* sc, const unsigned char* qn,
                   const unsigned char* on) {
    const int part = k / SUBS, i0 = 4 * (k % SUBS);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (part == 0) aop[u] = a_operand(i0 + u, qc, oc, 1);
      if (part == 1) cop[u] = c_operand(i0 + u, qc, oc, 0);
      if (part == 2) aop[u] = a_operand(i0 + u, qn, on, 0);
      if (part == 3) cop[u] = c_operand(i0 + u, qc, oc, 1);
    }
    if (part < 2) {
#pragma unroll
      for (int h = 0; h < GPS; ++h) {
        nl2[h] = stat(sc, part, GPS * (k % SUBS) + h, 0);
        ndl[h] = stat(sc, part, GPS * (k % SUBS) + h, 1);
      }
    }
  };
  auto step = [&](int t, unsigned char* qc, unsigned char* oc, float* sc, unsigned char* qn, unsigned char* on,
                  float* sn, unsigned char* qf_, unsigned char* of_, float* sf) {
    if (t + 2 < n_qt) load(t + 2, qf_, of_, sf);
    if (CAUSAL && t <= t_nomask) {  // (at t_nomask both come out all zeros)
      s_init[1] = mask_init(t, 1);
      s_init[0] = mask_init(t + 1, 0);
    }
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
      const int part = k / SUBS, i0 = 4 * (k % SUBS);
      u32x4 a_cur[4];
      bf16x8 c_cur[4];
      f32x4 l2[GPS], dl[GPS];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a_cur[u] = aop[u];
        c_cur[u] = cop[u];
      }
#pragma unroll
      for (int h = 0; h < GPS; ++h) {
        l2[h] = nl2[h];
        dl[h] = ndl[h];
      }
      // next sub-chunk's operands (sub-chunk NSUB is the next step's 0: tile t+1's A(1) and B(0) data)
      if (k < NSUB - 1)
        fetch(k + 1, qc, oc, sc, qn, on);
      else
        fetch(0, qn, on, sn, nullptr, nullptr);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (part == 0) a_mfma(i0 + u, 1, a_cur[u]);
        if (part == 1) c_mfma(i0 + u, 0, c_cur[u]);
        if (part == 2) a_mfma(i0 + u, 0, a_cur[u]);
        if (part == 3) c_mfma(i0 + u, 1, c_cur[u]);
      }
      if (part < 2) {
#pragma unroll
        for (int h = 0; h < GPS; ++h) b_group(part, GPS * (k % SUBS) + h, l2[h], dl[h]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  for (int gq = sp * heads; gq < (sp + 1) * heads; ++gq) {
    if (t_first >= n_qt) break;
    const int hq = hk * p.group + gq;
    const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;
    qbase = (const unsigned char*)p.q + qo_row0 * C::RB;
    obase = (const unsigned char*)p.dout + qo_row0 * C::RB;
    // wave 0 streams lse2, wave 1 delta: 64 floats per tile, one 4-byte DMA per lane
    stat_src = (wave == 0 ? p.lse2 : p.delta) + qo_row0;
    load(t_first, q_lds0, o_lds0, st_lds0);
    if (t_first + 1 < n_qt) load(t_first + 1, q_lds1, o_lds1, st_lds1);
    __syncthreads();
    // A(t_first, 0), then the first step's operands
    if (CAUSAL) s_init[0] = mask_init(t_first, 0);
    // (the operands in batches of eight, read before their MFMAs)
#pragma unroll
    for (int i0 = 0; i0 < NP; i0 += 8) {
      u32x4 a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = a_operand(i0 + u, q_lds0, o_lds0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) a_mfma(i0 + u, 0, a[u]);
    }
    fetch(0, q_lds0, o_lds0, st_lds0, nullptr, nullptr);
    for (int t = t_first;;) {
      step(t, q_lds0, o_lds0, st_lds0, q_lds1, o_lds1, st_lds1, q_lds2, o_lds2, st_lds2);
      if (++t >= n_qt) break;
      step(t, q_lds1, o_lds1, st_lds1, q_lds2, o_lds2, st_lds2, q_lds0, o_lds0, st_lds0);
      if (++t >= n_qt) break;
      step(t, q_lds2, o_lds2, st_lds2, q_lds0, o_lds0, st_lds0, q_lds1, o_lds1, st_lds1);
      if (++t >= n_qt) break;
    }
  }

  if (!wave_active) return;
  if (p.kv_split > 1) {
    // This subset's fp32 partial sums; attn_bwd_dkdv_reduce_kernel adds the
    // subsets in index order. Lane (i32, g) holds dims 32 db + 8 q4 + 4 g + [0, 4).
    if (kj >= p.Sk) return;
    const size_t rows = (size_t)p.B * p.Hkv * p.Sk;
    float* pk = p.dkv_part + ((size_t)sp * rows + kv_row0 + kj) * D;
    float* pv = pk + (size_t)p.kv_split * rows * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        *(float4*)(pk + d) = float4{dk[db][4 * q4] * p.dk_mul, dk[db][4 * q4 + 1] * p.dk_mul,
                                    dk[db][4 * q4 + 2] * p.dk_mul, dk[db][4 * q4 + 3] * p.dk_mul};
        *(float4*)(pv + d) = float4{dv[db][4 * q4] * p.dv_mul, dv[db][4 * q4 + 1] * p.dv_mul,
                                    dv[db][4 * q4 + 2] * p.dv_mul, dv[db][4 * q4 + 3] * p.dv_mul};
      }
    return;
  }
  // dK = dk_mul * dk, dV = dv_mul * dv. The Q and dO tiles are idle after the
  // last barrier: wave w stages its 32 dK rows in the Q tiles and its dV rows
  // in the dO tiles.
  const int half = (wave & 1) * (32 * C::RB);
  store_tile<D>(dk, p.dk_mul, (wave < 2 ? q_lds0 : q_lds1) + half, (unsigned char*)p.dk + (kv_row0 + kw) * C::RB,
                p.Sk - kw, lane);
  store_tile<D>(dv, p.dv_mul, (wave < 2 ? o_lds0 : o_lds1) + half, (unsigned char*)p.dv + (kv_row0 + kw) * C::RB,
                p.Sk - kw, lane);
}

// dK and dV from the fp32 partials of the query-head subsets, summed in
// subset order (deterministic) and rounded to bf16; 8 dims per thread.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void attn_bwd_dkdv_reduce_kernel(const BwdParams p,
                                                                                                   int d) {
  const size_t n8 = (size_t)p.B * p.Hkv * p.Sk * d / 8;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t part = n8 * 8;  // floats per subset and tensor
  for (int tensor = 0; tensor < 2; ++tensor) {
    const float* src = p.dkv_part + (size_t)tensor * p.kv_split * part + 8 * i;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.kv_split; ++sp) {
      const float4 a = *(const float4*)(src + sp * part);
      const float4 b = *(const float4*)(src + sp * part + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    unsigned char* dst = (unsigned char*)(tensor == 0 ? p.dk : p.dv) + 16 * i;
    *(u32x4*)dst = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7])};
  }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const BwdParams& bp, hipStream_t stream) {
  BwdParams arg = bp;
  void* args[] = {&arg};
  hipError_t e = hipLaunchKernel((const void*)&attn_bwd_dq_kernel<D, CAUSAL>,
                      dim3((unsigned)bp.n_qtiles * (unsigned)bp.B * (unsigned)bp.Hq), dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel((const void*)&attn_bwd_dkdv_kernel<D, CAUSAL>,
                      dim3((unsigned)bp.n_ktiles * (unsigned)bp.B * (unsigned)bp.Hkv * (unsigned)bp.kv_split),
                      dim3(256), args, 0, stream);
  if (e != hipSuccess || bp.kv_split == 1) return e;
  int d = D;
  void* rargs[] = {&arg, &d};
  const size_t n8 = (size_t)bp.B * bp.Hkv * bp.Sk * D / 8;
  return hipLaunchKernel((const void*)&attn_bwd_dkdv_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256),
                         rargs, 0, stream);
}

// fp8 codes -> bf16, 16 per thread: E4M3 (the forward format) for q, k, v and
// E5M2 (the gradient format) for dout. Both are exact: bf16 has more exponent
// range and more mantissa bits than either.
template <bool E5M2>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_bwd_widen_kernel(const unsigned char* src, unsigned char* dst, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 x = *(const u32x4*)(src + 16 * i);
  u32x4 lo, hi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 a, b;
    if (E5M2) {
      a = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x[w], 1.0f, false);
      b = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x[w], 1.0f, true);
    } else {
      a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false);
      b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true);
    }
    const uint32_t wa = __builtin_bit_cast(uint32_t, a), wb = __builtin_bit_cast(uint32_t, b);
    if (w < 2) {
      lo[2 * w] = wa;
      lo[2 * w + 1] = wb;
    } else {
      hi[2 * (w - 2)] = wa;
      hi[2 * (w - 2) + 1] = wb;
    }
  }
  *(u32x4*)(dst + 32 * i) = lo;
  *(u32x4*)(dst + 32 * i + 16) = hi;
}

template <bool E5M2>
hipError_t widen(const void* src, void* dst, size_t n, hipStream_t stream) {
  // n is a multiple of 16 (rows of 32, 64 or 128 elements)
  const size_t n16 = n / 16;
  const unsigned char* s8 = (const unsigned char*)src;
  unsigned char* d8 = (unsigned char*)dst;
  void* args[] = {&s8, &d8, (void*)&n16};
  return hipLaunchKernel((const void*)&attn_bwd_widen_kernel<E5M2>, dim3((unsigned)((n16 + 255) / 256)), dim3(256),
                         args, 0, stream);
}

}  // namespace bwd

hipError_t launch_attn_bwd_fp8(const BwdParams& bp, void* q16, void* k16, void* v16, void* do16, int d, bool causal,
                               hipStream_t stream) {
  const size_t nq = (size_t)bp.B * bp.Hq * bp.Sq * d, nk = (size_t)bp.B * bp.Hkv * bp.Sk * d;
  hipError_t e = bwd::widen<false>(bp.q, q16, nq, stream);
  if (e == hipSuccess) e = bwd::widen<false>(bp.k, k16, nk, stream);
  if (e == hipSuccess) e = bwd::widen<false>(bp.v, v16, nk, stream);
  if (e == hipSuccess) e = bwd::widen<true>(bp.dout, do16, nq, stream);
  if (e != hipSuccess) return e;
  BwdParams w = bp;
  w.q = q16;
  w.k = k16;
  w.v = v16;
  w.dout = do16;
  return launch_attn_bwd_bf16(w, d, causal, stream);
}

hipError_t launch_attn_bwd_bf16(const BwdParams& bp, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? bwd::launch_d<128, true>(bp, stream) : bwd::launch_d<128, false>(bp, stream);
  return causal ? bwd::launch_d<64, true>(bp, stream) : bwd::launch_d<64, false>(bp, stream);
}

}  // namespace sdpa18
