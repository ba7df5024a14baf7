// Fused scaled dot-product attention forward for gfx950: eight waves in
// matrix-core / vector-unit ping-pong over the two halves of a workgroup's
// keys, at head dims 64 and 128 on bf16 or fp8-e4m3fn inputs (bf16 output).
//
// The method is the FlashAttention forward pass ("Self-attention, CUDA kernels
// and FlashAttention", section 3): K and V stream through on-chip tiles, the
// scores of a tile exist only in registers, a running reference maximum and
// normaliser rescale the partial output as tiles arrive (online softmax), and
// only O and the per-row log-sum-exp are written. The arithmetic is the
// codelab's three steps ("Accelerate attention on GPU with cuDNN and
// TransformerEngine", intro and section 4) with the lower-triangular mask of
// its section 7 and the shared KV heads of its section 9.
//
// At d = 64 a tile's 16 MFMAs take half the time of its softmax on the vector
// unit, and a wave that runs both in turn leaves each unit idle while it runs
// the other. At d = 128 the 256-row ping-pong kernel of attn_fwd_bf16_pp.hip is
// faster on large grids, but on grids that do not fill the CUs this kernel's
// 128-row q-tiles double the workgroups and halve each one's chain of tiles.
// Here the two waves of a SIMD own the same 32 query rows and split the
// workgroup's key tiles: group 0 (waves 0-3) takes the first half, group 1
// (waves 4-7) the second. Each wave's chain of phases
//   M(m): O^T += V(m-1)^T . P(m-1)^T  and  S(m)^T = K(m) . Q^T - m_ref  (16 MFMAs; M0 only the scores)
//   V(m): mask, P(m) = exp2(c S(m)), row sums, reference check
// runs with group 0 in M on even global phases and group 1 in M on odd ones,
// so on every SIMD one wave feeds the matrix core while the other keeps the
// vector unit busy; a workgroup barrier separates phases. At the end group 1
// leaves its partial state (reference maximum, row sums, unnormalised O) in
// LDS and group 0 merges the two halves, as two blocks of the same softmax.
//
// K/V: each group streams its own tiles through its own two K and two V slots
// (8 KB each at d = 64, 64 KB for the workgroup with bf16 inputs; 16 KB and
// 128 KB at d = 128). Both groups load their K(n+1) and V(n) HBM -> LDS
// (buffer_load ... lds, 2 or 4 KB per wave and tensor) in global phase 2n,
// group 0 after the MFMAs of its M(n), group 1 at the start of its V(n-1), and
// wait for them at the barrier that ends phase 2n+1. Tile layouts and swizzles
// are those of the four-wave d = 64 kernel and of the 256-row d = 128
// ping-pong kernel: S^T and O^T are computed transposed on
// v_mfma_f32_32x32x16_bf16 so that one lane owns one query column, the
// bf16-rounded score accumulator is the P^T operand, and V^T comes from the
// row-major V tile through ds_read_b64_tr_b16.
//
// e4m3 inputs: S^T = K . Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// E8M0 scales, d / 64 MFMAs per 32-key block (K depth 64), into the same
// accumulator layout, so the softmax, P and the P.V MFMAs are those of the
// bf16 form. K tiles (4 or 8 KB of e4m3) go HBM -> LDS by DMA. V tiles go HBM
// -> registers (16 or 32 codes per lane) and are widened exactly to bf16 into
// the bf16 V layout at the end of an M phase, the short one at d = 64: group 0
// loads V(n+1) after its M(n) and stores it after its M(n+1), group 1 loads
// V(n) at the start of its V(n-1) and stores it after its M(n).
// The descales of Q and K are folded into the exponent's multiplier and that
// of V into the final 1/l.
//
// Softmax reference: as in the d = 128 ping-pong kernel, the first Q.K^T MFMA
// of a tile starts from -m_ref, the reference is set from the first tile with
// a visible key and moves only when a tile's partial row sums exceed 2^12.
// Under the causal mask a row may see no key of the second half's first tiles
// (or of the whole half); such a row keeps reference 0 and zero sums until its
// first visible key, and a half without one enters the merge with weight 0.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {
namespace ppk {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BM = 128;               // query rows per workgroup: four 32-row blocks, one per SIMD
constexpr int BN = 64;                // keys per tile
constexpr int kE8M0One = 127;         // E8M0 block scale 2^0 of the fp8 MFMA
constexpr int KB = BN / 32;           // 32-key blocks of a score tile
constexpr int KC = BN / 16;           // 16-key chunks (K depth of P.V)

constexpr int LA = 4;  // MFMAs whose LDS operand reads are in flight ahead of the matrix core
// A lane's partial row sum of one tile above this (or not finite) makes the
// wave move its reference maximum; below it every probability is <= 2^12.
constexpr float kSumLimit = 4096.0f;
constexpr int kBufferConfig = 0x00020000;  // word 3 of a raw buffer resource (gfx9 family)

// XOR swizzles of the 16-byte chunks of a K row (16 consecutive rows at one
// logical chunk hit 8 distinct chunks on each bank half of a 128-byte row, 16
// distinct chunks of a 256-byte one) and of a V row (the 4 rows of a
// transposing read hit disjoint 32-byte pairs).
template <int D>
__device__ __forceinline__ int k_swizzle(int row) { return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1)); }
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  return D == 128 ? ((0xCA60 >> (4 * (row & 3))) & 15) : ((0x6420 >> (4 * (row & 3))) & 15);
}
// e4m3 K rows: at d = 64 (64 bytes, 4 chunks) 16 consecutive rows at one logical
// chunk hit 4 rows per 256 bytes of banks, which the XOR with bits 2-3 of the row
// spreads; at d = 128 (128 bytes) the rows are laid out as bf16 rows at d = 64.
template <int D>
__device__ __forceinline__ int k8_swizzle(int row) { return D == 128 ? k_swizzle<64>(row) : ((row >> 2) & 3); }

// This wave's share of one K or V tile, HBM -> LDS: lane l of load t fills the
// 16 bytes at dst + 1024 t + 16 l. The buffer starts at the tile's first row
// and ends with the sequence's last, so rows at or past Sk load as zeros.
template <int NL>
__device__ __forceinline__ void dma_tile(const unsigned char* base, int tile_bytes, int kt, int limit,
                                         const unsigned* off, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + kt * tile_bytes), (short)0, limit - kt * tile_bytes, kBufferConfig);
#pragma unroll
  for (int t = 0; t < NL; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * t), 16, off[t], 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int kWaitLgkm0 = 0xC07F;     // lgkmcnt(0), others unconstrained
constexpr int kWaitVm0Lgkm0 = 0x0070;  // vmcnt(0) lgkmcnt(0)

// Workgroup barrier after the given s_waitcnt, without a memory fence (a release
// fence on LDS would also wait for the DMA still in flight into the other slots).
template <int WAIT>
__device__ __forceinline__ void barrier_after() {
  __builtin_amdgcn_s_waitcnt(WAIT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool FP8, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_ppk_kernel(const AttnParams p) {
  static_assert(D == 64 || D == 128, "head dims");
  constexpr int RB = D * 2;             // bytes per bf16 K/V row in LDS
  constexpr int CH = RB / 16;           // 16-byte chunks per row
  constexpr int TILE = BN * RB;         // 8 or 16 KB
  constexpr int DMA = TILE / 1024 / 4;  // 1 KB wave-wide loads per tensor per wave (a group's 4 waves fill a tile)
  constexpr int RB8 = D;                // bytes per e4m3 K/V row
  constexpr int TILE8 = BN * RB8;       // 4 or 8 KB
  constexpr int QS8 = D / 64;           // e4m3 score MFMAs (K depth 64) per 32x32 score block
  constexpr int PPR = RB8 / 16;         // 16-byte pieces of an e4m3 V row
  constexpr int VL = PPR / 4;           // e4m3 V loads per lane and tile (a group's 256 lanes, 16 rows per wave)
  constexpr int DB = D / 32;            // 32-wide output blocks
  constexpr int QS = D / 16;            // MFMAs per 32x32 score block
  constexpr int KTILE = FP8 ? TILE8 : TILE;     // K slot bytes
  constexpr int KDMA = KTILE / 1024 / 4;        // 1 KB K loads per wave
  constexpr int KCH = (FP8 ? RB8 : RB) / 16;    // 16-byte chunks per K row
  constexpr int IRB = FP8 ? RB8 : RB;           // bytes per input K/V row
  // Slots of group 0 (first key half) and group 1, each a fixed LDS object.
  __shared__ __attribute__((aligned(1024))) unsigned char k0_lds0[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k0_lds1[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v0_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v0_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k1_lds0[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k1_lds1[KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v1_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v1_lds1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;
  const int group = wave >> 2;  // key half
  const int si = wave & 3;      // SIMD and 32-row block

  // ---- work item: (q-tile, batch, query head), as in the four-wave d = 64 kernel
  int qt_seq, b, hq;
  if (p.xcd_remap) {
    // Workgroup i runs on XCD i % 8: each XCD gets whole KV heads (every query
    // head of a group), q-tiles outermost so every XCD starts on the heaviest.
    const int xcd = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;
    const int per_qt = (p.B * p.Hkv / 8) * p.group;
    qt_seq = j / per_qt;
    const int rem = j - qt_seq * per_qt;
    const int pair = (rem / p.group) * 8 + xcd;
    const int gq = rem - (rem / p.group) * p.group;
    b = pair / p.Hkv;
    hq = (pair - b * p.Hkv) * p.group + gq;
  } else {
    const int BH = p.B * p.Hq;
    qt_seq = blockIdx.x / BH;
    const int rem = blockIdx.x - qt_seq * BH;
    b = rem / p.Hq;
    hq = rem - b * p.Hq;
  }
  const int qt = CAUSAL ? (p.n_qtiles - 1 - qt_seq) : qt_seq;
  const int hk = hq / p.group;
  const int q0 = qt * BM;
  const int qw = q0 + si * 32;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);
  const int k_tile = BN * p.k_ss, v_tile = BN * p.v_ss;
  const int k_limit = (p.Sk - 1) * p.k_ss + IRB, v_limit = (p.Sk - 1) * p.v_ss + IRB;

  // Key tiles of the workgroup: [0, h) for group 0, [h, n_tiles) for group 1.
  // T counts this wave's tiles of its half (those up to the last one holding
  // a key visible to one of its rows); full_tiles the tiles, from 0, that no
  // mask touches for any of its rows.
  const int kv_end = CAUSAL ? min(p.Sk, q0 + BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int h = (n_tiles + 1) / 2;
  const int lo = group == 0 ? 0 : h;
  const int n_mine = group == 0 ? h : n_tiles - h;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles = CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / BN + 1) : n_tiles;
  const int T = !wave_active ? 0 : max(0, min(n_mine, wave_tiles - lo));
  const int full_tiles = CAUSAL ? min(p.Sk / BN, (qw + 1 + p.causal_off) / BN) : p.Sk / BN;

  // ---- DMA: wave si of a group writes 1 KB blocks DMA*si .. DMA*si+DMA-1 of each tile
  unsigned kdma_off[KDMA], vdma_off[DMA];
#pragma unroll
  for (int t = 0; t < KDMA; ++t) {
    const int row = (64 * (KDMA * si + t) + lane) / KCH;
    kdma_off[t] = row * p.k_ss + 16 * ((lane % KCH) ^ (FP8 ? k8_swizzle<D>(row) : k_swizzle<D>(row)));
  }
#pragma unroll
  for (int t = 0; t < DMA; ++t) {
    const int row = (64 * (DMA * si + t) + lane) / CH;
    vdma_off[t] = row * p.v_ss + 16 * ((lane % CH) ^ v_swizzle<D>(row));
  }
  const int kdma_dst = 1024 * KDMA * si, dma_dst = 1024 * DMA * si;
  // e4m3 V: in load t lane l of wave si takes 16 codes, dims [16 (l % PPR), +16)
  // of row 16 si + (64 / PPR) t + l / PPR, and stores them widened (exactly) to
  // bf16 as two 16-byte chunks of the row-major bf16 V tile.
  unsigned v8_ld[VL];
  int v8_st0[VL], v8_st1[VL];
  u32x4 v8reg[VL];
#pragma unroll
  for (int t = 0; t < VL; ++t) {
    const int row = 16 * si + (64 / PPR) * t + lane / PPR, piece = lane % PPR;
    v8_ld[t] = row * p.v_ss + 16 * piece;
    v8_st0[t] = row * RB + 16 * ((2 * piece) ^ v_swizzle<D>(row));
    v8_st1[t] = row * RB + 16 * ((2 * piece + 1) ^ v_swizzle<D>(row));
    v8reg[t] = u32x4{0, 0, 0, 0};
  }

  // ---- Q fragment (B operand of S^T): step s, half g holds dims [16s+8g, +8) of row qi
  const float c = p.qk_scale_log2;
  u32x4 qf[QS];
  i32x8 qf8[QS8];  // e4m3: step h holds dims [64h + 32g, +32) of row qi, the B operand of the fp8 score MFMA
  if constexpr (FP8) {
#pragma unroll
    for (int hs = 0; hs < QS8; ++hs) {
      qf8[hs] = i32x8{};
      if (qi < p.Sq) {
        const u32x4 a0 = *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 64 * hs + 32 * g);
        const u32x4 a1 = *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 64 * hs + 32 * g + 16);
        qf8[hs] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qf[s] = (qi < p.Sq) ? *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 32 * s + 16 * g) : u32x4{0, 0, 0, 0};
  }

  // ---- LDS operand offsets: K row 32kb + i32 at logical chunk 2s + g (e4m3:
  // chunk 4(s/2) + 2g + s%2); V^T through the transposing read (lane J of a
  // 16-lane group reads 4 dims of key row 4g + J/4).
  int k_rd[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s)
    k_rd[s] = FP8 ? i32 * RB8 + 16 * ((4 * (s >> 1) + 2 * g + (s & 1)) ^ k8_swizzle<D>(i32))
                  : i32 * RB + 16 * ((2 * s + g) ^ k_swizzle<D>(i32));
  const int J = lane & 15;
  int v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int row = 4 * g + (J >> 2);
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
    v_rd[db] = row * RB + 16 * ((d >> 3) ^ v_swizzle<D>(row)) + 2 * (d & 7);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  f32x16 s[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
  u32x4 pf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) pf[kc] = u32x4{0, 0, 0, 0};
  // Reference maximum m_ref (dot-product units, equal on both halves of a
  // query) and its negation over an accumulator block, where the first Q.K^T
  // MFMA of a tile starts.
  float m_ref = 0.f;
  f32x16 negm = f32x16{};
  float l_run = 0.f;
  bool seen = false;      // this lane's row has met a visible key of the half
  bool all_seen = false;  // every row of the wave has

  // M phase m with K(m) in kl and V(m-1) in vl.
  auto pv_part = [&](const unsigned char* vl) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc) * RB + v_rd[db]));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc + 8) * RB + v_rd[db]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
      }
  };
  auto qk_part = [&](const unsigned char* kl) {
    if constexpr (FP8) {
      // d / 64 fp8 MFMAs (K depth 64) per 32-key block; in step h lane (i32, g)
      // supplies key row i32's dims [64h + 32g, +32)
#pragma unroll
      for (int hs = 0; hs < QS8; ++hs)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 a0 = *(const u32x4*)(kl + kb * 32 * RB8 + k_rd[2 * hs]);
          const u32x4 a1 = *(const u32x4*)(kl + kb * 32 * RB8 + k_rd[2 * hs + 1]);
          const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[hs], hs == 0 ? negm : s[kb], 0, 0, 0,
                                                                  kE8M0One, 0, kE8M0One);
        }
    } else {
#pragma unroll
      for (int st = 0; st < QS; ++st)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 a = *(const u32x4*)(kl + kb * 32 * RB + k_rd[st]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf[st]), st == 0 ? negm : s[kb],
                                                          0, 0, 0);
        }
    }
  };
  // M phase m (1 <= m <= T): for m = T the K slot holds a stale tile whose
  // scores are never read. The LDS operand reads run LA MFMAs ahead of the
  // matrix core (two transposing reads per P.V MFMA, one per Q.K^T MFMA).
  auto m_phase = [&](int m, const unsigned char* kl, const unsigned char* vl) {
    if (m > T) return;
    pv_part(vl);
    qk_part(kl);
    constexpr int NQK = FP8 ? KB * QS8 : KB * QS, RQK = FP8 ? 2 : 1;  // score MFMAs, reads per score MFMA
    constexpr int NPV = KC * DB, NMF = KC * DB + NQK;
    static_assert(LA <= NPV, "the prologue reads belong to P.V MFMAs");
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int j = i + LA;
      if (j < NPV)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j < NMF)
        __builtin_amdgcn_sched_group_barrier(0x100, RQK, 0);
    }
  };
  // M(0): no probabilities yet, so only S(0).
  auto m_first = [&](const unsigned char* kl) {
    if (T == 0) return;
    qk_part(kl);
    if constexpr (!FP8) {
      constexpr int NQK = KB * QS;
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + LA < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // p = exp2(c S) for the whole tile: the P^T operand of the next M phase
  // (rounded to bf16) and this lane's partial row sum (fp32, unrounded).
  auto exp_tile = [&]() -> float {
    float lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r = 8 * j + 2 * e2;
          const float p0 = exp2_fast(s[kb][r] * c), p1 = exp2_fast(s[kb][r + 1] * c);
          pf[2 * kb + j][e2] = pack_bf16x2(p0, p1);
          lt[e2] += p0;
          lt[e2] += p1;
        }
    return (lt[0] + lt[1]) + (lt[2] + lt[3]);
  };
  // V phase v: mask, probabilities and row sums of S(v). The reference moves
  // while a row of the wave has seen no visible key (a row's first visible
  // key sets it to that tile's maximum) and when a tile's partial sums show
  // probabilities beyond 2^12; softmax does not depend on the reference.
  auto v_phase = [&](int v) {
    if (v < 0 || v >= T) return;
    const int gt = lo + v;  // tile index in the sequence
    if (gt >= full_tiles) {
      // Register r of block kb on half g holds key gt*BN + 4g + (32kb + 8(r/4) + r%4).
      const int limit = (CAUSAL ? min(p.Sk - 1, qi + p.causal_off) : p.Sk - 1) - gt * BN - 4 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3) <= limit) ? s[kb][r] : -INFINITY;
    }
    float l_tile = 0.f;
    bool rebase = !all_seen;
    if (!rebase) {
      l_tile = exp_tile();
      rebase = __builtin_amdgcn_ballot_w64(!(l_tile <= kSumLimit)) != 0;
    }
    if (rebase) {
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halfwave_max(mx);  // -inf: no key of this tile is visible to the row
      const bool vis = mx > -INFINITY;
      const float delta = seen ? fmaxf(mx, 0.f) : (vis ? mx : 0.f);
      const float alpha = seen ? exp2_fast(-delta * c) : 1.f;  // unseen rows hold zero sums and output
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_ref += delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
      seen = seen || vis;
      all_seen = __builtin_amdgcn_ballot_w64(!seen) == 0;
      l_tile = exp_tile();
    }
    l_run += l_tile;
  };
  // e4m3 V tile n of the half into registers, and from there into a slot.
  auto load_v8 = [&](int n) {
    if (n >= n_mine) return;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (lo + n) * v_tile), (short)0, v_limit - (lo + n) * v_tile, kBufferConfig);
#pragma unroll
    for (int t = 0; t < VL; ++t)
      v8reg[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, v8_ld[t], 0, 0));
  };
  auto store_v8 = [&](int n, unsigned char* dst) {
    __builtin_amdgcn_sched_barrier(0);
    if (n >= n_mine) return;
#pragma unroll
    for (int t = 0; t < VL; ++t) {
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v8reg[t][j], 1.0f, false));
        w[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v8reg[t][j], 1.0f, true));
      }
      *(u32x4*)(dst + v8_st0[t]) = u32x4{w[0], w[1], w[2], w[3]};
      *(u32x4*)(dst + v8_st1[t]) = u32x4{w[4], w[5], w[6], w[7]};
    }
  };
  // Loads of the group's K(n+1) and V (tile indices within its half): bf16 V(n)
  // by DMA; e4m3 V(n+1) (group 0, which stores it in M(n+1)) or V(n) (group 1,
  // which stores it in M(n)) into registers.
  auto dma_phase = [&](int n, unsigned char* k_dst, unsigned char* v_dst) {
    if (n + 1 < n_mine) dma_tile<KDMA>(kbase, k_tile, lo + n + 1, k_limit, kdma_off, k_dst + kdma_dst);
    if constexpr (FP8) {
      load_v8(group == 0 ? n + 1 : n);
    } else {
      if (n < n_mine) dma_tile<DMA>(vbase, v_tile, lo + n, v_limit, vdma_off, v_dst + dma_dst);
    }
  };
  // (bf16: nothing; the DMA writes the slot)
  auto store_v = [&](int n, unsigned char* dst) {
    if constexpr (FP8) store_v8(n, dst);
  };

  // ---- global phases --------------------------------------------------------
  // Group 0 runs M(m) in global phase 2m and V(v) in 2v+1, group 1 M(m) in
  // 2m+1 and V(v) in 2v+2. Both load K(n+1) and V(n) in phase 2n into the
  // slots their M(n-1) read (phase 2n-2 or 2n-1) and wait for them before the
  // barrier that ends phase 2n+1; M(n+1) reads them in phase 2n+2 or 2n+3.
  // So two K slots and two V slots per group suffice. Both groups run n_trips
  // trips of four phases and the same number of barriers (group 1 skips its
  // last, which would follow M(2 n_trips), a phase past every wave's last tile).
  const int n_trips = (h + 2) / 2;  // covers M(0..h) and V(0..h-1) of the longer half
  if (group == 0) {
    if (n_mine > 0) dma_tile<KDMA>(kbase, k_tile, lo, k_limit, kdma_off, k0_lds0 + kdma_dst);
    if constexpr (FP8) load_v8(0);
    barrier_after<kWaitVm0Lgkm0>();
    m_first(k0_lds0);
    store_v(0, v0_lds0);
    dma_phase(0, k0_lds1, v0_lds0);
    barrier_after<kWaitLgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      v_phase(2 * k);
      barrier_after<kWaitVm0Lgkm0>();
      m_phase(2 * k + 1, k0_lds1, v0_lds0);
      store_v(2 * k + 1, v0_lds1);
      dma_phase(2 * k + 1, k0_lds0, v0_lds1);
      barrier_after<kWaitLgkm0>();
      v_phase(2 * k + 1);
      barrier_after<kWaitVm0Lgkm0>();
      m_phase(2 * k + 2, k0_lds0, v0_lds1);
      store_v(2 * k + 2, v0_lds0);
      dma_phase(2 * k + 2, k0_lds1, v0_lds0);
      barrier_after<kWaitLgkm0>();
    }
  } else {
    if (n_mine > 0) dma_tile<KDMA>(kbase, k_tile, lo, k_limit, kdma_off, k1_lds0 + kdma_dst);
    barrier_after<kWaitVm0Lgkm0>();
    dma_phase(0, k1_lds1, v1_lds0);  // phase 0: no score tile yet
    barrier_after<kWaitLgkm0>();
    m_first(k1_lds0);
    store_v(0, v1_lds0);
    barrier_after<kWaitVm0Lgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      dma_phase(2 * k + 1, k1_lds0, v1_lds1);
      v_phase(2 * k);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 1, k1_lds1, v1_lds0);
      store_v(2 * k + 1, v1_lds1);
      barrier_after<kWaitVm0Lgkm0>();
      dma_phase(2 * k + 2, k1_lds1, v1_lds0);
      v_phase(2 * k + 1);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 2, k1_lds0, v1_lds1);
      if (k + 1 < n_trips) {  // M(2 n_trips) is past every T, and V(2 n_trips) past the half
        store_v(2 * k + 2, v1_lds0);
        barrier_after<kWaitVm0Lgkm0>();
      }
    }
  }
  barrier_after<kWaitVm0Lgkm0>();  // every slot idle

  // ---- merge of the two halves ----------------------------------------------
  // Group 1 leaves, register-major with the 64 lanes contiguous, its partial O
  // in group 0's slot si and its reference (log2 units; the most negative
  // float when no key of the half was visible) and row sums in k1_lds0; the
  // group 0 wave of the same rows rescales both halves to the larger
  // reference and adds.
  // (4 KB per 32-wide output block: group 0's K and V slots, or with e4m3 K,
  // whose slots are half the size, the four V slots)
  unsigned char* const acc_slot = FP8 ? (si == 0 ? v0_lds0 : si == 1 ? v0_lds1 : si == 2 ? v1_lds0 : v1_lds1)
                                      : (si == 0 ? k0_lds0 : si == 1 ? k0_lds1 : si == 2 ? v0_lds0 : v0_lds1);
  float* const m_acc = (float*)acc_slot;
  float* const m_ml = (float*)k1_lds0 + si * 128;
  if (group == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) m_acc[(db * 16 + r) * 64 + lane] = acc[db][r];
    m_ml[lane] = seen ? m_ref * c : -__FLT_MAX__;
    m_ml[64 + lane] = l_run;
  }
  barrier_after<kWaitLgkm0>();
  if (group == 1 || !wave_active) return;
  // Every row of the first half sees key 0, so its reference is a real maximum.
  const float m_a = m_ref * c, m_b = m_ml[lane], l_b = m_ml[64 + lane];
  const float m_new = fmaxf(m_a, m_b);
  const float fa = exp2_fast(m_a - m_new), fb = exp2_fast(m_b - m_new);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * fa + m_acc[(db * 16 + r) * 64 + lane] * fb;
  const float l_tot = halfwave_sum(l_run * fa + l_b * fb);

  // ---- epilogue -------------------------------------------------------------
  // O = acc / l rounded to bf16 (times the descale of e4m3 V, else 1), staged
  // through LDS and read back as whole rows for 1 KB row stores with the
  // non-temporal hint; 16-byte chunks are XOR-swizzled by row. The stage (32 rows)
  // is the region this wave has just read its partner's state from: no other
  // wave uses it after the barrier, and the wave's own reads return first.
  const float inv = p.o_scale / l_tot;
  unsigned char* stage = acc_slot;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int chunk = 4 * db + q4;  // dims 32 db + 8 q4 + [0, 8); this lane's 4 of them start at 4 g
      *(u32x2*)(stage + i32 * RB + 16 * (chunk ^ (i32 & (CH - 1))) + 8 * g) =
          u32x2{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)};
    }
  unsigned char* obase = (unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq);
  const int pchunk = lane % CH;
#pragma unroll
  for (int t = 0; t < 32 * RB / 1024; ++t) {
    const int r = (1024 / RB) * t + lane / CH;
    const u32x4 val = *(const u32x4*)(stage + r * RB + 16 * pchunk);
    if (qw + r < p.Sq)
      __builtin_nontemporal_store(val, (u32x4*)(obase + (size_t)(qw + r) * p.o_ss + 16 * (pchunk ^ (r & (CH - 1)))));
  }
  if (g == 0 && qi < p.Sq && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_new + __log2f(l_tot)) * kLn2;
}

}  // namespace ppk

template <int D, bool FP8>
static hipError_t launch_ppk(const AttnParams& p, bool causal, hipStream_t stream) {
  // Same grid as the four-wave d = 64 kernels: ceil(Sq / 128) x B x Hq workgroups.
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
  AttnParams arg = p;
  void* args[] = {&arg};
  const void* fn = causal ? (const void*)&ppk::attn_fwd_ppk_kernel<D, FP8, true>
                          : (const void*)&ppk::attn_fwd_ppk_kernel<D, FP8, false>;
  return hipLaunchKernel(fn, dim3(grid), dim3(512), args, 0, stream);
}

// d = 128: the shapes this kernel takes over from the 256-row ping-pong kernels
// (bf16 and e4m3), counted in q-tiles of 128 rows over all heads and batches.
// Unmasked, at most one pass over the 256 CUs; causal, at most two, since the
// heaviest tiles start first and the light ones fill the second pass. A/B per
// 128-row tile count (bf16 / e4m3): unmasked 256 tiles 29.0 -> 25.8 / 22.4 ->
// 18.6 us, 384 tiles 34.6 -> 44.2 / 24.7 -> 34.5 us; causal 512 tiles (B2 H8/2
// T4096) 90.4 -> 76.6 / 70.4 -> 58.1 us, 768 tiles 84.0 -> 98.6 / 61.1 -> 75.2 us.
// The count ignores the KV heads, so GQA and MHA on repeated K/V run the same kernel.
bool ppk_takes_d128(const AttnParams& p, bool causal) {
  const long long tiles = (long long)((p.Sq + 127) / 128) * p.B * p.Hq;
  return tiles <= (causal ? 512 : 256);
}

hipError_t launch_attn_bf16_ppk(const AttnParams& p, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_ppk<128, false>(p, causal, stream) : launch_ppk<64, false>(p, causal, stream);
}

hipError_t launch_attn_fp8_ppk(const AttnParams& p, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_ppk<128, true>(p, causal, stream) : launch_ppk<64, true>(p, causal, stream);
}

}  // namespace sdpa18

