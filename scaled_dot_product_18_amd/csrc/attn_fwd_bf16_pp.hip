// Fused scaled dot-product attention forward for gfx950, bf16, head dim 128:
// eight waves per workgroup in matrix-core / vector-unit ping-pong.
//
// The method is the FlashAttention forward pass ("Self-attention, CUDA kernels
// and FlashAttention", section 3): K and V stream through on-chip tiles, the
// scores of a tile exist only in registers, a running row maximum and
// normaliser rescale the partial output as tiles arrive (online softmax), and
// only O and the per-row log-sum-exp are written. The arithmetic is the
// codelab's three steps ("Accelerate attention on GPU with cuDNN and
// TransformerEngine", intro and section 4) with the lower-triangular mask of
// its section 7 and the shared KV heads of its section 9.
//
// Work of one wave (32 query rows) over its T key tiles of 64 keys is a chain
// of phases  M0 V0 M1 V1 ... M(T-1) V(T-1) MT:
//   M(m): O^T += V(m-1)^T . P(m-1)^T  and  S(m)^T = K(m) . Q^T - m_ref   (32 MFMAs;
//         M0 has only the scores, 16 MFMAs)
//   V(m): mask, P(m) = exp2(c S(m)), row sums, reference check
// A workgroup holds 8 waves, two per SIMD: group A (waves 0-3) runs M phases
// on even global phases and V phases on odd ones, group B (waves 4-7) the
// other way round, so on every SIMD one wave feeds the matrix core while the
// other keeps the vector unit busy. A workgroup barrier separates global
// phases. The two waves of a SIMD own adjacent 32-row blocks, so they have the
// same number of key tiles.
//
// Rows of a workgroup: 256 rows of one query head, or, under the causal mask
// when 2 or 4 query heads share a KV head, 128 or 64 rows of each of them. With
// one head the causal diagonal gives the four SIMDs 1, 2, 3 and 4 tiles of the
// last four, and the phase barriers make all of them wait for the fourth; with
// 64 rows of four heads every wave reads the same K/V tiles and needs the same
// number of them.
//
// K/V tiles: K(n+1) and V(n) are loaded HBM -> LDS (buffer_load ... lds, 2 KB
// per wave) during global phase 2n and waited for before the barrier
// that ends phase 2n+1; K(m) is read in phases 2m (A) and 2m+1 (B), V(m-1)
// likewise, so two K slots and two V slots suffice. The loop is unrolled over
// four phases so that every slot is a fixed LDS object and the compiler can
// see that a read never touches the slot being filled.
//
// Q: each wave loads its 32 rows once, as whole rows through the same DMA
// into a staging buffer (1 KB of four rows per load; a fragment-shaped load
// from HBM would touch 32 rows per instruction), and reads its Q fragment from
// there with the K tile's swizzle.
//
// Lane layout (unchanged from the four-wave kernel): S^T and O^T are computed
// transposed on v_mfma_f32_32x32x16_bf16 so that one lane owns one query
// column; the bf16-rounded score accumulator is directly the P^T operand; V^T
// comes from the row-major V tile through ds_read_b64_tr_b16; XOR swizzles
// keep the operand reads free of bank conflicts.
//
// Softmax reference: the first Q.K^T MFMA of a tile starts from an accumulator
// holding -m_ref, so the scores arrive relative to a reference maximum and the
// vector unit only multiplies by c = scale*log2(e) and exponentiates. The
// reference is set from the first tile's maximum and moves only when a tile's
// partial row sums show probabilities above 2^12; softmax does not depend on
// the reference point, so this is exact and the per-tile row maximum is gone.
// Row sums are fp32 adds of the probabilities (v_dot2 on the packed values
// would stall the partner wave's matrix core).
#include "kernel_common.h"
#include "launch.h"



namespace sdpa18 {
namespace pp {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int WAVES = 8;
constexpr int BM = 32 * WAVES;  // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int RB = D * 2;       // bytes per K/V row
constexpr int CH = RB / 16;     // 16-byte chunks per row
constexpr int TILE = BN * RB;   // 16 KB
constexpr int DMA = TILE / 1024 / WAVES;  // 1 KB wave-wide loads per tensor per wave
constexpr int KB = BN / 32;     // 32-key blocks of a score tile
constexpr int KC = BN / 16;     // 16-key chunks (K depth of P.V)
constexpr int DB = D / 32;      // 32-wide output blocks
constexpr int QS = D / 16;      // MFMAs per 32x32 score block
static_assert(DMA == 2, "8 waves x 2 loads cover a 16 KB tile");

constexpr int LA = 4;  // MFMAs whose LDS operand reads are in flight ahead of the matrix core
// A lane's partial row sum of one tile above this (or not finite) makes the
// wave move its reference maximum; below it every probability is <= 2^12.
constexpr float kSumLimit = 4096.0f;
constexpr int kBufferConfig = 0x00020000;  // word 3 of a raw buffer resource (gfx9 family)

// XOR swizzles of the 16-byte chunks of a K row (16 rows at one logical chunk
// hit 16 distinct chunks) and of a V row (the 4 rows of a transposing read hit
// disjoint 32-byte pairs), which keep the operand reads free of bank conflicts.
__device__ __forceinline__ int k_swizzle(int row) { return row & 15; }
__device__ __forceinline__ int v_swizzle(int row) { return (0xCA60 >> (4 * (row & 3))) & 15; }

// This wave's share of one K or V tile, HBM -> LDS: DMA wave-wide loads, lane l
// of load t filling the 16 bytes at dst + 1024 t + 16 l. The tile is read
// through a raw buffer that starts at its first row and ends at the end of
// the sequence, so rows at or past Sk fall outside it and load as zeros.
__device__ __forceinline__ void dma_tile(const unsigned char* base, int tile_bytes, int kt, int limit,
                                         const unsigned* off, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + kt * tile_bytes), (short)0, limit - kt * tile_bytes, kBufferConfig);
#pragma unroll
  for (int t = 0; t < DMA; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * t), 16, off[t], 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int kWaitLgkm0 = 0xC07F;       // lgkmcnt(0), others unconstrained
constexpr int kWaitVm0Lgkm0 = 0x0070;    // vmcnt(0) lgkmcnt(0)

// Workgroup barrier after the given s_waitcnt. No memory fence: a release
// fence on LDS would also wait for every LDS DMA still in flight, which the
// even phases must not do. The empty asm statements keep the compiler from
// moving memory accesses across the barrier; the explicit wait makes this
// wave's LDS reads (and, with vmcnt(0), its DMA into LDS) complete first.
template <int WAIT>
__device__ __forceinline__ void barrier_after() {
  __builtin_amdgcn_s_waitcnt(WAIT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool CAUSAL, int HP>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_pp_kernel(const AttnParams p) {
  // The larger alignment places the K/V slots first: the operand reads reach
  // them through 16-bit immediate offsets.
  __shared__ __attribute__((aligned(4096))) unsigned char k_lds0[TILE];
  __shared__ __attribute__((aligned(4096))) unsigned char k_lds1[TILE];
  __shared__ __attribute__((aligned(4096))) unsigned char v_lds0[TILE];
  __shared__ __attribute__((aligned(4096))) unsigned char v_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char q_stage[WAVES * 32 * RB];

  // HP query heads of one KV head share the workgroup, BM / HP rows each: SIMD
  // si serves head si / (4 / HP), and its two waves own adjacent 32-row blocks.
  static_assert(HP == 1 || HP == 2 || HP == 4, "heads per workgroup");
  constexpr int RPH = BM / HP;  // query rows per head
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;
  const int group = wave >> 2;                          // 0: M on even phases, 1: M on odd phases
  const int si = wave & 3;                              // SIMD
  const int row_block = 2 * (si % (4 / HP)) + group;    // 32-row block within the head's rows
  const int hsub = si / (4 / HP);                       // head within the workgroup

  // ---- work item: (q-tile, batch, HP query heads) -----------------------------
  const int gh = p.group / HP;  // head packs per KV head
  int qt_seq, b, hq;
  if (p.xcd_remap) {
    const int xcd = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;
    const int per_qt = (p.B * p.Hkv / 8) * gh;
    qt_seq = j / per_qt;
    const int rem = j - qt_seq * per_qt;
    const int pair = (rem / gh) * 8 + xcd;
    const int gq = rem - (rem / gh) * gh;
    b = pair / p.Hkv;
    hq = (pair - b * p.Hkv) * p.group + gq * HP + hsub;
  } else {
    const int BH = p.B * (p.Hq / HP);
    qt_seq = blockIdx.x / BH;
    const int rem = blockIdx.x - qt_seq * BH;
    b = rem / (p.Hq / HP);
    hq = (rem - b * (p.Hq / HP)) * HP + hsub;
  }
  const int qt = CAUSAL ? (p.n_qtiles - 1 - qt_seq) : qt_seq;
  const int hk = hq / p.group;

  const int q0 = qt * RPH;
  const int qw = q0 + row_block * 32;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);
  // A tile of BN rows spans BN strides; the buffer of K (V) ends with the last
  // key's row, so rows at or past Sk load as zeros.
  const int k_tile = BN * p.k_ss, v_tile = BN * p.v_ss;
  const int k_limit = (p.Sk - 1) * p.k_ss + RB, v_limit = (p.Sk - 1) * p.v_ss + RB;

  const int kv_end = CAUSAL ? min(p.Sk, q0 + RPH + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + BN - 1) / BN;  // tiles any wave of the workgroup needs
  const bool wave_active = qw < p.Sq;
  const int T = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / BN + 1) : n_tiles);
  const int full_tiles = CAUSAL ? min(p.Sk / BN, (qw + 1 + p.causal_off) / BN) : p.Sk / BN;

  // ---- DMA: wave w writes 1 KB blocks DMA*w .. DMA*w+DMA-1 of each tile ----
  unsigned kdma_off[DMA], vdma_off[DMA];
  const int dma_pchunk = lane % CH;
#pragma unroll
  for (int t = 0; t < DMA; ++t) {
    const int row = (64 * (DMA * wave + t) + lane) / CH;
    kdma_off[t] = row * p.k_ss + 16 * (dma_pchunk ^ k_swizzle(row));
    vdma_off[t] = row * p.v_ss + 16 * (dma_pchunk ^ v_swizzle(row));
  }
  const int dma_dst = 1024 * DMA * wave;

  // ---- Q rows of this wave HBM -> LDS as whole rows (1 KB per load, four
  // rows), 16-byte chunks swizzled as in a K tile; rows at or past Sq load as
  // zeros. The fragments are read from there after the prologue's barrier.
  const float c = p.qk_scale_log2;
  unsigned char* q_mine = q_stage + wave * (32 * RB);
  if (wave_active) {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qbase + (size_t)qw * p.q_ss), (short)0, (p.Sq - qw - 1) * p.q_ss + RB, kBufferConfig);
#pragma unroll
    for (int t = 0; t < 32 * RB / 1024; ++t) {
      const int row = 4 * t + (lane >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(q_mine + 1024 * t), 16,
                                               row * p.q_ss + 16 * ((lane & 15) ^ k_swizzle(row)), 0, 0, 0);
    }
  }
  u32x4 qf[QS];

  int k_rd[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) k_rd[s] = i32 * RB + 16 * ((2 * s + g) ^ k_swizzle(i32));
  const int J = lane & 15;
  int v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int row = 4 * g + (J >> 2);
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
    v_rd[db] = row * RB + 16 * ((d >> 3) ^ v_swizzle(row)) + 2 * (d & 7);
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
  // query) and its negation replicated over an accumulator block: the first
  // Q.K^T MFMA of a tile starts from it, so the scores arrive as s - m_ref.
  float m_ref = 0.f;
  f32x16 negm = f32x16{};
  float l_run = 0.f;

  // M phase m with K(m) in kl and V(m-1) in vl.
  auto pv_part = [&](const unsigned char* vl) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc) * RB + v_rd[db]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc + 8) * RB + v_rd[db]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
      }
  };
  auto qk_part = [&](const unsigned char* kl) {
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 a = *(const u32x4*)(kl + kb * 32 * RB + k_rd[st]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, qf[st]), st == 0 ? negm : s[kb],
                                                        0, 0, 0);
      }
  };
  // M phase m (1 <= m <= T; M(0) is m_first below), one straight-line shape
  // for every m: for m = T the K slot holds a stale tile and the scores it
  // yields are never read. The LDS operand reads run LA MFMAs ahead of the
  // matrix core (two transposing reads per P.V MFMA, one read per Q.K^T MFMA).
  auto m_phase = [&](int m, const unsigned char* kl, const unsigned char* vl) {
    if (m > T) return;
    pv_part(vl);
    qk_part(kl);
    constexpr int NPV = KC * DB, NMF = KC * DB + KB * QS;
    static_assert(LA <= NPV, "the prologue reads belong to P.V MFMAs");
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int j = i + LA;
      if (j < NPV)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j < NMF)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // M(0): no probabilities yet, so only S(0) = K(0).Q^T.
  auto m_first = [&](const unsigned char* kl) {
    if (T == 0) return;
    qk_part(kl);
    constexpr int NQK = KB * QS;
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LA < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
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

  // V phase v: mask, probabilities and row sums of S(v). The scores already
  // have m_ref subtracted; the reference only moves on the first tile and when
  // a tile's partial sums show probabilities beyond 2^12 (softmax does not
  // depend on the reference point, so the result is unchanged).
  auto v_phase = [&](int v) {
    if (v < 0 || v >= T) return;
    if (v >= full_tiles) {
      // Register r of block kb on half g holds key v*BN + 4g + (32kb + 8(r/4) + r%4);
      // the key is visible iff that offset <= last visible key - v*BN - 4g.
      const int limit = (CAUSAL ? min(p.Sk - 1, qi + p.causal_off) : p.Sk - 1) - v * BN - 4 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3) <= limit) ? s[kb][r] : -INFINITY;
    }
    float l_tile = 0.f;
    bool rebase = (v == 0);
    if (!rebase) {
      l_tile = exp_tile();
      rebase = __builtin_amdgcn_ballot_w64(!(l_tile <= kSumLimit)) != 0;
    }
    if (rebase) {
      // Tile 0 always holds a visible key of every row (key 0), so its maximum is finite.
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halfwave_max(mx);
      const float delta = (v == 0) ? mx : fmaxf(mx, 0.f);
      if (v > 0) {
        const float alpha = exp2_fast(-delta * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      m_ref += delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
      l_tile = exp_tile();
    }
    l_run += l_tile;
  };

  // DMA issued at the start of global phase 2n: K(n+1) and V(n).
  auto dma_phase = [&](int n, unsigned char* k_dst, unsigned char* v_dst) {
    if (n + 1 < n_tiles) dma_tile(kbase, k_tile, n + 1, k_limit, kdma_off, k_dst + dma_dst);
    if (n < n_tiles) dma_tile(vbase, v_tile, n, v_limit, vdma_off, v_dst + dma_dst);
  };

  // ---- prologue: K(0) into slot 0, published before phase 0 ------------------
  if (n_tiles > 0) dma_tile(kbase, k_tile, 0, k_limit, kdma_off, k_lds0 + dma_dst);
  barrier_after<kWaitVm0Lgkm0>();
  // Q fragment (B operand of S^T): step s, half g holds dims [16s+8g, +8) of row i32.
#pragma unroll
  for (int s = 0; s < QS; ++s) qf[s] = *(const u32x4*)(q_mine + k_rd[s]);

  // ---- global phases ----------------------------------------------------------
  // Global phase p ends with a barrier that waits for this wave's LDS reads
  // and, when p is odd, for the DMA issued in phase p-1. Group A issues its
  // share of that DMA after the phase's MFMAs (its matrix work starts without
  // waiting for the load issue), group B before its softmax.
  //   phase 4k   : DMA K(2k+1)->k1, V(2k)->v0 | A: M(2k)   [k0, v1] | B: V(2k-1)
  //   phase 4k+1 :                            | A: V(2k)            | B: M(2k)   [k0, v1]
  //   phase 4k+2 : DMA K(2k+2)->k0, V(2k+1)->v1 | A: M(2k+1) [k1, v0] | B: V(2k)
  //   phase 4k+3 :                            | A: V(2k+1)          | B: M(2k+1) [k1, v0]
  // M(0) has no P.V and stands before each group's loop, which is rotated to
  // start one phase later. Each group runs its own loop of four-phase trips,
  // so a score tile never crosses a trip; both groups execute n_trips * 4 + 2
  // barriers after the prologue's (group B skips its last, which would follow
  // M(2 n_trips), a phase past every wave's last tile).
  const int n_trips = (n_tiles + 2) / 2;  // covers M(0..n_tiles) and V(0..n_tiles-1)
  if (group == 0) {
    m_first(k_lds0);
    dma_phase(0, k_lds1, v_lds0);
    barrier_after<kWaitLgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      v_phase(2 * k);
      barrier_after<kWaitVm0Lgkm0>();
      m_phase(2 * k + 1, k_lds1, v_lds0);
      dma_phase(2 * k + 1, k_lds0, v_lds1);
      barrier_after<kWaitLgkm0>();
      v_phase(2 * k + 1);
      barrier_after<kWaitVm0Lgkm0>();
      m_phase(2 * k + 2, k_lds0, v_lds1);
      dma_phase(2 * k + 2, k_lds1, v_lds0);
      barrier_after<kWaitLgkm0>();
    }
  } else {
    dma_phase(0, k_lds1, v_lds0);  // phase 0: no score tile yet
    barrier_after<kWaitLgkm0>();
    m_first(k_lds0);
    barrier_after<kWaitVm0Lgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      dma_phase(2 * k + 1, k_lds0, v_lds1);
      v_phase(2 * k);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 1, k_lds1, v_lds0);
      barrier_after<kWaitVm0Lgkm0>();
      dma_phase(2 * k + 2, k_lds1, v_lds0);
      v_phase(2 * k + 1);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 2, k_lds0, v_lds1);
      if (k + 1 < n_trips) barrier_after<kWaitVm0Lgkm0>();  // M(2 n_trips) is past every T
    }
  }

  // ---- epilogue -------------------------------------------------------------
  // O = acc / l rounded to bf16. A lane holds 4-dim pieces of one query row,
  // so the wave first writes its 32 x 128 tile to LDS (the K/V slots are idle
  // once the last barrier has passed; wave w takes 8 KB of slot w/2) and reads
  // it back as whole rows: each global store then covers four 256-byte rows
  // instead of 16 bytes of 32 rows. 16-byte chunks are XOR-swizzled by row;
  // the stores carry the non-temporal hint (nothing in the kernel reads O back).
  if (!wave_active) return;
  const float l_tot = halfwave_sum(l_run);
  const float inv = 1.0f / l_tot;
  unsigned char* stage = (wave >> 1) == 0 ? k_lds0 : (wave >> 1) == 1 ? k_lds1 : (wave >> 1) == 2 ? v_lds0 : v_lds1;
  stage += (wave & 1) * (32 * RB);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int chunk = 4 * db + q4;  // dims 32 db + 8 q4 + [0, 8); this lane's 4 of them start at 4 g
      *(u32x2*)(stage + i32 * RB + 16 * (chunk ^ (i32 & 15)) + 8 * g) =
          u32x2{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)};
    }
  unsigned char* obase = (unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq);
  const int pchunk = lane & 15;
#pragma unroll
  for (int t = 0; t < 32 * RB / 1024; ++t) {
    const int r = 4 * t + (lane >> 4);
    const u32x4 val = *(const u32x4*)(stage + r * RB + 16 * pchunk);
    if (qw + r < p.Sq)
      __builtin_nontemporal_store(val, (u32x4*)(obase + (size_t)(qw + r) * p.o_ss + 16 * (pchunk ^ (r & 15))));
  }
  if (g == 0 && qi < p.Sq && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_ref * c + __log2f(l_tot)) * kLn2;
}

}  // namespace pp

int bf16_pp_block_m() { return pp::BM; }

hipError_t launch_attn_bf16_pp(const AttnParams& p, bool causal, hipStream_t stream) {
  // Under the causal mask the waves of a 256-row q-tile need different numbers
  // of key tiles and the phase barriers make every wave wait for the longest.
  // When four (two) query heads share a KV head, a workgroup instead takes 64
  // (128) rows of each of four (two) heads: the waves read the same K/V tiles
  // and need the same number of them (two numbers, one apart, with two heads).
  const int hp = !causal ? 1 : (p.group % 4 == 0) ? 4 : (p.group % 2 == 0) ? 2 : 1;
  AttnParams arg = p;
  arg.n_qtiles = (p.Sq + pp::BM / hp - 1) / (pp::BM / hp);
  const unsigned grid = (unsigned)arg.n_qtiles * (unsigned)p.B * (unsigned)(p.Hq / hp);
  void* args[] = {&arg};
  const void* fn = !causal   ? (const void*)&pp::attn_fwd_bf16_pp_kernel<false, 1>
                   : hp == 4 ? (const void*)&pp::attn_fwd_bf16_pp_kernel<true, 4>
                   : hp == 2 ? (const void*)&pp::attn_fwd_bf16_pp_kernel<true, 2>
                             : (const void*)&pp::attn_fwd_bf16_pp_kernel<true, 1>;
  return hipLaunchKernel(fn, dim3(grid), dim3(pp::WAVES * 64), args, 0, stream);
}

}  // namespace sdpa18
