// Fused scaled dot-product attention forward for gfx950 on fp8-e4m3fn inputs,
// head dim 128: eight waves per workgroup in matrix-core / vector-unit
// ping-pong, Q.K^T on fp8 matrix cores; P.V on bf16 or on fp8 matrix cores.
//
// The method is the FlashAttention forward pass ("Self-attention, CUDA kernels
// and FlashAttention", section 3): K and V stream through on-chip tiles, the
// scores of a tile exist only in registers, a reference maximum and a
// normaliser rescale the partial output as tiles arrive (online softmax), and
// only O and the per-row log-sum-exp are written. The arithmetic is the
// codelab's three steps ("Accelerate attention on GPU with cuDNN and
// TransformerEngine", intro and section 4) with the lower-triangular mask of
// its section 7, the shared KV heads of its section 9 and the E4M3 inputs
// with per-tensor scales of its section 10.
//
// Structure (shared with the bf16 ping-pong kernel): each wave owns 32 query
// rows and runs phases M0 V0 M1 V1 ... over its 64-key tiles; the two waves
// of a SIMD are one phase apart, so one feeds the matrix core while the other
// runs the softmax; a workgroup barrier separates phases.
//   M(m): O^T += V(m-1)^T . P(m-1)^T  (M0 has none)
//         S(m)^T = K(m) . Q^T - m_ref  (4 fp8 MFMAs 32x32x64, unit block scales)
//   V(m): mask, P(m) = exp2(c S(m)), fp32 row sums, reference check
// c = scale * descale_q * descale_k * log2(e); descale_v is applied to O.
//
// Two forms of P.V:
//  * bf16 (P8 = false): 16 bf16 MFMAs 32x32x16. V tiles are loaded into
//    registers, widened e4m3 -> bf16 (exact) and written to LDS transposed
//    (V^T, keys contiguous per dimension), once per workgroup; every P.V
//    operand is then one 16-byte LDS read.
//  * fp8 (P8 = true): 4 fp8 MFMAs 32x32x64 with P rounded to e4m3. V tiles
//    stay e4m3 and go HBM -> LDS by DMA like K; the V^T operand comes from
//    four transposing 8-bit reads (8 keys of one dimension each). P is kept
//    as 2 P (the factor folds into the reference, so it costs nothing) and a
//    score that would make a stored 2 P exceed 256 moves the reference
//    (tested on the lane's maximum score, before the exps), so no value
//    reaches the format's largest value 448. The row sums stay fp32 sums of
//    the unrounded values; the wave adds a tile's in its next M phase, beside
//    the MFMAs. It runs for the q-tiles whose first query sees at least
//    256 keys; workgroups of q-tiles that see fewer keys take the bf16 form.
//
// Memory path:
//  * K tiles (fp8, 64 x 128 B = 8 KB) go HBM -> LDS by buffer_load ... lds;
//    K rows are read in a bit-permuted order (bits 2 and 3 of the row swapped)
//    so that each lane's 8 consecutive score registers hold 8 consecutive keys.
//  * Every LDS layout carries an XOR swizzle of its 16-byte chunks that keeps
//    its operand reads free of bank conflicts.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {
namespace fp8pp {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = 128;
constexpr int WAVES = 8;
constexpr int BM = 32 * WAVES;       // query rows per workgroup
constexpr int BN = 64;               // keys per tile
constexpr int KRB = D;               // bytes per fp8 K row
constexpr int KTILE = BN * KRB;      // 8 KB
constexpr int VTRB = BN * 2;         // bytes per bf16 V^T row (64 keys)
constexpr int VTILE = D * VTRB;      // 16 KB
constexpr int KB = BN / 32;          // 32-key blocks of a score tile
constexpr int KC = BN / 16;          // 16-key chunks (K depth of P.V)
constexpr int DB = D / 32;           // 32-wide output blocks
constexpr int QS = D / 64;           // fp8 MFMA steps of a 32x32 score block
static_assert(KTILE == 1024 * WAVES, "one 1 KB K load per wave per tile");
static_assert(BN * D == 16 * 64 * WAVES, "each lane stages 4 keys x 4 dims of V per tile");

constexpr int LA = 4;                       // MFMAs whose LDS operand reads are in flight ahead
constexpr float kSumLimit = 4096.0f;        // see the bf16 ping-pong kernel
constexpr int kBufferConfig = 0x00020000;   // word 3 of a raw buffer resource (gfx9 family)
constexpr int kE8M0One = 127;               // E8M0 block scale 2^0
constexpr int kWaitLgkm0 = 0xC07F;          // s_waitcnt lgkmcnt(0)
constexpr int kWaitVm0Lgkm0 = 0x0070;       // s_waitcnt vmcnt(0) lgkmcnt(0)

// Chunk swizzle of both layouts: the 16 lanes of one read phase hit 8 even and
// 8 odd rows at one logical chunk; XOR with (row >> 1) & 7 spreads each set
// over all 8 chunk positions.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// fp8 V rows, read through the transposing 8-bit read: lanes 0-31 of one read
// cover 8 consecutive rows x 2 chunks; XOR with 2 ((row >> 1) & 3) puts the 4
// rows of each parity on 4 disjoint chunk pairs.
__device__ __forceinline__ int vswz(int row) { return ((row >> 1) & 3) << 1; }

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int WAIT>
__device__ __forceinline__ void barrier_after() {
  __builtin_amdgcn_s_waitcnt(WAIT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// q-tile of workgroup blockIdx.x (heaviest first under the causal mask).
__device__ __forceinline__ int work_qtile(const AttnParams& p, bool causal) {
  int qt_seq;
  if (p.xcd_remap) {
    qt_seq = (blockIdx.x >> 3) / ((p.B * p.Hkv / 8) * p.group);
  } else {
    qt_seq = blockIdx.x / (p.B * p.Hq);
  }
  return causal ? (p.n_qtiles - 1 - qt_seq) : qt_seq;
}

// One workgroup's work with either form of P.V. Each form has LDS slots of
// its own; the e4m3 form's come first (larger alignment), so its operand
// reads reach them through 16-bit immediate offsets.
template <bool CAUSAL, bool P8>
__device__ __forceinline__ void fp8_tile(const AttnParams& p) {
  constexpr int VSLOT = P8 ? KTILE : VTILE;  // e4m3 V rows, or the widened V^T
  constexpr int AL = P8 ? 4096 : 1024;
  __shared__ __attribute__((aligned(AL))) unsigned char k_lds0[KTILE];
  __shared__ __attribute__((aligned(AL))) unsigned char k_lds1[KTILE];
  __shared__ __attribute__((aligned(AL))) unsigned char v_lds0[VSLOT];
  __shared__ __attribute__((aligned(AL))) unsigned char v_lds1[VSLOT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;
  const int group = wave >> 2;                   // 0: M on even phases, 1: M on odd phases
  const int row_block = 2 * (wave & 3) + group;  // the SIMD's two waves own adjacent blocks

  // ---- work item: (q-tile, batch, query head) ------------------------------
  int qt_seq, b, hq;
  if (p.xcd_remap) {
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
  const int qw = q0 + row_block * 32;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);
  // A tile of BN rows spans BN strides; the buffer of K (V) ends with the last
  // key's row, so rows at or past Sk load as zeros.
  const int k_tile = BN * p.k_ss, v_tile = BN * p.v_ss;
  const int k_limit = (p.Sk - 1) * p.k_ss + KRB, v_limit = (p.Sk - 1) * p.v_ss + KRB;

  const int kv_end = CAUSAL ? min(p.Sk, q0 + BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const bool wave_active = qw < p.Sq;
  const int T = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / BN + 1) : n_tiles);
  const int full_tiles = CAUSAL ? min(p.Sk / BN, (qw + 1 + p.causal_off) / BN) : p.Sk / BN;

  // ---- K DMA: wave w fills rows 8w .. 8w+7 of a K tile (lane l: row 8w + l/8,
  // physical chunk l%8) ------------------------------------------------------
  const int kdma_row = 8 * wave + (lane >> 3);
  const unsigned kdma_off = kdma_row * p.k_ss + 16 * ((lane & 7) ^ swz(kdma_row));
  const int kdma_dst = 1024 * wave;
  auto dma_k = [&](int kt, unsigned char* dst) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + kt * k_tile), (short)0, k_limit - kt * k_tile, kBufferConfig);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + kdma_dst), 16, kdma_off, 0, 0, 0);
  };
  // fp8 P.V: V tiles as K tiles, with the V swizzle.
  const unsigned vdma_off = kdma_row * p.v_ss + 16 * ((lane & 7) ^ vswz(kdma_row));
  auto dma_v = [&](int kt, unsigned char* dst) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + kt * v_tile), (short)0, v_limit - kt * v_tile, kBufferConfig);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + kdma_dst), 16, vdma_off, 0, 0, 0);
  };

  // ---- V staging: lane l of wave w holds keys 4(l/4) .. +3 at dims 16w + 4(l%4) .. +3
  const int vkg = lane >> 2;
  const int vd0 = 16 * wave + 4 * (lane & 3);
  uint32_t vreg[4];
  auto load_v = [&](int kt) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + kt * v_tile), (short)0, v_limit - kt * v_tile, kBufferConfig);
#pragma unroll
    for (int j = 0; j < 4; ++j) vreg[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (4 * vkg + j) * p.v_ss + vd0, 0, 0);
  };
  // e4m3 -> bf16 (exact) and the transposed store: dimension vd0 + e gets the
  // 4 keys' values as one 8-byte unit at key offset 4 vkg of its V^T row.
  auto store_v = [&](unsigned char* dst) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[j], 1.0f, false));
      hi[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[j], 1.0f, true));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t* w = (e < 2) ? lo : hi;
      const u32x2 val = (e & 1) ? u32x2{pack_hi16(w[0], w[1]), pack_hi16(w[2], w[3])}
                                : u32x2{pack_lo16(w[0], w[1]), pack_lo16(w[2], w[3])};
      const int dd = vd0 + e;
      *(u32x2*)(dst + dd * VTRB + 16 * ((vkg >> 1) ^ swz(dd)) + 8 * (vkg & 1)) = val;
    }
  };

  // ---- Q fragment (B operand of S^T): step s, half g holds dims [64s+32g, +32)
  const float c = p.qk_scale_log2;
  i32x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    u32x4 q0v = u32x4{0, 0, 0, 0}, q1v = u32x4{0, 0, 0, 0};
    if (qi < p.Sq) {
      q0v = *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 64 * s + 32 * g);
      q1v = *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 64 * s + 32 * g + 16);
    }
    qf[s] = i32x8{(int)q0v[0], (int)q0v[1], (int)q0v[2], (int)q0v[3],
                  (int)q1v[0], (int)q1v[1], (int)q1v[2], (int)q1v[3]};
  }

  // ---- LDS operand offsets ---------------------------------------------------
  // K (A operand): row 32kb + swap_bits23(i32), logical chunks 4s + 2g and +1.
  const int krow = swap_bits23(i32);
  int k_rd[QS][2];
#pragma unroll
  for (int s = 0; s < QS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) k_rd[s][h] = krow * KRB + 16 * ((4 * s + 2 * g + h) ^ swz(krow));
  // V^T (A operand): row 32db + i32, logical chunk 2kc + g (keys 16kc + 8g .. +7).
  int v_rd[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) v_rd[kc] = i32 * VTRB + 16 * ((2 * kc + g) ^ swz(i32));
  // fp8 V^T (A operand, dims 32db + i32): in each 16-lane group (J = lane % 16,
  // G = bit 4 of the lane) lanes 2r and 2r+1 read bytes [8(J%2), +8) of chunk
  // 2db + G of row 8g + r (+ 16j for read j), and the transposing read hands
  // lane J that chunk's column J over the 8 rows: keys 16j + 8g + 0..7.
  int v8_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int J = lane & 15, G = (lane >> 4) & 1;
    const int row = 8 * g + (J >> 1);
    v8_rd[db] = row * KRB + 16 * ((2 * db + G) ^ vswz(row)) + 8 * (J & 1);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  f32x16 s[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
  u32x4 pf[KC];    // bf16 P^T operand: chunk kc <-> keys 16kc + 8g .. +7
  i32x8 pf8 = i32x8{};  // e4m3 P^T operand: bytes 8j + e <-> key 16j + 8g + e
  // Reference maximum m_ref (dot-product units of the fp8 codes, equal on
  // both halves of a query), and the start of the first Q.K^T MFMA of a tile,
  // replicated over an accumulator block: -m_ref, plus 1/c with e4m3 P, so
  // that exp2 yields 2 P there.
  const float lift = P8 ? 1.0f / c : 0.0f;
  float m_ref = 0.f;
  f32x16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = lift;
  float l_run = 0.f;

  auto pv_part = [&](const unsigned char* vl) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 a = *(const u32x4*)(vl + db * 32 * VTRB + v_rd[kc]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
      }
  };
  // With e4m3 P the tile's unrounded probabilities wait in pk until the
  // wave's next M phase adds them into l_run beside its MFMAs.
  float pk[KB * 16];
  auto add_pk = [&]() {
    float lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KB * 16; i += 2) {
      lt[(i >> 1) & 3] += pk[i];
      lt[(i >> 1) & 3] += pk[i + 1];
    }
    l_run += (lt[0] + lt[1]) + (lt[2] + lt[3]);
  };

  auto pv_part8 = [&](const unsigned char* vl) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x2 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vl + v8_rd[db] + 16 * KRB * j));
      const i32x8 a = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf8, acc[db], 0, 0, 0, kE8M0One, 0, kE8M0One);
    }
  };
  auto qk_part = [&](const unsigned char* kl) {
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 a0 = *(const u32x4*)(kl + kb * 32 * KRB + k_rd[st][0]);
        const u32x4 a1 = *(const u32x4*)(kl + kb * 32 * KRB + k_rd[st][1]);
        const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                              (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[st], st == 0 ? negm : s[kb], 0, 0, 0,
                                                                kE8M0One, 0, kE8M0One);
      }
  };
  // M phase m (1 <= m <= T), one straight-line shape for every m (for m = T
  // the scores are never read). LDS operand reads run LA MFMAs ahead.
  auto m_phase = [&](int m, const unsigned char* kl, const unsigned char* vl) {
    if (m > T) return;
    if constexpr (P8) {
      add_pk();  // the row sum of tile m-1, beside the MFMAs
      pv_part8(vl);
      qk_part(kl);
      constexpr int NPV = DB, NMF = DB + KB * QS, LA8 = 2;  // 4 reads per P.V MFMA, 2 per Q.K^T MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * LA8, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        const int j = i + LA8;
        if (j < NPV)
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        else if (j < NMF)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    } else {
      pv_part(vl);
      qk_part(kl);
      constexpr int NPV = KC * DB, NMF = KC * DB + KB * QS;
      static_assert(LA <= NPV, "the prologue reads belong to P.V MFMAs");
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        const int j = i + LA;
        if (j < NPV)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (j < NMF)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  // M(0): no probabilities yet, so only S(0) = K(0).Q^T.
  auto m_first = [&](const unsigned char* kl) {
    if (T == 0) return;
    qk_part(kl);
    constexpr int NQK = KB * QS;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 2 < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // p = exp2(c S) for the whole tile: the P^T operand (bf16) and this lane's
  // partial row sum (fp32, unrounded), or, with e4m3 P, the operand and pk.
  // Registers 8j .. 8j+7 of block kb hold keys 32kb + 16j + 8g .. +7, i.e.
  // P^T chunk kc = 2kb + j.
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
          if constexpr (P8) {
            // keys 16(2kb + j) + 8g + 2e2, +1: bytes 8(2kb + j) + 2e2, +1 of the operand
            const int w = 2 * (2 * kb + j) + (e2 >> 1);
            if (e2 & 1)
              pf8[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf8[w], true);
            else
              pf8[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf8[w], false);
            pk[16 * kb + r] = p0;
            pk[16 * kb + r + 1] = p1;
          } else {
            pf[2 * kb + j][e2] = pack_bf16x2(p0, p1);
            lt[e2] += p0;
            lt[e2] += p1;
          }
        }
    return (lt[0] + lt[1]) + (lt[2] + lt[3]);
  };

  // V phase v: mask, probabilities and row sums of S(v); the reference moves
  // on tile 0 and when a tile's partial sums show probabilities beyond 2^12.
  auto v_phase = [&](int v) {
    if (v < 0 || v >= T) return;
    if (v >= full_tiles) {
      // Register r of block kb on half g holds key v*BN + 32kb + 16(r/8) + 8g + r%8.
      const int limit = (CAUSAL ? min(p.Sk - 1, qi + p.causal_off) : p.Sk - 1) - v * BN - 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) <= limit) ? s[kb][r] : -INFINITY;
    }
    if constexpr (P8) {
      // The reference moves on tile 0 and when a stored 2P would exceed 256,
      // i.e. when c S > 8 for a score of the lane (tested before the exps).
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      if (v == 0 || __builtin_amdgcn_ballot_w64(!(mx * c <= 8.0f)) != 0) {
        // Tile 0 holds key 0, visible to every row, so its maximum is finite.
        mx = halfwave_max(mx) - lift;  // relative to m_ref
        const float delta = (v == 0) ? mx : fmaxf(mx, 0.f);
        if (v > 0) {
          const float alpha = exp2_fast(-delta * c);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        }
        m_ref += delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = lift - m_ref;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
      }
      exp_tile();
      return;
    }
    float l_tile = 0.f;
    bool rebase = (v == 0);
    if (!rebase) {
      l_tile = exp_tile();
      rebase = __builtin_amdgcn_ballot_w64(!(l_tile <= kSumLimit)) != 0;
    }
    if (rebase) {
      // Tile 0 holds key 0, visible to every row, so its maximum is finite.
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halfwave_max(mx) - lift;  // relative to m_ref
      const float delta = (v == 0) ? mx : fmaxf(mx, 0.f);
      if (v > 0) {
        const float alpha = exp2_fast(-delta * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
      m_ref += delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = lift - m_ref;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
      l_tile = exp_tile();
    }
    l_run += l_tile;
  };

  // Loads issued at the start of global phase 2n: K(n+1) and V(n). With bf16
  // P.V, V(n) goes to registers and is widened and stored at the end of phase
  // 2n+1; with e4m3 P.V it goes straight to its slot by DMA.
  auto dma_phase = [&](int n, unsigned char* k_dst, unsigned char* v_dst) {
    if (n + 1 < n_tiles) dma_k(n + 1, k_dst);
    if (n < n_tiles) {
      if constexpr (P8)
        dma_v(n, v_dst);
      else
        load_v(n);
    }
  };
  auto v_store_phase = [&](int n, unsigned char* v_dst) {
    if constexpr (!P8)
      if (n < n_tiles) store_v(v_dst);
  };

  // ---- prologue: K(0) into slot 0, published before phase 0 ------------------
  if (n_tiles > 0) dma_k(0, k_lds0);
  barrier_after<kWaitVm0Lgkm0>();

  // ---- global phases (as the bf16 ping-pong kernel) -------------------------
  //   phase 4k   : loads K(2k+1)->k1, V(2k)->v0     | A: M(2k)   [k0, v1] | B: V(2k-1)
  //   phase 4k+1 : (bf16 P.V: store V(2k) at the end) | A: V(2k)          | B: M(2k)   [k0, v1]
  //   phase 4k+2 : loads K(2k+2)->k0, V(2k+1)->v1   | A: M(2k+1) [k1, v0] | B: V(2k)
  //   phase 4k+3 : (bf16 P.V: store V(2k+1))        | A: V(2k+1)          | B: M(2k+1) [k1, v0]
  // M(0) has no P.V and stands before each group's loop, which is rotated to
  // start one phase later; both groups execute n_trips * 4 + 2 barriers after
  // the prologue's (group B skips its last, which would follow M(2 n_trips), a
  // phase past every wave's last tile).
  const int n_trips = (n_tiles + 2) / 2;
  if (group == 0) {
    dma_phase(0, k_lds1, v_lds0);
    m_first(k_lds0);
    barrier_after<kWaitLgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      v_phase(2 * k);
      v_store_phase(2 * k, v_lds0);
      barrier_after<kWaitVm0Lgkm0>();
      dma_phase(2 * k + 1, k_lds0, v_lds1);
      m_phase(2 * k + 1, k_lds1, v_lds0);
      barrier_after<kWaitLgkm0>();
      v_phase(2 * k + 1);
      v_store_phase(2 * k + 1, v_lds1);
      barrier_after<kWaitVm0Lgkm0>();
      dma_phase(2 * k + 2, k_lds1, v_lds0);
      m_phase(2 * k + 2, k_lds0, v_lds1);
      barrier_after<kWaitLgkm0>();
    }
  } else {
    dma_phase(0, k_lds1, v_lds0);
    barrier_after<kWaitLgkm0>();
    m_first(k_lds0);
    v_store_phase(0, v_lds0);
    barrier_after<kWaitVm0Lgkm0>();
    for (int k = 0; k < n_trips; ++k) {
      dma_phase(2 * k + 1, k_lds0, v_lds1);
      v_phase(2 * k);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 1, k_lds1, v_lds0);
      v_store_phase(2 * k + 1, v_lds1);
      barrier_after<kWaitVm0Lgkm0>();
      dma_phase(2 * k + 2, k_lds1, v_lds0);
      v_phase(2 * k + 1);
      barrier_after<kWaitLgkm0>();
      m_phase(2 * k + 2, k_lds0, v_lds1);
      v_store_phase(2 * k + 2, v_lds0);
      if (k + 1 < n_trips) barrier_after<kWaitVm0Lgkm0>();  // M(2 n_trips) is past every T
    }
  }

  // ---- epilogue -------------------------------------------------------------
  // O = descale_v * acc / l rounded to bf16. A lane holds 4-dim pieces of one
  // query row, so each half of the wave's 32 rows is written to 4 KB of an
  // idle V^T slot (no load or operand read is pending after the last barrier)
  // and read back as whole rows: each global store then covers four 256-byte
  // rows (with e4m3 P.V, whose V slots are 8 KB, wave w takes 4 KB of slot w/2
  // of the K and V slots). 16-byte chunks are XOR-swizzled by row; the stores
  // carry the non-temporal hint (nothing in the kernel reads O back).
  if (!wave_active) return;
  const float l_tot = halfwave_sum(l_run);
  const float inv = p.o_scale / l_tot;
  constexpr int ORB = 2 * D;  // bytes per bf16 output row
  unsigned char* stage;
  if constexpr (P8)
    stage = ((wave >> 1) == 0 ? k_lds0 : (wave >> 1) == 1 ? k_lds1 : (wave >> 1) == 2 ? v_lds0 : v_lds1) +
            (wave & 1) * (16 * ORB);
  else
    stage = (wave < 4 ? v_lds0 : v_lds1) + (wave & 3) * (16 * ORB);
  unsigned char* obase = (unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq);
  const int pchunk = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((i32 >> 4) == half) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int chunk = 4 * db + q4;  // dims 32 db + 8 q4 + [0, 8); this lane's 4 of them start at 4 g
          *(u32x2*)(stage + (i32 & 15) * ORB + 16 * (chunk ^ (i32 & 15)) + 8 * g) =
              u32x2{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                    pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)};
        }
    }
#pragma unroll
    for (int t = 0; t < 16 * ORB / 1024; ++t) {
      const int r = 4 * t + (lane >> 4);
      const u32x4 val = *(const u32x4*)(stage + r * ORB + 16 * pchunk);
      const int row = qw + 16 * half + r;
      if (row < p.Sq)
        __builtin_nontemporal_store(val, (u32x4*)(obase + (size_t)row * p.o_ss + 16 * (pchunk ^ r)));
    }
  }
  // l_tot sums 2^(c lift) P: the lift comes back out of the log-sum-exp.
  if (g == 0 && qi < p.Sq && p.lse != nullptr)
    p.lse[qo_row0 + qi] = (m_ref * c + __log2f(l_tot) - c * lift) * kLn2;
}

// q-tiles from p.p8_qtile on take P.V with e4m3 P, the earlier ones with bf16 P.
template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_pp_kernel(const AttnParams p) {
  if (work_qtile(p, CAUSAL) >= p.p8_qtile)
    fp8_tile<CAUSAL, true>(p);
  else
    fp8_tile<CAUSAL, false>(p);
}

}  // namespace fp8pp

int fp8_pp_block_m() { return fp8pp::BM; }

hipError_t launch_attn_fp8_pp(const AttnParams& p, bool causal, hipStream_t stream) {
  // P.V on fp8 matrix cores for the q-tiles whose first query sees at least
  // BM keys (causal: q-tile t's first query sees t BM + 1 + causal_off keys),
  // on bf16 matrix cores for the others, where softmax is concentrated on few
  // keys and P's three mantissa bits would show.
  constexpr int BM = fp8pp::BM;
  AttnParams arg = p;
  if (!causal) {
    arg.p8_qtile = p.Sk >= BM ? 0 : p.n_qtiles;
  } else {
    const int need = BM - 1 - p.causal_off;  // t BM >= need
    arg.p8_qtile = need <= 0 ? 0 : (need + BM - 1) / BM;
  }
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
  void* args[] = {&arg};
  const void* fn = causal ? (const void*)&fp8pp::attn_fwd_fp8_pp_kernel<true>
                          : (const void*)&fp8pp::attn_fwd_fp8_pp_kernel<false>;
  return hipLaunchKernel(fn, dim3(grid), dim3(fp8pp::WAVES * 64), args, 0, stream);
}

}  // namespace sdpa18
