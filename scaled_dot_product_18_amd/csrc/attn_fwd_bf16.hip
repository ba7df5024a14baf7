// Fused scaled dot-product attention forward for gfx950, bf16 inputs and output.
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
// Layout of the work on CDNA4:
//  * this kernel serves head dimensions 32 and 64 (the eight-wave ping-pong
//    kernel in attn_fwd_bf16_pp.hip serves 128, and the one in
//    attn_fwd_ppk.hip d = 64 grids of up to 768 workgroups over at
//    least 1024 keys), in three forms picked by the grid: four waves with
//    four resident per SIMD (large grids), four waves with the operand reads
//    run ahead (up to 768 workgroups), and eight waves splitting the keys in
//    two halves (up to 256 workgroups);
//  * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//    wave w owns rows [32w, 32w+32) and keeps their Q fragment in VGPRs;
//  * scores are computed transposed, S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16,
//    so each lane owns one query column: row max / row sum are in-lane plus one
//    v_permlane32_swap, and per-row factors are lane scalars;
//  * the accumulator registers of S^T, rounded to bf16, are directly the B
//    operand of O^T += V^T . P^T; the V^T operand comes from a row-major V tile
//    through ds_read_b64_tr_b16 (4 consecutive keys at one dimension per read);
//  * K and V tiles go HBM -> LDS with buffer_load_dwordx4 ... lds (no staging
//    registers, no per-lane address arithmetic: the tile offset lives in the
//    buffer descriptor), double buffered in two separate LDS objects so the
//    compiler never makes a read of one stage wait for the loads into the
//    other, one barrier per tile; rows past the end of the sequence fall
//    outside the buffer's range and load as zeros; both tiles carry an XOR
//    swizzle of their 16-byte chunks that keeps the MFMA operand reads free of
//    bank conflicts;
//  * the running maximum is only moved (and O, l rescaled) when a tile's
//    maximum exceeds it by more than 2^8 in probability units; otherwise the
//    stale maximum is kept. Softmax is invariant to the reference point, so
//    this is exact, and it removes the per-tile rescale of the accumulator;
//  * 64-key tiles keep a workgroup's double-buffered K and V at 32 KB of LDS,
//    so VGPRs, not LDS, bound the resident workgroups per CU;
//  * row sums add the fp32 probabilities in four independent partial sums;
//  * causal workgroups stop at the diagonal, run heaviest first, and query
//    heads that share a KV head are placed on the same XCD (same L2).
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct Bf16Cfg {
  static constexpr int BM = 128;             // query rows per workgroup
  static constexpr int BN = 64;              // keys per tile (32 KB of LDS per workgroup at d=64)
  static constexpr int RB = D * 2;           // bytes per K/V row
  static constexpr int CH = RB / 16;         // 16-byte chunks per row
  static constexpr int TILE = BN * RB;       // bytes of a K (or V) tile
  static constexpr int STAGE = 2 * TILE;     // K tile then V tile
  static constexpr int DMA = TILE / 1024 / 4;  // 1 KB wave-wide DMA instructions per tensor per wave
  static constexpr int ROWS_PER_DMA = 1024 / RB;
  static constexpr int KB = BN / 32;         // 32-key blocks of a score tile
  static constexpr int KC = BN / 16;         // 16-key chunks (K depth of P.V)
  static constexpr int DB = D / 32;          // 32-wide output blocks
  static constexpr int QS = D / 16;          // MFMAs per 32x32 score block
  static_assert(DMA * 4 * 1024 == TILE, "4 waves x DMA instructions cover a tile");
};

// Chunk swizzle of K rows: lanes 0..15 of an operand read hit 16 different rows
// at one logical chunk; XOR with a row-dependent value spreads them over all banks.
// At d = 32 a row is 64 bytes (4 chunks): rows 4 apart share banks, so the
// chunk is XORed with bits 2-3 of the row.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  return D == 128 ? (row & 15) : D == 64 ? ((row & 7) ^ ((row >> 3) & 1)) : ((row >> 2) & 3);
}
// Chunk swizzle of V rows: a 16-lane transposing read touches 4 consecutive rows
// at 32 consecutive bytes; the XOR values {0,6,10,12} (d=128) / {0,2,4,6} (d=64)
// place the 4 rows on disjoint banks for both 32- and 64-bank LDS. At d = 32
// four consecutive 64-byte rows already fall on disjoint banks.
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  return D == 128 ? ((0xCA60 >> (4 * (row & 3))) & 15) : D == 64 ? ((0x6420 >> (4 * (row & 3))) & 15) : 0;
}

constexpr float kRescaleThreshold = 8.0f;  // log2 units: keep the stale max unless exceeded by 2^8

constexpr int kBufferConfig = 0x00020000;  // word 3 of a raw buffer resource: 32-bit data format (gfx9 family)

// This wave's NLOAD wave-wide loads of one K or V tile, HBM -> LDS (lane l of load
// t fills the 16 bytes at dst + 1024 t + 16 l). The tile is read through a raw
// buffer that starts at its first row and ends at the end of the sequence, so
// rows at or past Sk fall outside the buffer and load as zeros. Called from
// the kernel body, not from a lambda: the host pass rejects a device function
// called from a lambda in a kernel template and then drops the launch stub.
template <int NLOAD>
__device__ __forceinline__ void dma_tile(const unsigned char* base, int tile_bytes, int kt, int limit,
                                         const unsigned* off, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + kt * tile_bytes), (short)0, limit - kt * tile_bytes, kBufferConfig);
#pragma unroll
  for (int t = 0; t < NLOAD; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * t), 16, off[t], 0, 0, 0);
}

// SPLIT = 2: eight waves, the workgroup's keys in two halves. Waves 0-3 take
// the first half of the key tiles and waves 4-7 the second, each with its
// own K/V stages, so every SIMD runs two independent chains of tiles; the two
// partial softmax states of a query row (reference maximum, normaliser,
// unnormalised output) are merged through LDS at the end. For grids of at
// most one workgroup per CU, where one wave per SIMD would leave the chain
// of dependent steps exposed.
template <int D, bool CAUSAL, bool READ_AHEAD, int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * SPLIT, 256 * SPLIT), amdgpu_waves_per_eu(2)))
void attn_fwd_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D>;
  static_assert(SPLIT == 1 || (SPLIT == 2 && READ_AHEAD), "the key split runs with read-ahead");
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[SPLIT * C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[SPLIT * C::STAGE];

  const int tid = threadIdx.x;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches and LDS bases
  const int half = wave_id >> 2;                                 // key half (0 unless SPLIT = 2)
  const int wave = wave_id & 3;                                  // 32-row block
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  // ---- work item: (q-tile, batch, query head) ------------------------------
  int qt_seq, b, hq;
  if (p.xcd_remap) {
    // Workgroup i runs on XCD i % 8. Give each XCD whole KV heads (all query
    // heads of a group), q-tiles outermost so every XCD starts on the heaviest.
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

  const int q0 = qt * C::BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + i32;

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);

  const int kv_end = CAUSAL ? min(p.Sk, q0 + C::BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + C::BN - 1) / C::BN;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / C::BN + 1) : n_tiles);
  // This half's key tiles [t_lo, t_hi); n_steps tiles per half (the first half takes the odd one).
  const int n_steps = SPLIT == 2 ? (n_tiles + 1) / 2 : n_tiles;
  const int t_lo = half * n_steps;
  const int t_hi = half == 0 ? n_steps : n_tiles;
  unsigned char* const st0 = smem0 + half * C::STAGE;
  unsigned char* const st1 = smem1 + half * C::STAGE;

  // ---- DMA assignment: wave w writes 1 KB blocks DMA*w .. DMA*w+DMA-1 of each tile
  // 16-byte slot s = 64*(DMA*w+t) + lane holds row s / CH, physical chunk s % CH.
  unsigned kdma_off[C::DMA], vdma_off[C::DMA];
  const int dma_pchunk = lane % C::CH;
#pragma unroll
  for (int t = 0; t < C::DMA; ++t) {
    const int row = (64 * (C::DMA * wave + t) + lane) / C::CH;
    kdma_off[t] = row * p.k_ss + 16 * (dma_pchunk ^ k_swizzle<D>(row));
    vdma_off[t] = row * p.v_ss + 16 * (dma_pchunk ^ v_swizzle<D>(row));
  }

  // ---- Q fragment (B operand of S^T): step s, half g holds dims [16s+8g, +8)
  u32x4 qf[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s)
    qf[s] = (qi < p.Sq) ? *(const u32x4*)(qbase + (size_t)qi * p.q_ss + 32 * s + 16 * g) : u32x4{0, 0, 0, 0};

  // ---- per-lane LDS operand offsets ------------------------------------------
  // K (A operand of S^T): row 32kb + i32, logical chunk 2s + g.
  int k_rd[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) k_rd[s] = i32 * C::RB + 16 * ((2 * s + g) ^ k_swizzle<D>(i32));
  // V (A operand of O^T through the transposing read): in each 16-lane group,
  // lane J reads 4 dims [dbase + 4(J%4), +4) of key row (row_base + J/4).
  const int J = lane & 15;
  int v_rd[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int row = 4 * g + (J >> 2);
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
    v_rd[db] = row * C::RB + 16 * ((d >> 3) ^ v_swizzle<D>(row)) + 2 * (d & 7);
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  // Reference maximum, log2 units of the scaled score. It starts at the most
  // negative finite value, not -inf: under the key split the second half's
  // first tiles can hide every key from a row, and exp2(c S - m) of those
  // -inf scores must still come out 0 (with m = -inf it would be exp2(NaN)).
  // The first tile with a visible key rescales by exp2(-FLT_MAX - m) = 0.
  float m_run = -__FLT_MAX__;
  float l_run = 0.f;        // this lane's share of the normaliser
  const float c = p.qk_scale_log2;

  auto compute_tile = [&](int kt, const unsigned char* stage) {
    const int kv0 = kt * C::BN;
    const unsigned char* kl = stage;
    const unsigned char* vl = stage + C::TILE;

    // S^T = K . Q^T. With READ_AHEAD every K operand is read first and the
    // MFMAs of the KB independent blocks alternate; the V^T operands of the
    // tile's P.V are read right behind them, so their latency hides under the
    // softmax (32 more VGPRs: three resident waves per SIMD instead of four).
    f32x16 s[C::KB];
    bf16x8 va[C::DB][C::KC];
    auto v_operand = [&](int db, int kc) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc) * C::RB + v_rd[db]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + (16 * kc + 8) * C::RB + v_rd[db]));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    if constexpr (READ_AHEAD) {
      u32x4 ka[C::KB][C::QS];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int st = 0; st < C::QS; ++st) ka[kb][st] = *(const u32x4*)(kl + kb * 32 * C::RB + k_rd[st]);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < C::QS; ++st)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[kb][st]),
                                                          __builtin_bit_cast(bf16x8, qf[st]), s[kb], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) va[db][kc] = v_operand(db, kc);
      __builtin_amdgcn_sched_group_barrier(0x100, C::KB * C::QS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, C::KB * C::QS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::DB * C::KC, 0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < C::QS; ++st) {
          const u32x4 a = *(const u32x4*)(kl + kb * 32 * C::RB + k_rd[st]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf[st]), s[kb], 0, 0, 0);
        }
      }
    }

    // register r of block kb on half g holds key kv0 + 32kb + 8(r/4) + 4g + r%4
    if ((CAUSAL && kv0 + C::BN - 1 > qw + p.causal_off) || kv0 + C::BN > p.Sk) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool ok = (key < p.Sk) && (!CAUSAL || key <= qi + p.causal_off);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float m_tile = halfwave_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
    }

    // P^T operand: chunk kc = 2kb + j, element e <-> key 16kc + 8(e/4) + 4g + e%4.
    // The row sum adds the unrounded fp32 probabilities (v_dot2 on the packed
    // bf16 values would stall the matrix core).
    u32x4 pf[C::KC];
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r = 8 * j + 2 * e2;
          const float p0 = exp2_fast(__builtin_fmaf(s[kb][r], c, -m_run));
          const float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], c, -m_run));
          pf[2 * kb + j][e2] = pack_bf16x2(p0, p1);
          lsum[e2] += p0;
          lsum[e2] += p1;
        }
    l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);

    // O^T += V^T . P^T
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(READ_AHEAD ? va[db][kc] : v_operand(db, kc),
                                                          __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
  };

  // ---- main loop: DMA of tile kt+1 overlaps compute of tile kt --------------
  // A tile of BN rows spans BN strides; the buffer of K (V) ends with the last
  // key's row, so rows at or past Sk load as zeros.
  const int k_tile = C::BN * p.k_ss, v_tile = C::BN * p.v_ss;
  const int k_limit = (p.Sk - 1) * p.k_ss + C::RB, v_limit = (p.Sk - 1) * p.v_ss + C::RB;
  if (t_lo < t_hi) {
    dma_tile<C::DMA>(kbase, k_tile, t_lo, k_limit, kdma_off, st0 + 1024 * C::DMA * wave);
    dma_tile<C::DMA>(vbase, v_tile, t_lo, v_limit, vdma_off, st0 + C::TILE + 1024 * C::DMA * wave);
  }
  __syncthreads();
  for (int i = 0; i < n_steps; i += 2) {
    const int kt = t_lo + i;
    if (kt + 1 < t_hi) {
      dma_tile<C::DMA>(kbase, k_tile, kt + 1, k_limit, kdma_off, st1 + 1024 * C::DMA * wave);
      dma_tile<C::DMA>(vbase, v_tile, kt + 1, v_limit, vdma_off, st1 + C::TILE + 1024 * C::DMA * wave);
    }
    if (kt < t_hi && kt < wave_tiles) compute_tile(kt, st0);
    __syncthreads();
    if (i + 1 >= n_steps) break;
    if (kt + 2 < t_hi) {
      dma_tile<C::DMA>(kbase, k_tile, kt + 2, k_limit, kdma_off, st0 + 1024 * C::DMA * wave);
      dma_tile<C::DMA>(vbase, v_tile, kt + 2, v_limit, vdma_off, st0 + C::TILE + 1024 * C::DMA * wave);
    }
    if (kt + 1 < t_hi && kt + 1 < wave_tiles) compute_tile(kt + 1, st1);
    __syncthreads();
  }

  // ---- merge of the two key halves (SPLIT = 2) -------------------------------
  // The second half's waves leave acc, m_run and l_run in LDS (register-major,
  // 64 lanes contiguous: acc in smem0, m and l at the end of smem1); the first
  // half's wave of the same rows rescales both to the larger reference and
  // adds. A row always has key 0, so the first half's reference is a real
  // score maximum; an empty second half (m = -FLT_MAX) gets the factor 0.
  if constexpr (SPLIT == 2) {
    float* const m_acc = (float*)smem0 + wave * (C::DB * 16 * 64);
    float* const m_ml = (float*)(smem1 + 2 * C::STAGE) - 8 * 64 + wave * (2 * 64);
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) m_acc[(db * 16 + r) * 64 + lane] = acc[db][r];
      m_ml[lane] = m_run;
      m_ml[64 + lane] = l_run;
    }
    __syncthreads();
    if (half == 1 || !wave_active) return;
    const float m_b = m_ml[lane], l_b = m_ml[64 + lane];
    const float m_new = fmaxf(m_run, m_b);
    const float fa = exp2_fast(m_run - m_new), fb = exp2_fast(m_b - m_new);
    m_run = m_new;
    l_run = l_run * fa + l_b * fb;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * fa + m_acc[(db * 16 + r) * 64 + lane] * fb;
  }

  // ---- epilogue -------------------------------------------------------------
  // O = acc / l rounded to bf16. A lane holds 4-dim pieces of one query row,
  // so the wave writes its 32-row tile to LDS (stage buffer 0 is idle after
  // the last barrier, buffer 1 after a merge; wave w takes rows [32w, 32w+32)
  // of it) and reads it back
  // as whole rows, so that each global store covers 1 KB of contiguous rows.
  // 16-byte chunks are XOR-swizzled by row. The stores carry the non-temporal
  // hint: nothing in the kernel reads O back.
  if (!wave_active) return;
  const float l_tot = halfwave_sum(l_run);
  const float inv = 1.0f / l_tot;
  unsigned char* stage = (SPLIT == 2 ? smem1 : smem0) + wave * (32 * C::RB);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int chunk = 4 * db + q4;  // dims 32 db + 8 q4 + [0, 8); this lane's 4 of them start at 4 g
      *(u32x2*)(stage + i32 * C::RB + 16 * (chunk ^ (i32 & (C::CH - 1))) + 8 * g) =
          u32x2{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)};
    }
  unsigned char* obase = (unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq);
  const int pchunk = lane % C::CH;
#pragma unroll
  for (int t = 0; t < 32 * C::RB / 1024; ++t) {
    const int r = C::ROWS_PER_DMA * t + lane / C::CH;
    const u32x4 val = *(const u32x4*)(stage + r * C::RB + 16 * pchunk);
    if (qw + r < p.Sq)
      __builtin_nontemporal_store(val, (u32x4*)(obase + (size_t)(qw + r) * p.o_ss + 16 * (pchunk ^ (r & (C::CH - 1)))));
  }
  if (g == 0 && qi < p.Sq && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// Grids that fit in one round at three workgroups per CU (768) are bound by
// each wave's chain of dependent steps: there the operand reads run ahead.
// Larger grids keep four resident waves per SIMD.
constexpr unsigned kReadAheadMaxGrid = 768;

// Grids of at most one workgroup per CU split each workgroup's keys over
// eight waves, when there are enough key tiles (six) to pay for the merge.
constexpr unsigned kSplitMaxGrid = 256;
constexpr int kSplitMinKeys = 384;

// d = 64 grids of up to 768 workgroups over at least 1024 keys run the
// ping-pong kernel (16 or more key tiles per row; on shorter rows, and on
// larger grids, where four waves per SIMD overlap without barriers, it is
// no faster).
constexpr unsigned kPingPongMaxGrid = 768;
constexpr int kPingPongMinKeys = 1024;

// attn_fwd_ppk.hip: bf16, d = 64 or 128, eight waves in ping-pong over the
// two halves of each workgroup's keys (n_qtiles counted in 128-row tiles).
hipError_t launch_attn_bf16_ppk(const AttnParams& p, int d, bool causal, hipStream_t stream);

template <int D, bool CAUSAL>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
  if (D == 64 && grid <= kPingPongMaxGrid && p.Sk >= kPingPongMinKeys)
    return launch_attn_bf16_ppk(p, 64, CAUSAL, stream);
  AttnParams arg = p;
  void* args[] = {&arg};
  if (grid <= kSplitMaxGrid && p.Sk >= kSplitMinKeys)
    return hipLaunchKernel((const void*)&attn_fwd_bf16_kernel<D, CAUSAL, true, 2>, dim3(grid), dim3(512), args, 0,
                           stream);
  const void* fn = grid <= kReadAheadMaxGrid ? (const void*)&attn_fwd_bf16_kernel<D, CAUSAL, true, 1>
                                             : (const void*)&attn_fwd_bf16_kernel<D, CAUSAL, false, 1>;
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream);
}

int bf16_block_m(int d) { return d == 128 ? bf16_pp_block_m() : Bf16Cfg<64>::BM; }

// attn_fwd_ppk.hip: whether a d = 128 shape is small enough for the key-half
// kernel (twice the workgroups of the 256-row kernel, half the key tiles each).
bool ppk_takes_d128(const AttnParams& p, bool causal);

hipError_t launch_attn_bf16(const AttnParams& p, int d, bool causal, hipStream_t stream) {
  // d = 128: the eight-wave ping-pong kernels (attn_fwd_bf16_pp.hip, attn_fwd_ppk.hip); d = 32 and 64 here.
  if (d == 128) {
    if (!ppk_takes_d128(p, causal)) return launch_attn_bf16_pp(p, causal, stream);
    AttnParams q = p;
    q.n_qtiles = (p.Sq + 127) / 128;
    return launch_attn_bf16_ppk(q, 128, causal, stream);
  }
  if (d == 32) return causal ? launch_one<32, true>(p, stream) : launch_one<32, false>(p, stream);
  return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace sdpa18
