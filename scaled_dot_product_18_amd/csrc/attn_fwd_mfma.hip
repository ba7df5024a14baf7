// Fused scaled dot-product attention forward for gfx950 on fp8-e4m3fn inputs
// at head dimensions 32 and 64 (fp8 MFMA for Q.K^T, bf16 MFMA for P.V with V
// widened exactly); head dimension 128 runs the ping-pong kernel of
// attn_fwd_fp8_pp.hip, and d = 64 over at least 1024 keys the one of
// attn_fwd_ppk.hip. The fp8 MFMA has a K depth of 64: at d = 32 the upper
// half-wave supplies zero operands, so each score is still one instruction.
// The template also has a bf16-input form (FP8 = false), which nothing
// launches.
//
// The method is the FlashAttention forward pass ("Self-attention, CUDA kernels
// and FlashAttention", section 3): Q, K, V are cut into tiles that fit on chip,
// scores exist only per tile, a running maximum and normaliser per query row
// rescale the partial output as each key tile arrives (online softmax), and
// only the output and the per-row log-sum-exp reach memory. The mathematics is
// the codelab's ("Accelerate attention on GPU with cuDNN and TransformerEngine",
// intro and section 4: score, scale + softmax, weighted sum), with the
// lower-triangular mask of its section 7 and the shared KV heads of section 9.
//
// Work decomposition: one workgroup = 4 waves = 128 query rows of one
// (batch, query head); wave w owns 32 rows. The scores are computed transposed,
// S^T = K . Q^T, on 32x32 MFMAs, so every lane owns one query column: the
// row max and row sum of the softmax are in-lane reductions plus one exchange
// with the other half-wave, and the per-row rescale factor is a lane scalar.
// The output is likewise accumulated transposed, O^T += V^T . P^T, and the
// score accumulator registers (converted to bf16) are directly the P^T operand:
// K rows are read in a bit-permuted order so that each lane's 8 consecutive
// accumulator registers hold 8 consecutive keys.
//
// Memory path: the Q fragment (B operand) is loaded once into VGPRs; K and V
// tiles are loaded from HBM into registers one tile ahead and written to a
// double-buffered LDS ring (K row-major with an XOR swizzle, V transposed to
// V^T with an XOR swizzle), one barrier per tile. Causal workgroups stop at the
// diagonal and are launched heaviest first.
//
// SPLIT = 2: eight waves, the workgroup's key tiles in two halves. Waves 0-3
// take the first half and waves 4-7 the second, each half with its own ring
// and its own 256 threads staging it, so every SIMD runs two independent
// chains of tiles; the two partial softmax states of a query row are merged
// through LDS at the end. For grids of at most one workgroup per CU, where
// one wave per SIMD would leave the chain of dependent steps exposed.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {

template <int D, bool FP8>
struct MfmaCfg {
  static constexpr int BM = 128;                    // query rows per workgroup
  static constexpr int BN = D == 32 ? 128 : 8192 / D;  // keys per tile: 64 (d=128), 128 (d=64, d=32)
  static constexpr int ES = FP8 ? 1 : 2;            // bytes per Q/K/V input element
  static constexpr int KRB = D * ES;                // bytes per K row in LDS
  static constexpr int KCH = KRB / 16;              // 16-byte chunks per K row
  static constexpr int KROWS_PER_PASS = 256 / KCH;  // K rows loaded per pass of 256 threads
  static constexpr int KPASS = BN / KROWS_PER_PASS; // 16-byte K loads per thread per tile
  static constexpr int KBYTES = BN * KRB;
  static constexpr int VTRB = BN * 2;               // bytes per V^T row (bf16 keys)
  static constexpr int VBYTES = D * VTRB;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int KC = BN / 16;                // 16-key chunks (K dim of P.V)
  static constexpr int DB = D / 32;                 // 32-wide output blocks
  static constexpr int QK_STEPS = FP8 ? (D + 63) / 64 : D / 16;  // MFMAs per 32x32 score block
  static constexpr int QREGS = FP8 ? 2 * QK_STEPS : QK_STEPS;  // 16-byte Q pieces per lane
  static constexpr int VU = BN / 4;                 // 4-key units per V^T row
  static constexpr int VTHREADS = VU * D / 8;       // threads that stage V (4 keys x 8 dims each)
  static_assert(KPASS >= 1 && KROWS_PER_PASS * KPASS == BN, "K staging must tile the key block");
  static_assert(VTHREADS <= 256 && VTHREADS * 32 == BN * D, "V staging: 4 keys x 8 dims per thread tile BN x D");
};

// E8M0 scale byte 127 = 2^0: the scaled fp8 MFMA with unit scales.
constexpr int kE8M0One = 127;

template <int D, bool CAUSAL, bool FP8, int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * SPLIT, 256 * SPLIT), amdgpu_waves_per_eu(2)))
void attn_fwd_mfma_kernel(const AttnParams p) {
  using C = MfmaCfg<D, FP8>;
  static_assert(SPLIT == 1 || SPLIT == 2, "one or two key halves");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SPLIT * 2 * C::STAGE];

  const int tid = threadIdx.x & 255;  // thread within the key half: the staging assignment below
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave_id >> 2;      // key half (0 unless SPLIT = 2)
  const int wave = wave_id & 3;       // 32-row block
  const int lane = tid & 63;
  const int i32 = lane & 31;  // MFMA row (A operand) / column (B operand, C)
  const int g = lane >> 5;    // half-wave

  // ---- which (q-tile, batch, head); causal tiles heaviest first -----------
  const int BH = p.B * p.Hq;
  const int seq = blockIdx.x / BH;
  const int rem = blockIdx.x - seq * BH;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - seq) : seq;
  const int b = rem / p.Hq;
  const int hq = rem - b * p.Hq;
  const int hk = hq / p.group;  // shared KV head of this query head

  const int q0 = qt * C::BM;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int qi = qw + i32;        // this lane's query row

  const size_t qo_row0 = ((size_t)b * p.Hq + hq) * (size_t)p.Sq;  // lse row of query 0
  const unsigned char* qbase = head_ptr(p.q, p.q_sb, p.q_sh, b, hq);
  const unsigned char* kbase = head_ptr(p.k, p.k_sb, p.k_sh, b, hk);
  const unsigned char* vbase = head_ptr(p.v, p.v_sb, p.v_sh, b, hk);

  const int kv_end = CAUSAL ? min(p.Sk, q0 + C::BM + p.causal_off) : p.Sk;
  const int n_tiles = (kv_end + C::BN - 1) / C::BN;
  const bool wave_active = qw < p.Sq;
  const int wave_tiles = !wave_active ? 0 : (CAUSAL ? min(n_tiles, (qw + 31 + p.causal_off) / C::BN + 1) : n_tiles);
  // This half's key tiles [t_lo, t_hi), n_steps loop steps for both halves (the first takes the odd tile).
  const int n_steps = SPLIT == 2 ? (n_tiles + 1) / 2 : n_tiles;
  const int t_lo = half * n_steps;
  const int t_hi = half == 0 ? n_steps : n_tiles;
  unsigned char* const ring = smem + half * (2 * C::STAGE);

  // ---- Q fragment: B operand of S^T = K.Q^T, resident for the whole loop ---
  // bf16: step s, lane half g holds dims [16s + 8g, +8); fp8: dims [64s + 32g, +32).
  u32x4 qf[C::QREGS];
#pragma unroll
  for (int s = 0; s < C::QREGS; ++s) {
    const int byte = FP8 ? (64 * (s >> 1) + 32 * g + 16 * (s & 1)) : (32 * s + 16 * g);
    // fp8 at d = 32: the upper half-wave holds the zero half of the 64-deep operand
    const bool in_row = !(FP8 && D == 32) || g == 0;
    qf[s] = (qi < p.Sq && in_row) ? *(const u32x4*)(qbase + (size_t)qi * p.q_ss + byte) : u32x4{0, 0, 0, 0};
  }

  // ---- staging assignment --------------------------------------------------
  const int kc_ = tid % C::KCH;   // K: 16-byte chunk within a row
  const int kr0 = tid / C::KCH;   // K: first row
  const int vu = tid % C::VU;     // V: 4-key unit
  const int vdc = tid / C::VU;    // V: 8-dim chunk
  const int vd0 = 8 * vdc;

  u32x4 kreg[C::KPASS];
  u32x4 vreg[4];  // bf16: 8 dims of 4 keys; fp8: .xy holds 8 codes of 4 keys

  auto stage_load = [&](int kv0) {
#pragma unroll
    for (int t = 0; t < C::KPASS; ++t) {
      const int kr = kv0 + kr0 + t * C::KROWS_PER_PASS;
      kreg[t] = (kr < p.Sk) ? *(const u32x4*)(kbase + (size_t)kr * p.k_ss + 16 * kc_) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kr = kv0 + 4 * vu + t;
      if (C::VTHREADS < 256 && tid >= C::VTHREADS) {
        vreg[t] = u32x4{0, 0, 0, 0};
      } else if (FP8) {
        u32x2 x = (kr < p.Sk) ? *(const u32x2*)(vbase + (size_t)kr * p.v_ss + vd0) : u32x2{0, 0};
        vreg[t] = u32x4{x[0], x[1], 0, 0};
      } else {
        vreg[t] = (kr < p.Sk) ? *(const u32x4*)(vbase + (size_t)kr * p.v_ss + 2 * vd0) : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto stage_store = [&](unsigned char* buf) {
    unsigned char* kl = buf;
    unsigned char* vl = buf + C::KBYTES;
#pragma unroll
    for (int t = 0; t < C::KPASS; ++t) {
      const int r = kr0 + t * C::KROWS_PER_PASS;
      const int phys = kc_ ^ (swap_bits23(r & 15) & (C::KCH - 1));
      *(u32x4*)(kl + r * C::KRB + 16 * phys) = kreg[t];
    }
    // V tile -> V^T: row = dim, 4 consecutive keys per 8-byte unit.
    if (C::VTHREADS < 256 && tid >= C::VTHREADS) return;
    uint32_t w[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (FP8) {
        // e4m3 -> bf16 is exact (bf16 has more exponent and mantissa bits).
        w[t][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[t][0], 1.0f, false));
        w[t][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[t][0], 1.0f, true));
        w[t][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[t][1], 1.0f, false));
        w[t][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vreg[t][1], 1.0f, true));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[t][j] = vreg[t][j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pw = j >> 1;
      u32x2 val;
      if (j & 1) {
        val = u32x2{pack_hi16(w[0][pw], w[1][pw]), pack_hi16(w[2][pw], w[3][pw])};
      } else {
        val = u32x2{pack_lo16(w[0][pw], w[1][pw]), pack_lo16(w[2][pw], w[3][pw])};
      }
      const int dd = vd0 + j;
      const int hsw = j ^ (vdc & 1);  // = (dd & 7) ^ ((dd >> 3) & 1)
      const int phys = vu ^ (2 * hsw);
      *(u32x2*)(vl + dd * C::VTRB + 8 * phys) = val;
    }
  };

  // ---- per-lane LDS read offsets (loop invariant) --------------------------
  // K (A operand of S^T): row 32*kb + pi(i32), chunk swizzled by i32.
  const int krow_off = swap_bits23(i32) * C::KRB;
  const int kswz = i32 & (C::KCH - 1);
  // V^T (A operand of O^T): row 32*db + i32, unit pair (4*kc + 2*g) swizzled.
  const int vrow_off = i32 * C::VTRB;
  const int vswz = 2 * ((i32 & 7) ^ ((i32 >> 3) & 1));

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  // Running row max, in log2 units of the scaled score. It starts at the most
  // negative float rather than -inf: a tile in which a row sees no key (the
  // second key half under the causal mask) then rescales by exp2(0) and gives
  // probabilities exp2(-inf) = 0, and the first tile with a visible key
  // rescales the zero state by exp2(-FLT_MAX - m) = 0.
  float m_run = -__FLT_MAX__;
  float l_run = 0.f;        // this lane's part of the running normaliser
  const float c = p.qk_scale_log2;

  if (t_lo < t_hi) {
    stage_load(t_lo * C::BN);
    stage_store(ring);
  }
  __syncthreads();

  for (int i = 0; i < n_steps; ++i) {
    const int kt = t_lo + i;
    const int kv0 = kt * C::BN;
    if (kt + 1 < t_hi) stage_load(kv0 + C::BN);

    if (kt < t_hi && kt < wave_tiles) {
      const unsigned char* kl = ring + (i & 1) * C::STAGE;
      const unsigned char* vl = kl + C::KBYTES;

      // S^T = K . Q^T for BN keys x 32 queries.
      f32x16 s[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = f32x16{};
        const unsigned char* krow = kl + kb * 32 * C::KRB + krow_off;
#pragma unroll
        for (int st = 0; st < C::QK_STEPS; ++st) {
          if (FP8) {
            // d = 32: both half-waves read the row's two chunks; the upper half's copy
            // meets the zero half of the Q operand, so it adds nothing
            const int c0 = D == 32 ? 0 : 4 * st + 2 * g;
            const u32x4 a0 = *(const u32x4*)(krow + 16 * (c0 ^ kswz));
            const u32x4 a1 = *(const u32x4*)(krow + 16 * ((c0 + 1) ^ kswz));
            const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                  (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            const u32x4 b0 = qf[2 * st], b1 = qf[2 * st + 1];
            const i32x8 bq = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq, s[kb], 0, 0, 0, kE8M0One, 0, kE8M0One);
          } else {
            const u32x4 a = *(const u32x4*)(krow + 16 * ((2 * st + g) ^ kswz));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, qf[st]), s[kb], 0, 0, 0);
          }
        }
      }

      // Mask keys beyond Sk and, when causal, keys after the query.
      // Accumulator register r of block kb on half g holds key 32kb + 16(r>>3) + 8g + (r&7).
      const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > qw + p.causal_off) || (kv0 + C::BN > p.Sk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
            const bool ok = (key < p.Sk) && (!CAUSAL || key <= qi + p.causal_off);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
      }

      // Online softmax: new running max, rescale factor, probabilities.
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halfwave_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;

      u32x4 pf[C::KC];  // P^T operand: chunk kc, element e <-> key 16kc + 8g + e
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = 8 * j + 2 * e2;
            const float p0 = exp2_fast(__builtin_fmaf(s[kb][r], c, -m_new));
            const float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], c, -m_new));
            rs += p0 + p1;
            pf[2 * kb + j][e2] = pack_bf16x2(p0, p1);
          }
      l_run = l_run * alpha + rs;

      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      }

      // O^T += V^T . P^T
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const unsigned char* vrow = vl + db * 32 * C::VTRB + vrow_off;
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
          const u32x4 a = *(const u32x4*)(vrow + 8 * ((4 * kc + 2 * g) ^ vswz));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < t_hi) stage_store(ring + ((i + 1) & 1) * C::STAGE);
    __syncthreads();
  }

  // ---- merge of the two key halves (SPLIT = 2) -------------------------------
  // The second half's waves leave acc, m_run and l_run in LDS (register-major,
  // 64 lanes contiguous: acc from the start of the first ring, m and l at the
  // end of the second); the first half's wave of the same rows rescales both
  // to the larger reference and adds. A row always sees key 0, so the first
  // half's reference is a real score maximum; a second half in which a row
  // saw no key keeps -FLT_MAX and gets the factor 0.
  if constexpr (SPLIT == 2) {
    float* const m_acc = (float*)smem + wave * (C::DB * 16 * 64);
    float* const m_ml = (float*)(smem + 4 * C::STAGE) - 8 * 64 + wave * (2 * 64);
    static_assert(4 * C::DB * 16 * 64 * 4 + 8 * 64 * 4 <= 2 * C::STAGE, "merge state fits beside the stage");
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

  // ---- epilogue: normalise, round to bf16, store O (and lse) ---------------
  // A lane holds 4-dim pieces of one query row, so the wave writes its 32-row
  // output tile to LDS (idle after the last barrier; with SPLIT = 2 the second
  // ring, clear of the merge state; wave w takes 32 * 2D bytes) and reads it
  // back as whole rows: each global store then covers 1 KB of contiguous rows. 16-byte chunks are XOR-swizzled by row; the stores
  // carry the non-temporal hint (nothing in the kernel reads O back).
  if (!wave_active) return;
  const float l_tot = halfwave_sum(l_run);
  const float inv = p.o_scale / l_tot;
  constexpr int ORB = 2 * D, OCH = ORB / 16;
  static_assert(4 * 32 * ORB + 8 * 64 * 4 <= 2 * C::STAGE, "the output stage fits below the merge's m and l");
  unsigned char* stage = smem + (SPLIT == 2 ? 2 * C::STAGE : 0) + wave * (32 * ORB);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int chunk = 4 * db + q4;  // dims 32 db + 8 q4 + [0, 8); this lane's 4 of them start at 4 g
      *(u32x2*)(stage + i32 * ORB + 16 * (chunk ^ (i32 & (OCH - 1))) + 8 * g) =
          u32x2{pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv)};
    }
  unsigned char* obase = (unsigned char*)head_ptr(p.o, p.o_sb, p.o_sh, b, hq);
  const int pchunk = lane % OCH;
#pragma unroll
  for (int t = 0; t < 32 * ORB / 1024; ++t) {
    const int r = (1024 / ORB) * t + lane / OCH;
    const u32x4 val = *(const u32x4*)(stage + r * ORB + 16 * pchunk);
    if (qw + r < p.Sq)
      __builtin_nontemporal_store(val, (u32x4*)(obase + (size_t)(qw + r) * p.o_ss + 16 * (pchunk ^ (r & (OCH - 1)))));
  }
  if (g == 0 && qi < p.Sq && p.lse != nullptr) p.lse[qo_row0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// Grids of at most one workgroup per CU over at least 3 key tiles split the
// keys over eight waves (the bf16 kernel's rule).
constexpr unsigned kSplitMaxGrid = 256;
constexpr int kSplitMinKeys = 384;

template <int D, bool CAUSAL, bool FP8>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.B * (unsigned)p.Hq;
  // hipLaunchKernel reports the status of this launch alone.
  AttnParams arg = p;
  void* args[] = {&arg};
  if (grid <= kSplitMaxGrid && p.Sk >= kSplitMinKeys)
    return hipLaunchKernel((const void*)&attn_fwd_mfma_kernel<D, CAUSAL, FP8, 2>, dim3(grid), dim3(512), args, 0,
                           stream);
  return hipLaunchKernel((const void*)&attn_fwd_mfma_kernel<D, CAUSAL, FP8, 1>, dim3(grid), dim3(256), args, 0,
                         stream);
}

int fp8_block_m(int d) { return d == 128 ? fp8_pp_block_m() : 128; }

// attn_fwd_ppk.hip: the key-half ping-pong kernel on e4m3 inputs, 128-row
// q-tiles (the grid of attn_fwd_mfma_kernel). At d = 64, unlike bf16, it also
// wins on large grids (B8 H16 S2048: 177 -> 156 us), where its scores run on
// the fp8 matrix cores.
hipError_t launch_attn_fp8_ppk(const AttnParams& p, int d, bool causal, hipStream_t stream);
// Whether a d = 128 shape is small enough for it (else the 256-row fp8 kernel).
bool ppk_takes_d128(const AttnParams& p, bool causal);

hipError_t launch_attn_fp8(const AttnParams& p, int d, bool causal, hipStream_t stream) {
  if (d == 128) {
    if (!ppk_takes_d128(p, causal)) return launch_attn_fp8_pp(p, causal, stream);
    AttnParams q = p;
    q.n_qtiles = (p.Sq + 127) / 128;
    return launch_attn_fp8_ppk(q, 128, causal, stream);
  }
  if (d == 64 && p.Sk >= 1024)
    return launch_attn_fp8_ppk(p, 64, causal, stream);
  if (d == 32) return causal ? launch_one<32, true, true>(p, stream) : launch_one<32, false, true>(p, stream);
  return causal ? launch_one<64, true, true>(p, stream) : launch_one<64, false, true>(p, stream);
}

}  // namespace sdpa18
