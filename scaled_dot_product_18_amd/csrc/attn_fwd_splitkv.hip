// Split-KV attention forward for a few queries against a long key sequence
// (decoding with a KV cache), bf16 inputs and output, gfx950.
//
// The arithmetic is that of the fused forward ("Accelerate attention on GPU
// with cuDNN and TransformerEngine", intro and sections 4, 7, 9; "Self-attention,
// CUDA kernels and FlashAttention", section 3): scores of a key block exist only
// in registers, an online softmax carries a running maximum and normaliser, and
// only O and the log-sum-exp leave the chip. What changes is how the work is
// spread when Sq is small and Sk is large (the KV-cache shapes of the codelab's
// section 9 and its closing next steps):
//  * the rows of all G query heads that share a KV head are packed into the
//    32 columns of one MFMA score tile (column c <-> query head hk*G + c / Sq,
//    query c % Sq), so a KV head's keys are read once for the whole group;
//  * the keys are cut into chunks, one workgroup per (chunk, column tile, KV
//    head, batch). With more than one chunk each workgroup writes its chunk's
//    normalised partial output and base-2 log-sum-exp to the caller's
//    workspace, and a second kernel merges the chunks with the identity the
//    online softmax uses between tiles: O = sum_s w_s O_s / sum_s w_s with
//    w_s = 2^(lse_s - max_s lse_s);
//  * inside a workgroup each of the 4 waves takes every 4th 32-key block of
//    the chunk and streams it HBM -> LDS with buffer_load ... lds into its own
//    two-slot ring, so the loop has no workgroup barrier; the four waves'
//    (max, sum, accumulator) merge through LDS at the end;
//  * scores are computed transposed as in the other bf16 kernels
//    (S^T = K . Q^T on v_mfma_f32_32x32x16_bf16, lane = query column, the score
//    accumulator rounded to bf16 is the P^T operand of O^T += V^T . P^T, V^T read
//    with ds_read_b64_tr_b16).
// The path is bound by the HBM reads of K and V: per 32-key block a wave moves
// 16 KB (d = 128) and spends 16 MFMAs on it, about a tenth of what the matrix
// cores could absorb at the HBM rate, so the unused columns of a tile cost
// nothing that matters.
#include "kernel_common.h"
#include "launch.h"

namespace sdpa18 {
namespace splitkv {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kBlock = 32;                 // keys per block: the rows of one score tile
constexpr int kBufferConfig = 0x00020000;  // word 3 of a raw buffer resource: 32-bit data format

template <int D>
struct Cfg {
  static constexpr int RB = 2 * D;           // bytes per K/V row
  static constexpr int CH = RB / 16;         // 16-byte chunks per row
  static constexpr int KBLK = kBlock * RB;   // bytes of a K (or V) block
  static constexpr int SLOT = 2 * KBLK;      // one ring slot: K block then V block
  static constexpr int NL = KBLK / 1024;     // 1 KB wave-wide DMA loads per block per tensor
  static constexpr int QS = D / 16;          // MFMAs per score tile
  static constexpr int DB = D / 32;          // 32-dim output blocks
  static_assert(DB * 16 * 64 * 4 == SLOT, "the merge stages one wave's accumulator in its slot");
};

// s_waitcnt immediate for vmcnt(n), other counters unconstrained (gfx9
// encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// XOR swizzles of the 16-byte chunks of a K row (MFMA operand reads: 16 lanes
// at 16 rows, one logical chunk) and of a V row (transposing reads: 4
// consecutive rows, 32 bytes each); both leave the reads free of bank conflicts.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((0xCA60 >> (4 * (row & 3))) & 15) : ((0x6420 >> (4 * (row & 3))) & 15);
}

// NL wave-wide loads HBM -> LDS of one block (lane l of load t fills dst + 1024 t
// + 16 l). The buffer ends at the chunk's last key, so rows past it load zeros.
template <int NL>
__device__ __forceinline__ void dma_block(const unsigned char* src, int bytes_left, const unsigned* off,
                                          unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, bytes_left, kBufferConfig);
#pragma unroll
  for (int t = 0; t < NL; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * t), 16, off[t], 0, 0, 0);
}

// DMA of key block kv0 (K then V) of one chunk into a ring slot; a block at or
// past the chunk's end gets an empty range and loads zeros.
template <int D>
__device__ __forceinline__ void issue_block(const unsigned char* kbase, const unsigned char* vbase, int kv0,
                                            int kv_end, const unsigned* koff, const unsigned* voff,
                                            unsigned char* slot) {
  using C = Cfg<D>;
  const int left = kv0 < kv_end ? (kv_end - kv0) * C::RB : 0;
  dma_block<C::NL>(kbase + (size_t)kv0 * C::RB, left, koff, slot);
  dma_block<C::NL>(vbase + (size_t)kv0 * C::RB, left, voff, slot + C::KBLK);
}

// Wait until at most n of this wave's vector-memory operations are in flight;
// the empty asm statement keeps later LDS reads from moving above the wait.
template <int N>
__device__ __forceinline__ void wait_vm_then() {
  __builtin_amdgcn_s_waitcnt(wait_vm(N));
  asm volatile("" ::: "memory");
}

// Wait until this wave's LDS reads have returned. A DMA into a slot is issued
// only after this: the compiler orders the DMA after the reads' issue, not
// after their completion, and the DMA's write could otherwise overtake a read
// of the block it replaces.
__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
  asm volatile("" ::: "memory");
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_fwd_splitkv_kernel(const SplitParams sp) {
  using C = Cfg<D>;
  // Two ring slots per wave, in two LDS objects: the compiler then never makes
  // a read of one slot wait for the DMA into the other.
  __shared__ __attribute__((aligned(1024))) unsigned char ring0[kWaves * C::SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char ring1[kWaves * C::SLOT];
  __shared__ float stat_m[kWaves][32];
  __shared__ float stat_l[kWaves][32];

  const AttnParams& p = sp.a;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  // ---- work item: (column tile, batch, KV head, key chunk) ---------------------
  const int per_tile = p.B * p.Hkv * sp.n_splits;
  const int ct = blockIdx.x / per_tile;
  const int rem = blockIdx.x - ct * per_tile;
  const int pair = rem / sp.n_splits;
  const int split = rem - pair * sp.n_splits;
  const int b = pair / p.Hkv;
  const int hk = pair - b * p.Hkv;

  // ---- this lane's query column ------------------------------------------------
  const int col = ct * 32 + i32;
  const bool col_ok = col < p.group * p.Sq;
  const int gq = col_ok ? col / p.Sq : 0;
  const int qi = col_ok ? col - gq * p.Sq : 0;
  const int hq = hk * p.group + gq;
  const size_t row = ((size_t)b * p.Hq + hq) * (size_t)p.Sq + qi;  // output row of this column
  const int lim = col_ok ? qi + p.causal_off : 0x7fffffff;          // last visible key (causal)

  const int kv_begin = split * sp.chunk;
  const int kv_end = min(p.Sk, kv_begin + sp.chunk);
  const int n_blocks = (kv_end - kv_begin + kBlock - 1) / kBlock;
  const int nw = n_blocks > wave ? (n_blocks - wave + kWaves - 1) / kWaves : 0;  // blocks of this wave

  const size_t kv_row0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Sk;
  const unsigned char* kbase = (const unsigned char*)p.k + kv_row0 * C::RB;
  const unsigned char* vbase = (const unsigned char*)p.v + kv_row0 * C::RB;

  // DMA slot s = 64 t + lane of a block: row s / CH, physical chunk s % CH.
  unsigned koff[C::NL], voff[C::NL];
#pragma unroll
  for (int t = 0; t < C::NL; ++t) {
    const int r = (64 * t + lane) / C::CH;
    const int pc = lane % C::CH;
    koff[t] = r * C::RB + 16 * (pc ^ k_swz<D>(r));
    voff[t] = r * C::RB + 16 * (pc ^ v_swz<D>(r));
  }

  // Q fragment (B operand of S^T): step s, half g holds dims [16s + 8g, +8).
  const unsigned char* qrow = (const unsigned char*)p.q + row * C::RB;
  u32x4 qf[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s)
    qf[s] = col_ok ? *(const u32x4*)(qrow + 32 * s + 16 * g) : u32x4{0, 0, 0, 0};

  // LDS operand offsets inside a slot. K: row i32, logical chunk 2s + g.
  int k_rd[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) k_rd[s] = i32 * C::RB + 16 * ((2 * s + g) ^ k_swz<D>(i32));
  // V^T through the transposing read: lane J of each 16-lane group reads dims
  // [dbase + 4(J%4), +4) of key row (row_base + J/4).
  const int J = lane & 15;
  int v_rd[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int r = 4 * g + (J >> 2);
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (J & 3);
    v_rd[db] = C::KBLK + r * C::RB + 16 * ((d >> 3) ^ v_swz<D>(r)) + 2 * (d & 7);
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running maximum, log2 units of the scaled score
  float l_run = 0.f;        // this lane's share of the normaliser
  const float c = p.qk_scale_log2;

  auto compute_block = [&](int j, const unsigned char* slot) {
    const int kv0 = kv_begin + kBlock * j;
    // S^T = K . Q^T; register r on half g holds key kv0 + 8(r/4) + 4g + r%4.
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < C::QS; ++st) {
      const u32x4 a = *(const u32x4*)(slot + k_rd[st]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]),
                                                  s, 0, 0, 0);
    }
    const bool tail = kv0 + kBlock > kv_end;
    const bool diag = CAUSAL && __builtin_amdgcn_ballot_w64(kv0 + kBlock - 1 > lim) != 0;
    if (tail || diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < kv_end && (!CAUSAL || key <= lim);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_new = fmaxf(m_run, halfwave_max(mx) * c);
    // A column with no visible key so far keeps m = -inf; exponentiate against
    // 0 then, so every probability is exp2(-inf) = 0 instead of NaN.
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;

    // P^T operand: chunk kc, element e <-> key 16kc + 8(e/4) + 4g + e%4.
    u32x4 pf[2];
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int r = 8 * kc + 2 * e2;
        const float p0 = exp2_fast(__builtin_fmaf(s[r], c, -m_use));
        const float p1 = exp2_fast(__builtin_fmaf(s[r + 1], c, -m_use));
        pf[kc][e2] = pack_bf16x2(p0, p1);
        lsum[e2] += p0;
        lsum[e2] += p1;
      }
    l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slot + 16 * kc * C::RB + v_rd[db]));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slot + (16 * kc + 8) * C::RB + v_rd[db]));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pf[kc]), acc[db], 0, 0, 0);
      }
  };

  // ---- this wave's blocks wave, wave + 4, ...: slot 0 for even i, slot 1 for odd
  unsigned char* const slot0 = ring0 + wave * C::SLOT;
  unsigned char* const slot1 = ring1 + wave * C::SLOT;
  // Two blocks are in flight ahead of the one being computed: block i + 2 is
  // issued into a slot as soon as the reads of block i from it have returned. A wave runs
  // an even number of blocks, the last one possibly past the end of the chunk;
  // such blocks get an empty buffer range (their DMA writes zeros) and the
  // key mask removes them. So the loop body is straight-line code, every wait
  // is the same vmcnt(2 NL), and no control-flow join hides from the compiler
  // which slot a pending DMA writes (it would then wait for all of them). The
  // DMA is issued from the kernel body, not from a lambda: the host pass
  // rejects a device function called from a lambda in a kernel template.
  const int kv_w = kv_begin + kBlock * wave;  // first key of this wave's block i is kv_w + 128 i
  constexpr int kStride = kBlock * kWaves;
  issue_block<D>(kbase, vbase, kv_w, kv_end, koff, voff, slot0);
  issue_block<D>(kbase, vbase, kv_w + kStride, kv_end, koff, voff, slot1);
  wait_vm_then<4 * C::NL>();  // Q has landed
  for (int i = 0; i < nw; i += 2) {
    wait_vm_then<2 * C::NL>();  // block i has landed; block i + 1 may still be in flight
    compute_block(wave + kWaves * i, slot0);
    wait_lds_reads();
    issue_block<D>(kbase, vbase, kv_w + kStride * (i + 2), kv_end, koff, voff, slot0);
    wait_vm_then<2 * C::NL>();
    compute_block(wave + kWaves * (i + 1), slot1);
    wait_lds_reads();
    issue_block<D>(kbase, vbase, kv_w + kStride * (i + 3), kv_end, koff, voff, slot1);
  }
  wait_vm_then<0>();

  // ---- merge the four waves ----------------------------------------------------
  // Every DMA of this wave has completed (vmcnt(0) above), so its slot 0 can
  // hold its accumulator: float index (16 db + r) * 64 + lane.
  const float l_w = halfwave_sum(l_run);
  float* const mine = (float*)slot0;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) mine[(16 * db + r) * 64 + lane] = acc[db][r];
  if (g == 0) {
    stat_m[wave][i32] = m_run;
    stat_l[wave][i32] = l_w;
  }
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, stat_m[w][i32]);
  float f[kWaves];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    f[w] = M == -INFINITY ? 0.f : exp2_fast(stat_m[w][i32] - M);
    L += f[w] * stat_l[w][i32];
  }
  if (!col_ok) return;
  const float inv = L > 0.f ? 1.0f / L : 0.f;

  // Wave w finishes registers 4w..4w+3 of every block: dims 32 db + 8w + 4g + (0..3).
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* src = (const float*)(ring0 + w * C::SLOT) + (16 * db + 4 * wave) * 64 + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] += f[w] * src[64 * q];
    }
    o *= inv;
    const int d = 32 * db + 8 * wave + 4 * g;
    if (sp.n_splits == 1) {
      *(u32x2*)((unsigned char*)p.o + row * C::RB + 2 * d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      *(f32x4*)(sp.part_o + (row * sp.n_splits + split) * D + d) = o;
    }
  }
  if (wave == 0 && g == 0) {
    const float lse2 = L > 0.f ? M + __log2f(L) : -INFINITY;
    if (sp.n_splits == 1) {
      if (p.lse != nullptr) p.lse[row] = lse2 * kLn2;
    } else {
      sp.part_lse[row * sp.n_splits + split] = lse2;
    }
  }
}

// Merge of the chunks: one wave per output row, lane l owns dims [D/64 * l, +D/64).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void attn_splitkv_merge_kernel(const SplitParams sp) {
  constexpr int E = D / 64;
  const size_t rows = (size_t)sp.a.B * sp.a.Hq * sp.a.Sq;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int ns = sp.n_splits;
  const float* pl = sp.part_lse + row * ns;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pl[s]);
  float L = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2_fast(pl[s] - M);  // a chunk with no visible key has lse -inf: weight 0
    L += w;
    const float* src = sp.part_o + (row * ns + s) * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += w * src[e];
  }
  const float inv = 1.0f / L;
  unsigned char* dst = (unsigned char*)sp.a.o + row * (2 * D) + 2 * E * lane;
  if constexpr (E == 2) {
    *(uint32_t*)dst = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    *(bf16_t*)dst = (bf16_t)(o[0] * inv);
  }
  if (lane == 0 && sp.a.lse != nullptr) sp.a.lse[row] = (M + __log2f(L)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch_d(const SplitParams& sp, hipStream_t stream) {
  const unsigned grid = (unsigned)sp.n_ctiles * (unsigned)sp.a.B * (unsigned)sp.a.Hkv * (unsigned)sp.n_splits;
  SplitParams arg = sp;
  void* args[] = {&arg};
  hipError_t e =
      hipLaunchKernel((const void*)&attn_fwd_splitkv_kernel<D, CAUSAL>, dim3(grid), dim3(256), args, 0, stream);
  if (e != hipSuccess || sp.n_splits == 1) return e;
  const size_t rows = (size_t)sp.a.B * sp.a.Hq * sp.a.Sq;
  return hipLaunchKernel((const void*)&attn_splitkv_merge_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256),
                         args, 0, stream);
}

}  // namespace splitkv

hipError_t launch_attn_splitkv_bf16(const SplitParams& sp, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? splitkv::launch_d<128, true>(sp, stream) : splitkv::launch_d<128, false>(sp, stream);
  return causal ? splitkv::launch_d<64, true>(sp, stream) : splitkv::launch_d<64, false>(sp, stream);
}

}  // namespace sdpa18
