// C ABI of the fused attention library: argument validation and dispatch.
//
// Every check runs on the host before anything is enqueued, so a rejected
// call has no effect on the stream. Unsupported requests are errors; there is
// no fallback path.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "kernel_common.h"
#include "launch.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* ptr) { return ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool positive_finite(float x) { return isfinite(x) && x > 0.0f; }

// Shared validation of attn_fwd and attn_fwd_fp8. Returns ATTN_OK or an error.
int validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq, int Hkv,
             int Sq, int Sk, int d, int causal) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return ATTN_ERR_SHAPE;
  // Row offsets inside one head and the grid size are 32-bit.
  const int64_t block_m = 128;
  const int64_t tiles = (Sq + block_m - 1) / block_m;
  if ((int64_t)Sq * d * 4 >= INT32_MAX || (int64_t)Sk * d * 4 >= INT32_MAX ||
      tiles * (int64_t)B * (int64_t)Hq >= INT32_MAX)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 32 && d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (causal && Sq > Sk) return ATTN_ERR_CAUSAL_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Element strides of q, k, v, o: {batch, head, position} for each, 12 values.
struct Strides {
  int64_t v[12];
};

Strides dense_strides(int Hq, int Hkv, int Sq, int Sk, int d) {
  const int64_t qo[3] = {(int64_t)Hq * Sq * d, (int64_t)Sq * d, d};
  const int64_t kv[3] = {(int64_t)Hkv * Sk * d, (int64_t)Sk * d, d};
  Strides s;
  for (int i = 0; i < 3; ++i) {
    s.v[i] = qo[i];
    s.v[3 + i] = kv[i];
    s.v[6 + i] = kv[i];
    s.v[9 + i] = qo[i];
  }
  return s;
}

// Every row 16-byte aligned (given aligned bases), rows of one head disjoint,
// and a head's rows within the kernels' 32-bit offsets.
bool strides_ok(const Strides& st, int Sq, int Sk, int d, int in_bytes, int out_bytes) {
  for (int t = 0; t < 4; ++t) {
    const int es = t == 3 ? out_bytes : in_bytes;
    const int S = (t == 0 || t == 3) ? Sq : Sk;
    const int64_t sb = st.v[3 * t], sh = st.v[3 * t + 1], ss = st.v[3 * t + 2];
    if (sb < 0 || sh < 0 || ss < d) return false;
    if ((sb * es) % 16 != 0 || (sh * es) % 16 != 0 || (ss * es) % 16 != 0) return false;
    if (((int64_t)S - 1) * ss * es + (int64_t)d * es >= INT32_MAX || 128 * ss * es >= INT32_MAX) return false;
  }
  return true;
}

sdpa18::AttnParams make_params(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int Sq, int Sk, int causal, float qk_scale, float o_scale, int block_m,
                               const Strides& st, int in_bytes, int out_bytes) {
  sdpa18::AttnParams p;
  p.q_sb = st.v[0] * in_bytes;
  p.q_sh = st.v[1] * in_bytes;
  p.q_ss = (int)(st.v[2] * in_bytes);
  p.k_sb = st.v[3] * in_bytes;
  p.k_sh = st.v[4] * in_bytes;
  p.k_ss = (int)(st.v[5] * in_bytes);
  p.v_sb = st.v[6] * in_bytes;
  p.v_sh = st.v[7] * in_bytes;
  p.v_ss = (int)(st.v[8] * in_bytes);
  p.o_sb = st.v[9] * out_bytes;
  p.o_sh = st.v[10] * out_bytes;
  p.o_ss = (int)(st.v[11] * out_bytes);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.group = Hq / Hkv;
  p.n_qtiles = (Sq + block_m - 1) / block_m;
  p.qk_scale_log2 = qk_scale * kLog2e;
  p.o_scale = o_scale;
  // Each XCD gets whole KV heads when they split evenly over the 8 XCDs.
  p.xcd_remap = ((B * Hkv) % 8 == 0) ? 1 : 0;
  // The queries are the last Sq of Sk positions: query i sits at position i + Sk - Sq.
  p.causal_off = causal ? Sk - Sq : 0;
  return p;
}

int launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Workspace of attn_bwd: per-row delta and lse * log2(e) (2 * B*Hq*Sq floats),
// then, when the dK/dV kernel splits the query heads of a KV head, 16-byte
// aligned fp32 partial dK and dV of every subset.
size_t bwd_part_offset(int B, int Hq, int Sq) { return (2 * (size_t)B * Hq * Sq * sizeof(float) + 15) / 16 * 16; }
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
  const int ks = sdpa18::bwd_kv_split(B, Hkv, Sk, Hq / Hkv);
  if (ks == 1) return 2 * (size_t)B * Hq * Sq * sizeof(float);
  return bwd_part_offset(B, Hq, Sq) + 2 * (size_t)ks * B * Hkv * Sk * d * sizeof(float);
}

constexpr int kMaxSplits = 128;

// Checks of attn_fwd_splitkv_plan and attn_fwd_splitkv beyond the shared ones.
int validate_split_sizes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_SPLITS;
  const int64_t ctiles = ((int64_t)(Hq / Hkv) * Sq + 31) / 32;
  if ((int64_t)Sq * d * 4 >= INT32_MAX || (int64_t)Sk * d * 4 >= INT32_MAX ||
      ctiles * B * Hkv * kMaxSplits >= INT32_MAX || (int64_t)B * Hq * Sq >= INT32_MAX)
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Key chunking of the split-KV path. num_splits = 0 picks enough chunks for
// one resident round of workgroups on the 256 CUs (one workgroup per CU at
// d = 128, where a workgroup holds 128 KB of LDS; two at d = 64), keeping at
// least 256 keys (two 32-key blocks per wave) in a chunk. Chunks hold a
// multiple of 32 keys; the count is what remains after rounding, so no chunk
// is empty.
struct SplitPlan {
  int n_splits, chunk, n_ctiles;
  size_t workspace;
};
SplitPlan plan_splits(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits) {
  SplitPlan pl;
  pl.n_ctiles = (int)(((int64_t)(Hq / Hkv) * Sq + 31) / 32);
  const int max_blocks = (Sk + 31) / 32;
  int ns;
  if (num_splits > 0) {
    ns = num_splits < max_blocks ? num_splits : max_blocks;
  } else {
    const int64_t items = (int64_t)B * Hkv * pl.n_ctiles;
    const int64_t target = d == 128 ? 256 : 512;
    int64_t want = (target + items - 1) / items;
    const int64_t by_len = (Sk + 255) / 256;
    if (want > by_len) want = by_len;
    if (want > kMaxSplits) want = kMaxSplits;
    ns = want < 1 ? 1 : (int)want;
  }
  pl.chunk = ((Sk + ns - 1) / ns + 31) / 32 * 32;
  pl.n_splits = (Sk + pl.chunk - 1) / pl.chunk;
  pl.workspace = pl.n_splits > 1 ? (size_t)B * Hq * Sq * pl.n_splits * (size_t)(d + 1) * sizeof(float) : 0;
  return pl;
}


// Shared path of attn_fwd, attn_fwd_fp8 and attn_fwd_strided (descales are 1 unless dtype is fp8).
int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Sq,
               int Sk, int d, const Strides& st, float scale, int causal, int dtype, float descale_q,
               float descale_k, float descale_v, hipStream_t stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  const int s = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal);
  if (s != ATTN_OK) return s;
  const int in_bytes = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  const int out_bytes = dtype == ATTN_F32 ? 4 : 2;
  if (!strides_ok(st, Sq, Sk, d, in_bytes, out_bytes)) return ATTN_ERR_STRIDE;
  if (!positive_finite(scale) || !positive_finite(descale_q) || !positive_finite(descale_k) ||
      !positive_finite(descale_v))
    return ATTN_ERR_SCALE;
  const float qk = scale * descale_q * descale_k;
  if (!positive_finite(qk * kLog2e)) return ATTN_ERR_SCALE;
  if (dtype == ATTN_F32) {
    const sdpa18::AttnParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, causal, qk, 1.0f,
                                             sdpa18::f32_block_m(), st, in_bytes, out_bytes);
    return launch_status(sdpa18::launch_attn_f32(p, d, causal != 0, stream));
  }
  if (dtype == ATTN_BF16) {
    const sdpa18::AttnParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, causal, qk, 1.0f,
                                             sdpa18::bf16_block_m(d), st, in_bytes, out_bytes);
    return launch_status(sdpa18::launch_attn_bf16(p, d, causal != 0, stream));
  }
  const sdpa18::AttnParams p = make_params(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, causal, qk, descale_v,
                                           sdpa18::fp8_block_m(d), st, in_bytes, out_bytes);
  return launch_status(sdpa18::launch_attn_fp8(p, d, causal != 0, stream));
}

// Workspace of attn_bwd_fp8: the bf16 backward's, then bf16 copies of q, k,
// v and dout (the fp8 codes widened), each from a 16-byte boundary.
size_t align16(size_t x) { return (x + 15) / 16 * 16; }
size_t bwd_fp8_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d) {
  const size_t nq = (size_t)B * Hq * Sq * d, nk = (size_t)B * Hkv * Sk * d;
  return align16(bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d)) + 2 * align16(2 * nq) + 2 * align16(2 * nk);
}

// Shared path of attn_bwd (bf16, fp32) and attn_bwd_fp8 (dtype ATTN_FP8_E4M3:
// e4m3 q, k, v and e5m2 dout with per-tensor descales, bf16 o and outputs).
int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
               int dtype, float ds_q, float ds_k, float ds_v, float ds_do, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  if (o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F32 && d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if ((int64_t)((Sk + 63) / 64) * B * Hkv >= INT32_MAX) return ATTN_ERR_SHAPE;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_ALIGN;
  if (!positive_finite(scale) || !positive_finite(ds_q) || !positive_finite(ds_k) || !positive_finite(ds_v) ||
      !positive_finite(ds_do))
    return ATTN_ERR_SCALE;
  const float qk = scale * ds_q * ds_k;
  if (!positive_finite(qk * kLog2e) || !positive_finite(scale * ds_do * ds_v * ds_k) ||
      !positive_finite(scale * ds_do * ds_v * ds_q))
    return ATTN_ERR_SCALE;
  const size_t rows = (size_t)B * Hq * Sq;
  const size_t need = dtype == ATTN_FP8_E4M3 ? bwd_fp8_workspace_bytes(B, Hq, Hkv, Sq, Sk, d)
                      : dtype == ATTN_F32    ? 2 * rows * sizeof(float)
                                             : bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  sdpa18::BwdParams bp;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.o = o;
  bp.dout = dout;
  bp.lse = lse;
  bp.delta = static_cast<float*>(workspace);
  bp.lse2 = static_cast<float*>(workspace) + rows;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.B = B;
  bp.Hq = Hq;
  bp.Hkv = Hkv;
  bp.Sq = Sq;
  bp.Sk = Sk;
  bp.group = Hq / Hkv;
  bp.causal_off = causal ? Sk - Sq : 0;
  bp.qk_scale_log2 = qk * kLog2e;
  // Real values: q = ds_q q', k = ds_k k', v = ds_v v', dout = ds_do dout'. With
  // delta' = rowsum(dout' o) / ds_v and dS' = P (dout' v'^T - delta'), the
  // gradients are dS = ds_do ds_v dS', dQ = scale dS K, dK = scale dS^T Q, dV = P^T dout.
  bp.delta_mul = 1.0f / ds_v;
  bp.dq_mul = scale * ds_do * ds_v * ds_k;
  bp.dk_mul = scale * ds_do * ds_v * ds_q;
  bp.dv_mul = ds_do;
  bp.n_qtiles = (Sq + 127) / 128;
  bp.n_ktiles = (Sk + 127) / 128;
  if (dtype == ATTN_F32) {
    bp.kv_split = 1;
    bp.dkv_part = nullptr;
    return launch_status(sdpa18::launch_attn_bwd_f32(bp, d, causal != 0, stream));
  }
  bp.kv_split = sdpa18::bwd_kv_split(B, Hkv, Sk, Hq / Hkv);
  bp.dkv_part = bp.kv_split > 1
                    ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + bwd_part_offset(B, Hq, Sq))
                    : nullptr;
  if (dtype == ATTN_BF16) return launch_status(sdpa18::launch_attn_bwd_bf16(bp, d, causal != 0, stream));
  const size_t nq = (size_t)B * Hq * Sq * d, nk = (size_t)B * Hkv * Sk * d;
  unsigned char* w = static_cast<unsigned char*>(workspace) + align16(bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d));
  unsigned char* q16 = w;
  unsigned char* do16 = q16 + align16(2 * nq);
  unsigned char* k16 = do16 + align16(2 * nq);
  unsigned char* v16 = k16 + align16(2 * nk);
  return launch_status(sdpa18::launch_attn_bwd_fp8(bp, q16, k16, v16, do16, d, causal != 0, stream));
}

// Scratch of attn_fwd_splitkv_noalloc: the key chunks' partial outputs and
// log-sum-exps, in a static device array instead of caller memory. Every GPU
// the library runs on holds its own copy until the process ends; in host code
// `scratch` names a host-side stand-in, so kernels receive the device address
// that hipGetSymbolAddress reports, taken once per device with that device
// current and kept below.
static __device__ __align__(256) unsigned char scratch[ATTN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (set up on the first call on
// that device). Returns ATTN_OK or ATTN_ERR_LAUNCH when the runtime refuses.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> guard(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return ATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// Shared path of attn_fwd_splitkv (caller workspace) and
// attn_fwd_splitkv_noalloc (use_scratch: the library's static scratch).
int splitkv_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Sq,
                   int Sk, int d, float scale, int causal, int dtype, int num_splits, void* workspace,
                   size_t workspace_bytes, bool use_scratch, hipStream_t stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  int st = validate(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal);
  if (st != ATTN_OK) return st;
  st = validate_split_sizes(B, Hq, Hkv, Sq, Sk, d, num_splits);
  if (st != ATTN_OK) return st;
  if (!positive_finite(scale) || !positive_finite(scale * kLog2e)) return ATTN_ERR_SCALE;
  const SplitPlan pl = plan_splits(B, Hq, Hkv, Sq, Sk, d, num_splits);
  if (use_scratch) {
    if (pl.workspace > ATTN_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    workspace = nullptr;
    if (pl.workspace > 0) {
      st = device_scratch(&workspace);
      if (st != ATTN_OK) return st;
    }
  } else if (pl.workspace > 0 &&
             (workspace == nullptr || !aligned16(workspace) || workspace_bytes < pl.workspace)) {
    return ATTN_ERR_WORKSPACE;
  }
  sdpa18::SplitParams sp;
  sp.a = make_params(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, causal, scale, 1.0f, 128, dense_strides(Hq, Hkv, Sq, Sk, d), 2,
                     2);
  const size_t rows = (size_t)B * Hq * Sq;
  sp.part_o = pl.workspace > 0 ? static_cast<float*>(workspace) : nullptr;
  sp.part_lse = pl.workspace > 0 ? static_cast<float*>(workspace) + rows * pl.n_splits * (size_t)d : nullptr;
  sp.n_splits = pl.n_splits;
  sp.chunk = pl.chunk;
  sp.n_ctiles = pl.n_ctiles;
  return launch_status(sdpa18::launch_attn_splitkv_bf16(sp, d, causal != 0, stream));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Sq,
             int Sk, int d, float scale, int causal, int dtype, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, dense_strides(Hq, Hkv, Sq, Sk, d), scale, causal, dtype,
                    1.0f, 1.0f, 1.0f, stream);
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse, int B, int Hq, int Hkv,
                 int Sq, int Sk, int d, float scale, int causal, float descale_q, float descale_k, float descale_v,
                 hipStream_t stream) {
  return fwd_common(q8, k8, v8, o_bf16, lse, B, Hq, Hkv, Sq, Sk, d, dense_strides(Hq, Hkv, Sq, Sk, d), scale, causal,
                    ATTN_FP8_E4M3, descale_q, descale_k, descale_v, stream);
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int d, const int64_t* strides, float scale, int causal, int dtype,
                     float descale_q, float descale_k, float descale_v, hipStream_t stream) {
  if (strides == nullptr) return ATTN_ERR_NULL;
  if (dtype != ATTN_FP8_E4M3 && (descale_q != 1.0f || descale_k != 1.0f || descale_v != 1.0f)) return ATTN_ERR_SCALE;
  Strides st;
  for (int i = 0; i < 12; ++i) st.v[i] = strides[i];
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, st, scale, causal, dtype, descale_q, descale_k,
                    descale_v, stream);
}

int attn_fwd_splitkv_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits, int* splits_used,
                          size_t* workspace_bytes) {
  const int st = validate_split_sizes(B, Hq, Hkv, Sq, Sk, d, num_splits);
  if (st != ATTN_OK) return st;
  const SplitPlan pl = plan_splits(B, Hq, Hkv, Sq, Sk, d, num_splits);
  if (splits_used != nullptr) *splits_used = pl.n_splits;
  if (workspace_bytes != nullptr) *workspace_bytes = pl.workspace;
  return ATTN_OK;
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int d, float scale, int causal, int dtype, int num_splits, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return splitkv_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, num_splits, workspace,
                        workspace_bytes, false, stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                             int Hkv, int Sq, int Sk, int d, float scale, int causal, int dtype, int num_splits,
                             hipStream_t stream) {
  return splitkv_common(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, num_splits, nullptr, 0, true,
                        stream);
}

int attn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d, size_t* workspace_bytes) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 32 && d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (workspace_bytes != nullptr) *workspace_bytes = bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d);
  return ATTN_OK;
}

int attn_bwd_fp8_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int d, size_t* workspace_bytes) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (workspace_bytes != nullptr) *workspace_bytes = bwd_fp8_workspace_bytes(B, Hq, Hkv, Sq, Sk, d);
  return ATTN_OK;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, 1.0f, 1.0f, 1.0f,
                    1.0f, workspace, workspace_bytes, stream);
}

int attn_bwd_fp8(const void* q8, const void* k8, const void* v8, const void* o, const void* dout8, const float* lse,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 float descale_q, float descale_k, float descale_v, float descale_do, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(q8, k8, v8, o, dout8, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, scale, causal, ATTN_FP8_E4M3,
                    descale_q, descale_k, descale_v, descale_do, workspace, workspace_bytes, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer (q, k, v, o; for attn_bwd also dout, lse, dq, dk, dv) is null";
    case ATTN_ERR_SHAPE: return "a size is < 1 or the problem exceeds 32-bit indexing";
    case ATTN_ERR_HEADS: return "Hq is not a multiple of Hkv";
    case ATTN_ERR_HEADDIM:
      return "head dimension d must be 32, 64 or 128 (64 or 128 for the split-KV and backward entry points)";
    case ATTN_ERR_CAUSAL_SHAPE: return "causal masking requires Sq <= Sk";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_SCALE: return "scale and descales must be finite and > 0";
    case ATTN_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case ATTN_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch (or the device query before it)";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL, not 16-byte aligned or smaller than the size query reports";
    case ATTN_ERR_SPLITS: return "num_splits must be in [0, 128]";
    case ATTN_ERR_STRIDE:
      return "a stride is negative, leaves rows overlapping or not 16-byte aligned, or spans 2 GiB within a head";
    case ATTN_ERR_SCRATCH:
      return "attn_fwd_splitkv_noalloc: the request needs more than the library's static scratch "
             "(ATTN_SCRATCH_BYTES = 16 MiB); use fewer splits or attn_fwd_splitkv with a workspace";
    default: return "unknown status";
  }
}

int attn_version(void) { return 200; }

}  // extern "C"
