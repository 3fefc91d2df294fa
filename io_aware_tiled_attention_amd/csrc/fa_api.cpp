// fa_api.cpp -- the C ABI declared in include/fa.h: validation, workspace
// carve-up and dispatch to the HIP launchers.  Every argument is checked
// before the first HIP call, so an invalid call enqueues nothing; no C++
// exception crosses the interface.
#include "fa.h"

#include <cmath>
#include <cstdint>

#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Threads per workgroup: the largest of the per-tile kernels (the 8-wave bf16
// dK/dV), and the decoding kernels'.
constexpr int64_t kMaxTileThreads = 512;
constexpr int64_t kDecodeThreads = 64;

// The bf16 kernels fold the score factor into base-2 exponentials:
// factor * log2(e) must be a finite float, or every probability would be NaN.
bool exp2_factor_finite(double factor) { return std::isfinite((float)(factor * 1.4426950408889634)); }

// Shape check shared by every entry point; `empty` is set for B*H*N == 0.
int check_shape(int B, int H, int N, int d, int dtype, float scale, bool* empty) {
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale) || scale < 0.f || !exp2_factor_finite(scale)) return FA_ERR_SCALE;
  // Sizes must fit the kernels' index arithmetic: rows and per-head byte
  // offsets use 32-bit ints, whole-tensor offsets 64-bit.  A ragged last
  // tile addresses up to kRowSlack rows past N (reads there are dropped by
  // the buffer range check), so those rows must fit too.  A launch's
  // work-item count (workgroups x threads) must fit in 32 bits: the largest
  // per-tile grid has one workgroup of kMaxTileThreads per 128 rows of a head
  // (the backward preprocess strides over its rows and has no such limit).
  constexpr int64_t kRowSlack = 256;
  const int64_t rows = (int64_t)B * H * N;
  const int64_t tiles = ((int64_t)N + 127) / 128 * B * H;
  const int64_t head_bytes = ((int64_t)N + kRowSlack) * d * (dtype == FA_BF16 ? 2 : 4);
  if ((int64_t)B * H > INT32_MAX || head_bytes > INT32_MAX || tiles * kMaxTileThreads > (int64_t)UINT32_MAX)
    return FA_ERR_SHAPE;
  *empty = rows == 0;
  return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Validation and launch for any subset of the backward stages.  A pointer is
// required (non-NULL, 16-byte aligned) exactly when a requested stage reads
// or writes it.
// Block-mask geometry shared by the block-sparse forward and backward.
int check_mask(int H, int N, int mask_heads, int block_q, int block_k) {
  if (block_q <= 0 || block_q % 32 != 0 || block_k <= 0 || block_k % 64 != 0 || N > fa::kSparseMaxN ||
      (mask_heads != 1 && mask_heads != H))
    return FA_ERR_MASK;
  return FA_OK;
}

// A block mask for the backward: `mask` non-NULL selects the block-sparse
// kernels (geometry already checked with check_mask).
struct BwdMask {
  const unsigned char* mask = nullptr;
  int mask_heads = 0, block_q = 0, block_k = 0;
};

int run_backward(int stages, const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                 float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                 const fa::DropParams& drop = fa::DropParams{}, const BwdMask& bm = BwdMask{}) {
  bool empty = false;
  const int st = check_shape(B, H, N, d, dtype, scale, &empty);
  if (st != FA_OK) return st;
  if (empty) return FA_OK;
  const bool pre = stages & fa::kStagePre, kv = stages & fa::kStageDkDv, dqs = stages & fa::kStageDq;
  const void* need[12];
  int n_need = 0;
  if (pre) {
    need[n_need++] = o;
    need[n_need++] = dout;
    need[n_need++] = lse;
  }
  if (kv || dqs) {
    const void* ptrs[] = {q, k, v, dout};
    for (const void* p : ptrs) need[n_need++] = p;
  }
  if (kv) {
    need[n_need++] = dk;
    need[n_need++] = dv;
  }
  if (dqs) need[n_need++] = dq;
  for (int i = 0; i < n_need; ++i)
    if (!need[i]) return FA_ERR_NULL;
  for (int i = 0; i < n_need; ++i)
    if (!aligned16(need[i])) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * N;
  if (!workspace || workspace_bytes < fa::ws_bytes(rows)) return FA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal ? 1 : 0, dtype, scale,
                reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + fa::ws_dsum_bytes(rows)), drop};
  a.mask = bm.mask;
  a.mask_heads = bm.mask_heads;
  a.block_q = bm.block_q;
  a.block_k = bm.block_k;
  return hip_status(fa::launch_backward(a, stages, static_cast<hipStream_t>(stream)));
}

// Dropout parameters: t = round(256 p) (float32 product, half away from
// zero) must lie in [0, 255]; t = 0 leaves dropout off (the plain kernels).
int make_drop(float p_drop, unsigned long long seed, unsigned offset, fa::DropParams* out) {
  if (!std::isfinite(p_drop)) return FA_ERR_DROPOUT;
  const float t = std::floor(p_drop * 256.0f + 0.5f);
  if (t < 0.f || t > 255.f) return FA_ERR_DROPOUT;
  out->k0 = (unsigned)(seed & 0xFFFFFFFFull);
  out->k1 = (unsigned)(seed >> 32);
  out->offset = offset;
  out->t = (unsigned)t;
  out->rs = 256.0f / (256.0f - t);
  out->on = out->t > 0;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
               int d, int causal, float scale, int dtype, void* stream) {
  bool empty = false;
  const int st = check_shape(B, H, N, d, dtype, scale, &empty);
  if (st != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, dtype, scale};
  return hip_status(fa::launch_forward(a, static_cast<hipStream_t>(stream)));
}

int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, int causal, float scale, int dtype, float p_drop, unsigned long long seed,
                       unsigned offset, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, dtype, scale, &empty);
  if (st != FA_OK) return st;
  fa::DropParams drop;
  st = make_drop(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, dtype, scale};
  a.drop = drop;
  return hip_status(fa::launch_forward(a, static_cast<hipStream_t>(stream)));
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   int causal, float scale, float q_descale, float k_descale, float v_descale, void* stream) {
  bool empty = false;
  // bf16 output: the per-head size check of the bf16 layout covers the one-byte inputs too
  const int st = check_shape(B, H, N, d, FA_BF16, scale, &empty);
  if (st != FA_OK) return st;
  const float ds[] = {q_descale, k_descale, v_descale};
  for (float x : ds)
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_SCALE;
  // the kernel's score factor scale * q_descale * k_descale * log2(e)
  if (!exp2_factor_finite((double)scale * q_descale * k_descale)) return FA_ERR_SCALE;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::Fp8Args a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, scale, q_descale, k_descale, v_descale};
  return hip_status(fa::launch_forward_fp8(a, static_cast<hipStream_t>(stream)));
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const unsigned char* block_mask, int mask_heads, int block_q, int block_k, int B,
                            int H, int N, int d, int causal, float scale, int dtype, void* stream) {
  bool empty = false;
  const int st = check_shape(B, H, N, d, dtype, scale, &empty);
  if (st != FA_OK) return st;
  const int ms = check_mask(H, N, mask_heads, block_q, block_k);
  if (ms != FA_OK) return ms;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, causal ? 1 : 0, dtype, scale, block_mask, mask_heads, block_q, block_k};
  return hip_status(fa::launch_forward(a, static_cast<hipStream_t>(stream)));
}

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, const unsigned char* block_mask,
                             int mask_heads, int block_q, int block_k, int B, int H, int N, int d, int causal,
                             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  const int st = check_shape(B, H, N, d, dtype, scale, &empty);
  if (st != FA_OK) return st;
  const int ms = check_mask(H, N, mask_heads, block_q, block_k);
  if (ms != FA_OK) return ms;
  if (empty) return FA_OK;
  if (!block_mask) return FA_ERR_NULL;
  return run_backward(fa::kStagePre | fa::kStageDkDv | fa::kStageDq, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d,
                      causal, scale, dtype, workspace, workspace_bytes, stream, fa::DropParams{},
                      BwdMask{block_mask, mask_heads, block_q, block_k});
}

// Decode shapes: Nq in [0, 32], Nk >= 1 unless the problem is empty, causal needs Nq <= Nk.
static int check_decode(int B, int H, int Nq, int Nk, int d, int causal, int dtype, float scale, bool* empty) {
  bool e1 = false, e2 = false;
  int st = check_shape(B, H, Nq, d, dtype, scale, &e1);
  if (st != FA_OK) return st;
  st = check_shape(B, H, Nk, d, dtype, scale, &e2);
  if (st != FA_OK) return st;
  if (Nq > fa::kDecodeMaxNq) return FA_ERR_SHAPE;
  *empty = e1;
  if (e1) return FA_OK;
  if (Nk < 1 || (causal && Nq > Nk)) return FA_ERR_SHAPE;
  return FA_OK;
}

// The two decoding grids, B*H*splits and B*H*Nq workgroups of kDecodeThreads,
// must each stay within 32-bit work-item counts.
static bool decode_grids_fit(int B, int H, int Nq, int splits) {
  const int64_t most = splits > Nq ? splits : Nq;
  return (int64_t)B * H * most * kDecodeThreads <= (int64_t)UINT32_MAX;
}

// Decode workspace: partial O [B*H*S*Nq][d] fp32, then partial lse
// [B*H*S*Nq] fp32, each region 256-byte aligned.  One chunk per head (S = 1)
// writes the outputs directly and needs none.
static size_t decode_ws_bytes(int B, int H, int Nq, int d, int splits) {
  if (splits == 1) return 0;
  const size_t rows = (size_t)B * H * splits * Nq;
  return fa::align256(rows * d * sizeof(float)) + fa::align256(rows * sizeof(float));
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits) {
  bool empty = false;
  if (num_splits < 0 || check_decode(B, H, Nq, Nk, d, 0, FA_BF16, 1.f, &empty) != FA_OK || empty) return 0;
  const int splits = fa::decode_splits(B, H, Nk, num_splits);
  if (!decode_grids_fit(B, H, Nq, splits)) return 0;
  return decode_ws_bytes(B, H, Nq, d, splits);
}

int fa_decode_num_splits(int B, int H, int Nk, int num_splits) {
  if (B <= 0 || H <= 0 || Nk <= 0 || num_splits < 0) return 0;
  return fa::decode_splits(B, H, Nk, num_splits);
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
              int causal, float scale, int dtype, int num_splits, void* workspace, size_t workspace_bytes,
              void* stream) {
  bool empty = false;
  const int st = check_decode(B, H, Nq, Nk, d, causal, dtype, scale, &empty);
  if (st != FA_OK) return st;
  if (num_splits < 0) return FA_ERR_SHAPE;
  if (empty) return FA_OK;
  const int splits = fa::decode_splits(B, H, Nk, num_splits);
  if (!decode_grids_fit(B, H, Nq, splits)) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const size_t need = decode_ws_bytes(B, H, Nq, d, splits);
  fa::DecArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, causal ? 1 : 0, dtype, splits, scale, nullptr, nullptr};
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    const size_t rows = (size_t)B * H * splits * Nq;
    const size_t o_bytes = fa::align256(rows * d * sizeof(float));
    a.opart = reinterpret_cast<float*>(ws);
    a.lpart = reinterpret_cast<float*>(ws + o_bytes);
  }
  return hip_status(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_shape(B, H, N, d, FA_BF16, 1.f, &empty) != FA_OK || empty) return 0;
  return fa::ws_bytes((size_t)B * H * N);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(fa::kStagePre | fa::kStageDkDv | fa::kStageDq, q, k, v, o, dout, lse, dq, dk, dv, B, H, N,
                      d, causal, scale, dtype, workspace, workspace_bytes, stream);
}

int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                        float scale, int dtype, float p_drop, unsigned long long seed, unsigned offset,
                        void* workspace, size_t workspace_bytes, void* stream) {
  fa::DropParams drop;
  const int st = make_drop(p_drop, seed, offset, &drop);
  if (st != FA_OK) {
    bool empty = false;
    const int shape = check_shape(B, H, N, d, dtype, scale, &empty);
    return shape != FA_OK ? shape : st;
  }
  return run_backward(fa::kStagePre | fa::kStageDkDv | fa::kStageDq, q, k, v, o, dout, lse, dq, dk, dv, B, H, N,
                      d, causal, scale, dtype, workspace, workspace_bytes, stream, drop);
}

int fa_backward_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N, int d, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(fa::kStagePre, nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr, nullptr, B, H, N, d,
                      0, 1.f, dtype, workspace, workspace_bytes, stream);
}

int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B, int H,
                     int N, int d, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return run_backward(fa::kStageDkDv, q, k, v, nullptr, dout, nullptr, nullptr, dk, dv, B, H, N, d, causal, scale,
                      dtype, workspace, workspace_bytes, stream);
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B, int H, int N,
                   int d, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return run_backward(fa::kStageDq, q, k, v, nullptr, dout, nullptr, dq, nullptr, nullptr, B, H, N, d, causal, scale,
                      dtype, workspace, workspace_bytes, stream);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, H or N negative, or the problem is too large";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_DTYPE: return "unsupported dtype: use FA_F32 or FA_BF16";
    case FA_ERR_SCALE: return "invalid scale: must be finite and >= 0 (FP8 descale factors: finite and > 0)";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_backward_workspace_size()";
    case FA_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned (workspace: 256-byte)";
    case FA_ERR_MASK:
      return "invalid block mask geometry: mask_heads must be 1 or H, block_q a positive multiple of 32, "
             "block_k a positive multiple of 64, and N at most 65536";
    case FA_ERR_DROPOUT: return "invalid dropout probability: round(256 p) must lie in [0, 255]";
    case FA_ERR_SCRATCH:
      return "fa_backward_noalloc: the problem needs more workspace than the library's built-in "
             "FA_NOALLOC_SCRATCH_BYTES; use fa_backward with a caller-owned workspace";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
