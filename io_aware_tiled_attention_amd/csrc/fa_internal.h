// fa_internal.h -- argument bundles and launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// Dropout on the attention probabilities, its mask regenerated from a
// counter-based generator (Philox4x32-10 keyed by the seed).
struct DropParams {
  unsigned k0 = 0, k1 = 0;   // seed, low and high word
  unsigned offset = 0;       // fourth counter word
  unsigned t = 0;            // an element is dropped when its random byte is < t (probability t / 256)
  float rs = 1.f;            // 1 / (1 - t / 256)
  bool on = false;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d, causal, dtype;
  float scale;
  // block-sparse forward only (mask == nullptr: dense)
  const unsigned char* mask = nullptr;
  int mask_heads = 0, block_q = 0, block_k = 0;
  DropParams drop{};
};

constexpr int kSparseMaxN = 65536;   // N limit of block-sparse attention (tile lists in LDS)

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d, causal, dtype;
  float scale;
  float* dsum;     // [B*H*N]   D_i = do_i . o_i          (workspace)
  float* nlse;     // [B*H*N]   -lse_i, exponent domain   (workspace)
  DropParams drop{};
  // block-sparse backward only (mask == nullptr: dense)
  const unsigned char* mask = nullptr;
  int mask_heads = 0, block_q = 0, block_k = 0;
};

// Forward with OCP E4M3 inputs (one byte per element) and bf16 output.
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;          // bf16 [B, H, N, d]
  float* lse;
  int B, H, N, d, causal;
  float scale, q_descale, k_descale, v_descale;
};

struct DecArgs {
  const void* q;     // [B, H, Nq, d]
  const void* k;     // [B, H, Nk, d]
  const void* v;
  void* o;           // [B, H, Nq, d]
  float* lse;        // [B, H, Nq]
  int B, H, Nq, Nk, d, causal, dtype, splits;
  float scale;
  float* opart;      // [B*H][splits][Nq][d]   partial outputs  (workspace; splits > 1)
  float* lpart;      // [B*H][splits][Nq]      partial lse      (workspace; splits > 1)
};

constexpr int kDecodeMaxNq = 32;      // query rows per decode call (one matrix-core tile)
constexpr int kDecodeTile = 32;       // keys per decode tile

// Number of key chunks of a decode call: `requested` if positive, else about
// 512 (head, chunk) workgroups -- two per CU, where the measured read rate
// of the long-cache shapes peaks (more concurrent streams read HBM more
// slowly) -- with at least 8 tiles (256 keys) per chunk; never more chunks
// than tiles.
inline int decode_splits(int B, int H, int Nk, int requested) {
  const long long tiles = ((long long)Nk + kDecodeTile - 1) / kDecodeTile;
  long long s = requested;
  if (s <= 0) {
    const long long bh = (long long)B * H;
    s = (512 + bh - 1) / bh;
    const long long cap = tiles / 8 > 1 ? tiles / 8 : 1;
    if (s > cap) s = cap;
  }
  if (s > tiles) s = tiles;
  return s < 1 ? 1 : (int)s;
}

// Workspace carve-up shared by fa_backward_workspace_size and fa_backward.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_dsum_bytes(size_t rows) { return align256(rows * sizeof(float)); }
inline size_t ws_bytes(size_t rows) { return 2 * ws_dsum_bytes(rows); }

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecArgs& a, hipStream_t stream);
hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream);
// backward stages (bit mask): D, dK/dV, dQ, run in that order.  All three
// (7) in bf16 run dQ first, with D folded into it, then dK/dV.
constexpr int kStagePre = 1, kStageDkDv = 2, kStageDq = 4;
hipError_t launch_backward(const BwdArgs& a, int stages, hipStream_t stream);

}  // namespace fa
