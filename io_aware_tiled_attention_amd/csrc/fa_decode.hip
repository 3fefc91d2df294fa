// fa_decode.hip -- split-KV decoding for gfx950 (MI355X).
//
// What is computed (per batch*head): Nq <= 32 new query rows attend to Nk
// cached keys and values,
//   O = softmax(scale * Q K^T) V,   lse_i = ln sum_j exp(scale * q_i . k_j),
// where the queries are the last Nq positions of the sequence: with the
// causal mask query i sees keys 0 .. Nk - Nq + i ("Как работает
// FlashAttention математически", section 9: FlashDecoding, K and V cached and
// Q the new token(s)).
//
// How: with a handful of query rows there is one matrix-core tile of queries
// per head, so the parallelism has to come from the keys.  The Nk keys of a
// head are cut into S consecutive chunks; one single-wave workgroup per
// (head, chunk) streams its K/V tiles of 32 keys through LDS (two stages,
// 32 KiB for bf16 d=128, so several workgroups share a CU and keep enough
// bytes in flight), computes S^T = K Q^T on the matrix cores with the query
// tile padded to 32 columns, runs the online softmax of the forward kernel
// and writes its partial result -- O_s normalised over the chunk and lse_s --
// to the workspace.  A second kernel merges the S partials of each row with
// the rule for concatenated key blocks ("Overview of Flash Attention
// series", Tiling): lse = ln sum_s e^(lse_s), O = sum_s e^(lse_s - lse) O_s.
// A chunk in which a query sees no key contributes lse_s = -inf (weight 0).
//
// The path is bound by HBM: K and V are read once, everything else is small.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecBC = 32;   // keys per tile
constexpr int kDecQ = 32;    // query columns of the matrix-core tile (Nq <= 32)

template <typename T, int D>
struct DecSmem {
  static constexpr int TILE = kDecBC * D * (int)sizeof(T);
  static constexpr int BYTES = 4 * TILE;   // [K st0][K st1][V st0][V st1]
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64)
void fa_decode_partial_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                              float* __restrict__ Opart, float* __restrict__ Lpart, int Nq, int Nk, int S,
                              float scale) {
  using M = Mfma<T>;
  using G = Tile<T, D>;
  using X = ExpDomain<T>;
  using L = DecSmem<T, D>;
  using Frag = typename M::Frag;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NDB = D / 32;
  constexpr int NC = D / KC;
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[L::BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int lane = threadIdx.x;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const int split = blockIdx.x % S;
  const int bh = blockIdx.x / S;

  // keys of this chunk: tiles [t0, t1) of the Nk keys
  const int ntiles_all = (Nk + kDecBC - 1) / kDecBC;
  const int t0 = (int)((long long)split * ntiles_all / S);
  const int t1 = (int)((long long)(split + 1) * ntiles_all / S);

  const size_t qhead = (size_t)bh * Nq * D;
  const size_t khead = (size_t)bh * Nk * D;
  const rsrc_t rq = make_rsrc(Q + qhead, (uint32_t)Nq * G::R);
  const u32x4 rk = rsrc_words(K + khead, (uint32_t)Nk * G::R);
  const u32x4 rv = rsrc_words(V + khead, (uint32_t)Nk * G::R);
  const float kfac = X::factor(scale);

  // Q^T as the B operand: column = query r32 (rows past Nq read as zero).
  Frag qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = M::load(rq, r32 * G::R + (c * KC + g * KPL) * (int)sizeof(T));

  // keys this lane's query may see: key <= last
  const int last = CAUSAL ? min(Nk - 1, Nk - Nq + r32) : Nk - 1;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float msub = kNegInf;
  float l_run = 0.f;

  auto load = [&](int t, int st) {
    tile_to_lds_async<T, D, kDecBC, 1>(rk, smem + st * L::TILE, t * kDecBC, 0, lane);
    tile_to_lds_async<T, D, kDecBC, 1>(rv, smem + (2 + st) * L::TILE, t * kDecBC, 0, lane);
  };

  if (t0 < t1) load(t0, 0);
  for (int t = t0; t < t1; ++t) {
    const int st = (t - t0) & 1;
    wait_vmem();                               // tile t landed (one wave: no barrier)
    if (t + 1 < t1) load(t + 1, st ^ 1);       // its stage was read in iteration t - 1
    const lds_u8* ks = smem + st * L::TILE;
    const lds_u8* vs = smem + (2 + st) * L::TILE;
    const int kv0 = t * kDecBC;

    // S^T = K Q^T: rows = the tile's 32 keys, column = this lane's query.
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = M::mma(M::lds(ks + G::off(r32, c * KC + g * KPL)), qf[c], s);
    if (kv0 + kDecBC - 1 > (CAUSAL ? Nk - Nq : Nk - 1)) {
      const int lim = last - (kv0 + 4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (acc_row(i, 0) > lim) ? kNegInf : s[i];
    }
    // online softmax (lazy shift, as in the forward kernel)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = pair_max(mx);
    const float cand = mx * kfac;
    const bool need = cand > msub + X::kLazy;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float newm = need ? cand : msub;
      const float alpha = (msub == kNegInf) ? 0.f : X::ex(msub - newm);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      msub = newm;
    }
    const float shift = (msub == kNegInf) ? 0.f : msub;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = X::ex(__builtin_fmaf(s[i], kfac, -shift));
      s[i] = p;
      psum += p;
    }
    l_run += psum;
    // O^T += V^T P^T
#pragma unroll
    for (int tt = 0; tt < 32 / KC; ++tt) {
      const Frag pb = M::pack(s, tt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        Frag va;
        if constexpr (sizeof(T) == 2) va = lds_tr_frag<D>(vs, 16 * tt, db * 32, lane);
        else va = M::lds(vs + G::off(acc_row(tt, g), db * 32 + r32));
        oacc[db] = M::mma(va, pb, oacc[db]);
      }
    }
  }

  // Partial result of this chunk: O_s normalised over its keys, lse_s; a
  // query with no visible key here gets O_s = 0, lse_s = -inf.
  const float l_tot = pair_sum(l_run);
  const bool no_key = !(l_tot > 0.f);
  const float inv = no_key ? 0.f : 1.f / l_tot;
  const size_t prow = ((size_t)bh * S + split) * Nq;   // first row of this chunk's partials
  const rsrc_t ro = make_rsrc(Opart + prow * D, (uint32_t)Nq * D * 4u);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = db * 32 + 8 * a + 4 * g;
      store4<float>(ro, (r32 * D + d0) * 4, oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                    oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
    }
  const rsrc_t rl = make_rsrc(Lpart + prow, (uint32_t)Nq * 4u);
  const float lse = no_key ? kNegInf : msub * X::kToNat + logf(l_tot);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, r32 * 4, 0, 0);
}

// Merge the S partials of each (head, query row): one workgroup of D/4
// threads per row, each thread owning 4 consecutive output elements.
template <typename T, int D>
__global__ __launch_bounds__(D / 4)
void fa_decode_combine_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                              T* __restrict__ O, float* __restrict__ LSE, int Nq, int S) {
  const int row = blockIdx.x;                 // bh * Nq + i
  const int bh = row / Nq, i = row % Nq;
  const int e = threadIdx.x * 4;
  float m = kNegInf;
  for (int s = 0; s < S; ++s) m = fmaxf(m, Lpart[((size_t)bh * S + s) * Nq + i]);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const size_t prow = ((size_t)bh * S + s) * Nq + i;
    const float ls = Lpart[prow];
    const float wgt = (ls == kNegInf) ? 0.f : expf(ls - m);
    tot += wgt;
    const f32x4 o = *reinterpret_cast<const f32x4*>(Opart + prow * D + e);
    acc += wgt * o;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;   // tot = 0 only if no chunk saw a key
  T* out = O + (size_t)row * D + e;
  out[0] = (T)(acc[0] * inv);
  out[1] = (T)(acc[1] * inv);
  out[2] = (T)(acc[2] * inv);
  out[3] = (T)(acc[3] * inv);
  if (threadIdx.x == 0) LSE[row] = tot > 0.f ? m + logf(tot) : kNegInf;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dec_t(const DecArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((fa_decode_partial_kernel<T, D, CAUSAL>), dim3(BH * a.splits), dim3(64), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.opart,
                     a.lpart, a.Nq, a.Nk, a.splits, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_decode_combine_kernel<T, D>), dim3(BH * a.Nq), dim3(D / 4), 0, stream, a.opart, a.lpart,
                     static_cast<T*>(a.o), a.lse, a.Nq, a.splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) return c ? launch_dec_t<bf16, 64, true>(a, stream) : launch_dec_t<bf16, 64, false>(a, stream);
    return c ? launch_dec_t<bf16, 128, true>(a, stream) : launch_dec_t<bf16, 128, false>(a, stream);
  }
  if (a.d == 64) return c ? launch_dec_t<float, 64, true>(a, stream) : launch_dec_t<float, 64, false>(a, stream);
  return c ? launch_dec_t<float, 128, true>(a, stream) : launch_dec_t<float, 128, false>(a, stream);
}

}  // namespace fa
