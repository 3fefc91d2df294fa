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
// head are cut into S chunks of 32-key tiles; one single-wave workgroup per
// (head, chunk) streams its K/V tiles through LDS (double-buffered),
// computes S^T = K Q^T on the matrix cores with the query tile padded to 32
// columns, and runs the online softmax of the forward kernel.  Each chunk's
// partial result -- O_s normalised over the chunk, and lse_s -- goes to the
// workspace, and a second kernel merges the partials of each row with the
// rule for concatenated key blocks ("Overview of Flash Attention series",
// Tiling): lse = ln sum_s e^(lse_s), O = sum_s e^(lse_s - lse) O_s.  A chunk
// in which a query sees no key contributes lse_s = -inf (weight 0).  With
// S = 1 the single chunk writes O and lse directly.
//
// Merging inside the partial kernel (the last chunk of a head to finish
// merges) measured slower: the device-scope release each workgroup needs
// writes back its L2, and the counters need clearing by a kernel anyway.
//
// The path is bound by HBM: K and V are read once, everything else is
// small.  Their copies carry the non-temporal hint: for a long read-once
// stream that measured about 15% more bandwidth than default caching.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecBC = 32;   // keys per tile
constexpr bool kDecInterleave = true;   // chunk s takes tiles s, s + S, ... (else consecutive tiles)

// K/V stages per wave: a wave keeps NST - 1 tiles in flight while it
// computes on one.  Two stages measured fastest on the long-cache shapes:
// with about two workgroups per CU the HBM stream, not the wave, sets the
// pace, and deeper rings (3 or 4 stages) only cost LDS.
template <typename T, int D>
struct DecSmem {
  static constexpr int NST = 2;
  static constexpr int TILE = kDecBC * D * (int)sizeof(T);
  static constexpr int BYTES = 2 * NST * TILE;   // [K stages][V stages]
  static constexpr int PER = 2 * TILE / 1024;    // copy instructions per K+V tile
  static_assert((NST - 2) * PER <= 63, "vmcnt is 6 bits");
};

template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Merge the S partial results of one (head, query row) with one wave: lanes
// read the S partial lse values in parallel (wave reductions give their max
// and the normaliser); each lane then accumulates its D/64 output elements
// over the chunks, with the chunk weights broadcast from the lane that holds
// them.  Partials live at row (bh * S + s) * Nq + i.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename T, int D>
__device__ __forceinline__ void merge_row(const float* Opart, const float* Lpart, T* O, float* LSE, int bh, int i,
                                          int Nq, int S, int lane) {
  constexpr int EPL = D / 64;                 // output elements per lane
  const float* lp = Lpart + (size_t)bh * S * Nq + i;                      // chunk s at lp[s * Nq]
  const float* op = Opart + ((size_t)bh * S * Nq + i) * D + lane * EPL;   // chunk s at op[s * Nq * D]
  const size_t ostride = (size_t)Nq * D;

  float m = kNegInf;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lp[(size_t)s * Nq]);
  m = wave_max(m);

  float tot = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const float ls = s < S ? lp[(size_t)s * Nq] : kNegInf;
    const float w = (ls == kNegInf) ? 0.f : expf(ls - m);   // a chunk with no visible key weighs 0
    tot += w;
    const int n = min(64, S - s0);
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
      const float* src = op + (size_t)(s0 + j) * ostride;
      if constexpr (EPL == 2) {
        const float2 o2 = *reinterpret_cast<const float2*>(src);
        acc[0] += wj * o2.x;
        acc[1] += wj * o2.y;
      } else {
        acc[0] += wj * src[0];
      }
    }
  }
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;   // tot = 0 only if no chunk saw a key
  const size_t row = (size_t)bh * Nq + i;
  T* out = O + row * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = (T)(acc[e] * inv);
  if (lane == 0) LSE[row] = tot > 0.f ? m + logf(tot) : kNegInf;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64)
void fa_decode_partial_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                              T* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart,
                              float* __restrict__ Lpart, int Nq, int Nk, int S, float scale) {
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

  // keys of this chunk: the 32-key tiles split, split + S, split + 2S, ...
  // (any partition of the keys merges to the same result).  The S
  // workgroups of a head then read neighbouring tiles at any moment, which
  // measured a little faster (about 2%) than consecutive chunks.
  const int ntiles_all = (Nk + kDecBC - 1) / kDecBC;
  const int n_my = kDecInterleave ? (split < ntiles_all ? (ntiles_all - split + S - 1) / S : 0)
                                  : (int)((long long)(split + 1) * ntiles_all / S) -
                                        (int)((long long)split * ntiles_all / S);
  const int t_first = kDecInterleave ? split : (int)((long long)split * ntiles_all / S);
  const int t_step = kDecInterleave ? S : 1;

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

  constexpr int NST = L::NST;
  auto load = [&](int t, int st) __attribute__((always_inline)) {
    tile_to_lds_async<T, D, kDecBC, 1, true>(rk, smem + st * L::TILE, t * kDecBC, 0, lane);
    tile_to_lds_async<T, D, kDecBC, 1, true>(rv, smem + (NST + st) * L::TILE, t * kDecBC, 0, lane);
  };

#pragma unroll
  for (int j = 0; j < NST - 1; ++j)
    if (j < n_my) load(t_first + j * t_step, j);
  // Take the compiler's wait for the Q loads here, once: left to itself it
  // places that wait at the first use inside the loop, where it runs on
  // every tile and also drains the K/V copies in flight.
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
  int st = 0;                                  // stage of tile t
  int st_next = NST - 1;                       // stage of tile t + NST - 1
  for (int j = 0; j < n_my; ++j) {
    // tile j landed once at most the copies of the NST - 2 tiles issued
    // after it are outstanding (copies complete in issue order; one wave:
    // no barrier)
    if (j + NST - 2 < n_my) wait_vmem_n<(NST - 2) * L::PER>();
    else wait_vmem();
    if (j + NST - 1 < n_my) load(t_first + (j + NST - 1) * t_step, st_next);   // stage read in iteration j - 1
    const lds_u8* ks = smem + st * L::TILE;
    const lds_u8* vs = smem + (NST + st) * L::TILE;
    const int kv0 = (t_first + j * t_step) * kDecBC;

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
    st = st + 1 == NST ? 0 : st + 1;
    st_next = st_next + 1 == NST ? 0 : st_next + 1;
  }

  const float l_tot = pair_sum(l_run);
  const bool no_key = !(l_tot > 0.f);           // no visible key in this chunk: O_s = 0, lse_s = -inf
  const float inv = no_key ? 0.f : 1.f / l_tot;
  const float lse = no_key ? kNegInf : msub * X::kToNat + logf(l_tot);

  if (S == 1) {
    // one chunk per head: its result is the final one
    const rsrc_t ro = make_rsrc(O + (size_t)bh * Nq * D, (uint32_t)Nq * G::R);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = db * 32 + 8 * a + 4 * g;
        store4<T>(ro, r32 * G::R + d0 * (int)sizeof(T), oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                  oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
      }
    const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4u);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, r32 * 4, 0, 0);
    return;
  }

  // Partial result of this chunk: O_s normalised over its keys, and lse_s.
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
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, r32 * 4, 0, 0);

}

// Merge kernel: one wave per (head, query row).
template <typename T, int D>
__global__ __launch_bounds__(64)
void fa_decode_combine_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                              T* __restrict__ O, float* __restrict__ LSE, int Nq, int S) {
  merge_row<T, D>(Opart, Lpart, O, LSE, blockIdx.x / Nq, blockIdx.x % Nq, Nq, S, threadIdx.x);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dec_t(const DecArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((fa_decode_partial_kernel<T, D, CAUSAL>), dim3(BH * a.splits), dim3(64), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<T*>(a.o), a.lse, a.opart, a.lpart, a.Nq, a.Nk, a.splits, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((fa_decode_combine_kernel<T, D>), dim3(BH * a.Nq), dim3(64), 0, stream, a.opart, a.lpart,
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
