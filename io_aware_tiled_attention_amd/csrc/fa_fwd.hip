// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// What is computed (per batch*head, Q,K,V in R^{N x d}):
//   O = softmax(scale * Q K^T) V,   lse_i = ln sum_j exp(scale * q_i . k_j)
// ("Overview of Flash Attention series", Standard Attention / Forward Pass;
// scale as in the "Transformer 入门" definitions), without ever writing the
// N x N matrices S or P to device memory.
//
// How (the tiling of "Overview of Flash Attention series", section Tiling,
// in the Q-outer "V2" loop order of the Transformer primer):
//   * a workgroup owns BR = 128 query rows (4 waves x 32 rows); each wave keeps
//     its 32 rows of Q, the running row max m, the running row sum l and the
//     un-normalised output O^T (d x 32, fp32) in registers for the whole
//     sweep over keys;
//   * K and V stream through LDS in tiles of BC = 64 keys, global -> LDS
//     directly (buffer_load ... lds), two stages deep at d = 128 and three at
//     d = 64 (bf16): while tile j is being consumed, K and V of the next one
//     or two tiles are in flight, and each wave waits with a counted vmcnt
//     for its own copies of tile j+1 only;
//   * per tile each wave computes S^T = K_j Q_i^T on the matrix cores, so
//     that each lane holds 32 scores of ONE query: the row max needs only an
//     in-lane reduction and one exchange with the partner lane l^32
//     (v_permlane32_swap), and the rescale of O by exp(m_old - m_new) is one
//     per-lane scalar;
//   * S of a tile is computed right before its softmax: issuing S of the
//     next tile first cost 32 registers and measured ~2% slower, the other
//     wave on the SIMD providing the overlap of matrix and vector work;
//   * the online-softmax update ("FlashAttention in NeurIPS 2022" section 2.1;
//     "Как работает FlashAttention математически" sections 3-4) keeps O
//     un-normalised and divides by l once at the end; the shift inside the
//     exponentials is the running max, raised only when a new score exceeds it
//     by more than 2^8 (then O and l are rescaled) -- the result is the same,
//     the per-tile rescale of O is skipped;
//   * the probabilities, rounded to the input type, are already in the B-operand
//     layout of the second product O^T += V_j^T P^T, so they never leave
//     registers; V^T fragments are read from the row-major V tile with the
//     gfx950 LDS transpose read (ds_read_b64_tr_b16);
//   * causal: tiles entirely above a wave's diagonal are skipped, diagonal and
//     ragged-tail tiles are masked (key > query or key >= N -> -inf).  Query
//     tiles are launched longest-first within XCD-aware head groups
//     (wg_order).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdQW = 32;                      // query rows per wave
constexpr int kFwdBR = kFwdWaves * kFwdQW;      // query rows per workgroup
constexpr int kFwdBC = 64;                      // keys per K/V tile
constexpr int kFwdThreads = kFwdWaves * 64;
// Block-sparse: the key tiles a workgroup visits are listed in LDS (TileList,
// N <= 64 * kListMax = 65536), with one bit per wave.

// K/V stages: NST - 1 tiles are in flight while one is consumed.  bf16 at
// d = 64 takes three: a tile then carries half the matrix work of d = 128,
// too little to cover the latency of the next tile's copy with one tile of
// prefetch, and three 16 KiB stages still leave room for three workgroups
// per CU.  d = 128 keeps two (64 KiB, two workgroups per CU).
template <typename T, int D>
constexpr int fwd_stages() { return (sizeof(T) == 2 && D == 64) ? 3 : 2; }

template <typename T, int D>
struct FwdSmem {
  static constexpr int NST = fwd_stages<T, D>();
  static constexpr int TILE = kFwdBC * D * (int)sizeof(T);   // bytes of one K or V tile
  // [K stages][V stages]
  static constexpr int BYTES = 2 * NST * TILE;
  // copy instructions each wave issues per K+V tile (1 KiB each)
  static constexpr int PER = 2 * (TILE / 1024) / kFwdWaves;
  static_assert((NST - 2) * PER <= 63, "vmcnt is 6 bits");
  __device__ static lds_u8* k(lds_u8* base, int st) { return base + st * TILE; }
  __device__ static lds_u8* v(lds_u8* base, int st) { return base + (NST + st) * TILE; }
};

template <int N>
__device__ __forceinline__ void fwd_wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// SPARSE: block-sparse attention ("Overview of Flash Attention series",
// Block-sparse Flashattention).  mask[mh][qb][kb] != 0 keeps the block of
// block_q query rows by block_k keys (mh = head if mask_heads > 1, else 0);
// key tiles whose block is zero for every wave of the workgroup are neither
// loaded nor computed, and a wave skips a loaded tile whose block is zero
// for its own rows -- the causal tile skip generalised to a block mask.
// block_q is a multiple of 32 (one mask row per wave) and block_k a multiple
// of 64 (one mask column per tile), so no tile is partly masked by the block
// mask.  A row that keeps no key gets O = 0 and lse = -inf.
//
// DROP: dropout on the probabilities ("Как работает FlashAttention
// математически", section 5; the mask is regenerated, not stored): after
// the row sum l has taken the undropped P, each entry of a dropped (query,
// key) pair is zeroed before P V, and O is scaled by 1 / (1 - t/256) in the
// epilogue; lse is that of the undropped scores.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kFwdThreads, sizeof(T) == 2 ? 2 : 1)
void fa_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                   T* __restrict__ O, float* __restrict__ LSE, int N, int BH, int n_qtiles, int group, float scale,
                   const unsigned char* __restrict__ mask, int H, int mask_heads, int block_q, int block_k,
                   DropParams dp) {
  using M = Mfma<T>;
  using L = FwdSmem<T, D>;
  using G = Tile<T, D>;
  using X = ExpDomain<T>;
  using Frag = typename M::Frag;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NKB = kFwdBC / 32;   // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;        // 32-wide d sub-blocks of O^T
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // Launch order: heads grouped per XCD, and longest-first for causal (rank
  // 0 = the last query tile, which sees the most keys).
  const WgOrder wo = wg_order(blockIdx.x, BH, n_qtiles, group);
  const int bh = wo.bh;
  const int qt = CAUSAL ? n_qtiles - 1 - wo.rank : wo.rank;
  const int q0 = qt * kFwdBR;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  // K/V tiles are copied with tile_to_lds_async; each wave waits for its
  // own copies (counted vmcnt) before the barrier that publishes a tile
  const u32x4 rk = rsrc_words(K + head, head_bytes);
  const u32x4 rv = rsrc_words(V + head, head_bytes);

  const int qw0 = q0 + w * kFwdQW;
  const int myq = qw0 + r32;
  const float kfac = X::factor(scale);
  if constexpr (!DROP) (void)dp;

  // Q^T as the B operand of S^T = K Q^T: column = query, KPL d-values of group g.
  Frag qf[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c) qf[c] = M::load(rq, (uint32_t)myq * G::R + (c * KC + g * KPL) * (int)sizeof(T));

  const int kv_end = CAUSAL ? min(N, q0 + kFwdBR) : N;
  const int ntiles = (kv_end + kFwdBC - 1) / kFwdBC;
  // last tile this wave needs (causal: keys up to its largest query)
  const int wave_last = CAUSAL ? min(ntiles - 1, (qw0 + kFwdQW - 1) / kFwdBC) : ntiles - 1;

  auto compute_st = [&](f32x16 (&s)[NKB], const lds_u8* ks) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / KC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = M::mma(M::lds(ks + G::off(kb * 32 + r32, c * KC + g * KPL)), qf[c], s[kb]);
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float msub = kNegInf;    // exponent shift (running max of scaled scores, raised lazily)
  float l_run = 0.f;       // this lane's share of the running row sum, relative to msub

  // The tiles this workgroup visits, in order: every tile up to kv_end
  // (dense), or the listed ones (block-sparse).  tile_of(i) is the i-th
  // visited tile, active(i) whether this wave computes it.
  const TileList tl = tile_list_at(smem + L::BYTES);
  int n_act = ntiles;
  if constexpr (SPARSE) {
    const int tk_n = (N + block_k - 1) / block_k;
    const int tq_n = (N + block_q - 1) / block_q;
    const unsigned char* mrow = mask_of_head(mask, bh, H, mask_heads, tq_n, tk_n);
    n_act = build_tile_list<kFwdWaves>(
        ntiles,
        [&](int j) -> unsigned {
          const int kb = j * kFwdBC / block_k;
          unsigned bits = 0;
#pragma unroll
          for (int w2 = 0; w2 < kFwdWaves; ++w2) {
            const int qw = q0 + w2 * kFwdQW;
            const bool reach = qw < N && !(CAUSAL && j * kFwdBC > qw + kFwdQW - 1);
            if (reach && mrow[(qw / block_q) * tk_n + kb] != 0) bits |= 1u << w2;
          }
          return bits;
        },
        tl, tid, w, lane);
  } else {
    (void)mask;
    (void)H;
    (void)mask_heads;
    (void)block_q;
    (void)block_k;
  }
  auto tile_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl.act[i]);
    else return i;
  };
  auto active = [&](int i) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane((int)tl.wbit[i]) >> w) & 1;
    else return i <= wave_last;
  };

  constexpr int NST = L::NST;
  auto load = [&](int i, int st) {
    tile_to_lds_async<T, D, kFwdBC, kFwdWaves>(rk, L::k(smem, st), tile_of(i) * kFwdBC, w, lane);
    tile_to_lds_async<T, D, kFwdBC, kFwdWaves>(rv, L::v(smem, st), tile_of(i) * kFwdBC, w, lane);
  };
  // Tile `it` has landed once at most the copies of the tiles issued after
  // it, up to NST - 2 of them, are outstanding (copies complete in issue
  // order).
  auto wait_tile = [&](int it) {
    if constexpr (NST > 2) {
      if (it + NST - 2 < n_act) {
        fwd_wait_vmem_n<(NST - 2) * L::PER>();
        return;
      }
    }
    wait_vmem();
  };

  // Prologue: the first NST - 1 visited tiles in flight, the first landed.
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < n_act) load(i, i);
  // Take the compiler's wait for the Q loads here, once: at their first use
  // inside the loop it would also drain the K/V copies in flight.
#pragma unroll
  for (int c = 0; c < D / KC; ++c) asm volatile("" : "+v"(qf[c]));
  f32x16 s_cur[NKB];
  if (n_act > 0) {
    wait_tile(0);
    __syncthreads();
  }

  int st = 0;                 // stage of tile it
  int st_next = NST - 1;      // stage of tile it + NST - 1 (read in iteration it - 1)
  for (int it = 0; it < n_act; ++it) {
    const int j = tile_of(it);
    const int kv0 = j * kFwdBC;
    if (it + NST - 1 < n_act) load(it + NST - 1, st_next);

    if (active(it)) {
      compute_st(s_cur, L::k(smem, st));
      const bool masked = (CAUSAL && kv0 + kFwdBC - 1 > qw0) || (kv0 + kFwdBC > N);
      if (masked) {
        // keys allowed for this lane: key <= min(N-1, myq) (causal) or key <= N-1
        const int last = CAUSAL ? min(N - 1, myq) : N - 1;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int lim = last - (kv0 + kb * 32 + 4 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            s_cur[kb][i] = (acc_row(i, 0) > lim) ? kNegInf : s_cur[kb][i];
        }
      }
      // Online softmax: running max over this tile's keys of this query.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
      mx = pair_max(mx);
      const float cand = mx * kfac;                 // kfac > 0: max commutes with the scaling
      const bool need = cand > msub + X::kLazy;     // false while both are -inf
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
      // a lane with no unmasked key yet keeps weight 0 for its -inf scores
      const float shift = (msub == kNegInf) ? 0.f : msub;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = X::ex(__builtin_fmaf(s_cur[kb][i], kfac, -shift));
          s_cur[kb][i] = p;
          psum += p;
        }
      l_run += psum;
      if constexpr (DROP) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 rb = drop_bytes_keys(dp.k0, dp.k1, dp.offset, (unsigned)bh, myq, kv0 + kb * 32, g, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) s_cur[kb][i] = drop_keep(rb, i, dp.t) ? s_cur[kb][i] : 0.f;
        }
      }

      // O^T += V^T P^T, with P^T straight from the registers of S^T.
      const lds_u8* vs = L::v(smem, st);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 32 / KC; ++t) {
          const Frag pb = M::pack(s_cur[kb], t);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            Frag va;
            if constexpr (sizeof(T) == 2) {
              va = lds_tr_frag<D>(vs, kb * 32 + 16 * t, db * 32, lane);
            } else {
              // fp32: one key per lane, key = acc_row(t, g) of this sub-block
              va = M::lds(vs + G::off(kb * 32 + acc_row(t, g), db * 32 + r32));
            }
            oacc[db] = M::mma(va, pb, oacc[db]);
          }
        }
    }

    if (it + 1 < n_act) wait_tile(it + 1);
    __syncthreads();
    st = st + 1 == NST ? 0 : st + 1;
    st_next = st_next + 1 == NST ? 0 : st_next + 1;
  }

  // Epilogue: O = O_acc / l (deferred normalisation), lse = shift + ln l;
  // a row that kept no key (block-sparse) gets O = 0 and lse = -inf.
  const float l_tot = pair_sum(l_run);
  const bool no_key = !(l_tot > 0.f);
  const float inv = no_key ? 0.f : (DROP ? dp.rs : 1.f) / l_tot;
  const rsrc_t ro = make_rsrc(O + head, head_bytes);
  if constexpr (sizeof(T) == 2 && D == 128) {
    // Every wave has passed the loop's last barrier and no copy is in
    // flight, so the K/V ring is idle: each wave stages its rows in a slice.
    // (At d = 64 the round trip through LDS lengthens the epilogue of a
    // workgroup whose LDS limits residency, and the direct stores measured
    // faster.)
    static_assert(kFwdWaves * kFwdQW * G::R <= L::BYTES, "O staging must fit in the K/V ring");
    store_rows_bf16<D>(smem + w * (kFwdQW * G::R), oacc, inv, ro, qw0, lane);
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = db * 32 + 8 * a + 4 * g;
        store4<T>(ro, (uint32_t)myq * G::R + d0 * (int)sizeof(T), oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                  oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
      }
  }
  // both lanes of a query pair write the same value
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const float lse = no_key ? kNegInf : msub * X::kToNat + logf(l_tot);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, myq * 4, 0, 0);
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using L = FwdSmem<T, D>;
  constexpr int bytes = L::BYTES + (SPARSE ? kListBytes : 0);
  auto kern = fa_fwd_kernel<T, D, CAUSAL, SPARSE, DROP>;
  // raise the dynamic-LDS limit once per instantiation (thread-safe static init)
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (attr_err != hipSuccess) return attr_err;
  const int BH = a.B * a.H;
  const int n_qtiles = (a.N + kFwdBR - 1) / kFwdBR;
  const dim3 grid(n_qtiles * BH), block(kFwdThreads);
  // resident workgroups per XCD: 32 CUs x (bf16: 2 at d = 128, 3 at d = 64; fp32: 1)
  const int group = wg_group(n_qtiles, 32 * (sizeof(T) == 2 ? (D == 64 ? 3 : 2) : 1));
  hipLaunchKernelGGL(kern, grid, block, bytes, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.o),
                     a.lse, a.N, BH, n_qtiles, group, a.scale, a.mask, a.H, a.mask_heads, a.block_q, a.block_k, a.drop);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_m(const FwdArgs& a, hipStream_t stream) {
  if (a.mask) return launch_fwd_t<T, D, CAUSAL, true, false>(a, stream);
  if (a.drop.on) return launch_fwd_t<T, D, CAUSAL, false, true>(a, stream);
  return launch_fwd_t<T, D, CAUSAL, false, false>(a, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) return c ? launch_fwd_m<bf16, 64, true>(a, stream) : launch_fwd_m<bf16, 64, false>(a, stream);
    return c ? launch_fwd_m<bf16, 128, true>(a, stream) : launch_fwd_m<bf16, 128, false>(a, stream);
  }
  if (a.d == 64) return c ? launch_fwd_m<float, 64, true>(a, stream) : launch_fwd_m<float, 64, false>(a, stream);
  return c ? launch_fwd_m<float, 128, true>(a, stream) : launch_fwd_m<float, 128, false>(a, stream);
}

}  // namespace fa
