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
//   * K and V stream through LDS in tiles of BC = 64 keys, double-buffered:
//     the global loads of tile j+1 are in flight while tile j is computed;
//   * per tile each wave computes S^T = K_j Q_i^T on the matrix cores, so
//     that each lane holds 32 scores of ONE query: the row max needs only an
//     in-lane reduction and one exchange with the partner lane l^32
//     (v_permlane32_swap), and the rescale of O by exp(m_old - m_new) is one
//     per-lane scalar;
//   * the online-softmax update ("FlashAttention in NeurIPS 2022" section 2.1;
//     "Как работает FlashAttention математически" sections 3-4) keeps O
//     un-normalised and divides by l once at the end;
//   * the probabilities, rounded to the input type, are already in the B-operand
//     layout of the second product O^T += V_j^T P^T, so they never leave
//     registers; V^T fragments are read from the row-major V tile with the
//     gfx950 LDS transpose read (ds_read_b64_tr_b16);
//   * causal: tiles entirely above the diagonal are skipped, the diagonal
//     tiles are masked (key > query -> -inf); ragged tails are masked the
//     same way.  Query tiles are launched longest-first.
//   * exponentials are exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdQW = 32;                      // query rows per wave
constexpr int kFwdBR = kFwdWaves * kFwdQW;      // query rows per workgroup
constexpr int kFwdBC = 64;                      // keys per K/V tile
constexpr int kFwdThreads = kFwdWaves * 64;

template <typename T, int D>
struct FwdSmem {
  static constexpr int ESZ = sizeof(T);
  static constexpr int KLD = D + 16 / ESZ;                           // K row stride (elements)
  static constexpr int VLD = D + (ESZ == 2 ? 64 : 16) / ESZ;         // V row stride (elements)
  static constexpr int KTILE = kFwdBC * KLD;
  static constexpr int VTILE = kFwdBC * VLD;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int BYTES = 2 * STAGE * ESZ;
  static constexpr int VE = 16 / ESZ;                                // elements per 16-byte chunk
  static constexpr int CPR = D / VE;                                 // chunks per row
  static constexpr int NCH = kFwdBC * CPR / kFwdThreads;             // chunks per thread per tensor
  static_assert(kFwdBC * CPR % kFwdThreads == 0, "tile must split evenly over threads");
};

// V^T fragment for bf16 PV: lane l (d row = db*32 + l%32, group g) needs the 8
// keys kb*32 + 16t + 8a + 4g + b (a in {0,1}, b in 0..3).  Two transpose
// reads of 4 keys x 16 d each deliver exactly that.
__device__ __forceinline__ bf16x8 load_vt_frag(const bf16* vs, int vld, int key0, int dcol0, int lane) {
  const int j = lane & 15;
  const int h = (lane >> 4) & 1;
  const int g = lane >> 5;
  const int col = dcol0 + 16 * h + 4 * (j & 3);
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const bf16* p0 = vs + (key0 + 4 * g + (j >> 2)) * vld + col;
  const bf16* p1 = p0 + 8 * vld;
  s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  union { s16x4 s[2]; bf16x8 b; } u;
  u.s[0] = r0;
  u.s[1] = r1;
  return u.b;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, sizeof(T) == 2 ? 2 : 1)
void fa_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                   T* __restrict__ O, float* __restrict__ LSE, int N, int BH, int n_qtiles,
                   float scale, float scale_log2) {
  using M = Mfma<T>;
  using L = FwdSmem<T, D>;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NKB = kFwdBC / 32;   // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;        // 32-wide d sub-blocks of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // Longest-first for causal: the last query tiles see the most keys.
  const int bh = blockIdx.x % BH;
  int qt = blockIdx.x / BH;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int q0 = qt * kFwdBR;
  const size_t head = (size_t)bh * N * D;
  const T* Qh = Q + head;
  const T* Kh = K + head;
  const T* Vh = V + head;

  const int qw0 = q0 + w * kFwdQW;
  const int myq = qw0 + r32;

  // Q^T as the B operand of S^T = K Q^T: column = query, KPL d-values of group g.
  typename M::Frag qf[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c)
    qf[c] = (myq < N) ? M::load(Qh + (size_t)myq * D + c * KC + g * KPL) : M::zero();

  const int kv_end = CAUSAL ? min(N, q0 + kFwdBR) : N;
  const int ntiles = (kv_end + kFwdBC - 1) / kFwdBC;

  uint4 kreg[L::NCH], vreg[L::NCH];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int r = 0; r < L::NCH; ++r) {
      const int c = tid + r * kFwdThreads;
      const int row = c / L::CPR;
      const int col = (c % L::CPR) * L::VE;
      const int key = kv0 + row;
      if (key < N) {
        kreg[r] = *reinterpret_cast<const uint4*>(Kh + (size_t)key * D + col);
        vreg[r] = *reinterpret_cast<const uint4*>(Vh + (size_t)key * D + col);
      } else {
        kreg[r] = make_uint4(0, 0, 0, 0);
        vreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    T* ks = smem + stage * L::STAGE;
    T* vs = ks + L::KTILE;
#pragma unroll
    for (int r = 0; r < L::NCH; ++r) {
      const int c = tid + r * kFwdThreads;
      const int row = c / L::CPR;
      const int col = (c % L::CPR) * L::VE;
      *reinterpret_cast<uint4*>(ks + row * L::KLD + col) = kreg[r];
      *reinterpret_cast<uint4*>(vs + row * L::VLD + col) = vreg[r];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  using X = ExpDomain<T>;
  const float kfac = X::factor(scale, scale_log2);
  float m_run = kNegInf;   // running max of raw scores q.k (unscaled)
  float m_shift = 0.f;     // m_run * kfac: the shift inside every exponent of l_run
  float l_run = 0.f;       // this lane's share of the running row sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * kFwdBC;
    if (j + 1 < ntiles) load_tile(kv0 + kFwdBC);

    const bool skip = CAUSAL && kv0 > qw0 + kFwdQW - 1;    // tile entirely above the diagonal
    if (!skip) {
      const T* ks = smem + (j & 1) * L::STAGE;
      const T* vs = ks + L::KTILE;

      // S^T (keys x queries) for the NKB 32-key sub-blocks.
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < D / KC; ++c) {
          typename M::Frag a = M::load(ks + (kb * 32 + r32) * L::KLD + c * KC + g * KPL);
          s[kb] = M::mma(a, qf[c], s[kb]);
        }
      }

      const bool masked = (CAUSAL && kv0 + kFwdBC - 1 > qw0) || (kv0 + kFwdBC > N);
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + kb * 32 + acc_row(i, g);
            const bool out = (key >= N) || (CAUSAL && key > myq);
            s[kb][i] = out ? kNegInf : s[kb][i];
          }
      }

      // Online softmax: new running max over this tile's keys of this query.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      // a row that has seen no key keeps weight 0 (never the case for row 0 of
      // the first tile, kept for safety); scale >= 0 so max commutes with it
      const float msub = (m_new == kNegInf) ? 0.f : m_new * kfac;
      const float alpha = (m_run == kNegInf) ? 0.f : X::ex(m_run * kfac - msub);
      m_run = m_new;
      m_shift = msub;

      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = X::ex(__builtin_fmaf(s[kb][i], kfac, -msub));
          if (masked) p = (s[kb][i] == kNegInf) ? 0.f : p;
          s[kb][i] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

      // O^T += V^T P^T, with P^T straight from the registers of S^T.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int t = 0; t < 32 / KC; ++t) {
          typename M::Frag pb = M::pack(s[kb], t);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            typename M::Frag va;
            if constexpr (sizeof(T) == 2) {
              va = load_vt_frag(reinterpret_cast<const bf16*>(vs), L::VLD, kb * 32 + 16 * t, db * 32, lane);
            } else {
              // fp32: one key per lane, key = acc_row(t, g) of this sub-block
              va = vs[(kb * 32 + acc_row(t, g)) * L::VLD + db * 32 + r32];
            }
            oacc[db] = M::mma(va, pb, oacc[db]);
          }
        }
      }
    }

    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l (deferred normalisation), lse = m*scale + ln l.
  const float l_tot = pair_sum(l_run);
  if (myq < N) {
    const float inv = 1.f / l_tot;
    T* orow = O + head + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = db * 32 + 8 * a + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int b = 0; b < 4; ++b) v4[b] = (bf16)(oacc[db][4 * a + b] * inv);
          *reinterpret_cast<bf16x4*>(orow + d0) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int b = 0; b < 4; ++b) v4[b] = oacc[db][4 * a + b] * inv;
          *reinterpret_cast<f32x4*>(orow + d0) = v4;
        }
      }
    // lse = ln(sum_j exp(scale*s_j)) = shift (converted to base e) + ln(l)
    const float shift = (sizeof(T) == 2) ? m_run * scale : m_shift;
    if (g == 0) LSE[(size_t)bh * N + myq] = shift + logf(l_tot);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using L = FwdSmem<T, D>;
  auto kern = fa_fwd_kernel<T, D, CAUSAL>;
  // raise the dynamic-LDS limit once per instantiation (thread-safe static init)
  static const hipError_t attr_err =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
  if (attr_err != hipSuccess) return attr_err;
  const int BH = a.B * a.H;
  const int n_qtiles = (a.N + kFwdBR - 1) / kFwdBR;
  const dim3 grid(n_qtiles * BH), block(kFwdThreads);
  hipLaunchKernelGGL(kern, grid, block, L::BYTES, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.o),
                     a.lse, a.N, BH, n_qtiles, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
  const bool c = a.causal != 0;
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) return c ? launch_fwd_t<bf16, 64, true>(a, stream) : launch_fwd_t<bf16, 64, false>(a, stream);
    return c ? launch_fwd_t<bf16, 128, true>(a, stream) : launch_fwd_t<bf16, 128, false>(a, stream);
  }
  if (a.d == 64) return c ? launch_fwd_t<float, 64, true>(a, stream) : launch_fwd_t<float, 64, false>(a, stream);
  return c ? launch_fwd_t<float, 128, true>(a, stream) : launch_fwd_t<float, 128, false>(a, stream);
}

}  // namespace fa
