// fa_bwd.hip -- exact attention backward for gfx950 (MI355X), with recomputation.
//
// What is computed (per batch*head; "Overview of Flash Attention series",
// section Backward Pass of flashattention), with S = scale * Q K^T:
//   P   = exp(S - lse)                       recomputed, never stored
//   dV  = P^T dO
//   dP  = dO V^T
//   D_i = do_i . o_i                         (the row term of the softmax Jacobian)
//   dS  = P o (dP - D)
//   dQ  = scale * dS K,   dK = scale * dS^T Q
// The N x N matrices P, dP and dS exist only tile by tile in registers and
// LDS; only the O(N) statistics lse and D are read from memory ("Как работает
// FlashAttention математически" section 5: recompute instead of store).
//
// Three launches on the caller's stream:
//   1. fa_bwd_pre: D_i = rowsum(dO o O) in fp32, and zero the fp32 dQ
//      accumulator (a plain store kernel, so the sequence is graph-capturable).
//   2. fa_bwd_main: a workgroup owns 128 keys (4 waves x 32) and keeps its
//      slice of K, V and the fp32 accumulators dK^T, dV^T in registers while
//      sweeping the query blocks that can see them (all blocks, or the blocks
//      at or below the diagonal when causal).  Per query block each wave
//      recomputes S and P for its 32 keys, forms dP and dS, and accumulates
//      dV^T += dO^T P and dK^T += Q^T dS on the matrix cores (the P and dS
//      registers are already in B-operand layout; Q^T and dO^T fragments come
//      from the row-major LDS tiles through the gfx950 transpose read).  dS is
//      then exchanged through LDS so that each wave forms one 32x32 tile of
//      dQ = dS K over all 128 keys and adds it to the fp32 accumulator with
//      atomics, one contribution per (query block, workgroup).
//   3. fa_bwd_dq: dQ = scale * accumulator, rounded to the element type.
// The loop order over (key block outer, query block inner) is the one whose
// dK/dV stay on chip; the pages leave the backward loop order open.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdKW = 32;                      // keys per wave
constexpr int kBwdBK = kBwdWaves * kBwdKW;      // keys per workgroup

template <typename T, int D>
struct BwdSmem {
  static constexpr int ESZ = sizeof(T);
  static constexpr int BQ = 32 * kBwdWaves * 32 / D;   // query rows per block: dQ tiles = waves
  static constexpr int QB = BQ / 32;                   // 32-row query sub-blocks
  static constexpr int QLD = D + 16 / ESZ;             // Q / dO row stride (elements)
  static constexpr int SLD = kBwdBK + 16 / ESZ;        // dS row stride (elements)
  // stage: Q tile, dO tile (T) then lse (in the exponent domain) and D (float)
  static constexpr int QTILE_B = BQ * QLD * ESZ;
  static constexpr int STAGE_B = 2 * QTILE_B + 2 * BQ * 4;
  static constexpr int DS_B = BQ * SLD * ESZ;
  static constexpr int BYTES = 2 * STAGE_B + DS_B;
  static constexpr int VE = 16 / ESZ;
  static constexpr int CPR = D / VE;
  static constexpr int NCH = BQ * CPR / kBwdThreads;
  static_assert(BQ * CPR % kBwdThreads == 0, "Q tile must split evenly over threads");
  static_assert((D / 32) * QB == kBwdWaves, "one dQ tile per wave");
  static_assert(QTILE_B % 16 == 0 && STAGE_B % 16 == 0, "16-byte aligned LDS regions");
};

// Transposed A fragment (M = d, K = rows) from a row-major bf16 LDS tile:
// lane l gets column dcol0 + l%32 of rows row0 + 8a + 4g + b (a in {0,1},
// b in 0..3), matching the accumulator rows acc_row(8t + e, g) of a 32-row
// sub-block when row0 = 16t.
__device__ __forceinline__ bf16x8 load_tr_frag(const bf16* base, int ld, int row0, int dcol0, int lane) {
  const int j = lane & 15;
  const int h = (lane >> 4) & 1;
  const int g = lane >> 5;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const bf16* p0 = base + (row0 + 4 * g + (j >> 2)) * ld + dcol0 + 16 * h + 4 * (j & 3);
  const bf16* p1 = p0 + 8 * ld;
  union { s16x4 s[2]; bf16x8 b; } u;
  u.s[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  u.s[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  return u.b;
}

// ---------------------------------------------------------------- 1. preprocess
template <typename T, int D>
__global__ __launch_bounds__(256)
void fa_bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ dsum,
                       float* __restrict__ dq_acc, size_t rows) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int CPR = D / VE;                 // threads per row
  constexpr int RPB = 256 / CPR;              // rows per block
  const int tid = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * RPB + tid / CPR;
  const int col = (tid % CPR) * VE;
  float part = 0.f;
  if (row < rows) {
    Vec16<T> o, d;
    o.raw = *reinterpret_cast<const uint4*>(O + row * D + col);
    d.raw = *reinterpret_cast<const uint4*>(dO + row * D + col);
#pragma unroll
    for (int e = 0; e < VE; ++e) part += (float)o.get(e) * (float)d.get(e);
    float4* z = reinterpret_cast<float4*>(dq_acc + row * D + col);
#pragma unroll
    for (int e = 0; e < VE / 4; ++e) z[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if (row < rows && tid % CPR == 0) dsum[row] = part;
}

// ---------------------------------------------------------------- 2. main loop
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1)
void fa_bwd_main_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                        const T* __restrict__ dO, const float* __restrict__ LSE,
                        const float* __restrict__ dsum, float* __restrict__ dq_acc,
                        T* __restrict__ dK, T* __restrict__ dV, int N, int BH, float scale,
                        float scale_log2) {
  using M = Mfma<T>;
  using L = BwdSmem<T, D>;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NDB = D / 32;
  constexpr int BQ = L::BQ, QB = L::QB;
  const float kfac = ExpDomain<T>::factor(scale, scale_log2);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 5;
  const int r32 = lane & 31;

  const int bh = blockIdx.x % BH;
  const int kt = blockIdx.x / BH;             // causal: low key tiles (most work) first
  const int k0 = kt * kBwdBK;
  const int kw0 = k0 + w * kBwdKW;
  const int mykey = kw0 + r32;
  const size_t head = (size_t)bh * N * D;
  const T* Qh = Q + head;
  const T* Kh = K + head;
  const T* Vh = V + head;
  const T* dOh = dO + head;
  const float* lse_h = LSE + (size_t)bh * N;
  const float* dsum_h = dsum + (size_t)bh * N;
  float* dq_h = dq_acc + head;

  // K and V rows of this wave as B operands (column = key, KPL d-values of group g).
  typename M::Frag kf[D / KC], vf[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c) {
    const bool ok = mykey < N;
    kf[c] = ok ? M::load(Kh + (size_t)mykey * D + c * KC + g * KPL) : M::zero();
    vf[c] = ok ? M::load(Vh + (size_t)mykey * D + c * KC + g * KPL) : M::zero();
  }
  // K^T for this wave's dQ tile (column d = dblk*32 + l%32, KPL keys of group g
  // per step, all 128 keys of the workgroup) as the B operand of dQ = dS K.
  const int dblk = w % NDB;
  const int qblk = w / NDB;
  typename M::Frag ktf[kBwdBK / KC];
#pragma unroll
  for (int kc = 0; kc < kBwdBK / KC; ++kc) {
    if constexpr (sizeof(T) == 2) {
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = k0 + kc * 16 + 8 * g + e;
        f[e] = key < N ? Kh[(size_t)key * D + dblk * 32 + r32] : (bf16)0.f;
      }
      ktf[kc] = f;
    } else {
      const int key = k0 + kc * 2 + g;
      ktf[kc] = key < N ? Kh[(size_t)key * D + dblk * 32 + r32] : 0.f;
    }
  }

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv_acc[db] = f32x16{};
    dk_acc[db] = f32x16{};
  }

  T* ds_s = reinterpret_cast<T*>(smem_raw + 2 * L::STAGE_B);
  auto stage_q = [&](int st) { return reinterpret_cast<T*>(smem_raw + st * L::STAGE_B); };
  auto stage_do = [&](int st) { return reinterpret_cast<T*>(smem_raw + st * L::STAGE_B + L::QTILE_B); };
  auto stage_lse = [&](int st) { return reinterpret_cast<float*>(smem_raw + st * L::STAGE_B + 2 * L::QTILE_B); };
  auto stage_dd = [&](int st) { return stage_lse(st) + BQ; };

  uint4 qreg[L::NCH], doreg[L::NCH];
  float lse_reg = 0.f, dd_reg = 0.f;
  auto load_block = [&](int q0b) {
#pragma unroll
    for (int r = 0; r < L::NCH; ++r) {
      const int c = tid + r * kBwdThreads;
      const int row = c / L::CPR;
      const int col = (c % L::CPR) * L::VE;
      const int q = q0b + row;
      if (q < N) {
        qreg[r] = *reinterpret_cast<const uint4*>(Qh + (size_t)q * D + col);
        doreg[r] = *reinterpret_cast<const uint4*>(dOh + (size_t)q * D + col);
      } else {
        qreg[r] = make_uint4(0, 0, 0, 0);
        doreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BQ) {
      const int q = q0b + tid;
      // rows past the end get lse = +inf, hence P = 0
      lse_reg = q < N ? ExpDomain<T>::from_lse(lse_h[q]) : __builtin_inff();
      dd_reg = q < N ? dsum_h[q] : 0.f;
    }
  };
  auto store_block = [&](int st) {
    T* qs = stage_q(st);
    T* dos = stage_do(st);
#pragma unroll
    for (int r = 0; r < L::NCH; ++r) {
      const int c = tid + r * kBwdThreads;
      const int row = c / L::CPR;
      const int col = (c % L::CPR) * L::VE;
      *reinterpret_cast<uint4*>(qs + row * L::QLD + col) = qreg[r];
      *reinterpret_cast<uint4*>(dos + row * L::QLD + col) = doreg[r];
    }
    if (tid < BQ) {
      stage_lse(st)[tid] = lse_reg;
      stage_dd(st)[tid] = dd_reg;
    }
  };

  const int q_begin = CAUSAL ? k0 : 0;   // queries below k0 see none of these keys
  const int nblocks = (N - q_begin + BQ - 1) / BQ;

  load_block(q_begin);
  store_block(0);
  __syncthreads();

  for (int jb = 0; jb < nblocks; ++jb) {
    const int q0b = q_begin + jb * BQ;
    const int st = jb & 1;
    if (jb + 1 < nblocks) load_block(q0b + BQ);

    const T* qs = stage_q(st);
    const T* dos = stage_do(st);
    const float* lse_s = stage_lse(st);
    const float* dd_s = stage_dd(st);

    const bool skip = CAUSAL && (q0b + BQ - 1 < kw0);   // every query precedes every key of the wave
    if (!skip) {
      const bool masked = (CAUSAL && q0b < kw0 + kBwdKW - 1) || (kw0 + kBwdKW > N);
#pragma unroll
      for (int qs_i = 0; qs_i < QB; ++qs_i) {
        // S = Q K^T and dP = dO V^T: rows = queries, column = this lane's key.
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int c = 0; c < D / KC; ++c) {
          typename M::Frag aq = M::load(qs + (qs_i * 32 + r32) * L::QLD + c * KC + g * KPL);
          typename M::Frag ado = M::load(dos + (qs_i * 32 + r32) * L::QLD + c * KC + g * KPL);
          s = M::mma(aq, kf[c], s);
          dp = M::mma(ado, vf[c], dp);
        }
        // P = exp(S - lse) and dS = P (dP - D), row by row of the accumulator.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = qs_i * 32 + acc_row(i, g);
          float p = ExpDomain<T>::ex(__builtin_fmaf(s[i], kfac, -lse_s[ql]));
          if (masked) {
            const int q = q0b + ql;
            const bool out = (mykey >= N) || (CAUSAL && mykey > q);
            p = out ? 0.f : p;
          }
          s[i] = p;
          dp[i] = p * (dp[i] - dd_s[ql]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (k = the 32 queries of the sub-block).
#pragma unroll
        for (int t = 0; t < 32 / KC; ++t) {
          typename M::Frag pb = M::pack(s, t);
          typename M::Frag dsb = M::pack(dp, t);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            typename M::Frag a_do, a_q;
            if constexpr (sizeof(T) == 2) {
              a_do = load_tr_frag(reinterpret_cast<const bf16*>(dos), L::QLD, qs_i * 32 + 16 * t, db * 32, lane);
              a_q = load_tr_frag(reinterpret_cast<const bf16*>(qs), L::QLD, qs_i * 32 + 16 * t, db * 32, lane);
            } else {
              const int row = qs_i * 32 + acc_row(t, g);
              a_do = dos[row * L::QLD + db * 32 + r32];
              a_q = qs[row * L::QLD + db * 32 + r32];
            }
            dv_acc[db] = M::mma(a_do, pb, dv_acc[db]);
            dk_acc[db] = M::mma(a_q, dsb, dk_acc[db]);
          }
        }
        // dS to LDS as [query][key] for the dQ product.
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ds_s[(qs_i * 32 + acc_row(i, g)) * L::SLD + w * kBwdKW + r32] = (T)dp[i];
      }
    } else {
#pragma unroll
      for (int qs_i = 0; qs_i < QB; ++qs_i)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ds_s[(qs_i * 32 + acc_row(i, g)) * L::SLD + w * kBwdKW + r32] = (T)0.f;
    }
    __syncthreads();

    // dQ tile (queries qblk*32.., d dblk*32..) = dS K over the 128 keys.
    {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < kBwdBK / KC; ++kc) {
        typename M::Frag a = M::load(ds_s + (qblk * 32 + r32) * L::SLD + kc * KC + g * KPL);
        acc = M::mma(a, ktf[kc], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0b + qblk * 32 + acc_row(i, g);
        if (q < N) unsafeAtomicAdd(dq_h + (size_t)q * D + dblk * 32 + r32, acc[i]);
      }
    }

    if (jb + 1 < nblocks) store_block(st ^ 1);
    __syncthreads();
  }

  // dK = scale * dK_acc, dV = dV_acc; lane holds key mykey, d = db*32 + acc_row(i, g).
  if (mykey < N) {
    T* dk_row = dK + head + (size_t)mykey * D;
    T* dv_row = dV + head + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = db * 32 + 8 * a + 4 * g;
        if constexpr (sizeof(T) == 2) {
          bf16x4 k4, v4;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            k4[b] = (bf16)(dk_acc[db][4 * a + b] * scale);
            v4[b] = (bf16)dv_acc[db][4 * a + b];
          }
          *reinterpret_cast<bf16x4*>(dk_row + d0) = k4;
          *reinterpret_cast<bf16x4*>(dv_row + d0) = v4;
        } else {
          f32x4 k4, v4;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            k4[b] = dk_acc[db][4 * a + b] * scale;
            v4[b] = dv_acc[db][4 * a + b];
          }
          *reinterpret_cast<f32x4*>(dk_row + d0) = k4;
          *reinterpret_cast<f32x4*>(dv_row + d0) = v4;
        }
      }
  }
}

// ---------------------------------------------------------------- 3. dQ finalise
template <typename T>
__global__ __launch_bounds__(256)
void fa_bwd_dq_kernel(const float* __restrict__ dq_acc, T* __restrict__ dq, size_t n4, float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 x = reinterpret_cast<const float4*>(dq_acc)[i];
  if constexpr (sizeof(T) == 2) {
    bf16x4 y;
    y[0] = (bf16)(x.x * scale);
    y[1] = (bf16)(x.y * scale);
    y[2] = (bf16)(x.z * scale);
    y[3] = (bf16)(x.w * scale);
    reinterpret_cast<bf16x4*>(dq)[i] = y;
  } else {
    reinterpret_cast<float4*>(dq)[i] = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  using L = BwdSmem<T, D>;
  const int BH = a.B * a.H;
  const size_t rows = (size_t)BH * a.N;
  if (stages & kStagePre) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL((fa_bwd_pre_kernel<T, D>), grid, dim3(256), 0, stream, static_cast<const T*>(a.o),
                       static_cast<const T*>(a.dout), a.dsum, a.dq_acc, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageMain) {
    auto kern = fa_bwd_main_kernel<T, D, CAUSAL>;
    static const hipError_t attr_err =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    if (attr_err != hipSuccess) return attr_err;
    const int n_ktiles = (a.N + kBwdBK - 1) / kBwdBK;
    hipLaunchKernelGGL(kern, dim3(n_ktiles * BH), dim3(kBwdThreads), L::BYTES, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<const T*>(a.dout), a.lse, a.dsum, a.dq_acc, static_cast<T*>(a.dk),
                       static_cast<T*>(a.dv), a.N, BH, a.scale, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageFinal) {
    const size_t n4 = rows * D / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T>), grid, dim3(256), 0, stream, a.dq_acc, static_cast<T*>(a.dq),
                       n4, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, int stages, hipStream_t s) {
  const bool c = a.causal != 0;
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) return c ? launch_bwd_t<bf16, 64, true>(a, stages, s) : launch_bwd_t<bf16, 64, false>(a, stages, s);
    return c ? launch_bwd_t<bf16, 128, true>(a, stages, s) : launch_bwd_t<bf16, 128, false>(a, stages, s);
  }
  if (a.d == 64) return c ? launch_bwd_t<float, 64, true>(a, stages, s) : launch_bwd_t<float, 64, false>(a, stages, s);
  return c ? launch_bwd_t<float, 128, true>(a, stages, s) : launch_bwd_t<float, 128, false>(a, stages, s);
}

}  // namespace fa
