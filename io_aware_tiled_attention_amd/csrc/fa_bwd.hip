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
//      at or below the diagonal when causal), BQ query rows at a time.  Per
//      32-row sub-block each wave recomputes S and P for its 32 keys, forms dP
//      and dS, and accumulates dV^T += dO^T P and dK^T += Q^T dS on the matrix
//      cores (P and dS are already in B-operand layout; dO^T and Q^T come from
//      the row-major LDS tiles through the gfx950 transpose read).  dS^T goes
//      to LDS; in the next iteration each wave reads it back, transposed, as
//      the A operand of dQ = dS K over all 128 keys and adds its tiles to the
//      fp32 accumulator with buffer atomics -- one contribution per (query
//      block, workgroup), one barrier per query block.
//      Query blocks are swept from the last one downwards: all key tiles of a
//      head run at the same time on one XCD and reach the same query block
//      together, so their dQ atomics meet in that XCD's L2.
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
struct BwdCfg {
  static constexpr int ESZ = sizeof(T);
  static constexpr int BQ = ESZ == 2 ? 64 : 32;        // query rows per block
  static constexpr int QB = BQ / 32;                   // 32-row sub-blocks
  static constexpr int NDB = D / 32;                   // 32-wide d blocks
  static constexpr int NDQ = NDB * QB;                 // 32x32 dQ tiles per block
  static constexpr int TPW = (NDQ + kBwdWaves - 1) / kBwdWaves;   // dQ tiles per wave
  static constexpr int QTILE = BQ * D * ESZ;           // bytes of the Q (or dO) tile
  static constexpr int STATS = 2 * 64 * 4;             // lse, D: 64 floats each
  static constexpr int STAGE = 2 * QTILE + STATS;
  static constexpr int DST = kBwdBK * BQ * ESZ;        // dS^T tile [keys][queries]
  static constexpr int BYTES = 2 * STAGE + 2 * DST;
  static_assert(ESZ != 2 || kBwdBK * D * ESZ <= 2 * DST, "K staging fits in the dS^T buffers");
  static_assert(NDB % 1 == 0 && (NDQ <= kBwdWaves || NDQ % kBwdWaves == 0), "dQ tiles split over waves");
  static_assert(kBwdWaves % NDB == 0 || NDB % kBwdWaves == 0, "one d block per wave");
  __device__ static lds_u8* q(lds_u8* b, int st) { return b + st * STAGE; }
  __device__ static lds_u8* dout(lds_u8* b, int st) { return b + st * STAGE + QTILE; }
  __device__ static lds_u8* lse(lds_u8* b, int st) { return b + st * STAGE + 2 * QTILE; }
  __device__ static lds_u8* dd(lds_u8* b, int st) { return b + st * STAGE + 2 * QTILE + 256; }
  __device__ static lds_u8* dst(lds_u8* b, int k) { return b + 2 * STAGE + k * DST; }
};

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
    union { uint4 u; T t[VE]; } o, d;
    o.u = *reinterpret_cast<const uint4*>(O + row * D + col);
    d.u = *reinterpret_cast<const uint4*>(dO + row * D + col);
#pragma unroll
    for (int e = 0; e < VE; ++e) part += (float)o.t[e] * (float)d.t[e];
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
                        T* __restrict__ dK, T* __restrict__ dV, int N, int BH, float scale) {
  using M = Mfma<T>;
  using C = BwdCfg<T, D>;
  using G = Tile<T, D>;                 // Q, dO and K tiles: rows x D
  using GS = Tile<T, C::BQ>;            // dS^T tile: 128 key rows x BQ query columns
  using X = ExpDomain<T>;
  using Frag = typename M::Frag;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NDB = C::NDB, BQ = C::BQ, QB = C::QB;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;

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
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  const rsrc_t rk = make_rsrc(K + head, head_bytes);
  const rsrc_t rv = make_rsrc(V + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const rsrc_t rlse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rdd = make_rsrc(dsum + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rdq = make_rsrc(dq_acc + head, (uint32_t)N * D * 4u);
  const float kfac = X::factor(scale);

  // K and V rows of this wave as B operands (column = key, KPL d-values of group g).
  Frag kf[D / KC], vf[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c) {
    const int off = mykey * G::R + (c * KC + g * KPL) * (int)sizeof(T);
    kf[c] = M::load(rk, off);
    vf[c] = M::load(rv, off);
  }

  // K^T for this wave's dQ tiles (column d = dblk*32 + l%32) as the B operand of
  // dQ = dS K; k-step kc covers keys kc*KC.., in the order of the dS fragments.
  const int dblk = w % NDB;
  Frag ktf[kBwdBK / KC];
  if constexpr (sizeof(T) == 2) {
    // stage the workgroup's 128 K rows in the (not yet used) dS^T buffers and
    // read them back transposed: lane gets keys kc*16 + 8a + 4g + b
    lds_u8* kst = C::dst(smem, 0);
    tile_to_lds<T, D, kBwdBK, kBwdWaves>(rk, kst, k0, w, lane);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < kBwdBK / KC; ++kc) ktf[kc] = lds_tr_frag<D>(kst, kc * 16, dblk * 32, lane);
    __syncthreads();
  } else {
#pragma unroll
    for (int kc = 0; kc < kBwdBK / KC; ++kc)
      ktf[kc] = M::load(rk, (k0 + kc * 2 + g) * G::R + (dblk * 32 + r32) * (int)sizeof(T));
  }

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv_acc[db] = f32x16{};
    dk_acc[db] = f32x16{};
  }

  auto load_block = [&](int q0b, int st) {
    tile_to_lds<T, D, BQ, kBwdWaves>(rq, C::q(smem, st), q0b, w, lane);
    tile_to_lds<T, D, BQ, kBwdWaves>(rdo, C::dout(smem, st), q0b, w, lane);
    // lse and D of the block's rows, one float per lane (rows past N read 0)
    if (w == 0) lds_dma4(rlse, C::lse(smem, st), (q0b + lane) * 4);
    if (w == 1) lds_dma4(rdd, C::dd(smem, st), (q0b + lane) * 4);
  };

  // dQ tiles of the block whose dS^T is in buffer `buf`: tile t = w + 4u covers
  // d block t % NDB (= dblk) and query sub-block t / NDB.
  auto dq_block = [&](int q0b, int buf) {
    const lds_u8* ds = C::dst(smem, buf);
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = w + kBwdWaves * u;
      if (t < C::NDQ) {
        const int qblk = t / NDB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kc = 0; kc < kBwdBK / KC; ++kc) {
          Frag a;
          if constexpr (sizeof(T) == 2) a = lds_tr_frag<BQ>(ds, kc * 16, qblk * 32, lane);
          else a = M::lds(ds + GS::off(kc * 2 + g, qblk * 32 + r32));
          acc = M::mma(a, ktf[kc], acc);
        }
        // lane holds column d = dblk*32 + r32 of query rows acc_row(i, g)
        const int qrow = q0b + qblk * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          atomic_add_f32(rdq, ((qrow + acc_row(i, g)) * D + dblk * 32 + r32) * 4, acc[i]);
      }
    }
  };

  // Query blocks from the last one down to the first that sees these keys.
  const int nqb_total = (N + BQ - 1) / BQ;
  const int qb_first = CAUSAL ? k0 / BQ : 0;
  const int nblocks = nqb_total - qb_first;
  auto block_start = [&](int it) { return (nqb_total - 1 - it) * BQ; };

  load_block(block_start(0), 0);
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < nblocks; ++it) {
    const int q0b = block_start(it);
    const int st = it & 1;
    if (it + 1 < nblocks) load_block(block_start(it + 1), st ^ 1);
    if (it > 0) dq_block(block_start(it - 1), st ^ 1);

    const lds_u8* qs = C::q(smem, st);
    const lds_u8* dos = C::dout(smem, st);
    const lds_u8* lse_s = C::lse(smem, st);
    const lds_u8* dd_s = C::dd(smem, st);
    lds_u8* ds_out = C::dst(smem, st);

#pragma unroll
    for (int qs_i = 0; qs_i < QB; ++qs_i) {
      const int qsb = q0b + qs_i * 32;
      if (CAUSAL && qsb + 31 < kw0) {
        // every query of the sub-block precedes every key of the wave: dS = 0
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int off = GS::off(w * kBwdKW + r32, qs_i * 32 + 8 * a + 4 * g);
          if constexpr (sizeof(T) == 2) *(lds_u32x2*)(ds_out + off) = u32x2{0u, 0u};
          else *(lds_u32x4*)(ds_out + off) = u32x4{0u, 0u, 0u, 0u};
        }
        continue;
      }
      // S = Q K^T and dP = dO V^T: rows = queries, column = this lane's key.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / KC; ++c) {
        const int off = G::off(qs_i * 32 + r32, c * KC + g * KPL);
        s = M::mma(M::lds(qs + off), kf[c], s);
        dp = M::mma(M::lds(dos + off), vf[c], dp);
      }
      // P = exp(S - lse), dS = P (dP - D); masked entries (key > query, or a
      // key past the end) get P = 0.
      const bool masked = (CAUSAL && qsb < kw0 + kBwdKW - 1) || (kw0 + kBwdKW > N);
      const int lim = (mykey >= N) ? 64 : (CAUSAL ? mykey - (qsb + 4 * g) : -1);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 lz = *(const lds_f32x4*)(lse_s + (qs_i * 32 + 8 * a + 4 * g) * 4);
        const f32x4 dz = *(const lds_f32x4*)(dd_s + (qs_i * 32 + 8 * a + 4 * g) * 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          float p = X::ex(__builtin_fmaf(s[i], kfac, -X::from_lse(lz[b])));
          if (masked) p = (acc_row(i, 0) < lim) ? 0.f : p;
          s[i] = p;
          dp[i] = p * (dp[i] - dz[b]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (k = the 32 queries of the sub-block).
#pragma unroll
      for (int t = 0; t < 32 / KC; ++t) {
        const Frag pb = M::pack(s, t);
        const Frag dsb = M::pack(dp, t);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          Frag a_do, a_q;
          if constexpr (sizeof(T) == 2) {
            a_do = lds_tr_frag<D>(dos, qs_i * 32 + 16 * t, db * 32, lane);
            a_q = lds_tr_frag<D>(qs, qs_i * 32 + 16 * t, db * 32, lane);
          } else {
            const int off = G::off(qs_i * 32 + acc_row(t, g), db * 32 + r32);
            a_do = M::lds(dos + off);
            a_q = M::lds(qs + off);
          }
          dv_acc[db] = M::mma(a_do, pb, dv_acc[db]);
          dk_acc[db] = M::mma(a_q, dsb, dk_acc[db]);
        }
      }
      // dS^T (row = key, 4 consecutive query columns per store) for the dQ product.
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int off = GS::off(w * kBwdKW + r32, qs_i * 32 + 8 * a + 4 * g);
        if constexpr (sizeof(T) == 2) {
          const bf16x4 v4 = {(bf16)dp[4 * a], (bf16)dp[4 * a + 1], (bf16)dp[4 * a + 2], (bf16)dp[4 * a + 3]};
          *(lds_u32x2*)(ds_out + off) = __builtin_bit_cast(u32x2, v4);
        } else {
          const f32x4 v4 = {dp[4 * a], dp[4 * a + 1], dp[4 * a + 2], dp[4 * a + 3]};
          *(lds_u32x4*)(ds_out + off) = __builtin_bit_cast(u32x4, v4);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
  dq_block(block_start(nblocks - 1), (nblocks - 1) & 1);

  // dK = scale * dK_acc, dV = dV_acc; lane holds key mykey, d = db*32 + acc_row(i, g).
  const rsrc_t rdk = make_rsrc(dK + head, head_bytes);
  const rsrc_t rdv = make_rsrc(dV + head, head_bytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int off = mykey * G::R + (db * 32 + 8 * a + 4 * g) * (int)sizeof(T);
      store4<T>(rdk, off, dk_acc[db][4 * a] * scale, dk_acc[db][4 * a + 1] * scale, dk_acc[db][4 * a + 2] * scale,
                dk_acc[db][4 * a + 3] * scale);
      store4<T>(rdv, off, dv_acc[db][4 * a], dv_acc[db][4 * a + 1], dv_acc[db][4 * a + 2], dv_acc[db][4 * a + 3]);
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
    const bf16x4 y = {(bf16)(x.x * scale), (bf16)(x.y * scale), (bf16)(x.z * scale), (bf16)(x.w * scale)};
    reinterpret_cast<bf16x4*>(dq)[i] = y;
  } else {
    reinterpret_cast<float4*>(dq)[i] = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  using C = BwdCfg<T, D>;
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
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
    if (attr_err != hipSuccess) return attr_err;
    const int n_ktiles = (a.N + kBwdBK - 1) / kBwdBK;
    hipLaunchKernelGGL(kern, dim3(n_ktiles * BH), dim3(kBwdThreads), C::BYTES, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<const T*>(a.dout), a.lse, a.dsum, a.dq_acc, static_cast<T*>(a.dk),
                       static_cast<T*>(a.dv), a.N, BH, a.scale);
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
