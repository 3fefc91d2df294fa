// fa_fwd_fp8.hip -- attention forward with 8-bit float inputs for gfx950 (MI355X).
//
// What is computed: exact attention ("Overview of Flash Attention series",
// Standard Attention / Forward Pass) of Q, K, V stored in the OCP 8-bit float
// E4M3, each tensor with one descale factor (value = stored number times its
// factor):  O = softmax(scale sq sk Q8 K8^T) sv V8,  lse of the scaled
// scores.  O is written in bfloat16.  FP8 is named on the pages only as a
// feature of FlashAttention-3 on Hopper ("Как работает FlashAttention
// математически", section 9); the format and the scaling rule are this
// library's.
//
// How: the loop of the bf16 forward (fa_fwd.hip) on the gfx950 8-bit matrix
// core, v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 per instruction, twice the
// bf16 rate):
//   * S^T = K Q^T: each lane supplies 32 consecutive d-bytes of its key (A)
//     and of its query (B); any k-order shared by both operands sums over d;
//   * the probabilities, in (0, 2^8] under the lazy shift, are rounded to
//     E4M3 (v_cvt_pk_fp8_f32, round to nearest even) for O^T += V^T P^T.  The
//     S^T accumulators leave each lane four keys of every group of eight; one
//     v_permlane32_swap per four keys gives each lane 32 consecutive keys,
//     the layout the V^T operand can be read in;
//   * V^T comes from the row-major V tile through the 8-bit LDS transpose
//     read ds_read_b64_tr_b8: within 16 lanes, lane L reads 8 bytes of key
//     row L/2 and output lane i receives byte i%8 of the reads of lanes
//     2e + i/8 (e = 0..7) -- 8 consecutive keys of one d column;
//   * l sums the unrounded probabilities, so only P's rounding enters O.
// K/V tiles are 64 keys x D bytes, swizzled so that both the 16-byte K reads
// and the transpose reads are free of bank conflicts.  S of a tile is
// computed right before its softmax (no second set of S registers), which
// leaves room for three waves per SIMD: the vector work of one wave then
// overlaps the matrix work of another more often.
#include <algorithm>
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kF8Waves = 4;
constexpr int kF8QW = 32;                     // query rows per wave
constexpr int kF8BR = kF8Waves * kF8QW;       // query rows per workgroup
constexpr int kF8BC = 64;                     // keys per K/V tile
constexpr int kF8Threads = kF8Waves * 64;

// Row-major tile of D one-byte elements per row; 16-byte chunk c of row r is
// stored at chunk c ^ swz(r) (periodic in 32 rows).
template <int D> struct Tile8 {
  static constexpr int R = D;
  static constexpr int NCH = R / 16;
  __device__ __forceinline__ static constexpr int swz(int row) {
    if constexpr (D == 128) return (row >> 1) & 7;
    else return ((row >> 1) ^ (row >> 3)) & 3;
  }
  __device__ __forceinline__ static constexpr int off(int row, int byte) {
    return row * R + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
  }
};

template <int D> struct F8Smem {
  static constexpr int TILE = kF8BC * D;      // bytes of one K or V tile
  static constexpr int BYTES = 4 * TILE;      // [K st0][K st1][V st0][V st1]
  __device__ static lds_u8* k(lds_u8* b, int st) { return b + st * TILE; }
  __device__ static lds_u8* v(lds_u8* b, int st) { return b + (2 + st) * TILE; }
};

// rows [row0, row0 + kF8BC) of one head's [N, D] byte tensor into an LDS
// tile, 1 KiB per wave instruction; rows past the end read as zero.
template <int D>
__device__ __forceinline__ void tile8_to_lds(rsrc_t src, lds_u8* tile, int row0, int w, int lane) {
  using G = Tile8<D>;
  constexpr int SEGS = kF8BC * G::R / 1024;
  static_assert(SEGS % kF8Waves == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int r = 0; r < SEGS / kF8Waves; ++r) {
    const int s = w * (SEGS / kF8Waves) + r;
    const int o = s * 1024 + lane * 16;
    const int row = o / G::R;
    const int chunk = ((o % G::R) >> 4) ^ G::swz(row);
    lds_dma16(src, tile + s * 1024, (uint32_t)(row0 + row) * G::R + chunk * 16);
  }
}

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four probabilities -> four E4M3 bytes of one word (round to nearest even).
// Each conversion writes one half of the word and keeps the other; the first
// is seeded with a's own bits (both halves end up overwritten), which spares
// the register a zero seed would need.
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 3)
void fa_fwd_fp8_kernel(const unsigned char* __restrict__ Q, const unsigned char* __restrict__ K,
                       const unsigned char* __restrict__ V, bf16* __restrict__ O, float* __restrict__ LSE, int N,
                       int BH, int n_qtiles, int group, float kfac, float v_descale) {
  using L = F8Smem<D>;
  using G = Tile8<D>;
  using X = ExpDomain<bf16>;                   // base-2 exponent domain
  constexpr int NC = D / 64;                   // k-chunks of the S product
  constexpr int NKB = kF8BC / 32;              // 32-key blocks per tile
  constexpr int NDB = D / 32;                  // 32-wide d blocks of O^T
  // Static LDS: its base is known when the kernel is compiled, so with the
  // loop below unrolled over the two stages every LDS read is one per-lane
  // offset register plus an immediate.
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[F8Smem<D>::BYTES];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // heads grouped per XCD, longest-first for causal
  const WgOrder wo = wg_order(blockIdx.x, BH, n_qtiles, group);
  const int bh = wo.bh;
  const int qt = CAUSAL ? n_qtiles - 1 - wo.rank : wo.rank;
  const int q0 = qt * kF8BR;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  const rsrc_t rk = make_rsrc(K + head, head_bytes);
  const rsrc_t rv = make_rsrc(V + head, head_bytes);

  const int qw0 = q0 + w * kF8QW;
  const int myq = qw0 + r32;

  // Q^T as the B operand: column = query, d-bytes 64c + 32g .. +31.
  i32x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t qo = (uint32_t)myq * G::R + 64 * c + 32 * g;
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qo + 16, 0, 0));
    qf[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // Per-lane LDS offsets, the same for every tile (the swizzle is periodic in 32 rows):
  //   ka[c][h]: 16 bytes of this lane's key row r32 (add kb*32 rows), k-chunk c, half h;
  //   vt[t][db]: transpose read t of d block db: key row 32g + 8t + (j >> 1),
  //              columns db*32 + 16*hh + 8*(j & 1), j = lane % 16, hh = (lane / 16) % 2.
  int ka[NC][2], vt[4][NDB];
  {
    const int j = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) ka[c][h] = G::off(r32, 64 * c + 32 * g + 16 * h);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vt[t][db] = G::off(32 * g + 8 * t + (j >> 1), db * 32 + 16 * hh + 8 * (j & 1));
  }

  const int kv_end = CAUSAL ? min(N, q0 + kF8BR) : N;
  const int ntiles = (kv_end + kF8BC - 1) / kF8BC;
  const int wave_last = CAUSAL ? min(ntiles - 1, (qw0 + kF8QW - 1) / kF8BC) : ntiles - 1;

  auto compute_st = [&](f32x16 (&s)[NKB], const lds_u8* ks) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 lo = *(const lds_u32x4*)(ks + kb * 32 * G::R + ka[c][0]);
        const u32x4 hi = *(const lds_u32x4*)(ks + kb * 32 * G::R + ka[c][1]);
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kb] = mma8(a, qf[c], s[kb]);
      }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float msub = kNegInf;   // exponent shift (running max of scaled scores, raised lazily)
  float l_run = 0.f;      // this lane's share of the running row sum, relative to msub

  f32x16 s_cur[NKB];
  tile8_to_lds<D>(rk, L::k(smem, 0), 0, w, lane);
  tile8_to_lds<D>(rv, L::v(smem, 0), 0, w, lane);
  wait_vmem();
  __syncthreads();

  // One tile: K/V of tile it in stage ST, those of tile it+1 copied into the other.
  auto step = [&](const int it, auto stage) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    const int kv0 = it * kF8BC;
    if (it + 1 < ntiles) {
      tile8_to_lds<D>(rk, L::k(smem, 1 - ST), (it + 1) * kF8BC, w, lane);
      tile8_to_lds<D>(rv, L::v(smem, 1 - ST), (it + 1) * kF8BC, w, lane);
    }

    if (it <= wave_last) {
      compute_st(s_cur, L::k(smem, ST));
      const bool masked = (CAUSAL && kv0 + kF8BC - 1 > qw0) || (kv0 + kF8BC > N);
      if (masked) {
        const int last = CAUSAL ? min(N - 1, myq) : N - 1;   // keys allowed: key <= last
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int lim = last - (kv0 + kb * 32 + 4 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i) s_cur[kb][i] = (acc_row(i, 0) > lim) ? kNegInf : s_cur[kb][i];
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
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
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = X::ex(__builtin_fmaf(s_cur[kb][i], kfac, -shift));
          s_cur[kb][i] = p;
          psum += p;
        }
      l_run += psum;

      // P^T as the B operand: word w of lane (query, g) = keys 32g + 4w .. 4w+3.
      // Word a of block kb holds keys kb*32 + 8a + 4g + 0..3; swapping the upper
      // lanes of block 0 with the lower lanes of block 1 leaves block g's keys
      // in order (words 2a: 8a..8a+3 and 2a+1: 8a+4..8a+7).
      i32x8 pb;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int w0 = pack4_e4m3(s_cur[0][4 * a], s_cur[0][4 * a + 1], s_cur[0][4 * a + 2], s_cur[0][4 * a + 3]);
        const int w1 = pack4_e4m3(s_cur[1][4 * a], s_cur[1][4 * a + 1], s_cur[1][4 * a + 2], s_cur[1][4 * a + 3]);
        const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)w0, (unsigned)w1, false, false);
        pb[2 * a] = (int)sw[0];
        pb[2 * a + 1] = (int)sw[1];
      }
      // O^T += V^T P^T: V^T bytes 8t..8t+7 of lane (d, g) = keys 32g + 8t .. +7 of column d.
      const lds_u8* vs = L::v(smem, ST);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8 va;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vs + vt[t][db]));
          va[2 * t] = x[0];
          va[2 * t + 1] = x[1];
        }
        oacc[db] = mma8(va, pb, oacc[db]);
      }
    }

    wait_vmem();
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < ntiles) step(it, std::integral_constant<int, 0>{});

  // O = v_descale * O_acc / l, lse = shift + ln l (natural log units).
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? v_descale / l_tot : 0.f;
  const rsrc_t ro = make_rsrc(O + head, (uint32_t)N * D * 2u);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = db * 32 + 8 * a + 4 * g;
      store4<bf16>(ro, (myq * D + d0) * 2, oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                   oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
    }
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const float lse = msub * X::kToNat + logf(l_tot);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, myq * 4, 0, 0);
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_t(const Fp8Args& a, hipStream_t stream) {
  auto kern = fa_fwd_fp8_kernel<D, CAUSAL>;   // LDS: static, F8Smem<D>::BYTES
  const int BH = a.B * a.H;
  const int n_qtiles = (a.N + kF8BR - 1) / kF8BR;
  // the scores' factor in the base-2 domain: scale * q_descale * k_descale * log2(e)
  const float kfac = std::max(a.scale * a.q_descale * a.k_descale * kLog2e, kMinFactor);
  hipLaunchKernelGGL(kern, dim3(n_qtiles * BH), dim3(kF8Threads), 0, stream,
                     static_cast<const unsigned char*>(a.q), static_cast<const unsigned char*>(a.k),
                     static_cast<const unsigned char*>(a.v), static_cast<bf16*>(a.o), a.lse, a.N, BH, n_qtiles,
                     wg_group(n_qtiles, 32 * 3), kfac, a.v_descale);   // 3 workgroups per CU
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch_fp8_t<64, true>(a, stream) : launch_fp8_t<64, false>(a, stream);
  return a.causal ? launch_fp8_t<128, true>(a, stream) : launch_fp8_t<128, false>(a, stream);
}

}  // namespace fa
