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
// The N x N matrices P, dP and dS exist only tile by tile in registers; only
// the O(N) statistics lse and D are read from memory ("Как работает
// FlashAttention математически" section 5: recompute instead of store).
//
// Three launches on the caller's stream, none of them with atomics:
//   1. fa_bwd_pre: D_i = rowsum(dO o O) in fp32 and -lse_i (in the exponent
//      domain) into the workspace.
//   2. fa_bwd_dkdv: a workgroup owns 128 keys and keeps the fp32
//      accumulators dK^T, dV^T of its keys in registers while sweeping the
//      query blocks that can see them (all blocks, or the blocks at or below
//      the diagonal when causal) through double-buffered LDS.  Per 32-row
//      sub-block a wave recomputes S and P for its 32 keys, forms dP and dS,
//      and accumulates dV^T += dO^T P and dK^T += Q^T dS on the matrix cores:
//      P and dS are already in B-operand layout, dO^T and Q^T come from the
//      row-major LDS tiles through the gfx950 transpose read.  bf16
//      (fa_bwd_dkdv_bf16_kernel): 8 waves, K and V resident in LDS, the two
//      waves of a SIMD taking the two 32-row halves of each 64-row block and
//      summing their partials through LDS at the end.  fp32: 4 waves with K
//      and V in registers.
//   3. fa_bwd_dq: the same recomputation in the transposed orientation, one
//      workgroup per 128 query rows (like the forward): S^T = K Q^T and
//      dP^T = V dO^T leave each lane with one query's scores, lse and D are
//      per-lane scalars, and dQ^T += K^T dS^T takes dS^T straight from
//      registers (K^T from the K tile through the transpose read).  dQ is
//      written once.
// Splitting dQ from dK/dV costs the two products S and dP a second time but
// needs no cross-workgroup reduction: on this GPU fp32 atomics are executed at
// the memory side, and the fused form spent most of its time waiting on them.
// The pages leave the backward loop order open (their figure is missing).
// Every grid is launched in the XCD-aware order of wg_order (longest work
// first within head groups).  SPARSE instantiations (block-sparse attention,
// "Overview of Flash Attention series", Block-sparse Flashattention) visit
// only the tiles a block mask keeps, from per-workgroup lists in LDS
// (build_tile_list); DROP ones regenerate the forward's dropout mask.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdKW = 32;                      // keys per wave
constexpr int kBwdBK = kBwdWaves * kBwdKW;      // keys per workgroup
constexpr int kBwdListCap = 2 * kListMax;         // block-sparse list of 32-row query blocks (fp32)

template <typename T, int D>
struct BwdCfg {
  static constexpr int ESZ = sizeof(T);
  static constexpr int BQ = ESZ == 2 ? 64 : 32;        // query rows per block
  static constexpr int QB = BQ / 32;                   // 32-row sub-blocks
  static constexpr int NDB = D / 32;                   // 32-wide d blocks
  static constexpr int QTILE = BQ * D * ESZ;           // bytes of the Q (or dO) tile
  static constexpr int STATS = 2 * 64 * 4;             // lse, D: 64 floats each
  static constexpr int STAGE = 2 * QTILE + STATS;
  static constexpr int BYTES = 2 * STAGE;
  __device__ static lds_u8* q(lds_u8* b, int st) { return b + st * STAGE; }
  __device__ static lds_u8* dout(lds_u8* b, int st) { return b + st * STAGE + QTILE; }
  __device__ static lds_u8* lse(lds_u8* b, int st) { return b + st * STAGE + 2 * QTILE; }
  __device__ static lds_u8* dd(lds_u8* b, int st) { return b + st * STAGE + 2 * QTILE + 256; }
};

// ---------------------------------------------------------------- 1. preprocess
// Row statistics in the workspace: dsum[i] = D_i = do_i . o_i, and
// nlse[i] = -lse_i in the exponent domain of T, so that the later kernels
// form P = ex(s * factor + nlse) with one FMA.  Blocks of RPB rows; the grid
// is capped at kPreMaxBlocks and strides over the rest (a launch's work-item
// count must fit in 32 bits).
constexpr unsigned kPreMaxBlocks = 1u << 16;
template <typename T, int D>
__global__ __launch_bounds__(256)
void fa_bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO, const float* __restrict__ LSE,
                       float* __restrict__ dsum, float* __restrict__ nlse, size_t rows) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int CPR = D / VE;                 // threads per row
  constexpr int RPB = 256 / CPR;              // rows per block
  const int tid = threadIdx.x;
  const int col = (tid % CPR) * VE;
  for (size_t blk = blockIdx.x; blk * RPB < rows; blk += gridDim.x) {   // block-uniform trip count
    const size_t row = blk * RPB + tid / CPR;
    float part = 0.f;
    if (row < rows) {
      union { uint4 u; T t[VE]; } o, d;
      o.u = *reinterpret_cast<const uint4*>(O + row * D + col);
      d.u = *reinterpret_cast<const uint4*>(dO + row * D + col);
#pragma unroll
      for (int e = 0; e < VE; ++e) part += (float)o.t[e] * (float)d.t[e];
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (row < rows && tid % CPR == 0) {
      dsum[row] = part;
      nlse[row] = -ExpDomain<T>::from_lse(LSE[row]);
    }
  }
}

// ---------------------------------------------------------------- 2. dK, dV
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kBwdThreads, 2)
void fa_bwd_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                        const T* __restrict__ dO, const float* __restrict__ dsum, const float* __restrict__ nlse,
                        T* __restrict__ dK, T* __restrict__ dV, int N, int BH, int n_ktiles, int group, float scale,
                        SparseArgs sp, DropParams dpar) {
  using M = Mfma<T>;
  using C = BwdCfg<T, D>;
  using G = Tile<T, D>;                 // Q and dO tiles: BQ rows x D
  using X = ExpDomain<T>;
  using Frag = typename M::Frag;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NDB = C::NDB, BQ = C::BQ, QB = C::QB;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // heads grouped per XCD; causal: low key tiles (most work) first
  const WgOrder wo = wg_order(blockIdx.x, BH, n_ktiles, group);
  const int bh = wo.bh;
  const int kt = wo.rank;
  const int k0 = kt * kBwdBK;
  const int kw0 = k0 + w * kBwdKW;
  const int mykey = kw0 + r32;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  const rsrc_t rk = make_rsrc(K + head, head_bytes);
  const rsrc_t rv = make_rsrc(V + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const rsrc_t rnl = make_rsrc(nlse + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rdd = make_rsrc(dsum + (size_t)bh * N, (uint32_t)N * 4u);
  const float kfac = X::factor(scale);
  int q_blk = 0;   // first query row of the current block (dropout counters)
  if constexpr (!DROP) (void)dpar;

  // K and V rows of this wave as B operands (column = key, KPL d-values of group g).
  Frag kf[D / KC], vf[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c) {
    const uint32_t off = (uint32_t)mykey * G::R + (c * KC + g * KPL) * (int)sizeof(T);
    kf[c] = M::load(rk, off);
    vf[c] = M::load(rv, off);
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
    // -lse and D of the block's rows, one float per lane (rows past N read 0)
    if (w == 0) lds_dma4(rnl, C::lse(smem, st), (q0b + lane) * 4);
    if (w == 1) lds_dma4(rdd, C::dd(smem, st), (q0b + lane) * 4);
  };

  // S = Q K^T and dP = dO V^T for 32-row sub-block qs_i: rows = queries,
  // column = this lane's key.  All A-operand fragments are read from LDS
  // before the products are issued, so the LDS latency is paid once.
  auto sdp = [&](const lds_u8* qs, const lds_u8* dos, int qs_i, f32x16& s, f32x16& dp) {
    Frag aq[D / KC], ado[D / KC];
#pragma unroll
    for (int c = 0; c < D / KC; ++c) {
      const int off = G::off(qs_i * 32 + r32, c * KC + g * KPL);
      aq[c] = M::lds(qs + off);
      ado[c] = M::lds(dos + off);
    }
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int c = 0; c < D / KC; ++c) {
      s = M::mma(aq[c], kf[c], s);
      dp = M::mma(ado[c], vf[c], dp);
    }
  };
  // P = ex(S*factor - lse) and dS = P (dP - D) in place; with `lim` >= 0
  // entries whose row offset acc_row(i, 0) < lim (key > query) get P = 0.
  // DROP: the P kept for dV is P o Z (1 / (1 - t/256) applied at the end),
  // and dS = P (dP o Z / (1 - t/256) - D).
  auto softmax_grad = [&](const lds_u8* nl_s, const lds_u8* dd_s, int qs_i, f32x16& s, f32x16& dp, bool masked,
                          int lim) {
    u32x4 rb = {};
    if constexpr (DROP)
      rb = drop_bytes_queries(dpar.k0, dpar.k1, dpar.offset, (unsigned)bh, mykey, q_blk + qs_i * 32, g, lane);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 lz = *(const lds_f32x4*)(nl_s + (qs_i * 32 + 8 * a + 4 * g) * 4);
      const f32x4 dz = *(const lds_f32x4*)(dd_s + (qs_i * 32 + 8 * a + 4 * g) * 4);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = 4 * a + b;
        float p = X::ex(__builtin_fmaf(s[i], kfac, lz[b]));
        if (masked) p = (acc_row(i, 0) < lim) ? 0.f : p;
        if constexpr (DROP) {
          const bool keep = drop_keep(rb, i, dpar.t);
          s[i] = keep ? p : 0.f;
          dp[i] = p * ((keep ? dp[i] * dpar.rs : 0.f) - dz[b]);
        } else {
          s[i] = p;
          dp[i] = p * (dp[i] - dz[b]);
        }
      }
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS (k = the 32 queries of the sub-block);
  // the transposed fragments of one k-step are read before its products.
  auto accumulate = [&](const lds_u8* qs, const lds_u8* dos, int qs_i, const f32x16& s, const f32x16& dp) {
#pragma unroll
    for (int t = 0; t < 32 / KC; ++t) {
      Frag a_do[NDB], a_q[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (sizeof(T) == 2) {
          a_do[db] = lds_tr_frag<D>(dos, qs_i * 32 + 16 * t, db * 32, lane);
          a_q[db] = lds_tr_frag<D>(qs, qs_i * 32 + 16 * t, db * 32, lane);
        } else {
          const int off = G::off(qs_i * 32 + acc_row(t, g), db * 32 + r32);
          a_do[db] = M::lds(dos + off);
          a_q[db] = M::lds(qs + off);
        }
      }
      const Frag pb = M::pack(s, t);
      const Frag dsb = M::pack(dp, t);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv_acc[db] = M::mma(a_do[db], pb, dv_acc[db]);
        dk_acc[db] = M::mma(a_q[db], dsb, dk_acc[db]);
      }
    }
  };

  // Query blocks from the first one that sees these keys to the end.
  const int q_begin = CAUSAL ? k0 : 0;
  const int nblocks = (N - q_begin + BQ - 1) / BQ;

  // The query blocks visited: all from q_begin (dense), or those the block
  // mask keeps for some (sub-block, wave) pair, bit qs_i * waves + wave
  // (block-sparse; each 32-row sub-block lies in one mask row, each wave's
  // 32 keys in one mask column).
  const TileList tl = tile_list_at<kBwdListCap>(smem + C::BYTES);
  int n_act = nblocks;
  if constexpr (SPARSE) {
    const int tk_n = (N + sp.block_k - 1) / sp.block_k;
    const int tq_n = (N + sp.block_q - 1) / sp.block_q;
    const unsigned char* mrow = mask_of_head(sp.mask, bh, sp.H, sp.mask_heads, tq_n, tk_n);
    n_act = build_tile_list<kBwdWaves>(
        nblocks,
        [&](int b) -> unsigned {
          unsigned bits = 0;
#pragma unroll
          for (int qs_i = 0; qs_i < QB; ++qs_i)
#pragma unroll
            for (int w2 = 0; w2 < kBwdWaves; ++w2) {
              const int kw = k0 + w2 * kBwdKW;
              const int qs = q_begin + b * BQ + qs_i * 32;
              const bool reach = kw < N && qs < N && !(CAUSAL && qs + 31 < kw);
              if (reach && mrow[(qs / sp.block_q) * tk_n + kw / sp.block_k] != 0)
                bits |= 1u << (qs_i * kBwdWaves + w2);
            }
          return bits;
        },
        tl, tid, w, lane);
  } else {
    (void)sp;
  }
  auto block_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl.act[i]);
    else return i;
  };

  if (n_act > 0) load_block(q_begin + block_of(0) * BQ, 0);
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < n_act; ++it) {
    const int q0b = q_begin + block_of(it) * BQ;
    q_blk = q0b;
    const int st = it & 1;
    if (it + 1 < n_act) load_block(q_begin + block_of(it + 1) * BQ, st ^ 1);
    unsigned wbits = 0xFFu;
    if constexpr (SPARSE) wbits = (unsigned)__builtin_amdgcn_readfirstlane((int)tl.wbit[it]);

    const lds_u8* qs = C::q(smem, st);
    const lds_u8* dos = C::dout(smem, st);
    const lds_u8* nl_s = C::lse(smem, st);
    const lds_u8* dd_s = C::dd(smem, st);

    // every (query, key) pair of the block visible to this wave: no masks
    const bool full = (!CAUSAL || q0b >= kw0 + kBwdKW - 1) && (kw0 + kBwdKW <= N);
#pragma unroll
    for (int qs_i = 0; qs_i < QB; ++qs_i) {
      const int qsb = q0b + qs_i * 32;
      // every query of the sub-block precedes every key of the wave: nothing to add
      if (CAUSAL && !full && qsb + 31 < kw0) continue;
      if (SPARSE && !((wbits >> (qs_i * kBwdWaves + w)) & 1)) continue;   // block masked out
      __builtin_amdgcn_iglp_opt(2);   // interleave the exponentials with the products
      f32x16 s, dp;
      sdp(qs, dos, qs_i, s, dp);
      const int lim = (mykey >= N) ? 64 : (CAUSAL ? mykey - (qsb + 4 * g) : -1);
      softmax_grad(nl_s, dd_s, qs_i, s, dp, !full, lim);
      accumulate(qs, dos, qs_i, s, dp);
    }
    wait_vmem();
    __syncthreads();
  }

  // dK = scale * dK_acc, dV = dV_acc; lane holds key mykey, d = db*32 + acc_row(i, g).
  const rsrc_t rdk = make_rsrc(dK + head, head_bytes);
  const rsrc_t rdv = make_rsrc(dV + head, head_bytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t off = (uint32_t)mykey * G::R + (db * 32 + 8 * a + 4 * g) * (int)sizeof(T);
      store4<T>(rdk, off, dk_acc[db][4 * a] * scale, dk_acc[db][4 * a + 1] * scale, dk_acc[db][4 * a + 2] * scale,
                dk_acc[db][4 * a + 3] * scale);
      const float vs = DROP ? dpar.rs : 1.f;
      store4<T>(rdv, off, dv_acc[db][4 * a] * vs, dv_acc[db][4 * a + 1] * vs, dv_acc[db][4 * a + 2] * vs,
                dv_acc[db][4 * a + 3] * vs);
    }
}

// ---------------------------------------------------------------- 2b. dK, dV (bf16)
// Eight waves over 128 keys: waves w and w + 4 own the same 32 keys (slice
// w % 4) and take the first and the second 32-row query sub-block of every
// 64-row block, so each SIMD runs two waves of a workgroup.  K and V stay
// resident in LDS; at d = 128 each wave holds its K slice as B fragments in
// registers (read once) and reads its V fragments per block -- holding both
// would not leave room for two waves per SIMD.  At d = 64 (no dropout) two
// workgroups share a CU instead (kv_two_per_cu), and every operand is read
// from LDS where it is used.  Every LDS address is a
// per-lane offset computed once plus a compile-time constant: the block loop
// is unrolled over the two staging buffers, and blocks that cross no diagonal
// and no end of the sequence run a body without any masking.  At the end the
// two waves of a slice exchange partial sums through LDS: the first group
// finishes dK, the second dV.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;

template <int D>
struct KvCfg {
  using G = Tile<bf16, D>;
  static constexpr int BQ = 64;                         // query rows per block (2 sub-blocks)
  static constexpr int KTILE = kBwdBK * G::R;           // K (or V) rows of the workgroup
  static constexpr int QTILE = BQ * G::R;
  static constexpr int STAGE = 1024 + 2 * QTILE;       // -lse, D (1 KiB slot), Q, dO
  // [stage 0][stage 1][K][V]: stage-relative addresses fit the 16-bit
  // immediate offset of ds_read; K and V get a base register of their own.
  static constexpr int NL0 = 0;
  static constexpr int DD0 = 256;
  static constexpr int Q0 = 1024;
  static constexpr int DO0 = 1024 + QTILE;
  static constexpr int KOFF = 2 * STAGE;
  static constexpr int VOFF = KOFF + KTILE;
  static constexpr int BYTES = 2 * STAGE + 2 * KTILE;
  static constexpr int NACC = D / 32 * 16;              // accumulator registers per lane (dK or dV)
  static_assert(4 * NACC * 64 * 4 <= 2 * KTILE && 4 * NACC * 64 * 4 <= 2 * STAGE, "exchange fits");
  static_assert(STAGE + DO0 + 16 * G::R < 65536, "stage offsets fit the ds_read immediate");
};

// Two workgroups per CU at d = 64 (four waves per SIMD, at most 128
// registers): the second workgroup covers the first's waits on its staged
// blocks.  To fit, each wave reads its K fragments from LDS at every use
// instead of holding them, and reads its other operands without a
// one-step-ahead copy.  The dropout instantiations, which would spill at 128
// registers, keep one workgroup per CU and the d = 128 layout.
template <int D, bool DROP>
constexpr bool kv_two_per_cu() { return D == 64 && !DROP; }

template <int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kKvThreads, (kv_two_per_cu<D, DROP>() ? 4 : 1))
void fa_bwd_dkdv_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                             const bf16* __restrict__ dO, const float* __restrict__ dsum,
                             const float* __restrict__ nlse, bf16* __restrict__ dK, bf16* __restrict__ dV, int N,
                             int BH, int n_ktiles, int group, float scale, SparseArgs sp, DropParams dpar) {
  using M = Mfma<bf16>;
  using C = KvCfg<D>;
  using G = Tile<bf16, D>;
  using X = ExpDomain<bf16>;
  using Frag = M::Frag;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NDB = D / 32, NC = D / KC, BQ = C::BQ;
  // static, so that every LDS address is known at compile time (block-sparse:
  // the query-block list follows)
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[C::BYTES + (SPARSE ? kListBytes : 0)];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int slice = w & 3;                                   // 32-key slice
  const int grp = w >> 2;                                    // query sub-block of each block
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // heads grouped per XCD; causal: low key tiles (most work) first
  const WgOrder wo = wg_order(blockIdx.x, BH, n_ktiles, group);
  const int bh = wo.bh;
  const int kt = wo.rank;
  const int k0 = kt * kBwdBK;
  const int kw0 = k0 + slice * kBwdKW;
  const int mykey = kw0 + r32;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  // copies into LDS are issued with lds_dma*_async and waited for at the
  // end of each block (wait_vmem), so reads of the current block never wait
  // for the next block's copy
  const u32x4 rq = rsrc_words(Q + head, head_bytes);
  const u32x4 rk = rsrc_words(K + head, head_bytes);
  const u32x4 rv = rsrc_words(V + head, head_bytes);
  const u32x4 rdo = rsrc_words(dO + head, head_bytes);
  const u32x4 rnl = rsrc_words(nlse + (size_t)bh * N, (uint32_t)N * 4u);
  const u32x4 rdd = rsrc_words(dsum + (size_t)bh * N, (uint32_t)N * 4u);
  const float kfac = X::factor(scale);
  if constexpr (!DROP) (void)dpar;

  // Loop-invariant per-lane LDS offsets.  The swizzle depends on the row
  // modulo 16 only, so an offset computed for rows 0..31 holds for every
  // 16-row-aligned shift of them.
  //   qa[c]: A fragment (row r32 of this wave's query sub-block, k-chunk c)
  //   ka[c]: B fragment (row r32 of this wave's key slice) in the K tile
  //   tq[db][e]: transposed fragment reads (rows 4g + (j>>2) + 8e, columns
  //              db*32 + 16h + 4(j&3)) of this wave's query sub-block
  int qa[NC], ka[NC], tq[NDB][2];
  {
    const int j = lane & 15, h = (lane >> 4) & 1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qa[c] = G::off(grp * 32 + r32, c * KC + g * KPL);
      ka[c] = C::KOFF + G::off(slice * 32 + r32, c * KC + g * KPL);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) tq[db][e] = G::off(grp * 32 + 4 * g + (j >> 2) + 8 * e, db * 32 + 16 * h + 4 * (j & 3));
  }
  const int stat_off = (grp * 32 + 4 * g) * 4;

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv_acc[db] = f32x16{};
    dk_acc[db] = f32x16{};
  }

  auto load_block = [&](int q0b, int st) {
    lds_u8* sb = smem + st * C::STAGE;
    tile_to_lds_async<bf16, D, BQ, kKvWaves>(rq, sb + C::Q0, q0b, w, lane);
    tile_to_lds_async<bf16, D, BQ, kKvWaves>(rdo, sb + C::DO0, q0b, w, lane);
    if (w == 0) lds_dma4_async(rnl, sb + C::NL0, (q0b + lane) * 4);
    if (w == 1) lds_dma4_async(rdd, sb + C::DD0, (q0b + lane) * 4);
  };

  const int q_begin = CAUSAL ? k0 : 0;
  const int nblocks = (N - q_begin + BQ - 1) / BQ;

  // The query blocks this workgroup visits: all from q_begin (dense), or the
  // ones the block mask keeps for some wave (block-sparse; a wave's 32 keys
  // lie in one mask column since block_k is a multiple of 64, its 32-row
  // half of a block in one mask row since block_q is a multiple of 32).
  const TileList tl = tile_list_at(smem + C::BYTES);
  int n_act = nblocks;
  if constexpr (SPARSE) {
    const int tk_n = (N + sp.block_k - 1) / sp.block_k;
    const int tq_n = (N + sp.block_q - 1) / sp.block_q;
    const unsigned char* mrow = mask_of_head(sp.mask, bh, sp.H, sp.mask_heads, tq_n, tk_n);
    n_act = build_tile_list<kKvWaves>(
        nblocks,
        [&](int b) -> unsigned {
          unsigned bits = 0;
#pragma unroll
          for (int w2 = 0; w2 < kKvWaves; ++w2) {
            const int kw = k0 + (w2 & 3) * kBwdKW;
            const int qs = q_begin + b * BQ + (w2 >> 2) * 32;
            const bool reach = kw < N && qs < N && !(CAUSAL && qs + 31 < kw);
            if (reach && mrow[(qs / sp.block_q) * tk_n + kw / sp.block_k] != 0) bits |= 1u << w2;
          }
          return bits;
        },
        tl, tid, w, lane);
  } else {
    (void)sp;
  }
  auto block_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl.act[i]);
    else return i;
  };

  tile_to_lds_async<bf16, D, kBwdBK, kKvWaves>(rk, smem + C::KOFF, k0, w, lane);
  tile_to_lds_async<bf16, D, kBwdBK, kKvWaves>(rv, smem + C::VOFF, k0, w, lane);
  if (n_act > 0) load_block(q_begin + block_of(0) * BQ, 0);
  wait_vmem();
  __syncthreads();
  constexpr bool KREG = !kv_two_per_cu<D, DROP>();
  Frag kf[KREG ? NC : 1];   // this wave's K slice as B fragments, read once
  if constexpr (KREG) {
#pragma unroll
    for (int c = 0; c < NC; ++c) kf[c] = M::lds(smem + ka[c]);
  }

  // Visited query block number `it` (64 rows from q_begin + block_of(it) * 64)
  // from staging buffer ST; MASKED also handles the causal diagonal and keys
  // past the end of the sequence.
  auto block = [&](int it, auto st_c, auto masked_c) {
    constexpr int ST = decltype(st_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    const int q0b = q_begin + block_of(it) * BQ;
    if (it + 1 < n_act) load_block(q_begin + block_of(it + 1) * BQ, ST ^ 1);
    const int qsb = q0b + grp * 32;   // this wave's 32 query rows
    bool run = true, diag = false;
    if constexpr (MASKED) {
      run = !(CAUSAL && qsb + 31 < kw0);   // some query reaches some key of the slice
      diag = (CAUSAL && qsb < kw0 + kBwdKW - 1) || (kw0 + kBwdKW > N);
    }
    if constexpr (SPARSE) run = run && ((__builtin_amdgcn_readfirstlane((int)tl.wbit[it]) >> w) & 1);
    if (run) {
      const lds_u8* sb = smem + ST * C::STAGE;
      // DROP: this block's random bytes, generated before the products so
      // that the generator's temporaries are not live next to S and dP.
      u32x4 rb = {};
      if constexpr (DROP) rb = drop_bytes_queries(dpar.k0, dpar.k1, dpar.offset, (unsigned)bh, mykey, qsb, g, lane);
      // S = Q K^T and dP = dO V^T: rows = queries, column = this lane's key.
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (KREG) {
        Frag fq[2], fd[2], fv[2];
        fq[0] = M::lds(sb + C::Q0 + qa[0]);
        fd[0] = M::lds(sb + C::DO0 + qa[0]);
        fv[0] = M::lds(smem + ka[0] + C::KTILE);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int cur = c & 1;
          if (c + 1 < NC) {
            fq[cur ^ 1] = M::lds(sb + C::Q0 + qa[c + 1]);
            fd[cur ^ 1] = M::lds(sb + C::DO0 + qa[c + 1]);
            fv[cur ^ 1] = M::lds(smem + ka[c + 1] + C::KTILE);
          }
          s = M::mma(fq[cur], kf[c], s);
          dp = M::mma(fd[cur], fv[cur], dp);
          __builtin_amdgcn_sched_barrier(0);   // keep the reads one step ahead
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          s = M::mma(M::lds(sb + C::Q0 + qa[c]), M::lds(smem + ka[c]), s);
          dp = M::mma(M::lds(sb + C::DO0 + qa[c]), M::lds(smem + ka[c] + C::KTILE), dp);
        }
      }
      // P = ex(S*factor - lse), dS = P (dP - D); masked (key > query, or a key
      // past the end) -> P = 0.
      const int lim = (mykey >= N) ? 64 : (CAUSAL ? mykey - (qsb + 4 * g) : -1);
      // DROP: P o Z for dV (1 / (1 - t/256) applied at the end), and
      // dS = P (dP o Z / (1 - t/256) - D).
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 lz = *(const lds_f32x4*)(sb + C::NL0 + stat_off + 32 * a);
        const f32x4 dz = *(const lds_f32x4*)(sb + C::DD0 + stat_off + 32 * a);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          float p = X::ex(__builtin_fmaf(s[i], kfac, lz[b]));
          if constexpr (MASKED) {
            if (diag) p = (acc_row(i, 0) < lim) ? 0.f : p;
          }
          if constexpr (DROP) {
            const bool keep = drop_keep(rb, i, dpar.t);
            s[i] = keep ? p : 0.f;
            dp[i] = p * ((keep ? dp[i] * dpar.rs : 0.f) - dz[b]);
          } else {
            s[i] = p;
            dp[i] = p * (dp[i] - dz[b]);
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows.
      auto tr = [&](int base, int t, int db) {
        union { s16x4 h[2]; Frag f; } u;
        u.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + base + tq[db][0] + t * 16 * G::R));
        u.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + base + tq[db][1] + t * 16 * G::R));
        return u.f;
      };
#pragma unroll
      for (int t = 0; t < 32 / KC; ++t) {
        const Frag pb = M::pack(s, t);
        const Frag dsb = M::pack(dp, t);
        if constexpr (KREG) {
          Frag td[2], tqf[2];
          td[0] = tr(C::DO0, t, 0);
          tqf[0] = tr(C::Q0, t, 0);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int cur = db & 1;
            if (db + 1 < NDB) {
              td[cur ^ 1] = tr(C::DO0, t, db + 1);
              tqf[cur ^ 1] = tr(C::Q0, t, db + 1);
            }
            dv_acc[db] = M::mma(td[cur], pb, dv_acc[db]);
            dk_acc[db] = M::mma(tqf[cur], dsb, dk_acc[db]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dv_acc[db] = M::mma(tr(C::DO0, t, db), pb, dv_acc[db]);
            dk_acc[db] = M::mma(tr(C::Q0, t, db), dsb, dk_acc[db]);
          }
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Msk = std::integral_constant<bool, true>;
  using NoMsk = std::integral_constant<bool, false>;
  // Blocks 0 and 1 hold the causal diagonal of the 128 keys; a key tile that
  // reaches past the end of the sequence is masked throughout.  Block-sparse:
  // the visited blocks among those two (the list is in increasing order),
  // rounded up to an even count -- the masked body is correct for any block.
  const bool ktail = k0 + kBwdBK > N;
  int n_masked = ktail ? n_act : (CAUSAL ? min(2, n_act) : 0);
  if constexpr (SPARSE) {
    if (!ktail && CAUSAL) n_masked = (n_act > 0 && block_of(0) < 2) ? min(2, n_act) : 0;
  }
  int it = 0;
  for (; it < n_masked; it += 2) {
    block(it, S0{}, Msk{});
    if (it + 1 >= n_masked) { ++it; break; }
    block(it + 1, S1{}, Msk{});
  }
  // n_masked is even unless it covers every block, so the unmasked blocks
  // start on staging buffer 0.
  for (; it < n_act; it += 2) {
    block(it, S0{}, NoMsk{});
    if (it + 1 >= n_act) break;
    block(it + 1, S1{}, NoMsk{});
  }

  // Combine the two query halves of each slice: group 1 hands its dK partial to
  // group 0 (through the K/V area), group 0 hands its dV partial to group 1
  // (through the staging area); partials are laid out [slice][reg/4][lane][4].
  lds_u8* xk = smem + C::KOFF + slice * (C::NACC * 64 * 4);
  lds_u8* xv = smem + slice * (C::NACC * 64 * 4);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int off = ((db * 4 + a) * 64 + lane) * 16;
      if (grp == 1) {
        const f32x4 x = {dk_acc[db][4 * a], dk_acc[db][4 * a + 1], dk_acc[db][4 * a + 2], dk_acc[db][4 * a + 3]};
        *(lds_f32x4*)(xk + off) = x;
      } else {
        const f32x4 x = {dv_acc[db][4 * a], dv_acc[db][4 * a + 1], dv_acc[db][4 * a + 2], dv_acc[db][4 * a + 3]};
        *(lds_f32x4*)(xv + off) = x;
      }
    }
  __syncthreads();
  // Each wave adds its partner's partial, then writes its 32 rows whole
  // through the exchange slot it has just read, which no other wave touches.
  auto finish = [&](f32x16 (&acc)[NDB], lds_u8* x, float mul, bf16* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 o = *(const lds_f32x4*)(x + ((db * 4 + a) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * a + e] += o[e];
      }
    store_rows_bf16<D>(x, acc, mul, make_rsrc(dst + head, head_bytes), kw0, lane);
  };
  static_assert(32 * G::R <= C::NACC * 64 * 4, "a wave's rows fit its exchange slot");
  if constexpr (D == 128) {
    if (grp == 0) finish(dk_acc, xk, scale, dK);
    else finish(dv_acc, xv, DROP ? dpar.rs : 1.f, dV);
  } else {
    // d = 64 runs at 128 registers, where the staging spills: direct stores.
    const rsrc_t rdk = make_rsrc(dK + head, head_bytes);
    const rsrc_t rdv = make_rsrc(dV + head, head_bytes);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int xo = ((db * 4 + a) * 64 + lane) * 16;
        const uint32_t off = (uint32_t)mykey * G::R + (db * 32 + 8 * a + 4 * g) * 2;
        if (grp == 0) {
          const f32x4 o = *(const lds_f32x4*)(xk + xo);
          store4<bf16>(rdk, off, (dk_acc[db][4 * a] + o[0]) * scale, (dk_acc[db][4 * a + 1] + o[1]) * scale,
                       (dk_acc[db][4 * a + 2] + o[2]) * scale, (dk_acc[db][4 * a + 3] + o[3]) * scale);
        } else {
          const f32x4 o = *(const lds_f32x4*)(xv + xo);
          const float vs = DROP ? dpar.rs : 1.f;
          store4<bf16>(rdv, off, (dv_acc[db][4 * a] + o[0]) * vs, (dv_acc[db][4 * a + 1] + o[1]) * vs,
                       (dv_acc[db][4 * a + 2] + o[2]) * vs, (dv_acc[db][4 * a + 3] + o[3]) * vs);
        }
      }
  }
}

// ---------------------------------------------------------------- 3. dQ
// K/V stages of the bf16 dQ kernel: three at d = 64 (each 64-key tile then
// carries half the matrix work of d = 128, too little to cover the next
// tile's copy with one tile of prefetch; 48 KiB still fits three workgroups
// per CU), two at d = 128 (64 KiB, two workgroups per CU).
template <int D>
constexpr int dq_stages() { return D == 64 ? 3 : 2; }
constexpr int kDqWaves = 4;
constexpr int kDqQW = 32;                       // query rows per wave
constexpr int kDqBR = kDqWaves * kDqQW;         // query rows per workgroup
constexpr int kDqBC = 64;                       // keys per K/V tile
constexpr int kDqThreads = kDqWaves * 64;

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kDqThreads, sizeof(T) == 2 ? 2 : 1)
void fa_bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                      const T* __restrict__ dO, const float* __restrict__ dsum, const float* __restrict__ nlse,
                      T* __restrict__ dQ, int N, int BH, int n_qtiles, int group, float scale, SparseArgs sp,
                      DropParams dpar) {
  using M = Mfma<T>;
  using G = Tile<T, D>;
  using X = ExpDomain<T>;
  using Frag = typename M::Frag;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NKB = kDqBC / 32;
  constexpr int NDB = D / 32;
  constexpr int TILE = kDqBC * G::R;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;      // [K st0][K st1][V st0][V st1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // heads grouped per XCD; causal: longest first
  const WgOrder wo = wg_order(blockIdx.x, BH, n_qtiles, group);
  const int bh = wo.bh;
  const int qt = CAUSAL ? n_qtiles - 1 - wo.rank : wo.rank;
  const int q0 = qt * kDqBR;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  const rsrc_t rk = make_rsrc(K + head, head_bytes);
  const rsrc_t rv = make_rsrc(V + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const int qw0 = q0 + w * kDqQW;
  const int myq = qw0 + r32;
  const float kfac = X::factor(scale);

  // Q^T and dO^T as B operands (column = query, KPL d-values of group g);
  // this lane's lse (in the exponent domain) and D are scalars.
  Frag qf[D / KC], dof[D / KC];
#pragma unroll
  for (int c = 0; c < D / KC; ++c) {
    const uint32_t off = (uint32_t)myq * G::R + (c * KC + g * KPL) * (int)sizeof(T);
    qf[c] = M::load(rq, off);
    dof[c] = M::load(rdo, off);
  }
  const rsrc_t rnl = make_rsrc(nlse + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rdd = make_rsrc(dsum + (size_t)bh * N, (uint32_t)N * 4u);
  const float nl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rnl, myq * 4, 0, 0));
  const float dd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdd, myq * 4, 0, 0));
  if constexpr (!DROP) (void)dpar;

  const int kv_end = CAUSAL ? min(N, q0 + kDqBR) : N;
  const int ntiles = (kv_end + kDqBC - 1) / kDqBC;
  const int wave_last = CAUSAL ? min(ntiles - 1, (qw0 + kDqQW - 1) / kDqBC) : ntiles - 1;

  // The key tiles visited: all up to kv_end (dense) or those the block mask
  // keeps for some wave (block-sparse, as in the bf16 kernel).
  const TileList tl = tile_list_at(smem + 4 * TILE);
  int n_act = ntiles;
  if constexpr (SPARSE) {
    const int tk_n = (N + sp.block_k - 1) / sp.block_k;
    const int tq_n = (N + sp.block_q - 1) / sp.block_q;
    const unsigned char* mrow = mask_of_head(sp.mask, bh, sp.H, sp.mask_heads, tq_n, tk_n);
    n_act = build_tile_list<kDqWaves>(
        ntiles,
        [&](int jj) -> unsigned {
          const int kb = jj * kDqBC / sp.block_k;
          unsigned bits = 0;
#pragma unroll
          for (int w2 = 0; w2 < kDqWaves; ++w2) {
            const int qw = q0 + w2 * kDqQW;
            const bool reach = qw < N && !(CAUSAL && jj * kDqBC > qw + kDqQW - 1);
            if (reach && mrow[(qw / sp.block_q) * tk_n + kb] != 0) bits |= 1u << w2;
          }
          return bits;
        },
        tl, tid, w, lane);
  } else {
    (void)sp;
  }
  auto tile_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl.act[i]);
    else return i;
  };
  auto active = [&](int i) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane((int)tl.wbit[i]) >> w) & 1;
    else return i <= wave_last;
  };

  auto load_tile = [&](int j, int st) {
    tile_to_lds<T, D, kDqBC, kDqWaves>(rk, smem + st * TILE, j * kDqBC, w, lane);
    tile_to_lds<T, D, kDqBC, kDqWaves>(rv, smem + (2 + st) * TILE, j * kDqBC, w, lane);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  if (n_act > 0) load_tile(tile_of(0), 0);
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < n_act; ++it) {
    const int st = it & 1;
    const int j = tile_of(it);
    const int kv0 = j * kDqBC;
    if (it + 1 < n_act) load_tile(tile_of(it + 1), st ^ 1);
    if (active(it)) {
      const lds_u8* ks = smem + st * TILE;
      const lds_u8* vs = smem + (2 + st) * TILE;
      // S^T = K Q^T and dP^T = V dO^T: rows = keys, column = this lane's query.
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
#pragma unroll
      for (int c = 0; c < D / KC; ++c)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int off = G::off(kb * 32 + r32, c * KC + g * KPL);
          s[kb] = M::mma(M::lds(ks + off), qf[c], s[kb]);
          dp[kb] = M::mma(M::lds(vs + off), dof[c], dp[kb]);
        }
      const bool masked = (CAUSAL && kv0 + kDqBC - 1 > qw0) || (kv0 + kDqBC > N);
      if (masked) {
        // keys allowed for this lane: key <= min(N-1, myq) (causal) or key <= N-1
        const int last = CAUSAL ? min(N - 1, myq) : N - 1;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int lim = last - (kv0 + kb * 32 + 4 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = (acc_row(i, 0) > lim) ? kNegInf : s[kb][i];
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // DROP: dS = P (dP o Z / (1 - t/256) - D)
        u32x4 rb = {};
        if constexpr (DROP)
          rb = drop_bytes_keys(dpar.k0, dpar.k1, dpar.offset, (unsigned)bh, myq, kv0 + kb * 32, g, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // masked scores are -inf and kfac > 0, so P = 0 there
          const float p = X::ex(__builtin_fmaf(s[kb][i], kfac, nl));
          if constexpr (DROP) dp[kb][i] = p * ((drop_keep(rb, i, dpar.t) ? dp[kb][i] * dpar.rs : 0.f) - dd);
          else dp[kb][i] = p * (dp[kb][i] - dd);
        }
      }
      // dQ^T += K^T dS^T, dS^T straight from registers (B operand), K^T from
      // the K tile through the transpose read (A operand).
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 32 / KC; ++t) {
          const Frag dsb = M::pack(dp[kb], t);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            Frag a;
            if constexpr (sizeof(T) == 2) a = lds_tr_frag<D>(ks, kb * 32 + 16 * t, db * 32, lane);
            else a = M::lds(ks + G::off(kb * 32 + acc_row(t, g), db * 32 + r32));
            acc[db] = M::mma(a, dsb, acc[db]);
          }
        }
    }
    wait_vmem();
    __syncthreads();
  }

  // dQ = scale * acc; lane holds query myq, d = db*32 + acc_row(i, g).
  const rsrc_t rdq = make_rsrc(dQ + head, head_bytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4<T>(rdq, (uint32_t)myq * G::R + (db * 32 + 8 * a + 4 * g) * (int)sizeof(T), acc[db][4 * a] * scale,
                acc[db][4 * a + 1] * scale, acc[db][4 * a + 2] * scale, acc[db][4 * a + 3] * scale);
}

// bf16 dQ: the same sweep with every LDS address a per-lane offset computed
// once plus a compile-time constant (static LDS, the tile loop unrolled over
// the two staging buffers), masking only on the tiles that cross the diagonal
// or the end of the sequence, and operand reads issued one product ahead.
// The two 32-key halves of a tile are processed one after the other so that
// the first half's dS is already packed to bf16 while the second half's
// products run.
//
// PRE: this kernel also does the preprocess pass (it runs first then, before
// dK/dV): each lane forms D_i = do_i . o_i and -lse_i for its own query from O
// and lse, uses them, and writes them to the workspace for the dK/dV kernel.
// The sum follows the preprocess kernel's order exactly (8-element chunks,
// then the chunks 8, 4, 2 and 1 apart combined), so the gradients equal
// those of the staged entry points bit for bit.
template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool PRE>
__global__ __launch_bounds__(kDqThreads, 2)
void fa_bwd_dq_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                           const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ LSE,
                           float* __restrict__ dsum, float* __restrict__ nlse, bf16* __restrict__ dQ, int N, int BH,
                           int n_qtiles, int group, float scale, SparseArgs sp, DropParams dpar) {
  using M = Mfma<bf16>;
  using G = Tile<bf16, D>;
  using X = ExpDomain<bf16>;
  using Frag = M::Frag;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  constexpr int KPL = M::KPL, KC = M::KC;
  constexpr int NKB = kDqBC / 32;
  constexpr int NDB = D / 32, NC = D / KC;
  constexpr int TILE = kDqBC * G::R;
  // K/V stages: NST - 1 tiles in flight while one is consumed (three at
  // d = 64, whose tiles carry half the matrix work of d = 128)
  constexpr int NST = dq_stages<D>();
  constexpr int PER = 2 * (TILE / 1024) / kDqWaves;   // copy instructions per wave per K+V tile
  static_assert((NST - 2) * PER <= 63, "vmcnt is 6 bits");
  // [K stages][V stages] (block-sparse: then the tile list)
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[2 * NST * TILE + (SPARSE ? kListBytes : 0)];
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 5;
  const int r32 = lane & 31;

  // heads grouped per XCD; causal: longest first
  const WgOrder wo = wg_order(blockIdx.x, BH, n_qtiles, group);
  const int bh = wo.bh;
  const int qt = CAUSAL ? n_qtiles - 1 - wo.rank : wo.rank;
  const int q0 = qt * kDqBR;
  if constexpr (!SPARSE) (void)sp;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * G::R;
  const rsrc_t rq = make_rsrc(Q + head, head_bytes);
  // K/V tiles are copied with lds_dma16_async and waited for at the end of
  // each tile (wait_vmem), so reads of tile j never wait for tile j+1's copy
  const u32x4 rk = rsrc_words(K + head, head_bytes);
  const u32x4 rv = rsrc_words(V + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const int qw0 = q0 + w * kDqQW;
  const int myq = qw0 + r32;
  const float kfac = X::factor(scale);

  // Q^T and dO^T as B operands (column = query, KPL d-values of group g);
  // this lane's lse (in the exponent domain) and D are scalars.
  Frag qf[NC], dof[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t off = (uint32_t)myq * G::R + (c * KC + g * KPL) * 2;
    qf[c] = M::load(rq, off);
    dof[c] = M::load(rdo, off);
  }
  const rsrc_t rnl = make_rsrc(nlse + (size_t)bh * N, (uint32_t)N * 4u);
  const rsrc_t rdd = make_rsrc(dsum + (size_t)bh * N, (uint32_t)N * 4u);
  float nl, dd;
  if constexpr (PRE) {
    // lane group g holds the 8-element chunks t = 2c + g of its query's row
    const rsrc_t ro = make_rsrc(O + head, head_bytes);
    const rsrc_t rls = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
    float part[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const Frag of = M::load(ro, (uint32_t)myq * G::R + (c * KC + g * KPL) * 2);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)of[e] * (float)dof[c][e];
      part[c] = acc;
    }
    // chunks 8, 4 and 2 apart (c 4, 2 and 1 apart), then the partner lane's (1 apart)
#pragma unroll
    for (int h = NC / 2; h > 0; h >>= 1)
#pragma unroll
      for (int c = 0; c < h; ++c) part[c] = part[c] + part[c + h];
    dd = pair_sum(part[0]);
    nl = -X::from_lse(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rls, myq * 4, 0, 0)));
    if (g == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dd), rdd, myq * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nl), rnl, myq * 4, 0, 0);
    }
  } else {
    (void)O;
    (void)LSE;
    nl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rnl, myq * 4, 0, 0));
    dd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdd, myq * 4, 0, 0));
  }
  if constexpr (!DROP) (void)dpar;

  // Loop-invariant per-lane LDS offsets (the swizzle depends on the row
  // modulo 16 only): ka[c] = row r32, k-chunk c of a tile; tk[db][e] = the
  // transposed reads of rows 4g + (j>>2) + 8e, columns db*32 + 16h + 4(j&3).
  int ka[NC], tk[NDB][2];
  {
    const int j = lane & 15, h = (lane >> 4) & 1;
#pragma unroll
    for (int c = 0; c < NC; ++c) ka[c] = G::off(r32, c * KC + g * KPL);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) tk[db][e] = G::off(4 * g + (j >> 2) + 8 * e, db * 32 + 16 * h + 4 * (j & 3));
  }

  const int kv_end = CAUSAL ? min(N, q0 + kDqBR) : N;
  const int ntiles = (kv_end + kDqBC - 1) / kDqBC;
  const int wave_last = CAUSAL ? min(ntiles - 1, (qw0 + kDqQW - 1) / kDqBC) : ntiles - 1;

  // The key tiles this workgroup visits: all up to kv_end (dense) or the
  // ones the block mask keeps for some wave (block-sparse; each wave's 32
  // rows lie in one mask row since block_q is a multiple of 32, and each
  // 64-key tile in one mask column since block_k is a multiple of 64).  A
  // wave that reaches a tile has every one of its rows past the tile's first
  // key, so no row it computes has lse = -inf.
  const TileList tl = tile_list_at(smem + 2 * NST * TILE);
  int n_act = ntiles;
  if constexpr (SPARSE) {
    const int tk_n = (N + sp.block_k - 1) / sp.block_k;
    const int tq_n = (N + sp.block_q - 1) / sp.block_q;
    const unsigned char* mrow = mask_of_head(sp.mask, bh, sp.H, sp.mask_heads, tq_n, tk_n);
    n_act = build_tile_list<kDqWaves>(
        ntiles,
        [&](int j) -> unsigned {
          const int kb = j * kDqBC / sp.block_k;
          unsigned bits = 0;
#pragma unroll
          for (int w2 = 0; w2 < kDqWaves; ++w2) {
            const int qw = q0 + w2 * kDqQW;
            const bool reach = qw < N && !(CAUSAL && j * kDqBC > qw + kDqQW - 1);
            if (reach && mrow[(qw / sp.block_q) * tk_n + kb] != 0) bits |= 1u << w2;
          }
          return bits;
        },
        tl, tid, w, lane);
  }
  auto tile_of = [&](int i) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tl.act[i]);
    else return i;
  };
  auto active = [&](int i) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane((int)tl.wbit[i]) >> w) & 1;
    else return i <= wave_last;
  };

  auto load_tile = [&](int j, int st) {
    tile_to_lds_async<bf16, D, kDqBC, kDqWaves>(rk, smem + st * TILE, j * kDqBC, w, lane);
    tile_to_lds_async<bf16, D, kDqBC, kDqWaves>(rv, smem + (NST + st) * TILE, j * kDqBC, w, lane);
  };
  // Tile `it` has landed once at most the copies of the tiles issued after
  // it, up to NST - 2 of them, are outstanding (copies complete in issue
  // order).
  auto wait_tile = [&](int it) {
    if constexpr (NST > 2) {
      if (it + NST - 2 < n_act) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * PER) : "memory");
        return;
      }
    }
    wait_vmem();
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < n_act) load_tile(tile_of(i), i);
  // Take the compiler's waits for the Q, dO and statistics loads here, once:
  // at their first use inside the loop they would also drain the K/V copies
  // in flight.
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]), "+v"(dof[c]));
  asm volatile("" : "+v"(nl), "+v"(dd));
  if (n_act > 0) wait_tile(0);
  __syncthreads();

  // Visited tile number `it` (tile_of(it)) from staging buffer ST.
  auto tile = [&](int it, auto st_c, auto masked_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int KB = ST * TILE, VB = (NST + ST) * TILE;
    const int j = tile_of(it);
    const int kv0 = j * kDqBC;
    // the stage of tile it + NST - 1 held tile it - 1, read in the last iteration
    if (it + NST - 1 < n_act) load_tile(tile_of(it + NST - 1), (ST + NST - 1) % NST);
    if (!MASKED || active(it)) {
      bool msk = false;
      int last = 0;
      if constexpr (MASKED) {
        msk = (CAUSAL && kv0 + kDqBC - 1 > qw0) || (kv0 + kDqBC > N);
        last = CAUSAL ? min(N - 1, myq) : N - 1;   // keys allowed: key <= last
      }
      // S^T = K Q^T and dP^T = V dO^T for the 32 keys of half kb: rows = keys,
      // column = this lane's query; operand reads run one product ahead.
      auto sdp = [&](int kb, f32x16& s, f32x16& dp) {
        s = f32x16{};
        dp = f32x16{};
        Frag fk[2], fv[2];
        fk[0] = M::lds(smem + KB + kb * 32 * G::R + ka[0]);
        fv[0] = M::lds(smem + VB + kb * 32 * G::R + ka[0]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int cur = c & 1;
          if (c + 1 < NC) {
            fk[cur ^ 1] = M::lds(smem + KB + kb * 32 * G::R + ka[c + 1]);
            fv[cur ^ 1] = M::lds(smem + VB + kb * 32 * G::R + ka[c + 1]);
          }
          s = M::mma(fk[cur], qf[c], s);
          dp = M::mma(fv[cur], dof[c], dp);
        }
      };
      // P = ex(S*factor - lse) (masked scores are -inf and factor > 0, so
      // P = 0 there), dS = P (dP - D), packed to bf16 B fragments.
      auto softmax = [&](int kb, f32x16& s, f32x16& dp, Frag* ds, const u32x4& rb) {
        if constexpr (MASKED) {
          if (msk) {
            const int lim = last - (kv0 + kb * 32 + 4 * g);
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = (acc_row(i, 0) > lim) ? kNegInf : s[i];
          }
        }
        // DROP: dS = P (dP o Z / (1 - t/256) - D)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = X::ex(__builtin_fmaf(s[i], kfac, nl));
          if constexpr (DROP) dp[i] = p * ((drop_keep(rb, i, dpar.t) ? dp[i] * dpar.rs : 0.f) - dd);
          else dp[i] = p * (dp[i] - dd);
        }
        ds[0] = M::pack(dp, 0);
        ds[1] = M::pack(dp, 1);
      };
      // dQ^T += K^T dS^T: K^T through the transpose read (A operand), dS^T
      // straight from registers (B operand).
      auto tr = [&](int kb, int t, int db) {
        union { s16x4 h[2]; Frag f; } u;
        const int base = KB + (kb * 32 + 16 * t) * G::R;
        u.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + base + tk[db][0]));
        u.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + base + tk[db][1]));
        return u.f;
      };
      auto dq_mma = [&](int kb, const Frag* ds) {
        Frag fa[2];
        fa[0] = tr(kb, 0, 0);
#pragma unroll
        for (int n = 0; n < 2 * NDB; ++n) {
          const int cur = n & 1;
          if (n + 1 < 2 * NDB) fa[cur ^ 1] = tr(kb, (n + 1) / NDB, (n + 1) % NDB);
          acc[n % NDB] = M::mma(fa[cur], ds[n / NDB], acc[n % NDB]);
        }
      };
      Frag ds[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // DROP: the half's random bytes before its products (generator
        // temporaries not live next to S and dP)
        u32x4 rb = {};
        if constexpr (DROP)
          rb = drop_bytes_keys(dpar.k0, dpar.k1, dpar.offset, (unsigned)bh, myq, kv0 + kb * 32, g, lane);
        f32x16 st, dpt;
        sdp(kb, st, dpt);
        softmax(kb, st, dpt, ds[kb], rb);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) dq_mma(kb, ds[kb]);
    }
    if (it + 1 < n_act) wait_tile(it + 1);
    __syncthreads();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using Msk = std::integral_constant<bool, true>;
  using NoMsk = std::integral_constant<bool, false>;
  // Leading tiles that no wave needs to mask: keys below the workgroup's
  // first query (causal), or all whole tiles (non-causal).  Block-sparse:
  // every visited tile takes the masked body, which also skips the waves
  // the mask leaves out (the causal / tail masking inside is a uniform
  // branch taken only where needed).
  const int n_plain = SPARSE ? 0 : (CAUSAL ? min(ntiles, q0 / kDqBC) : N / kDqBC);
  int j = 0;
  if constexpr (NST == 2) {
    for (; j + 1 < n_plain; j += 2) {
      tile(j, S0{}, NoMsk{});
      tile(j + 1, S1{}, NoMsk{});
    }
    if (j < n_plain) {
      tile(j, S0{}, NoMsk{});
      ++j;
    }
    for (; j < n_act; ++j) {
      if (j & 1) tile(j, S1{}, Msk{});
      else tile(j, S0{}, Msk{});
    }
  } else {
    // The stage of visited tile j is j % NST; the plain run is unrolled over
    // the stages so that every LDS address is a compile-time offset.
    for (; j + NST - 1 < n_plain; j += NST) {
      tile(j, S0{}, NoMsk{});
      tile(j + 1, S1{}, NoMsk{});
      tile(j + 2, S2{}, NoMsk{});
    }
    for (; j < n_act; ++j) {
      const int st = j % NST;
      if (j < n_plain) {
        if (st == 0) tile(j, S0{}, NoMsk{});
        else if (st == 1) tile(j, S1{}, NoMsk{});
        else tile(j, S2{}, NoMsk{});
      } else {
        if (st == 0) tile(j, S0{}, Msk{});
        else if (st == 1) tile(j, S1{}, Msk{});
        else tile(j, S2{}, Msk{});
      }
    }
  }

  // dQ = scale * acc; lane holds query myq, d = db*32 + acc_row(i, g).
  const rsrc_t rdq = make_rsrc(dQ + head, head_bytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4<bf16>(rdq, (uint32_t)myq * G::R + (db * 32 + 8 * a + 4 * g) * 2, acc[db][4 * a] * scale,
                   acc[db][4 * a + 1] * scale, acc[db][4 * a + 2] * scale, acc[db][4 * a + 3] * scale);
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  const int BH = a.B * a.H;
  const size_t rows = (size_t)BH * a.N;
  const int n_ktiles = (a.N + kBwdBK - 1) / kBwdBK;
  const int n_qtiles = (a.N + kDqBR - 1) / kDqBR;
  SparseArgs sp;
  if constexpr (SPARSE) sp = SparseArgs{a.mask, a.H, a.mask_heads, a.block_q, a.block_k};
  // The whole bf16 backward runs dQ first, with the preprocess pass folded
  // into it (PRE), then dK/dV, which reads the statistics dQ wrote.
  if constexpr (sizeof(T) == 2) {
    if (stages == (kStagePre | kStageDkDv | kStageDq)) {
      hipLaunchKernelGGL((fa_bwd_dq_bf16_kernel<D, CAUSAL, SPARSE, DROP, true>), dim3(n_qtiles * BH),
                         dim3(kDqThreads), 0, stream, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout),
                         static_cast<const bf16*>(a.o), a.lse, a.dsum, a.nlse, static_cast<bf16*>(a.dq), a.N, BH,
                         n_qtiles, wg_group(n_qtiles, 32 * (D == 64 ? 3 : 2)), a.scale, sp, a.drop);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      stages = kStageDkDv;
    }
  }
  if (stages & kStagePre) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const size_t blocks = (rows + RPB - 1) / RPB;
    const dim3 grid((unsigned)(blocks < kPreMaxBlocks ? blocks : kPreMaxBlocks));
    hipLaunchKernelGGL((fa_bwd_pre_kernel<T, D>), grid, dim3(256), 0, stream, static_cast<const T*>(a.o),
                       static_cast<const T*>(a.dout), a.lse, a.dsum, a.nlse, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDkDv) {
    if constexpr (sizeof(T) == 2) {
      hipLaunchKernelGGL((fa_bwd_dkdv_bf16_kernel<D, CAUSAL, SPARSE, DROP>), dim3(n_ktiles * BH), dim3(kKvThreads),
                         0, stream, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout), a.dsum, a.nlse,
                         static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N, BH, n_ktiles,
                         wg_group(n_ktiles, 32 * ((kv_two_per_cu<D, DROP>()) ? 2 : 1)), a.scale, sp,
                         a.drop);   // 2 or 1 workgroups per CU
    } else {
      using C = BwdCfg<T, D>;
      constexpr int bytes = C::BYTES + (SPARSE ? list_bytes(kBwdListCap) : 0);
      auto kern = fa_bwd_dkdv_kernel<T, D, CAUSAL, SPARSE, DROP>;
      static const hipError_t attr_err =
          hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (attr_err != hipSuccess) return attr_err;
      hipLaunchKernelGGL(kern, dim3(n_ktiles * BH), dim3(kBwdThreads), bytes, stream,
                         static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                         static_cast<const T*>(a.dout), a.dsum, a.nlse, static_cast<T*>(a.dk),
                         static_cast<T*>(a.dv), a.N, BH, n_ktiles, wg_group(n_ktiles, 32), a.scale, sp, a.drop);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDq) {
    if constexpr (sizeof(T) == 2) {
      hipLaunchKernelGGL((fa_bwd_dq_bf16_kernel<D, CAUSAL, SPARSE, DROP, false>), dim3(n_qtiles * BH),
                         dim3(kDqThreads), 0, stream, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dout), nullptr, nullptr,
                         a.dsum, a.nlse, static_cast<bf16*>(a.dq), a.N, BH, n_qtiles,
                         wg_group(n_qtiles, 32 * (D == 64 ? 3 : 2)), a.scale, sp, a.drop);   // 3 / 2 workgroups per CU
    } else {
      constexpr int bytes = 4 * kDqBC * D * (int)sizeof(T) + (SPARSE ? kListBytes : 0);
      auto kern = fa_bwd_dq_kernel<T, D, CAUSAL, SPARSE, DROP>;
      static const hipError_t attr_err =
          hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (attr_err != hipSuccess) return attr_err;
      hipLaunchKernelGGL(kern, dim3(n_qtiles * BH), dim3(kDqThreads), bytes, stream, static_cast<const T*>(a.q),
                         static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<const T*>(a.dout),
                         a.dsum, a.nlse, static_cast<T*>(a.dq), a.N, BH, n_qtiles, wg_group(n_qtiles, 32),
                         a.scale, sp, a.drop);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Instantiations: dense (with and without dropout) and block-sparse (no dropout).
template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_c(const BwdArgs& a, int stages, hipStream_t s) {
  if (a.mask) return launch_bwd_t<T, D, CAUSAL, true, false>(a, stages, s);
  if (a.drop.on) return launch_bwd_t<T, D, CAUSAL, false, true>(a, stages, s);
  return launch_bwd_t<T, D, CAUSAL, false, false>(a, stages, s);
}

template <typename T, int D>
hipError_t launch_bwd_d(const BwdArgs& a, int stages, hipStream_t s) {
  return a.causal ? launch_bwd_c<T, D, true>(a, stages, s) : launch_bwd_c<T, D, false>(a, stages, s);
}

hipError_t launch_backward(const BwdArgs& a, int stages, hipStream_t s) {
  if (a.dtype == kDtypeBF16) return a.d == 64 ? launch_bwd_d<bf16, 64>(a, stages, s) : launch_bwd_d<bf16, 128>(a, stages, s);
  return a.d == 64 ? launch_bwd_d<float, 64>(a, stages, s) : launch_bwd_d<float, 128>(a, stages, s);
}

}  // namespace fa
