// fa_common.h -- device helpers shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA family):
//   * A operand (M x K): lane l supplies row m = l % 32 and KPL consecutive
//     k-elements of the lane group g = l / 32.
//   * B operand (K x N): lane l supplies column n = l % 32 and the same KPL
//     k-elements of group g.  Only the agreement between A and B matters for
//     the sum over k, so any k-assignment that both operands share is valid.
//   * C/D (32 x 32 fp32, 16 registers): register i of lane l holds
//     row acc_row(i, g) = 8*(i/4) + 4*g + (i%4), column l % 32.
// bf16 uses v_mfma_f32_32x32x16_bf16 (KPL = 8); fp32 uses
// v_mfma_f32_32x32x2_f32 (KPL = 1).  Accumulation is always fp32.
//
// Memory: every global access goes through a buffer resource that covers
// exactly one head's tensor, so rows past the end read as zero and writes
// past the end are dropped by the hardware range check -- no per-element
// branches.  K/V (forward) and Q/dO (backward) tiles move global -> LDS with
// buffer_load ... lds (no register staging) into row-major tiles whose
// 16-byte chunks are XOR-swizzled per row (see Tile below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Smallest exponent factor used: keeps masked scores (-inf) at -inf after the
// scaling even for scale = 0, while every finite score times it rounds to 0.
constexpr float kMinFactor = 0x1p-100f;

// Raw buffer resource over [base, base + bytes): gfx9 "raw" descriptor
// (stride 0, 32-bit data format word), range-checked per access.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;   // k elements per lane per instruction
  static constexpr int KC = 16;   // k per instruction
  using Frag = bf16x8;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // KPL consecutive elements at byte offset `off` of a buffer (16 bytes)
  __device__ __forceinline__ static Frag load(rsrc_t r, int off) {
    return __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ static Frag lds(const lds_u8* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) Frag*>(p);
  }
  // registers i = KPL*t .. KPL*t+KPL-1 of an accumulator, rounded to bf16 (RNE)
  __device__ __forceinline__ static Frag pack(const f32x16& x, int t) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)x[8 * t + e];
    return f;
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KC = 2;
  using Frag = float;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag load(rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  __device__ __forceinline__ static Frag lds(const lds_u8* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(p);
  }
  __device__ __forceinline__ static Frag pack(const f32x16& x, int t) { return x[t]; }
};

// Row of accumulator register i for lane group g (see the header comment).
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Row-major LDS tile of D elements per row, R = D*sizeof(T) bytes per row,
// no padding.  For bf16 the 16-byte chunk c of row r is stored at chunk
// c ^ swz(r).  The swizzle makes both access patterns conflict-free:
//   * 16 lanes reading one 16-byte chunk each from 16 consecutive rows
//     (MFMA operand fragments, ds_read_b128), and
//   * the transpose read ds_read_b64_tr_b16, where 32 lanes read 8 bytes each
//     from rows r0..r0+3 (r0 % 4 == 0) and 4 consecutive chunks.
// With 256-byte rows (d = 128) a row spans all 64 banks, so only the chunk
// index matters; with 128-byte rows (d = 64) rows of one parity share a half
// of the banks.  fp32 tiles are not swizzled.
template <typename T, int D> struct Tile {
  static constexpr int R = D * (int)sizeof(T);
  __device__ __forceinline__ static constexpr int swz(int row) {
    if constexpr (sizeof(T) != 2) return 0;
    else if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
  // byte offset of element (row, col); col * sizeof(T) must not straddle a chunk
  __device__ __forceinline__ static constexpr int off(int row, int col) {
    const int b = col * (int)sizeof(T);
    return row * R + (((b >> 4) ^ swz(row)) << 4) + (b & 15);
  }
};

// One global -> LDS transfer per lane: `bytes` (4 or 16) from byte offset
// `voff` of buffer `src` to dst + lane*bytes (dst wave-uniform).  Kept out of
// templates: the host pass rejects this builtin with dependent arguments.
__device__ __forceinline__ void lds_dma16(rsrc_t src, lds_u8* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(rsrc_t src, lds_u8* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)dst, 4, voff, 0, 0, 0);
}

// The same global -> LDS copy issued through inline assembly, on a buffer
// descriptor held as four words.  The compiler does not see this LDS write,
// so it never makes later LDS reads wait for it: the caller waits itself
// (wait_vmem) before the copied rows are read.  M0 holds the LDS address;
// one wait state separates its write from the copy.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)base;
  return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
__device__ __forceinline__ void lds_dma16_async(u32x4 src, const lds_u8* dst, int voff) {
  const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(voff), "s"(src) : "memory", "m0");
}
// lds_dma16_async with the non-temporal hint, for data that is read exactly
// once: a long stream of such copies runs markedly closer to the HBM peak.
__device__ __forceinline__ void lds_dma16_async_nt(u32x4 src, const lds_u8* dst, int voff) {
  const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(m), "v"(voff), "s"(src) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_async(u32x4 src, const lds_u8* dst, int voff) {
  const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m), "v"(voff), "s"(src) : "memory", "m0");
}

// Copy rows [row0, row0 + ROWS) of one head's [N, D] tensor (buffer `src`)
// into an LDS tile, spread over NW waves: each wave moves 1 KiB per
// instruction, lane i landing at byte 16*i of the wave's segment.  Rows past
// the end of the tensor read as zero.  Completion is tracked by vmcnt.
template <typename T, int D, int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds(rsrc_t src, lds_u8* tile, int row0, int w, int lane) {
  using G = Tile<T, D>;
  constexpr int SEGS = ROWS * G::R / 1024;
  static_assert(SEGS % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int r = 0; r < SEGS / NW; ++r) {
    const int s = w * (SEGS / NW) + r;
    const int o = s * 1024 + lane * 16;
    const int row = o / G::R;
    const int chunk = ((o % G::R) >> 4) ^ G::swz(row);
    lds_dma16(src, tile + s * 1024, (uint32_t)(row0 + row) * G::R + chunk * 16);
  }
}

// tile_to_lds through lds_dma16_async (see there for the waiting rule);
// STREAM: with the non-temporal hint (rows read once).
template <typename T, int D, int ROWS, int NW, bool STREAM = false>
__device__ __forceinline__ void tile_to_lds_async(u32x4 src, lds_u8* tile, int row0, int w, int lane) {
  using G = Tile<T, D>;
  constexpr int SEGS = ROWS * G::R / 1024;
  static_assert(SEGS % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int r = 0; r < SEGS / NW; ++r) {
    const int s = w * (SEGS / NW) + r;
    const int o = s * 1024 + lane * 16;
    const int row = o / G::R;
    const int chunk = ((o % G::R) >> 4) ^ G::swz(row);
    if constexpr (STREAM) lds_dma16_async_nt(src, tile + s * 1024, (uint32_t)(row0 + row) * G::R + chunk * 16);
    else lds_dma16_async(src, tile + s * 1024, (uint32_t)(row0 + row) * G::R + chunk * 16);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposed bf16 A fragment (M = columns, K = rows) from a swizzled tile:
// lane l gets column col0 + l%32 of rows row0 + 8a + 4g + b (a in {0,1},
// b in 0..3) -- the rows that accumulator registers 8t..8t+7 of lane group g
// hold for a 32-row block when row0 = 16t.  Two ds_read_b64_tr_b16: within
// each 16-lane group the instruction hands output lane 4p+q element e of
// input lane 4e+p's 4-element read (element q), i.e. a 4x16 transpose.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_frag(const lds_u8* tile, int row0, int col0, int lane) {
  using G = Tile<bf16, D>;
  const int j = lane & 15;
  const int h = (lane >> 4) & 1;
  const int g = lane >> 5;
  const int row = row0 + 4 * g + (j >> 2);
  const int col = col0 + 16 * h + 4 * (j & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  union { s16x4 s[2]; bf16x8 b; } u;
  u.s[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + G::off(row, col)));
  u.s[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + G::off(row + 8, col)));
  return u.b;
}

// Both lanes l and l^32 receive f(x[l & 31], x[(l & 31) + 32]) with the
// operands in the same order, so the two halves of a wave agree bit for bit.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exponent domain of the softmax.  bf16 inputs: base 2 with scale*log2(e)
// folded into one FMA and the hardware v_exp_f32.  fp32 inputs: base e with
// the accurate expf, so that the fp32 path keeps about 1e-7 relative error
// in every probability (the fp32 tolerance is 1e-5 absolute).
// kLazy: the running max used as the exponent shift is only raised when a
// new score exceeds it by more than this (in the domain's units), so the
// un-normalised probabilities stay <= 2^8 and the output accumulator is
// rescaled only on those rare tiles.
template <typename T> struct ExpDomain;
template <> struct ExpDomain<bf16> {
  static constexpr float kLazy = 8.0f;
  static constexpr float kToNat = kLn2;          // shift (log2 units) -> natural-log units
  __device__ __forceinline__ static float factor(float scale) { return fmaxf(scale * kLog2e, kMinFactor); }
  __device__ __forceinline__ static float ex(float x) { return fast_exp2(x); }
  __device__ __forceinline__ static float from_lse(float lse) { return lse * kLog2e; }
};
template <> struct ExpDomain<float> {
  static constexpr float kLazy = 8.0f * kLn2;
  static constexpr float kToNat = 1.0f;
  __device__ __forceinline__ static float factor(float scale) { return fmaxf(scale, kMinFactor); }
  __device__ __forceinline__ static float ex(float x) { return expf(x); }
  __device__ __forceinline__ static float from_lse(float lse) { return lse; }
};

// ---------------------------------------------------------------- launch order
// Workgroup b of a launch goes to XCD b % 8 (round-robin dispatch), and each
// of the 8 XCDs has its own L2.  A grid of (head, tile) workgroups therefore
// deals the heads out to the XCDs when B*H is a multiple of 8 (head h to XCD
// h % 8), and each XCD walks its heads in groups of `group`: the tiles of a
// group in order of decreasing work (rank 0 first), the group's heads
// interleaved.  The workgroups resident on one XCD at a time then share the
// K/V of a few heads in its L2, instead of taking one tile each of many
// heads.  Otherwise the heads are interleaved over the whole grid (rank
// b / BH).  Either way the map is a bijection onto [0, BH) x [0, n_tiles).
struct WgOrder {
  int bh, rank;
};
__device__ __forceinline__ WgOrder wg_order(int b, int BH, int n_tiles, int group) {
  if ((BH & 7) != 0) return {b % BH, b / BH};
  const int xcd = b & 7, i = b >> 3;
  const int hx = BH >> 3;                       // heads per XCD
  const int per_group = group * n_tiles;
  const int gi = i / per_group;
  const int hg = min(group, hx - gi * group);   // heads in this group (the last one may be short)
  const int r = i - gi * per_group;
  return {(gi * group + r % hg) * 8 + xcd, r / hg};
}
// Group size: at least 4 heads (one head at a time was ~1% slower at 16K,
// every resident workgroup then reading the same K/V lines at once), and for
// causal work enough that the last group's longest tile still ends with the
// rest of its XCD's work (slots = workgroups resident per XCD; checked with a
// list-scheduling simulation).  Measured on the causal forward: +4% at
// B*H = 128, N = 4096, +13% at B*H = 128, N = 8192, +48% at B*H = 512,
// N = 4096, unchanged at B*H = 32, N = 16384.
inline int wg_group(int n_tiles, int slots_per_xcd) {
  const int fit = (slots_per_xcd + n_tiles - 1) / n_tiles;
  return fit > 4 ? fit : 4;
}

// ---------------------------------------------------------------- block-sparse tile lists
// Block-sparse attention ("Overview of Flash Attention series", Block-sparse
// Flashattention) visits only the tiles a block mask keeps.  Each workgroup
// lists its tiles in LDS, in increasing order: act[i] = tile index,
// wbit[i] = which of its waves compute that tile (bit w; at most 8 waves).
// The mask is uint8 [mask_heads][ceil(N/block_q)][ceil(N/block_k)], non-zero
// keeps a block; mask_heads = 1 shares one mask, otherwise head h of every
// batch uses mask h.
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) int lds_i32;
// A list of up to CAP entries takes list_bytes(CAP) bytes of LDS: act (u16),
// wbit (u8), then 8 per-wave counters.  CAP = kListMax covers N <= 65536 in
// tiles of 64; lists of 32-row blocks take 2 * kListMax.
constexpr int kListMax = 1024;
constexpr int list_bytes(int cap) { return (3 * cap + 8 * 4 + 255) / 256 * 256; }
constexpr int kListBytes = list_bytes(kListMax);

struct TileList {
  lds_u16* act;
  lds_u8* wbit;
  lds_i32* cnt;
};
template <int CAP = kListMax>
__device__ __forceinline__ TileList tile_list_at(lds_u8* base) {
  return {(lds_u16*)base, base + 2 * CAP, (lds_i32*)(base + 3 * CAP)};
}
// The mask as the kernels take it (mask == nullptr: dense).
struct SparseArgs {
  const unsigned char* mask = nullptr;
  int H = 1, mask_heads = 1, block_q = 32, block_k = 64;
};
// This head's mask rows (each ceil(N/block_k) entries).
__device__ __forceinline__ const unsigned char* mask_of_head(const unsigned char* mask, int bh, int H, int mask_heads,
                                                             int tq_n, int tk_n) {
  return mask + (size_t)(mask_heads > 1 ? bh % H : 0) * tq_n * tk_n;
}
// Lists the tiles j in [0, n) with bits_of(j) != 0; every thread of the NW
// waves calls it.  Returns the number of listed tiles.
template <int NW, typename BitsFn>
__device__ int build_tile_list(int n, BitsFn bits_of, const TileList& tl, int tid, int w, int lane) {
  constexpr int NT = NW * 64;
  int n_act = 0;
  for (int base = 0; base < n; base += NT) {
    const int j = base + tid;
    const unsigned bits = j < n ? bits_of(j) : 0u;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(bits != 0);
    if (lane == 0) tl.cnt[w] = __builtin_popcountll(bal);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const int c = tl.cnt[w2];
      off += w2 < w ? c : 0;
      tot += c;
    }
    if (bits) {
      const int pos = n_act + off + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
      tl.act[pos] = (unsigned short)j;
      tl.wbit[pos] = (unsigned char)bits;
    }
    n_act += tot;
    __syncthreads();
  }
  return n_act;
}

// ---------------------------------------------------------------- dropout
// The dropout mask is never stored: every kernel regenerates the bits it
// needs from the counter-based generator Philox4x32-10 (Salmon, Moraes,
// Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).
// Element (i, j) of head bh takes byte 4 (i % 4) + (j % 4) of the 16 output
// bytes (words little-endian) at counter (j / 4, i / 4, bh, offset) with the
// 64-bit seed as key, and is dropped when that byte is < t.

// One Philox4x32-10 evaluation; the key (k0, k1) is wave-uniform.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const unsigned long long p0 = (unsigned long long)0xD2511F53u * c[0];
    const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c[2];
    c = u32x4{(unsigned)(p1 >> 32) ^ c[1] ^ k0, (unsigned)p1, (unsigned)(p0 >> 32) ^ c[3] ^ k1, (unsigned)p0};
  }
  return c;
}

// Within each quad of lanes (x = lane & 3), lane x holds row x of a 4 x 4
// matrix of words; returns column x (word a = row a's word x).  Two
// butterfly stages of quad-permute DPP moves.
__device__ __forceinline__ unsigned dpp_quad_xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ unsigned dpp_quad_xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ u32x4 quad_transpose(u32x4 m, int x) {
  const bool b0 = x & 1, b1 = x & 2;
  const unsigned r0 = dpp_quad_xor1(b0 ? m[0] : m[1]);
  const unsigned r1 = dpp_quad_xor1(b0 ? m[2] : m[3]);
  // column (x & 1) and (x & 1) + 2 of rows (x & ~1) and (x | 1)
  const unsigned t0 = b0 ? r0 : m[0], t1 = b0 ? m[1] : r0;
  const unsigned t2 = b0 ? r1 : m[2], t3 = b0 ? m[3] : r1;
  const unsigned q0 = dpp_quad_xor2(b1 ? t0 : t2);
  const unsigned q1 = dpp_quad_xor2(b1 ? t1 : t3);
  return b1 ? u32x4{q0, q1, t2, t3} : u32x4{t0, t1, q0, q1};
}

// 4 x 4 byte transpose within one lane: byte w of result word y = byte y of word w.
__device__ __forceinline__ u32x4 byte_transpose(u32x4 w) {
  const unsigned a = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);   // w0.b0 w1.b0 w0.b1 w1.b1
  const unsigned b = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);   // w0.b2 w1.b2 w0.b3 w1.b3
  const unsigned c = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const unsigned d = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(c, a, 0x05040100u), __builtin_amdgcn_perm(c, a, 0x07060302u),
               __builtin_amdgcn_perm(d, b, 0x05040100u), __builtin_amdgcn_perm(d, b, 0x07060302u)};
}

// Random bytes of the 16 accumulator entries a lane holds for one 32 x 32
// block, laid out so that entry i is byte (i & 3) of word (i >> 2).
// Rows along keys (S^T layout: lane = query `qi`, rows = keys k0 + acc_row(i, g)):
__device__ __forceinline__ u32x4 drop_bytes_keys(unsigned k0s, unsigned k1s, unsigned offset, unsigned bh, int qi,
                                                 int key0, int g, int lane) {
  const int x = lane & 3;
  const u32x4 c = {(unsigned)(key0 / 4 + 2 * x + g), (unsigned)qi >> 2, bh, offset};
  return quad_transpose(philox4x32_10(c, k0s, k1s), x);
}
// Rows along queries (S layout: lane = key `kj`, rows = queries q0 + acc_row(i, g)):
__device__ __forceinline__ u32x4 drop_bytes_queries(unsigned k0s, unsigned k1s, unsigned offset, unsigned bh, int kj,
                                                    int q0, int g, int lane) {
  const int x = lane & 3;
  const u32x4 c = {(unsigned)kj >> 2, (unsigned)(q0 / 4 + 2 * x + g), bh, offset};
  return quad_transpose(byte_transpose(philox4x32_10(c, k0s, k1s)), x);
}
__device__ __forceinline__ bool drop_keep(const u32x4& bytes, int i, unsigned t) {
  return ((bytes[i >> 2] >> (8 * (i & 3))) & 0xFFu) >= t;
}

// Store 4 consecutive fp32 values, rounded to T, at byte offset `off` of a buffer.
template <typename T>
__device__ __forceinline__ void store4(rsrc_t r, int off, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
  } else {
    f32x4 v = {a, b, c, d};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  }
}

// Store a wave's 32 output rows, rows row0..row0+31 of a [N, D] bf16 tensor
// (buffer `dst`), from the transposed accumulator layout: acc[db] register i
// of lane l is element (row l % 32, column db*32 + acc_row(i, g)), times
// `mul`.  Stored directly, every instruction would write 16-byte pieces of
// 32 rows; instead the wave transposes the block through `buf` (its own
// 32*D*2 bytes of idle LDS, laid out as a swizzled Tile) and writes whole
// rows, 16 bytes per lane.  Rows past the end are dropped by the range check.
template <int D>
__device__ __forceinline__ void store_rows_bf16(lds_u8* buf, const f32x16 (&acc)[D / 32], float mul, rsrc_t dst,
                                                int row0, int lane) {
  using G = Tile<bf16, D>;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  const int g = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const bf16x4 x = {(bf16)(acc[db][4 * a] * mul), (bf16)(acc[db][4 * a + 1] * mul),
                        (bf16)(acc[db][4 * a + 2] * mul), (bf16)(acc[db][4 * a + 3] * mul)};
      *(lds_bf16x4*)(buf + G::off(r32, db * 32 + 8 * a + 4 * g)) = x;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int LPR = G::R / 16;   // lanes per row
  constexpr int RPI = 64 / LPR;    // rows per store
  const int chunk = lane % LPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = lane / LPR + RPI * i;
    const u32x4 x = *(const lds_u32x4*)(buf + row * G::R + ((chunk ^ G::swz(row)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(x, dst, (uint32_t)(row0 + row) * G::R + chunk * 16, 0, 0);
  }
}

}  // namespace fa
