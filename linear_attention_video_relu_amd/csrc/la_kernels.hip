// HIP kernels for block-causal ReLU linear attention with RoPE on gfx950.
//
// Three kernels make one forward pass ("Implementing Block Causal Linear
// Attention for Long Video Generation with Sana", sections "The Linear
// Attention Kernel" and "Chunk-Wise Causality"):
//
//   k_block_state  reads K and V once.  For a two-head group and a chunk of one
//                  block it forms phi(k), rotates it, and accumulates the partial
//                  state S_c = V^T . R phi(K) on MFMA (fp32 accumulate) and the
//                  un-rotated key sum z_c = sum phi(k).
//   k_prefix       sums the chunk partials of each block, in a fixed order, and
//                  writes the inclusive prefix Sbar_j, zbar_j of every block,
//                  starting from an optional carried state (streaming) and
//                  optionally writing the final state back (save).
//   k_readout      reads Q once, forms phi(q), the normaliser zbar_j . phi(q) +
//                  eps from un-rotated phi(q), rotates phi(q), multiplies by
//                  Sbar_j on MFMA and writes out = num / den.
//
// Data in HBM: q, k, v, out are (B, N, H, D) row-major with D = 32 or 64.  A
// workgroup owns 64 channels of every token row (a pair of heads at D = 32,
// one head at D = 64): 128 contiguous bytes in bf16 (256 in fp32), so a lane
// moves 16-byte pieces of fully used 128-byte lines.  Q, K, V and out are reached through buffer resources that span one
// workgroup's token range: the hardware range check turns reads past the end
// into zeros and drops writes past the end, so ragged tails need no branches,
// and lane offsets stay 32-bit.
//
// bf16 arithmetic: bf16 MFMA operands that are not exact bf16 values (the
// rotated keys and queries, the prefix state) are split as x = hi + lo with
// both parts bf16 (hi rounded to nearest, lo the rounded remainder), and the
// products hi.hi + hi.lo + lo.hi are accumulated in fp32, so each operand
// carries ~17 significant bits instead of 8.
// fp32 inputs use the fp32 MFMA (v_mfma_f32_*_f32) and are exact fp32 products.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "la_internal.h"

namespace lavr {
namespace {

constexpr int D = 32;                // channels of one lane chunk's half (a head at head dim 32)
constexpr int NT = 256;              // threads of the state and readout workgroups
constexpr int kReadAlBytes = 2 * 8 * 64 * 16;   // head dim 64, bf16: Sbar hi and lo tiles of a readout workgroup
constexpr int kReadZBytes = 2 * 2 * 4 * 16;     // packed path: zbar hi and lo slices of a readout workgroup (2 heads or halves)
constexpr int STEP = 64;             // tokens per step of the state kernel
constexpr int TCOLS = 2 * D;         // an LDS tile row holds two heads
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer: 32-bit data, range checked
// Cache policy of the streaming q/k/v loads and of the large output stores
// (out, dq, dk, dv, the convolution's y): 0 = default, 2 = non-temporal.
// Non-temporal output stores keep a call's written tensors from sitting dirty
// in L2/MALL, where their write-back competed with the next kernel's loads
// (block-state kernel after a readout: 0.636 -> 0.599 ms); non-temporal loads
// were slower (0.676 ms).
#ifndef LAVR_LOAD_CPOL
#define LAVR_LOAD_CPOL 0
#endif
#ifndef LAVR_STORE_CPOL
#define LAVR_STORE_CPOL 2
#endif
// k_bw_q with bf16 inputs: 16-token groups of q/g loads in flight per wave, at
// head dim 32 and 64.  A third group took the minute backward (d 32) from 2.91
// to 2.89 ms and measured the same at 64; fp32 inputs keep two (a third spills
// at 2 waves per SIMD).
#ifndef LAVR_BWQ_PF
#define LAVR_BWQ_PF 3
#endif
#ifndef LAVR_BWQ_PF64
#define LAVR_BWQ_PF64 2
#endif
#ifndef LAVR_STATE_PF
#define LAVR_STATE_PF 2   // block-state: 64-token steps of K/V loads in flight
#endif
#ifndef LAVR_READ_PF
#define LAVR_READ_PF 2    // readout: 16-token groups of Q loads in flight per wave
#endif

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef short s16x2 __attribute__((ext_vector_type(2)));

// Token position bookkeeping shared by the kernels: how to split a token index
// into (frame, row, col), and the step that advances it by 64 tokens.
struct PosArgs {
  int tpf, gw, ghd;          // tokens per frame, row length, rows per frame
  int adv_f, adv_r, adv_c;   // 64 tokens = adv_f frames + adv_r rows + adv_c tokens
  long long t0;              // frame offset (frames already streamed)
  uint64_t mag_tpf, mag_gw;
};

struct StateArgs {
  const void* k;
  const void* v;
  float* part;
  const float* scale;        // normalised k: per-token 1 / rms of the token's k row
  const float* gamma;        // normalised k: per-channel weight (H * head_dim floats)
  int H, N, L, L0, nb, cpb, Tc, hg;   // L0: tokens of the first block
  int row_in;                // elements from one token row of k (and v) to the next
  PosArgs pos;
  RopeDev rope;
  // Fingerprint of what the block prefixes are formed from, stored in the
  // workspace header for the backward that reuses them.
  uint64_t* fp_dst;
  uint64_t fp0, fp1;
};

struct PrefixArgs {
  const float* part;
  float* prefix;
  const float* S_init;
  const float* z_init;
  float* S_save;
  float* z_save;
  int H, nb, cpb;
  int hd, rec;               // head dim, floats per record (hd * hd + hd)
  int rev;                   // 1: sums over blocks j >= i (last block first)
};

struct ReadArgs {
  const void* q;
  void* out;
  const float* prefix;
  const float* scale;        // normalised q: per-token 1 / rms of the token's q row
  const float* gamma;        // normalised q: per-channel weight (H * head_dim floats)
  float eps;
  int H, N, L, L0, nb, rpb, Tr, hg;   // L0: tokens of the first block
  int row_in;                // elements from one token row of q to the next
  uint64_t mag_hg, mag_rpb;  // floor(2^42 / hg) + 1, floor(2^42 / rpb) + 1 (fast_div)
  PosArgs pos;
  RopeDev rope;
};

// ------------------------------------------------------------------ helpers

// Chunk partial records are stored chunk-major: record (chunk ci, batch row *
// H + head bh) at ci * BH + bh, BH = batch rows * H.  The workgroups that
// finish together (the head groups of one chunk index) then write one
// contiguous range; a head-major layout scattered those writes across the
// workspace, and the write bursts slowed the K/V read stream around them.
__device__ __forceinline__ size_t part_rec(size_t bh, int ci, size_t BH) { return (size_t)ci * BH + bh; }

__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint64_t mag) {
  // floor(n / d) with mag = floor(2^42 / d) + 1; exact while n * d < 2^42.
  return (uint32_t)(((uint64_t)n * mag) >> 42);
}

// Two floats rounded to bf16 (nearest, ties to even; v_cvt_pk_bf16_f32), packed
// low = a, high = b.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Split 8 floats into bf16 operands hi = rne(x) and lo = rne(x - hi); the pair
// holds x to about 2^-17 relative.
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = pack_bf16(x[2 * i], x[2 * i + 1]);
    hi[i] = h;
    lo[i] = pack_bf16(x[2 * i] - __uint_as_float(h << 16), x[2 * i + 1] - __uint_as_float(h & 0xffff0000u));
  }
}

// split8 with the remainders formed by v_dot2c_f32_bf16: x - hi is the dot
// product of the packed hi pair with (-1, 0) or (0, -1), accumulated onto x.
// The products are exact and x - hi is representable in fp32, so the result
// is the exact remainder in one instruction, where a subtraction needs the hi
// part widened first: four instructions per pair instead of six.  Used where
// the instruction count matters (the readout's packed path).
//
// The unused half of each multiplier is -0, not +0: a pair with a zero high
// half is encoded as an inline constant, which v_dot2c reads as the fp32 value
// (1.0 -> 0x3f800000, the pair (0, 1)); a literal is read bit for bit.  x - h
// plus -0 * h' is still exactly x - h.
__device__ __forceinline__ void split8d(const float* x, u32x4& hi, u32x4& lo) {
  const bf16x2 m0 = __builtin_bit_cast(bf16x2, 0x8000bf80u);   // (-1, -0)
  const bf16x2 m1 = __builtin_bit_cast(bf16x2, 0xbf808000u);   // (-0, -1)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = pack_bf16(x[2 * i], x[2 * i + 1]);
    hi[i] = h;
    const bf16x2 hb = __builtin_bit_cast(bf16x2, h);
    lo[i] = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(hb, m0, x[2 * i], false),
                      __builtin_amdgcn_fdot2_f32_bf16(hb, m1, x[2 * i + 1], false));
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// First token of block j when the first block holds L0 tokens and every later
// one L.
__device__ __forceinline__ int block_start(int j, int L0, int L) { return j == 0 ? 0 : L0 + (j - 1) * L; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_WORD3);
}

// ------------------------------------------------------------ lane chunks
//
// Both the block-state loader and the readout give a lane channels 8c .. 8c+7
// (c = 0..3) of one token, for each of the two heads of its group.  A chunk of
// 8 elements is one 16-byte load in bf16 and two in fp32.

template <typename T> struct Raw8 { u32x4 r[sizeof(T) / 2]; };

template <typename T>
__device__ __forceinline__ Raw8<T> bload8(__amdgpu_buffer_rsrc_t rs, int off) {
  Raw8<T> o;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) o.r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, LAVR_LOAD_CPOL);
  return o;
}

// phi = ReLU on the raw bits (a sign bit set means <= 0; the integer max with 0
// clears it), then widen to fp32.
__device__ __forceinline__ void relu_widen(const Raw8<uint16_t>& r, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copy the element to a scalar first: bit-casting a subscripted vector
    // element directly reads element 0 with this compiler
    const uint32_t ri = r.r[0][i];
    const s16x2 z = {0, 0};
    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, ri), z));
    x[2 * i] = __uint_as_float(w << 16);
    x[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}
// Normalised input: x = phi(s * gamma * raw) for a token scale s = 1 / rms and
// the channels' weights; the weight may be negative, so phi comes last.
__device__ __forceinline__ void norm_relu_widen(const Raw8<uint16_t>& r, const float* gam, float s, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ri = r.r[0][i];
    x[2 * i] = __uint_as_float(ri << 16);
    x[2 * i + 1] = __uint_as_float(ri & 0xffff0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = fmaxf(x[i] * (s * gam[i]), 0.f);
}
__device__ __forceinline__ void norm_relu_widen(const Raw8<float>& r, const float* gam, float s, float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = fmaxf(__uint_as_float(r.r[i >> 2][i & 3]) * (s * gam[i]), 0.f);
}

// The 8 weights of channels c0 .. c0+7 (zeros for a half that holds no head).
__device__ __forceinline__ void load_gamma8(const float* gamma, int c0, bool live, float* g) {
  const float* src = gamma + (live ? c0 : 0);    // a dead half reads channel 0 and drops it
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g[i] = live ? a[i] : 0.f;
    g[4 + i] = live ? b[i] : 0.f;
  }
}

__device__ __forceinline__ void relu_widen(const Raw8<float>& r, float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    x[i] = __uint_as_float((uint32_t)__builtin_elementwise_max((int)r.r[i >> 2][i & 3], 0));
}

// Two transposing LDS reads (ds_read_b64_tr_b16) at element offsets e0 and
// e1 of a bf16 tile, joined into one 8-element MFMA operand.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ u32x4 tr_pair(const T* tile, int e0, int e1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + e0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + e1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// --------------------------------------------------------------------- RoPE
//
// A workgroup stages the rows of the rotary table it needs in LDS: the t rows
// of the frames its tokens span, then the whole h and w sections.  Pair gp of
// a head (channels 2gp, 2gp+1) reads (cos, sin) at base + pos * stride, with
// pos the token's local frame, row or column depending on its section.

struct TabWindow {
  int f_lo;   // first local frame staged
  int nf;     // frames staged
};

// Rotary entry for rotating a packed bf16 pair (a, b) = (x_2i, x_2i+1) with
// v_dot2_f32_bf16 (exact bf16 products, fp32 sum).  cos and sin are split into
// bf16 parts c = ch + cl, s = sh + sl (ch, sh rounded to nearest, cl, sl the
// rounded remainders, together ~2^-17 relative), and
//   a c - b s = dot(a b, ch -sh) + dot(a b, cl -sl),
//   a s + b c = dot(a b, sh  ch) + dot(a b, sl  cl).
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ u32x4 rope_words(float2 cs) {
  const float ch = bf16_round(cs.x), sh = bf16_round(cs.y);
  const float cl = cs.x - ch, sl = cs.y - sh;
  return u32x4{pack_bf16(ch, -sh), pack_bf16(cl, -sl), pack_bf16(sh, ch), pack_bf16(sl, cl)};
}

// (frame, row, col) of a lane's token, advanced 64 tokens at a time without
// divisions: the carries are at most one row and one frame per step.
struct TokPos {
  int f, row, col;
  __device__ void init(int n, const PosArgs& p) {
    f = (int)fast_div((uint32_t)n, p.mag_tpf);
    const int rem = n - f * p.tpf;
    row = (int)fast_div((uint32_t)rem, p.mag_gw);
    col = rem - row * p.gw;
  }
  __device__ void advance(const PosArgs& p) {
    col += p.adv_c;
    const bool c1 = col >= p.gw;
    col = c1 ? col - p.gw : col;
    row += p.adv_r + (int)c1;
    const bool c2 = row >= p.ghd;
    row = c2 ? row - p.ghd : row;
    f += p.adv_f + (int)c2;
  }
};

// Per lookup: byte offset in the staged window = base + fl * sf + row * sr +
// col * sc, where only the stride of the lookup's own section is non-zero (no
// per-lane branches); ESZ is the window's entry size (8 bytes for (cos, sin)
// pairs, 16 for rope_words), folded into base and the strides so that a
// lookup is three 24-bit multiply-adds.
// P2: every section has an even number of pairs, so the pairs (4c, 4c+1) and
// (4c+2, 4c+3) share a section, sit side by side in the table, and one LDS
// read fetches a couple (two for rope_words); otherwise each pair is read on
// its own.
template <bool P2, int ESZ = 8>
struct RopeLane {
  static constexpr int NL = P2 ? 2 : 4;   // lookups per lane
  int base[NL], sf[NL], sr[NL], sc[NL];

  __device__ void init(const RopeDev& r, const TabWindow& w, int c) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int gp = 4 * c + (P2 ? 2 * i : i);
      const bool in_t = gp < r.pt, in_h = !in_t && gp < r.pt + r.ph, in_w = !in_t && !in_h;
      base[i] = ESZ * (in_t ? gp : (in_h ? w.nf * r.pt + (gp - r.pt) : w.nf * r.pt + r.gh * r.ph + (gp - r.pt - r.ph)));
      sf[i] = in_t ? ESZ * r.pt : 0;
      sr[i] = in_h ? ESZ * r.ph : 0;
      sc[i] = in_w ? ESZ * r.pw : 0;
    }
  }

  __device__ int off(int i, int fl, const TokPos& tp) const {
    return __umul24(fl, sf[i]) + (__umul24(tp.row, sr[i]) + (__umul24(tp.col, sc[i]) + base[i]));
  }

  // (cos, sin) of the lane's 4 pairs at the token's local frame (clamped into
  // the staged window, so tokens past the range read valid rows), row and column.
  __device__ void fetch(const float2* lds, const TokPos& tp, const TabWindow& w, float2* cs) const {
    static_assert(ESZ == 8, "a (cos, sin) window has 8-byte entries");
    const int fl = min(tp.f - w.f_lo, w.nf - 1);
    const char* base_p = reinterpret_cast<const char*>(lds);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const char* e = base_p + off(i, fl, tp);
      if constexpr (P2) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(e);
        cs[2 * i] = make_float2(v[0], v[1]);
        cs[2 * i + 1] = make_float2(v[2], v[3]);
      } else {
        cs[i] = *reinterpret_cast<const float2*>(e);
      }
    }
  }

  // The same lookups in a window staged as rope_words: T[p] holds the
  // rope_words of the lane's pair p.
  __device__ void fetch16(const u32x4* lds, const TokPos& tp, const TabWindow& w, u32x4* T) const {
    static_assert(ESZ == 16, "a rope_words window has 16-byte entries");
    const int fl = min(tp.f - w.f_lo, w.nf - 1);
    const char* base_p = reinterpret_cast<const char*>(lds);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const u32x4* e = reinterpret_cast<const u32x4*>(base_p + off(i, fl, tp));
      if constexpr (P2) {
        T[2 * i] = e[0];
        T[2 * i + 1] = e[1];
      } else {
        T[i] = e[0];
      }
    }
  }
};

// phi = ReLU of 8 packed bf16 values, kept packed (integer max with 0 clears
// every value whose sign bit is set).
__device__ __forceinline__ u32x4 relu_pk(u32x4 r) {
  const s16x2 z = {0, 0};
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ri = r[i];
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, ri), z));
  }
  return o;
}

// Rotate the 8 packed values of p (pairs p[i]) with their rope_words T[i]
// into fp32 x.
// dot(a, b) of two packed bf16 pairs with a zero addend.  The builtin would
// become the accumulating v_dot2c_f32_bf16 after a register cleared to zero;
// the three-operand form takes the zero as an inline constant.
__device__ __forceinline__ float dot2_bf16_z(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ void rotate_pk(const u32x4& p, const u32x4* T, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pi = p[i];
    const bf16x2 ab = __builtin_bit_cast(bf16x2, pi);
    const uint32_t w0 = T[i][0], w1 = T[i][1], w2 = T[i][2], w3 = T[i][3];
    x[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(ab, __builtin_bit_cast(bf16x2, w1), dot2_bf16_z(pi, w0), false);
    x[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(ab, __builtin_bit_cast(bf16x2, w3), dot2_bf16_z(pi, w2), false);
  }
}

__device__ __forceinline__ void rotate8(float* x, const float2* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * cs[i].x - b * cs[i].y;
    x[2 * i + 1] = a * cs[i].y + b * cs[i].x;
  }
}

// Normaliser of the packed paths: the MFMA's A operand holds zbar's hi part in
// rows 0-7 and its lo part in rows 8-15, so lane l (rows 4(l/16)..) holds
// hi . phi(q) below lane 32 and lo . phi(q) from lane 32 on, for token l mod
// 16; their sum (the same in both lanes) is the token's zbar . phi(q).
__device__ __forceinline__ float den_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Sum over the four lanes l, l^16, l^32, l^48 that hold one token's chunks.
__device__ __forceinline__ float sum4_lanes(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the 16 lanes of a wave that share (lane mod 4): two DPP rotations
// inside each 16-lane row (row_ror 4, 8), then the four rows.
__device__ __forceinline__ float sum16_lanes_mod4(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
  return sum4_lanes(v);
}

// Rotary window staged in two phases: the global reads go to registers
// first, so that a prologue can issue its other loads before the LDS writes
// wait for these (with at most PER entries per thread in registers; a larger
// window loads the rest in commit).  commit() writes (cos, sin) pairs,
// commit16() the same pairs as rope_words.
struct TabStage {
  static constexpr int PER = 4;   // entries a thread holds in registers
  float2 v[PER];
  int nt, tot;
  TabWindow w;
  const float2* tab;
  int tb, hb;                     // table index of the window's first t row, of the h/w rows
  // Table index of window entry i (the t rows, then the h and w sections).
  __device__ int src(int i) const { return i + (i < nt ? tb : hb - nt); }

  __device__ void issue(const RopeDev& r, long long t0, int n0, int n1, uint64_t mag_tpf) {
    w = TabWindow{0, 0};
    nt = tot = 0;
    if (r.table == nullptr || n1 <= n0) return;
    w.f_lo = (int)fast_div((uint32_t)n0, mag_tpf);
    w.nf = (int)fast_div((uint32_t)(n1 - 1), mag_tpf) - w.f_lo + 1;
    tab = reinterpret_cast<const float2*>(r.table);
    tb = (int)(t0 + w.f_lo) * r.pt;
    hb = r.max_frames * r.pt;
    nt = w.nf * r.pt;
    tot = nt + r.gh * r.ph + r.gw * r.pw;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < tot) v[k] = tab[src(i)];
    }
  }
  __device__ void commit(float2* lds) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < tot) lds[i] = v[k];
    }
    for (int i = threadIdx.x + PER * NT; i < tot; i += NT) lds[i] = tab[src(i)];
  }
  // The same window written as rope_words (16 bytes per pair).
  __device__ void commit16(u32x4* lds) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x + k * NT;
      if (i < tot) lds[i] = rope_words(v[k]);
    }
    for (int i = threadIdx.x + PER * NT; i < tot; i += NT) lds[i] = rope_words(tab[src(i)]);
  }
};

// --------------------------------------------------------- k_block_state
//
// Grid: x = chunk * hg + head group, y = batch.  256 threads.  A workgroup owns
// 64 channels (128 bytes of bf16) of every token row: two heads at head dim 32,
// one head at 64, whose two 32-channel halves take the place of the two heads
// in the loads and tiles.  Each 64-token step: thread t loads channels
// 8(t&3) .. +7 of each 32-channel half of token (t>>2) of K and V, applies
// ReLU, adds to its key sums, rotates, and writes V and R phi(K) into LDS tiles
// [token][64].  Loads run two steps ahead of the tiles.  MFMA with
// A[e][n] = V[n][e], B[n][f] = R phi(K)[n][f], C = S: at head dim 32, wave w
// takes head (w & 1) and tokens 32*(w >> 1) .. +31 of the step (two waves per
// head, added at the end); at 64, wave w takes the quadrant (e half w >> 1,
// f half w & 1) of S over all 64 tokens.  A lane supplies one channel over 8
// tokens, read across LDS rows; odd groups of 8 rows store the two halves
// swapped, so the two half-waves read disjoint LDS banks.  Tokens past the
// chunk read as zeros (buffer range check) and add nothing.

// TS: LDS tile sets (2: double buffered, one barrier per step; 1: single
// buffered, so that more workgroups fit per CU for launches of one round).
template <typename TIn, bool P2, int DH, bool NRM, int TS>
__global__ __launch_bounds__(NT, sizeof(TIn) == 2 ? ((P2 && DH == 32 && !NRM && TS == 1) ? 4 : (NRM && DH == 64) ? 2 : 3) : 2) void k_block_state(StateArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr bool W64 = DH == 64;
  constexpr int RECN = DH * DH + DH;
  constexpr int ES = (int)sizeof(TIn);
  constexpr int NTILE = BF ? 3 : 2;      // V, R phi(K) (hi, lo for bf16)
  constexpr int TILE_ELEMS = STEP * TCOLS;
  constexpr int TILE_BYTES = NTILE * TILE_ELEMS * ES;
  constexpr int W16 = 16 / ES;           // elements per 16 bytes
  // Steps of loads in flight: a launch of one resident round (single-buffered
  // tiles, four workgroups per CU) runs faster with one; longer launches keep two.
  constexpr int PF = (BF && P2 && !W64 && !NRM) ? (TS == 1 ? 1 : LAVR_STATE_PF) : 2;
  static_assert(PF >= 1 && PF <= 3, "block-state prefetch depth: one to three register buffers");
  // bf16 keys that are not normalised stay packed: ReLU on the packed pairs,
  // key sums and rotation by v_dot2_f32_bf16 against a rope_words window.
  constexpr bool PK = BF && !NRM;

  extern __shared__ __align__(16) unsigned char smem[];
  // Tile set in use (two sets alternate per step when double buffered).
  TIn* tV = reinterpret_cast<TIn*>(smem);
  TIn* tK = tV + TILE_ELEMS;
  TIn* tKl = tK + TILE_ELEMS;            // bf16 only
  float2* tab = reinterpret_cast<float2*>(smem + TS * TILE_BYTES);
  u32x4* tab16 = reinterpret_cast<u32x4*>(smem + TS * TILE_BYTES);

  const int g = blockIdx.x % a.hg;
  const int ci = blockIdx.x / a.hg;
  const int b = blockIdx.y;
  const int j = ci / a.cpb;
  const int c = ci - j * a.cpb;
  const int blk0 = block_start(j, a.L0, a.L);
  const int blk1 = min(blk0 + (j == 0 ? a.L0 : a.L), a.N);
  const int c0 = min(blk0 + c * a.Tc, blk1);
  const int c1 = min(c0 + a.Tc, blk1);
  const int h0 = W64 ? g : 2 * g;        // first head of the group
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lrow = t >> 2, lc = t & 3;   // loader: token row of the step, channel chunk
  const int nh = W64 ? 2 : min(2, a.H - h0);   // 32-channel halves that hold data
  const bool rope_on = a.rope.table != nullptr;

  // K and V of this chunk: rows c0 .. c1-1 of batch b.
  const int RB = a.row_in * ES;
  const size_t base = ((size_t)b * a.N + c0) * RB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + base, (uint32_t)(c1 - c0) * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + base, (uint32_t)(c1 - c0) * RB);
  int voff = lrow * RB + (g * 64 + 8 * lc) * ES;
  // Normalised k: the token scales of the chunk (past it they read 0, and so
  // does the key) and this thread's 16 channel weights.
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(NRM ? a.scale + (size_t)b * a.N + c0 : nullptr, NRM ? (uint32_t)(c1 - c0) * 4 : 0u);
  int soff = lrow * 4;
  float gam[2][8];
  if constexpr (NRM) {
#pragma unroll
    for (int h = 0; h < 2; ++h) load_gamma8(a.gamma, g * 64 + h * D + 8 * lc, h < nh, gam[h]);
  }

  struct Buf { Raw8<TIn> k[2], v[2]; float s; };
  auto load_step = [&](Buf& bf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf.k[h] = bload8<TIn>(rk, voff + h * D * ES);
      bf.v[h] = bload8<TIn>(rv, voff + h * D * ES);
    }
    voff += STEP * RB;
    if constexpr (NRM) {
      bf.s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0));
      soff += STEP * 4;
    }
  };
  // Rotary window reads first, then the K/V loads, then the window's LDS
  // writes: the writes wait only for the window reads.
  TabStage ts;
  ts.issue(a.rope, a.pos.t0, c0, c1, a.pos.mag_tpf);
  const TabWindow win = ts.w;

  // Register buffers: loads run PF steps ahead of the LDS tiles.  Every load
  // is issued, also past the chunk (those read zeros and touch no memory), so
  // the number of loads in flight is fixed and each wait covers only the
  // oldest step.
  Buf b0, b1, b2;
  load_step(b0);
  if constexpr (PF > 1) load_step(b1);
  if constexpr (PF > 2) load_step(b2);

  if constexpr (PK) ts.commit16(tab16);
  else ts.commit(tab);
  RopeLane<P2, PK ? 16 : 8> rl, rl1;    // rl1: the second half at head dim 64
  TokPos tp;
  if (rope_on) {
    rl.init(a.rope, win, lc);
    if constexpr (W64) rl1.init(a.rope, win, lc + 4);
    tp.init(c0 + lrow, a.pos);
  }
  __syncthreads();

  float zacc[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) zacc[h][i] = 0.f;
  f32x16 acc = {};
  const int hh = w & 1, th = w >> 1, cl = lane & 31, q = lane >> 5;
  const int ha = W64 ? (w >> 1) : hh;    // half of the channels feeding A (V, rows e of S)
  const int hb = W64 ? (w & 1) : hh;     // half of the channels feeding B (R phi(K), columns f)
  const int rbase = W64 ? 0 : th * 32;   // first token row of the wave's share of a step

  auto run_step_pk = [&](const auto& bf) {   // generic: instantiated only where called
    u32x4 T[4], T1[4];
    if (rope_on) {
      rl.fetch16(tab16, tp, win, T);
      if constexpr (W64) rl1.fetch16(tab16, tp, win, T1);
      tp.advance(a.pos);
    }
    // (1, -0) and (-0, 1): literals, not inline constants (as in split8d)
    const bf16x2 one0 = __builtin_bit_cast(bf16x2, 0x80003f80u);
    const bf16x2 one1 = __builtin_bit_cast(bf16x2, 0x3f808000u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 kp = relu_pk(bf.k[h].r[0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 kb = __builtin_bit_cast(bf16x2, (uint32_t)kp[i]);
        zacc[h][2 * i] = __builtin_amdgcn_fdot2_f32_bf16(kb, one0, zacc[h][2 * i], false);
        zacc[h][2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(kb, one1, zacc[h][2 * i + 1], false);
      }
      const int col = (h * D + 8 * lc) ^ (((lrow >> 3) & 1) << 5);
      *reinterpret_cast<u32x4*>(tV + lrow * TCOLS + col) = bf.v[h].r[0];
      u32x4 hi = kp, lo = {0u, 0u, 0u, 0u};
      if (rope_on) {
        float x[8];
        rotate_pk(kp, (W64 && h == 1) ? T1 : T, x);
        split8d(x, hi, lo);
      }
      *reinterpret_cast<u32x4*>(tK + lrow * TCOLS + col) = hi;
      *reinterpret_cast<u32x4*>(tKl + lrow * TCOLS + col) = lo;
    }
  };

  auto run_step_wide = [&](const auto& bf) {   // generic: instantiated only where called
    float2 cs[4], cs1[4];
    if (rope_on) {
      rl.fetch(tab, tp, win, cs);
      if constexpr (W64) rl1.fetch(tab, tp, win, cs1);
      tp.advance(a.pos);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[8];
      if constexpr (NRM) norm_relu_widen(bf.k[h], gam[h], bf.s, x);
      else relu_widen(bf.k[h], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) zacc[h][i] += x[i];
      if (rope_on) rotate8(x, (W64 && h == 1) ? cs1 : cs);
      const int col = (h * D + 8 * lc) ^ (((lrow >> 3) & 1) << 5);
      TIn* dv = tV + lrow * TCOLS + col;
#pragma unroll
      for (int i = 0; i < ES / 2; ++i) *reinterpret_cast<u32x4*>(dv + i * W16) = bf.v[h].r[i];
      if constexpr (BF) {
        u32x4 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<u32x4*>(tK + lrow * TCOLS + col) = hi;
        *reinterpret_cast<u32x4*>(tKl + lrow * TCOLS + col) = lo;
      } else {
        f32x4* dk = reinterpret_cast<f32x4*>(tK + lrow * TCOLS + col);
        dk[0] = f32x4{x[0], x[1], x[2], x[3]};
        dk[1] = f32x4{x[4], x[5], x[6], x[7]};
      }
    }
  };

  auto run_step = [&](const Buf& bf) {
    if constexpr (PK) run_step_pk(bf);
    else run_step_wide(bf);
  };

  auto mfma_step = [&]() {
    if constexpr (BF) {
      // ds_read_b64_tr_b16: in each 16-lane group, lane 4r+s reads channels
      // c0+4s .. +3 of token row r, and the hardware hands lane i channel c0+i
      // of the 4 rows.  Group G = lane >> 4 takes channels 16(G&1) .. +15 of a
      // half and tokens 8(G>>1) .. +7 of the 16-token MFMA step (two reads of 4
      // rows), which is the 32x32x16 operand layout: lane l holds channel l%32
      // over tokens 8(l/32) .. +7.
      const int G = lane >> 4, jr = (lane >> 2) & 3, js = lane & 3;
      const int sw = (G >> 1) << 5;
      const int colA = ((ha * D) ^ sw) + 16 * (G & 1) + 4 * js;
      const int colB = ((hb * D) ^ sw) + 16 * (G & 1) + 4 * js;
#pragma unroll
      for (int m = 0; m < (W64 ? 4 : 2); ++m) {
        const int row0 = rbase + m * 16 + 8 * (G >> 1) + jr;
        const int eA = row0 * TCOLS + colA, eB = row0 * TCOLS + colB;
        const u32x4 av = tr_pair(tV, eA, eA + 4 * TCOLS);
        const u32x4 bh = tr_pair(tK, eB, eB + 4 * TCOLS);
        const u32x4 bl = tr_pair(tKl, eB, eB + 4 * TCOLS);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bl), acc, 0, 0, 0);
      }
    } else {
      const float* Vf = reinterpret_cast<const float*>(tV);
      const float* Kf = reinterpret_cast<const float*>(tK);
#pragma unroll
      for (int s = 0; s < (W64 ? 32 : 16); ++s) {
        const int row = rbase + 2 * s + q;
        const int swr = ((row >> 3) & 1) << 5;
        const int iA = row * TCOLS + ((ha * D + cl) ^ swr);
        const int iB = row * TCOLS + ((hb * D + cl) ^ swr);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vf[iA], Kf[iB], acc, 0, 0, 0);
      }
    }
  };

  // Whole rounds of PF steps; steps past the chunk hold zeros and add nothing.
  // With two tile sets, the barrier after step s+1's tile writes also orders
  // every wave's step-s MFMA reads before step s+2 rewrites that set.
  auto one_step = [&](Buf& bf) {
    run_step(bf);
    __syncthreads();
    load_step(bf);
    mfma_step();
    if constexpr (TS == 2) {
      const int off = (tV == reinterpret_cast<TIn*>(smem)) ? TILE_BYTES : 0;
      tV = reinterpret_cast<TIn*>(smem + off);
      tK = tV + TILE_ELEMS;
      tKl = tK + TILE_ELEMS;
    } else {
      __syncthreads();
    }
  };
  for (int s0 = c0; s0 < c1; s0 += PF * STEP) {
    one_step(b0);
    if constexpr (PF > 1) one_step(b1);
    if constexpr (PF > 2) one_step(b2);
  }

  if constexpr (TS == 2) __syncthreads();   // last MFMA reads before red reuses the tiles

  // Head dim 32: combine the two waves of each head through LDS.  Key sums:
  // first across the 16 lanes of a wave that hold the same channel chunk
  // (cross-lane adds), then across the four waves through LDS.
  float* red = reinterpret_cast<float*>(smem);   // [2 waves][16][64]
  float* zred = red + 2 * 16 * 64;               // [4 waves][4 chunks][16]
  if (!W64 && w >= 2) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((w - 2) * 16 + v) * 64 + lane] = acc[v];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float zs = sum16_lanes_mod4(zacc[h][i]);
      if (lane < 4) zred[(w * 4 + lane) * 16 + h * 8 + i] = zs;
    }
  __syncthreads();

  // Records: S (DH x DH, row e, column f) then z (DH).
  if constexpr (W64) {
    float* dst = a.part + part_rec((size_t)(b * a.H + h0), ci, (size_t)gridDim.y * a.H) * RECN;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      dst[(ha * D + e) * DH + hb * D + (lane & 31)] = acc[v];
    }
  } else if (w < 2 && w < nh) {
    float* dst = a.part + part_rec((size_t)(b * a.H + h0 + w), ci, (size_t)gridDim.y * a.H) * RECN;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      dst[e * D + (lane & 31)] = acc[v] + red[(w * 16 + v) * 64 + lane];
    }
  }
  if (t < 2 * D && t / D < nh) {
    const int hd = t / D, ch = t % D;
    const int lc2 = ch >> 3, el = ch & 7;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) s += zred[(ww * 4 + lc2) * 16 + hd * 8 + el];
    const size_t zi = W64 ? part_rec((size_t)(b * a.H + h0), ci, (size_t)gridDim.y * a.H) * RECN + DH * DH + hd * D + ch
                          : part_rec((size_t)(b * a.H + h0 + hd), ci, (size_t)gridDim.y * a.H) * RECN + D * D + ch;
    a.part[zi] = s;
  }
  if (a.fp_dst != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && t == 0) {
    a.fp_dst[0] = a.fp0;
    a.fp_dst[1] = a.fp1;
  }
}

// -------------------------------------------------------------- k_prefix
//
// Grid: x = element group (17 x 64 covers the 1056 floats of a record),
// y = head, z = batch; 256 threads.  For each run of 32 blocks, the four waves
// form block sums p_0 + p_1 + ... (chunk order) for blocks w, w+4, ... of the
// run into LDS, reading the (block, chunk) partials of a wave 24 at a time so
// that their latencies overlap (all of them at once for 8 blocks of 3 chunks,
// the minute-length clip's 30 blocks); then wave 0 walks the run in block order:
// prefix = previous prefix + block sum.  A streaming call starts from the
// carried cache, so one block streamed on top of a cache adds exactly as the
// one-shot prefix does.

constexpr int PFX_NT = 256;
constexpr int PFX_RUN = 32;

__global__ __launch_bounds__(PFX_NT) void k_prefix(PrefixArgs a) {
  __shared__ float bs[PFX_RUN][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int el = blockIdx.x * 64 + lane;
  const int REC = a.rec;
  const bool ok = el < REC;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  // (lanes past the record read its last element and discard it)
  const size_t cstride = (size_t)gridDim.z * a.H * REC;   // from one chunk's record to the next
  const float* part = a.part + bh * REC + min(el, REC - 1);
  float* o = a.prefix + bh * a.nb * REC + el;
  float acc = 0.f;
  if (w == 0 && ok && a.S_init != nullptr)
    acc = el < a.hd * a.hd ? a.S_init[bh * a.hd * a.hd + el] : a.z_init[bh * a.hd + el - a.hd * a.hd];
  constexpr int BATCH = 24;
  for (int r0 = 0; r0 < a.nb; r0 += PFX_RUN) {
    const int nr = min(PFX_RUN, a.nb - r0);
    // Items of this wave: (block bi, chunk c) for its blocks r0 + w + 4 bi, in
    // block-major, chunk-minor order; item q sits at block w + 4 (q / cpb).
    const int items = (nr > w ? (nr - w + 3) / 4 : 0) * a.cpb;
    float s = 0.f;
    int bi = 0, c = 0;                    // (block, chunk) of the next item to add
    for (int q0 = 0; q0 < items; q0 += BATCH) {
      // Unconditional loads (items past the end reread the last one) keep the
      // batch in flight together.
      float v[BATCH];
      int lb = bi, lcn = c;               // (block, chunk) of the next item to load
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int jb = a.rev ? a.nb - 1 - (r0 + w + 4 * lb) : r0 + w + 4 * lb;
        v[i] = part[((size_t)jb * a.cpb + lcn) * cstride];
        if (q0 + i + 1 < items && ++lcn == a.cpb) { lcn = 0; ++lb; }
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (q0 + i < items) {
          s += v[i];
          if (++c == a.cpb) {
            bs[w + 4 * bi][lane] = s;
            s = 0.f;
            c = 0;
            ++bi;
          }
        }
      }
    }
    __syncthreads();
    if (w == 0 && ok) {
      for (int jj = 0; jj < nr; ++jj) {
        acc += bs[jj][lane];
        o[(size_t)(a.rev ? a.nb - 1 - (r0 + jj) : r0 + jj) * REC] = acc;
      }
    }
    __syncthreads();
  }
  if (w == 0 && ok && a.S_save != nullptr) {
    if (el < a.hd * a.hd) a.S_save[bh * a.hd * a.hd + el] = acc;
    else a.z_save[bh * a.hd + el - a.hd * a.hd] = acc;
  }
}

// Single-block calls (a streamed block, or a one-shot call of one block): no
// scan over blocks, so every thread takes one element of one record, sums the
// block's chunk partials in chunk order (sixteen loads in flight) and adds the
// carried state, in the same order as k_prefix.  Grid: x = element group of
// 256, y = head, z = batch.
__global__ __launch_bounds__(256) void k_prefix1(PrefixArgs a) {
  const int el = blockIdx.x * 256 + threadIdx.x;
  const int REC = a.rec;
  if (el >= REC) return;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  const size_t cstride = (size_t)gridDim.z * a.H * REC;   // from one chunk's record to the next
  const float* part = a.part + bh * REC + el;
  const bool inS = el < a.hd * a.hd;
  const size_t si = bh * a.hd * a.hd + el, zi = bh * a.hd + el - a.hd * a.hd;
  // the carried state is read first, so that its load is in flight with the
  // partials' (one memory latency for the whole kernel)
  float acc = 0.f;
  if (a.S_init != nullptr) acc = inS ? a.S_init[si] : a.z_init[zi];
  constexpr int BATCH = 16;
  float s = 0.f;
  for (int c0 = 0; c0 < a.cpb; c0 += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) v[i] = part[(size_t)min(c0 + i, a.cpb - 1) * cstride];
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (c0 + i < a.cpb) s += v[i];
  }
  acc += s;
  a.prefix[bh * REC + el] = acc;
  if (a.S_save != nullptr) {
    if (inS) a.S_save[si] = acc;
    else a.z_save[zi] = acc;
  }
}

// ------------------------------------------------------------- k_readout
//
// Grid: x = tile * hg + head group, y = batch.  256 threads; a workgroup owns
// 64 channels of every token row (two heads at head dim 32, one at 64, as in
// the block-state kernel).  Wave w takes the tile's 16-token groups w, w+4, ...
// with loads two groups ahead.  MFMA 16x16x32: A = Sbar rows (e) x 32 channels
// (f), B = 32 channels (f) x tokens: lane l holds channels 8(l>>4) .. +7 of
// each 32-channel half of token (l & 15), one 16-byte load of bf16 q per half.
// At head dim 32 each half is a head; at 64 every 16-row tile of the output
// sums the products of both halves.  The Sbar rows are staged so that the
// output lane holds channels 8(l>>4) .. +7 of each 32-channel half for token
// (l & 15) (four from each of the half's two tiles).  Tokens past the tile
// read as zeros and their stores are dropped by the buffer range check.
//
// bf16 inputs that are not normalised take the packed path: phi(q) stays
// packed bf16 (exact) and feeds the normaliser's MFMA, whose A operand (from
// LDS) holds zbar's hi bf16 part in the even rows and its lo part in the odd
// rows (one MFMA per 32-channel half), so each output lane receives its own
// token's hi and lo parts of zbar . phi(q) side by side; the rotation is
// v_dot2_f32_bf16 on the packed pairs against the rope_words table, so phi(q)
// is never widened.  This path spends about a third fewer VALU instructions
// per token than widening to fp32, which matters because the kernel's time
// grows as the shader clock drops (the clock dips under a sudden heavy load).
// Other inputs widen phi(q) to fp32, form the normaliser with fp32 FMAs summed
// over the four lanes of a token, and rotate in fp32.
//
// RO: RoPE on, a compile-time switch so the loop carries no branch on it.

template <typename TIn, typename TOut, bool P2, int DH, bool NRM, bool RO>
__global__ __launch_bounds__(NT, (sizeof(TIn) == 2 && !NRM) ? 4 : (!NRM && DH == 32 && P2) ? 3 : 2) void k_readout(
    ReadArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr bool W64 = DH == 64;
  constexpr bool FAST = BF && !NRM;      // packed bf16 phi(q)
  constexpr int RECN = DH * DH + DH;
  constexpr int ES = (int)sizeof(TIn), EO = (int)sizeof(TOut);
  constexpr int NA = W64 ? 8 : 4;        // Sbar tiles of 16 rows x 32 channels a lane holds
  extern __shared__ __align__(16) unsigned char smem[];
  // bf16 at head dim 64, and the packed path: the hi and lo parts of the Sbar
  // tiles live in LDS (one copy per workgroup, lane-major: slot (2 i + part) *
  // 64 + lane), and on the packed path zbar's bf16 parts too ([head or half]
  // [part][lane row] slices), which keeps the kernel within 128 registers
  // without spills.
  constexpr bool A_LDS = BF && (W64 || FAST);
  constexpr bool Z_LDS = FAST;
  constexpr int A_BYTES = A_LDS ? 2 * NA * 64 * 16 : 0;
  constexpr int PRE = A_BYTES + (Z_LDS ? kReadZBytes : 0);
  u32x4* lds_a = reinterpret_cast<u32x4*>(smem);
  u32x4* lds_z = reinterpret_cast<u32x4*>(smem + A_BYTES);
  float2* tab = reinterpret_cast<float2*>(smem + PRE);
  u32x4* tab16 = reinterpret_cast<u32x4*>(smem + PRE);

  // (tile, head group) and (block, tile in block) from the workgroup index by
  // multiply-shift divisions (fast_div) instead of the compiler's division
  const int ti = (int)fast_div(blockIdx.x, a.mag_hg);
  const int g = blockIdx.x - ti * a.hg;
  const int b = blockIdx.y;
  const int j = (int)fast_div((uint32_t)ti, a.mag_rpb);
  const int r = ti - j * a.rpb;
  const int blk0 = block_start(j, a.L0, a.L);
  const int blk1 = min(blk0 + (j == 0 ? a.L0 : a.L), a.N);
  const int t0 = min(blk0 + r * a.Tr, blk1);
  const int t1 = min(t0 + a.Tr, blk1);
  if (t0 >= t1) return;

  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: kept in a scalar register, so
  // that the group loop and the per-group buffer resources below are scalar work
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tl = lane & 15, ch = lane >> 4;
  const int h0 = W64 ? g : 2 * g;        // first head of the group
  const int nh = W64 ? 2 : min(2, a.H - h0);   // 32-channel halves that hold data
  const int ngroups = (t1 - t0 + 15) >> 4;

  // Q, the token scales and out are reached through one buffer resource per
  // 16-token group, starting at the group's first row and ending at the
  // tile's end (no bytes past it: a group past the end reads zeros and drops
  // its stores).  The resources are formed in scalar registers, and a lane's
  // offsets inside them stay fixed, so advancing a group costs no vector
  // instruction.
  const int RB = a.row_in * ES, RO_ = a.H * DH * EO;
  const char* q_tile = static_cast<const char*>(a.q) + ((size_t)b * a.N + t0) * RB;
  char* o_tile = static_cast<char*>(a.out) + ((size_t)b * a.N + t0) * RO_;
  const int n_tok = t1 - t0;
  auto q_rsrc = [&](int gr) { return make_rsrc(q_tile + (size_t)(16 * gr) * RB, (uint32_t)max(n_tok - 16 * gr, 0) * RB); };
  auto o_rsrc = [&](int gr) { return make_rsrc(o_tile + (size_t)(16 * gr) * RO_, (uint32_t)max(n_tok - 16 * gr, 0) * RO_); };
  const int qlane = tl * RB + (g * 64 + 8 * ch) * ES;
  // Output offsets of this lane: channels 8ch .. 8ch+7 of each 32-channel half
  // of token tl (the Sbar rows are staged in the order that puts them there).
  // fp32: stored as two 16-byte pieces per half.  bf16 (after the exchange in
  // store_pk): tokens tl & 7 (first store) and 8 + (tl & 7) (second store) of
  // half tl >> 3, so each store instruction writes whole 128-byte lines
  // (8 tokens x the group's 64 channels).
  const int o_one = tl * RO_ + (g * 64 + 8 * ch) * EO;
  // The last group of an odd head count (head dim 32) holds one head: its
  // second half is computed on whatever the loads return, and every store of
  // that half is sent past the buffer range, where the hardware drops it (an
  // offset of 2^31 + x, x < 2^31, exceeds any range a call plans).  One loop
  // then serves every group.
  const bool two = W64 || nh == 2;
  constexpr int kDrop = (int)0x80000000u;
  const int o_pair = (two || tl < 8) ? (tl & 7) * RO_ + (g * 64 + (tl >> 3) * D + 8 * ch) * EO : kDrop;
  const int o_pair2 = o_pair + 8 * RO_;       // second bf16 store: tokens 8 .. 15
  const int o_half1 = two ? D * EO : kDrop;   // fp32 stores: offset of half 1

  // Prologue: the rotary window and the prefix record (zbar and the Sbar
  // tiles) are loaded together, so that their latencies overlap, and the
  // first Q groups follow once both are in LDS.  (Issuing the Q loads before
  // those waits measured slower at the minute-length workload.)
  TabStage ts;
  if constexpr (RO) ts.issue(a.rope, a.pos.t0, t0, t1, a.pos.mag_tpf);
  else ts.w = TabWindow{0, 0};
  const TabWindow win = ts.w;
  RopeLane<P2, FAST ? 16 : 8> rl, rl1;  // rl1: the second half at head dim 64

  // Key-sum slices zb[h] (channels 32h + 8ch .. +7 of the half's z; packed
  // path: their bf16 parts zh, zl) and Sbar tiles.  A tile is 16 rows of one
  // 32-row half of Sbar: tile row m of the half's tile hf is Sbar row
  // 8 (m / 4) + 4 hf + m % 4 of the half, so that the MFMA's output lane
  // (rows 4 (l / 16) .. +3 of each tile) receives rows 8 (l / 16) .. +7, eight
  // consecutive channels of its token, with no exchange between lanes.  Head
  // dim 32: tile 2h + hf of head h, channels 8ch .. +7.  Head dim 64: tile
  // 2et + kt = half et >> 1, tile et & 1, channels 32kt + 8ch .. +7.
  const float* pre[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int hd = W64 ? 0 : min(h, nh - 1);
    pre[h] = a.prefix + ((size_t)(b * a.H + h0 + hd) * a.nb + j) * RECN;
  }
  auto tile_row = [&](int hf) { return 8 * (tl >> 2) + 4 * hf + (tl & 3); };
  auto tile_src = [&](int i) -> const float* {
    if constexpr (W64) return pre[0] + (32 * (i >> 2) + tile_row((i >> 1) & 1)) * DH + (i & 1) * D + 8 * ch;
    else return ((i >> 1) ? pre[1] : pre[0]) + tile_row(i & 1) * D + 8 * ch;
  };
  float zb[2][8];
  f32x4 zr[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* zp = pre[h] + DH * DH + (W64 ? h * D : 0) + 8 * ch;
    zr[h][0] = *reinterpret_cast<const f32x4*>(zp);
    zr[h][1] = *reinterpret_cast<const f32x4*>(zp + 4);
  }
  // Tiles in LDS are split and written by one wave each (wave i mod 4), so a
  // wave loads only tiles w, w + 4, ...; register tiles are loaded by every wave.
  constexpr int NL = A_LDS ? NA / 4 : NA;
  auto tile_of = [&](int m) { return A_LDS ? w + 4 * m : m; };
  f32x4 tr[NL][2];
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    const float* src = tile_src(tile_of(m));
    tr[m][0] = *reinterpret_cast<const f32x4*>(src);
    tr[m][1] = *reinterpret_cast<const f32x4*>(src + 4);
  }

  // Normalised q: token scales of the tile (0 past it) and the lane's weights.
  const float* s_tile = NRM ? a.scale + (size_t)b * a.N + t0 : nullptr;
  auto s_rsrc = [&](int gr) { return make_rsrc(s_tile + 16 * gr, NRM ? (uint32_t)max(n_tok - 16 * gr, 0) * 4 : 0u); };
  float gam[2][8];
  if constexpr (NRM) {
#pragma unroll
    for (int h = 0; h < 2; ++h) load_gamma8(a.gamma, g * 64 + h * D + 8 * ch, h < nh, gam[h]);
  }

  struct Buf { Raw8<TIn> x[2]; float s; };
  int gload = w;                         // next group to load (uniform)
  auto load_group = [&](Buf& bf) {
    const __amdgpu_buffer_rsrc_t rq = q_rsrc(gload);
#pragma unroll
    for (int h = 0; h < 2; ++h) bf.x[h] = bload8<TIn>(rq, qlane + h * D * ES);
    if constexpr (NRM) bf.s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s_rsrc(gload), tl * 4, 0, 0));
    gload += 4;
  };
  auto widen_q = [&](const Buf& bf, int h, float* x) {
    if constexpr (NRM) norm_relu_widen(bf.x[h], gam[h], bf.s, x);
    else relu_widen(bf.x[h], x);
  };
  // Register buffers: loads run RPF groups ahead of the arithmetic.  Every
  // load is issued, also past the tile (those read zeros and touch no memory),
  // so the number of loads in flight is fixed.
  // One group in flight on the packed path at head dim 32 (with more
  // workgroups per CU: see kReadOccN), two or three elsewhere.
  constexpr int RPF = (FAST && !W64) ? 1 : BF ? LAVR_READ_PF : 2;
  static_assert(RPF >= 1 && RPF <= 3, "readout prefetch depth: one to three buffers");
  Buf b0, b1, b2;

  // The waits, oldest loads first: the window, then the record.
  TokPos tp;
  if constexpr (RO) {
    if constexpr (FAST) ts.commit16(tab16);
    else ts.commit(tab);
    rl.init(a.rope, win, ch);
    if constexpr (W64) rl1.init(a.rope, win, ch + 4);
    tp.init(t0 + w * 16 + tl, a.pos);
  }
  u32x4 zh[2], zl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { zb[h][i] = zr[h][0][i]; zb[h][4 + i] = zr[h][1][i]; }
    if constexpr (Z_LDS) {
      if (w == 0) {                      // uniform: only wave 0 stores the slices
        split8d(zb[h], zh[h], zl[h]);
        if (tl == 0) {
          lds_z[(2 * h) * 4 + ch] = zh[h];
          lds_z[(2 * h + 1) * 4 + ch] = zl[h];
        }
      }
    }
  }
  u32x4 Ah[NA], Al[NA];
  float As[NA][8];
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    float sv[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) { sv[k] = tr[m][0][k]; sv[4 + k] = tr[m][1][k]; }
    if constexpr (A_LDS) {
      const int i = tile_of(m);
      u32x4 hi, lo;
      split8d(sv, hi, lo);
      lds_a[(2 * i) * 64 + lane] = hi;
      lds_a[(2 * i + 1) * 64 + lane] = lo;
    } else if constexpr (BF) {
      split8(sv, Ah[m], Al[m]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) As[m][k] = sv[k];
    }
  }
  load_group(b0);
  if constexpr (RPF > 1) load_group(b1);
  if constexpr (RPF > 2) load_group(b2);

  __syncthreads();

  // Output of one 32-channel half h (o: its two 16-row tiles, channels
  // 8ch .. 8ch+3 and 8ch+4 .. 8ch+7 of token tl) scaled by inv: bf16 pieces go
  // to pk[h] for the paired store, fp32 is stored at once.
  auto emit = [&](int h, const f32x4* o, float inv, u32x4* pk, __amdgpu_buffer_rsrc_t ro) {
    if constexpr (EO == 2) {
      pk[h] = u32x4{pack_bf16(o[0][0] * inv, o[0][1] * inv), pack_bf16(o[0][2] * inv, o[0][3] * inv),
                    pack_bf16(o[1][0] * inv, o[1][1] * inv), pack_bf16(o[1][2] * inv, o[1][3] * inv)};
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 ov = o[hf] * inv;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ov), ro,
                                               o_one + (h ? o_half1 : 0) + 4 * hf * EO, 0, LAVR_STORE_CPOL);
      }
    }
  };

  // bf16 stores of a group.  Lanes tl and
  // tl ^ 8 (DPP row rotate by 8 inside each 16-lane row) trade one piece: the
  // low lane keeps half 0 of tokens tl and tl + 8, the high lane half 1 of
  // tokens tl - 8 and tl.  The bank masks limit each rotated move to the lanes
  // that take the partner's piece (banks 2-3 = lanes 8-15 of a row, banks 0-1
  // = lanes 0-7); the other lanes keep their own.
  auto store_pk = [&](const u32x4* pk, __amdgpu_buffer_rsrc_t ro) {
    if constexpr (EO == 2) {
      uint32_t first[4], second[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p0 = pk[0][i], p1 = pk[1][i];
        first[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)p0, (int)p1, 0x128, 0xf, 0xc, false);
        second[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)p1, (int)p0, 0x128, 0xf, 0x3, false);
      }
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{first[0], first[1], first[2], first[3]}, ro,
                                             o_pair, 0, LAVR_STORE_CPOL);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{second[0], second[1], second[2], second[3]}, ro,
                                             o_pair2, 0, LAVR_STORE_CPOL);
    }
  };

  // Normaliser of the packed path: the MFMA's A operand holds zbar's hi part
  // in the tile rows m with m % 2 == 0 and its lo part in the odd rows (lane
  // tl supplies row tl), so each output lane's elements 0 and 1 are its
  // token's hi . phi(q) and lo . phi(q), and the accumulator starts at
  // (eps, 0, 0, 0): den = dd[0] + dd[1] with no exchange between lanes.
  const f32x4 dd_init = {a.eps, 0.f, 0.f, 0.f};

  // One 16-token group (gc: its index in the tile), packed bf16 path.
  auto run_fast = [&](const auto& bf, int gc) {   // generic: instantiated only where called
    const __amdgpu_buffer_rsrc_t ro = o_rsrc(gc);
    u32x4 T[4], T1[4];
    if constexpr (RO) {
      rl.fetch16(tab16, tp, win, T);
      if constexpr (W64) rl1.fetch16(tab16, tp, win, T1);
      tp.advance(a.pos);
    }
    u32x4 pk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if constexpr (W64) {
      // one head: den over both halves, every output tile from both halves
      // (one normaliser MFMA per half, A operand read from LDS)
      u32x4 qp[2], bh[2], bl[2];
      f32x4 dd = dd_init;
      int zrow = ch + ((tl & 1) << 2);
      asm volatile("" : "+v"(zrow));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        qp[h] = relu_pk(bf.x[h].r[0]);
        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lds_z[8 * h + zrow]), as_bf16x8(qp[h]), dd, 0, 0, 0);
        if constexpr (RO) {
          float x[8];
          rotate_pk(qp[h], h ? T1 : T, x);
          // (the dot2c form needs more registers: with fp32 outputs it spills)
          if constexpr (EO == 2) split8d(x, bh[h], bl[h]);
          else split8(x, bh[h], bl[h]);
        } else {
          bh[h] = qp[h];
        }
      }
      const float inv = __builtin_amdgcn_rcpf(dd[0] + dd[1]);
      // The Sbar operands are read from LDS in every group: an opaque copy of
      // the lane index keeps the compiler from hoisting them into registers.
      int aslot = lane;
      asm volatile("" : "+v"(aslot));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 o[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int et = 2 * h + hf;
          f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const u32x4 ah = lds_a[(2 * (et * 2 + kt)) * 64 + aslot];
            const u32x4 al = lds_a[(2 * (et * 2 + kt) + 1) * 64 + aslot];
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bh[kt]), cc, 0, 0, 0);
            if constexpr (RO) cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bl[kt]), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(bh[kt]), cc, 0, 0, 0);
          }
          o[hf] = cc;
        }
        emit(h, o, inv, pk, ro);
      }
    } else {
      // Sbar and zbar operands from LDS in every group: opaque copies of the
      // lane's byte offsets keep the compiler from hoisting them into registers.
      int zb_off = 16 * (ch + ((tl & 1) << 2)), ab_off = 16 * lane;
      asm volatile("" : "+v"(zb_off), "+v"(ab_off));
      const u32x4* zsl = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(lds_z) + zb_off);
      const u32x4* asl = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(lds_a) + ab_off);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 qp = relu_pk(bf.x[h].r[0]);
        const u32x4 zs = zsl[8 * h];
        const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(zs), as_bf16x8(qp), dd_init, 0, 0, 0);
        f32x4 o[2];
        if constexpr (RO) {
          float x[8];
          rotate_pk(qp, T, x);
          u32x4 bh, bl;
          split8d(x, bh, bl);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const u32x4 ah = asl[(2 * (2 * h + hf)) * 64];
            const u32x4 al = asl[(2 * (2 * h + hf) + 1) * 64];
            f32x4 cc = {0.f, 0.f, 0.f, 0.f};
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bh), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bl), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(bh), cc, 0, 0, 0);
            o[hf] = cc;
          }
        } else {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const u32x4 ah = asl[(2 * (2 * h + hf)) * 64];
            const u32x4 al = asl[(2 * (2 * h + hf) + 1) * 64];
            f32x4 cc = {0.f, 0.f, 0.f, 0.f};
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(qp), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(qp), cc, 0, 0, 0);
            o[hf] = cc;
          }
        }
        emit(h, o, __builtin_amdgcn_rcpf(dd[0] + dd[1]), pk, ro);
      }
    }
    store_pk(pk, ro);
  };

  // One 16-token group (gc: its index in the tile), fp32 path (fp32 or
  // normalised inputs).
  auto run_wide = [&](const auto& bf, int gc) {   // generic: instantiated only where called
    const __amdgpu_buffer_rsrc_t ro = o_rsrc(gc);
    float2 cs[4], cs1[4];
    if constexpr (RO) {
      rl.fetch(tab, tp, win, cs);
      if constexpr (W64) rl1.fetch(tab, tp, win, cs1);
      tp.advance(a.pos);
    }
    u32x4 pk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if constexpr (W64) {
      // one head: den over both halves, every output tile from both halves
      float den = 0.f;
      int aslot = lane;
      if constexpr (A_LDS) asm volatile("" : "+v"(aslot));
      u32x4 bh[2], bl[2];
      float xs[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x[8];
        widen_q(bf, h, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) den += zb[h][i] * x[i];
        if constexpr (RO) rotate8(x, h ? cs1 : cs);
        if constexpr (BF) {
          split8(x, bh[h], bl[h]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) xs[h][i] = x[i];
        }
      }
      den = sum4_lanes(den);
      const float inv = __builtin_amdgcn_rcpf(den + a.eps);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 o[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int et = 2 * h + hf;
          f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if constexpr (BF) {
              const u32x4 ah = lds_a[(2 * (et * 2 + kt)) * 64 + aslot];
              const u32x4 al = lds_a[(2 * (et * 2 + kt) + 1) * 64 + aslot];
              cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bh[kt]), cc, 0, 0, 0);
              cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bl[kt]), cc, 0, 0, 0);
              cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(bh[kt]), cc, 0, 0, 0);
            } else {
#pragma unroll
              for (int s = 0; s < 8; ++s)
                cc = __builtin_amdgcn_mfma_f32_16x16x4f32(As[et * 2 + kt][s], xs[kt][s], cc, 0, 0, 0);
            }
          }
          o[hf] = cc;
        }
        emit(h, o, inv, pk, ro);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x[8];
        widen_q(bf, h, x);
        float den = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) den += zb[h][i] * x[i];
        if constexpr (RO) rotate8(x, cs);
        f32x4 o[2];
        if constexpr (BF) {
          u32x4 bh, bl;
          split8(x, bh, bl);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            f32x4 cc = {0.f, 0.f, 0.f, 0.f};
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Ah[2 * h + hf]), as_bf16x8(bh), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Ah[2 * h + hf]), as_bf16x8(bl), cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Al[2 * h + hf]), as_bf16x8(bh), cc, 0, 0, 0);
            o[hf] = cc;
          }
        } else {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) cc = __builtin_amdgcn_mfma_f32_16x16x4f32(As[2 * h + hf][s], x[s], cc, 0, 0, 0);
            o[hf] = cc;
          }
        }
        den = sum4_lanes(den);
        emit(h, o, __builtin_amdgcn_rcpf(den + a.eps), pk, ro);
      }
    }
    store_pk(pk, ro);
  };

  auto run_group = [&](const Buf& bf, int gc) {
    if constexpr (FAST) run_fast(bf, gc);
    else run_wide(bf, gc);
  };

  // Whole rounds of RPF groups; groups past the tile read zeros and their
  // stores are dropped by the range check.
  for (int gi = w; gi < ngroups; gi += 4 * RPF) {
    run_group(b0, gi);
    load_group(b0);
    if constexpr (RPF > 1) {
      run_group(b1, gi + 4);
      load_group(b1);
    }
    if constexpr (RPF > 2) {
      run_group(b2, gi + 8);
      load_group(b2);
    }
  }
}

// =================================================================== backward

//
// The exact derivative of the forward for an output gradient g, per (batch,
// head); for token n of block j (p = phi(q_n), r = R p, den = zbar_j . p + eps,
// out = Sbar_j r / den):
//   a = g / den, beta = -(g . out) / den,
//   dq = [q > 0] (R^T Sbar_j^T a + beta zbar_j),
//   G_j = sum_n a r^T, gz_j = sum_n beta p,
//   dS_i = sum_{j >= i} G_j, dz_i = sum_{j >= i} gz_j   (block j reads every block <= j),
//   dv = dS_i kappa, dk = [k > 0] (R^T dS_i^T v + dz_i), kappa = R phi(k).
// Sbar, zbar come from the forward's block-state and prefix kernels (run again
// by the backward entry point); dS, dz from the prefix kernel run over the
// blocks in reverse on the chunk partials of (G, gz).

struct BwQArgs {
  const void* q;
  const void* g;
  void* dq;
  const float* prefix;       // Sbar_j, zbar_j records
  float* part;               // out: chunk partials of (G, gz)
  float eps;
  int H, N, L, L0, nb, cpb, Tc, hg;
  PosArgs pos;
  RopeDev rope;
};

struct BwKVArgs {
  const void* k;
  const void* v;
  void* dk;
  void* dv;
  const float* suffix;       // dS_i, dz_i records
  int H, N, L, L0, nb, rpb, Tr, hg;
  PosArgs pos;
  RopeDev rope;
};

__device__ __forceinline__ void unrotate8(float* x, const float2* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * cs[i].x + b * cs[i].y;
    x[2 * i + 1] = b * cs[i].x - a * cs[i].y;
  }
}

__device__ __forceinline__ void widen8(const Raw8<uint16_t>& r, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ri = r.r[0][i];
    x[2 * i] = __uint_as_float(ri << 16);
    x[2 * i + 1] = __uint_as_float(ri & 0xffff0000u);
  }
}
__device__ __forceinline__ void widen8(const Raw8<float>& r, float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(r.r[i >> 2][i & 3]);
}

// Matrix-vector products in the token layout (lane l: token l & 15, channels
// 8(l >> 4) .. +7).  MFMA 16x16x32 output row i of tile t is loaded from matrix
// row 8(i >> 2) + 4t + (i & 3), so the output lane of chunk ch holds channels
// 8ch + 4t .. +3: with both tiles, exactly the channels its inputs hold.
__device__ __forceinline__ int perm_row(int t, int i) { return 8 * (i >> 2) + 4 * t + (i & 3); }

constexpr int OPS_BLOCK = 4 * 64;                   // u32x4 slots of one block's operand tiles

// c[t] += (block, tile t) x for the lane's token; x as bf16 hi/lo (xl may be
// null: x exact in bf16) or 8 floats.  Output tile t, lane row ch holds the
// block's output channels 8ch + 4t .. +3 (row-permuted operands).
template <bool BF>
__device__ __forceinline__ void mv_acc(const u32x4* op, int lane, u32x4 xh, const u32x4* xl, const float* xf,
                                       f32x4* c) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u32x4 p0 = op[(t * 2) * 64 + lane], p1 = op[(t * 2 + 1) * 64 + lane];
    if constexpr (BF) {
      c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p0), as_bf16x8(xh), c[t], 0, 0, 0);
      if (xl != nullptr) c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p0), as_bf16x8(*xl), c[t], 0, 0, 0);
      c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p1), as_bf16x8(xh), c[t], 0, 0, 0);
    } else {
      const f32x4 f0 = __builtin_bit_cast(f32x4, p0), f1 = __builtin_bit_cast(f32x4, p1);
#pragma unroll
      for (int s = 0; s < 4; ++s) c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(f0[s], xf[s], c[t], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) c[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(f1[s], xf[4 + s], c[t], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void take8(const f32x4* c, float* y) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) y[4 * t + v] = c[t][v];
}

// Operand blocks of a matrix per workgroup: at head dim 32 one 32 x 32 block
// per head of the pair, at 64 the four quadrants (a, b) of the head's 64 x 64
// matrix (block 2a + b maps input half b to output half a).  NMAT = 2: blocks
// 0 .. NB-1 hold the matrix, NB .. 2NB-1 its transpose; NMAT = 1: blocks 0 ..
// NB-1 hold the transpose only.  The four waves form them: block bo by wave
// bo mod 4.  A block's operand tiles (both 16-row tiles), parked in LDS: slot
// (tile * 2 + part) holds, per lane, the bf16 hi (part 0) and lo (part 1) of
// the lane's 8 values, or for fp32 values 0-3 (part 0) and 4-7 (part 1);
// 16-byte slots per lane keep the reads conflict-free.  In two steps, so that
// a prologue issues these loads with its others and waits for them later:
// issue() loads the wave's values into registers, commit() writes the tiles.
template <bool BF, bool W64, int NMAT>
struct OpsStage {
  static constexpr int NB = W64 ? 4 : 2;
  static constexpr int TOT = NMAT * NB;
  static constexpr int K = (TOT + 3) / 4;   // blocks per wave (at most)
  float sv[K][2][8];

  __device__ void issue(const float* rec0, const float* rec1, int w, int lane) {
    const int i = lane & 15, kc = lane >> 4;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int bo = w + 4 * k;
      if (bo >= TOT) break;
      const bool tr = NMAT == 2 ? bo >= NB : true;
      const int blk = bo % NB;
      // Element [r][c] of the block is m[r * ld + c], of its transpose
      // m[c * ld + r].  At 64, block (qa, qb) of M: rows 32qa.., columns
      // 32qb..; of M^T: the transpose of M's block (qb, qa).
      const float* m;
      int ld;
      if constexpr (W64) {
        const int qa = blk >> 1, qb = blk & 1;
        m = tr ? rec0 + (32 * qb) * 64 + 32 * qa : rec0 + (32 * qa) * 64 + 32 * qb;
        ld = 64;
      } else {
        m = blk == 0 ? rec0 : rec1;
        ld = 32;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = perm_row(t, i);
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[k][t][e] = m[tr ? (8 * kc + e) * ld + row : row * ld + 8 * kc + e];
      }
    }
  }

  __device__ void commit(u32x4* ops, int w, int lane) const {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int bo = w + 4 * k;
      if (bo >= TOT) break;
      u32x4* op = ops + bo * OPS_BLOCK;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float* v = sv[k][t];
        if constexpr (BF) {
          u32x4 hi, lo;
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = v[e];
          split8(x, hi, lo);
          op[(t * 2) * 64 + lane] = hi;
          op[(t * 2 + 1) * 64 + lane] = lo;
        } else {
          op[(t * 2) * 64 + lane] = __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
          op[(t * 2 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]});
        }
      }
    }
  }
};

// Store the 8 channels y of the lane's token for half h: bf16 pieces are
// collected in pk for the paired store; fp32 goes out at once.
template <int EO>
__device__ __forceinline__ void put8(const float* y, int h, u32x4* pk, __amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (EO == 2) {
    pk[h] = u32x4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}), rs, off, 0,
                                           LAVR_STORE_CPOL);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{y[4], y[5], y[6], y[7]}), rs, off + 16, 0,
                                           LAVR_STORE_CPOL);
  }
}

// Paired bf16 store of both halves' pieces as whole 128-byte lines (lanes tl
// and tl ^ 8 trade one piece, as in the readout), or one half alone.
__device__ __forceinline__ void store_pair(const u32x4* pk, int nh, int tl, __amdgpu_buffer_rsrc_t rs,
                                           int off_pair, int off_one, int RO) {
  if (nh == 2) {
    const bool lo = tl < 8;
    uint32_t first[4], second[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p0 = pk[0][i], p1 = pk[1][i];
      const uint32_t snd = lo ? p1 : p0;
      const uint32_t rcv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd, 0x128, 0xf, 0xf, false);
      first[i] = lo ? p0 : rcv;
      second[i] = lo ? rcv : p1;
    }
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{first[0], first[1], first[2], first[3]}, rs, off_pair, 0,
                                           LAVR_STORE_CPOL);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{second[0], second[1], second[2], second[3]}, rs,
                                           off_pair + 8 * RO, 0, LAVR_STORE_CPOL);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(pk[0], rs, off_one, 0, LAVR_STORE_CPOL);
  }
}

// ------------------------------------------------------------------ k_bw_kv
//
// Grid and token layout as k_readout (tiles of one block; a head pair at head
// dim 32, one head at 64).  Per token: kappa = R phi(k), dv = dS kappa,
// dkappa = dS^T v, dk = [k > 0] (R^T dkappa + dz), both products on MFMA with
// row-permuted operand blocks of dS and dS^T read from LDS (at head dim 64 each
// output half sums the products of both input halves).

template <typename TIn, typename TOut, bool P2, int DH>
__global__ __launch_bounds__(NT, 2) void k_bw_kv(BwKVArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr bool W64 = DH == 64;
  constexpr int NB = W64 ? 4 : 2;
  constexpr int RECN = DH * DH + DH;
  constexpr int ES = (int)sizeof(TIn), EO = (int)sizeof(TOut);
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* ops = reinterpret_cast<u32x4*>(smem);                      // [2 NB blocks][4 slots][64 lanes]
  float2* tab = reinterpret_cast<float2*>(ops + 2 * NB * OPS_BLOCK);

  const int g = blockIdx.x % a.hg;
  const int ti = blockIdx.x / a.hg;
  const int b = blockIdx.y;
  const int j = ti / a.rpb;
  const int r = ti - j * a.rpb;
  const int blk0 = block_start(j, a.L0, a.L);
  const int blk1 = min(blk0 + (j == 0 ? a.L0 : a.L), a.N);
  const int t0 = min(blk0 + r * a.Tr, blk1);
  const int t1 = min(t0 + a.Tr, blk1);
  if (t0 >= t1) return;
  const bool rope_on = a.rope.table != nullptr;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tl = lane & 15, ch = lane >> 4;
  const int h0 = W64 ? g : 2 * g;
  const int nh = W64 ? 2 : min(2, a.H - h0);      // 32-channel halves that hold data
  const int ngroups = (t1 - t0 + 15) >> 4;

  const int RB = a.H * DH * ES, RO = a.H * DH * EO;
  const size_t row0 = (size_t)b * a.N + t0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + row0 * RB, (uint32_t)(t1 - t0) * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + row0 * RB, (uint32_t)(t1 - t0) * RB);
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc(static_cast<char*>(a.dk) + row0 * RO, (uint32_t)(t1 - t0) * RO);
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc(static_cast<char*>(a.dv) + row0 * RO, (uint32_t)(t1 - t0) * RO);
  int ioff = (w * 16 + tl) * RB + (g * 64 + 8 * ch) * ES;
  int ooff = (w * 16) * RO + g * 64 * EO;
  const int o_one = tl * RO + 8 * ch * EO;
  const int o_pair = (tl & 7) * RO + ((tl >> 3) * D + 8 * ch) * EO;

  // Prologue: the rotary window and the block's suffix record (dS, dz) are
  // loaded together, so that one memory latency covers both, then the window
  // and the operand blocks go to LDS, then the first K/V groups are loaded.
  TabStage ts;
  ts.issue(a.rope, a.pos.t0, t0, t1, a.pos.mag_tpf);
  const TabWindow win = ts.w;

  // dS and dS^T operand blocks of block j in LDS; dz slices per half.
  const float* rec0 = a.suffix + ((size_t)(b * a.H + h0) * a.nb + j) * RECN;
  const float* rec1 = a.suffix + ((size_t)(b * a.H + h0 + (nh - 1)) * a.nb + j) * RECN;
  OpsStage<BF, W64, 2> os;
  os.issue(rec0, rec1, w, lane);
  float dzb[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* zp = W64 ? rec0 + DH * DH + h * D : (h == 0 ? rec0 : rec1) + D * D;
#pragma unroll
    for (int i = 0; i < 8; ++i) dzb[h][i] = zp[8 * ch + i];
  }

  ts.commit(tab);
  RopeLane<P2> rl, rl1;                  // rl1: the second half at head dim 64
  TokPos tp;
  if (rope_on) {
    rl.init(a.rope, win, ch);
    if constexpr (W64) rl1.init(a.rope, win, ch + 4);
    tp.init(t0 + w * 16 + tl, a.pos);
  }
  os.commit(ops, w, lane);

  struct Buf { Raw8<TIn> k[2], v[2]; };
  auto load_group = [&](Buf& bf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf.k[h] = bload8<TIn>(rk, ioff + h * D * ES);
      bf.v[h] = bload8<TIn>(rv, ioff + h * D * ES);
    }
    ioff += 64 * RB;
  };
  Buf b0, b1;
  load_group(b0);
  load_group(b1);
  __syncthreads();

  auto run_group = [&](const Buf& bf) {
    // At head dim 64 the operand blocks (32 tiles) are read from LDS where they
    // are used; an empty asm with a memory clobber keeps the compiler from
    // hoisting those reads out of the loop into 128 registers.
    if constexpr (W64) __asm__ volatile("" ::: "memory");
    float2 cs[4], cs1[4];
    if (rope_on) {
      rl.fetch(tab, tp, win, cs);
      if constexpr (W64) rl1.fetch(tab, tp, win, cs1);
      tp.advance(a.pos);
    }
    float kx[2][8], kap[2][8], vx[2][8];
    u32x4 kh[2], kl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      relu_widen(bf.k[h], kx[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) kap[h][i] = kx[h][i];
      if (rope_on) rotate8(kap[h], (W64 && h == 1) ? cs1 : cs);
      if constexpr (BF) split8(kap[h], kh[h], kl[h]);
      else widen8(bf.v[h], vx[h]);
    }
    u32x4 pkk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}}, pkv[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {                   // output half
      if (h >= nh) break;
      f32x4 cv[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, ck[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int x = 0; x < (W64 ? 2 : 1); ++x) {     // input half
        const int xi = W64 ? x : h;
        const int blk = W64 ? 2 * h + x : h;
        if constexpr (BF) {
          mv_acc<true>(ops + blk * OPS_BLOCK, lane, kh[xi], &kl[xi], nullptr, cv);
          mv_acc<true>(ops + (NB + blk) * OPS_BLOCK, lane, bf.v[xi].r[0], nullptr, nullptr, ck);   // v exact in bf16
        } else {
          mv_acc<false>(ops + blk * OPS_BLOCK, lane, u32x4{}, nullptr, kap[xi], cv);
          mv_acc<false>(ops + (NB + blk) * OPS_BLOCK, lane, u32x4{}, nullptr, vx[xi], ck);
        }
      }
      float dv[8], dka[8];
      take8(cv, dv);
      take8(ck, dka);
      if (rope_on) unrotate8(dka, (W64 && h == 1) ? cs1 : cs);
#pragma unroll
      for (int i = 0; i < 8; ++i) dka[i] = kx[h][i] > 0.f ? dka[i] + dzb[h][i] : 0.f;
      put8<EO>(dka, h, pkk, rdk, ooff + o_one + h * D * EO);
      put8<EO>(dv, h, pkv, rdv, ooff + o_one + h * D * EO);
    }
    if constexpr (EO == 2) {
      store_pair(pkk, nh, tl, rdk, ooff + o_pair, ooff + o_one, RO);
      store_pair(pkv, nh, tl, rdv, ooff + o_pair, ooff + o_one, RO);
    }
    ooff += 64 * RO;
  };

  for (int gi = w; gi < ngroups; gi += 8) {
    run_group(b0);
    load_group(b0);
    run_group(b1);
    load_group(b1);
  }
}

// ------------------------------------------------------------------- k_bw_q
//
// Grid as k_block_state (chunks of one block; a head pair at head dim 32, one
// head at 64); token layout as k_readout, wave w taking the chunk's 16-token
// groups w, w+4, ...  One matrix-vector product per token does both jobs of
// Sbar: u = Sbar^T g (MFMA, row-permuted operand blocks of Sbar^T from LDS)
// gives g . num = u . r (num = Sbar r) and Sbar^T a = u / den, so
//   beta = -(u . r) / den^2,  dq = [q > 0] (R^T u / den + beta zbar).
// G = sum a r^T = sum g (r / den)^T goes through a per-wave LDS tile [16
// tokens][2 halves x 32] holding g (exact in bf16, or fp32) and r / den (bf16
// hi and lo, or fp32), read back transposed into 32x32 MFMAs over the group's
// tokens: one 32 x 32 block per head at head dim 32; at 64 wave w takes
// quadrant w of the 64 x 64 G over the four waves' tiles.  gz = sum beta p
// stays in registers.  At the end the waves' partials are added through LDS
// (over the tiles, no longer needed) and written as the chunk's (G, gz) records.

template <typename TIn, typename TOut, bool P2, int DH>
__global__ __launch_bounds__(NT, 2) void k_bw_q(BwQArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr bool W64 = DH == 64;
  constexpr int NB = W64 ? 4 : 2;                    // operand blocks of Sbar^T
  constexpr int RECN = DH * DH + DH;
  constexpr int ES = (int)sizeof(TIn), EO = (int)sizeof(TOut);
  constexpr int WT = 16 * TCOLS;                     // elements of one wave tile array
  constexpr int WAVE_BYTES = BF ? 3 * WT * 2 : 2 * WT * 4;   // g, r/den hi, lo (bf16) or g, r/den (fp32)
  constexpr int RED_FLOATS = W64 ? DH * DH : 4 * 2 * D * D;  // waves' G partials at the end
  constexpr int PFQ = !BF ? 2 : W64 ? LAVR_BWQ_PF64 : LAVR_BWQ_PF;   // 16-token groups of loads in flight per wave
  static_assert(PFQ == 2 || PFQ == 3, "k_bw_q prefetch depth: two or three register buffers");
  static_assert(4 * WAVE_BYTES + NB * OPS_BLOCK * 16 >= RED_FLOATS * 4, "reduction space");
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* ops = reinterpret_cast<u32x4*>(smem + 4 * WAVE_BYTES);   // [NB blocks][4 slots][64 lanes]
  float* zred = reinterpret_cast<float*>(ops + NB * OPS_BLOCK);    // [4 waves][2 halves][32]
  float* zl = zred + 4 * 2 * D;                                     // zbar of the block (head dim 64)
  // bf16 at head dim 32: the normaliser zbar . phi(q) on MFMA; zbar's hi and lo
  // bf16 parts as its A operand ([head][part][lane row], 256 bytes) take the
  // slot that holds zbar at 64.
  constexpr bool PKD = BF && !W64;
  u32x4* zsel = reinterpret_cast<u32x4*>(zl);
  float2* tab = reinterpret_cast<float2*>(zl + 2 * D);
  float* red = reinterpret_cast<float*>(smem);       // after the loop, over tiles + operands

  const int g = blockIdx.x % a.hg;
  const int ci = blockIdx.x / a.hg;
  const int b = blockIdx.y;
  const int j = ci / a.cpb;
  const int c = ci - j * a.cpb;
  const int blk0 = block_start(j, a.L0, a.L);
  const int blk1 = min(blk0 + (j == 0 ? a.L0 : a.L), a.N);
  const int c0 = min(blk0 + c * a.Tc, blk1);
  const int c1 = min(c0 + a.Tc, blk1);
  const bool rope_on = a.rope.table != nullptr;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tl = lane & 15, ch = lane >> 4;
  const int h0 = W64 ? g : 2 * g;
  const int nh = W64 ? 2 : min(2, a.H - h0);      // 32-channel halves that hold data
  const int ngroups = (c1 - c0 + 15) >> 4;
  unsigned char* wtile = smem + w * WAVE_BYTES;

  const int RB = a.H * DH * ES, RO = a.H * DH * EO;
  const size_t row0 = (size_t)b * a.N + c0;
  const uint32_t span = (uint32_t)(c1 - c0);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + row0 * RB, span * RB);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(static_cast<const char*>(a.g) + row0 * RB, span * RB);
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(static_cast<char*>(a.dq) + row0 * RO, span * RO);
  int ioff = (w * 16 + tl) * RB + (g * 64 + 8 * ch) * ES;
  int ooff = (w * 16) * RO + g * 64 * EO;
  const int o_one = tl * RO + 8 * ch * EO;
  const int o_pair = (tl & 7) * RO + ((tl >> 3) * D + 8 * ch) * EO;

  // Prologue: the rotary window and the block's prefix record (Sbar, zbar)
  // are loaded together, so that one memory latency covers both, then the
  // window and the operand blocks go to LDS, then the first q/g groups are
  // loaded.
  TabStage ts;
  ts.issue(a.rope, a.pos.t0, c0, c1, a.pos.mag_tpf);
  const TabWindow win = ts.w;

  // Sbar^T operand blocks of block j in LDS (the same for every wave); zbar
  // slices per half: in registers at 32, at 64 in LDS, read per group
  // (registers are the limit there).
  const float* rec0 = a.prefix + ((size_t)(b * a.H + h0) * a.nb + j) * RECN;
  const float* rec1 = a.prefix + ((size_t)(b * a.H + h0 + (nh - 1)) * a.nb + j) * RECN;
  OpsStage<BF, W64, 1> os;
  os.issue(rec0, rec1, w, lane);
  float zb[2][8];
  float z64 = 0.f;
  if constexpr (W64) {
    z64 = rec0[DH * DH + (threadIdx.x & (DH - 1))];
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* zp = (h == 0 ? rec0 : rec1) + D * D;
#pragma unroll
      for (int i = 0; i < 8; ++i) zb[h][i] = zp[8 * ch + i];
    }
  }

  ts.commit(tab);
  RopeLane<P2> rl, rl1;                  // rl1: the second half at head dim 64
  TokPos tp;
  if (rope_on) {
    rl.init(a.rope, win, ch);
    if constexpr (W64) rl1.init(a.rope, win, ch + 4);
    tp.init(c0 + w * 16 + tl, a.pos);
  }
  os.commit(ops, w, lane);
  if constexpr (W64) {
    if (threadIdx.x < DH) zl[threadIdx.x] = z64;
  } else if constexpr (PKD) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (w == 0 && tl == 0) {
        u32x4 hi, lo;
        split8d(zb[h], hi, lo);
        zsel[(2 * h) * 4 + ch] = hi;
        zsel[(2 * h + 1) * 4 + ch] = lo;
      }
    }
  }

  struct Buf { Raw8<TIn> q[2], g[2]; };
  auto load_group = [&](Buf& bf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf.q[h] = bload8<TIn>(rq, ioff + h * D * ES);
      bf.g[h] = bload8<TIn>(rg, ioff + h * D * ES);
    }
    ioff += 64 * RB;
  };
  // The lane's token within the chunk, for the group being processed: tokens
  // past the chunk read zeros and must add nothing to G (1/den is taken as 0
  // there, which also keeps eps = 0 from turning them into NaN).
  int tok = w * 16 + tl;
  Buf b0, b1, b2;
  load_group(b0);
  load_group(b1);
  if constexpr (PFQ > 2) load_group(b2);
  __syncthreads();

  // G accumulators: at 32 each wave adds both heads' blocks over its own
  // tokens; at 64 wave w adds quadrant w (g's half w >> 1 against (r/den)'s
  // half w & 1) over the tokens of all four waves' tiles.
  constexpr int NACC = W64 ? 1 : NB;
  f32x16 gacc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) gacc[q] = f32x16{};
  float zacc[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) zacc[h][i] = 0.f;

  // Per-wave tile: row tl, columns h*32 + 8ch .. +7; odd groups of 8 rows keep
  // the two halves swapped (as the block-state tiles) so transposed reads of
  // the two half-waves hit different banks.  Arrays: 0 = g, 1 = r/den (hi), 2
  // = r/den (lo) in bf16; 0 = g, 1 = r/den in fp32.
  const int tcol = (8 * ch) ^ (((tl >> 3) & 1) << 5);
  auto tile_put16 = [&](int arr, int h, u32x4 x) {      // bf16 arrays
    uint16_t* t16 = reinterpret_cast<uint16_t*>(wtile) + arr * WT;
    *reinterpret_cast<u32x4*>(t16 + tl * TCOLS + (tcol ^ (h * D))) = x;
  };
  auto tile_put32 = [&](int arr, int h, const float* x) {   // fp32 arrays
    float* t32 = reinterpret_cast<float*>(wtile) + arr * WT;
    f32x4* dst = reinterpret_cast<f32x4*>(t32 + tl * TCOLS + (tcol ^ (h * D)));
    dst[0] = f32x4{x[0], x[1], x[2], x[3]};
    dst[1] = f32x4{x[4], x[5], x[6], x[7]};
  };

  auto run_group = [&](const Buf& bf) {
    if constexpr (W64) {
      __asm__ volatile("" ::: "memory");   // operand and zbar reads stay in the loop
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zl + h * D + 8 * ch);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zl + h * D + 8 * ch + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { zb[h][i] = z0[i]; zb[h][4 + i] = z1[i]; }
      }
    }
    float2 cs[4], cs1[4];
    if (rope_on) {
      rl.fetch(tab, tp, win, cs);
      if constexpr (W64) rl1.fetch(tab, tp, win, cs1);
      tp.advance(a.pos);
    }
    float p[2][8], rr[2][8], gx[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      relu_widen(bf.q[h], p[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) rr[h][i] = p[h][i];
      if (rope_on) rotate8(rr[h], (W64 && h == 1) ? cs1 : cs);
      if constexpr (BF) tile_put16(0, h, bf.g[h].r[0]);        // g, exact in bf16
      else {
        widen8(bf.g[h], gx[h]);
        tile_put32(0, h, gx[h]);
      }
    }
    // u = Sbar^T g per output half (at 64 both input halves contribute), then
    // u . r and z . phi(q)
    float u[2][8], ur[2], den_h[2];
    // PKD: a lane's A operand is zbar's hi part for output rows 0-7 (tl < 8)
    // and its lo part for rows 8-15; an opaque copy of the row index keeps the
    // compiler from hoisting the reads into registers.
    int zrow = ch + ((tl >> 3) << 2);
    if constexpr (PKD) asm volatile("" : "+v"(zrow));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 cc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int x = 0; x < (W64 ? 2 : 1); ++x) {
        const int xi = W64 ? x : h, blk = W64 ? 2 * h + x : h;
        mv_acc<BF>(ops + blk * OPS_BLOCK, lane, bf.g[xi].r[0], nullptr, gx[xi], cc);
      }
      take8(cc, u[h]);
      ur[h] = 0.f;
      den_h[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ur[h] += u[h][i] * rr[h][i];
      if constexpr (PKD) {
        const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(zsel[8 * h + zrow]),
                                                                 as_bf16x8(relu_pk(bf.q[h].r[0])),
                                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        den_h[h] = den_rows(dd[0]);             // the whole head's sum
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) den_h[h] += zb[h][i] * p[h][i];
      }
    }
    // 1/den and beta: per head at 32, over both halves at 64 (v_rcp_f32, as in the readout)
    const bool live = tok < (int)span;
    tok += 64;
    float inv[2], beta[2];
    if constexpr (W64) {
      const float dsum = sum4_lanes(den_h[0] + den_h[1]), usum = sum4_lanes(ur[0] + ur[1]);
      const float iv = live ? __builtin_amdgcn_rcpf(dsum + a.eps) : 0.f;
      inv[0] = inv[1] = iv;
      beta[0] = beta[1] = -usum * (iv * iv);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float dsum = PKD ? den_h[h] : sum4_lanes(den_h[h]), usum = sum4_lanes(ur[h]);
        inv[h] = live ? __builtin_amdgcn_rcpf(dsum + a.eps) : 0.f;
        beta[h] = -usum * (inv[h] * inv[h]);
      }
    }
    u32x4 pk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // r / den into the tile for G
      float rs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rs[i] = rr[h][i] * inv[h];
      if constexpr (BF) {
        u32x4 hi, lo;
        split8d(rs, hi, lo);
        tile_put16(1, h, hi);
        tile_put16(2, h, lo);
      } else {
        tile_put32(1, h, rs);
      }
      // dq = [q > 0] (R^T u / den + beta zbar); gz += beta phi(q)
      float sa[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sa[i] = u[h][i] * inv[h];
      if (rope_on) unrotate8(sa, (W64 && h == 1) ? cs1 : cs);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sa[i] = p[h][i] > 0.f ? sa[i] + beta[h] * zb[h][i] : 0.f;
        zacc[h][i] += beta[h] * p[h][i];
      }
      if (h < nh) put8<EO>(sa, h, pk, rdq, ooff + o_one + h * D * EO);
    }
    if constexpr (EO == 2) store_pair(pk, nh, tl, rdq, ooff + o_pair, ooff + o_one, RO);
    ooff += 64 * RO;
  };

  // G += g (r/den)^T over 16 tokens of tile `src` (a wave's tile): block (qa,
  // qb) takes g's half qa against (r/den)'s half qb into accumulator q.
  auto g_block = [&](const unsigned char* src, int q, int qa, int qb) {
    if constexpr (BF) {
      const uint16_t* t16 = reinterpret_cast<const uint16_t*>(src);
      const int Gq = lane >> 4, jr = (lane >> 2) & 3, js = lane & 3;
      const int r0 = 8 * (Gq >> 1) + jr;
      const int ca = ((qa * D) ^ ((Gq >> 1) << 5)) + 16 * (Gq & 1) + 4 * js;
      const int cb = ((qb * D) ^ ((Gq >> 1) << 5)) + 16 * (Gq & 1) + 4 * js;
      const int ea = r0 * TCOLS + ca, eb = r0 * TCOLS + cb;
      const u32x4 gA = tr_pair(t16, ea, ea + 4 * TCOLS);
      const u32x4 rH = tr_pair(t16 + WT, eb, eb + 4 * TCOLS), rL = tr_pair(t16 + 2 * WT, eb, eb + 4 * TCOLS);
      gacc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(gA), as_bf16x8(rH), gacc[q], 0, 0, 0);
      gacc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(gA), as_bf16x8(rL), gacc[q], 0, 0, 0);
    } else {
      const float* af = reinterpret_cast<const float*>(src);
      const float* rf = af + WT;
      const int cl = lane & 31, qq = lane >> 5;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int row = 2 * s + qq;
        const int sw = ((row >> 3) & 1) << 5;
        gacc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[row * TCOLS + ((qa * D + cl) ^ sw)],
                                                       rf[row * TCOLS + ((qb * D + cl) ^ sw)], gacc[q], 0, 0, 0);
      }
    }
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // After a group's tiles are written: at 32 the wave's own two head blocks; at
  // 64 quadrant w over the four waves' tiles, between workgroup barriers (so
  // every wave runs the same number of groups; groups past the chunk are zeros).
  auto g_step = [&]() {
    if constexpr (W64) {
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) g_block(smem + tt * WAVE_BYTES, 0, w >> 1, w & 1);
      __syncthreads();
    } else {
      wave_sync();
#pragma unroll
      for (int q = 0; q < NB; ++q) g_block(wtile, q, q, q);
      wave_sync();
    }
  };

  // PFQ groups per wave per iteration (4 PFQ per workgroup); uniform at 64
  const int iters = W64 ? (ngroups + 4 * PFQ - 1) / (4 * PFQ) : (ngroups - w + 4 * PFQ - 1) / (4 * PFQ);
  for (int it = 0; it < iters; ++it) {
    run_group(b0);
    g_step();
    load_group(b0);
    run_group(b1);
    g_step();
    load_group(b1);
    if constexpr (PFQ > 2) {
      run_group(b2);
      g_step();
      load_group(b2);
    }
  }

  // Sum the four waves: G through LDS (over the tiles and operand blocks), gz
  // across the 16 lanes of a row (the chunk's tokens) and then the waves.
  // red holds each wave's G as [32 NB / 2 rows][...]: at 32 two 32 x 32 heads,
  // at 64 the 64 x 64 matrix.
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NACC; ++q) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      // at 64: wave w's quadrant straight into the one 64 x 64 G (the four
      // waves hold the four quadrants, already summed over every token)
      if constexpr (W64) red[(32 * (w >> 1) + e) * DH + 32 * (w & 1) + (lane & 31)] = gacc[q][v];
      else red[((w * 2 + q) * D + e) * D + (lane & 31)] = gacc[q][v];
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = zacc[h][i];
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x121, 0xf, 0xf, false));
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x122, 0xf, 0xf, false));
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x124, 0xf, 0xf, false));
      s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x128, 0xf, 0xf, false));
      if (tl == 0) zred[(w * 2 + h) * D + 8 * ch + i] = s;
    }
  }
  __syncthreads();
  if constexpr (W64) {
    // one record: G (64 x 64) then gz (64)
    for (int o = threadIdx.x; o < RECN; o += NT) {
      float s;
      if (o < DH * DH) {
        s = red[o];
      } else {
        const int f = o - DH * DH;
        s = zred[f] + zred[2 * D + f] + zred[4 * D + f] + zred[6 * D + f];
      }
      a.part[part_rec((size_t)(b * a.H + h0), ci, (size_t)gridDim.y * a.H) * RECN + o] = s;
    }
  } else {
    for (int el = threadIdx.x; el < 2 * RECN; el += NT) {
      const int h = el / RECN, o = el - h * RECN;
      if (h >= nh) break;
      float s;
      if (o < D * D) {
        s = red[((0 * 2 + h) * D * D) + o] + red[((1 * 2 + h) * D * D) + o] + red[((2 * 2 + h) * D * D) + o] +
            red[((3 * 2 + h) * D * D) + o];
      } else {
        const int f = o - D * D;
        s = zred[(0 * 2 + h) * D + f] + zred[(1 * 2 + h) * D + f] + zred[(2 * 2 + h) * D + f] +
            zred[(3 * 2 + h) * D + f];
      }
      a.part[part_rec((size_t)(b * a.H + h0 + h), ci, (size_t)gridDim.y * a.H) * RECN + o] = s;
    }
  }
}

// ---------------------------------------------------------------- helpers

__global__ void k_rope_table(float2* tab, int pt, int ph, int pw, int max_frames, int gh, int gw,
                             double base) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nt = (long long)max_frames * pt, nh = (long long)gh * ph, nw = (long long)gw * pw;
  if (i >= nt + nh + nw) return;
  long long pos;
  int pair, np;
  if (i < nt) {
    pos = i / pt; pair = (int)(i % pt); np = pt;
  } else if (i < nt + nh) {
    pos = (i - nt) / ph; pair = (int)((i - nt) % ph); np = ph;
  } else {
    pos = (i - nt - nh) / pw; pair = (int)((i - nt - nh) % pw); np = pw;
  }
  // pair `pair` of a section of width d_s = 2 np turns by pos * base^(-2 pair / d_s)
  const double theta = pow(base, -(2.0 * pair) / (2.0 * np));
  const double ang = (double)pos * theta;
  tab[i] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ void k_fill_zero(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------- k_tconv
//
// Cached temporal convolution of the causal Mix-FFN: depthwise along frames,
// y[t] = sum_i w[i] * x[t + i - 1] over the kt taps (kt = 3: frames t-1, t,
// t+1; kt = 2: t-1, t), plus an optional bias.  Inside a block the taps see the
// block's frames; before the first frame of the call they see the cache (the
// previous block's last frame, or zeros), before a later block's first frame
// the last frame of the block before, and after a block's last frame zeros.
// Grid: x = 256-thread groups over (spatial position, 8-channel piece), y =
// batch.  A thread owns one position's 8 channels and walks the call's frames
// in order with the window (prev, cur, next) in registers and loads running
// PF frames ahead, so every input element is read from memory once and every
// output written once; consecutive threads cover consecutive 16-byte pieces of
// a token row.  The frame after the call reads zero through the buffer range.
struct ConvArgs {
  const void* x;
  void* y;
  const float* w;            // (kt, Ch) taps, tap 0 = previous frame
  const float* bias;         // (Ch) or nullptr
  const void* cache_in;      // (B, P, Ch) in x's dtype, or nullptr (zeros)
  void* cache_out;           // (B, P, Ch): receives the call's last frame, or nullptr
  int F, P, Ch;              // frames of the call, tokens per frame, channels
  int F0, BF;                // frames of the first block and of later blocks
  int kt;
  int seg;                   // frames per segment (grid z); a segment re-reads the frame before it
};

template <typename TIn, typename TOut>
__global__ __launch_bounds__(NT) void k_tconv(ConvArgs a) {
  constexpr int ES = (int)sizeof(TIn), EO = (int)sizeof(TOut);
  constexpr int PF = 4;                                // ring of raw frames f .. f + 3
  const int pieces = a.Ch / 8;
  const int gid = blockIdx.x * NT + threadIdx.x;
  if (gid >= a.P * pieces) return;
  const int b = blockIdx.y;
  const int pos = gid / pieces, cp = gid - pos * pieces;
  const int c0 = 8 * cp;
  // This thread's frames [fs, fe): segment blockIdx.z of a.seg frames.
  const int fs = blockIdx.z * a.seg;
  const int fe = min(a.F, fs + a.seg);
  const uint32_t frame_in = (uint32_t)a.P * a.Ch * ES, frame_out = (uint32_t)a.P * a.Ch * EO;
  const uint32_t col_in = (uint32_t)(pos * a.Ch + c0) * ES, col_out = (uint32_t)(pos * a.Ch + c0) * EO;
  // Loads see frames up to fe (the next tap of the segment's last frame);
  // stores only the segment's own frames.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char*>(a.x) + (size_t)b * a.F * frame_in,
                                              (uint32_t)min(a.F, fe + 1) * frame_in);
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(static_cast<char*>(a.y) + (size_t)b * a.F * frame_out, (uint32_t)fe * frame_out);

  float w0[8], w1[8], w2[8], bs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w0[i] = a.w[c0 + i];
    w1[i] = a.w[a.Ch + c0 + i];
    w2[i] = a.kt == 3 ? a.w[2 * a.Ch + c0 + i] : 0.f;
    bs[i] = a.bias != nullptr ? a.bias[c0 + i] : 0.f;
  }
  // The window stays in its raw input form (widened where used).  The frame
  // before the segment: the previous frame of the call, else the cache, else 0.
  Raw8<TIn> prev;
  if (fs > 0) {
    prev = bload8<TIn>(rx, (uint32_t)(fs - 1) * frame_in + col_in);
  } else if (a.cache_in != nullptr) {
    const TIn* cin = static_cast<const TIn*>(a.cache_in) + ((size_t)b * a.P + pos) * a.Ch + c0;
#pragma unroll
    for (int i = 0; i < ES / 2; ++i) prev.r[i] = *reinterpret_cast<const u32x4*>(cin + i * (16 / ES));
  } else {
#pragma unroll
    for (int i = 0; i < ES / 2; ++i) prev.r[i] = u32x4{0u, 0u, 0u, 0u};
  }
  Raw8<TIn> ring[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) ring[k] = bload8<TIn>(rx, (uint32_t)(fs + k) * frame_in + col_in);
  // frames left in the block holding frame fs
  int rem = fs < a.F0 ? a.F0 - fs : a.BF - (fs - a.F0) % a.BF;
  // Whole passes of PF frames; frames past the segment compute on what the
  // load range gives and their stores fall outside the store range (dropped),
  // so no load is conditional.  Slot k holds frame f when frame f is produced,
  // slot k + 1 frame f + 1; slot k is then refilled with frame f + PF.
  for (int f0 = fs; f0 < fe; f0 += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int f = f0 + k;
      const bool block_end = rem == 1;
      float xp[8], xc[8], xn[8], o[8];
      widen8(prev, xp);
      widen8(ring[k], xc);
      widen8(ring[(k + 1) % PF], xn);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = bs[i] + w0[i] * xp[i] + w1[i] * xc[i] + (block_end ? 0.f : w2[i] * xn[i]);
      if constexpr (EO == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])},
            ry, (uint32_t)f * frame_out + col_out, 0, LAVR_STORE_CPOL);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{o[0], o[1], o[2], o[3]}), ry,
                                               (uint32_t)f * frame_out + col_out, 0, LAVR_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{o[4], o[5], o[6], o[7]}), ry,
                                               (uint32_t)f * frame_out + col_out + 16, 0, LAVR_STORE_CPOL);
      }
      rem = block_end ? a.BF : rem - 1;
      prev = ring[k];
      ring[k] = bload8<TIn>(rx, (uint32_t)(f + PF) * frame_in + col_in);   // zeros past the load range
    }
  }
  if (a.cache_out != nullptr && fe == a.F) {
    // the call's last frame, read again (cache_out may be cache_in: this thread
    // read its element of the old cache above)
    const Raw8<TIn> r = bload8<TIn>(rx, (uint32_t)(a.F - 1) * frame_in + col_in);
    TIn* cout = static_cast<TIn*>(a.cache_out) + ((size_t)b * a.P + pos) * a.Ch + c0;
#pragma unroll
    for (int i = 0; i < ES / 2; ++i) *reinterpret_cast<u32x4*>(cout + i * (16 / ES)) = r.r[i];
  }
}

// ---------------------------------------------------------------- k_qk_rms
//
// Token scales of the q/k RMSNorm: 1 / sqrt(mean(x^2) + norm_eps) of each
// token's q row and k row over its C channels.  One wave per token, grid-stride
// over the tokens: lane l reads the 8-channel pieces l, l + 64, ... of both
// rows, adds their squares in fp32, and the wave adds its lanes.  A tensor that
// is not normalised gets an empty buffer range (its loads read zeros and touch
// no memory).  The channel weights are applied where q and k are consumed.
struct RmsArgs {
  const void* q;
  const void* k;
  float* sq;
  float* sk;
  long long ntok;            // token rows (B * N)
  int row_in;                // elements from one token row to the next
  int C;                     // channels per row (a multiple of 8)
  float norm_eps;
};

template <typename TIn>
__global__ __launch_bounds__(NT) void k_qk_rms(RmsArgs a) {
  constexpr int ES = (int)sizeof(TIn);
  const int lane = threadIdx.x & 63;
  const long long nwaves = (long long)gridDim.x * (NT / 64);
  const int pieces = a.C / 8;
  const uint32_t row_bytes = (uint32_t)a.C * ES;
  const char* bq = static_cast<const char*>(a.q != nullptr ? a.q : a.k);
  const char* bk = static_cast<const char*>(a.k != nullptr ? a.k : a.q);
  const float inv_c = 1.0f / (float)a.C;
  for (long long tok = ((long long)blockIdx.x * NT + threadIdx.x) >> 6; tok < a.ntok; tok += nwaves) {
    const size_t off = (size_t)tok * a.row_in * ES;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(bq + off, a.q != nullptr ? row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(bk + off, a.k != nullptr ? row_bytes : 0u);
    float sq = 0.f, sk = 0.f;
#pragma unroll 4
    for (int pc = lane; pc < pieces; pc += 64) {
      float fq[8], fk[8];
      widen8(bload8<TIn>(rq, pc * 8 * ES), fq);
      widen8(bload8<TIn>(rk, pc * 8 * ES), fk);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sq += fq[i] * fq[i];
        sk += fk[i] * fk[i];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sq += __shfl_xor(sq, m, 64);
      sk += __shfl_xor(sk, m, 64);
    }
    if (lane == 0) {
      if (a.sq != nullptr) a.sq[tok] = 1.0f / sqrtf(sq * inv_c + a.norm_eps);
      if (a.sk != nullptr) a.sk[tok] = 1.0f / sqrtf(sk * inv_c + a.norm_eps);
    }
  }
}

// Timing events of one launch.  A caller's events are bound to the kernel's
// own dispatch (hipExtLaunchKernel): they take its start and end times and add
// no command to the stream, where an event record between two kernels leaves
// a gap of several microseconds in the timeline.
struct KEv {
  hipEvent_t start = nullptr, stop = nullptr;
  bool any() const { return start != nullptr || stop != nullptr; }
};

#define LAVR_LAUNCH(KER, GRID, LDS, S, EV, ARG)                                            \
  do {                                                                                     \
    if ((EV).any()) hipExtLaunchKernelGGL(KER, GRID, dim3(NT), LDS, S, (EV).start, (EV).stop, 0u, ARG); \
    else hipLaunchKernelGGL(KER, GRID, dim3(NT), LDS, S, ARG);                             \
  } while (0)

template <typename TIn, typename TOut, int DH, bool NRM>
hipError_t launch_readout(const ReadArgs& ra, bool p2, dim3 grid, int lds, hipStream_t s, KEv ev) {
  if (ra.rope.table == nullptr) LAVR_LAUNCH((k_readout<TIn, TOut, true, DH, NRM, false>), grid, lds, s, ev, ra);
  else if (p2) LAVR_LAUNCH((k_readout<TIn, TOut, true, DH, NRM, true>), grid, lds, s, ev, ra);
  else LAVR_LAUNCH((k_readout<TIn, TOut, false, DH, NRM, true>), grid, lds, s, ev, ra);
  return hipGetLastError();
}

template <int DH, bool NRM>
hipError_t launch_state_n(const StateArgs& sa, bool in_bf16, bool p2, dim3 grid, int lds, int lds1, hipStream_t s,
                          KEv ev) {
  // Packed bf16 at head dim 32: a launch of at most one round at four
  // workgroups per CU takes single-buffered tiles (lds1 bytes), so that it runs
  // as one round; longer launches keep two tile sets per workgroup.
  if constexpr (DH == 32 && !NRM) {
    if (in_bf16 && p2 && (long long)grid.x * grid.y <= 4LL * 256) {
      LAVR_LAUNCH((k_block_state<uint16_t, true, DH, NRM, 1>), grid, lds1, s, ev, sa);
      return hipGetLastError();
    }
  }
  if (in_bf16 && p2) LAVR_LAUNCH((k_block_state<uint16_t, true, DH, NRM, kStateTileSets>), grid, lds, s, ev, sa);
  else if (in_bf16) LAVR_LAUNCH((k_block_state<uint16_t, false, DH, NRM, kStateTileSets>), grid, lds, s, ev, sa);
  else if (p2) LAVR_LAUNCH((k_block_state<float, true, DH, NRM, kStateTileSets>), grid, lds, s, ev, sa);
  else LAVR_LAUNCH((k_block_state<float, false, DH, NRM, kStateTileSets>), grid, lds, s, ev, sa);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_state(const StateArgs& sa, bool in_bf16, bool p2, dim3 grid, int lds, int lds1, hipStream_t s,
                        KEv ev = {}) {
  return sa.scale != nullptr ? launch_state_n<DH, true>(sa, in_bf16, p2, grid, lds, lds1, s, ev)
                             : launch_state_n<DH, false>(sa, in_bf16, p2, grid, lds, lds1, s, ev);
}

template <int DH, bool NRM>
hipError_t launch_readouts_n(const ReadArgs& ra, bool in_bf16, bool out_bf16, bool p2, dim3 grid, int lds,
                             hipStream_t s, KEv ev) {
  if (in_bf16 && out_bf16) return launch_readout<uint16_t, uint16_t, DH, NRM>(ra, p2, grid, lds, s, ev);
  if (in_bf16) return launch_readout<uint16_t, float, DH, NRM>(ra, p2, grid, lds, s, ev);
  if (out_bf16) return launch_readout<float, uint16_t, DH, NRM>(ra, p2, grid, lds, s, ev);
  return launch_readout<float, float, DH, NRM>(ra, p2, grid, lds, s, ev);
}

template <int DH>
hipError_t launch_readouts(const ReadArgs& ra, bool in_bf16, bool out_bf16, bool p2, dim3 grid, int lds,
                           hipStream_t s, KEv ev = {}) {
  return ra.scale != nullptr ? launch_readouts_n<DH, true>(ra, in_bf16, out_bf16, p2, grid, lds, s, ev)
                             : launch_readouts_n<DH, false>(ra, in_bf16, out_bf16, p2, grid, lds, s, ev);
}

PosArgs pos_args(const Plan& p) {
  PosArgs q;
  q.tpf = p.tpf;
  q.gw = p.gw_div;
  q.ghd = p.tpf / p.gw_div;
  q.adv_f = 64 / p.tpf;
  const int rr = 64 % p.tpf;
  q.adv_r = rr / p.gw_div;
  q.adv_c = rr % p.gw_div;
  q.t0 = p.t0;
  q.mag_tpf = p.mag_tpf;
  q.mag_gw = p.mag_gw;
  return q;
}

}  // namespace

int launch_rope_table(float* table, int pt, int ph, int pw, int max_frames, int gh, int gw,
                      double base, void* stream) {
  const long long tot = (long long)max_frames * pt + (long long)gh * ph + (long long)gw * pw;
  if (tot == 0) return (int)hipSuccess;
  const int nt = 256;
  const long long nblk = (tot + nt - 1) / nt;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)nblk), dim3(nt), 0, (hipStream_t)stream,
                     reinterpret_cast<float2*>(table), pt, ph, pw, max_frames, gh, gw, base);
  return (int)hipGetLastError();
}

// Threads a long temporal-convolution call aims for (about 5 waves per SIMD;
// measured on the 240-frame, 436800-column call: 3 segments 0.662 ms, 1 segment
// 0.678, 8 segments 0.713, 15 segments 0.869).
#ifndef TCONV_TARGET_THREADS
#define TCONV_TARGET_THREADS (5LL * 256 * 4 * 256)
#endif
int launch_tconv(const ConvPlan& c, const void* x, void* y, int in_bf16, int out_bf16, const float* w,
                 const float* bias, const void* cache_in, void* cache_out, void* stream) {
  ConvArgs a;
  a.x = x; a.y = y; a.w = w; a.bias = bias; a.cache_in = cache_in; a.cache_out = cache_out;
  a.F = c.F; a.P = c.P; a.Ch = c.Ch; a.F0 = c.F0; a.BF = c.BF; a.kt = c.kt;
  // Frame segments multiply the threads of a long call; each re-reads one
  // frame.  A call with a cache runs as one segment: its first segment reads
  // the cache that its last one may overwrite.
  const long long threads = (long long)c.P * (c.Ch / 8);
  long long nseg = (TCONV_TARGET_THREADS + threads * c.B / 2) / (threads * c.B);   // rounded
  nseg = std::max(1LL, std::min(nseg, (long long)c.F / 16));
  if (cache_in != nullptr || cache_out != nullptr) nseg = 1;
  a.seg = (int)((c.F + nseg - 1) / nseg);
  const dim3 grid((unsigned)((threads + NT - 1) / NT), (unsigned)c.B, (unsigned)((c.F + a.seg - 1) / a.seg));
  hipStream_t s = (hipStream_t)stream;
  if (in_bf16 && out_bf16) hipLaunchKernelGGL((k_tconv<uint16_t, uint16_t>), grid, dim3(NT), 0, s, a);
  else if (in_bf16) hipLaunchKernelGGL((k_tconv<uint16_t, float>), grid, dim3(NT), 0, s, a);
  else if (out_bf16) hipLaunchKernelGGL((k_tconv<float, uint16_t>), grid, dim3(NT), 0, s, a);
  else hipLaunchKernelGGL((k_tconv<float, float>), grid, dim3(NT), 0, s, a);
  return (int)hipGetLastError();
}

int launch_zero(float* p, size_t n, void* stream) {
  if (n == 0) return (int)hipSuccess;
  const int nt = 256;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + nt - 1) / nt)), dim3(nt), 0,
                     (hipStream_t)stream, p, n);
  return (int)hipGetLastError();
}

// Prefix (or, reversed, suffix) sums of the block states: one element per
// thread for a single block, the run-wise scan otherwise.
hipError_t launch_prefix(const PrefixArgs& pa, const Plan& p, hipStream_t s) {
  if (p.nb == 1) {
    const dim3 g((unsigned)((p.rec + 255) / 256), (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL(k_prefix1, g, dim3(256), 0, s, pa);
  } else {
    const dim3 g((unsigned)((p.rec + 63) / 64), (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL(k_prefix, g, dim3(PFX_NT), 0, s, pa);
  }
  return hipGetLastError();
}

// 128-bit fingerprint (two FNV-1a hashes) of everything the block prefixes of
// a call depend on: shape, block schedule, rotary table and offset, the k and v
// tensors and their normalisation.
struct Fnv {
  uint64_t h;
  void add(const void* x, size_t n) {
    const unsigned char* c = static_cast<const unsigned char*>(x);
    for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 0x100000001b3ULL;
  }
  template <typename T> void val(T v) { add(&v, sizeof(v)); }
};

void prefix_fingerprint(const Plan& p, const void* k, const void* v, int in_bf16, const Prologue* pro,
                        uint64_t* f0, uint64_t* f1) {
  Fnv a{0xcbf29ce484222325ULL}, b{0x84222325cbf29ce4ULL};
  for (Fnv* f : {&a, &b}) {
    f->val(p.B); f->val(p.H); f->val(p.D); f->val(p.N); f->val(p.row_in); f->val(p.tpf); f->val(p.gw_div);
    f->val(p.L); f->val(p.L0); f->val(p.nb); f->val(p.cpb); f->val(p.Tc); f->val(p.t0);
    f->val(p.rope.table); f->val(p.rope.pt); f->val(p.rope.ph); f->val(p.rope.pw);
    f->val(p.rope.max_frames); f->val(p.rope.gh); f->val(p.rope.gw);
    f->val(k); f->val(v); f->val(in_bf16);
    const float* kg = pro != nullptr ? pro->k_gamma : nullptr;
    f->val(kg);
    f->val(kg != nullptr ? pro->norm_eps : 0.f);
  }
  *f0 = a.h;
  *f1 = b.h;
}

// Dynamic LDS of a readout launch of `wgs` workgroups: the packed path at head
// dim 32 asks for at least the occupancy floor, so that kReadOcc workgroups
// share a CU in a launch of one such round and kReadOccN in a longer one.
int read_lds(bool floor, long long wgs, int bytes) {
  if (!floor) return bytes;
  const int f = wgs <= (long long)kReadOcc * 256 ? kReadOccLds : kReadOccLdsN;
  return bytes < f ? f : bytes;
}

int launch_forward(const Plan& p, const void* q, const void* k, const void* v, void* out,
                   int in_bf16, int out_bf16, float eps, void* ws,
                   const float* S_init, const float* z_init, float* S_save, float* z_save,
                   void* stream, void* const* events, const Prologue* pro) {
  hipStream_t s = (hipStream_t)stream;
  // events[0] / [1]: start and end of the block-state kernel, [2] / [3]: of the
  // readout, each bound to the kernel's dispatch
  auto ev = [&](int i) -> hipEvent_t { return events ? reinterpret_cast<hipEvent_t>(events[i]) : nullptr; };
  const KEv ev_state{ev(0), ev(1)}, ev_read{ev(2), ev(3)};
  hipError_t e = hipSuccess;
  const bool nq = pro != nullptr && pro->q_gamma != nullptr;
  const bool nk = pro != nullptr && pro->k_gamma != nullptr;
  if (nq || nk) {
    RmsArgs ra;
    ra.q = nq ? q : nullptr;
    ra.k = nk ? k : nullptr;
    ra.sq = nq ? pro->q_scale : nullptr;
    ra.sk = nk ? pro->k_scale : nullptr;
    ra.ntok = (long long)p.B * p.N;
    ra.row_in = p.row_in;
    ra.C = p.H * p.D;
    ra.norm_eps = pro->norm_eps;
    const long long waves = ra.ntok;
    const unsigned grid = (unsigned)std::min<long long>((waves + 3) / 4, 256LL * 8);
    if (in_bf16) hipLaunchKernelGGL(k_qk_rms<uint16_t>, dim3(grid), dim3(NT), 0, s, ra);
    else hipLaunchKernelGGL(k_qk_rms<float>, dim3(grid), dim3(NT), 0, s, ra);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_part);
  float* prefix = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_prefix);
  const PosArgs pa_pos = pos_args(p);

  StateArgs sa;
  sa.k = k; sa.v = v; sa.part = part;
  sa.scale = nk ? pro->k_scale : nullptr;
  sa.gamma = nk ? pro->k_gamma : nullptr;
  sa.H = p.H; sa.N = p.N; sa.L = p.L; sa.L0 = p.L0; sa.nb = p.nb; sa.cpb = p.cpb; sa.Tc = p.Tc; sa.hg = p.hg;
  sa.row_in = p.row_in;
  sa.pos = pa_pos;
  sa.rope = p.rope;
  sa.fp_dst = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + p.ws_fp);
  prefix_fingerprint(p, k, v, in_bf16, nk ? pro : nullptr, &sa.fp0, &sa.fp1);
  const dim3 gs((unsigned)(p.hg * p.nb * p.cpb), (unsigned)p.B);
  const bool p2 = ((p.rope.pt | p.rope.ph | p.rope.pw) & 1) == 0;
  e = p.D == 64 ? launch_state<64>(sa, in_bf16, p2, gs, p.lds_state, p.lds_state1, s, ev_state)
                : launch_state<32>(sa, in_bf16, p2, gs, p.lds_state, p.lds_state1, s, ev_state);
  if (e != hipSuccess) return (int)e;

  PrefixArgs pa;
  pa.part = part; pa.prefix = prefix; pa.S_init = S_init; pa.z_init = z_init;
  pa.S_save = S_save; pa.z_save = z_save; pa.H = p.H; pa.nb = p.nb; pa.cpb = p.cpb;
  pa.hd = p.D; pa.rec = p.rec; pa.rev = 0;
  e = launch_prefix(pa, p, s);
  if (e != hipSuccess) return (int)e;

  ReadArgs ra;
  ra.q = q; ra.out = out; ra.prefix = prefix; ra.eps = eps;
  ra.scale = nq ? pro->q_scale : nullptr;
  ra.gamma = nq ? pro->q_gamma : nullptr;
  ra.H = p.H; ra.N = p.N; ra.L = p.L; ra.L0 = p.L0; ra.nb = p.nb; ra.rpb = p.rpb; ra.Tr = p.Tr; ra.hg = p.hg;
  ra.row_in = p.row_in;
  ra.mag_hg = (uint64_t)((1LL << 42) / p.hg) + 1;
  ra.mag_rpb = (uint64_t)((1LL << 42) / p.rpb) + 1;
  ra.pos = pa_pos;
  ra.rope = p.rope;
  const dim3 gr((unsigned)(p.hg * p.nb * p.rpb), (unsigned)p.B);
  // bf16 inputs without a q norm stage the rotary window as rope_words (16
  // bytes per pair instead of 8)
  const bool packed = in_bf16 && !nq;
  const int lds_tab = packed ? p.lds_read16 : p.lds_read;
  e = p.D == 64 ? launch_readouts<64>(ra, in_bf16, out_bf16, p2, gr,
                                     read_lds(false, 0, lds_tab + (in_bf16 ? kReadAlBytes : 0) + (packed ? kReadZBytes : 0)), s,
                                     ev_read)
                : launch_readouts<32>(ra, in_bf16, out_bf16, p2, gr,
                                      read_lds(packed, (long long)gr.x * gr.y, lds_tab + (packed ? kReadAlBytes / 2 + kReadZBytes : 0)), s,
                                      ev_read);
  return (int)e;
}

// Guard of the training-path backward: the block prefixes it reused are the
// ones a matching forward formed only if the workspace's fingerprint equals
// the one of this call's arguments; otherwise dq, dk and dv (n16 16-byte
// pieces each) are overwritten with NaN, so a foreign workspace cannot give
// plausible wrong gradients.  On a match every thread leaves at once.
__global__ __launch_bounds__(256) void k_fp_guard(const uint64_t* fp, uint64_t f0, uint64_t f1, u32x4* dq,
                                                  u32x4* dk, u32x4* dv, size_t n16, uint32_t nan_word) {
  if (fp[0] == f0 && fp[1] == f1) return;
  const u32x4 nn = {nan_word, nan_word, nan_word, nan_word};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
    dq[i] = nn;
    dk[i] = nn;
    dv[i] = nn;
  }
}

template <int DH>
hipError_t launch_bw_q(const BwQArgs& qa, bool in_bf16, bool grad_bf16, bool p2, dim3 grid, int lds, hipStream_t s) {
  if (in_bf16 && grad_bf16) hipLaunchKernelGGL((p2 ? k_bw_q<uint16_t, uint16_t, true, DH> : k_bw_q<uint16_t, uint16_t, false, DH>), grid, dim3(NT), lds, s, qa);
  else if (in_bf16) hipLaunchKernelGGL((p2 ? k_bw_q<uint16_t, float, true, DH> : k_bw_q<uint16_t, float, false, DH>), grid, dim3(NT), lds, s, qa);
  else if (grad_bf16) hipLaunchKernelGGL((p2 ? k_bw_q<float, uint16_t, true, DH> : k_bw_q<float, uint16_t, false, DH>), grid, dim3(NT), lds, s, qa);
  else hipLaunchKernelGGL((p2 ? k_bw_q<float, float, true, DH> : k_bw_q<float, float, false, DH>), grid, dim3(NT), lds, s, qa);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_bw_kv(const BwKVArgs& ka, bool in_bf16, bool grad_bf16, bool p2, dim3 grid, int lds, hipStream_t s) {
  if (in_bf16 && grad_bf16) hipLaunchKernelGGL((p2 ? k_bw_kv<uint16_t, uint16_t, true, DH> : k_bw_kv<uint16_t, uint16_t, false, DH>), grid, dim3(NT), lds, s, ka);
  else if (in_bf16) hipLaunchKernelGGL((p2 ? k_bw_kv<uint16_t, float, true, DH> : k_bw_kv<uint16_t, float, false, DH>), grid, dim3(NT), lds, s, ka);
  else if (grad_bf16) hipLaunchKernelGGL((p2 ? k_bw_kv<float, uint16_t, true, DH> : k_bw_kv<float, uint16_t, false, DH>), grid, dim3(NT), lds, s, ka);
  else hipLaunchKernelGGL((p2 ? k_bw_kv<float, float, true, DH> : k_bw_kv<float, float, false, DH>), grid, dim3(NT), lds, s, ka);
  return hipGetLastError();
}

int launch_backward(const Plan& p, const void* q, const void* k, const void* v, const void* dout,
                    void* dq, void* dk, void* dv, int in_bf16, int grad_bf16, float eps, void* ws,
                    void* stream, bool have_prefix) {
  hipStream_t s = (hipStream_t)stream;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_part);
  float* prefix = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_prefix);
  float* suffix = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_suffix);
  const PosArgs pa_pos = pos_args(p);
  const bool p2 = ((p.rope.pt | p.rope.ph | p.rope.pw) & 1) == 0;
  hipError_t e;

  // Sbar, zbar of every block, as the forward forms them (unless the forward's
  // are still in the workspace).
  StateArgs sa;
  sa.k = k; sa.v = v; sa.part = part;
  sa.scale = nullptr; sa.gamma = nullptr; sa.row_in = p.row_in;
  sa.H = p.H; sa.N = p.N; sa.L = p.L; sa.L0 = p.L0; sa.nb = p.nb; sa.cpb = p.cpb; sa.Tc = p.Tc; sa.hg = p.hg;
  sa.pos = pa_pos;
  sa.rope = p.rope;
  sa.fp_dst = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + p.ws_fp);
  prefix_fingerprint(p, k, v, in_bf16, nullptr, &sa.fp0, &sa.fp1);
  const dim3 gs((unsigned)(p.hg * p.nb * p.cpb), (unsigned)p.B);
  PrefixArgs pa;
  pa.part = part; pa.prefix = prefix; pa.S_init = nullptr; pa.z_init = nullptr;
  pa.S_save = nullptr; pa.z_save = nullptr; pa.H = p.H; pa.nb = p.nb; pa.cpb = p.cpb;
  pa.hd = p.D; pa.rec = p.rec; pa.rev = 0;
  if (!have_prefix) {
    e = p.D == 64 ? launch_state<64>(sa, in_bf16, p2, gs, p.lds_state, p.lds_state1, s)
                  : launch_state<32>(sa, in_bf16, p2, gs, p.lds_state, p.lds_state1, s);
    if (e == hipSuccess) e = launch_prefix(pa, p, s);
    if (e != hipSuccess) return (int)e;
  }

  // dq and the chunk partials of (G, gz) (over the forward's partials, which
  // the prefix kernel has consumed).
  BwQArgs qa;
  qa.q = q; qa.g = dout; qa.dq = dq; qa.prefix = prefix; qa.part = part; qa.eps = eps;
  qa.H = p.H; qa.N = p.N; qa.L = p.L; qa.L0 = p.L0; qa.nb = p.nb; qa.cpb = p.cpb; qa.Tc = p.Tc; qa.hg = p.hg;
  qa.pos = pa_pos;
  qa.rope = p.rope;
  const int nbk = p.D == 64 ? 4 : 2;                  // operand blocks per matrix
  const int lds_ops = 2 * nbk * OPS_BLOCK * 16;
  const int wave_tile = in_bf16 ? 3 * 16 * TCOLS * 2 : 2 * 16 * TCOLS * 4;
  const int lds_q = 4 * wave_tile + nbk * OPS_BLOCK * 16 + (4 * 2 * D + 2 * D) * 4 + p.tab_state;   // tiles, Sbar^T, gz, zbar, table
  e = p.D == 64 ? launch_bw_q<64>(qa, in_bf16, grad_bf16, p2, gs, lds_q, s)
                : launch_bw_q<32>(qa, in_bf16, grad_bf16, p2, gs, lds_q, s);
  if (e != hipSuccess) return (int)e;

  // dS, dz: sums over the blocks at or after each block.
  pa.prefix = suffix; pa.rev = 1;
  e = launch_prefix(pa, p, s);
  if (e != hipSuccess) return (int)e;

  BwKVArgs ka;
  ka.k = k; ka.v = v; ka.dk = dk; ka.dv = dv; ka.suffix = suffix;
  ka.H = p.H; ka.N = p.N; ka.L = p.L; ka.L0 = p.L0; ka.nb = p.nb; ka.rpb = p.rpb; ka.Tr = p.Tr; ka.hg = p.hg;
  ka.pos = pa_pos;
  ka.rope = p.rope;
  const dim3 gr((unsigned)(p.hg * p.nb * p.rpb), (unsigned)p.B);
  const int lds_kv = lds_ops + p.lds_read;
  e = p.D == 64 ? launch_bw_kv<64>(ka, in_bf16, grad_bf16, p2, gr, lds_kv, s)
                : launch_bw_kv<32>(ka, in_bf16, grad_bf16, p2, gr, lds_kv, s);
  if (e != hipSuccess || !have_prefix) return (int)e;

  // reused prefixes: check that a matching forward formed them
  uint64_t f0, f1;
  prefix_fingerprint(p, k, v, in_bf16, nullptr, &f0, &f1);
  const size_t n16 = (size_t)p.B * p.N * p.H * p.D * (grad_bf16 ? 2 : 4) / 16;
  const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 1024);
  hipLaunchKernelGGL(k_fp_guard, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint64_t*>(static_cast<char*>(ws) + p.ws_fp), f0, f1,
                     static_cast<u32x4*>(dq), static_cast<u32x4*>(dk), static_cast<u32x4*>(dv), n16,
                     grad_bf16 ? 0x7fc07fc0u : 0x7fc00000u);
  return (int)hipGetLastError();
}

// ------------------------------------------------- allocation-free workspace
//
// The workspace of la_block_causal_forward_noalloc: a file-scope device array,
// one copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device memory: its device
// address on each GPU comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address reaches the kernels.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int noalloc_workspace(void* stream, void** ws) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return LAVR_NOALLOC_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LAVR_NOALLOC_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return LAVR_NOALLOC_HIP;
    if (sdev != dev) return LAVR_NOALLOC_WRONG_DEVICE;   // the stream must belong to the current device
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return LAVR_NOALLOC_HIP;
    addr[dev].store(p, std::memory_order_release);
  }
  *ws = p;
  return 0;
}

}  // namespace lavr
