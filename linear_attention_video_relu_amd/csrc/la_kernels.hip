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
// Data in HBM: q, k, v, out are (B, N, H, 32) row-major.  A token's two-head
// slice is 128 contiguous bytes in bf16 (256 in fp32), so each workgroup owns
// a pair of heads and every global access is a whole 16-byte lane chunk of a
// fully used 128-byte line.
//
// bf16 arithmetic: bf16 MFMA operands that are not exact bf16 values (the
// rotated keys and queries, the prefix state) are split as x = hi + lo with
// both parts bf16 (hi rounded to nearest, lo the rounded remainder), and the
// products hi.hi + hi.lo + lo.hi are accumulated in fp32, so each operand
// carries ~17 significant bits instead of 8.
// fp32 inputs use the fp32 MFMA (v_mfma_f32_*_f32) and are exact fp32 products.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_internal.h"

namespace lavr {
namespace {

constexpr int D = kHeadDim;
constexpr int REC = kRec;
constexpr int NT = 256;              // threads of the state and readout workgroups
constexpr int STEP = 64;             // tokens per step of the state kernel
constexpr int TCOLS = 2 * D;         // an LDS tile row holds two heads
constexpr int SCAN_NT = 64;          // threads of the prefix workgroups

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

struct StateArgs {
  const void* k;
  const void* v;
  float* part;
  int H, N, L, nb, cpb, Tc, hg, tpf, gw;
  long long t0;
  uint64_t mag_tpf, mag_gw;
  RopeDev rope;
};

struct PrefixArgs {
  const float* part;
  float* prefix;
  const float* S_init;
  const float* z_init;
  float* S_save;
  float* z_save;
  int H, nb, cpb;
};

struct ReadArgs {
  const void* q;
  void* out;
  const float* prefix;
  float eps;
  int H, N, L, nb, rpb, Tr, hg, tpf, gw;
  long long t0;
  uint64_t mag_tpf, mag_gw;
  RopeDev rope;
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint64_t mag) {
  // floor(n / d) with mag = floor(2^42 / d) + 1; exact while n * d < 2^42.
  return (uint32_t)(((uint64_t)n * mag) >> 42);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Loads 16 bytes of element type T and widens them to floats.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void widen(u32x4 r, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void widen(u32x4 r, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

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

__device__ __forceinline__ TabWindow stage_table(float2* lds, const RopeDev& r, long long t0,
                                                 int n0, int n1, uint64_t mag_tpf) {
  TabWindow w{0, 0};
  if (r.table == nullptr || n1 <= n0) return w;
  w.f_lo = (int)fast_div((uint32_t)n0, mag_tpf);
  w.nf = (int)fast_div((uint32_t)(n1 - 1), mag_tpf) - w.f_lo + 1;
  const float2* tab = reinterpret_cast<const float2*>(r.table);
  const float2* tsrc = tab + (size_t)(t0 + w.f_lo) * r.pt;
  const float2* hwsrc = tab + (size_t)r.max_frames * r.pt;
  const int nt = w.nf * r.pt;
  const int tot = nt + r.gh * r.ph + r.gw * r.pw;
  for (int i = threadIdx.x; i < tot; i += blockDim.x) lds[i] = i < nt ? tsrc[i] : hwsrc[i - nt];
  return w;
}

template <int NP>
struct PairLut {
  int base[NP], stride[NP], sel[NP];
  __device__ void init(const RopeDev& r, const TabWindow& w, int p0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int gp = p0 + i;
      if (gp < r.pt) {
        sel[i] = 0; base[i] = gp; stride[i] = r.pt;
      } else if (gp < r.pt + r.ph) {
        sel[i] = 1; base[i] = w.nf * r.pt + (gp - r.pt); stride[i] = r.ph;
      } else {
        sel[i] = 2; base[i] = w.nf * r.pt + r.gh * r.ph + (gp - r.pt - r.ph); stride[i] = r.pw;
      }
    }
  }
  // Rotate NP adjacent pairs x[0..2NP) of token n (local index in the call).
  __device__ void rotate(float* x, const float2* lds, int n, int f_lo, int tpf, int gw,
                         uint64_t mag_tpf, uint64_t mag_gw) const {
    const int f = (int)fast_div((uint32_t)n, mag_tpf);
    const int rem = n - f * tpf;
    const int row = (int)fast_div((uint32_t)rem, mag_gw);
    const int col = rem - row * gw;
    const int pos3[3] = {f - f_lo, row, col};
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pos = sel[i] == 0 ? pos3[0] : (sel[i] == 1 ? pos3[1] : pos3[2]);
      const float2 cs = lds[base[i] + pos * stride[i]];
      const float a = x[2 * i], b = x[2 * i + 1];
      x[2 * i] = a * cs.x - b * cs.y;
      x[2 * i + 1] = a * cs.y + b * cs.x;
    }
  }
};

// --------------------------------------------------------- k_block_state
//
// Grid: x = chunk * hg + head group, y = batch.  256 threads.  Each 64-token
// step: every thread loads 16-byte chunks of K and V (8 lanes cover one
// token's two-head bf16 row), applies ReLU, adds to its key-sum, rotates, and
// writes V and R phi(K) into LDS tiles [token][2 heads x 32].  Then wave w
// takes head (w & 1) and tokens 32*(w >> 1) .. +31 of the step and feeds
// MFMA: A[e][n] = V[n][e], B[n][f] = R phi(K)[n][f], so C = S (32 x 32).
// A lane supplies one channel over 8 tokens, read across LDS rows.  Odd
// groups of 8 rows store the two heads swapped, so the two half-waves read
// disjoint LDS banks.

template <typename TIn>
__global__ __launch_bounds__(NT) void k_block_state(StateArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int VEC = Vec16<TIn>::N;     // elements per 16 bytes
  constexpr int CPH = D / VEC;           // 16-byte chunks per head row
  constexpr int LPR = 2 * CPH;           // lanes per two-head row
  constexpr int TPP = NT / LPR;          // tokens per load pass
  constexpr int NPASS = STEP / TPP;
  constexpr int NP = VEC / 2;            // rotary pairs per chunk
  constexpr int NTILE = BF ? 3 : 2;      // V, R phi(K) (hi, lo for bf16)
  constexpr int TILE_ELEMS = STEP * TCOLS;
  constexpr int TILE_BYTES = NTILE * TILE_ELEMS * (int)sizeof(TIn);

  extern __shared__ __align__(16) unsigned char smem[];
  TIn* tV = reinterpret_cast<TIn*>(smem);
  TIn* tK = tV + TILE_ELEMS;
  TIn* tKl = tK + TILE_ELEMS;            // bf16 only
  float2* tab = reinterpret_cast<float2*>(smem + TILE_BYTES);

  const int g = blockIdx.x % a.hg;
  const int ci = blockIdx.x / a.hg;
  const int b = blockIdx.y;
  const int j = ci / a.cpb;
  const int c = ci - j * a.cpb;
  const int blk0 = j * a.L;
  const int blk1 = min(blk0 + a.L, a.N);
  const int c0 = min(blk0 + c * a.Tc, blk1);
  const int c1 = min(c0 + a.Tc, blk1);
  const int h0 = g * kHeadsPerGroup;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;

  // loader role of this thread
  const int lr = t % LPR, ltok = t / LPR, lhh = lr / CPH, lcc = lr % CPH;
  const bool lhead_ok = h0 + lhh < a.H;
  const bool rope_on = a.rope.table != nullptr;

  const TabWindow win = stage_table(tab, a.rope, a.t0, c0, c1, a.mag_tpf);
  PairLut<NP> lut;
  if (rope_on) lut.init(a.rope, win, lcc * NP);
  __syncthreads();

  const size_t tok_stride = (size_t)a.H * D;
  const size_t off = ((size_t)b * a.N) * tok_stride + (size_t)(h0 + lhh) * D + lcc * VEC;
  const TIn* kp = reinterpret_cast<const TIn*>(a.k) + off;
  const TIn* vp = reinterpret_cast<const TIn*>(a.v) + off;

  float zacc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) zacc[i] = 0.f;
  f32x16 acc = {};

  const int hh = w & 1, th = w >> 1, cl = lane & 31, q = lane >> 5;

  for (int s0 = c0; s0 < c1; s0 += STEP) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int row = p * TPP + ltok;
      const int tok = s0 + row;
      const bool ok = tok < c1 && lhead_ok;
      u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
      if (ok) {
        kr = ld16(kp + (size_t)tok * tok_stride);
        vr = ld16(vp + (size_t)tok * tok_stride);
      }
      float x[VEC];
      Vec16<TIn>::widen(kr, x);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        x[i] = fmaxf(x[i], 0.f);
        zacc[i] += x[i];
      }
      if (rope_on && ok) lut.rotate(x, tab, tok, win.f_lo, a.tpf, a.gw, a.mag_tpf, a.mag_gw);
      const int col = (lhh * D + lcc * VEC) ^ (((row >> 3) & 1) << 5);
      *reinterpret_cast<u32x4*>(tV + row * TCOLS + col) = vr;
      if constexpr (BF) {
        u32x4 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<u32x4*>(tK + row * TCOLS + col) = hi;
        *reinterpret_cast<u32x4*>(tKl + row * TCOLS + col) = lo;
      } else {
        u32x4 xr;
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = __float_as_uint(x[i]);
        *reinterpret_cast<u32x4*>(tK + row * TCOLS + col) = xr;
      }
    }
    __syncthreads();
    if constexpr (BF) {
      const uint16_t* V16 = reinterpret_cast<const uint16_t*>(tV);
      const uint16_t* Kh16 = reinterpret_cast<const uint16_t*>(tK);
      const uint16_t* Kl16 = reinterpret_cast<const uint16_t*>(tKl);
      const int col = (hh * D + cl) ^ (q << 5);  // rows 8q..8q+7 of a 16-row group
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r0 = th * 32 + m * 16 + 8 * q;
        u32x4 av, bh, bl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = (r0 + 2 * e) * TCOLS + col, i1 = i0 + TCOLS;
          av[e] = (uint32_t)V16[i0] | ((uint32_t)V16[i1] << 16);
          bh[e] = (uint32_t)Kh16[i0] | ((uint32_t)Kh16[i1] << 16);
          bl[e] = (uint32_t)Kl16[i0] | ((uint32_t)Kl16[i1] << 16);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bl), acc, 0, 0, 0);
      }
    } else {
      const float* Vf = reinterpret_cast<const float*>(tV);
      const float* Kf = reinterpret_cast<const float*>(tK);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int row = th * 32 + 2 * s + q;
        const int i0 = row * TCOLS + ((hh * D + cl) ^ (((row >> 3) & 1) << 5));
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Vf[i0], Kf[i0], acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Combine the two waves of each head, and the key-sum lanes, through LDS.
  float* red = reinterpret_cast<float*>(smem);   // [2 waves][16][64]
  float* zred = red + 2 * 16 * 64;               // [NT][VEC]
  if (w >= 2) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((w - 2) * 16 + v) * 64 + lane] = acc[v];
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) zred[t * VEC + i] = zacc[i];
  __syncthreads();

  const int nchunk = a.nb * a.cpb;
  if (w < 2 && h0 + w < a.H) {
    float* dst = a.part + ((size_t)(b * a.H + h0 + w) * nchunk + ci) * REC;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      dst[e * D + (lane & 31)] = acc[v] + red[(w * 16 + v) * 64 + lane];
    }
  }
  if (t < 2 * D && h0 + t / D < a.H) {
    const int hd = t / D, ch = t % D;
    const int r = hd * CPH + ch / VEC, el = ch % VEC;
    float s = 0.f;
    for (int tp = 0; tp < TPP; ++tp) s += zred[(tp * LPR + r) * VEC + el];
    a.part[((size_t)(b * a.H + h0 + hd) * nchunk + ci) * REC + D * D + ch] = s;
  }
}

// -------------------------------------------------------------- k_prefix
//
// Grid: x = element group (17 x 64 covers the 1056 floats of a record),
// y = head, z = batch.  One thread owns one element of (S, z) for one head
// and walks the blocks in order: block sum = p_0 + p_1 + ... (chunk order),
// prefix = previous prefix + block sum.  A streaming call starts from the
// carried cache, so one block streamed on top of a cache adds exactly as the
// one-shot prefix does.

__global__ __launch_bounds__(SCAN_NT) void k_prefix(PrefixArgs a) {
  const int el = blockIdx.x * SCAN_NT + threadIdx.x;
  if (el >= REC) return;
  const size_t bh = (size_t)blockIdx.z * a.H + blockIdx.y;
  float acc = 0.f;
  if (a.S_init != nullptr) acc = el < D * D ? a.S_init[bh * D * D + el] : a.z_init[bh * D + el - D * D];
  const float* p = a.part + bh * a.nb * a.cpb * REC + el;
  float* o = a.prefix + bh * a.nb * REC + el;
  for (int j = 0; j < a.nb; ++j) {
    float bs = p[0];
    for (int c = 1; c < a.cpb; ++c) bs += p[(size_t)c * REC];
    p += (size_t)a.cpb * REC;
    acc += bs;
    o[(size_t)j * REC] = acc;
  }
  if (a.S_save != nullptr) {
    if (el < D * D) a.S_save[bh * D * D + el] = acc;
    else a.z_save[bh * D + el - D * D] = acc;
  }
}

// ------------------------------------------------------------- k_readout
//
// Grid: x = tile * hg + head group, y = batch.  256 threads; wave w takes head
// (w & 1) and every other 16-token group of the tile starting at (w >> 1).
// MFMA 16x16x32: A = Sbar rows (e) x channels (f), B = channels (f) x tokens:
// lane l holds channels 8(l>>4) .. +7 of token (l & 15), which is one 16-byte
// load of bf16 q.  The output lane holds channels 4(l>>4) .. +3 of each 16-row
// half for token (l & 15), so the normaliser of that token, summed over the
// four lanes that share it, is already in place.

template <typename TIn, typename TOut>
__global__ __launch_bounds__(NT) void k_readout(ReadArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  extern __shared__ __align__(16) unsigned char smem[];
  float2* tab = reinterpret_cast<float2*>(smem);

  const int g = blockIdx.x % a.hg;
  const int ti = blockIdx.x / a.hg;
  const int b = blockIdx.y;
  const int j = ti / a.rpb;
  const int r = ti - j * a.rpb;
  const int blk0 = j * a.L;
  const int blk1 = min(blk0 + a.L, a.N);
  const int t0 = min(blk0 + r * a.Tr, blk1);
  const int t1 = min(t0 + a.Tr, blk1);
  const bool rope_on = a.rope.table != nullptr;

  const TabWindow win = stage_table(tab, a.rope, a.t0, t0, t1, a.mag_tpf);
  __syncthreads();

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hh = w & 1, sub = w >> 1;
  const int head = g * kHeadsPerGroup + hh;
  if (head >= a.H || t0 >= t1) return;
  const int tl = lane & 15, ch = lane >> 4;

  PairLut<4> lut;
  if (rope_on) lut.init(a.rope, win, 4 * ch);

  const float* pre = a.prefix + ((size_t)(b * a.H + head) * a.nb + j) * REC;
  float zb[8];
  {
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(pre + D * D + 8 * ch);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(pre + D * D + 8 * ch + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { zb[i] = z0[i]; zb[4 + i] = z1[i]; }
  }
  // Sbar operands: row e = 16 * half + tl, channels 8 ch .. 8 ch + 7.
  u32x4 Ah[2], Al[2];
  float As[2][8];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float* srow = pre + (16 * hf + tl) * D + 8 * ch;
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(srow);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(srow + 4);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { sv[i] = s0[i]; sv[4 + i] = s1[i]; }
    if constexpr (BF) {
      split8(sv, Ah[hf], Al[hf]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) As[hf][i] = sv[i];
    }
  }

  const size_t tok_stride = (size_t)a.H * D;
  const TIn* qp = reinterpret_cast<const TIn*>(a.q) + (size_t)b * a.N * tok_stride + (size_t)head * D + 8 * ch;
  TOut* op = reinterpret_cast<TOut*>(a.out) + (size_t)b * a.N * tok_stride + (size_t)head * D + 4 * ch;

  for (int gi = sub; t0 + gi * 16 < t1; gi += 2) {
    const int tok = t0 + gi * 16 + tl;
    const bool ok = tok < t1;
    float x[8];
    if constexpr (BF) {
      u32x4 qr = {0u, 0u, 0u, 0u};
      if (ok) qr = ld16(qp + (size_t)tok * tok_stride);
      Vec16<uint16_t>::widen(qr, x);
    } else {
      u32x4 q0 = {0u, 0u, 0u, 0u}, q1 = {0u, 0u, 0u, 0u};
      if (ok) {
        q0 = ld16(qp + (size_t)tok * tok_stride);
        q1 = ld16(qp + (size_t)tok * tok_stride + 4);
      }
      Vec16<float>::widen(q0, x);
      Vec16<float>::widen(q1, x + 4);
    }
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = fmaxf(x[i], 0.f);
      den += zb[i] * x[i];
    }
    if (rope_on && ok) lut.rotate(x, tab, tok, win.f_lo, a.tpf, a.gw, a.mag_tpf, a.mag_gw);

    f32x4 o[2];
    if constexpr (BF) {
      u32x4 bh, bl;
      split8(x, bh, bl);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Ah[hf]), as_bf16x8(bh), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Ah[hf]), as_bf16x8(bl), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Al[hf]), as_bf16x8(bh), c, 0, 0, 0);
        o[hf] = c;
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(As[hf][s], x[s], c, 0, 0, 0);
        o[hf] = c;
      }
    }
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const float inv = 1.0f / (den + a.eps);
    if (ok) {
      TOut* dst = op + (size_t)tok * tok_stride;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (sizeof(TOut) == 2) {
          u32x2 pk;
          pk[0] = pack_bf16(o[hf][0] * inv, o[hf][1] * inv);
          pk[1] = pack_bf16(o[hf][2] * inv, o[hf][3] * inv);
          *reinterpret_cast<u32x2*>(dst + 16 * hf) = pk;
        } else {
          f32x4 ov = o[hf] * inv;
          *reinterpret_cast<f32x4*>(dst + 16 * hf) = ov;
        }
      }
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

template <typename TIn, typename TOut>
hipError_t launch_readout(const ReadArgs& ra, dim3 grid, int lds, hipStream_t s) {
  hipLaunchKernelGGL((k_readout<TIn, TOut>), grid, dim3(NT), lds, s, ra);
  return hipGetLastError();
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

int launch_zero(float* p, size_t n, void* stream) {
  if (n == 0) return (int)hipSuccess;
  const int nt = 256;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + nt - 1) / nt)), dim3(nt), 0,
                     (hipStream_t)stream, p, n);
  return (int)hipGetLastError();
}

int launch_forward(const Plan& p, const void* q, const void* k, const void* v, void* out,
                   int in_bf16, int out_bf16, float eps, void* ws,
                   const float* S_init, const float* z_init, float* S_save, float* z_save,
                   void* stream, void* const* events) {
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return (int)e;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_part);
  float* prefix = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_prefix);

  StateArgs sa;
  sa.k = k; sa.v = v; sa.part = part;
  sa.H = p.H; sa.N = p.N; sa.L = p.L; sa.nb = p.nb; sa.cpb = p.cpb; sa.Tc = p.Tc; sa.hg = p.hg;
  sa.tpf = p.tpf; sa.gw = p.gw_div; sa.t0 = p.t0; sa.mag_tpf = p.mag_tpf; sa.mag_gw = p.mag_gw;
  sa.rope = p.rope;
  const dim3 gs((unsigned)(p.hg * p.nb * p.cpb), (unsigned)p.B);
  if (in_bf16) hipLaunchKernelGGL(k_block_state<uint16_t>, gs, dim3(NT), p.lds_state, s, sa);
  else hipLaunchKernelGGL(k_block_state<float>, gs, dim3(NT), p.lds_state, s, sa);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return (int)e;

  PrefixArgs pa;
  pa.part = part; pa.prefix = prefix; pa.S_init = S_init; pa.z_init = z_init;
  pa.S_save = S_save; pa.z_save = z_save; pa.H = p.H; pa.nb = p.nb; pa.cpb = p.cpb;
  const dim3 gp((REC + SCAN_NT - 1) / SCAN_NT, (unsigned)p.H, (unsigned)p.B);
  hipLaunchKernelGGL(k_prefix, gp, dim3(SCAN_NT), 0, s, pa);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return (int)e;

  ReadArgs ra;
  ra.q = q; ra.out = out; ra.prefix = prefix; ra.eps = eps;
  ra.H = p.H; ra.N = p.N; ra.L = p.L; ra.nb = p.nb; ra.rpb = p.rpb; ra.Tr = p.Tr; ra.hg = p.hg;
  ra.tpf = p.tpf; ra.gw = p.gw_div; ra.t0 = p.t0; ra.mag_tpf = p.mag_tpf; ra.mag_gw = p.mag_gw;
  ra.rope = p.rope;
  const dim3 gr((unsigned)(p.hg * p.nb * p.rpb), (unsigned)p.B);
  if (in_bf16 && out_bf16) e = launch_readout<uint16_t, uint16_t>(ra, gr, p.lds_read, s);
  else if (in_bf16) e = launch_readout<uint16_t, float>(ra, gr, p.lds_read, s);
  else if (out_bf16) e = launch_readout<float, uint16_t>(ra, gr, p.lds_read, s);
  else e = launch_readout<float, float>(ra, gr, p.lds_read, s);
  if (e == hipSuccess) e = mark(3);
  return (int)e;
}

}  // namespace lavr
