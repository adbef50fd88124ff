// Internal interface between the host API layer (la_api.cpp) and the HIP
// kernels (la_kernels.hip).  Not installed; the public ABI is include/la_vr.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lavr {

// Head dims built: 32 (two heads per workgroup) and 64 (one head per
// workgroup).  Either way a workgroup owns 64 channels = 128 bytes of bf16 of
// every token row.
constexpr bool head_dim_built(int d) { return d == 32 || d == 64; }
constexpr int rec_floats(int d) { return d * d + d; }   // floats of one (S, z) record

// Workspace header: 256 bytes holding the 16-byte fingerprint of the block
// prefixes; the data follows.
constexpr size_t kWsHeader = 256;

// Block-state LDS tiles: 1 = one set (two barriers per step), 2 = double
// buffered (one barrier per step).
#ifndef LAVR_STATE_DB
#define LAVR_STATE_DB 2
#endif
constexpr int kStateTileSets = LAVR_STATE_DB == 2 ? 2 : 1;

// Readout workgroups resident per CU on the packed bf16 path at head dim 32,
// set by an LDS floor (its registers would allow six).  The readout streams Q
// in and the output out at once, and the HBM serves that mix best with few
// requests in flight: each wave keeps one 16-token group of loads in flight,
// four workgroups share a CU in a launch of several rounds, and a launch that
// fits one round at three per CU runs at three.  At head dim 64 the launch
// keeps its register-bound four per CU and two groups in flight.
constexpr int kReadOcc = 3;    // one-round launches (at most kReadOcc * 256 workgroups)
constexpr int kReadOccN = 4;   // longer launches
constexpr int kCuLds = 160 * 1024;   // LDS bytes per CU (gfx950)
// Dynamic LDS floors of a packed readout workgroup: one more would not fit.
constexpr int kReadOccLds = kCuLds / (kReadOcc + 1) + 256;
constexpr int kReadOccLdsN = kCuLds / (kReadOccN + 1) + 256;
static_assert(kReadOcc * kReadOccLds <= kCuLds && kReadOccN * kReadOccLdsN <= kCuLds, "readout occupancy floors");

// Rotary table as the kernels see it.
struct RopeDev {
  const float* table;   // (cos, sin) pairs; nullptr = RoPE off
  int pt, ph, pw;       // pairs per section (d_t/2, d_h/2, d_w/2)
  int max_frames;       // rows of the t section
  int gh, gw;           // rows of the h and w sections
};

// Everything a launch needs; filled by the host planner.
struct Plan {
  int B, H;
  int D;                // head dim (32 or 64)
  int rec;              // floats of one (S, z) record: D * D + D
  int N;                // tokens per sequence in this call
  int row_in;           // elements from one input token row to the next (H * D, or 3 * H * D fused)
  int tpf;              // tokens per frame
  int gw_div;           // divisor for row/col (grid_w, or 1 without spatial sections)
  int L;                // tokens per block (after the first)
  int L0;               // tokens of the first block
  int nb;               // blocks in this call
  int hg;               // workgroup head groups: ceil(H / 2) at D = 32, H at D = 64
  int cpb, Tc;          // block-state chunks per block, tokens per chunk
  int rpb, Tr;          // readout tiles per block, tokens per tile
  long long t0;         // frame offset of token 0 (frames already streamed)
  uint64_t mag_tpf;     // floor(2^42 / tpf) + 1
  uint64_t mag_gw;      // floor(2^42 / gw_div) + 1
  RopeDev rope;
  int lds_state;        // dynamic LDS bytes of the block-state kernel
  int lds_state1;       // the same with one tile set (single-round launches)
  int tab_state;        // of which the rotary window of a chunk
  int lds_read;         // dynamic LDS bytes of the readout kernel's rotary window ((cos, sin) pairs)
  int lds_read16;       // the same window as rope_words (16 bytes per pair)
  size_t ws_fp;         // byte offset of the 16-byte fingerprint of the block prefixes (in the header)
  size_t ws_part;       // byte offset of the per-chunk partial states
  size_t ws_prefix;     // byte offset of the per-block prefix states
  size_t ws_suffix;     // byte offset of the per-block suffix sums (backward only)
  size_t ws_total_bw;   // workspace bytes of the backward
  size_t ws_total;      // workspace bytes
  size_t ws_scale;      // byte offset of the q/k token scales (fused prologue only)
  size_t ws_total_qkv;  // workspace bytes of the fused-prologue forward
};

// q/k RMSNorm prologue of a forward call (null weights: that tensor is not
// normalised).  The scales live in the workspace.
struct Prologue {
  const float* q_gamma;
  const float* k_gamma;
  float* q_scale;       // B * N floats
  float* k_scale;       // B * N floats
  float norm_eps;
};

// Launchers; each returns a hipError_t value (0 = success).
int launch_rope_table(float* table, int pt, int ph, int pw, int max_frames, int gh, int gw,
                      double base, void* stream);
int launch_forward(const Plan& p, const void* q, const void* k, const void* v, void* out,
                   int in_bf16, int out_bf16, float eps, void* ws,
                   const float* S_init, const float* z_init, float* S_save, float* z_save,
                   void* stream, void* const* events = nullptr, const Prologue* pro = nullptr);
int launch_zero(float* p, size_t n, void* stream);

// Allocation-free forward: the workspace is a device array of kScratchBytes,
// one per GPU (la_kernels.hip).  noalloc_workspace() returns its address on
// the current device (0), or one of the codes below.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int LAVR_NOALLOC_HIP = 1;            // a HIP query failed
constexpr int LAVR_NOALLOC_UNSUPPORTED = 2;    // device index beyond the library's table
constexpr int LAVR_NOALLOC_WRONG_DEVICE = 3;   // the stream belongs to another device
int noalloc_workspace(void* stream, void** ws);

// Cached temporal convolution of one call: F frames of P tokens x Ch channels
// per batch row, blocks of F0 then BF frames, kt taps.
struct ConvPlan {
  int B, F, P, Ch, F0, BF, kt;
};
int launch_tconv(const ConvPlan& c, const void* x, void* y, int in_bf16, int out_bf16, const float* w,
                 const float* bias, const void* cache_in, void* cache_out, void* stream);
// have_prefix: ws already holds the block prefixes the forward wrote (the
// block-state and prefix kernels are skipped).
int launch_backward(const Plan& p, const void* q, const void* k, const void* v, const void* dout,
                    void* dq, void* dk, void* dv, int in_bf16, int grad_bf16, float eps, void* ws,
                    void* stream, bool have_prefix = false);

}  // namespace lavr
