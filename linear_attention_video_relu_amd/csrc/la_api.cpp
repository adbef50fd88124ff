// Host side of liblavr: argument checks, launch planning, workspace sizing and
// the C entry points declared in include/la_vr.h.  Every check runs before any
// HIP call, so a bad call returns a status without touching the GPU.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "la_internal.h"
#include "la_vr.h"

using lavr::Plan;

namespace {

// Work split.  A block-state chunk or readout tile holds at most kStateMax /
// kReadMax tokens (long chunks keep the partial-state traffic and the prefix
// kernel small), and the launch is split finer until it has at least kMinWg
// workgroups, so that a single streamed block still fills 256 CUs.  kMinWg is
// about one resident round of the block-state kernel (3 workgroups per CU);
// measured on a streamed 3-frame block (B = 2, 70 heads): 1024 -> 56-57 us,
// 700 -> 54 us, 1536 -> 59 us per call.  Readout tiles of at most 512 tokens
// at head dim 32 (25 per 8-frame block of the minute-long clip), whose
// prologue overlaps its loads: 0.599-0.603 ms against 0.605-0.614 at 640,
// 0.623-0.626 at 448 and 896, 0.604 at 384, 0.643 at 1280; at head dim 64,
// 640 (0.651-0.653 ms against 0.657 at 512).
#ifndef LAVR_STATE_MAX
#define LAVR_STATE_MAX 4200
#endif
#ifndef LAVR_READ_MAX
#define LAVR_READ_MAX 512
#endif
#ifndef LAVR_READ_MAX64
#define LAVR_READ_MAX64 640
#endif
#ifndef LAVR_MIN_WG
#define LAVR_MIN_WG 700
#endif
constexpr int kStateMax = LAVR_STATE_MAX;
constexpr int kReadMax = LAVR_READ_MAX, kReadMax64 = LAVR_READ_MAX64;
constexpr int kMinWg = LAVR_MIN_WG;
// readout workgroups resident in one round on the packed path: kReadOcc per CU
// at head dim 32 (the occupancy a launch of one round takes), four at 64
constexpr long long kReadSlots32 = lavr::kReadOcc * 256, kReadSlots64 = 4 * 256;
constexpr int kTabLdsMax = 32768;      // LDS bytes for a staged rotary window ((cos, sin) pairs)
constexpr int kTabLdsMax16 = 49152;    // the same for a readout tile's rope_words (with the 16 KB Sbar
                                       // copy at head dim 64, at most 64 KB per workgroup)
constexpr int kStep = 64;              // block-state kernel step (tokens)
constexpr long long kTwo42 = 1LL << 42;
constexpr long long kMaxTokens = 1LL << 30;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

long long round_up(long long a, long long m) { return cdiv(a, m) * m; }

bool rope_on(const la_rope* r) { return r != nullptr && r->table != nullptr; }

int esize(la_dtype dt) { return dt == LA_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == LA_F32 || dt == LA_BF16; }

// Validate the rotary description for a call covering frames [t0, t0 + frames).
int check_rope(const la_rope* r, int head_dim, int tpf, long long t0, long long frames) {
  if (!rope_on(r)) return LA_OK;
  if (!aligned(r->table, 16)) return LA_ERR_INVALID_ARG;
  if (r->d_t < 0 || r->d_h < 0 || r->d_w < 0) return LA_ERR_INVALID_ARG;
  if ((r->d_t | r->d_h | r->d_w) & 1) return LA_ERR_INVALID_ARG;
  if (r->d_t + r->d_h + r->d_w != head_dim) return LA_ERR_INVALID_ARG;
  if (r->max_frames < 1 || r->grid_h < 1 || r->grid_w < 1) return LA_ERR_INVALID_ARG;
  if (r->d_h + r->d_w > 0 && (long long)r->grid_h * r->grid_w != tpf) return LA_ERR_INVALID_ARG;
  if (t0 < 0 || t0 + frames > r->max_frames) return LA_ERR_INVALID_ARG;
  // the kernels index the table's (cos, sin) pairs with 32-bit integers
  const long long pairs = (long long)r->max_frames * (r->d_t / 2) + (long long)r->grid_h * (r->d_h / 2) +
                          (long long)r->grid_w * (r->d_w / 2);
  if (pairs >= (1LL << 31)) return LA_ERR_INVALID_ARG;
  return LA_OK;
}

// Pairs of the rotary table a workgroup covering `tokens` consecutive tokens stages.
long long tab_pairs(const la_rope* r, int tpf, int tokens) {
  if (!rope_on(r)) return 0;
  const long long nf = (tokens - 1) / tpf + 2;
  return nf * (r->d_t / 2) + (long long)r->grid_h * (r->d_h / 2) + (long long)r->grid_w * (r->d_w / 2);
}

// Split a block of L tokens into n chunks of T tokens (a multiple of `mult`):
// at most max_tokens per chunk, at least min_n chunks, the rotary window of a
// chunk fits in LDS and its byte span (plus the 256 tokens a kernel may run
// ahead) stays within the 32-bit buffer offsets the kernels use; row_bytes is
// the widest token row (fp32).  Returns false if no split fits.
bool split_block(int L, int max_tokens, long long min_n, int mult, const la_rope* r, int tpf,
                 long long row_bytes, int entry_bytes, int tab_cap, int* n_out, int* T_out) {
  long long n = cdiv(L, max_tokens);
  if (n < min_n) n = min_n;
  for (;;) {
    const long long T = round_up(cdiv(L, n), mult);
    if (tab_pairs(r, tpf, (int)T) * entry_bytes <= tab_cap && (T + 256) * row_bytes < (1LL << 31)) {
      *n_out = (int)cdiv(L, T);
      *T_out = (int)T;
      return true;
    }
    if (T <= mult) return false;
    n = cdiv(L, T - mult);
  }
}

// Small launches run a few resident rounds of workgroups, and a last round that
// has barely begun costs almost a whole round.  If fewer, longer pieces (at most
// twice max_tokens) drop that round, take them.  `rows` workgroups share each
// piece index; `slots` is one resident round.
void fit_rounds(int L, int max_tokens, long long rows, long long slots, int mult, const la_rope* r, int tpf,
                long long row_bytes, int entry_bytes, int tab_cap, int* n, int* T) {
  const long long R = cdiv(rows * *n, slots);
  if (R <= 1 || R > 4) return;
  const long long n2 = (R - 1) * slots / rows;
  if (n2 < 1) return;
  const long long T2 = round_up(cdiv(L, n2), mult);
  if (T2 > 2LL * max_tokens || tab_pairs(r, tpf, (int)T2) * entry_bytes > tab_cap ||
      (T2 + 256) * row_bytes >= (1LL << 31))
    return;
  *n = (int)cdiv(L, T2);
  *T = (int)T2;
}

// first_block_frames: frames of the first block (0 = block_frames).  row_mult:
// input token rows hold row_mult * H * head_dim elements (3 for fused q|k|v).
// stream_chunks: split every block into the chunks a streamed call of that one
// block takes (the chunk count is planned as for a launch of one block), so that
// the block states, and every output, equal the streamed ones bit for bit.
int make_plan(Plan* p, int B, int H, int head_dim, int frames, int tpf, int block_frames,
              int first_block_frames, const la_rope* rope, long long t0, la_dtype in_dt,
              int row_mult = 1, bool stream_chunks = false) {
  if (B < 1 || H < 1 || head_dim < 1 || frames < 1 || tpf < 1 || block_frames < 1 ||
      first_block_frames < 0)
    return LA_ERR_INVALID_ARG;
  if (first_block_frames == 0) first_block_frames = block_frames;
  if (!lavr::head_dim_built(head_dim)) return LA_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535 || (long long)B * H > (1LL << 24)) return LA_ERR_UNSUPPORTED;
  const long long N = (long long)frames * tpf;
  if (N > kMaxTokens || N * tpf >= kTwo42) return LA_ERR_UNSUPPORTED;
  int st = check_rope(rope, head_dim, tpf, t0, frames);
  if (st != LA_OK) return st;
  const int gw_div = (rope_on(rope) && rope->d_h + rope->d_w > 0) ? rope->grid_w : 1;
  if ((long long)tpf * gw_div >= kTwo42) return LA_ERR_UNSUPPORTED;

  std::memset(p, 0, sizeof(*p));
  p->B = B;
  p->H = H;
  p->D = head_dim;
  p->rec = lavr::rec_floats(head_dim);
  p->N = (int)N;
  p->row_in = row_mult * H * head_dim;
  p->tpf = tpf;
  p->gw_div = gw_div;
  p->L = (int)((long long)(block_frames < frames ? block_frames : frames) * tpf);
  p->L0 = (int)((long long)(first_block_frames < frames ? first_block_frames : frames) * tpf);
  p->nb = N <= p->L0 ? 1 : 1 + (int)cdiv(N - p->L0, p->L);
  const int Lmax = p->L0 > p->L ? p->L0 : p->L;   // chunks and tiles are planned for the longest block
  p->hg = head_dim == 32 ? (H + 1) / 2 : H;
  p->t0 = t0;
  p->mag_tpf = (uint64_t)(kTwo42 / tpf) + 1;
  p->mag_gw = (uint64_t)(kTwo42 / gw_div) + 1;
  const long long row_bytes = (long long)p->row_in * 4;
  const long long min_n = cdiv(kMinWg, (long long)B * p->hg * (stream_chunks ? 1 : p->nb));
  // Rotary windows are staged as (cos, sin) pairs (8 bytes), or as rope_words
  // (16 bytes) by the readout tiles and, for bf16 inputs, the block-state chunks.
  const bool bf16_in = in_dt == LA_BF16;
  const int state_entry = bf16_in ? 16 : 8;
  if (!split_block(Lmax, kStateMax, min_n, kStep, rope, tpf, row_bytes, state_entry,
                   bf16_in ? kTabLdsMax16 : kTabLdsMax, &p->cpb, &p->Tc))
    return LA_ERR_UNSUPPORTED;
  const int read_max = head_dim == 32 ? kReadMax : kReadMax64;
  if (!split_block(Lmax, read_max, min_n, 64, rope, tpf, row_bytes, 16, kTabLdsMax16, &p->rpb, &p->Tr))
    return LA_ERR_UNSUPPORTED;
  fit_rounds(Lmax, read_max, (long long)B * p->hg * p->nb, head_dim == 32 ? kReadSlots32 : kReadSlots64, 64, rope, tpf, row_bytes, 16, kTabLdsMax16,
             &p->rpb, &p->Tr);
  if ((long long)p->hg * p->nb * p->cpb > 0x7fffffffLL || (long long)p->hg * p->nb * p->rpb > 0x7fffffffLL)
    return LA_ERR_UNSUPPORTED;

  if (rope_on(rope)) {
    p->rope.table = rope->table;
    p->rope.pt = rope->d_t / 2;
    p->rope.ph = rope->d_h / 2;
    p->rope.pw = rope->d_w / 2;
    p->rope.max_frames = rope->max_frames;
    p->rope.gh = rope->grid_h;
    p->rope.gw = rope->grid_w;
  }
  const int tiles = (in_dt == LA_BF16 ? 3 : 2) * kStep * 64 * esize(in_dt);   // 64 channels per row
  p->tab_state = (int)(tab_pairs(rope, tpf, p->Tc) * 8);
  p->lds_state = lavr::kStateTileSets * tiles + (int)(tab_pairs(rope, tpf, p->Tc) * state_entry);
  p->lds_state1 = tiles + (int)(tab_pairs(rope, tpf, p->Tc) * state_entry);
  p->lds_read = (int)(tab_pairs(rope, tpf, p->Tr) * 8);
  p->lds_read16 = 2 * p->lds_read;

  const size_t rec = (size_t)p->rec * sizeof(float);
  const size_t part = (size_t)B * H * p->nb * p->cpb * rec;
  const size_t prefix = (size_t)B * H * p->nb * rec;
  // Header: the fingerprint of the block prefixes (what a backward reusing
  // them checks), then the chunk records and the prefixes.
  p->ws_fp = 0;
  p->ws_part = lavr::kWsHeader;
  p->ws_prefix = p->ws_part + align256(part);
  p->ws_total = p->ws_prefix + align256(prefix);
  p->ws_suffix = p->ws_total;
  p->ws_total_bw = p->ws_suffix + align256(prefix);
  p->ws_scale = p->ws_total;
  p->ws_total_qkv = p->ws_scale + 2 * align256((size_t)B * N * sizeof(float));
  return LA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_tensors(const void* q, const void* k, const void* v, void* out, la_dtype in_dt,
                  la_dtype out_dt, const Plan& p) {
  if (!q || !k || !v || !out) return LA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return LA_ERR_INVALID_ARG;
  const size_t elems = (size_t)p.B * p.N * p.H * p.D;
  const size_t nin = elems * esize(in_dt), nout = elems * esize(out_dt);
  if (overlaps(out, nout, q, nin) || overlaps(out, nout, k, nin) || overlaps(out, nout, v, nin))
    return LA_ERR_INVALID_ARG;
  return LA_OK;
}

int hip_status(int e) { return e == 0 ? LA_OK : LA_ERR_HIP; }

// Bytes of one (B, N, H, head_dim) tensor of dtype dt (rows * row_mult for
// the fused q|k|v input).
size_t tensor_bytes(const Plan& p, la_dtype dt, int row_mult = 1) {
  return (size_t)p.B * p.N * row_mult * p.H * p.D * esize(dt);
}

// A byte range a call touches.
struct Span {
  const void* p;
  size_t n;
};

// True if the range w, which the call writes, shares bytes with any of the
// others (null or empty ranges are skipped).
bool clashes(Span w, std::initializer_list<Span> others) {
  if (!w.p || !w.n) return false;
  for (const Span& o : others)
    if (o.p && o.n && overlaps(w.p, w.n, o.p, o.n)) return true;
  return false;
}

Span rope_span(const la_rope* r) {
  if (!rope_on(r)) return {nullptr, 0};
  return {r->table, 8 * ((size_t)r->max_frames * (r->d_t / 2) + (size_t)r->grid_h * (r->d_h / 2) +
                         (size_t)r->grid_w * (r->d_w / 2))};
}

// The workspace (the part the call uses) against the call's tensors and the
// rotary table, the output against the rotary table, and a carried state
// (written when `save` is set) against all of them.
int check_scratch(const Plan& p, void* ws, size_t used, Span out, std::initializer_list<Span> tensors,
                  const la_rope* rope, const la_state* st = nullptr) {
  const Span r = rope_span(rope);
  if (clashes({ws, used}, tensors) || clashes({ws, used}, {out, r}) || clashes(out, {r}))
    return LA_ERR_INVALID_ARG;
  if (st) {
    const Span S{st->S, (size_t)p.B * p.H * p.D * p.D * 4}, z{st->z, (size_t)p.B * p.H * p.D * 4};
    if (clashes({ws, used}, {S, z}) || clashes(S, tensors) || clashes(z, tensors) || clashes(S, {out, r}) ||
        clashes(z, {out, r}))
      return LA_ERR_INVALID_ARG;
  }
  return LA_OK;
}

// Fused (B, N, 3, C) input, its output and the optional norm weights; fills
// the prologue (scales in the workspace) and the q, k, v row pointers.
int check_fused(const void* qkv, void* out, la_dtype in_dt, la_dtype out_dt, const Plan& p,
                const float* q_gamma, const float* k_gamma, float norm_eps, void* ws,
                size_t ws_bytes, lavr::Prologue* pro, const void** q, const void** k,
                const void** v) {
  if (!qkv || !out || !aligned(qkv, 16) || !aligned(out, 16)) return LA_ERR_INVALID_ARG;
  const size_t C = (size_t)p.H * p.D;
  const size_t nin = (size_t)p.B * p.N * 3 * C * esize(in_dt), nout = (size_t)p.B * p.N * C * esize(out_dt);
  if (overlaps(out, nout, qkv, nin)) return LA_ERR_INVALID_ARG;
  for (const float* gm : {q_gamma, k_gamma}) {
    if (gm == nullptr) continue;
    if (!aligned(gm, 16) || overlaps(out, nout, gm, C * sizeof(float))) return LA_ERR_INVALID_ARG;
  }
  if ((q_gamma || k_gamma) && (!std::isfinite(norm_eps) || !(norm_eps > 0.f))) return LA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total_qkv) return LA_ERR_INVALID_ARG;
  float* sc = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ws_scale);
  pro->q_gamma = q_gamma;
  pro->k_gamma = k_gamma;
  pro->q_scale = sc;
  pro->k_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(sc) + align256((size_t)p.B * p.N * sizeof(float)));
  pro->norm_eps = norm_eps;
  const char* base = static_cast<const char*>(qkv);
  *q = base;
  *k = base + C * esize(in_dt);
  *v = base + 2 * C * esize(in_dt);
  return LA_OK;
}

// Shared checks of the temporal convolution entry points.
int check_conv(const void* x, const void* y, la_dtype in_dt, la_dtype out_dt, int B, int frames,
               int tpf, int ch, int kt, const float* w, const float* bias) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (B < 1 || frames < 1 || tpf < 1 || ch < 8 || (ch % 8) != 0) return LA_ERR_INVALID_ARG;
  if (kt != 2 && kt != 3) return LA_ERR_INVALID_ARG;
  if (!x || !y || !w || !aligned(x, 16) || !aligned(y, 16) || !aligned(w, 16)) return LA_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 16)) return LA_ERR_INVALID_ARG;
  if (B > 65535) return LA_ERR_UNSUPPORTED;
  const int wide = esize(in_dt) > esize(out_dt) ? esize(in_dt) : esize(out_dt);
  if ((long long)(frames + 16) * tpf * ch * wide >= (1LL << 32)) return LA_ERR_UNSUPPORTED;
  if ((long long)tpf * (ch / 8) > 0x7fffffffLL - 256) return LA_ERR_UNSUPPORTED;
  const size_t n = (size_t)B * frames * tpf * ch;
  const size_t nx = n * esize(in_dt), ny = n * esize(out_dt);
  if (overlaps(y, ny, x, nx) || overlaps(y, ny, w, (size_t)kt * ch * 4)) return LA_ERR_INVALID_ARG;
  if (bias && overlaps(y, ny, bias, (size_t)ch * 4)) return LA_ERR_INVALID_ARG;
  return LA_OK;
}


int backward_common(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                    void* dv, la_dtype in_dt, la_dtype grad_dt, int B, int H, int head_dim, int frames,
                    int tokens_per_frame, int block_frames, int first_block_frames, const la_rope* rope,
                    float eps, void* ws, size_t ws_bytes, void* stream, bool have_prefix) {
  if (!valid_dtype(in_dt) || !valid_dtype(grad_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                     rope, 0, in_dt);
  if (st != LA_OK) return st;
  // inputs q, k, v, dout; gradient outputs dq, dk, dv: each output checked
  // against the inputs (as the forward checks out) and against the others.
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  const size_t elems = (size_t)p.B * p.N * p.H * p.D;
  const size_t nin = elems * esize(in_dt), nout = elems * esize(grad_dt);
  for (const void* x : ins)
    if (!x || !aligned(x, 16)) return LA_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i) {
    if (!outs[i] || !aligned(outs[i], 16)) return LA_ERR_INVALID_ARG;
    for (const void* x : ins)
      if (overlaps(outs[i], nout, x, nin)) return LA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], nout, outs[j], nout)) return LA_ERR_INVALID_ARG;
    if (ws && overlaps(outs[i], nout, ws, ws_bytes)) return LA_ERR_INVALID_ARG;
  }
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total_bw) return LA_ERR_INVALID_ARG;
  st = check_scratch(p, ws, p.ws_total_bw, {nullptr, 0}, {{q, nin}, {k, nin}, {v, nin}, {dout, nin}}, rope);
  if (st != LA_OK) return st;
  for (int i = 0; i < 3; ++i)
    if (clashes({outs[i], nout}, {rope_span(rope)})) return LA_ERR_INVALID_ARG;
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_backward(p, q, k, v, dout, dq, dk, dv, in_dt == LA_BF16,
                                          grad_dt == LA_BF16, eps, ws, stream, have_prefix));
}
}  // namespace

extern "C" {

size_t rope_table_bytes(int d_t, int d_h, int d_w, int max_frames, int grid_h, int grid_w) {
  if (d_t < 0 || d_h < 0 || d_w < 0 || ((d_t | d_h | d_w) & 1)) return 0;
  if (max_frames < 1 || grid_h < 1 || grid_w < 1) return 0;
  return 8 * ((size_t)max_frames * (d_t / 2) + (size_t)grid_h * (d_h / 2) + (size_t)grid_w * (d_w / 2));
}

int rope_table_build(la_rope* out, float* table_dev, size_t bytes, int head_dim, int d_t, int d_h,
                     int d_w, int max_frames, int grid_h, int grid_w, double base, void* stream) {
  if (!out || !table_dev || !aligned(table_dev, 16)) return LA_ERR_INVALID_ARG;
  if (head_dim < 1) return LA_ERR_INVALID_ARG;
  if (!lavr::head_dim_built(head_dim)) return LA_ERR_UNSUPPORTED;
  if (d_t + d_h + d_w != head_dim) return LA_ERR_INVALID_ARG;
  const size_t need = rope_table_bytes(d_t, d_h, d_w, max_frames, grid_h, grid_w);
  if (need == 0 || bytes < need) return LA_ERR_INVALID_ARG;
  if (!(base > 0.0) || !std::isfinite(base)) return LA_ERR_INVALID_ARG;
  if ((long long)max_frames * (d_t / 2) > 0x7fffffffLL) return LA_ERR_UNSUPPORTED;
  const int e = lavr::launch_rope_table(table_dev, d_t / 2, d_h / 2, d_w / 2, max_frames, grid_h,
                                        grid_w, base, stream);
  if (e != 0) return LA_ERR_HIP;
  out->table = table_dev;
  out->d_t = d_t;
  out->d_h = d_h;
  out->d_w = d_w;
  out->max_frames = max_frames;
  out->grid_h = grid_h;
  out->grid_w = grid_w;
  return LA_OK;
}

size_t la_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                          int block_frames, int first_block_frames, const la_rope* rope) {
  Plan p;
  if (make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                rope, 0, LA_BF16) != LA_OK)
    return 0;
  return p.ws_total;
}

int la_block_causal_forward(const void* q, const void* k, const void* v, void* out,
                            la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                            int frames, int tokens_per_frame, int block_frames,
                            int first_block_frames, const la_rope* rope, float eps, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                     rope, 0, in_dt);
  if (st != LA_OK) return st;
  st = check_tensors(q, k, v, out, in_dt, out_dt, p);
  if (st != LA_OK) return st;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return LA_ERR_INVALID_ARG;
  const size_t nin = tensor_bytes(p, in_dt), nout = tensor_bytes(p, out_dt);
  st = check_scratch(p, ws, p.ws_total, {out, nout}, {{q, nin}, {k, nin}, {v, nin}}, rope);
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps,
                                         ws, nullptr, nullptr, nullptr, nullptr, stream));
}

size_t la_replay_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                                 int block_frames, const la_rope* rope) {
  if (block_frames < 1 || frames < 1 || frames % block_frames != 0) return 0;
  Plan p;
  if (make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, 0, rope, 0, LA_BF16, 1,
                true) != LA_OK)
    return 0;
  return p.ws_total;
}

int la_block_causal_forward_replay(const void* q, const void* k, const void* v, void* out,
                                   la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                                   int frames, int tokens_per_frame, int block_frames,
                                   const la_rope* rope, float eps, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  if (block_frames < 1 || frames < 1 || frames % block_frames != 0) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, 0, rope, 0, in_dt, 1,
                     true);
  if (st != LA_OK) return st;
  st = check_tensors(q, k, v, out, in_dt, out_dt, p);
  if (st != LA_OK) return st;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return LA_ERR_INVALID_ARG;
  const size_t nin = tensor_bytes(p, in_dt), nout = tensor_bytes(p, out_dt);
  st = check_scratch(p, ws, p.ws_total, {out, nout}, {{q, nin}, {k, nin}, {v, nin}}, rope);
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps,
                                         ws, nullptr, nullptr, nullptr, nullptr, stream));
}

int la_block_causal_forward_timed(const void* q, const void* k, const void* v, void* out,
                                  la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                                  int frames, int tokens_per_frame, int block_frames,
                                  int first_block_frames, const la_rope* rope, float eps,
                                  void* ws, size_t ws_bytes, void* stream, void* const* events) {
  if (!events) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                     rope, 0, in_dt);
  if (st != LA_OK) return st;
  st = check_tensors(q, k, v, out, in_dt, out_dt, p);
  if (st != LA_OK) return st;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return LA_ERR_INVALID_ARG;
  const size_t nin = tensor_bytes(p, in_dt), nout = tensor_bytes(p, out_dt);
  st = check_scratch(p, ws, p.ws_total, {out, nout}, {{q, nin}, {k, nin}, {v, nin}}, rope);
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps,
                                         ws, nullptr, nullptr, nullptr, nullptr, stream, events));
}

int la_block_causal_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                                    la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                                    int frames, int tokens_per_frame, int block_frames,
                                    int first_block_frames, const la_rope* rope, float eps,
                                    void* stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                     rope, 0, in_dt);
  if (st != LA_OK) return st;
  st = check_tensors(q, k, v, out, in_dt, out_dt, p);
  if (st != LA_OK) return st;
  if (p.ws_total > lavr::kScratchBytes) return LA_ERR_UNSUPPORTED;   // beyond the fixed workspace
  void* ws = nullptr;
  switch (lavr::noalloc_workspace(stream, &ws)) {
    case 0: break;
    case lavr::LAVR_NOALLOC_WRONG_DEVICE: return LA_ERR_INVALID_ARG;
    case lavr::LAVR_NOALLOC_UNSUPPORTED: return LA_ERR_UNSUPPORTED;
    default: return LA_ERR_HIP;
  }
  const size_t nin = tensor_bytes(p, in_dt), nout = tensor_bytes(p, out_dt);
  st = check_scratch(p, ws, p.ws_total, {out, nout}, {{q, nin}, {k, nin}, {v, nin}}, rope);
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps,
                                         ws, nullptr, nullptr, nullptr, nullptr, stream));
}

size_t la_backward_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                                   int block_frames, int first_block_frames, const la_rope* rope) {
  Plan p;
  if (make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                rope, 0, LA_BF16) != LA_OK)
    return 0;
  return p.ws_total_bw;
}

int la_block_causal_backward(const void* q, const void* k, const void* v, const void* dout,
                             void* dq, void* dk, void* dv, la_dtype in_dt, la_dtype grad_dt,
                             int B, int H, int head_dim, int frames, int tokens_per_frame,
                             int block_frames, int first_block_frames, const la_rope* rope,
                             float eps, void* ws, size_t ws_bytes, void* stream) {
  return backward_common(q, k, v, dout, dq, dk, dv, in_dt, grad_dt, B, H, head_dim, frames,
                         tokens_per_frame, block_frames, first_block_frames, rope, eps, ws, ws_bytes,
                         stream, false);
}

int la_block_causal_backward_from_forward(const void* q, const void* k, const void* v,
                                          const void* dout, void* dq, void* dk, void* dv,
                                          la_dtype in_dt, la_dtype grad_dt, int B, int H,
                                          int head_dim, int frames, int tokens_per_frame,
                                          int block_frames, int first_block_frames,
                                          const la_rope* rope, float eps, void* ws, size_t ws_bytes,
                                          void* stream) {
  return backward_common(q, k, v, dout, dq, dk, dv, in_dt, grad_dt, B, H, head_dim, frames,
                         tokens_per_frame, block_frames, first_block_frames, rope, eps, ws, ws_bytes,
                         stream, true);
}

size_t la_qkv_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                              int block_frames, int first_block_frames, const la_rope* rope) {
  Plan p;
  if (make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                rope, 0, LA_BF16, 3) != LA_OK)
    return 0;
  return p.ws_total_qkv;
}

int la_block_causal_forward_qkv(const void* qkv, void* out, la_dtype in_dt, la_dtype out_dt, int B,
                                int H, int head_dim, int frames, int tokens_per_frame,
                                int block_frames, int first_block_frames, const la_rope* rope,
                                float eps, const float* q_gamma, const float* k_gamma,
                                float norm_eps, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(&p, B, H, head_dim, frames, tokens_per_frame, block_frames, first_block_frames,
                     rope, 0, in_dt, 3);
  if (st != LA_OK) return st;
  lavr::Prologue pro;
  const void *q, *k, *v;
  st = check_fused(qkv, out, in_dt, out_dt, p, q_gamma, k_gamma, norm_eps, ws, ws_bytes, &pro, &q, &k, &v);
  if (st != LA_OK) return st;
  const size_t C4 = (size_t)p.H * p.D * 4;
  st = check_scratch(p, ws, p.ws_total_qkv, {out, tensor_bytes(p, out_dt)},
                     {{qkv, tensor_bytes(p, in_dt, 3)}, {q_gamma, C4}, {k_gamma, C4}}, rope);
  if (st != LA_OK) return st;
  return hip_status(lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps,
                                         ws, nullptr, nullptr, nullptr, nullptr, stream, nullptr, &pro));
}

int la_state_init(la_state* st, float* S_dev, float* z_dev, int B, int H, int head_dim,
                  void* stream) {
  if (!st || !S_dev || !z_dev || !aligned(S_dev, 16) || !aligned(z_dev, 16)) return LA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || head_dim < 1) return LA_ERR_INVALID_ARG;
  if (!lavr::head_dim_built(head_dim)) return LA_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535 || (long long)B * H > (1LL << 24)) return LA_ERR_UNSUPPORTED;
  const size_t nS = (size_t)B * H * head_dim * head_dim, nz = (size_t)B * H * head_dim;
  if (overlaps(S_dev, nS * 4, z_dev, nz * 4)) return LA_ERR_INVALID_ARG;
  int e = lavr::launch_zero(S_dev, nS, stream);
  if (e == 0) e = lavr::launch_zero(z_dev, nz, stream);
  if (e != 0) return LA_ERR_HIP;
  st->S = S_dev;
  st->z = z_dev;
  st->B = B;
  st->H = H;
  st->head_dim = head_dim;
  st->frames_done = 0;
  return LA_OK;
}

int la_stream_block(la_state* st, const void* q, const void* k, const void* v, void* out,
                    la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                    int block_frames, int tokens_per_frame, const la_rope* rope, float eps,
                    int save, void* ws, size_t ws_bytes, void* stream) {
  if (!st || !st->S || !st->z) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  if (st->frames_done < 0) return LA_ERR_INVALID_ARG;
  if (B != st->B || H != st->H || head_dim != st->head_dim) return LA_ERR_STATE_MISMATCH;
  Plan p;
  int rc = make_plan(&p, B, H, head_dim, block_frames, tokens_per_frame, block_frames, 0, rope,
                     st->frames_done, in_dt);
  if (rc != LA_OK) return rc;
  rc = check_tensors(q, k, v, out, in_dt, out_dt, p);
  if (rc != LA_OK) return rc;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.ws_total) return LA_ERR_INVALID_ARG;
  const size_t nin = tensor_bytes(p, in_dt), nout = tensor_bytes(p, out_dt);
  rc = check_scratch(p, ws, p.ws_total, {out, nout}, {{q, nin}, {k, nin}, {v, nin}}, rope, st);
  if (rc != LA_OK) return rc;
  const int e = lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps, ws,
                                     st->S, st->z, save ? st->S : nullptr, save ? st->z : nullptr,
                                     stream);
  if (e != 0) return LA_ERR_HIP;
  if (save) st->frames_done += block_frames;
  return LA_OK;
}

int la_stream_block_qkv(la_state* st, const void* qkv, void* out, la_dtype in_dt, la_dtype out_dt,
                        int B, int H, int head_dim, int block_frames, int tokens_per_frame,
                        const la_rope* rope, float eps, const float* q_gamma, const float* k_gamma,
                        float norm_eps, int save, void* ws, size_t ws_bytes, void* stream) {
  if (!st || !st->S || !st->z) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return LA_ERR_INVALID_ARG;
  if (st->frames_done < 0) return LA_ERR_INVALID_ARG;
  if (B != st->B || H != st->H || head_dim != st->head_dim) return LA_ERR_STATE_MISMATCH;
  Plan p;
  int rc = make_plan(&p, B, H, head_dim, block_frames, tokens_per_frame, block_frames, 0, rope,
                     st->frames_done, in_dt, 3);
  if (rc != LA_OK) return rc;
  lavr::Prologue pro;
  const void *q, *k, *v;
  rc = check_fused(qkv, out, in_dt, out_dt, p, q_gamma, k_gamma, norm_eps, ws, ws_bytes, &pro, &q, &k, &v);
  if (rc != LA_OK) return rc;
  const size_t C4 = (size_t)p.H * p.D * 4;
  rc = check_scratch(p, ws, p.ws_total_qkv, {out, tensor_bytes(p, out_dt)},
                     {{qkv, tensor_bytes(p, in_dt, 3)}, {q_gamma, C4}, {k_gamma, C4}}, rope, st);
  if (rc != LA_OK) return rc;
  const int e = lavr::launch_forward(p, q, k, v, out, in_dt == LA_BF16, out_dt == LA_BF16, eps, ws,
                                     st->S, st->z, save ? st->S : nullptr, save ? st->z : nullptr,
                                     stream, nullptr, &pro);
  if (e != 0) return LA_ERR_HIP;
  if (save) st->frames_done += block_frames;
  return LA_OK;
}

int la_temporal_conv(const void* x, void* y, la_dtype in_dt, la_dtype out_dt, int B, int frames,
                     int tokens_per_frame, int channels, int block_frames, int first_block_frames,
                     int kt, const float* w, const float* bias, void* stream) {
  if (block_frames < 1 || first_block_frames < 0) return LA_ERR_INVALID_ARG;
  const int st = check_conv(x, y, in_dt, out_dt, B, frames, tokens_per_frame, channels, kt, w, bias);
  if (st != LA_OK) return st;
  lavr::ConvPlan c{B, frames, tokens_per_frame, channels,
                   first_block_frames == 0 ? block_frames : first_block_frames, block_frames, kt};
  return hip_status(lavr::launch_tconv(c, x, y, in_dt == LA_BF16, out_dt == LA_BF16, w, bias, nullptr,
                                       nullptr, stream));
}

int la_conv_state_init(la_conv_state* st, void* last_dev, la_dtype dtype, int B, int tokens_per_frame,
                       int channels, void* stream) {
  if (!st || !last_dev || !aligned(last_dev, 16) || !valid_dtype(dtype)) return LA_ERR_INVALID_ARG;
  if (B < 1 || tokens_per_frame < 1 || channels < 8 || (channels % 8) != 0) return LA_ERR_INVALID_ARG;
  const size_t bytes = (size_t)B * tokens_per_frame * channels * esize(dtype);
  if (lavr::launch_zero(static_cast<float*>(last_dev), bytes / 4, stream) != 0) return LA_ERR_HIP;
  st->last = last_dev;
  st->B = B;
  st->tokens_per_frame = tokens_per_frame;
  st->channels = channels;
  st->dtype = dtype;
  st->frames_done = 0;
  return LA_OK;
}

int la_temporal_conv_stream_block(la_conv_state* st, const void* x, void* y, la_dtype out_dt, int B,
                                  int block_frames, int tokens_per_frame, int channels, int kt,
                                  const float* w, const float* bias, int save, void* stream) {
  if (!st || !st->last || !aligned(st->last, 16) || st->frames_done < 0) return LA_ERR_INVALID_ARG;
  if (block_frames < 1) return LA_ERR_INVALID_ARG;
  if (B != st->B || tokens_per_frame != st->tokens_per_frame || channels != st->channels)
    return LA_ERR_STATE_MISMATCH;
  const la_dtype in_dt = st->dtype;
  const int rc = check_conv(x, y, in_dt, out_dt, B, block_frames, tokens_per_frame, channels, kt, w, bias);
  if (rc != LA_OK) return rc;
  const size_t ny = (size_t)B * block_frames * tokens_per_frame * channels * esize(out_dt);
  const size_t nc = (size_t)B * tokens_per_frame * channels * esize(in_dt);
  if (overlaps(y, ny, st->last, nc)) return LA_ERR_INVALID_ARG;
  lavr::ConvPlan c{B, block_frames, tokens_per_frame, channels, block_frames, block_frames, kt};
  const int e = lavr::launch_tconv(c, x, y, in_dt == LA_BF16, out_dt == LA_BF16, w, bias, st->last,
                                   save ? st->last : nullptr, stream);
  if (e != 0) return LA_ERR_HIP;
  if (save) st->frames_done += block_frames;
  return LA_OK;
}

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG: invalid argument";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: not supported by this library";
    case LA_ERR_STATE_MISMATCH: return "LA_ERR_STATE_MISMATCH: state shape does not match the call";
    case LA_ERR_HIP: return "LA_ERR_HIP: HIP launch or runtime error";
    default: return "unknown la_status";
  }
}

const char* la_version(void) { return "0.5.0"; }

}  // extern "C"
