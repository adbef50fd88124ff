/*
 * la_vr.h -- C ABI of liblavr: block-causal ReLU linear attention with RoPE
 * (forward, one-shot and streaming; its backward; a fused q/k/v input with the
 * q/k RMSNorm prologue) and the cached temporal convolution of the causal
 * Mix-FFN, on AMD MI355X (gfx950).
 *
 * What is computed.  For every batch row b and head h, with phi = ReLU applied
 * elementwise to queries and keys ("Implementing Block Causal Linear Attention
 * for Long Video Generation with Sana", sections "What is Block Causal Linear
 * Attention?" and "The Linear Attention Kernel"), and R the rotary embedding
 * applied to phi(q) and phi(k) right after the ReLU (same page, "Rotary
 * Position Embeddings"):
 *
 *   block j of the sequence adds   S_j = sum_{n in j} v_n (R phi(k_n))^T   (d x d)
 *                                  z_j = sum_{n in j} phi(k_n)             (d)
 *   the prefix over blocks <= j    Sbar_j = sum_{j' <= j} S_j',  zbar_j likewise
 *   a token n of block j reads     out_n = Sbar_j (R phi(q_n)) / (zbar_j . phi(q_n) + eps)
 *
 * Tokens of block j see every token of blocks <= j, their own block included,
 * and nothing later (same page, "Chunk-Wise Causality"; "Block Causal Linear
 * Attention", happyin.space, "What SANA-Video Actually Uses": a block needs the
 * cumulative attention state and key summaries of earlier blocks).  The
 * normaliser uses the un-rotated phi(q), phi(k).  A streaming caller carries the
 * constant-size (S, z) cache between calls ("[feat] LongSANA: a minute-length
 * real-time video generation model", diffusers pull request 12723: the cache is
 * passed in and handed back on every call and an enable-save flag decides
 * whether a call updates it).
 *
 * Layouts.  q, k, v and out are contiguous row-major (B, N, H, head_dim) with
 * N = frames * tokens_per_frame; tokens are frame-major, then raster order
 * (row, col) inside a frame.  This is the (B, N, C) activation with C = H *
 * head_dim.  head_dim 32 and 64 are built (the per-head widths the walkthrough
 * names, "Integration into Sana's Video Backbone").
 *
 * Size limits.  A call takes at most 2^30 tokens per batch row (N = frames *
 * tokens_per_frame), B <= 65535 and B * H <= 2^24, and N * tokens_per_frame must
 * stay below 2^42 (exact integer division of token indices); past them a call
 * returns LA_ERR_UNSUPPORTED and the workspace-size queries return 0.  A batch
 * row may hold more than 4 GiB.
 *
 * RoPE.  head_dim is split into consecutive sections of d_t, d_h and d_w
 * channels that follow the token's frame index t, row and column.  Pair i
 * (channels 2i, 2i+1 of a section of width d_s) turns by the angle
 * pos * base^(-2i/d_s):  (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos).
 * A 1-D RoPE over the token index is tokens_per_frame = 1, d_t = head_dim,
 * d_h = d_w = 0.  The pages fix neither pairing nor frequencies; this is the
 * library's convention.
 *
 * Calling convention.  Every pointer argument named *_dev, q, k, v, out, ws,
 * S, z or table is device memory owned by the caller; the library never
 * allocates or frees device memory and keeps no global state (apart from the
 * fixed workspace of la_block_causal_forward_noalloc).  Every call
 * checks its arguments on the host first and returns an error code without
 * touching the GPU if they are wrong; otherwise it enqueues its kernels on
 * `stream` (a hipStream_t, NULL = default stream) and returns at once.  The
 * library never aborts and never prints.  A call enqueues kernels only (no
 * allocation, memset, copy or synchronisation), so calls on different streams
 * with their own workspaces run side by side, and one-shot forward and backward
 * calls can be captured into a HIP graph and replayed.  A streamed call reads
 * and advances la_state.frames_done on the host, so a captured one would replay
 * with the rotary frame offset it was captured with.
 */
#ifndef LA_VR_H
#define LA_VR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,     /* null/misaligned pointer, bad size, overlap, small workspace */
  LA_ERR_UNSUPPORTED = 2,     /* valid request the library does not build (head_dim not 32 or 64, ...) */
  LA_ERR_STATE_MISMATCH = 3,  /* la_state shape does not match the call */
  LA_ERR_HIP = 4              /* a HIP launch or runtime call failed */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Description of a rotary table built by rope_table_build.  table == NULL turns
 * RoPE off (identity rotation).  A table of 2^31 or more (cos, sin) pairs is
 * rejected (LA_ERR_INVALID_ARG): the kernels index it with 32-bit integers. */
typedef struct {
  const float* table;          /* device; (cos, sin) float pairs, see rope_table_bytes */
  int d_t, d_h, d_w;           /* even section widths, d_t + d_h + d_w == head_dim */
  int max_frames;              /* rows of the t section: frames 0 .. max_frames-1 */
  int grid_h, grid_w;          /* rows / columns of a frame (1, 1 for 1-D RoPE) */
} la_rope;

/* Streaming cache of one generation stream ("Block Causal Linear Attention",
 * happyin.space, "Integration Contract": one cache per stream, never shared).
 * S is [B][H][head_dim][head_dim] fp32 (S[e][f] multiplies channel f of the
 * rotated query), z is [B][H][head_dim] fp32, frames_done counts committed
 * frames and is the frame offset of the next call's RoPE.  (S, z, frames_done)
 * is the complete resumable state. */
typedef struct {
  float* S;
  float* z;
  int B, H, head_dim;
  long long frames_done;
} la_state;

/* Bytes of the rotary table: 8 * (max_frames*d_t/2 + grid_h*d_h/2 + grid_w*d_w/2).
 * Returns 0 for invalid sizes. */
size_t rope_table_bytes(int d_t, int d_h, int d_w, int max_frames, int grid_h, int grid_w);

/* Fill `table_dev` (bytes >= rope_table_bytes(...), 16-byte aligned) with cos and
 * sin of every (section, position, pair) angle, computed in float64 on the GPU
 * and rounded to float32, and describe it in *out.  The t section covers frames
 * 0 .. max_frames-1, the h section rows 0 .. grid_h-1, the w section columns
 * 0 .. grid_w-1.  base > 0 (10000 in every SANA configuration).  Layout: the
 * t section as [max_frames][d_t/2] pairs, then h as [grid_h][d_h/2], then w as
 * [grid_w][d_w/2]; a pair is (cos, sin). */
int rope_table_build(la_rope* out, float* table_dev, size_t bytes, int head_dim,
                     int d_t, int d_h, int d_w, int max_frames, int grid_h, int grid_w,
                     double base, void* stream);

/* Workspace bytes needed by la_block_causal_forward for this shape, block
 * schedule and rotary description (for la_stream_block pass frames =
 * block_frames and first_block_frames = 0).  rope is the description the call
 * will take (NULL or a NULL table = RoPE off): a block's work is split so that
 * each piece's rotary window fits on chip, and with short frames that can need
 * more pieces, and so more workspace, than without RoPE.  Only rope's fields
 * are read, not its table.  0 for invalid sizes or descriptions. */
size_t la_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                          int block_frames, int first_block_frames, const la_rope* rope);

/* One-shot block-causal forward over `frames` frames, starting from an empty
 * cache.  Blocks: the first holds first_block_frames frames (0 means
 * block_frames: a uniform schedule), every later one block_frames frames, and
 * the last may be shorter.  A first chunk one frame longer than the others is
 * the schedule the SANA-WM pipeline pull request (huggingface/diffusers 13881,
 * review thread) names as its configuration; a block of frames sees itself and
 * every earlier block ("Implementing Block Causal Linear Attention for Long
 * Video Generation with Sana", "Chunk-Wise Causality").
 * q, k, v have dtype in_dt, out has dtype out_dt (LA_BF16 out is rounded to
 * nearest even from the fp32 result).  All accumulation is fp32.  eps >= 0 is
 * added to the normaliser (1e-8 in SANA).  ws (256-byte aligned, ws_bytes >=
 * la_workspace_bytes) is scratch owned by the caller and must not be touched
 * by other work until the call's kernels finish.  out must not overlap q, k, v;
 * the used part of ws must not overlap q, k, v, out or the rotary table, nor
 * out the table (LA_ERR_INVALID_ARG).
 * If rope->table is non-NULL, frames <= rope->max_frames and, when d_h + d_w >
 * 0, grid_h * grid_w == tokens_per_frame.  rope may be NULL (RoPE off). */
int la_block_causal_forward(const void* q, const void* k, const void* v, void* out,
                            la_dtype in_dt, la_dtype out_dt,
                            int B, int H, int head_dim, int frames, int tokens_per_frame,
                            int block_frames, int first_block_frames, const la_rope* rope,
                            float eps, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of la_block_causal_forward_replay (0 if the shape is invalid,
 * including frames not a multiple of block_frames). */
size_t la_replay_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                                 int block_frames, const la_rope* rope);

/* One-shot forward for deterministic replay ("Block Causal Linear Attention",
 * happyin.space, "Integration Contract" and "Acceptance Checks": streaming must
 * reproduce the one-shot result).  Its output equals, bit for bit, the outputs
 * of streaming the same clip block by block with la_stream_block (save = 1,
 * from a zeroed state, the same B, H, head_dim, block_frames, tokens_per_frame,
 * rotary table, eps and output dtype).  la_block_causal_forward splits each
 * block into chunks sized for the whole clip's launch, a streamed call into
 * chunks sized for one block, and the fp32 block sums then round differently
 * (about one bf16 step apart); this entry point takes the streamed split for
 * every block, at the cost of more, shorter chunks on long clips.  The clip
 * must consist of whole blocks (frames a multiple of block_frames, else
 * LA_ERR_INVALID_ARG); arguments and errors are otherwise those of
 * la_block_causal_forward, with ws sized by la_replay_workspace_bytes.  Its
 * workspace is not one that la_block_causal_backward_from_forward accepts. */
int la_block_causal_forward_replay(const void* q, const void* k, const void* v, void* out,
                                   la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                                   int frames, int tokens_per_frame, int block_frames,
                                   const la_rope* rope, float eps, void* ws, size_t ws_bytes,
                                   void* stream);

/* la_block_causal_forward that also times its two large kernels with
 * caller-created hipEvent_t events: events[0] and events[1] take the start and
 * end of the block-state kernel, events[2] and events[3] the start and end of
 * the readout, so hipEventElapsedTime gives each kernel's duration, and the
 * span from events[1] to events[2] the prefix kernel with the launch
 * boundaries around it.  The events are bound to the kernels' own dispatches
 * (hipExtLaunchKernel), so they add no command between the kernels and the
 * timed call runs the same timeline as la_block_causal_forward.  events must
 * not be NULL; an entry that is NULL is not recorded.  Not for HIP graph
 * capture (use la_block_causal_forward there). */
int la_block_causal_forward_timed(const void* q, const void* k, const void* v, void* out,
                                  la_dtype in_dt, la_dtype out_dt,
                                  int B, int H, int head_dim, int frames, int tokens_per_frame,
                                  int block_frames, int first_block_frames, const la_rope* rope,
                                  float eps, void* ws, size_t ws_bytes, void* stream,
                                  void* const* events);

/* la_block_causal_forward for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  The caller passes inputs and outputs only; the workspace is a
 * fixed device array inside the library, 64 MiB on each GPU the library runs
 * on (enough for a 240-frame 480p clip at 70 heads), set up on the first call
 * on a device and held until the process ends.  The call allocates nothing and
 * makes no allocating library call.  Every call on one GPU shares that GPU's
 * array, so calls whose kernels overlap on one GPU (concurrent streams, or
 * other threads) race and give wrong results: serialise them.  stream must
 * belong to the current device (else LA_ERR_INVALID_ARG).  A shape whose
 * workspace (la_workspace_bytes) exceeds 64 MiB returns LA_ERR_UNSUPPORTED
 * before any HIP call.  Arguments, results and other status codes as for
 * la_block_causal_forward. */
int la_block_causal_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                                    la_dtype in_dt, la_dtype out_dt,
                                    int B, int H, int head_dim, int frames, int tokens_per_frame,
                                    int block_frames, int first_block_frames, const la_rope* rope,
                                    float eps, void* stream);

/* Workspace bytes needed by la_block_causal_backward (and by a forward whose
 * workspace la_block_causal_backward_from_forward will reuse) for this shape,
 * schedule and rotary description (rope as for la_workspace_bytes; 0 for
 * invalid sizes). */
size_t la_backward_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                                   int block_frames, int first_block_frames, const la_rope* rope);

/* Gradients of sum(dout * out) with respect to q, k and v, where out is what
 * la_block_causal_forward returns for the same arguments.  The pages state the
 * forward only ("Implementing Block Causal Linear Attention for Long Video
 * Generation with Sana", "The Linear Attention Kernel" and "Chunk-Wise
 * Causality"); this is its exact derivative (ReLU's derivative taken as 0 at
 * 0), for training.  q, k, v and dout have dtype in_dt and layout (B, N, H,
 * head_dim); dq, dk, dv have dtype grad_dt and the same layout, and must not
 * overlap the inputs or each other.  Head dims 32 and 64 are built, as for the
 * forward.  The block states are formed again from
 * k and v.  ws (256-byte aligned, ws_bytes >= la_backward_workspace_bytes) is
 * caller-owned scratch; its used part must not overlap the inputs, the
 * gradients or the rotary table, nor the gradients the table.  Same status
 * codes and stream semantics as the forward. */
int la_block_causal_backward(const void* q, const void* k, const void* v, const void* dout,
                             void* dq, void* dk, void* dv, la_dtype in_dt, la_dtype grad_dt,
                             int B, int H, int head_dim, int frames, int tokens_per_frame,
                             int block_frames, int first_block_frames, const la_rope* rope,
                             float eps, void* ws, size_t ws_bytes, void* stream);

/* la_block_causal_backward for training, where the forward has just run: ws
 * (ws_bytes >= la_backward_workspace_bytes) must be the workspace that a
 * la_block_causal_forward call with the same q, k, v and arguments (out dtype
 * aside) wrote, left untouched since; the block prefixes it holds are used as
 * they are instead of being formed again from k and v.  The result is the one
 * la_block_causal_backward gives, bit for bit.  The forward stores a 128-bit
 * fingerprint of what its prefixes were formed from (shape, block schedule,
 * rotary table and offset, the k and v pointers, the input dtype and any k
 * norm) in the workspace; if the fingerprint does not match this call's
 * arguments (another shape or schedule, another k or v, a fused-input forward,
 * a workspace no forward wrote), the call still returns LA_OK but fills dq, dk
 * and dv with NaN.  Contents of k or v changed in place since the forward are
 * not detected. */
int la_block_causal_backward_from_forward(const void* q, const void* k, const void* v,
                                          const void* dout, void* dq, void* dk, void* dv,
                                          la_dtype in_dt, la_dtype grad_dt, int B, int H,
                                          int head_dim, int frames, int tokens_per_frame,
                                          int block_frames, int first_block_frames,
                                          const la_rope* rope, float eps, void* ws, size_t ws_bytes,
                                          void* stream);

/* Bind the caller's device buffers S_dev ([B][H][d][d] fp32) and z_dev
 * ([B][H][d] fp32), both 16-byte aligned, to *st, zero them on `stream`, and set
 * frames_done = 0. */
int la_state_init(la_state* st, float* S_dev, float* z_dev, int B, int H, int head_dim,
                  void* stream);

/* Streaming step: q, k, v, out hold exactly one block of block_frames frames,
 * shape (B, block_frames * tokens_per_frame, H, head_dim); (B, H, head_dim) must
 * equal the state's, else LA_ERR_STATE_MISMATCH.  The block
 * reads the cache plus its own contribution; RoPE frame offset is
 * st->frames_done.  With save != 0 the cache becomes cache + this block and
 * st->frames_done advances by block_frames (on the host, at enqueue time);
 * with save == 0 the cache is left unchanged (several denoising steps of one
 * block may reuse it, [feat] LongSANA pull request: timesteps per chunk).
 * The result is the one-shot result of the concatenated blocks.  Workspace as
 * for la_block_causal_forward with frames = block_frames; the state's S and z
 * must not overlap q, k, v, out, the workspace or the rotary table. */
int la_stream_block(la_state* st, const void* q, const void* k, const void* v, void* out,
                    la_dtype in_dt, la_dtype out_dt, int B, int H, int head_dim,
                    int block_frames, int tokens_per_frame, const la_rope* rope, float eps,
                    int save, void* ws, size_t ws_bytes, void* stream);

/* Fused prologue.  The projection of x (B, N, C) to queries, keys and values
 * ("Implementing Block Causal Linear Attention for Long Video Generation with
 * Sana", "The Linear Attention Kernel", step 1) hands over one contiguous
 * (B, N, 3, C) tensor qkv: each token row holds q (C = H * head_dim channels,
 * heads in order), then k, then v.  The attention module's qk_norm flag (same
 * page, "Direct Instantiation of ChunkCausalAttention") is taken as RMSNorm of
 * each token's q and k over its C channels, with one weight per channel:
 *   x_hat = x / sqrt(mean_C(x^2) + norm_eps) * gamma,
 * applied before phi (a weight may be negative).  The pages name the flag
 * only; this reading is the library's.  The kernels read q, k, v in place
 * from the fused rows, so neither a split copy nor normalised q and k make a
 * round trip through memory; a small pre-pass forms the per-token 1 / rms
 * values (8 bytes per token in the workspace). */

/* Workspace bytes of la_block_causal_forward_qkv (for la_stream_block_qkv pass
 * frames = block_frames and first_block_frames = 0; rope as for
 * la_workspace_bytes).  0 for invalid sizes. */
size_t la_qkv_workspace_bytes(int B, int H, int head_dim, int frames, int tokens_per_frame,
                              int block_frames, int first_block_frames, const la_rope* rope);

/* la_block_causal_forward from the fused input qkv (B, N, 3, H * head_dim) of
 * dtype in_dt (16-byte aligned).  q_gamma and k_gamma are device arrays of
 * H * head_dim fp32 weights (16-byte aligned), or NULL to leave that tensor
 * unnormalised; norm_eps must be finite and > 0 when either is given.  out is
 * (B, N, H, head_dim) of dtype out_dt and must not overlap qkv or the weights.
 * ws (256-byte aligned, ws_bytes >= la_qkv_workspace_bytes) is caller-owned
 * scratch; its used part must not overlap qkv, out, the weights or the
 * rotary table.  Block schedule, RoPE, eps, status codes and stream semantics as
 * for la_block_causal_forward. */
int la_block_causal_forward_qkv(const void* qkv, void* out, la_dtype in_dt, la_dtype out_dt,
                                int B, int H, int head_dim, int frames, int tokens_per_frame,
                                int block_frames, int first_block_frames, const la_rope* rope,
                                float eps, const float* q_gamma, const float* k_gamma,
                                float norm_eps, void* ws, size_t ws_bytes, void* stream);

/* la_stream_block from the fused input: qkv is (B, block_frames *
 * tokens_per_frame, 3, H * head_dim); weights and norm_eps as for
 * la_block_causal_forward_qkv; cache semantics as for la_stream_block. */
int la_stream_block_qkv(la_state* st, const void* qkv, void* out, la_dtype in_dt, la_dtype out_dt,
                        int B, int H, int head_dim, int block_frames, int tokens_per_frame,
                        const la_rope* rope, float eps, const float* q_gamma,
                        const float* k_gamma, float norm_eps, int save, void* ws,
                        size_t ws_bytes, void* stream);

/* Cached temporal convolution of the causal Mix-FFN.  The pages say that the
 * causal Mix-FFN keeps the previous block's last frame for its temporal
 * convolution ("Block Causal Linear Attention", happyin.space, "What SANA-Video
 * Actually Uses"; "[feat] LongSANA ..." pull request: causal logic for the
 * Mix-FFN, block CachedGLUMBConvTemp).  The library's reading: a depthwise
 * convolution along frames at every spatial position,
 *   y[t] = bias + sum_{i < kt} w[i] * x[t + i - 1],
 * kt = 3 (frames t-1, t, t+1) or kt = 2 (t-1, t).  Inside a block the taps see
 * the block's frames; before a block's first frame they see the previous
 * block's last frame (zeros before the first block of a stream), after its
 * last frame zeros.  x and y are contiguous (B, frames * tokens_per_frame,
 * channels), frame-major tokens as for attention; w is (kt, channels) fp32,
 * bias (channels) fp32 or NULL; channels is a multiple of 8; accumulation is
 * fp32 and a bf16 y is rounded to nearest even.  All pointers 16-byte aligned;
 * y must not overlap x, w, bias or the cache.  One batch row of x or y
 * (plus 16 frames) must stay below 4 GiB, else LA_ERR_UNSUPPORTED. */

/* Streaming cache of the temporal convolution: `last` is the last frame of the
 * last committed block, (B, tokens_per_frame, channels) in `dtype` (device,
 * caller-owned); frames_done counts committed frames. */
typedef struct {
  void* last;
  int B, tokens_per_frame, channels;
  la_dtype dtype;
  long long frames_done;
} la_conv_state;

/* One-shot convolution over `frames` frames in blocks (first_block_frames as
 * for la_block_causal_forward; the first block starts from zeros). */
int la_temporal_conv(const void* x, void* y, la_dtype in_dt, la_dtype out_dt, int B, int frames,
                     int tokens_per_frame, int channels, int block_frames, int first_block_frames,
                     int kt, const float* w, const float* bias, void* stream);

/* Bind and zero the caller's cache buffer last_dev (B * tokens_per_frame *
 * channels elements of dtype) on `stream`; frames_done = 0. */
int la_conv_state_init(la_conv_state* st, void* last_dev, la_dtype dtype, int B, int tokens_per_frame,
                       int channels, void* stream);

/* One streamed block of block_frames frames: x (B, block_frames *
 * tokens_per_frame, channels) in the cache's dtype.  The block's first frame
 * reads the cache; with save != 0 the cache becomes the block's last frame and
 * frames_done advances (on the host, at enqueue time), with save == 0 the cache
 * is unchanged.  (B, tokens_per_frame, channels) must equal the cache's, else
 * LA_ERR_STATE_MISMATCH. */
int la_temporal_conv_stream_block(la_conv_state* st, const void* x, void* y, la_dtype out_dt, int B,
                                  int block_frames, int tokens_per_frame, int channels, int kt,
                                  const float* w, const float* bias, int save, void* stream);

/* Static, human-readable name of a status code. */
const char* la_status_string(int status);

/* Library version as "major.minor.patch". */
const char* la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_VR_H */
