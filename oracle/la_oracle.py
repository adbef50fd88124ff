"""fp64 CPU oracle for block-causal ReLU linear attention with RoPE.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the HIP library and imports nothing from it: callers hand it plain numpy
arrays (bf16/fp32 values widened exactly to float64).

Pages cited (short tags used below):
  [ImplBCLA]  "Implementing Block Causal Linear Attention for Long Video
              Generation with Sana" (instagit.com walkthrough of the Sana repo).
  [BCLA]      "Block Causal Linear Attention" (happyin.space).
  [LongSANA]  "[feat] LongSANA: a minute-length real-time video generation
              model" (huggingface/diffusers pull request 12723).
  [SANA-WM]   the SANA-WM pipeline pull request (huggingface/diffusers 13881).

What is computed, per (batch b, head h), with phi = ReLU:
  fq = phi(q), fk = phi(k)                  [ImplBCLA, "The Linear Attention Kernel", steps 3]
  rq = R(fq), rk = R(fk)  (RoPE after phi)  [ImplBCLA, "Rotary Position Embeddings"]
  running over blocks j = 0, 1, ... in order:
     S += v_j^T . rk_j      (d x d)         [ImplBCLA, "The Linear Attention Kernel", vk line]
     z += sum_n fk_n        (d)             [ImplBCLA, same listing, key-sum in the z line]
     out_j = (rq_j . S^T) / (fq_j . z + eps)
  i.e. tokens of block j read the inclusive prefix of blocks <= j
  [ImplBCLA, "Chunk-Wise Causality" and "Summary"; BCLA, "What SANA-Video Actually
  Uses": cumulative attention-state and key summaries].

Readings where the pages are silent or ambiguous (each one is restated where it
is used):
  - causality is across blocks only; inside a block every token sees the whole
    block (a block of one token is the token-causal form);
  - the prefix is inclusive (a block sees itself);
  - the numerator uses the rotated vectors, the normaliser the un-rotated ones;
  - RoPE rotates adjacent channel pairs (2i, 2i+1) by +angle; the head dim is
    split into consecutive sections t, h, w; pair i of a section of width d_s
    turns by pos * base**(-2i/d_s);  positions are 0-based, tokens are frame-major
    then raster (row, col) in the frame, t is the absolute latent-frame index;
    RoPE convention: parity unpinned by the pages (a documented convention,
    checked only for internal consistency and its textbook special cases);
  - a last block shorter than the others is allowed;
  - eps = 1e-8 is added to the normaliser ([ImplBCLA], constructor default).
"""

import numpy as np

EPS_DEFAULT = 1e-8  # [ImplBCLA, "Architecture and Implementation Details"]


# --------------------------------------------------------------------------- RoPE

def token_positions(n_tokens, tokens_per_frame, grid_w, t0=0):
    """(t, row, col) of each token: frame-major, raster order inside a frame.

    Token n sits in frame n // tpf at raster index n % tpf = row * grid_w + col.
    t is shifted by t0 (the number of frames already streamed).
    """
    n = np.arange(n_tokens, dtype=np.int64)
    t = n // tokens_per_frame + t0
    r = n % tokens_per_frame
    if grid_w > 0:
        row, col = r // grid_w, r % grid_w
    else:
        row, col = np.zeros_like(r), np.zeros_like(r)
    return t, row, col


def rope_rotate(x, pos_t, pos_h, pos_w, split, base):
    """Rotate adjacent channel pairs of x (n, d) section by section.

    split = (d_t, d_h, d_w): channels [0, d_t) follow t, [d_t, d_t+d_h) follow the
    row, the rest the column ([SANA-WM] names a 3-D t/h/w rotary embedding).
    Pair i of a section of width d_s turns by pos * base**(-2 i / d_s); cos and sin
    are taken in float64.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    off = 0
    for d_s, pos in zip(split, (pos_t, pos_h, pos_w)):
        for i in range(d_s // 2):
            theta = float(base) ** (-2.0 * i / d_s)
            ang = np.asarray(pos, dtype=np.float64) * theta
            c, s = np.cos(ang), np.sin(ang)
            a, b = off + 2 * i, off + 2 * i + 1
            xa, xb = x[:, a].copy(), x[:, b].copy()
            x[:, a] = xa * c - xb * s
            x[:, b] = xa * s + xb * c
        off += d_s
    return x


def _rotate_tokens(x, rope, tokens_per_frame, t0):
    """Apply RoPE (or nothing when rope is None) to x (n, d)."""
    if rope is None:
        return np.array(x, dtype=np.float64, copy=True)
    t, row, col = token_positions(x.shape[0], tokens_per_frame, rope["grid"][1], t0)
    return rope_rotate(x, t, row, col, rope["split"], rope["base"])


def _relu(x):
    # phi = ReLU on queries and keys [ImplBCLA, "What is Block Causal Linear Attention?"]
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


# ------------------------------------------------------------------ one-shot forward

def block_bounds(n_tokens, block_tokens, first_tokens=None):
    """Token ranges [s, e) of the blocks; the last one may be shorter.

    first_tokens (default block_tokens) is the length of the first block: a
    schedule whose first chunk holds one frame more than the others is named in
    [SANA-WM] (review thread: the configuration uses "first_chunk_plus_one").
    """
    first = block_tokens if first_tokens is None else first_tokens
    bounds = [(0, min(first, n_tokens))]
    s = first
    while s < n_tokens:
        bounds.append((s, min(s + block_tokens, n_tokens)))
        s += block_tokens
    return bounds


def _head_forward(q, k, v, tokens_per_frame, block_frames, rope, eps, t0, S, z,
                  first_block_frames=None):
    """One (batch, head) stream: q, k, v are (n, d); S (d, d) and z (d) are updated in place."""
    fq, fk = _relu(q), _relu(k)
    rq = _rotate_tokens(fq, rope, tokens_per_frame, t0)
    rk = _rotate_tokens(fk, rope, tokens_per_frame, t0)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    first = None if first_block_frames is None else first_block_frames * tokens_per_frame
    for s, e in block_bounds(q.shape[0], block_frames * tokens_per_frame, first):
        S += v[s:e].T @ rk[s:e]          # S[e_, f] += sum_n v[n, e_] * rk[n, f]
        z += fk[s:e].sum(axis=0)         # un-rotated key-sum
        num = rq[s:e] @ S.T              # num[n, e_] = sum_f S[e_, f] * rq[n, f]
        den = fq[s:e] @ z + eps          # un-rotated query in the normaliser
        out[s:e] = num / den[:, None]
    return out


def forward(q, k, v, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
            first_block_frames=None):
    """Block-causal forward over whole sequences.

    q, k, v: (B, N, H, d) arrays (any float dtype; taken as float64).
    rope: None (no rotation) or {"split": (d_t, d_h, d_w), "grid": (rows, cols),
    "base": float}.  first_block_frames: frames of the first block (default
    block_frames).  Returns out (B, N, H, d) float64.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            S, z = np.zeros((d, d)), np.zeros(d)
            out[b, :, h] = _head_forward(q[b, :, h], k[b, :, h], v[b, :, h],
                                         tokens_per_frame, block_frames, rope, eps, 0, S, z,
                                         first_block_frames)
    return out


def forward_head(q, k, v, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
                 first_block_frames=None):
    """Same as forward for one (batch, head) slice: q, k, v are (N, d)."""
    d = q.shape[1]
    S, z = np.zeros((d, d)), np.zeros(d)
    return _head_forward(q, k, v, tokens_per_frame, block_frames, rope, eps, 0, S, z,
                         first_block_frames)


def block_states(k, v, tokens_per_frame, block_frames, rope=None, t0=0, first_block_frames=None):
    """Inclusive prefix states (S_bar_j, z_bar_j) of every block of one head (k, v: (N, d))."""
    fk = _relu(k)
    rk = _rotate_tokens(fk, rope, tokens_per_frame, t0)
    v = np.asarray(v, dtype=np.float64)
    d = k.shape[1]
    S, z = np.zeros((d, d)), np.zeros(d)
    Ss, zs = [], []
    first = None if first_block_frames is None else first_block_frames * tokens_per_frame
    for s, e in block_bounds(k.shape[0], block_frames * tokens_per_frame, first):
        S = S + v[s:e].T @ rk[s:e]
        z = z + fk[s:e].sum(axis=0)
        Ss.append(S.copy())
        zs.append(z.copy())
    return np.array(Ss), np.array(zs)


def readout_tokens(q, n_idx, S_bar, z_bar, tokens_per_frame, rope=None, eps=EPS_DEFAULT, t0=0):
    """Outputs of chosen tokens n_idx of one head, given that head's block prefix state.

    q: (m, d) rows of the tokens n_idx; S_bar (d, d), z_bar (d) is the inclusive
    prefix of the block those tokens sit in.  Used to check sampled outputs of large runs.
    """
    fq = _relu(q)
    if rope is None:
        rq = fq
    else:
        t, row, col = token_positions(int(np.max(n_idx)) + 1, tokens_per_frame, rope["grid"][1], t0)
        n_idx = np.asarray(n_idx)
        rq = rope_rotate(fq, t[n_idx], row[n_idx], col[n_idx], rope["split"], rope["base"])
    return (rq @ S_bar.T) / (fq @ z_bar + eps)[:, None]


# ------------------------------------------------------------------------ backward

def _unrotate_tokens(y, rope, tokens_per_frame, t0):
    """R^T y: each pair turns by minus its angle (the transpose of a rotation)."""
    if rope is None:
        return np.array(y, dtype=np.float64, copy=True)
    t, row, col = token_positions(y.shape[0], tokens_per_frame, rope["grid"][1], t0)
    return rope_rotate(y, -t, -row, -col, rope["split"], rope["base"])


def backward_head(q, k, v, g, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
                  first_block_frames=None):
    """Gradients (dq, dk, dv) of sum(g * out) for one (batch, head); q, k, v, g: (N, d).

    The pages give the forward only; this is its exact derivative, written out
    from the forward's definition (token n of block j, p = phi(q_n), r = R p,
    den = zbar_j . p + eps, out = Sbar_j r / den):
      a = g / den, beta = -(g . out) / den,
      dq = [q > 0] * (R^T Sbar_j^T a + beta zbar_j),
      G_j = sum_n a r^T, gz_j = sum_n beta p over block j,
      dS_i = sum_{j >= i} G_j, dz_i = sum_{j >= i} gz_j (blocks at or after i see block i),
      dv_m = dS_i kappa_m, dk_m = [k > 0] * (R^T dS_i^T v_m + dz_i), kappa = R phi(k).
    ReLU's derivative is taken as 0 at 0.
    """
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    N, d = q.shape
    fq, fk = _relu(q), _relu(k)
    rq = _rotate_tokens(fq, rope, tokens_per_frame, 0)
    rk = _rotate_tokens(fk, rope, tokens_per_frame, 0)
    first = None if first_block_frames is None else first_block_frames * tokens_per_frame
    bounds = block_bounds(N, block_frames * tokens_per_frame, first)
    S, z = np.zeros((d, d)), np.zeros(d)
    Sbar, zbar = [], []
    for s, e in bounds:
        S = S + v[s:e].T @ rk[s:e]
        z = z + fk[s:e].sum(axis=0)
        Sbar.append(S)
        zbar.append(z)
    dr, dp = np.zeros((N, d)), np.zeros((N, d))
    G, gz = [], []
    for jb, (s, e) in enumerate(bounds):
        den = fq[s:e] @ zbar[jb] + eps
        out = (rq[s:e] @ Sbar[jb].T) / den[:, None]
        a = g[s:e] / den[:, None]
        beta = -np.sum(g[s:e] * out, axis=1) / den
        dr[s:e] = a @ Sbar[jb]                 # row n: Sbar^T a_n
        dp[s:e] = beta[:, None] * zbar[jb][None, :]
        G.append(a.T @ rq[s:e])                # G[e, f] = sum_n a_n[e] r_n[f]
        gz.append(beta @ fq[s:e])
    nb = len(bounds)
    dS, dz = [None] * nb, [None] * nb
    accS, accz = np.zeros((d, d)), np.zeros(d)
    for i in reversed(range(nb)):
        accS = accS + G[i]
        accz = accz + gz[i]
        dS[i], dz[i] = accS, accz
    dv, dkr, dku = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for i, (s, e) in enumerate(bounds):
        dv[s:e] = rk[s:e] @ dS[i].T            # dv_m[e] = sum_f dS[e, f] kappa_m[f]
        dkr[s:e] = v[s:e] @ dS[i]              # d kappa_m[f] = sum_e dS[e, f] v_m[e]
        dku[s:e] = dz[i][None, :]
    dq = (q > 0) * (_unrotate_tokens(dr, rope, tokens_per_frame, 0) + dp)
    dk = (k > 0) * (_unrotate_tokens(dkr, rope, tokens_per_frame, 0) + dku)
    return dq, dk, dv


def backward(q, k, v, g, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
             first_block_frames=None):
    """backward_head over (B, N, H, d) arrays; returns dq, dk, dv (float64)."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    B, N, H, d = q.shape
    dq, dk, dv = (np.empty((B, N, H, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = backward_head(
                q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], tokens_per_frame, block_frames,
                rope, eps, first_block_frames)
    return dq, dk, dv


# ------------------------------------------------------------------------ streaming

class StreamState:
    """Constant-size cache carried between streamed blocks.

    Holds S (B, H, d, d), z (B, H, d) and the number of frames already committed
    ([BCLA, "What SANA-Video Actually Uses"]; [LongSANA]: the cache is passed in and
    returned on every call, an enable-save flag decides whether it is updated).
    """

    def __init__(self, B, H, d):
        self.S = np.zeros((B, H, d, d))
        self.z = np.zeros((B, H, d))
        self.frames_done = 0


def stream_block(state, q, k, v, tokens_per_frame, rope=None, eps=EPS_DEFAULT, save=True):
    """Process one block (all of q, k, v's N tokens form one block) against the cache.

    The block reads old state + its own contribution (inclusive prefix).  With
    save, the sum is committed and frames_done advances; without it the cache is
    left as it was (several denoising steps may reuse one committed cache).
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, d = q.shape
    frames = N // tokens_per_frame
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            S, z = state.S[b, h].copy(), state.z[b, h].copy()
            out[b, :, h] = _head_forward(q[b, :, h], k[b, :, h], v[b, :, h], tokens_per_frame,
                                         frames, rope, eps, state.frames_done, S, z)
            if save:
                state.S[b, h], state.z[b, h] = S, z
    if save:
        state.frames_done += frames
    return out


# ------------------------------------------------------ fused q/k/v prologue
#
# The projection of x (B, N, C) to q, k, v gives one (B, N, 3, C) tensor: per
# token row q (C channels), then k, then v ([ImplBCLA], "The Linear Attention
# Kernel", step 1: x projects to Q/K/V through learned weights; the (3, C) order
# inside a row is a reading, the pages do not fix it).  qk_norm ([ImplBCLA],
# "Direct Instantiation of ChunkCausalAttention", the qk_norm flag) is read as
# RMSNorm -- the norm class the pages name ([SANA-WM], review thread) -- over
# the C channels of each token's q and of its k, before the split into heads,
# with one learned weight per channel.  The pages give no eps for it; it is an
# argument here.

NORM_EPS_DEFAULT = 1e-6


def qk_rms_norm(x, gamma, norm_eps=NORM_EPS_DEFAULT):
    """RMSNorm over the last axis: x / sqrt(mean(x**2) + norm_eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + norm_eps) * np.asarray(gamma, dtype=np.float64)


def split_qkv(qkv, heads):
    """(B, N, 3, C) projection output -> q, k, v as (B, N, C) float64 arrays."""
    qkv = np.asarray(qkv, dtype=np.float64)
    B, N, three, C = qkv.shape
    if three != 3 or C % heads:
        raise ValueError("qkv must be (B, N, 3, heads * head_dim)")
    return qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]


def _prologue(qkv, heads, q_gamma, k_gamma, norm_eps):
    q, k, v = split_qkv(qkv, heads)
    if q_gamma is not None:
        q = qk_rms_norm(q, q_gamma, norm_eps)
    if k_gamma is not None:
        k = qk_rms_norm(k, k_gamma, norm_eps)
    B, N, C = q.shape
    d = C // heads
    return tuple(a.reshape(B, N, heads, d) for a in (q, k, v))


def forward_qkv(qkv, heads, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
                q_gamma=None, k_gamma=None, norm_eps=NORM_EPS_DEFAULT, first_block_frames=None):
    """Block-causal forward from the fused (B, N, 3, C) projection output, with
    the optional q/k RMSNorm (a None weight leaves that tensor as it is).
    Returns out (B, N, heads, C // heads) float64."""
    q, k, v = _prologue(qkv, heads, q_gamma, k_gamma, norm_eps)
    return forward(q, k, v, tokens_per_frame, block_frames, rope, eps,
                   first_block_frames=first_block_frames)


def stream_block_qkv(state, qkv, heads, tokens_per_frame, rope=None, eps=EPS_DEFAULT,
                     q_gamma=None, k_gamma=None, norm_eps=NORM_EPS_DEFAULT, save=True):
    """stream_block from the fused projection output (see forward_qkv)."""
    q, k, v = _prologue(qkv, heads, q_gamma, k_gamma, norm_eps)
    return stream_block(state, q, k, v, tokens_per_frame, rope, eps, save)


# ----------------------------------------------- cached temporal convolution
#
# The causal Mix-FFN keeps the previous block's last frame for its temporal
# convolution ([BCLA] "What SANA-Video Actually Uses"; [LongSANA], the pull
# request description: causal logic for the Mix-FFN, the conv in the MLP, and
# its block name CachedGLUMBConvTemp).  Reading: a depthwise (per-channel)
# convolution along the frame axis at every spatial position, y[t] = sum_i
# w[i] * x[t + i - 1] over the taps i < kt, with kt = 3 (frames t-1, t, t+1)
# or kt = 2 (frames t-1, t).  Inside a block the taps see the block's own
# frames; before the block's first frame they see the previous block's last
# frame (the cache; zeros before the first block), after its last frame zeros
# (the next block does not exist yet).  So, like the attention, it is
# bidirectional inside a block and causal across blocks, and one cached frame
# is all it needs.  An optional per-channel bias is added.  The 1x1
# projections and the gate around it are ordinary matrix products and are not
# part of this oracle.


def temporal_conv_block(x, w, cache=None, bias=None):
    """Temporal conv of one block: x (B, F, P, Ch) frames of P spatial positions,
    w (kt, Ch), cache (B, P, Ch) = the previous block's last frame (None: zeros).
    Returns y (B, F, P, Ch) float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kt = w.shape[0]
    if kt not in (2, 3):
        raise ValueError("kt must be 2 or 3")
    B, F, P, Ch = x.shape
    prev = np.zeros((B, 1, P, Ch)) if cache is None else np.asarray(cache, dtype=np.float64)[:, None]
    padded = np.concatenate([prev, x, np.zeros((B, 1, P, Ch))], axis=1)     # frames -1 .. F
    y = np.zeros_like(x)
    for i in range(kt):
        y += w[i] * padded[:, i:i + F]          # tap i reads frame t + i - 1
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)
    return y


def temporal_conv(x, w, tokens_per_frame, block_frames, bias=None, first_block_frames=None):
    """One-shot temporal conv over a whole sequence x (B, N, Ch) of frame-major
    tokens (N = frames * tokens_per_frame), block by block, each block reading
    the last frame of the one before.  Returns y (B, N, Ch) float64."""
    x = np.asarray(x, dtype=np.float64)
    B, N, Ch = x.shape
    frames = N // tokens_per_frame
    xf = x.reshape(B, frames, tokens_per_frame, Ch)
    y = np.empty_like(xf)
    cache = None
    for s, e in block_bounds(frames, block_frames, first_block_frames):
        y[:, s:e] = temporal_conv_block(xf[:, s:e], w, cache, bias)
        cache = xf[:, e - 1]
    return y.reshape(B, N, Ch)


class ConvCache:
    """The temporal conv's streaming cache: the last frame of the last committed
    block, (B, P, Ch), zeros at the start."""

    def __init__(self, B, P, Ch):
        self.last = np.zeros((B, P, Ch))
        self.frames_done = 0


def temporal_conv_stream_block(cache, x, w, tokens_per_frame, bias=None, save=True):
    """One streamed block x (B, F * P, Ch) against the cache; with save the cache
    becomes this block's last frame."""
    x = np.asarray(x, dtype=np.float64)
    B, n, Ch = x.shape
    F = n // tokens_per_frame
    xf = x.reshape(B, F, tokens_per_frame, Ch)
    y = temporal_conv_block(xf, w, cache.last, bias)
    if save:
        cache.last = xf[:, -1].copy()
        cache.frames_done += F
    return y.reshape(B, n, Ch)


# ------------------------------------------------------------- independent checks

def brute_force(q, k, v, tokens_per_frame, block_frames, rope=None, eps=EPS_DEFAULT,
                first_block_frames=None):
    """O(N^2) masked form, for tiny inputs.

    out_i = sum_j M_ij <rk_j, rq_i> v_j / (sum_j M_ij <fk_j, fq_i> + eps),
    M_ij = [block(j) <= block(i)].  Written token by token, with no prefix state;
    the block of a token comes from its frame index: frames below the first
    block's end are block 0, then one block per block_frames frames.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, d = q.shape
    f0 = block_frames if first_block_frames is None else first_block_frames
    frame = np.arange(N) // tokens_per_frame
    blk = np.where(frame < f0, 0, 1 + (frame - f0) // block_frames)
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            fq, fk = _relu(q[b, :, h]), _relu(k[b, :, h])
            rq = _rotate_tokens(fq, rope, tokens_per_frame, 0)
            rk = _rotate_tokens(fk, rope, tokens_per_frame, 0)
            for i in range(N):
                num = np.zeros(d)
                den = 0.0
                for j in range(N):
                    if blk[j] <= blk[i]:
                        num += float(np.dot(rk[j], rq[i])) * v[b, j, h]
                        den += float(np.dot(fk[j], fq[i]))
                out[b, i, h] = num / (den + eps)
    return out


def token_causal_cumsum(q, k, v, tokens_per_frame, rope=None, eps=EPS_DEFAULT):
    """Token-causal linear attention through running sums (np.cumsum over tokens).

    Equals the block form with blocks of one token; written without blocks.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            fq, fk = _relu(q[b, :, h]), _relu(k[b, :, h])
            rq = _rotate_tokens(fq, rope, tokens_per_frame, 0)
            rk = _rotate_tokens(fk, rope, tokens_per_frame, 0)
            outer = v[b, :, h][:, :, None] * rk[:, None, :]      # (N, d, d)
            Sc = np.cumsum(outer, axis=0)
            zc = np.cumsum(fk, axis=0)
            num = np.einsum("nef,nf->ne", Sc, rq)
            den = np.einsum("nf,nf->n", zc, fq) + eps
            out[b, :, h] = num / den[:, None]
    return out


def lite_la_single_block(q, k, v, tokens_per_frame, rope=None, eps=EPS_DEFAULT):
    """Non-causal ReLU linear attention over the whole sequence: the normalised
    readout of [ImplBCLA, "The Linear Attention Kernel"] with one block that
    holds every token, so every query reads the state formed by all keys:

        out_n = sum_m v_m <R phi(k_m), R phi(q_n)> / (<sum_m phi(k_m), phi(q_n)> + eps)

    (rotated vectors in the numerator, un-rotated ones in the normaliser).  A
    block spanning the whole sequence must give this.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            fq, fk = _relu(q[b, :, h]), _relu(k[b, :, h])
            rq = _rotate_tokens(fq, rope, tokens_per_frame, 0)
            rk = _rotate_tokens(fk, rope, tokens_per_frame, 0)
            num = np.einsum("me,mf,nf->ne", v[b, :, h], rk, rq, optimize=True)
            den = np.einsum("mf,nf->n", fk, fq, optimize=True) + eps
            out[b, :, h] = num / den[:, None]
    return out


def rel_err(got, ref):
    """max |got - ref| / RMS(ref) over the whole tensor (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / rms
