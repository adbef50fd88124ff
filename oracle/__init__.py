"""fp64 CPU oracle (test infrastructure only; see la_oracle's header)."""
from .la_oracle import *  # noqa: F401,F403
from .la_oracle import (EPS_DEFAULT, NORM_EPS_DEFAULT, StreamState, backward, backward_head, block_bounds,
                        block_states, brute_force, forward_qkv, qk_rms_norm, split_qkv,
                        stream_block_qkv, ConvCache, temporal_conv, temporal_conv_block,
                        temporal_conv_stream_block,
                        forward, forward_head, lite_la_single_block, readout_tokens, rel_err,
                        rope_rotate, stream_block, token_causal_cumsum, token_positions)
