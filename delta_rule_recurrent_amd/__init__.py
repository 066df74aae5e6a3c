"""MI355X-native gated delta-rule recurrent state update.

Entry points over the gdnrt HIP library (C ABI in include/gdnrt.h):
``gdn_decode_step``, ``gla_chunk_fwd``, ``gla_chunk_bwd``, ``gdn_chunk_fwd``, ``gdn_chunk_bwd``,
``leapq_decode_step``,
``leapq_window_flush``, ``kda_decode_step``, ``kda_chunk_fwd``,
``kda_leapq_decode_step``, ``kda_leapq_window_flush``, the window-closing
``leapq_decode_flush`` and ``kda_leapq_decode_flush``, and the per-device calls of ZeCO's
sequence-parallel GLA forward: ``gla_shard_local`` (``gla_chunk_fwd`` from zero and
``gla_shard_decay``), ``gla_all_scan_step`` and ``gla_shard_output_correct``, and its
backward's phase 1, ``gla_shard_bwd_state`` (then ``gla_shard_bwd_grads``). ``synth``
draws the seeded synthetic workloads.
"""
from .binding import (  # noqa: F401
    GdnrtError,
    LeapqBuffers,
    code_row_bytes,
    gdn_chunk_bwd,
    gdn_chunk_bwd_workspace,
    gdn_chunk_fwd,
    gdn_chunk_fwd_noalloc,
    gdn_chunk_workspace,
    gdn_decode_step,
    gdn_decode_step_bf16_state,
    gdn_decode_step_int_state,
    gla_chunk_bwd,
    gla_chunk_bwd_workspace,
    gla_chunk_fwd,
    gla_chunk_workspace,
    gla_all_scan_step,
    gla_shard_bwd_grads,
    gla_shard_bwd_state,
    gla_shard_decay,
    gla_shard_local,
    gla_shard_output_correct,
    hbm_stream,
    kda_chunk_fwd,
    kda_chunk_workspace,
    kda_decode_step,
    kda_leapq_decode_flush,
    kda_leapq_decode_step,
    kda_leapq_window_flush,
    leapq_decode_flush,
    leapq_decode_step,
    leapq_window_flush,
    lib,
)
