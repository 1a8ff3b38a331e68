"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Nothing here performs any step of the packed-attention method: no prefix sums,
segment ids, positions, labels, rotations or attention.  The module only draws
random numbers and lays them out as sample lengths, pad flags, token ids and
bf16 q/k/v buffers.
"""

from .generators import (  # noqa: F401
    CONFIG_NAMES,
    EOS_ID,
    PAD_ID,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    logits_bits,
    make_prefill,
    prefill_bits,
    Prefill,
    make_workload,
    qkv_bits,
    token_ids,
)
