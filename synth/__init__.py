"""Seeded synthetic inputs for the MARS hot path.

This module draws the random inputs (Q/K/V, paged KV caches, hidden states,
LM-head weights, logits, thresholds) that both the CPU oracle's checks and the
HIP path consume. It holds none of the method's arithmetic: no masking, no
softmax, no acceptance rule, no cache commit. It only draws numbers, rounds
them to the storage precision and lays them out.

The workloads are synthetic stand-ins shaped like the Qwen2.5-0.5B / 7B models
that "MARS: Enabling Autoregressive Models Multi-Token Generation" evaluates
(gist.science explainer, section 4 Experimental Results; papernotes.org notes,
主实验 table); no model weights, tokenizer or benchmark item is used.
"""

from .generators import (  # noqa: F401
    bf16_round,
    bf16_bits_to_f32,
    two_stream_qkv,
    sequence_qkv,
    decode_inputs,
    layered_commit_inputs,
    LayeredCommitInputs,
    lmhead_inputs,
    normal_logits,
    PeakedLogitsPool,
    tau_schedule,
    decode_step_tensors,
    sample_pairs,
    Tensor,
    DecodeInputs,
)
