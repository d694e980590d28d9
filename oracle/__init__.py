"""Plain, slow, fp64 CPU oracle for exact attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The GPU library never routes through it, and it shares no code
with the HIP path: no kernels, headers, helpers, tables or pre/post-processing.

Contents
--------
exact          -- the plain definition: S = scale*Q K^T materialised per head,
                  masked, stable softmax, P V and the natural-log LSE.
online         -- the online-softmax recurrence over key blocks (running max m,
                  running sum l, rescaled output), used only to pin that the
                  blockwise algorithm reproduces the plain definition.
e4m3           -- decoding of OCP FP8 E4M3FN codes to exact float64 values.
keyrange       -- attention over one range of the keys (causal alignment of the
                  whole problem) and the log-sum-exp merge of such partial
                  results (split-KV, chunked prefill).
quant          -- the fp8 input pipeline: signed Hadamard rotation of Q and K,
                  e4m3 encoding (nearest, ties to even, saturating) and
                  quantisation with one descale per 64-row block.
backward       -- gradients dQ, dK, dV: the chain rule through the forward
                  definition, P materialised per head.
fp8p           -- attention with e4m3 probabilities, one power-of-two scale
                  per 64-key block of each row, exact or Lean P codes.
polyexp        -- the cubic base-2 exponential of the polynomial-exp variant.

Every function cites the passage of the source pages it follows, by page title
and section.  No function here is "parity unpinned": each one is pinned by a
test in ``tests/test_oracle_pins.py`` (closed forms, invariants, brute force,
a library cross-check and a hand-worked example under ``tests/golden/``).
"""
from .exact import attention, attention_head, kv_head_of, visible_mask
from .online import online_attention_head
from .e4m3 import e4m3fn_decode, E4M3FN_MAX
from .keyrange import attention_range, attention_range_head, key_range_mask, merge
from .quant import dequantize_blocks, e4m3fn_encode, hadamard, quantize_blocks, rotation
from .backward import attention_backward, attention_backward_head, probabilities_head, row_delta
from .fp8p import fp8p_attention, fp8p_attention_head, fp8p_attention_head_f32
from .polyexp import poly_exp2

__all__ = [
    "attention",
    "attention_head",
    "kv_head_of",
    "visible_mask",
    "online_attention_head",
    "e4m3fn_decode",
    "E4M3FN_MAX",
    "attention_range",
    "attention_range_head",
    "key_range_mask",
    "merge",
    "e4m3fn_encode",
    "hadamard",
    "rotation",
    "quantize_blocks",
    "dequantize_blocks",
    "attention_backward",
    "attention_backward_head",
    "probabilities_head",
    "row_delta",
    "fp8p_attention",
    "fp8p_attention_head",
    "fp8p_attention_head_f32",
    "poly_exp2",
]
