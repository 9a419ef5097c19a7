"""CPU oracle for DiT dense joint text+image attention (TEST INFRASTRUCTURE).

Plain, slow, obviously correct float64 code. Only the test suite, the smoke
check of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library and its Python binding never do, and this package
imports nothing from them. It shares no code with the GPU path: its inputs
come from the separate ``workloads`` module, which holds no attention
arithmetic.

Pins (what each function is checked against, in tests/test_oracle*.py):
* ``attention``: literal brute force with correctly rounded sums on tiny
  shapes; torch's float64 CPU scaled-dot-product attention; closed forms
  (N = 1, N = 2 logistic, constant V, identical keys, scale -> 0, dominating
  key); invariants (rows of p sum to 1, joint K/V permutation, query
  permutation, key shift). Planted mistakes are shown to fail these pins.
* ``formats``: all 256 e4m3 codes against torch.float8_e4m3fn; e4m3 and
  bf16 rounding against torch's casts; OCP special values (golden file).
* ``quantize_per_tensor``: absmax code is 448, scale round trip, torch cast.
* ``attention_fp8_pipeline``: with P unrounded it equals ``attention`` on the
  dequantised inputs; the P rounding error obeys the e4m3 bound; closed forms
  with identical keys and N = 1; with the rounded denominator a constant V is
  returned exactly and rows differ from the default by one bounded factor.
* ``attention_blocksparse``: torch's float64 CPU scaled-dot-product attention
  with the boolean key mask (a library routine); full lists give
  ``attention``; one listed block of one valid key gives that key's V row
  and logit; the merge identity over two disjoint lists; permuted and
  repeated list entries change nothing; empty lists give 0 / -inf.
* ``mx_quantize``: torch's float8_e4m3fn cast of each value divided by its
  block's power of two; the block maximum's code in the top binade; the
  half-step error bound; power-of-two invariance; exact blocks; zero blocks;
  the token-blocked scale layout on columns of known magnitude.
* ``attention_mx_pipeline``: with P unrounded it equals ``attention`` on the
  dequantised inputs; with every scale 2^0 it equals
  ``attention_fp8_pipeline`` with unit descales; doubling every V scale
  doubles O; moving 2^k from ``scale`` into every Q scale changes nothing.
"""
from .attention import attention, attention_bruteforce, softmax_probabilities
from .formats import (E4M3_MAX, bf16_round, e4m3_decode, e4m3_encode,
                      quantize_per_tensor)
from .blocksparse import attention_blocksparse, key_set
from .fp8_attention import P_SCALE, attention_fp8_pipeline
from .mx import attention_mx_pipeline, mx_dequantize, mx_quantize, shared_exponent

__all__ = [
    "attention", "attention_bruteforce", "softmax_probabilities",
    "E4M3_MAX", "bf16_round", "e4m3_decode", "e4m3_encode", "quantize_per_tensor",
    "P_SCALE", "attention_fp8_pipeline", "attention_blocksparse", "key_set",
    "attention_mx_pipeline", "mx_dequantize", "mx_quantize", "shared_exponent",
]
