"""CPU oracle for the RAM-Net layer recurrence.  TEST INFRASTRUCTURE ONLY.

A plain fp64 C implementation (ramnet_oracle.c) wrapped with ctypes;
projections.py (numpy fp64) for the dense steps either side of the layer;
backward.py (torch fp64 autograd through a token loop) for the gradients.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .oracle import (  # noqa: F401
    build, load, slot_weights, digit_probs, decode_one, decode_all, cape,
    layer, scan_given, round_bf16, max_threads, TOPK_BRUTE, TOPK_TREE,
)
