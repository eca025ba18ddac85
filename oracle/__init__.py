"""CPU oracle of the tiered KV-cache decode path (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .ref import (T0, T1, T2, T3, Policy, TieredSequence, assign_tiers, attention,
                  budgets, dequantize_rows, gather_rows, keep_order,
                  protected_mask, quantize_rows, score_increment, widen)

__all__ = ["T0", "T1", "T2", "T3", "Policy", "TieredSequence", "assign_tiers", "attention",
           "budgets", "dequantize_rows", "gather_rows", "keep_order",
           "protected_mask", "quantize_rows", "score_increment", "widen"]
