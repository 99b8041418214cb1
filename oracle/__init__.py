"""fp64 CPU oracle and brute-force replay of the H2O KV-cache path.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package. The product path never does.
"""
from .h2o_oracle import (H2OOracle, PrefillResult, StepResult, causal_attention_probs,
                         choose_victim, eligible_slots, prefill_column_sums, select_prefill)
from .brute import brute_run

__all__ = ["H2OOracle", "PrefillResult", "StepResult", "causal_attention_probs",
           "choose_victim", "eligible_slots", "prefill_column_sums", "select_prefill",
           "brute_run"]
