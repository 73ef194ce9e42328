"""fp64 CPU oracle of the activation-sparse FFN (PowerInfer's neuron-aware FFN).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
restatement of what the sparse FFN computes. The only code that may import
it is the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``. The HIP path never calls it and shares no code with it.
The seeded input generator in ``synth`` is the only thing both sides use.

Every function works in float64 with numpy. Each one names the passage of the
pages it restates. The pages are:

* P1: "Tüketici sınıfı GPU takılı PC'lerde yüksek hızlı büyük dil modeli
  serving" (GeekNews summary of the PowerInfer README)
* P2: "PowerInfer: Fast Large Language Model Serving with a Consumer-grade
  GPU" (КПД Telegram post)
* P3: "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen" (unite.ai)

Where a step is not fixed by the pages, the module docstring of
:mod:`oracle.ffn` states the reading taken.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_synth_calibration.py`` and ``tests/test_stack_chain.py``: hand-worked
fixtures under ``tests/golden`` (``band`` by ``band.json``: exactly 1e-4 away is
outside, 5e-5 off a nonzero theta inside, inf and NaN outside; ``stack_forward`` and
``glue`` by ``stack_two_layers.json``: two layers, two tokens, the chaining vector,
the all-zero pass-through and a predictor miss), the textbook dense FFN, brute-force
loops, closed forms and invariants. None is "parity unpinned".
"""
from .ffn import (  # noqa: F401
    THRESHOLD_BAND,
    band,
    compact,
    decision_values,
    dequant_q4_0,
    glue,
    hot_first_order,
    layer_forward,
    mask_words,
    per_token_ffn,
    permute_layer,
    predictor_logits,
    rows_f64,
    sparse_ffn,
    stack_forward,
    threshold,
    true_preactivation,
    union,
    words_to_mask,
)
