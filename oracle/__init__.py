"""CPU oracle for the DFlash-style lossless speculative-decoding step.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The GPU path never does: it shares no code, header, helper or table with
this package, and this package imports nothing from the GPU package.

What it computes (all in float64 unless a step is documented as float32):

* ``ops``       RMSNorm, rotate-half RoPE, SiLU, masked multi-head attention
                with grouped KV heads, row-wise linear maps.
* ``model``     a Qwen3-like pre-norm decoder with a position-indexed KV cache
                (the target), and the block-diffusion drafter whose every
                layer's KV cache receives projected target hidden states
                (KV injection).
* ``sampling``  Philox4x64-10, the temperature / top-k / top-p candidate
                distribution (float32, sequential sums), and the
                accept / resample rule for deterministic drafts.
* ``spec``      the draft -> verify -> accept loop, the plain autoregressive
                loop, and exact enumeration of both output laws.

Pins (tests/test_oracle_*.py) tie each part to something other than itself;
see the per-module headers.  Parity unpinned: the drafter's wiring (which
target layers feed it, where the fc projection and norms sit) has no printed
reference implementation or worked example; it cannot affect the output
law, only how many drafts are accepted.
"""
