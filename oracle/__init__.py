"""CPU oracle for the Kimi K2 sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy implementation of what the layer computes, written from the source
pages ("Kimi K2 · Architecture", "Kimi-K2-Base", "Kimi K2 · Dense
transformer block").  It exists to check the HIP implementation: only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it.
It shares no code with the HIP path and never runs on the product path.

Precision policy: every sum is formed in float64 and rounded once to the
precision in which the layer stores that quantity (fp32 for sums, scores,
activations and outputs; bf16 for the normalised hidden state and the layer
output; e4m3 codes with fp32 scales for quantised activations).  Every
decision that turns floating point into an integer (top-k selection, an FP8
code) is taken on the fp32 value, as the layer takes it.

Parity pins: see tests/test_oracle_*.py.  The exact operation order of the
fp32 sums and of RMSNorm is not fixed by the pages; those parts are
"parity unpinned" beyond the invariants and closed forms the tests check.
"""
