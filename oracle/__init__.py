"""CPU oracle for the CSA + HCA hybrid-attention path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 reference
of what the GPU library computes. Only the test suite, the smoke check and
the CPU-baseline leg of the benchmark may import it; the product path never
does. It shares no code with the HIP library: it imports nothing from
``long_context_attention_hca_amd`` and nothing there imports it.

Sources (the only description of the method): the hyper.ai paper page for
arXiv 2606.19348, "DeepSeek-V4", section 方法 (Method):

* the CSA paragraph: every m tokens of KV are compressed into one entry with
  learnable compression weights and a position bias; a "lightning indexer"
  picks the top-k compressed entries; core attention is MQA with shared keys
  and values;
* the HCA paragraph: every m' >> m tokens merge into one entry without
  overlap, with dense attention over all of them; both mechanisms add a
  sliding-window attention branch;
* the efficiency paragraph: BF16 for the RoPE dimensions, FP8 for the rest,
  FP4 for the lightning indexer.

The DeepSeek-V4-Pro model card mirror (hugingapi.com, "Tensor type" list)
names F8_E4M3, F8_E8M0 and I8 tensors, which supports reading FP8 as OCP
E4M3 and FP4 as MX E2M1 with E8M0 block scales.

Readings of points the pages leave open are stated in each module.

Pins: every function here is checked by the CPU test suite against closed
forms, special cases that reduce to library routines, invariants and brute
force (tests/test_oracle_*.py). The whole-workload compositions of
pipeline.py are pinned by rebuilding queries from whole raw sequences
(tests/test_oracle_pipeline.py): with k >= n_vis they equal textbook
attention over the explicitly listed rows, a chunk's entries equal those of
the whole sequence, and with one entry per token and no window they reduce
to causal MQA through torch's scaled_dot_product_attention. The golden
fixture under tests/golden is a regression record written by this oracle,
not a pin.
"""

from . import codecs, compress, indexer, attention  # noqa: F401
