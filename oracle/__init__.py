"""CPU oracle for FlashSampling (fused LM-head matmul + exact Gumbel-max sampling).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
fp64 implementation of what the sampler computes. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the HIP library and its Python binding) never does, and this package
imports nothing from the product.

What it computes (FlashSampling, arXiv 2603.15854, Section 3 "method"):
the logits are l = H W^T; the sample for a row is the Gumbel-max
argmax_v (l_v / T + g_v) over the whole vocabulary, with i.i.d. Gumbel noise
g. The fused kernel reaches exactly this maximiser because argmax decomposes
over any partition of the vocabulary into tiles (exactness paragraph of the
same section). The noise g is a pure function of (seed, step, row, vocab
index) built from Philox4x32-10 (Salmon et al., SC'11).

Modules:
  philox   Philox4x32-10 keyed and countered per vocab element.
  gumbel   word -> uniform on the open unit interval -> Gumbel, in fp64.
  sampler  exact logits, perturbed scores, the direct sample and its top-2
           margin, and the two-stage tiled form used to pin the partition
           argument.
  grouped  the grouped (hierarchical) variant: per vocabulary group a local
           sample and a local log-mass, then a Gumbel-max draw of the group
           from its own noise stream.

Every function is pinned by a CPU test against something other than itself
(rocRAND's Philox for the words, closed forms of the Gumbel law, exact
rational dot products, chi-square against softmax, the T -> 0 limit,
brute-force argmax over random partitions, and for the grouped variant its
two index-exact reductions, scipy's logsumexp and chi-square).
"""
from .philox import philox4x32_10, philox_words, philox4x32_10_scalar  # noqa: F401
from .gumbel import word_to_uniform, uniform_to_gumbel, gumbel_from_words  # noqa: F401
from .sampler import (  # noqa: F401
    SampleResult,
    exact_logits,
    gumbel_noise,
    perturbed_scores,
    argmax_lowest,
    sample,
    sample_two_stage,
)
from .grouped import (  # noqa: F401
    GroupedResult,
    group_noise,
    group_philox_words,
    log_mass,
    sample_grouped,
)
