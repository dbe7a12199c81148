"""fp64 CPU oracle for replay-free block verification of a hybrid conv/IIR/attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the ``smoke()`` check of the entry
module and the CPU-baseline leg of the benchmark use it.  It shares no code
with the HIP library or its Python binding.

What it computes follows the EvSpark digest ("EvSpark: Lossless Speculative
Decoding for Hybrid DNA Foundation Models"): one initial-state block forward
over the anchor and gamma drafts (Interpretation), lossless acceptance with a
sampled correction as the next anchor (Figure 1(c)), and slicing of the three
state classes -- FIR windows, modal IIR state, KV cache -- to the accepted
index without replay (Figure 1(d)).  The acceptance rules follow the ReaDy
summary (section 3.1 for greedy verification, section D.2 for the
speculative-sampling rule).

Everything is plain numpy in float64.  bf16 inputs arrive as uint16 bit
patterns and are widened exactly.

Pinning (see tests/test_oracle_*.py):
  * FIR: brute-force full convolution from zero state, delta taps.
  * IIR: closed form y = h * g with the materialised impulse response,
    lfilter for one pole, lambda = 0 and beta = 0 special cases.
  * attention: explicit full softmax matrix per query and torch's
    scaled_dot_product_attention in fp64, plus invariants.
  * greedy / rejection acceptance: brute force for forced k, the exact
    first-token distribution identity, a Monte-Carlo chi-square test.
  * slicing: the Figure 1(d) worked example; block+slice equals sequential steps.
  * prefill: equals the prompt's sequential single-position steps; the long
    FIR equals the plain FIR; the IIR scan equals the state-keeping scan.
  * linear / rmsnorm: a pure-Python triple loop on small shapes, permutation
    and identity weights; RMS of the output = 1 with unit gains, scale
    invariance of the input.
  * model stack: block forward + slice at k equals k+1 one-row steps for
    every k (rounding off, fp64), each sublayer equals the pinned single-layer
    pieces; bf16 rounding equals torch's conversion on fp32-exact values.
  * drafter: the sampled draft's law equals softmax((z + B[prev]) / T)
    exactly, for the first draft and for the second given the first (decision
    boundaries by bisection); the trunk is causal in the block rows and sees
    every window row; its pieces are the pinned ones.  Architecture reading:
    parity unpinned beyond these.
  * multi-candidate selection (largest accepted count, lowest index on ties):
    parity unpinned -- the pages give no rule for choosing among candidates.
  * recursive multi-candidate acceptance: reduces to the one-candidate rule;
    exact first-token distribution = target over every draft combination
    (decision boundaries found by bisection); Monte-Carlo joint law of the
    first two emitted tokens under a toy prefix-keyed target and drafter.
  * token trees: every node's forward equals the chain forward over its
    root-to-node path (chains, stars, random trees, trees deeper than the
    outer window); the tree mask; greedy and sampling acceptance reduce to the
    one-block rules on a chain, greedy matches a brute-force search on random
    trees, the first emitted token is exactly target-distributed over every
    combination of children tokens (each child with its own draft
    distribution), a Monte-Carlo joint law of two emitted tokens on depth-2
    trees; tree forward + slice along the accepted path equals sequential
    steps over the path.
"""
from .layer import (depthwise_fir, modal_iir, block_attention, verify_block,
                    as_f64, Layer, SeqState)
from .acceptance import greedy_accept, rejection_accept, recursive_accept, accept_candidates
from .slicing import slice_state, sequential_steps
from .prefill import depthwise_fir_long, iir_scan, prefill_state
from .linear import linear, rmsnorm
from . import model
from . import drafter
from . import tree

__all__ = [
    "depthwise_fir", "modal_iir", "block_attention", "verify_block", "as_f64",
    "Layer", "SeqState", "greedy_accept", "rejection_accept", "recursive_accept", "accept_candidates",
    "slice_state", "sequential_steps", "depthwise_fir_long", "iir_scan", "prefill_state", "linear", "rmsnorm",
]
