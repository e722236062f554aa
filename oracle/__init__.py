"""CPU oracle for the DFlash 2 draft-path selector.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy (fp64) statement of what the selector
computes, used to check the HIP library.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does,
and this package shares no code with the HIP library.

Source: the blog post "DFlash 2: Keep Drafting Parallel" (Inco AI, 2026) and
its translations; see each function for the passage it follows.

Pinning status (what each function is checked against, in tests/):
  top16          full stable sort == heapq.nlargest; sorted rows; ties; -inf; +-0
  gate           W_h = 0 -> 0.5; one-hot h; scipy.special.expit(h @ W); odd symmetry
  pair_scores    scalar triple loop with math.fsum; zero bilinear -> U; closed forms
  walk (greedy)  zero bilinear -> per-position top-1; planted chain; lexicographic
                 brute force over all 16^L paths for L <= 4
  walk (gumbel)  Gumbel-max frequencies vs softmax (chi-square); T -> 0 == greedy
  viterbi        brute force (math.fsum) over all 16^L paths for L <= 4; zero
                 bilinear -> per-position top-1; a planted path greedy misses;
                 per-position shifts change nothing; all-equal scores -> slot 0
  philox4x32_10  rocRAND's header-only Philox4x32-10 compiled for the host
  recall         hand-counted blocks (recall@k, accepted lengths, oracle selector)
  verify         the speculative-sampling theorem (emitted tokens follow the target,
                 chi-square), acceptance rate = sum min(p, q), q = p -> all accepted,
                 target mass off the candidates -> rejected at once, inverse CDF by
                 definition, draft_probs = scipy softmax
  conv2          static kernel == numpy.convolve along the block; identity and shift
                 kernels exact; a planted one-weight case fixes taps, groups and
                 predecessors; one group's weights move exactly its 16 channels by
                 a closed form; x_prev reaches position 0 only; scalar fsum loops
  lmhead         one-hot hidden states select a weight column (closed form); scalar
                 fsum dot products; top-16 == heapq.nlargest of the brute-force logits
"""
from . import conv, lmhead, recall, verify
from .philox import gumbel, philox4x32_10, uniform_from_word
from .selector import (
    SequenceResult,
    gate,
    pair_scores,
    select,
    select_sequence,
    top16,
    top16_rows,
    viterbi,
    walk,
    widen,
)

__all__ = [
    "SequenceResult",
    "conv",
    "gate",
    "gumbel",
    "lmhead",
    "pair_scores",
    "philox4x32_10",
    "recall",
    "verify",
    "select",
    "select_sequence",
    "top16",
    "top16_rows",
    "uniform_from_word",
    "viterbi",
    "walk",
    "widen",
]
