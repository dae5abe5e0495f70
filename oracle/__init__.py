"""fp64 CPU oracle for hybrid-batch (chunked prefill + decode) attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The GPU library never routes
through it and shares no code with it: no kernels, headers, helpers, tables or
pre/post-processing.  The only thing both sides read is the seeded input bits
produced by ``prefill_decode_amd.inputs`` (which holds none of the method's
arithmetic).

Sources (web pages, cited by title and section):

* [POD] "POD-Attention: Unlocking Full Prefill-Decode Overlap for Faster LLM
  Inference" (ASPLOS 2025; bookshelf summary page).  Section "Why this problem
  is worth solving": for each query token attention forms a weighted
  combination of the keys and values of all earlier tokens, held in the
  KV-cache; prefill processes a prompt chunk, decode one new token that looks
  at the whole cache.  Section "The argument in one glance" / "Why it fell
  short": every token looks back at all prior tokens (causal).
* [POD] "How POD-Attention overlaps" > "Cap prefill splitting to avoid
  contention": attention may be split along the KV dimension
  (FlashDecoding-style); partial results are then combined.
* [PAT] "PAT: Accelerating LLM Decoding via Prefix-Aware Attention ..."
  (catalogue record, abstract): the split partials are merged by an online
  softmax (log-sum-exp) merge.

The pages never print the attention equation, so the oracle is the textbook
definition (scaled dot-product attention with a softmax over the visible keys),
written out plainly in float64 with no tiling, no online softmax and no
splitting.  The readings taken where the pages are silent are listed in the
module docstring of :mod:`oracle.attention`.

Pins (tests/test_oracle*.py, all ``-m "not gpu"``): brute force with
``math.fsum`` on tiny shapes, softmax rows summing to one, a single key
returning its value exactly, a decode row equal to the last prefill row,
split/merge invariance, the identical-keys closed form, a boundary probe,
GQA == MHA with repeated KV heads, ``torch`` float64 SDPA with an explicit
mask, page-table invariance, and the row-sampling entry point against brute
force and against the whole-batch oracle.  Planted-mistake tests check that
each plausible bug in the oracle is caught by at least one pin.  The pages
print no worked example with numbers, so ``tests/golden/`` holds only a
regression snapshot written from this oracle by ``make_golden.py``; it pins
nothing.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    fp8_e4m3_bits_to_f64,
    kv_head_of,
    visible_key_count,
    attention_rows,
    attention_partial,
    merge_partials,
    gather_request_kv,
    batch_attention,
    sample_batch_attention,
)
