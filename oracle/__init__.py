"""Plain CPU oracle for one layer of compressed sparse attention decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The library
under ``compressed_sparse_long_c4a_amd`` never calls it and shares no code
with it: the two are written independently from the same pages.

Everything here is numpy in float64, written for readability rather than
speed.  Each function names the passage of the pages it follows:

* "DeepSeek V4 in vLLM: Efficient Long-context Attention" (digest of the
  vLLM blog post), cited as [vLLM-V4] with its section headings: design
  principles (section 2), keeping the KV cache packed (section 3, part 1),
  keeping the GPU busy (section 3, part 2), and the appendix (why inverse
  RoPE; exact position ranges and causality; exact k values; why the short
  window; the 8.7x memory arithmetic).
* "SGLang KV Cache storage pool architecture" notes, cited as
  [SGLang-pools] with section numbers (section 3: the MLA row; section 4:
  the DSA indexer row).
* A second digest of the vLLM post, cited as [V4-digest-2].

Where the pages leave a step open the oracle takes one plain reading, and
the docstring of the function that takes it says which.  Readings that
nothing on the pages can arbitrate are marked "parity unpinned":

* ``rope.rope``: rotated dimensions are the last ``rope_dims`` of a row,
  rotated in consecutive pairs (2i, 2i+1).
* ``compress.rms_norm``: epsilon and the span (the whole row).
* the indexer key's RoPE span (the last 64 of its 128 dimensions).
* the softmax scale, which is a caller input.
"""

from . import formats, rope, geometry, paged, compress, indexer, attention, sizes  # noqa: F401
