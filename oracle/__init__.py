"""CPU oracle for LLVQ (Leech-lattice vector quantization) decode and dequant-GEMV.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The HIP library never calls it, and this package never
imports the HIP library or its binding: the two share no code, tables or helpers.
The only thing both sides consume is the seeded input generator
(``weight_decompression_amd/synth.py``), which holds none of the method's arithmetic.

It is deliberately plain and slow: pure Python integers for every exact step, numpy
only for bulk float work, fp64 for every floating-point result.

Sources (the paper "Leech Lattice Vector Quantization for Efficient LLM Compression",
arXiv 2603.11021, as summarised on five web pages):

* papernotes.org page ("Leech Lattice Vector Quantization for Efficient LLM
  Compression", NeurIPS 2026 notes), section 方法详解: 整体框架 (24-dim blocking,
  shape-gain), 关键设计 1 (shell union from squared norm 4 up to 2M, angular search),
  关键设计 2 (shell -> class -> Golay / sign / permutation index and its div/mod
  inverse), 关键设计 4 (fused dequantization kernel).
* gist.science page (German summary), section "Methodik": 1. Struktur des
  Leech-Gitters (Golay construction, even/odd cosets, shells of norm 2m),
  2. Multi-Shell Search (Euclidean vs. angular modes), 3. Indexierungsschema,
  4. Dequantisierungskernel.
* gptget.net page, section 原文摘要 (the English abstract: indexing to and from
  bitstrings without materialising the codebook).

Every convention the pages leave open (Golay generator, coordinate order, class
order, sign-bit order, permutation order inside even classes, bit packing, bf16
rounding) is stated in the docstring of the module that implements it.

Module map:
  golay.py      extended binary Golay code, sorted codeword table T
  leech.py      integer-coordinate membership, shell sizes (closed form and DP)
  classes.py    class table per shell (leader multiset + parity)
  bijection.py  unrank (index -> point) and rank (point -> index)
  search.py     exact angular / Euclidean search over the shell union
  reference.py  bitstream reader, fp64 GEMV, bf16 decode emulation, tolerances
  cpu_baseline.py  timed oracle decode + GEMV used as the reported CPU baseline
"""


