"""CPU oracle for dynamic block-sparse attention selected from block means.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously-correct
definition that the HIP path is checked against. Only the test suite, the
package-level smoke check and the benchmark's CPU-baseline leg may import it;
the library itself never calls it and has no CPU fallback.

The method (the pages describe it only in prose; no formula, code or listing):

* page "600倍加速，720p视频实时生成！单卡也能带的动14B模型" (66bd.net news article),
  section on the single-card path, paragraph on dynamic sparse quantized
  attention: importance of attention is estimated from block-level means of
  Query and Key, the important blocks are chosen at run time, only the activated
  tiles are computed, and they are computed densely; typical sparsity 80-90 %,
  i.e. 10-20 % of blocks kept;
* same page, paragraph on efficient inference operators: the long-sequence
  self-attention judges block relevance from the current Q/K, keeps about 10 %
  of the blocks, and computes with Q/K in INT8 and V in FP8;
* page "Run Wan2.2-A14B on One RTX 5090: 720p Video in 3.8s", section
  "3. Dynamic sparse attention": block importance from Q/K block-level means,
  top 10-20 % of blocks kept, dense computation inside the kept blocks.

Everything the pages leave open (token order, block sizes, score function,
selection count and ties, quantizer granularity and rounding, the FP8 format,
the softmax state) is a reading, listed in the design notes and restated at
each function below.

Parity unpinned: the pages print no worked example and no output of their own
kernel, so no function here is pinned to the pages' implementation; each is
pinned to its definition (closed forms, library routines, brute force,
invariants) by the tests.
"""
from .blocksparse import (  # noqa: F401
    LOG2E,
    attend_exact,
    attend_masked_dense,
    attend_quantized,
    block_bounds,
    block_scores,
    bf16_rne,
    dequantize_blocks,
    e4m3_bits,
    e4m3_decode,
    e4m3_rne,
    fp8_block_exponent,
    n_keep,
    plan,
    pool_block_means,
    quantize_fp8_blocks,
    quantize_int8_blocks,
    quantized_error_bound,
    select_top_blocks,
)

from . import ulysses  # noqa: E402  (Light-Ulysses FP8 packing)
from . import prologue  # noqa: E402,F401
from . import nvfp4  # noqa: E402,F401
