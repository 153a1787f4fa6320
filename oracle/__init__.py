"""fp64 CPU oracle for the ternary-expert MoE block.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of the package entry file and the CPU-baseline
leg of the benchmark may import this package.  The product path (the C-ABI
library and its Python binding) never imports, links or calls it, and this
package shares no code with it: the oracle has its own container codec, its own
routing and its own expert evaluation, written from the release pages:

  * containers: Scion-35B-A3B card, "Weight Representation: ternary PQ2_0 +
    trained corrections" and "About the Hub's quant chip" (PQ2_0: 2-bit codes,
    one fp16 scale per 128 weights, 2.125 bpw); Scion-FlashNext-176B-A6B card,
    "Highlights" and "Weight Representation: ternary PTQ1_0 + trained
    corrections + Q4_0 PLE" (PTQ1_0: 24 bytes of 5-trit data, 2 bytes of
    remaining trits, 2-byte scale = 28 bytes per 128 weights);
  * router + router delta, rank-r residual correction on the MoE block output:
    Scion project README, "The idea"; Scion-35B-A3B card, "Weight
    Representation"; "What the experiments established" (placement rule);
  * top-k routing with an always-on shared expert: FlashNext card "Model
    Overview" (top-10 routed + 1 shared); 35B-A3B card "Model Overview";
  * per-expert grouping of tokens (mul_mat_id): Scion README "Serving notes";
  * the ternary quantizers (absmean, Lloyd over groups of 128): project README,
    "What the experiments established" (quant.py);
  * the Q4_0 per-row n-gram table decode: FlashNext card, "Model Overview" and
    "Weight Representation" (ple.py);
  * the k=1 draft head (fc1, gelu, fc2): 35B-A3B card, "Shipped Components"
    (mtp.py).

Where the pages are silent the readings are those listed in the package's design
notes (two's-complement 2-bit codes, little-endian base-3 digits, SwiGLU,
softmax over the selected k, ties to the lower expert index, correction input =
block input).  Everything is evaluated in float64 from the exact bits the GPU
receives.
"""
from . import codec, moe, mtp, ple, quant  # noqa: F401
