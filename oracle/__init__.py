"""Plain, slow CPU oracle for the QLoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import or call anything in this package.  The
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product path.

Modules:
  nf4     -- NF4 codebook, blockwise absmax quantization, double quantization,
             double dequantization (bit-exact definitions).
  linear  -- forward and backward of the QLoRA linear in float64.

Every function cites the passage it follows by page title and section.
The page titles used in citations:
  [Explainer]  "QLoRA: Efficient Finetuning of Quantized LLMs" (intuitivepapers.ai)
  [Review]     "QLoRA Review: 4-Bit Finetuning for 65B Models on One GPU" (tildalice.io)
  [Addaly]     "QLoRA: quantising the part you are not training" (addaly.com)
  [Glossary]   "4-bit QLoRA" (inferensys.com glossary)
"""
from . import nf4, linear  # noqa: F401
