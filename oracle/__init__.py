"""CPU oracle for the MXFP8 Mixture-of-Experts expert path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is plain NumPy (fp64 for real arithmetic, integers for codes) and
shares no code with the HIP library.  Sources it follows:

* "1.5x faster MoE training on Blackwell with MXFP8 kernels built from
  scratch" (engineering.fyi digest), sections "Key Questions Answered" and
  "Technologies & Tools": MXFP8 microscaling, i.e. a scale per fine-grained
  sub-block of a tensor.
* pytorch/ao PR #3203 "[mxfp8 moe training] bench and profile mxfp8 a2a fwd
  and bwd separately", stacked-PR list and "Next steps": separate MXFP8
  quantize / dequantize kernels, an e8m0 -> fp32 scale decode, a token
  shuffle that stays in MXFP8, and a scaled grouped GEMM that accepts
  pre-quantized (data, scale) pairs.
* NVIDIA/TransformerEngine issue #556, first maintainer reply: an fp8
  all-to-all is pure byte movement as long as the scales travel with the
  bytes (the permute copies codes and scales together).

The pages do not define the MX encoding numerically.  The numeric rules used
here are the OCP Microscaling v1.0 rules as restated in the build target:
32-element blocks, E4M3 elements, one E8M0 power-of-two scale per block with
exponent floor(log2(amax)) - 8 clamped to the E8M0 range, and a
round-to-nearest-even, saturating E4M3 cast.  Every reading taken where the
text is silent is listed in the design notes and in the docstring of the
function that takes it.
"""

from . import mxfp8  # noqa: F401
