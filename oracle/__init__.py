"""Plain, slow CPU oracle for the simulated-quantization hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``fp4_fake_quant_amd``
package, its HIP kernels or its C-ABI library) imports, calls, links or executes
anything in this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP path.

What it computes follows the QATFactory project page ("Method" section and the
"Supported formats" table): weights (and optionally activations) are rounded
onto a 4-bit format's grid and dequantized back to BF16 (QDQ) in the forward
pass, gradients pass straight through (STE) in the backward pass, LoRA adapters
are merged into the frozen base before quantization, one MoE expert at a time,
and the codes and scales are packed into an engine-style layout.  The table
fixes the formats only at the level of element type, block size, scale types,
symmetry and bits per weight; every bit-level rule below it is a stated reading
(see each module's docstring).

Numerics: every step is a sequence of IEEE-754 binary32 operations with
round-to-nearest-even, done with numpy float32 arrays (numpy never contracts a
multiply and an add), plus exact integer and bit operations.  Reference GEMMs
and adapter gradients are computed in float64.

Modules
-------
primitives  number formats: bf16, fp16, E4M3, E8M0, E2M1 encode/decode
nvfp4       tensor scale (tied groups), block-16 QDQ, pack/unpack
mxfp4       block-32 QDQ with a shared power-of-two scale, pack/unpack
q4k         256-element super-blocks of eight 32-element sub-blocks, pack/unpack
ste         straight-through estimator backward
lora        LoRA merge (W + B.A) and adapter gradients (float64)
gemm        float64 reference for Y = QDQ(X) . QDQ(W)^T and its error bound

Parity status of each function is listed in the module docstrings.  Functions
with no independent pin say "parity unpinned".
"""

from . import primitives, nvfp4, mxfp4, q4k, ste, lora, gemm  # noqa: F401
