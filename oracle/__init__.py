"""CPU oracle for the block-scaled quantization hot path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
NumPy restatement of what the quantization pipeline and the expert GEMMs
compute, written from the text of "End-to-End 4-Bit Training" (Thinking
Machines Lab). It exists to check the HIP library. Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library itself never calls it and has no CPU fallback.

It shares no code with the HIP path: no kernels, headers, tables, constant
generators or pre/post-processing. Seeded inputs come from ``synth``, which
holds no arithmetic of the method.

Modules
-------
formats  E2M1 / E4M3 / E8M0 codecs (section "Low-precision formats on Blackwell").
rng      Philox4x32-10 counter-based generator (Salmon et al., SC'11) and the
         16-bit uniform draw used by stochastic rounding.
quant    NVFP4 round-to-nearest quantize, dequantize, MXFP8 quantize (RN/SR),
         dequantize-transpose-SR-requantize (sections "Block-scaled backward
         passes" and "Re-quantization with stochastic rounding").
gemm     fp64 references of the NVFP4 grouped GEMM and the MXFP8 DGRAD/WGRAD.
route    top-k routing -> per-expert token segments ("Quantized communications").

Parity status: every function here is pinned by a CPU test under tests/
(worked examples of the pages, closed forms, brute force on tiny inputs,
known-answer vectors, statistical tests). The only exception is the exact
bit stream of the RNG beyond the published Philox known-answer vectors,
which the pages do not fix.
"""
