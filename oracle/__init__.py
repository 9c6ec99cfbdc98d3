"""CPU oracle for bit-plane GEMV -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy implementations of what the GPU library
computes: the weight quantizers, the per-token activation quantizer, the
bit-plane contraction and the GEMV itself (explicit dequantization followed by
an fp64 dot product, or an exact int64 dot product for integer partials).

Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of
bench.py may import this package.  It shares no code with the library
(bit_plane_gemv_amd/): the two meet only through the seeded inputs of the
`synth` package and through the documented packed-blob layout, which
oracle/layout.py re-implements on its own.

Sources (cited below by the short name in brackets):
  [RaBiT]  "RaBiT框架：突破2比特量化性能瓶颈的LLM部署方案"
           (RaBiT: 2-path residual binarization)
  [HGF]    "1.58位LLM混合门控流优化技术解析"
           (Hybrid Gated Flow: ternary weights, int8 activations)
  [ABQ]    "ABQ-LLM：用于大語言模型的任意比特量化推理加速"
           (arbitrary-bit W/A quantization, binary-TensorCore-equivalent GEMM)
  [BVSR]   "BVSR：面向分布感知的大语言模型权重量化的比特向量求和表示"
           (bitvector-sum representation, Neurocomputing)
  [BitNet] "1-bit LLM的端侧推理革命" (BitNet 1-bit edge deployment)

Precision policy: floating-point results are computed in fp64 unless a step is
specified in a narrower type (fp32 activation quantizer, fp16/fp32 storage of
coefficients); integer results are exact int64.

Parity status: every function in this package is pinned by tests under
tests/ (test_oracle_*.py) against identities, closed forms, brute force or a
library routine; none is "parity unpinned".
"""
from . import common, bitserial, act, weights, gemv, layout  # noqa: F401
