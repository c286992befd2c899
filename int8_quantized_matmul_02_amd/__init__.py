"""MI355X (gfx950) LLM.int8() mixed-precision decomposition matmul.

The computation runs in hand-written HIP kernels behind the C ABI of
``libllmint8.so`` (include/llmint8.h); ``llmint8`` holds the thin Python
binding with the same function names, ``linear`` the ``Linear8bitLt``
module built on it.  ``workloads`` draws the seeded synthetic inputs.
"""
from .llmint8 import (  # noqa: F401
    ACT_NONE,
    ACT_RELU,
    PATH_AUTO,
    PATH_DECODE,
    PATH_GEMM,
    LLMInt8Error,
    llmint8_igemm_i32,
    llmint8_matmul_e4m3,
    llmint8_matmul_e4m3_path,
    llmint8_matmul,
    llmint8_matmul_act,
    llmint8_matmul_path,
    llmint8_matmul_f8,
    llmint8_matmul_f8_path,
    llmint8_matmul_zp,
    llmint8_matmul_zp_path,
    llmint8_quantize_act,
    llmint8_quantize_act_e4m3,
    llmint8_quantize_act_f8,
    llmint8_quantize_act_workspace_bytes,
    llmint8_quantize_act_zp,
    llmint8_quantize_weight,
    llmint8_quantize_weight_e4m3,
    llmint8_quantize_weight_f8,
    llmint8_quantize_weight_zp,
    llmint8_status_string,
    llmint8_workspace_bytes,
)
from .linear import Linear8bitLt  # noqa: F401
