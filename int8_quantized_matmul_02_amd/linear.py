"""Linear8bitLt: a torch.nn.Module over the library's C ABI.

The Hugging Face write-up of LLM.int8() (agentlenshq.com, "Hugging Face,
LLM.int8() 8-bit matrix multiplication integrated into Transformers and
Accelerate", section "Integration into transformers") describes the
user-facing piece: a drop-in replacement for torch.nn.Linear that stores the
weight as int8 CB plus per-output-column scales SCB when it is moved to the
GPU (has_fp16_weights=False), runs the decomposition matmul with a
`threshold` (6.0 by default) and adds the bias.  With has_fp16_weights=True
the fp16 weight stays the parameter and is quantized again on every call
(the mode for weights that still change).

Everything computed runs in libllmint8's HIP kernels: weight quantization
(llmint8_quantize_weight), the whole decomposition (llmint8_matmul_act), and
an optional ReLU fused into its output rounding for the feed-forward
expansion layers.  `quant` selects the 8-bit part's quantizer: "absmax" (the
method's vector-wise absmax int8), or the library's two variants,
"zeropoint" (asymmetric int8, llmint8_matmul_zp), "fp8" (E5M2,
llmint8_matmul_f8) and "fp8_e4m3" (E4M3, llmint8_matmul_e4m3); the variants
have no fused activation.  This module only holds the tensors, flattens leading
dimensions into rows, and shares one workspace buffer per (device, stream)
among all instances, grown as needed, so that steady-state calls allocate
nothing but their output and a model needs one workspace, not one per layer.
Calls on one stream run in order, so they may share it; calls on different
streams get different buffers.
"""
import torch

from . import llmint8 as L

# (device, stream handle) -> uint8 workspace tensor shared by every module
_WORKSPACES = {}


def _shared_workspace(nbytes, device):
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        # a larger buffer replaces the old one; work already enqueued on this
        # stream keeps the old one alive through the caching allocator
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws

_ACTS = {None: L.ACT_NONE, "none": L.ACT_NONE, "relu": L.ACT_RELU}
_QUANTS = ("absmax", "zeropoint", "fp8", "fp8_e4m3")
# the FP8 quantizers: the binding's function-name suffix of each format
_FP8 = {"fp8": "f8", "fp8_e4m3": "e4m3"}


class Linear8bitLt(torch.nn.Module):
    """y = act(x W^T + b) through the LLM.int8() decomposition.

    in_features and out_features must be multiples of 64 (the library's
    tile granularity), in_features at most 133,144.  Inputs are fp16 on a
    HIP device with in_features as the last dimension; the output is fp16.
    """

    def __init__(self, in_features, out_features, bias=True, has_fp16_weights=False,
                 threshold=6.0, activation=None, device=None, quant="absmax"):
        super().__init__()
        if quant not in _QUANTS:
            raise ValueError("quant must be one of %s, got %r" % (_QUANTS, quant))
        if quant != "absmax" and _ACTS.get(activation, None) not in (L.ACT_NONE,):
            raise ValueError("the %s variant has no fused activation" % quant)
        if quant == "zeropoint" and in_features > 33286:
            raise ValueError("in_features must be at most 33286 for the zero-point variant")
        if in_features % 64 or out_features % 64 or in_features <= 0 or out_features <= 0:
            raise ValueError("in_features and out_features must be positive multiples of 64, "
                             "got %d and %d" % (in_features, out_features))
        if in_features > 133144:
            raise ValueError("in_features must be at most 133144 (int32-exact accumulation)")
        if activation not in _ACTS:
            raise ValueError("activation must be None, 'none' or 'relu', got %r" % (activation,))
        if not threshold >= 0.0:
            raise ValueError("threshold must be >= 0 (float('inf') disables outliers)")
        self.in_features = in_features
        self.out_features = out_features
        self.has_fp16_weights = has_fp16_weights
        self.threshold = float(threshold)
        self.activation = activation
        self.quant = quant
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=torch.float16, device=device),
            requires_grad=False)
        torch.nn.init.normal_(self.weight, 0.0, 0.02)
        if bias:
            self.bias = torch.nn.Parameter(
                torch.zeros((out_features,), dtype=torch.float16, device=device),
                requires_grad=False)
        else:
            self.register_parameter("bias", None)
        self.register_buffer("CB", None)    # int8 codes (fp8 / fp8_e4m3: E5M2 / E4M3 codes, uint8)
        self.register_buffer("SCB", None)   # absmax: column absmax; zero-point: nd; fp8: 2^-e
        self.register_buffer("ZP", None)    # zero-point variant: zero points and code sums
        self.register_buffer("RS", None)

    @classmethod
    def from_linear(cls, linear, has_fp16_weights=False, threshold=6.0, activation=None,
                    quant="absmax"):
        """A Linear8bitLt holding torch.nn.Linear `linear`'s weight and bias
        (cast to fp16); quantized on the first forward call, or by
        quantize_()."""
        m = cls(linear.in_features, linear.out_features, bias=linear.bias is not None,
                has_fp16_weights=has_fp16_weights, threshold=threshold, activation=activation,
                device=linear.weight.device, quant=quant)
        with torch.no_grad():
            m.weight.copy_(linear.weight.to(torch.float16))
            if linear.bias is not None:
                m.bias.copy_(linear.bias.to(torch.float16))
        return m

    def quantize_(self):
        """Quantize the fp16 weight into CB and SCB (on its device).  Without
        fp16 weights the fp16 parameter is released afterwards, as the
        write-up's Int8Params does when the weight is moved to the GPU."""
        if self.weight is None:
            return self
        if self.weight.device.type != "cuda":
            raise RuntimeError("Linear8bitLt: move the module to a HIP device before quantizing")
        w = self.weight.detach().contiguous()
        if self.CB is None or self.CB.device != w.device:
            dt = torch.uint8 if self.quant in _FP8 else torch.int8
            self.CB = torch.empty((self.out_features, self.in_features), dtype=dt, device=w.device)
            self.SCB = torch.empty((self.out_features,), dtype=torch.float32, device=w.device)
            if self.quant == "zeropoint":
                self.ZP = torch.empty((self.out_features,), dtype=torch.int32, device=w.device)
                self.RS = torch.empty((self.out_features,), dtype=torch.int32, device=w.device)
        if self.quant == "zeropoint":
            L.llmint8_quantize_weight_zp(w, CB=self.CB, ND=self.SCB, ZP=self.ZP, RS=self.RS)
        elif self.quant in _FP8:
            getattr(L, "llmint8_quantize_weight_" + _FP8[self.quant])(w, CB8=self.CB, SC8=self.SCB)
        else:
            L.llmint8_quantize_weight(w, CB=self.CB, SCB=self.SCB)
        if not self.has_fp16_weights:
            self.weight = None
        return self

    def _workspace(self, T, device):
        return _shared_workspace(L.llmint8_workspace_bytes(T, self.in_features, self.out_features),
                                 device)

    def forward(self, x):
        if x.dtype != torch.float16:
            raise TypeError("Linear8bitLt expects fp16 input, got %s" % x.dtype)
        if x.shape[-1] != self.in_features:
            raise ValueError("last dimension %d != in_features %d" % (x.shape[-1], self.in_features))
        if self.has_fp16_weights or self.CB is None:
            # fp16 weights are quantized on every call (they may have changed)
            self.quantize_()
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        T = x2.shape[0]
        if T == 0:
            return x.new_empty(lead + (self.out_features,))
        ws = self._workspace(T, x2.device)
        if self.quant == "zeropoint":
            out = L.llmint8_matmul_zp(x2, self.CB, self.SCB, self.ZP, self.RS, self.threshold,
                                      bias=self.bias, ws=ws)
        elif self.quant in _FP8:
            out = getattr(L, "llmint8_matmul_" + _FP8[self.quant])(
                x2, self.CB, self.SCB, self.threshold, bias=self.bias, ws=ws)
        else:
            out = L.llmint8_matmul_act(x2, self.CB, self.SCB, self.threshold,
                                       _ACTS[self.activation], bias=self.bias, ws=ws)
        return out.reshape(lead + (self.out_features,))

    def extra_repr(self):
        return ("in_features=%d, out_features=%d, bias=%s, has_fp16_weights=%s, threshold=%g, "
                "activation=%s, quant=%s" % (self.in_features, self.out_features,
                                             self.bias is not None, self.has_fp16_weights,
                                             self.threshold, self.activation, self.quant))
