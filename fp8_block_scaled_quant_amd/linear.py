"""FP8 linear layer over the block-scaled kernels.

The page "DeepSeek-V3 quantization_config Parameters Explained" (section
"Integrating with Linear Layers") shows the layer a user of the method calls:
``Linear(in_features, out_features, dtype="fp8")`` holding an E4M3 weight and
its block scales, whose forward pass manages quantization itself.  The page
"Understanding Dynamic and Static Activation Quantization Schemes in
DeepSeek-V3" (section "How Dynamic Activation Quantization Works") has the
linear wrapper call act_quant on the activations before the FP8 GEMM; the page
"How weight_dequant Handles Per-Block Scaling in DeepSeek-V3 FP8 GEMM"
(sections "Relationship to FP8 GEMM Operations" and "Practical Usage Example")
gives the alternative of dequantizing the weight and using a plain linear
product, for layer types or debugging the FP8 product does not serve.

This module's forward runs ``act_quant_gemm`` (one C-ABI call: act_quant of the
activations, the block-scaled GEMM, the bias added in the GEMM's epilogue);
``gemm_impl="dequant"`` instead dequantizes the weight with
``weight_dequant`` and calls ``torch.nn.functional.linear``.  Nothing falls
back to the CPU: tensors on the CPU raise.
"""

import torch

from . import act_quant_gemm, weight_dequant, weight_quant

BLOCK = 128


class Linear(torch.nn.Module):
    """``y = x W^T (+ b)`` with ``W`` held as E4M3 codes and 128x128 block scales.

    Parameters (frozen; this is an inference layer):

    * ``weight``       float8_e4m3fn ``[out_features, in_features]``;
    * ``weight_scale`` float32 ``[ceil(out/128), ceil(in/128)]`` -- the stored
      inverse scale of each weight tile (weight_scale_inv): dequantized weight
      = code * scale;
    * ``bias``         ``[out_features]`` of ``dtype``, or None.

    ``scale_fmt`` is the activations' act_quant scale format (None or "ue8m0");
    ``dtype`` the output (and bias) dtype, bf16 or fp32.
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = False,
                 dtype: torch.dtype = torch.bfloat16, scale_fmt=None, gemm_impl: str = "fp8",
                 device=None):
        super().__init__()
        if in_features % BLOCK != 0:
            raise ValueError(f"in_features must be a multiple of {BLOCK} (act_quant blocks)")
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be bfloat16 or float32")
        if scale_fmt not in (None, "ue8m0"):
            raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
        if gemm_impl not in ("fp8", "dequant"):
            raise ValueError("gemm_impl must be 'fp8' or 'dequant'")
        self.in_features, self.out_features = in_features, out_features
        self.dtype, self.scale_fmt, self.gemm_impl = dtype, scale_fmt, gemm_impl
        grid = (-(-out_features // BLOCK), -(-in_features // BLOCK))
        self.weight = torch.nn.Parameter(
            torch.zeros(out_features, in_features, dtype=torch.float8_e4m3fn, device=device),
            requires_grad=False)
        self.weight_scale = torch.nn.Parameter(
            torch.ones(grid, dtype=torch.float32, device=device), requires_grad=False)
        if bias:
            self.bias = torch.nn.Parameter(torch.zeros(out_features, dtype=dtype, device=device),
                                           requires_grad=False)
        else:
            self.register_parameter("bias", None)

    @classmethod
    def from_weight(cls, weight: torch.Tensor, bias: torch.Tensor = None, weight_scale_fmt=None,
                    **kwargs) -> "Linear":
        """Quantize a bf16/fp32 GPU weight ``[out, in]`` per 128x128 tile
        (``weight_quant``) into a new layer; ``bias`` is copied in ``dtype``."""
        out_features, in_features = weight.shape
        layer = cls(in_features, out_features, bias=bias is not None, device=weight.device, **kwargs)
        y, s = weight_quant(weight.contiguous(), BLOCK, weight_scale_fmt)
        layer.weight.data.copy_(y)
        layer.weight_scale.data.copy_(s)
        if bias is not None:
            layer.bias.data.copy_(bias.to(layer.dtype))
        return layer

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        if self.gemm_impl == "dequant":
            w = weight_dequant(self.weight, self.weight_scale, BLOCK, self.dtype)
            return torch.nn.functional.linear(x.to(self.dtype), w, self.bias)
        if x.dtype not in (torch.bfloat16, torch.float32):
            x = x.to(self.dtype)
        c, _, _ = act_quant_gemm(x.contiguous(), self.weight, self.weight_scale, self.scale_fmt,
                                 self.dtype, self.bias)
        return c

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, dtype={self.dtype}, scale_fmt={self.scale_fmt}, "
                f"gemm_impl={self.gemm_impl}")
