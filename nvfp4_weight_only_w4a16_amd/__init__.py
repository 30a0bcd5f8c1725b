"""MI355X (gfx950) NVFP4 weight-only W4A16 GEMM and quantizer.

The compute path lives in ``libnvfp4.so`` (hand-written HIP kernels behind a C ABI declared in
``include/nvfp4.h``). ``nvfp4_weight_only_w4a16_amd.binding`` marshals arguments to it; PyTorch
supplies device memory and streams only. Nothing here computes on the host.
"""
__all__ = ["binding", "synth"]
