"""W12 lossless 12-bit weights on MI355X: HIP kernels behind a C ABI (libw12.so).

Submodules:
  w12    -- ctypes binding of libw12.so over torch device tensors (encode, decode, gemm, q8_gemm,
            bf16_gemm, read_probe)
  synth  -- seeded synthetic inputs (no W12 arithmetic)
  build  -- hipcc build of libw12.so for gfx950
"""
