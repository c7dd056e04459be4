"""MI355X (gfx950) Qwen3-style decoder block: HIP kernels behind a C ABI.

binding  - ctypes binding of include/sttd.h (same names as the C ABI)
device   - torch-held device memory and streams around the ABI calls
synth    - seeded synthetic inputs (weights, rows, KV fills)
workloads- the decoder shapes and workloads
"""
