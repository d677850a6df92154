"""TurboQuant hot path for AMD Instinct MI355X (gfx950).

The compute lives in libtq.so (HIP kernels behind the C ABI of include/tq.h);
`api` wraps it for PyTorch device tensors and `synth` draws the seeded
synthetic inputs used by tests and benchmarks.
"""
__version__ = "0.1.0"
