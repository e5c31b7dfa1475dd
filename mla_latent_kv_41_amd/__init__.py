"""MI355X (gfx950) absorbed Multi-head Latent Attention decode.

libmla.so (HIP kernels + C ABI, include/mla.h) does the work; ``mla`` is its
Python binding, ``synth`` draws seeded synthetic workloads, ``harness`` sets one
decode step up on the GPU. Submodules are imported on demand so that importing
the package needs neither a GPU nor torch.
"""
__all__ = ["mla", "synth", "harness", "build"]
