"""MI355X-native (gfx950) KDA forward scan: HIP kernels behind a C ABI.

``inputs`` (seeded synthetic workloads) imports without the GPU library; the
binding in ``kda`` loads ``libkda.so`` on first use and fails loudly when it is
missing.
"""
__all__ = ["inputs", "kda"]
