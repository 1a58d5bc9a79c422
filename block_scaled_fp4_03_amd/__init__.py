"""MI355X (gfx950) NVFP4 mixture-of-experts expert pipeline.

The compute lives in ``libnvfp4moe.so`` (hand-written HIP, C ABI declared in
``include/nvfp4moe.h``); ``ops`` is a thin ctypes binding over it that takes
torch tensors for device memory and streams.  ``workloads`` draws the seeded
synthetic inputs.  The library is loaded lazily on the first op call, and a
missing library is an error: there is no fallback path.
"""
__all__ = ["ops", "workloads", "lib"]
