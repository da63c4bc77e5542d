"""MI355X-native forward pass of one mixture-of-experts feed-forward layer.

The hot path lives in libmoe.so (HIP kernels for gfx950 behind a C ABI, declared
in include/moe.h); ``_lib`` binds it with ctypes and ``layer`` chains its calls.
The library is loaded on first use: importing this package needs no GPU.
"""
