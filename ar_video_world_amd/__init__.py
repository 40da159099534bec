"""MI355X-native KV-memory hot path of WorldKV-style autoregressive video world
models: World Compression, pose retrieval, window assembly and chunk attention
as hand-written HIP kernels for gfx950 behind a C ABI (include/wkv.h).

The binding lives in ``ar_video_world_amd.wkv`` (importing it requires the
built ``libwkv.so``); ``ar_video_world_amd.build`` compiles the library.
"""
__all__ = ["wkv", "build"]
