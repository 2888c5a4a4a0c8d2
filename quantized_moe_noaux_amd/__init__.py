"""MI355X-native quantised MoE layer: HIP kernels for gfx950 behind a C ABI.

The layer (GeekNews #31297 "Show HN: running GLM 5.2 on a slow computer",
implemented features; wpnews.pro "Colibri - GLM-5.2 744B MoE on 25GB RAM",
model spec table): noaux_tc sigmoid router with correction bias and
group-limited top-k, Q8_0-style int8 block-32 activations, routed and shared
SwiGLU experts over packed int4 / int8 / int2 codes with per-row scales, and
a weighted combine.  `moe` is the ctypes binding of include/moe.h.
"""
from . import moe
from .moe import *  # noqa: F401,F403
