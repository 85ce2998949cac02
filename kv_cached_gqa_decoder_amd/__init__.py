"""MI355X-native KV-cached GQA decoder: C-ABI library (libvla.so, HIP for gfx950)
and its thin ctypes binding. See include/vla.h for the entry points."""
from .vla import *  # noqa: F401,F403
from .vla import Model, VlaError, load, make_config, preset, PRESETS  # noqa: F401
