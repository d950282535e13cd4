"""MI355X-native block-wise decoding forward (AR / block diffusion /
self-speculation) behind a C ABI (include/sdm.h, libsdm.so).

Importing the package does not touch the GPU; ``Model`` loads libsdm.so and
fails loudly if it has not been built (``python -m self_speculative_amd.build``).
"""
import importlib

from ._lib import (SDM_BF16, SDM_BIDIR, SDM_CAUSAL, SDM_F32, SdmConfig, SdmError, lib)  # noqa: F401

__all__ = ["Model", "SdmError", "lib", "decode"]


def __getattr__(name):
    if name == "Model":
        return importlib.import_module(".model", __name__).Model
    if name == "decode":
        return importlib.import_module(".decode", __name__)
    raise AttributeError(name)
