"""MI355X-native multi-head latent attention over a shared latent cache.

The path runs in hand-written HIP kernels for gfx950 behind the C-ABI in
``include/mla.h`` (``libmla_amd.so``); this package is its thin Python
binding.  Build the library with ``python -m head_latent_attention_cache_amd.build``.
"""
from ._lib import (MLA_BF16, MLA_CACHE_DENSE, MLA_CACHE_INT4, MLA_F32, MLAError, MlaDims,  # noqa: F401
                   MlaGeom, SIGNATURES, load)


def __getattr__(name):
    # the torch-facing wrappers (and torch) are imported on first use
    import importlib
    api = importlib.import_module(__name__ + ".api")
    if name == "api":
        return api
    return getattr(api, name)
