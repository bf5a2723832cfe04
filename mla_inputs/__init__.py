"""Seeded synthetic workloads for MLA over a shared latent cache.

This module is the only code shared by the CPU oracle and the HIP path.  It
holds workload shapes and a deterministic random generator, and none of the
method's arithmetic: no projection, no rotary embedding, no attention, no
quantisation.  Floating-point inputs are drawn as float32 normals, scaled, and
handed out either as float32 or as bfloat16 bit patterns (uint16) so that both
sides receive identical bits.
"""
from .configs import MLAConfig, CONFIGS, EXTRA_CONFIGS, SMALL_CONFIGS, get_config  # noqa: F401
from .generate import make_workload, bf16_bits_from_f32, bf16_bits_to_f32  # noqa: F401
