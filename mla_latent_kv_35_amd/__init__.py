"""MI355X-native MLA absorbed decode.

The compute path lives in the HIP/C-ABI library built from csrc/ (loaded by
`binding`); `synth` draws seeded synthetic workloads. Importing the package
does not load the library: `from mla_latent_kv_35_amd import binding` does,
and fails loudly when it is missing.
"""
__all__ = ["synth", "binding"]
