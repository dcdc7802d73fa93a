"""MI355X-native layerwise QK-Norm (fused Q+K RMSNorm with logical shards).

The compute path is the HIP library ``libqknorm.so`` (kernels for gfx950);
``ops`` is a thin binding with the library's names. Importing the package
does not load the library; the first op call does, and raises if it is
missing.
"""
__all__ = ["ops", "inputs"]
