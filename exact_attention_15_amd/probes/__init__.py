"""Measurement probes of gfx950's ceilings, for reading the kernels'
rooflines: HBM read bandwidth (``stream``), vector / transcendental / MFMA
issue rates and their co-issue (``units``), and LDS read rates, plain,
transposing and feeding MFMAs (``lds``).  They are standalone HIP programs,
not part of the library; ``python -m exact_attention_15_amd.probes NAME``
builds one for gfx950 (in ``_build/probes``) and runs it.
"""
