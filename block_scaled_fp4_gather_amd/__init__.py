"""Block-scaled FP4 (MXFP4 / NVFP4) mixture-of-experts layer for AMD MI355X.

The compute path is the HIP library ``libmoe_fp4.so`` built from ``csrc/``;
``moe`` is its thin ctypes binding (argument marshalling only).  ``synth``
draws seeded synthetic inputs.
"""
