"""Block-scaled FP4 (MXFP4 / NVFP4) mixture-of-experts layer for AMD MI355X.

The compute path is the HIP library ``libmoe_fp4.so`` built from ``csrc/``;
``moe`` is its thin ctypes binding (argument marshalling only): ``Desc``
(shape, weight format, activation format "bf16" / "mxfp8", activation
function), ``Fp4MoE`` (prepared weights + workspace, callable), and the
entry points one to one.  ``synth`` draws seeded synthetic inputs.
"""
