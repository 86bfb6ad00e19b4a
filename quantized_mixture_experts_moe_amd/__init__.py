"""Grouped, weight-quantized Mixture-of-Experts FFN for MI355X (gfx950).

The compute path is the C-ABI library ``libqmoe.so`` (hand-written HIP);
``ops`` is a thin ctypes binding with the same call names.  ``shapes`` and
``synth`` describe and draw the synthetic workloads.
"""
