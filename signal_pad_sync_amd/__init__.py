"""MI355X one-shot W-way bf16 reduction with signal-pad synchronisation.

The compute path is libarx.so (hand-written HIP for gfx950, C ABI declared in
include/arx.h); ``signal_pad_sync_amd.arx`` is its thin ctypes binding.
``signal_pad_sync_amd.workloads`` holds the seeded synthetic inputs.
"""
