"""MI355X-native RWKV-7 WKV time-mix recurrence (prefill and single-token step).

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI in
include/rwkv7_wkv.h (librwkv7_wkv.so, built by `python -m linear_rnn_amd.build`).
`linear_rnn_amd.wkv` is the thin ctypes binding; `linear_rnn_amd.inputs` holds
the seeded synthetic workloads.
"""
__all__ = ["wkv", "inputs", "build"]
