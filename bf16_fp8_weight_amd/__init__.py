"""MI355X-native parameter preparation for RL weight transfer.

The GPU library (``libwt.so``, C ABI declared in ``include/wt.h``) is loaded by
``bf16_fp8_weight_amd.wt``; importing this package alone loads nothing, so the
seeded workload generators in ``bf16_fp8_weight_amd.workloads`` can be used
without a GPU.
"""
