"""MI355X-native node-local data path of TIDE's layout-aware FSDP2
collectives: fused bf16->fp32 dim-0-shard reduce-scatter and all-gather
placement, behind a C-ABI HIP library (``libtide.so``).

Submodules: ``configs`` and ``synth`` (workload shapes, seeded inputs) import
without the HIP library; ``api`` (the binding) loads it and fails loudly when
it is missing.
"""
