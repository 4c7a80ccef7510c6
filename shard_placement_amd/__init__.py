"""MI355X-native node-local data path of TIDE's layout-aware FSDP2
collectives: fused bf16->fp32 dim-0-shard reduce-scatter and all-gather
placement, behind a C-ABI HIP library (``libtide.so``).

The heavy pieces load lazily: ``configs`` and ``synth`` import without the
HIP library; ``api`` loads it and fails loudly if it is missing.
"""
__all__ = ["configs", "synth", "api"]


def __getattr__(name):
    if name == "api":
        from . import api
        return api
    raise AttributeError(name)
