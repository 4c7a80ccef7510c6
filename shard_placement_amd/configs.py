"""Synthetic workloads: parameter shapes of the layers the paper trains.

The paper's Abstract ("The Endgame of FSDP Communication", weekinpapers.com)
and the kongchang.com article's "Performance" section name Llama-3.1 70B,
Wan2.2 and Qwen3-30B-A3B.  They print no gradient data, so these synthetic
layers, shaped after the public architectures, stand in for them; gradients
are seeded random values (see ``synth``).  A shape is a tuple of ints; its
first dimension is the one that is sharded.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

Shape = Tuple[int, ...]


@dataclass(frozen=True)
class Workload:
    key: int                 # 1..5; seeds derive from it
    name: str
    R: int                   # simulated ranks
    names: Tuple[str, ...]   # parameter names, registration order
    shapes: Tuple[Shape, ...]
    sigma: float             # standard deviation of the synthetic gradients
    slot_reuse: bool = False  # fp32 shards staged in vacated gathered buffers
    note: str = ""

    @property
    def P(self) -> int:
        return len(self.shapes)

    def numel(self) -> int:
        total = 0
        for shp in self.shapes:
            n = 1
            for d in shp:
                n *= d
            total += n
        return total


def _llama70b_layer() -> List[Tuple[str, Shape]]:
    h, kv, ffn = 8192, 1024, 28672
    return [("q_proj", (h, h)), ("k_proj", (kv, h)), ("v_proj", (kv, h)),
            ("o_proj", (h, h)), ("gate_proj", (ffn, h)), ("up_proj", (ffn, h)),
            ("down_proj", (h, ffn)), ("input_norm", (h,)), ("post_attn_norm", (h,))]


def _qwen3_moe_layer() -> List[Tuple[str, Shape]]:
    h, experts, inter = 2048, 128, 768
    out = [("q_proj", (4096, h)), ("k_proj", (512, h)), ("v_proj", (512, h)),
           ("o_proj", (h, 4096))]
    for e in range(experts):
        out += [("experts.%d.gate" % e, (inter, h)), ("experts.%d.up" % e, (inter, h)),
                ("experts.%d.down" % e, (h, inter))]
    out.append(("router", (experts, h)))
    return out


def _wan22_block() -> List[Tuple[str, Shape]]:
    d, ffn = 5120, 13824
    out = []
    for blk in ("self_attn", "cross_attn"):
        for w in ("q", "k", "v", "o"):
            out.append(("%s.%s" % (blk, w), (d, d)))
    out += [("ffn.0", (ffn, d)), ("ffn.2", (d, ffn)), ("modulation", (6, d)),
            ("norm1", (d,)), ("norm2", (d,))]
    return out


def _mk(key, name, R, pairs, sigma, slot_reuse=False, note=""):
    return Workload(key=key, name=name, R=R, names=tuple(n for n, _ in pairs),
                    shapes=tuple(s for _, s in pairs), sigma=sigma,
                    slot_reuse=slot_reuse, note=note)


WORKLOADS = {
    1: _mk(1, "tiny", 4, [("a", (37, 16)), ("b", (64, 64)), ("c", (5,))], 1.0,
           note="R=4, three small params; ragged and all-padding shards"),
    2: _mk(2, "llama3.1-70b-layer", 8, _llama70b_layer(), 1e-3,
           note="one Llama-3.1-70B decoder layer, R=8"),
    3: _mk(3, "qwen3-30b-a3b-moe-layer", 16, _qwen3_moe_layer(), 1e-3,
           note="Qwen3-30B-A3B-style MoE layer, 128 experts, R=16"),
    4: _mk(4, "wan2.2-14b-dit-block", 32, _wan22_block(), 1e-3,
           note="Wan2.2-14B-style DiT block, R=32; two norms"),
    5: _mk(5, "llama3.1-70b-layer-ragged-r64", 64,
           _llama70b_layer() + [("ragged", (1001, 8192))], 1e-3, slot_reuse=True,
           note="Llama-3.1-70B layer plus a ragged [1001,8192] param, R=64, "
                "fp32 shards staged in vacated gathered buffers"),
}


def get(key) -> Workload:
    if isinstance(key, str):
        for w in WORKLOADS.values():
            if w.name == key or str(w.key) == key:
                return w
        raise KeyError(key)
    return WORKLOADS[int(key)]
