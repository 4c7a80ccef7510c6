"""Write tests/golden/tiny_oracle.json: the oracle's outputs on the tiny
workload (R=4; params [37,16], [64,64], [5]; bf16 N(0,1); rank q seeded
1000*1+q; gathered buffer seeded 1000*1+999), as SHA-256 digests of the
output bits plus a few leading values per shard.

Calls only the oracle package (and the seeded input generator).  Rerun it
only when a change to the oracle's arithmetic is justified by a reading of
the pages, and say which in the commit message.
"""
import hashlib
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from shard_placement_amd import configs, synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_inputs():
    w = configs.get(1)
    grads = []
    for q in range(w.R):
        arena = torch.empty(synth.arena_numel(w.shapes), dtype=torch.bfloat16)
        synth.fill_normal_(arena, synth.SEED_STRIDE * w.key + q, w.sigma)
        grads.append(arena.view(torch.int16).numpy().view(np.uint16).copy())
    _, _, _, S = oracle.layout(w.shapes, w.R)
    g = torch.empty(w.R * S, dtype=torch.bfloat16)
    synth.fill_normal_(g, synth.SEED_STRIDE * w.key + synth.GATHERED_SEED_OFFSET, w.sigma)
    gathered = g.view(torch.int16).numpy().view(np.uint16).copy()
    return w, grads, gathered


def split(arena, shapes):
    out, pos = [], 0
    for shp in shapes:
        n = int(np.prod(shp))
        out.append(arena[pos:pos + n])
        pos += n
    return out


def main():
    w, arenas, gathered = tiny_inputs()
    grads = [split(a, w.shapes) for a in arenas]
    s, m, off, S = oracle.layout(w.shapes, w.R)
    rec = {"workload": w.name, "R": w.R, "shapes": [list(x) for x in w.shapes],
           "slot_numel": S, "input_sha256": [sha(a) for a in arenas],
           "gathered_sha256": sha(gathered)}
    for order in ("fixed", "tree"):
        out = oracle.rs(w.shapes, w.R, grads, order=order)
        rec["rs_%s_sha256" % order] = [sha(o.view(np.uint32)) for o in out]
        rec["rs_%s_head" % order] = {
            "%d/%d" % (r, p): [format(int(x), "08x") for x in out[r].view(np.uint32)[off[p]:off[p] + min(4, m[p])]]
            for r in range(w.R) for p in range(w.P)}
    placed = oracle.ag(w.shapes, w.R, gathered)
    rec["ag_sha256"] = [sha(x) for x in placed]
    with open(OUT, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
