"""Writes image_chain_rows.npz: sampled rows of the 28-block image-DiT
forward computed by the oracle (fp64), for the chained-forward GPU test.
Calls only synth (inputs) and oracle (the computation).

    python tests/golden/make_image_chain.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import dit as D, layout as OL  # noqa: E402

ROWS = (0, 1, 1023, 2048, 3071, 4094, 4095)


def main():
    wl = synth.workload("image")
    shapes = list(wl.blocks)
    x = synth.activations(wl.tokens, shapes[0].d_model).astype(np.float64)
    cond = synth.conditioning(shapes[0].d_cond)
    rows = np.array(ROWS)
    for b, shp in enumerate(shapes):
        flat = synth.block_weights(wl.wid, b, OL.block_numel(shp))
        if b + 1 < len(shapes):
            x = D.dit_block(flat, shp, x, cond)
        else:
            x = D.dit_block(flat, shp, x, cond, rows=rows)
        print(f"block {b} done", flush=True)
    np.savez_compressed(os.path.join(HERE, "image_chain_rows.npz"), rows=rows, out=x.astype(np.float64))


if __name__ == "__main__":
    main()
