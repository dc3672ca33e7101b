"""Write tests/golden/tiny_greedy.json from the oracle alone.

The pages print no worked numbers for the decode step, so this fixture is a
regression anchor for the oracle, not a pin: it records the tiny fp32
decoder's greedy run (8 uniform prompt ids, 32 greedy steps, seeds of the
synthetic workload) so that any later change to the oracle's arithmetic shows
up as a diff of this file.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import Decoder, top2_margin  # noqa: E402
from persistent_megakernel_loop_amd import workload as wl  # noqa: E402


def tiny_greedy():
    shape = wl.TINY
    weights = wl.make_weights(shape)
    prompt = wl.make_prompt_ids(shape)
    dec = Decoder.from_shape(shape, weights)
    first, logits, _ = dec.prefill(prompt)
    ids, margins, cur = [first], [top2_margin(logits)], first
    for _ in range(shape.steps):
        lg, _ = dec.step(dec.input_row(cur))
        cur = int(np.argmax(lg.astype(np.float32)))
        ids.append(cur)
        margins.append(top2_margin(lg))
    return {"workload": shape.name, "prompt": [int(v) for v in prompt], "ids": ids,
            "margins": [round(m, 6) for m in margins]}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_greedy.json"), "w") as f:
        d = tiny_greedy()
        f.write("{\n" + ",\n".join(f' "{k}": {json.dumps(v)}' for k, v in d.items()) + "\n}\n")
