"""Writes tests/golden/config0_session.json by running the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
The stored values guard the oracle against unnoticed changes; they are never
produced by, or compared with anything but, the oracle itself.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth                      # noqa: E402
from oracle import dflash as O    # noqa: E402


def main():
    wl = synth.workload(0)
    model = O.Model(wl.shape, synth.weights(wl.shape, wl.seed), keep=True)
    sess = O.Session(model, wl, keep_outputs=True)
    steps = []
    for _ in range(wl.steps):
        r = sess.step()
        steps.append({"tau": r.tau.tolist(), "ctx_len": r.ctx_len.tolist(),
                      "cap": r.cap.tolist(), "draft": r.draft.tolist(),
                      "logits_head": r.logits[0, :, :8].tolist()})
    out = {"workload": wl.name, "seed": wl.seed, "steps": steps,
           "_note": "written by tests/golden/make_golden.py from the fp64 oracle"}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "config0_session.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
