"""Writes the stored expected values under tests/golden/.

Calls only the oracle (and the seeded input generator for its inputs); no
value here ever comes from the HIP library.  Re-run after a change to the
oracle's arithmetic that the Prox pages justify:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))


def toy_case():
    """512 x 1376 fp32 layer, one token, int8 row proxy, keep 0.5, sparsity 0.5, seed 0."""
    w = synth.WORKLOADS["toy_fp32"]
    wg, wu, wd = synth.make_weights(w.d, w.F, w.std, w.dtype, seed=0)
    x = synth.make_x(1, w.d, w.dtype, seed=0)
    qg, scg = oracle.quantize(wg, "int8_row")
    qu, scu = oracle.quantize(wu, "int8_row")
    r = oracle.prox_forward(x, wg, wu, wd, (qg, scg, qu, scu), w.input_keep, w.sparsities[0], "int8_row")
    return {
        "what": "Prox forward, 512x1376 fp32 layer, B=1, int8 per-row proxy, input_keep 0.5, ffn_sparsity 0.5, "
                "inputs synth seed 0 layer 0",
        "written_by": "tests/golden/make_golden.py (oracle only)",
        "k_in": r["k_in"], "k": r["k"], "T": r["T"],
        "sel": r["sel"].tolist(),
        "score_head": [float(v) for v in r["score"][:32]],
        "y": [float(v) for v in r["y"][0]],
        "codes_gate_row0": qg[0].tolist(), "scale_gate_row0": float(scg[0]),
    }


if __name__ == "__main__":
    with open(os.path.join(OUT, "toy_fp32_seed0.json"), "w") as f:
        json.dump(toy_case(), f, indent=0)
    print("wrote", os.path.join(OUT, "toy_fp32_seed0.json"))
