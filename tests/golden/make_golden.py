"""Writes tests/golden/tiny_oracle.json: digests of the oracle's outputs on the
tiny workload (B1 H2 N256 D64, seed 0).  Calls only `oracle` and `synth`.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    q, k, v = synth.make_qkv(0)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    o = oracle.attn_tiled(qk, vq)
    e = oracle.attn_exact(q, k, v)
    rec = {k2: digest(qk[k2]) for k2 in ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean")}
    rec.update({k2: digest(vq[k2]) for k2 in ("v_fp8", "v_scale", "v_mean")})
    rec["attn_tiled_rel_l2_vs_exact"] = round(oracle.rel_l2(o, e), 6)
    rec["attn_tiled_first_row"] = [round(float(x), 9) for x in o[0, 0, 0, :8]]
    return rec


if __name__ == "__main__":
    rec = {"workload": "tiny B1 H2 N256 D64 seed 0", "source": "oracle (sage_oracle.c) via make_golden.py",
           **compute()}
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
