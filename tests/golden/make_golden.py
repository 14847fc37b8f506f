"""Write tiny_oracle.json: oracle outputs on the tiny fp32 workload (seed 0).

Calls only ``oracle`` and ``synth``.  The file is a regression fixture of the
oracle; the pins that tie the oracle to the pages are in tests/test_oracle_*.py.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from synth import make_workload  # noqa: E402


def tiny_reference():
    wl = make_workload("tiny", seed=0)
    c = wl.cfg
    Ks = [t.double().numpy() for t in wl.group_kv(0, "K", 0)]
    Vs = [t.double().numpy() for t in wl.group_kv(0, "V", 0)]
    ck, cv = oracle.compress_group(Ks, c.rank), oracle.compress_group(Vs, c.rank)
    out = {"rel_err_K": ck["rel_err"], "rel_err_V": cv["rel_err"],
           "eigvals_K_top": ck["eigvals"][: c.rank + 4].tolist(), "layers": []}
    exact = [t for t in range(c.T) if t < c.n_sink or t >= c.T - c.n_local]
    for l in range(c.n_layers):
        lm = oracle.landmarks(Ks[l], c.n_kv_heads, c.head_dim, c.chunk)
        res = oracle.sr_decode_layer(
            wl.query(0, l, 0).double().numpy(), T=c.T, n_gen=0, n_kv_heads=c.n_kv_heads,
            chunk=c.chunk, top_k=c.top_k, n_sink=c.n_sink, n_local=c.n_local, landmarks_l=lm,
            A_k=ck["A"], B_k_l=ck["B"][:, l * c.d_kv:(l + 1) * c.d_kv],
            A_v=cv["A"], B_v_l=cv["B"][:, l * c.d_kv:(l + 1) * c.d_kv],
            k_exact={t: Ks[l][t] for t in exact}, v_exact={t: Vs[l][t] for t in exact})
        out["layers"].append({"sel": res["sel"].tolist(), "out": res["out"].tolist(),
                              "scores": res["scores"].tolist()})
    return out


if __name__ == "__main__":
    ref = tiny_reference()
    ref["generated_by"] = "tests/golden/make_golden.py (oracle + synth only)"
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(ref, f, indent=1)
    print("wrote tiny_oracle.json")
