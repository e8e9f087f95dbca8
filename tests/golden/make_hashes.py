"""Write tests/golden/oracle_hashes.json: SHA-256 digests of the CPU oracle's outputs for one
seeded input set per configuration (inputs: tests/golden/cases.py).

A bitwise regression baseline (the Meituan page's "key practices" list asks for bitwise
regression checks with continuous monitoring of numeric drift): the CPU test recomputes
these digests from the oracle and the GPU test from the HIP library, and both must equal the
stored ones.  This script calls only the oracle; no stored value comes from the GPU.

Run: python tests/golden/make_hashes.py        (rewrites the JSON file)
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

from cases import HASH_FILE, LM_KEYS, cases, digest  # noqa: E402


def oracle_digest(kind, d):
    from oracle import oracle as orc
    if kind == "lmhead":
        r = orc.lmhead(d["h"], d["w"], d["target"], tau=d["tau"])
        return digest(*[r[k] for k in LM_KEYS])
    if kind == "attention":
        return digest(orc.attention(d["q"], d["k"], d["v"]))
    if kind == "gemm":
        return digest(orc.gemm(d["x"], d["w"]))
    if kind == "decoder":
        outs = []
        for b in range(d["tokens"].shape[0]):
            r = orc.decoder(d["tokens"][b], d["model"])
            outs += [r[k] for k in LM_KEYS]
        return digest(*outs)
    raise ValueError(kind)


def main():
    out = {}
    for name, (desc, kind, build) in cases().items():
        print("oracle:", name, flush=True)
        out[name] = dict(description=desc, kind=kind, sha256=oracle_digest(kind, build()))
    with open(HASH_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", HASH_FILE)


if __name__ == "__main__":
    main()
