"""Write full_size_sha256.json: the SHA-256 of the CPU oracle's outputs for
every full-size workload of the parity tests, in exact and fast mode.

It calls only the oracle (inputs from synth); nothing here comes from the GPU
library.  Run from the repository root:

    python tests/golden/make_full_size_hashes.py [workload ...]

With names, only those entries are recomputed and the rest kept.
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
for p in (ROOT, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)

import full_size  # noqa: E402
import oracle  # noqa: E402


def main(names):
    orc = oracle.get()
    out = full_size.stored() if os.path.exists(full_size.STORED) else {}
    out["_about"] = ("SHA-256 of the oracle's outputs (binary32 bit patterns, C order, layers "
                     "in order) per workload and mode; written by make_full_size_hashes.py "
                     "from the inputs of synth.py")
    todo = names or list(full_size.GEMMS) + list(full_size.CONVS)
    for name in todo:
        out[name] = {}
        for mname, mode in full_size.MODES.items():
            t0 = time.time()
            out[name][mname] = full_size.oracle_digest(orc, name, mode)
            print(f"{name} {mname} {out[name][mname][:16]} ({time.time() - t0:.1f} s)", flush=True)
    with open(full_size.STORED, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
