"""Writes workload_hashes.json: sha256 prefixes of head 0 of each workload's
generator output at L=600, and the ragged batch's drawn lengths.  It freezes
the input recipe; it computes no expected values of the method."""
import hashlib
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from prompt_kv_selection_amd import workloads as WL  # noqa: E402


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def main():
    out = {}
    for name, w in WL.WORKLOADS.items():
        if w.ragged:
            out[name] = digest(*WL.head_arrays(w, 0, L=600))
        else:
            out[name] = digest(*WL.head_arrays(WL.reduced(w, L=600), 0))
    out["ragged_lengths"] = WL.seq_lengths(WL.get("ragged_b8_h32_l4k_64k"))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_hashes.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
