"""Writes tests/golden/tiny_oracle.json: digests of the oracle's tables, blob and
decoded tensors for the tiny workload.  Calls only the oracle and the seeded
generator; a change of these digests means the oracle's arithmetic changed."""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402


def digests():
    w = synth.workload("tiny")
    k, v = synth.gen_kv(w)
    t = oracle.build_tables(oracle.params_for(w), k, v)
    blob = oracle.encode_chunk(t, k, v, 0, 0)
    ko, vo = np.zeros_like(k), np.zeros_like(v)
    oracle.decode_blob(t, blob, ko, vo)
    sha = lambda b: hashlib.sha256(b).hexdigest()
    return {"workload": "tiny [2,64,128] seed 0", "input_sha256": sha(k.tobytes() + v.tobytes()),
            "tables_bytes": len(t), "tables_sha256": sha(t), "blob_bytes": len(blob),
            "blob_sha256": sha(blob), "decoded_sha256": sha(ko.tobytes() + vo.tobytes())}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(digests(), f, indent=1)
        f.write("\n")
