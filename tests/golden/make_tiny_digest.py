"""Write tiny_oracle_digest.json: SHA-256 of the CPU oracle's outputs on the tiny workload.

Calls only oracle/ and the input generator. Rerun it (and say why in the commit) only when
the oracle's arithmetic or the generator changes on purpose.
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from bitwise_consistent_linear_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402


def digests():
    w = W.tiny()
    o, cs, fs = O.scan(w.cu_seqlens, w.q, w.k, w.v, w.a, w.b, chunk=w.chunk,
                       want_chunk_states=True, want_final_state=True)
    return {
        "workload": "tiny: N=1, T=64, Hk=Hv=2, d=16, C=16, float32, seed 0",
        "o_sha256": hashlib.sha256(o.tobytes()).hexdigest(),
        "chunk_states_sha256": hashlib.sha256(cs.tobytes()).hexdigest(),
        "final_state_sha256": hashlib.sha256(fs.tobytes()).hexdigest(),
        "o_first4_hex": [f"0x{x:08x}" for x in o.reshape(-1)[:4].view("uint32")],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle_digest.json"), "w") as f:
        json.dump(digests(), f, indent=1)
        f.write("\n")
