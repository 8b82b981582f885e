"""Write contract_identity.json: the library's contract digests for every admitted (C, d_k).

A change of these digests means the contract text changed; rerun this script only then,
and say in the commit which reading of the pages changed.
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from bitwise_consistent_linear_amd import api  # noqa: E402

if __name__ == "__main__":
    ids = {f"{c},{d}": api.contract_identity(c, d).hex()
           for c in (16, 32, 64, 128, 256) for d in (16, 32, 64, 128)}
    with open(os.path.join(HERE, "contract_identity.json"), "w") as f:
        json.dump({"about": "SHA-256 of gdn_contract_string(chunk, d_k), keyed 'chunk,d_k'",
                   "identities": ids}, f, indent=1)
        f.write("\n")
