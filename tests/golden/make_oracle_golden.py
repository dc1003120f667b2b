"""Write the oracle's own regression fixture for the tiny workload (T=8,
hidden 512, intermediate 256, 8 experts, top-2). It calls only the CPU oracle
and the seeded input generator; the pages print no worked numerical example of
the MoE block, so this fixture records the oracle's present answer, and any
later change to it must name the passage that justifies the new arithmetic.

Run from the repository root:  python tests/golden/make_oracle_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_expert_ffn_route_amd import synth  # noqa: E402


def digest(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def main():
    case = synth.workload_case(0)
    r = oracle.forward(case, trace=True)
    P = r["P"]
    rec = {
        "workload": "tiny_w8a8_moe T=8 H=512 I=256 E=8 K=2 seed=1234",
        "expert_token_nums": r["expert_token_nums"].tolist(),
        "sorted_pair": r["sorted_pair"].tolist(),
        "output_bf16_sha256": digest(r["output"]),
        "output_row0_first8_bf16": [int(v) for v in r["output"][0, :8]],
        "q_x_sha256": digest(r["q_x"][:P]),
        "acc1_sha256": digest(r["acc1"][:P]),
        "q_h_sha256": digest(r["q_h"][:P]),
        "acc2_sha256": digest(r["acc2"][:P]),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg0_oracle.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
