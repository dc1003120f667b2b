"""The oracle still gives its recorded answer on the tiny workload
(tests/golden/cfg0_oracle.json, written by make_oracle_golden.py from the
oracle alone)."""
import hashlib
import json
import os

import oracle
from moe_expert_ffn_route_amd import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cfg0_oracle.json")


def test_oracle_matches_recorded_fixture():
    with open(GOLD) as f:
        g = json.load(f)
    r = oracle.forward(synth.workload_case(0), trace=True)
    P = r["P"]
    h = lambda a: hashlib.sha256(a.tobytes()).hexdigest()
    assert r["expert_token_nums"].tolist() == g["expert_token_nums"]
    assert r["sorted_pair"].tolist() == g["sorted_pair"]
    assert h(r["q_x"][:P]) == g["q_x_sha256"]
    assert h(r["acc1"][:P]) == g["acc1_sha256"]
    assert h(r["q_h"][:P]) == g["q_h_sha256"]
    assert h(r["acc2"][:P]) == g["acc2_sha256"]
    assert h(r["output"]) == g["output_bf16_sha256"]
