"""CPU check that every repository path the documentation names exists
(profiles, sources, tests), so a renamed or removed file cannot leave a
dangling reference behind."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DOCS = ["DESIGN.md", "README.md", os.path.join("profiles", "INDEX.md")]
# backquoted repository paths: a known top-level folder, then a file name
PATH = re.compile(r"`((?:profiles|tests|oracle|include|moe_expert_ffn_route_amd)/[A-Za-z0-9_./-]+\.(?:md|py|c|h|hip|txt|json))`")
# kernel sources named relative to the package, and test files by name
CSRC = re.compile(r"`(csrc/[A-Za-z0-9_]+\.(?:hip|h))`")
TEST = re.compile(r"`(test_[A-Za-z0-9_]+\.py)`")


def named_paths():
    out = set()
    for d in DOCS:
        with open(os.path.join(ROOT, d), encoding="utf-8") as f:
            text = f.read()
        out |= {(d, m) for m in PATH.findall(text)}
        out |= {(d, "moe_expert_ffn_route_amd/" + m) for m in CSRC.findall(text)}
        out |= {(d, "tests/" + m) for m in TEST.findall(text)}
    return out


def test_documented_paths_exist():
    paths = named_paths()
    assert len(paths) > 10
    missing = sorted(f"{doc}: {p}" for doc, p in paths if not os.path.exists(os.path.join(ROOT, p)))
    assert not missing, missing


def test_profile_index_lists_every_profile():
    with open(os.path.join(ROOT, "profiles", "INDEX.md"), encoding="utf-8") as f:
        index = f.read()
    stems = {re.sub(r"__.*", "", n) for n in os.listdir(os.path.join(ROOT, "profiles")) if n != "INDEX.md"}
    for stem in stems:
        assert stem in index, stem
