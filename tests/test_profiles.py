"""The rocprofv3 summaries under profiles/ name the commands that made them;
each must run committed files only, with options bench.py still accepts."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith(".md"))


def _bench_options():
    src = open(os.path.join(ROOT, "bench.py")).read()
    return set(re.findall(r'add_argument\(\s*"(--[a-z0-9-]+)"', src))


def _commands(text):
    """Shell commands of the fenced blocks, continuation lines joined and a
    B="..." assignment substituted where $B is used."""
    cmds = []
    for block in re.findall(r"```\n(.*?)```", text, flags=re.S):
        joined = re.sub(r"\\\n\s*", " ", block)
        assigns = dict(re.findall(r'^(\w+)="([^"]*)"', joined, flags=re.M))
        for line in joined.splitlines():
            line = line.strip()
            if not line or re.match(r'^\w+="', line):
                continue
            for k, v in assigns.items():
                line = line.replace("$" + k, v)
            cmds.append(line)
    return cmds


def test_every_profile_has_a_command():
    assert PROFILES
    for name in PROFILES:
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert any("rocprofv3" in c for c in _commands(text)), name


@pytest.mark.parametrize("name", PROFILES)
def test_profile_commands_run_committed_files(name):
    text = open(os.path.join(ROOT, "profiles", name)).read()
    opts = _bench_options()
    for cmd in _commands(text):
        if "rocprofv3" not in cmd:
            continue
        prog = cmd.split(" -- ", 1)[1].split()
        assert prog[0] in ("python3", "python"), cmd
        rel = prog[1].replace("$R/", "")
        assert not rel.startswith(("_work", "gpurun_out")), cmd
        assert os.path.isfile(os.path.join(ROOT, rel)), cmd
        if rel == "bench.py":
            for tok in prog[2:]:
                if tok.startswith("--"):
                    assert tok in opts, f"{name}: bench.py has no option {tok}"
