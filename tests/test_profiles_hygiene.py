"""The committed rocprofv3 summaries are short text that names, for each figure, the command
that made it; that command runs committed files only (bench.py from the repository root),
and nothing under profiles/ is raw profiler output or runnable."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _summaries():
    names = sorted(os.listdir(PROFILES))
    assert names, "no profile summaries"
    return names


def test_only_short_text_summaries():
    for name in _summaries():
        assert name.endswith((".md", ".txt")), name
        assert os.path.getsize(os.path.join(PROFILES, name)) < 16 * 1024, name


def test_each_summary_names_a_committed_command():
    for name in _summaries():
        text = open(os.path.join(PROFILES, name)).read()
        cmds = re.findall(r"^rocprofv3 .*$", text, flags=re.M)
        assert cmds, f"{name}: no rocprofv3 command"
        for c in cmds:
            prog = c.split(" -- ", 1)
            assert len(prog) == 2, f"{name}: no program after --: {c}"
            assert prog[1].startswith("python3 bench.py"), f"{name}: {c}"
            assert "_work" not in c and "/root/reference" not in c, f"{name}: {c}"


def test_summaries_are_named_for_kind_and_workload():
    from virtual_expert_routed_amd import configs
    workloads = {c.name for c in configs.CONFIGS}
    for name in _summaries():
        m = re.match(r"^(kernel_trace|pmc_traffic)_(.+)\.md$", name)
        assert m and m.group(2) in workloads, name
