"""The commands quoted in profiles/ must run committed files with valid arguments.

Each summary under profiles/ gives the rocprofv3 and bench.py commands that
produced its figures.  These checks keep them runnable: every script they
name exists in the repository (outside the ignored working folder), every
`bench.py --only` leg and digest name is one bench.py knows, and every
counter pass stays within what one rocprofv3 pass can collect on this chip
(8 SQ counters, 4 TCC counters with FETCH_SIZE taking 3 and WRITE_SIZE 2,
2 GRBM counters), without a trace domain beside --pmc.
"""
import os
import re
import shlex

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# Trace options that may not share a run with --pmc.
TRACE_OPTS = {"-s", "--sys-trace", "-r", "--runtime-trace", "--hip-trace", "--hsa-trace", "--memory-copy-trace",
              "--scratch-memory-trace", "--marker-trace"}
# TCC counters each derived counter occupies.
TCC_COST = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}


def commands():
    """(file, line) for every line inside a fenced code block of a summary."""
    out = []
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        inside = False
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                if line.strip().startswith("```"):
                    inside = not inside
                    continue
                if inside and line.strip():
                    out.append((name, line.strip()))
    return out


def bench_choices():
    src = open(os.path.join(ROOT, "bench.py")).read()
    m = re.search(r'"--only".*?choices=\[(.*?)\]', src, re.S)
    assert m, "bench.py declares its --only legs"
    return set(re.findall(r'"([a-z0-9_]+)"', m.group(1)))


def test_every_summary_quotes_its_commands():
    names = [n for n in os.listdir(PROFILES) if n.endswith(".md")]
    assert names
    with_cmds = {f for f, _ in commands()}
    assert set(names) <= with_cmds, f"summaries without a command block: {sorted(set(names) - with_cmds)}"


def test_quoted_scripts_are_committed_files():
    seen = 0
    for f, line in commands():
        for tok in shlex.split(line.replace("$", "")):
            if tok.endswith(".py") and not tok.startswith("-"):
                seen += 1
                assert not tok.startswith("_work"), f"{f}: {line} runs a working file"
                assert os.path.isfile(os.path.join(ROOT, tok)), f"{f}: {tok} is not in the repository"
    assert seen > 0


def test_bench_legs_and_digest_names_exist():
    legs = bench_choices()
    names = set(bench.TRAFFIC_KERNELS)
    for f, line in commands():
        toks = shlex.split(line)
        for i, tok in enumerate(toks[:-1]):
            nxt = toks[i + 1]
            if nxt.startswith("$"):
                continue
            if tok == "--only":
                assert nxt in legs, f"{f}: unknown bench leg {nxt}"
            if tok in ("--digest-traffic", "--digest-cycles"):
                assert nxt in names, f"{f}: unknown kernel entry {nxt}"


def test_counter_passes_fit_one_rocprofv3_run():
    passes = 0
    for f, line in commands():
        if "rocprofv3" not in line or "--pmc" not in line:
            continue
        toks = shlex.split(line)
        prof = toks[toks.index("rocprofv3"):]
        if "--" in prof:
            prof = prof[:prof.index("--")]
        assert not TRACE_OPTS & set(prof), f"{f}: --pmc beside a trace domain: {line}"
        i = prof.index("--pmc") + 1
        counters = []
        while i < len(prof) and not prof[i].startswith("-"):
            counters.append(prof[i])
            i += 1
        if any(c.startswith("$") for c in counters):
            continue
        passes += 1
        sq = sum(c.startswith("SQ_") for c in counters)
        grbm = sum(c.startswith("GRBM_") for c in counters)
        tcc = sum(TCC_COST.get(c, 1 if c.startswith("TCC_") else 0) for c in counters)
        assert sq <= 8 and grbm <= 2 and tcc <= 4, f"{f}: too many counters for one pass: {counters}"
    assert passes > 0
