"""Turns the parity report that the GPU suite writes (SPECV_PARITY_REPORT=<file>.json) into a
markdown table: one line per comparison against the oracle, with the sequences compared and
the near-boundary cases counted by kind.

    python tests/parity_report.py <report.json> "<command that produced it>" ["<build>"] > <summary.md>

The kinds: "acceptance" = an acceptance test whose uniform lies within 1e-5 of min(1, p/q);
"topp" = a drafted token whose probability lies within 1e-5 of a top-p cut on p or q; "draw"
= a residual or bonus draw whose uniform lies within 1e-5 of a cumulative-mass boundary;
"draw_topp" = the drawn row's own top-p cut within 1e-5; "expansion" (tree drafting) = a
top-k choice between candidates whose fp64 path scores differ by less than 1e-12. Decisions
before a sequence's first such case are compared exactly; after it only validity is checked.
"""
import json
import sys

CONFIGS = (("c1 ", "C1 Markov B=1 gamma=4 V=4"), ("c2 ", "C2 B=64 gamma=4 V=32000"),
           ("c3 ", "C3 B=256 gamma=8 V=128256 top-p"), ("c4 ", "C4 tree B=128 V=151936 + KV"),
           ("c5 ", "C5 ragged B=1024 V=128256"))


def main(path, command, build=""):
    rep = json.load(open(path))
    ent = rep["entries"]
    kinds = sorted({k for e in ent for k in e["boundary"]})
    print("# Parity against the fp64 oracle: near-boundary cases per comparison\n")
    print(f"Command (GPU suite, one process, exit status {rep['exitstatus']}):\n")
    print(f"    {command}\n")
    if build:
        print(f"Build: {build}\n")
    print("A comparison with no near-boundary case matched the oracle exactly: tokens, "
          "accepted counts, committed lengths and bytes bit for bit, probabilities within "
          "1e-5. A near-boundary case (margin below 1e-5) is compared up to that decision and "
          "checked for validity after it.\n")
    print("A draw is counted near its boundary when its uniform lies within 1e-5 of the "
          "cumulative mass before or after the drawn token. Without a cut, at V=128256, most "
          "tokens carry less than 2e-5 of the mass, so a good share of whole-row draws are "
          "counted (C5); the tests bound the count by its expectation, the sum over draws of "
          "min(1, 2e-5 / w) for the drawn token's mass w, plus slack.\n")
    print("\"Disagreeing\" counts the near-boundary cases whose GPU result after that decision "
          "differs from the oracle's (accepted count, emitted count or tokens); blank where the "
          "comparison does not count it.\n")
    dis = lambda e: str(e["disagreed"]) if "disagreed" in e else ""  # noqa: E731
    print("## The five configurations\n")
    print("| config | comparison | sequences / rounds | near-boundary cases | disagreeing |")
    print("|---|---|---|---|---|")
    for prefix, name in CONFIGS:
        for e in ent:
            if e["label"].lower().startswith(prefix):
                b = ", ".join(f"{k} {v}" for k, v in e["boundary"].items() if v) or "none"
                print(f"| {name} | {e['label']} ({e['kind']}) | {e['sequences']} | {b} | "
                      f"{dis(e)} |")
    print("\n## Every comparison\n")
    print("| comparison | kind | sequences | " + " | ".join(kinds) + " | disagreeing |")
    print("|---|---|---|" + "---|" * (len(kinds) + 1))
    for e in ent:
        cells = " | ".join(str(e["boundary"].get(k, "")) for k in kinds)
        print(f"| {e['label']} | {e['kind']} | {e['sequences']} | {cells} | {dis(e)} |")
    tot = {k: sum(e["boundary"].get(k, 0) for e in ent) for k in kinds}
    seqs = sum(e["sequences"] for e in ent)
    tdis = sum(e.get("disagreed", 0) for e in ent)
    print(f"| **total** ({len(ent)} comparisons) | | {seqs} | "
          + " | ".join(str(tot[k]) for k in kinds) + f" | {tdis} |")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "", sys.argv[3] if len(sys.argv) > 3 else "")
