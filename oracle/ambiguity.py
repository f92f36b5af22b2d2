"""How often a verify decision lies within a window of its boundary (oracle only).

TEST INFRASTRUCTURE: run by hand; imports the oracle and the workload generators.

For each sampling workload, counts the rows whose draw margin (distance of u
from the ends of the chosen token's interval of the normalised CDF) or accept
margin (|r - alpha|) is below the window. This fraction is a property of the
inputs: at vocabularies of 10^4-10^5 tokens many tokens carry more mass than the
window, so a uniform often lands near one of them.

    python -m oracle.ambiguity [--window 1e-6] [--rounds 1:200,2:40,3:4,4:1]
"""
from __future__ import annotations

import argparse

from oracle.verify import oracle_sample
from workloads import make_sample_inputs


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--window", type=float, default=1e-6)
    ap.add_argument("--rounds", default="1:200,2:40,3:4,4:1")
    a = ap.parse_args()
    for item in a.rounds.split(","):
        cfg, rounds = (int(x) for x in item.split(":"))
        rows = draw = acc = 0
        for rnd in range(rounds):
            s = make_sample_inputs(cfg, rnd)
            r = oracle_sample(s.target_f32(), s.draft_f32(), s.draft_tokens, s.uniforms, s.temperature,
                              with_probs=False)
            rows += len(r.n_accepted)
            draw += int((r.draw_margin < a.window).sum())
            acc += int((r.accept_margin.min(axis=1) < a.window).sum())
        print(f"workload {cfg}: rows {rows}  draw margin < {a.window:g}: {draw / rows:.4f}  "
              f"accept margin < {a.window:g}: {acc / rows:.4f}", flush=True)


if __name__ == "__main__":
    main()
