"""Markdown summary of a rocprofv3 `--kernel-trace --stats --output-format csv`
kernel_stats.csv: per-kernel time per step, share, calls and average.

    python -m transformer_lm_pretraining_gpt2_amd.profile_summary STATS_CSV --steps N [--top 25]
"""
import argparse
import csv
import re


def short(name):
    name = re.sub(r"gpt2k::\(anonymous namespace\)::", "", name)
    name = re.sub(r"_ZN5gpt2k12_GLOBAL__N_1\d+", "", name)
    return name[:110]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("stats_csv")
    ap.add_argument("--steps", type=float, required=True, help="training steps the profiled run executed")
    ap.add_argument("--top", type=int, default=25)
    a = ap.parse_args(argv)
    rows = list(csv.DictReader(open(a.stats_csv)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"Kernel time per step: {tot / a.steps / 1e6:.3f} ms (sum over {len(rows)} kernels)\n")
    print("| ms/step | share | calls/step | avg us | kernel |")
    print("|---:|---:|---:|---:|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:a.top]:
        t = float(r["TotalDurationNs"])
        print(f"| {t / a.steps / 1e6:.3f} | {100 * t / tot:.1f}% | {int(r['Calls']) / a.steps:g} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | `{short(r['Name'])}` |")


if __name__ == "__main__":
    main()
