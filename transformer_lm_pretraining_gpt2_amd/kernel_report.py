"""Per-kernel report of one profiled training step: time, MFMA utilisation and
achieved HBM bandwidth, from rocprofv3 runs of the same bench command.

Inputs (all from `python3 bench.py --steps S --warmup W --no-cpu-baseline
--copy-mib N` under rocprofv3):
  * a `--kernel-trace --stats` run: per-kernel call counts and durations;
  * a `--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32` run:
    MFMA FLOPs executed per dispatch (MOPS x 512, rocprofv3's own MfmaFlops
    definition; padded or masked tile work included), which over the traced
    duration and the dense MFMA peak gives the MFMA utilisation;
  * a `--pmc FETCH_SIZE` and a `--pmc WRITE_SIZE` run: HBM bytes per dispatch,
    scaled by what the counters read for the plain N MiB device copy (see
    traffic.py).
Achieved GB/s = (fetch + write bytes per dispatch) / average traced duration,
and its fraction of the 8 TB/s HBM peak (the roofline of the memory-bound
kernels: LayerNorm, cross-entropy, AdamW, reductions, embeddings).

    python -m transformer_lm_pretraining_gpt2_amd.kernel_report STATS_CSV MFMA_CSV FETCH_CSV WRITE_CSV \\
        --copy-mib 1024 --steps 7
"""
import argparse
import collections
import csv
import re

from transformer_lm_pretraining_gpt2_amd.config import (MI355X_BF16_PEAK_FLOPS, MI355X_FP32_MFMA_PEAK_FLOPS,
                                                        MI355X_HBM_BYTES_PER_S)
from transformer_lm_pretraining_gpt2_amd.traffic import COPY, read


def short(name):
    name = re.sub(r"gpt2k::\(anonymous namespace\)::", "", name)
    name = re.sub(r"_ZN5gpt2k12_GLOBAL__N_1\d+", "", name)
    name = re.sub(r"\(.*", "", name)
    return name[:90]


def per_dispatch(path):
    """{dispatch id: (kernel name, {counter: value})}; SQ counters summed over
    their instances, GRBM counters maxed (one clock per XCC)."""
    out = {}
    for r in csv.DictReader(open(path)):
        k = r["Dispatch_Id"]
        name, vals = out.setdefault(k, (r["Kernel_Name"], {}))
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        if c.startswith("GRBM"):
            vals[c] = max(vals.get(c, 0.0), v)
        else:
            vals[c] = vals.get(c, 0.0) + v
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("stats_csv")
    ap.add_argument("mfma_csv")
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--steps", type=float, required=True, help="training steps the traced run executed")
    ap.add_argument("--peak-bf16", type=float, default=MI355X_BF16_PEAK_FLOPS)
    ap.add_argument("--peak-f32", type=float, default=MI355X_FP32_MFMA_PEAK_FLOPS)
    ap.add_argument("--top", type=int, default=30)
    a = ap.parse_args(argv)

    stats = list(csv.DictReader(open(a.stats_csv)))
    mf = collections.defaultdict(list)  # executed MFMA work per dispatch, in seconds at peak
    for name, vals in per_dispatch(a.mfma_csv).values():
        mf[name].append(vals.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / a.peak_bf16 +
                        vals.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512 / a.peak_f32)
    (fetch, fetch_id), (write, write_id) = read(a.fetch_csv, "FETCH_SIZE"), read(a.write_csv, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    did, (_, cw) = max(((i, nv) for i, nv in write_id.items() if COPY in nv[0]), key=lambda t: t[1][1])
    cf = fetch_id[did][1]
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)

    tot = sum(float(r["TotalDurationNs"]) for r in stats)
    print(f"Kernel time per step: {tot / a.steps / 1e6:.3f} ms; counter scales: FETCH x{fs:.3f}, WRITE x{ws:.3f}\n")
    print("| ms/step | share | calls/step | avg us | MFMA util | HBM GB/s | HBM frac | kernel |")
    print("|---:|---:|---:|---:|---:|---:|---:|---|")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:a.top]:
        name, t, avg = r["Name"], float(r["TotalDurationNs"]), float(r["AverageNs"])
        u = mf.get(name)
        util = (sum(u) / len(u)) / (avg * 1e-9) if u and avg > 0 else None
        fb = [v for v, _ in fetch.get(name, [])]
        wb = [v for v, _ in write.get(name, [])]
        gbs = None
        if fb and wb and avg > 0:
            bytes_ = (sum(fb) / len(fb)) * 1024 * fs + (sum(wb) / len(wb)) * 1024 * ws
            gbs = bytes_ / avg  # bytes per ns = GB/s
        print(f"| {t / a.steps / 1e6:.3f} | {100 * t / tot:.1f}% | {int(r['Calls']) / a.steps:g} | {avg / 1e3:.1f} | "
              f"{'' if util is None or util < 0.005 else f'{100 * util:.1f}%'} | "
              f"{'' if gbs is None else f'{gbs:,.0f}'} | "
              f"{'' if gbs is None else f'{gbs * 1e9 / MI355X_HBM_BYTES_PER_S:.2f}'} | `{short(name)}` |")


if __name__ == "__main__":
    main()
