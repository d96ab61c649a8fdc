"""HBM traffic per launch of one kernel from two rocprofv3 counter runs.

The bench is run twice under rocprofv3, once collecting FETCH_SIZE and once
WRITE_SIZE (KiB per dispatch), with `bench.py --copy-mib N`, which performs
one plain device copy of N MiB before the steps.  The copy's readings against
its known size give one scale factor per counter; the kernel's readings,
averaged over its dispatches and scaled, give its HBM bytes per launch.  The
result is stored with a hash of the kernel source, so bench.py reports it only
while the kernel is unchanged.

    python -m transformer_lm_pretraining_gpt2_amd.traffic FETCH_CSV WRITE_CSV \\
        --copy-mib 1024 --kernel gemm_tn_f32 --workload gpt2_124m --out profiles/traffic.json
"""
import argparse
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel id -> (mangled-name fragments of the instantiations it launches for
# the GPT-2 124M bf16 workload, most workgroups per launch or None); a launch
# of any of them counts as one launch
KERNELS = {
    # a layer's four weight gradients in one grouped launch: the 8-wave 256x256
    # tile, BK = 32, each product split over the reduction so the group makes
    # one round of at most one block per CU (the tied head's weight gradient
    # is a separate, ungrouped kernel)
    "gemm_tn_f32": (["gemm_group_kernelIDF16bLi256ELi256ELi32ELi2ELi4ELi1ELi1ELi4E"], None),
    "attn_bwd_dkv": (["attn_dkv_kernelIDF16bLi64E"], None),
}
COPY = "copyBuffer"  # the runtime's device-to-device copy kernel, used by dst.copy_(src)


def read(path, counter):
    out, by_id = {}, {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        blocks = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
        out.setdefault(r["Kernel_Name"], []).append((float(r["Counter_Value"]), blocks))
        by_id[r["Dispatch_Id"]] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return out, by_id


def per_dispatch(rows, spec):
    frags, max_blocks = spec
    vals = [v for name, vs in rows.items() if any(f in name for f in frags)
            for v, blocks in vs if max_blocks is None or blocks <= max_blocks]
    if not vals:
        raise SystemExit(f"no dispatch matching {frags}")
    return sum(vals) / len(vals), len(vals)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--kernel", default="gemm_tn_f32")
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash

    (fetch, fetch_id), (write, write_id) = read(a.fetch_csv, "FETCH_SIZE"), read(a.write_csv, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    # the calibration copy: the copy dispatch writing the most, and the same
    # dispatch (same position in the run) in the fetch run
    did, (_, cw) = max(((i, nv) for i, nv in write_id.items() if COPY in nv[0]), key=lambda t: t[1][1])
    name, cf = fetch_id[did]
    if COPY not in name:
        raise SystemExit("the two runs do not line up on the calibration copy")
    f_scale, w_scale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    kf, nf = per_dispatch(fetch, KERNELS[a.kernel])
    kw, nw = per_dispatch(write, KERNELS[a.kernel])
    entry = {
        "bytes_per_launch": kf * 1024 * f_scale + kw * 1024 * w_scale,
        "fetch_bytes_per_launch": kf * 1024 * f_scale,
        "write_bytes_per_launch": kw * 1024 * w_scale,
        "fetch_kib_raw": kf, "write_kib_raw": kw, "dispatches": [nf, nw],
        "copy_mib": a.copy_mib, "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "source_hash": kernel_source_hash(a.kernel),
    }
    d = json.load(open(a.out)) if os.path.exists(a.out) else {}
    d.setdefault(a.workload, {})[a.kernel] = entry
    with open(a.out, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


if __name__ == "__main__":
    main()
