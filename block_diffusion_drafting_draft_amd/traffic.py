"""HBM traffic of a kernel from rocprofv3 counter runs, scaled by a plain copy of known size.

Two `rocprofv3 --pmc` runs of the benchmark give the derived counters FETCH_SIZE and WRITE_SIZE
(KiB per dispatch) of every dispatch; two more runs of `bench.py --copy-calibration MIB` give the same
counters for a device-to-device copy of MIB MiB. The copy reads and writes exactly that many bytes,
so bytes = KiB_kernel * copy_bytes / KiB_copy per counter. The record is written as JSON together
with the SHA-256 prefix of the attention source it was measured on; bench.py reports it only while
that source is unchanged.

  python -m block_diffusion_drafting_draft_amd.traffic --workload NAME --kernel attn_kernel \
      --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --out OUT.json
"""

import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))


KERNEL_SOURCES = ("attn.hip", "attn_tiles.h")  # the attention kernel's source text


def source_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def per_dispatch(path, counter, name_part):
    """Counter value of every dispatch whose kernel name contains name_part (summed over the
    counter's instances within one dispatch)."""
    vals = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter or name_part not in row["Kernel_Name"]:
                continue
            key = row["Dispatch_Id"]
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named like {name_part!r}")
    return list(vals.values())


def main():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--workload", required=True)
    p.add_argument("--kernel", default="attn_kernel")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", required=True)
    p.add_argument("--copy-write", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--copy-kernel", default="copyBuffer")
    p.add_argument("--out", required=True)
    a = p.parse_args()
    f_k = statistics.median(per_dispatch(a.fetch, "FETCH_SIZE", a.kernel))
    w_k = statistics.median(per_dispatch(a.write, "WRITE_SIZE", a.kernel))
    f_c = statistics.median(per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel))
    w_c = statistics.median(per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel))
    sf, sw = a.copy_bytes / (f_c * 1024.0), a.copy_bytes / (w_c * 1024.0)
    rec = {
        "workload": a.workload,
        "kernel": a.kernel,
        "source_digest": source_digest(),
        "fetch_kib_per_dispatch": f_k,
        "write_kib_per_dispatch": w_k,
        "copy_bytes": a.copy_bytes,
        "copy_fetch_kib": f_c,
        "copy_write_kib": w_c,
        "fetch_scale": sf,
        "write_scale": sw,
        "bytes_per_launch": round(f_k * 1024.0 * sf + w_k * 1024.0 * sw),
    }
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
