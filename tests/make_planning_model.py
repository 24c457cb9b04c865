"""Writes tests/planning_model_mi355x.json: the planning model of the device
this runs on, i.e. its compute-unit count and, per kernel variant, the
workgroups per compute unit that the HIP occupancy query reports for the
variant's data-parallel kernel (gemm_variant_occupancy).  These are
properties of the device and of the compiled kernels (registers, LDS), not
results of any computation.  The CPU tests load the file into
gemm_set_planning_model to check the selection rules on a host without the
device; a GPU test checks that the file still matches the device.  Run on an
MI355X after the kernels change:

    python tests/make_planning_model.py
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))


def main() -> int:
    import torch

    import dense_gemm_11_amd as g

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    occ = {name: g.gemm_variant_occupancy(i) for i, name, _, _ in g.variants()}
    bad = [n for n, o in occ.items() if o <= 0]
    if bad:
        print(f"occupancy query failed for {bad}", file=sys.stderr)
        return 1
    model = {"device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
             "compute_units": props.multi_processor_count, "occupancy": occ}
    path = os.path.join(HERE, "planning_model_mi355x.json")
    with open(path, "w") as f:
        json.dump(model, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {path}: {len(occ)} variants, {props.multi_processor_count} compute units")
    return 0


if __name__ == "__main__":
    sys.exit(main())
