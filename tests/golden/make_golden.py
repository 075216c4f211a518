"""Write the stored expected values under tests/golden/.

Every value here comes from the fp64 oracle (``oracle/``) run on the seeded
inputs of ``workloads.py``; nothing comes from the GPU path.  The pages print
no worked example, so these fixtures guard the oracle against drift and give
the GPU tests a fixed expectation for the 1x64x16x4 workload.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.get("tiny_fwd")
    inp = workloads.make_inputs(w)
    y, hT = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], nthreads=1)
    doc = {
        "what": "fp64 oracle forward of the tiny workload (B=1, T=64, D=16, DS=4, fp32 inputs, "
                "A[d,n] = -(n+1), h0 = 0, delta = softplus(N(-1,1)), seed 1)",
        "definition": "pssa-100m/pssa_kernels.py page, module docstring: "
                      "h_t = exp(delta_t A) h_{t-1} + delta_t b_t x_t, y_t = <h_t, c_t>",
        "written_by": "tests/golden/make_golden.py (calls only oracle/)",
        "workload": w.name,
        "shape": {"B": w.B, "T": w.T, "D": w.D, "DS": w.DS},
        "y": [float(v) for v in y.ravel()],
        "hT": [float(v) for v in hT.ravel()],
    }
    with open(os.path.join(HERE, "tiny_fwd_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
