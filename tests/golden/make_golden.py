"""Write tests/golden/tiny_oracle.json from the CPU oracle only.

Run: python tests/golden/make_golden.py
The fixture records digests and a few values of the oracle's outputs on the
tiny workload (A [16,256] ~ N(0,1), W [256,256] ~ N(0,0.02), seed 0, group 64),
so later changes to the oracle's arithmetic show up as a test failure.
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from w4a8_quantized_gemm_quantize_amd import inputs  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    a, w, spec = inputs.workload_inputs("tiny", seed=0)
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    a_q, a_s, acc, y = oracle.w4a8_gemm_bf16act(a, q, sg, sch, 64)
    qa32, sa32 = oracle.quantize_act_blockwise(a, 32)
    return {
        "inputs_sha256": {"a_bf16": digest(a), "w_bf16": digest(w)},
        "act_per_token": {"q_sha256": digest(a_q), "scales_hex": [float(v).hex() for v in a_s]},
        "act_block32": {"q_sha256": digest(qa32), "scales_sha256": digest(sa32)},
        "weights": {"q_sha256": digest(q), "s_g_sha256": digest(sg), "s_ch_sha256": digest(sch),
                    "s_g_histogram": np.bincount(sg.reshape(-1), minlength=17).tolist()},
        "gemm": {"acc_sha256": digest(acc), "acc_first_row": acc[0, :8].tolist(),
                 "y_first_row_hex": [float(v).hex() for v in y[0, :8]]},
    }


if __name__ == "__main__":
    out = compute()
    out["_about"] = ("Written by tests/golden/make_golden.py from the CPU oracle on the tiny "
                     "workload (seed 0); regression fixture for the oracle's arithmetic.")
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print("wrote tiny_oracle.json")
