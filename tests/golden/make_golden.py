"""Write the golden fixtures in this folder.

Every value here is transcribed from the pages (cited in each fixture's
"source" field); nothing is computed by the HIP path or by the oracle.
Run: python tests/golden/make_golden.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    s3 = math.sqrt(3.0)
    fixtures = {
        "mod3_rotation.json": {
            "source": "DeltaProduct study notes (arXiv 2502.10297v7), sec. 2.4 'why products can "
                      "express rotations': teaching example of mod-3 counting with two reflections "
                      "(principle Fig.3; construction App.B.2)",
            "k1": [1.0, 0.0],
            "k2": [0.5, s3 / 2.0],
            "beta": 2.0,
            "B_i": "zero (no write)",
            "F2F1_printed": [[-0.5, -s3 / 2.0], [s3 / 2.0, -0.5]],
            "rotation_degrees": 120.0,
            "start_state": [1.0, 0.0],
            "period_tokens": 3,
        },
        "osdn_teaching_example.json": {
            "source": "OSDN study notes (arXiv 2605.13473v1), sec. 2.4 teaching example (not a paper "
                      "experiment): one-step residual ratio q = (1 - a)^2 with a = beta <d, k*k>",
            "k": [1.0, 0.0],
            "beta": 0.5,
            "cases": [{"d": [1.0, 1.0], "q": 0.25}, {"d": [1.5, 1.0], "q": 0.0625}],
        },
        "osdn_oscillation.json": {
            "source": "OSDN study notes (arXiv 2605.13473v1), sec. 3.3 (App.D.4): K = V = 1, "
                      "k_t = 1, v_t = (-1)^t; even with exact writes S_t oscillates between -1 and +1",
            "K": 1,
            "V": 1,
            "k": 1.0,
            "beta_exact_write": 1.0,
            "v_rule": "(-1)^t, t = 1, 2, ...",
            "S_rule": "(-1)^t",
        },
    }
    for name, fx in fixtures.items():
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fx, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
