"""Fresh-process half of the resume test: load a step-64 checkpoint of the byte
LM into a new model and run steps 65-128, writing their records as JSON."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from bitwise_reproducible_fp32_amd import inputs as I  # noqa: E402
import bitwise_reproducible_fp32_amd as mlb  # noqa: E402
from test_gpu_model import run_gpu  # noqa: E402


def main():
    ck, out = sys.argv[1], sys.argv[2]
    cfg = I.make_config("c0")
    m = mlb.Model(cfg, I.init_params(cfg, seed=12345))   # different step-0 values: load must replace them
    with open(ck, "rb") as f:
        m.load(f.read())
    assert m.step == 64
    _, recs = run_gpu("c2", cfg, 64, model=m, start=65, data_name="c0")
    with open(out, "w") as f:
        json.dump(recs, f)
    print("resumed", len(recs), "steps", flush=True)


if __name__ == "__main__":
    main()
