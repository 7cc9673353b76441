"""Writes the stored expected values of the end-to-end parity tests.

Every value here comes from the CPU oracle (oracle/), run on the seeded inputs
of bitwise_reproducible_fp32_amd.inputs; nothing is taken from the HIP path.
Usage: python tests/golden/make_golden.py c0 c2 c3 c4 tables [--threads N]
(c4, two full steps of the 162M decoder, takes about three hours per step on 8 threads.)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from bitwise_reproducible_fp32_amd import inputs as I  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE_SEED = 20241


def hx(x) -> str:
    return np.float32(x).tobytes()[::-1].hex()


def sha(a: np.ndarray) -> str:
    return oracle.sha256(np.ascontiguousarray(a).tobytes())


def run(name: str, cfg: dict, steps: int, model=None, start: int = 1, log=None, log_micro=False):
    m = model or oracle.Model(cfg, I.init_params(cfg))
    recs = []
    for s in range(start, start + steps):
        t0 = time.time()
        losses = []
        for mb in range(cfg["micro"]):
            x, y = I.batch_for(name if name != "c2" else "c0", cfg, s, mb)
            losses.append(m.forward(x, y))
            m.backward()
            if log and log_micro:
                log(f"{name} step {s} micro-batch {mb} loss {float(losses[-1]):.6f} {time.time() - t0:.1f}s")
        grad = sha(m.grad)
        lr = I.lr_at(name if name != "c2" else "c0", s)
        m.adamw(lr)
        rec = dict(step=s, lr=hx(lr), losses=[hx(l) for l in losses], grad=grad, params=sha(m.params),
                   adam_m=sha(m.adam_m), adam_v=sha(m.adam_v), ckpt=oracle.sha256(m.save()))
        recs.append(rec)
        if log:
            log(f"{name} step {s} loss0 {float(losses[0]):.6f} {time.time() - t0:.1f}s")
    return m, recs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("configs", nargs="+")
    ap.add_argument("--threads", type=int, default=1)
    a = ap.parse_args()
    oracle.set_threads(a.threads)
    for name in a.configs:
        t0 = time.time()
        if name == "c0":
            cfg = I.make_config("c0")
            _, recs = run("c0", cfg, 4, log=print)
            out = dict(config="c0", cfg=cfg, init_seed=I.INIT_SEED, steps=recs)
        elif name == "c2":
            cfg = I.make_config("c0")
            _, full = run("c2", cfg, 128)
            half, first = run("c2", cfg, 64)
            blob = half.save()
            fresh = oracle.Model(cfg, I.init_params(cfg, seed=1))
            fresh.load(blob)
            _, second = run("c2", cfg, 64, model=fresh, start=65)
            assert first + second == full, "resume identity failed in the oracle"
            out = dict(config="c2", cfg=cfg, init_seed=I.INIT_SEED, steps=full,
                       ckpt_step64=oracle.sha256(blob))
        elif name == "c3":
            cfg = I.make_config("c3")
            _, recs = run("c3", cfg, 3, log=print)
            out = dict(config="c3", cfg=cfg, init_seed=I.INIT_SEED, steps=recs)
        elif name == "tables":
            # Digests of the bytes that come from the host's binary64 libm (the
            # rotary tables and the profile's seeded step-0 parameters) and of
            # the seeded input parameters, per config: a host whose libm or
            # numpy rounds one value differently fails against these loudly.
            out = dict(config="tables", seed=TABLE_SEED, steps=[])
            for c in ("c0", "c3", "c4"):
                cfg = I.make_config(c)
                cs, sn = oracle.rope_table(cfg["seq_len"], cfg["head_dim"], cfg["rope_theta"])
                out[c] = dict(rope_cos=sha(cs), rope_sin=sha(sn),
                              seeded_params=sha(oracle.seed_params(cfg, TABLE_SEED)),
                              init_params=sha(I.init_params(cfg)))
                print(c, out[c], flush=True)
        elif name == "c4":
            # Steps 1 and 2 of the 162M decoder; the record is rewritten after
            # each step so that step 1 is kept if step 2 is cut short.
            cfg = I.make_config("c4")
            model, recs = None, []
            for s in (1, 2):
                model, rec = run("c4", cfg, 1, model=model, start=s,
                                 log=lambda t: print(t, flush=True), log_micro=True)
                recs += rec
                part = dict(config="c4", cfg=cfg, init_seed=I.INIT_SEED, steps=recs,
                            oracle_threads=a.threads)
                with open(os.path.join(HERE, "c4.json"), "w") as f:
                    json.dump(part, f, indent=1)
            out = dict(config="c4", cfg=cfg, init_seed=I.INIT_SEED, steps=recs)
        else:
            raise SystemExit(f"unknown config {name}")
        out["oracle_threads"] = a.threads
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(out, f, indent=1)
        print(f"{name}: wrote {len(out['steps'])} steps in {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
