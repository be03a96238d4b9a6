"""Writes the expected prompt-key gradients of the P = 32768 and P = 131072 workloads.

Calls only the fp64 oracle (oracle.prompt_key_grads) on the seeded inputs of
workloads.make_inputs; the GPU parity test compares the library's dK_P / dV_P at these keys.
For one key/value head, 4096 prompt keys are sampled so that every 256-key block (the
workgroup tile of the prompt K/V gradient kernels) and so every row chunk of the prefill K/V
gradient walk is covered: each block's first and last key, the keys either side of its
32-key wave boundary, and further keys drawn from a seeded generator.

Run from the repository root:  python tests/golden/make_prompt_key_grads.py [4] [5]
(about 2 minutes for the P = 32768 tree and 15 to 20 for the P = 131072 tree on 8 cores).
"""
from __future__ import annotations

import os
import random
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import prompt_key_grads  # noqa: E402
from workloads import make_inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
PLAN = {4: dict(kv_head=3, per_block=32), 5: dict(kv_head=6, per_block=8)}
NAMES = ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r"]


def fingerprint(w):
    """fp64 sums of every input tensor: the test checks that it regenerated the same inputs."""
    return np.array([float(getattr(w, n).double().sum()) for n in NAMES] +
                    [float(getattr(w, n).double().abs().sum()) for n in NAMES], dtype=np.float64)


def sample_keys(P: int, per_block: int, seed: int):
    rng = random.Random(seed)
    keys = []
    for b0 in range(0, P, 256):
        b1 = min(P, b0 + 256)
        pick = {b0, b1 - 1}
        if per_block >= 4 and b1 - b0 > 33:
            pick |= {b0 + 31, b0 + 32}
        rest = [j for j in range(b0, b1) if j not in pick]
        pick |= set(rng.sample(rest, min(len(rest), per_block - len(pick))))
        keys.extend(sorted(pick))
    return keys


def main(cfgs):
    torch.set_num_threads(min(8, os.cpu_count() or 1))
    for cfg in cfgs:
        plan = PLAN[cfg]
        t0 = time.time()
        w = make_inputs(cfg)
        keys = sample_keys(w.shape.P, plan["per_block"], 20260600 + cfg)
        g = prompt_key_grads(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, keys, w.do_p, w.do_r,
                             kv_heads=[plan["kv_head"]], slab=256)
        out = os.path.join(HERE, f"prompt_key_grads_cfg{cfg}.npz")
        np.savez_compressed(out, cfg=np.int32(cfg), kv_head=np.int32(plan["kv_head"]),
                            keys=g["keys"].numpy().astype(np.int32),
                            dk_p=g["dk_p"][:, 0].numpy().astype(np.float32),
                            dv_p=g["dv_p"][:, 0].numpy().astype(np.float32),
                            fingerprint=fingerprint(w), offsets=np.array(w.shape.offsets, dtype=np.int64))
        print(f"config {cfg}: {len(keys)} keys of kv head {plan['kv_head']} in {time.time() - t0:.0f} s -> {out}",
              flush=True)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [4, 5])
