"""Helpers of the GPU parity tests: device copies of the seeded inputs, one
walk through the C ABI, and an optional JSON-lines report of what each
full-size check covered (set DSW_PARITY_REPORT to a file path)."""
import json
import os
import sys

import numpy as np

DEV = "cuda:0"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def report(record: dict) -> None:
    path = os.environ.get("DSW_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def int8_dev(torch, Q, scale):
    return torch.from_numpy(np.ascontiguousarray(Q)).to(DEV), torch.from_numpy(scale).to(DEV)


def round_dev(torch, inp):
    return (bf16_dev(torch, inp["base"]), torch.from_numpy(inp["anchor"]).to(DEV),
            torch.from_numpy(inp["T"]).to(DEV), torch.from_numpy(inp["uniforms"]).to(DEV))


def logits_host(torch, logits):
    return logits.view(torch.int16).cpu().numpy().view(np.uint16)


def run(torch, walker, W1d, W2d, inp, want_logits=True, scale=None, check_status=True):
    base, anchor, T, uni = round_dev(torch, inp)
    tokens, logits = walker.walk(W1d, W2d, base, anchor, T, uni, w2_scale=scale, want_logits=want_logits)
    torch.cuda.synchronize()
    if check_status:
        st = walker.status()
        assert st == 0, f"device status {st}"
    lg = None if logits is None else logits_host(torch, logits)
    return tokens.cpu().numpy(), lg
