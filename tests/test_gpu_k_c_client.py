"""The library driven from plain C on the GPU: tests/c_client/step_client, a
C99 program linked against libzero_shard.so and the HIP runtime only (no
Python, no torch in its process), runs check -> decision -> step through the
C ABI on inputs this test writes, with an overflow planted in one step.  Its
flags, decisions, loss scale, step counter and final state must meet the
parity bar against the oracle and the host policy.  build() compiles the
program; a missing program fails the test.
"""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, log

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "step_client")


def test_c_client_steps_match_oracle(tmp_path):
    assert os.path.exists(CLIENT), "tests/c_client/step_client is missing: run build() first"
    psi, n, rank = 1_000_003, 8, 7                 # the ragged last rank: 124,996 elements, 5 padding
    dtype, steps, S0, growth = "bf16", 5, 65536.0, 2
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    cnt = oracle.layout(psi, n, rank).count
    grads = []
    for s in range(steps):
        g = synth.fill_normal_(torch.empty(cnt, dtype=torch.bfloat16), 1e-3, 50_000 + s)
        if s == 2:
            synth.inject_nonfinite_(g, 1e-4, 50_100 + s)   # this step must be skipped
        grads.append(synth.to_numpy_u16(g))
    master0 = synth.fill_normal_(torch.empty(cnt), 0.02, 50_200).numpy()
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<QIIIIfIfffff", psi, n, rank, 1, steps, S0, growth, hp["lr"],
                            hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]))
        for g in grads:
            f.write(g.tobytes())
        f.write(master0.astype("<f4").tobytes())
    out = tmp_path / "out.bin"
    log(f"running the C client on {cnt} elements, {steps} steps")
    r = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    raw = open(out, "rb").read()
    decisions = np.frombuffer(raw[:8 * steps], np.int32).reshape(steps, 2)
    S_end, t_end = struct.unpack("<fQ", raw[8 * steps:8 * steps + 12])
    body = raw[8 * steps + 12:]
    assert len(body) == cnt * 14
    got = dict(w16=np.frombuffer(body[:2 * cnt], np.uint16),
               master=np.frombuffer(body[2 * cnt:6 * cnt], np.float32),
               m=np.frombuffer(body[6 * cnt:10 * cnt], np.float32),
               v=np.frombuffer(body[10 * cnt:], np.float32))

    ref = dict(master=master0.copy(), m=np.zeros(cnt, np.float32), v=np.zeros(cnt, np.float32),
               w16=np.zeros(cnt, np.uint16))
    st = oracle.ScalerState(S0, growth_interval=growth)
    for s, g in enumerate(grads):
        S = st.loss_scale
        flag, _ = oracle.overflow_check(g, dtype, S)
        apply = oracle.policy(st, flag)
        assert tuple(decisions[s]) == (flag, int(apply)), (s, decisions[s])
        if apply:
            oracle.adam_step(ref["w16"], g, ref["master"], ref["m"], ref["v"], dtype,
                             step=st.step, loss_scale=S, **hp)
    assert decisions[2, 0] == 1 and decisions[2, 1] == 0
    assert (S_end, t_end) == (np.float32(st.loss_scale), st.step)
    log("  C client", assert_close(got, ref, dtype, "C client"))
