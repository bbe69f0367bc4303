"""Failure handling of the one-launch decode schedule, forced from the host.

The schedule's group barrier waits, with a bounded spin, for per-member epoch flags in
the workspace's control block. Here the host sets one member's flag to a value the
other members never reach, so that barrier can never be satisfied: every workgroup
still exits after its bounded wait, the outputs become NaN, and the workspace's status
word makes blockffn_workspace_check report BLOCKFFN_ETIMEOUT. A zero-filled workspace
then gives the same bits as before.
"""
import numpy as np
import pytest
import torch

import chunk_level_activation_amd as bf
from chunk_level_activation_amd import inputs
from gpu_helpers import DEV, dev

pytestmark = pytest.mark.gpu

# The control block's layout (plan.h): 16384 words; the decode schedule's region starts
# at word 8192 with 32 output-tile counters, then the group-barrier flags [group][member].
DECODE_FLAGS_WORD = 8192 + 32
STATUS_WORD = 16383


def test_timeout_is_reported_and_a_zeroed_workspace_recovers():
    inp = inputs.make_workload("decode", seed=4)
    T, d_h, E, d_e, n = inp.T, inp.d_h, inp.E, inp.d_e, inp.n
    b16 = torch.bfloat16
    x, s = dev(inp.x, b16), dev(inp.scores)
    w1, w2 = dev(inp.w1, b16), dev(inp.w2, b16)
    ws = bf.blockffn_chunk_ffn_workspace(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16, DEV)
    y_ok = bf.blockffn_chunk_ffn(x, s, w1, w2, n, workspace=ws)
    bf.blockffn_workspace_check(ws)                       # no time-out: returns
    words = ws.view(torch.int32)
    assert int(words[STATUS_WORD]) == 0
    print("forcing a group-barrier time-out (member 1 of group 0)", flush=True)
    words[DECODE_FLAGS_WORD + 1] = 1 << 20
    y_bad = bf.blockffn_chunk_ffn(x, s, w1, w2, n, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y_bad.float()).all()
    with pytest.raises(bf.BlockFFNError) as err:
        bf.blockffn_workspace_check(ws)
    assert err.value.status == 5
    assert "zero-fill" in str(err.value)
    ws.zero_()
    y_again = bf.blockffn_chunk_ffn(x, s, w1, w2, n, workspace=ws)
    bf.blockffn_workspace_check(ws)
    assert torch.equal(y_again, y_ok)
    assert np.isfinite(y_ok.float().cpu().numpy()).all()


def test_init_is_idempotent():
    bf.blockffn_init()
    bf.blockffn_init()
    assert bf.blockffn_layer_forward_fused(32, 2048, 64, 128, 32, bf.BLOCKFFN_BF16)
