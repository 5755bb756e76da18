"""The synthetic input recipe (CPU): correlated multi-token decode inputs."""
import dataclasses

import torch

import dsa_inputs as DI


def _small(name):
    c = DI.CASES[name]
    return dataclasses.replace(c, seqlens_k=(4096, 4096), seqlens_q=(4, 4))


def test_shared_query_tokens_copy_the_stated_fraction():
    """Token j > 0 of a sequence copies each indexer entry of token j-1 with probability
    q_share (0.9 here); entries drawn independently agree by chance (1/9 for q_I uniform over
    the 9 integers -4..4, 1/5 for w over -2..2); tokens of different sequences are independent."""
    d = DI.make_inputs(_small("mtp_b32_l16k_q4_shared"), "cpu", layers=1)
    q, w = d["q_idx"].float(), d["w"]
    for t in (1, 2, 3, 5, 6, 7):
        eq = (q[t] == q[t - 1]).float().mean().item()
        assert abs(eq - (0.9 + 0.1 / 9)) < 0.02, (t, eq)
    assert abs((w[1:4] == w[0:3]).float().mean().item() - (0.9 + 0.1 / 5)) < 0.06
    cross = (q[4] == q[3]).float().mean().item()      # first token of sequence 1 vs last of 0
    assert abs(cross - 1 / 9) < 0.02, cross


def test_independent_query_tokens():
    d = DI.make_inputs(_small("mtp_b32_l16k_q4"), "cpu", layers=1)
    q = d["q_idx"].float()
    for t in range(1, 8):
        assert abs((q[t] == q[t - 1]).float().mean().item() - 1 / 9) < 0.02


def test_q_share_leaves_the_other_tensors_alone():
    """The shared case draws k_idx, kv and q exactly as the independent one (same seed base)."""
    a = DI.make_inputs(_small("mtp_b32_l16k_q4"), "cpu", layers=1)
    b = DI.make_inputs(_small("mtp_b32_l16k_q4_shared"), "cpu", layers=1)
    assert torch.equal(a["k_idx"], b["k_idx"]) and torch.equal(a["kv"][0], b["kv"][0])
    assert torch.equal(a["q"][0], b["q"][0])
    assert torch.equal(a["q_idx"][0], b["q_idx"][0]) and torch.equal(a["q_idx"][4], b["q_idx"][4])
