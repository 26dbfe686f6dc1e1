"""The seeded input generator: determinism, shapes and statistics (CPU)."""

import math

import numpy as np
import torch

from workloads import WORKLOADS, make_inputs


def test_shapes_and_derived_sizes():
    w = WORKLOADS
    assert (w["tiny_fp32"].L, w["tiny_fp32"].T, w["tiny_fp32"].k) == (1024, 16, 4)
    assert (w["image_4608"].L, w["image_4608"].T, w["image_4608"].k) == (4608, 72, 18)
    assert (w["video480p_32760"].L, w["video480p_32760"].T, w["video480p_32760"].k) == (32760, 512, 64)
    assert (w["video720p_75600"].L, w["video720p_75600"].T, w["video720p_75600"].k) == (75600, 1182, 148)
    assert (w["video_long_118800"].L, w["video_long_118800"].T, w["video_long_118800"].k) == (118800, 1857, 186)
    assert w["video_long_118800_dense"].k == 1857
    # last block sizes: full, full, 56, 16, 16
    assert [x.L - 64 * (x.T - 1) for x in (w["tiny_fp32"], w["image_4608"], w["video480p_32760"],
                                            w["video720p_75600"], w["video_long_118800"])] == [64, 64, 56, 16, 16]


def test_deterministic_and_head_subsets():
    q1, k1, v1 = make_inputs("tiny_fp32")
    q2, k2, v2 = make_inputs("tiny_fp32", threads=1)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    qs, ks, vs = make_inputs("tiny_fp32", heads=[1])
    assert torch.equal(qs[0, 0], q1[0, 1]) and torch.equal(vs[0, 0], v1[0, 1])
    assert q1.dtype == torch.float32 and q1.shape == (1, 2, 1024, 64)


def test_bf16_statistics_and_text_tokens():
    w = WORKLOADS["image_4608"]
    q, k, v = make_inputs(w, heads=[0, 5])
    assert q.dtype == torch.bfloat16 and q.shape == (1, 2, 4608, 128)
    # values are exactly bf16 (the float32 view round-trips)
    assert torch.equal(q.float().to(torch.bfloat16), q)
    vf = v.float()
    assert abs(vf.mean().item()) < 0.01 and abs(vf.std().item() - 1.0) < 0.01
    # text tokens: iid N(0, 1) queries/keys
    qt = q[0, 0, 4096:].float()
    assert abs(qt.std().item() - 1.0) < 0.03
    # image logits q'.k have the spread of smooth DiT keys (std ~ 0.7)
    qi = q[0, 0, :4096:16].double().numpy()
    ki = k[0, 0, :4096].double().numpy()
    lg = qi @ ki.T / math.sqrt(128)
    assert 0.4 < lg.std() < 1.2
