"""The seeded input generator: bf16 rounding, determinism, shapes and the head-scale recipe."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties between two bf16 neighbours, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-38, -3.4e38, 65504.0], dtype=np.float32),
    ])
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    assert (W.bf16_to_f32(ours) == torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()


def test_shapes_and_determinism():
    w = W.workload(0)
    a = W.generate(w)
    b = W.generate(w)
    assert a["q16"].shape == (1, 256, 2, 64)
    for key in ("q16", "k16", "v16"):
        assert (a[key] == b[key]).all()
    assert list(a["s"]) == [0.5, 3.0]
    assert w.nb == 16 and w.tiles == 32


def test_workload_table():
    shapes = {w.name: (w.N, w.nb, w.tiles) for w in W.WORKLOADS}
    assert shapes["480p-12h"] == (32760, 512, 6144)
    assert shapes["720p-40h"] == (75600, 1182, 47280)
    assert shapes["long6x-12h"] == (196560, 1536, 18432)
    skew = W.workload("720p-40h-skew")
    s = W._signal_scales(skew, np.random.default_rng(0))
    assert (s[:35] == 5.0).all() and (s[35:] == 0.3).all()
