"""The seeded generator: determinism, shapes and that its codes are valid."""

import numpy as np
import torch

import synth
from oracle import e2m1_table, e4m3_table, e8m0_value
from oracle.gemm import decode_activations, decode_weights


def test_deterministic_and_shapes():
    p1 = synth.make_problem("tiny")
    p2 = synth.make_problem("tiny")
    for a, b in [(p1.topk_ids, p2.topk_ids), (p1.A, p2.A), (p1.SA, p2.SA), (p1.B, p2.B),
                 (p1.SB, p2.SB)]:
        assert torch.equal(a, b)
    assert p1.A.shape == (64, 512) and p1.SA.shape == (64, 4)
    assert p1.B.shape == (8, 256, 256) and p1.SB.shape == (8, 256, 16)
    assert p1.topk_ids.shape == (32, 2) and p1.topk_ids.dtype == torch.int32


def test_routing_kinds():
    u = synth.make_routing("uniform", 200, 12, 8, 3)
    for row in u.tolist():
        assert len(set(row)) == 8 and all(0 <= v < 12 for v in row)
    b = synth.make_routing("biased", 2000, 32, 8, 1)
    for row in b[:50].tolist():
        assert len(set(row)) == 8
    cnt = np.bincount(b.reshape(-1).numpy(), minlength=32)
    assert cnt.max() > 4 * max(cnt.min(), 1)          # strongly skewed


def test_fp8_quantizer_codes():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(16, 512, generator=g)
    x[3, 128:256] = 0
    codes, s = synth.quantize_fp8_rows(x)
    lut = e4m3_table()
    c = codes.numpy()
    assert not np.any((c & 0x7F) == 0x7F)                  # no NaN codes
    back = decode_activations(c, s.numpy())
    err = np.abs(back - x.double().numpy())
    assert np.all(err <= np.abs(x.double().numpy()) * 2.0 ** -4 + 1e-9 + s.double().repeat_interleave(128, 1).numpy() * 2.0 ** -10)
    assert s[3, 1] == 1.0 and np.all(c[3, 128:256] == 0)
    # the largest element of each group maps to +-448
    amax_codes = np.abs(lut[c]).reshape(16, 4, 128).max(axis=2)
    assert np.all((amax_codes == 448) | (s.numpy() == 1.0))


def test_mxfp4_quantizer_rule():
    g = torch.Generator().manual_seed(1)
    w = 0.02 * torch.randn(8, 256, generator=g)
    w[0, :32] = 0
    w[1, 32:64] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)
    packed, sb = synth.quantize_mxfp4(w)
    wd = decode_weights(packed.numpy(), sb.numpy())
    amax = w.abs().reshape(8, 8, 32).amax(2).double().numpy()
    scale = e8m0_value(sb.numpy())
    nz = amax > 0
    # scale = 2^(floor(log2 amax) - 2): amax/scale lies in [4, 8)
    assert np.all((amax[nz] / scale[nz] >= 4) & (amax[nz] / scale[nz] < 8))
    assert sb[0, 0] == 127 and np.all(wd[0, :32] == 0)
    # row 1 block 1: amax 7 -> scale 2^0; ties go to the even code, 7 saturates to 6
    assert sb[1, 1] == 127
    assert list(wd[1, 32:40]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    lut4 = e2m1_table()
    assert set(np.unique(np.abs(wd / np.repeat(scale, 32, axis=1)))) <= set(np.abs(lut4))


def test_wide_routing_is_a_top_k_selection():
    for skew in (False, True):
        a = synth.make_wide_routing(300, 5000, 8, seed=3, skew=skew)
        b = synth.make_wide_routing(300, 5000, 8, seed=3, skew=skew)
        assert a.dtype == torch.int32 and a.shape == (300, 8) and torch.equal(a, b)
        s = torch.sort(a, dim=1).values
        assert bool((s[:, 1:] != s[:, :-1]).all()) and int(a.min()) >= 0 and int(a.max()) < 5000
    assert synth.make_wide_routing(0, 64, 4, seed=1).shape == (0, 4)
    # skew concentrates slots on heavy experts
    u = torch.bincount(synth.make_wide_routing(2000, 2048, 8, 5).reshape(-1).long(), minlength=2048)
    w = torch.bincount(synth.make_wide_routing(2000, 2048, 8, 5, skew=True).reshape(-1).long(), minlength=2048)
    assert int(w.max()) > 4 * int(u.max())


def test_nvfp4_quantizer_gives_valid_codes_and_a_positive_tensor_scale():
    g = torch.Generator().manual_seed(8)
    w = 0.02 * torch.randn((64, 256), generator=g)
    B, SB, gs = synth.quantize_nvfp4(w)
    assert B.shape == (64, 128) and SB.shape == (64, 16) and gs > 0
    assert not torch.any((SB & 0x7F) == 0x7F)          # no NaN scale codes
    assert not torch.any(SB & 0x80)                     # block scales are amaxes: no sign
    p = synth.make_a16_problem("tiny", 1)
    assert p.SB.shape == (p.E, p.N, p.K // 16) and torch.all(p.GS > 0)
    p0 = synth.make_a16_problem("tiny", 0)
    assert p0.SB.shape == (p0.E, p0.N, p0.K // 32) and torch.all(p0.GS == 1)
