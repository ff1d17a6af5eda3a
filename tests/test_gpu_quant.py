"""GPU activation quantizer with gather (w4a8_quantize_gather): E4M3 codes and
fp32 scales bit for bit equal to the oracle (oracle/quant.py), in both scale
layouts, at small sizes in full and at the large prefill size on sampled
tokens."""

import numpy as np
import pytest
import torch

import synth
from oracle import quantize_gather, quantize_tokens

pytestmark = pytest.mark.gpu


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _tokens(T, K, seed):
    """N(0,1) tokens with groups scaled over a wide range, all-zero groups,
    negative zeros and groups whose values fall in the E4M3 subnormal range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    G = K // 128
    scale = np.exp2(rng.integers(-30, 20, size=(T, G))).astype(np.float32)
    x = (x.reshape(T, G, 128) * scale[:, :, None]).reshape(T, K)
    x[0, :128] = 0.0
    if T > 1:
        x[1, 128:256] = -0.0
    if T > 2:
        x[2, :128] = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** -12)
        x[2, 0] = np.float32(448.0)  # tiny values beside a large amax: codes in the subnormal range
    return _bf16_bits(x)


def _run(lib, bits, ids, E, layout, R_extra=0):
    T, K = bits.shape
    k = ids.shape[1]
    _, off, ros = lib.route_prep(torch.from_numpy(ids).to("cuda"), E)
    R = int(off[-1].item()) + R_extra
    A0 = torch.full((R, K), 0x5A, dtype=torch.uint8, device="cuda")
    G = K // 128
    S0 = torch.full((R * G,), -7.0, dtype=torch.float32, device="cuda")
    A, SA = lib.quantize_gather(torch.from_numpy(bits.view(np.int16)).to("cuda"), ros, k, R, layout,
                                A=A0, SA=S0.view((R, G) if layout == 0 else (G, R)))
    torch.cuda.synchronize()
    return A.cpu().numpy(), SA.cpu().numpy().reshape(-1), ros.cpu().numpy(), R


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("T,K,E,k,seed", [
    (1, 128, 4, 1, 1),
    (37, 512, 8, 2, 2),
    (64, 6144, 32, 8, 3),     # decode gate/up activations
    (150, 3584, 12, 8, 4),    # E=12 W13 activations (28 groups: a partial pass of 32)
])
def test_quantize_gather_bit_exact(gpu_lib, layout, T, K, E, k, seed):
    bits = _tokens(T, K, seed)
    ids = synth.make_routing("uniform" if E >= k else "biased", T, E, k, seed).numpy()
    ids[0, 0] = -1  # an ignored slot: its row map entry is -1 and it writes nothing
    A, SA, ros, R = _run(gpu_lib, bits, ids, E, layout, R_extra=1)
    A_ref, SA_ref = quantize_gather(bits, ros, k, R, layout,
                                    A_init=np.full((R, K), 0x5A, np.uint8),
                                    SA_init=np.full(R * (K // 128), -7.0, np.float32))
    assert np.array_equal(A, A_ref)
    assert np.array_equal(SA.view(np.uint32), SA_ref.view(np.uint32))
    assert np.all(A[R - 1] == 0x5A)  # the extra row is named by no slot


def test_quantize_ties_and_extremes_bit_exact(gpu_lib):
    """Scaled values exactly on every midpoint between neighbouring E4M3
    codes (scale a power of two), just beside them, and the amax element."""
    table = np.array([v for v in np.unique(np.abs(_e4m3_values())) if v <= 448.0])
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    mb = _bf16_bits(mids)
    beside = np.concatenate([mb + 1, mb[mb > 0] - 1]).astype(np.uint16)  # one bf16 step off each midpoint
    beside = (beside.astype(np.uint32) << 16).view(np.float32)
    vals = np.concatenate([mids, -mids, beside, table.astype(np.float32)])
    groups = []
    for shift in (-3, 0, 5):
        for i in range(0, len(vals), 127):
            g = np.zeros(128, np.float32)
            chunk = vals[i:i + 127]
            g[:len(chunk)] = chunk * np.float32(2.0 ** shift)
            g[127] = np.float32(448.0 * 2.0 ** shift)  # amax: scale exactly 2^shift
            groups.append(g)
    while len(groups) % 4:
        groups.append(np.zeros(128, np.float32))
    x = np.stack(groups).reshape(-1, 512)
    bits = _bf16_bits(x)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x)  # exact in bf16
    T = x.shape[0]
    ros = torch.arange(T, dtype=torch.int32, device="cuda")
    A, SA = gpu_lib.quantize_gather(torch.from_numpy(bits.view(np.int16)).to("cuda"), ros, 1, T, 0)
    codes, s = quantize_tokens(bits)
    assert np.array_equal(A.cpu().numpy(), codes)
    assert np.array_equal(SA.cpu().numpy().view(np.uint32), s.view(np.uint32))


def _e4m3_values():
    from oracle import e4m3_table
    t = e4m3_table()
    return t[~np.isnan(t)]


def test_quantize_prefill_size_sampled(gpu_lib):
    """16384 tokens x 6144, top-8 biased routing over 32 experts (the large
    prefill gate/up activations), M-major scales: every row of 48 sampled
    tokens against the oracle."""
    cfg = synth.CONFIGS["prefill_gateup"]
    T, K, E, k = cfg["T"], cfg["K"], cfg["E"], cfg["top_k"]
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((T, K), dtype=np.float32)).to(torch.bfloat16)
    ids = synth.make_routing(cfg["routing"], T, E, k, cfg["seed"])
    _, off, ros = gpu_lib.route_prep(ids.to("cuda"), E)
    R = int(off[-1].item())
    A, SA = gpu_lib.quantize_gather(x.to("cuda"), ros, k, R, 1)
    torch.cuda.synchronize()
    G = K // 128
    ros_np = ros.cpu().numpy().reshape(T, k)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    sample = rng.choice(T, size=48, replace=False)
    codes, s = quantize_tokens(xb[sample])
    rows = ros_np[sample]
    A_rows = A[torch.from_numpy(rows.reshape(-1)).long().to("cuda")].cpu().numpy().reshape(48, k, K)
    SA_cols = SA.view(G, R)[:, torch.from_numpy(rows.reshape(-1)).long().to("cuda")].cpu().numpy()
    SA_cols = SA_cols.T.reshape(48, k, G)
    for i in range(48):
        for j in range(k):
            assert np.array_equal(A_rows[i, j], codes[i])
            assert np.array_equal(SA_cols[i, j].view(np.uint32), s[i].view(np.uint32))


def test_quantize_empty_inputs(gpu_lib):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    ros = torch.zeros(0, dtype=torch.int32, device="cuda")
    A, SA = gpu_lib.quantize_gather(x, ros, 2, 4, 0)
    torch.cuda.synchronize()
    assert not A.any() and not SA.any()
