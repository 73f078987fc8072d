"""The measurement references on the GPU: zdo_device_copy and
zdo_stream_probe (the step's stream shape with trivial arithmetic, in its
three store modes). Not
part of the method; checked against the transform include/zdo.h states,
evaluated with numpy, and for their argument errors."""

import numpy as np
import pytest
import torch

from test_gpu_parity import DEV, free, to_dev

pytestmark = pytest.mark.gpu


def probe_numpy(reads, state, n):
    """state gains the exponent bits of the XOR of the reads' 16-byte chunk
    of each lane; out holds the old state bits XOR words of that chunk."""
    D = len(reads)
    tiles = n // 512
    x = np.zeros((tiles, 64, 4), np.uint32)
    for r in reads:
        x ^= r[:n].view(np.uint32).reshape(tiles, 64, 4)
    f = ((x[..., 0] ^ x[..., 1] ^ x[..., 2] ^ x[..., 3]) & np.uint32(0x3F000000)).view(np.float32)   # [tiles, 64]
    new = [s.copy() for s in state]
    out = np.zeros(n, np.uint16)
    o32 = out.view(np.uint32).reshape(tiles, 2, 64, 2)
    for i in range(3):
        q = state[i][:n].reshape(tiles, 2, 64, 4)
        new[i][:n] = (q + f[:, None, :, None]).reshape(-1)
    for h in range(2):
        q0 = state[0][:n].reshape(tiles, 2, 64, 4)[:, h, :, 0].view(np.uint32)
        q1 = state[1][:n].reshape(tiles, 2, 64, 4)[:, h, :, 1].view(np.uint32)
        o32[:, h, :, 0] = q0 ^ x[..., 2 * h]
        o32[:, h, :, 1] = q1 ^ x[..., 2 * h + 1]
    return new, out


def probe_numpy_parts(reads, state, n, stores, out0):
    """The two store modes without state stores: with PROBE_STORE_OUT quad h
    of each lane gets x[2h] ^ S_h and x[2h+1] ^ S_h (S_h: XOR of the quad's
    12 state words); with PROBE_STORE_NONE only word t of out (elements
    2t, 2t+1) changes, to the XOR over the tile's lanes of
    x[0]^x[1]^x[2]^x[3]^S_0^S_1."""
    tiles = n // 512
    x = np.zeros((tiles, 64, 4), np.uint32)
    for r in reads:
        x ^= r[:n].view(np.uint32).reshape(tiles, 64, 4)
    sx = np.zeros((tiles, 2, 64), np.uint32)
    for st in state:
        q = st[:n].view(np.uint32).reshape(tiles, 2, 64, 4)
        sx ^= q[..., 0] ^ q[..., 1] ^ q[..., 2] ^ q[..., 3]
    out = out0.copy()
    if stores == 1:
        o32 = out.view(np.uint32).reshape(tiles, 2, 64, 2)
        for h in range(2):
            o32[:, h, :, 0] = x[..., 2 * h] ^ sx[:, h]
            o32[:, h, :, 1] = x[..., 2 * h + 1] ^ sx[:, h]
    else:
        v = x[..., 0] ^ x[..., 1] ^ x[..., 2] ^ x[..., 3] ^ sx[:, 0] ^ sx[:, 1]
        out.view(np.uint32)[:tiles] = np.bitwise_xor.reduce(v, axis=1)
    return out


@pytest.mark.parametrize("D", [8, 16, 32])
def test_stream_probe_transform(gpu, D):
    rng = np.random.default_rng(D)
    n = 512 * 37
    reads = [rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16) for _ in range(D)]
    state = [(rng.standard_normal(n) * 0.02).astype(np.float32) for _ in range(3)]
    rd = [to_dev(r) for r in reads]
    sd = [to_dev(s) for s in state]
    od = torch.zeros(n, dtype=torch.int16, device=DEV)
    for cap in (0, 4):
        for x, s in zip(sd, state):
            x.copy_(torch.from_numpy(s))
        gpu.stream_probe(rd, sd, od, n, cap)
        want_s, want_o = probe_numpy(reads, state, n)
        for x, w in zip(sd, want_s):
            assert np.array_equal(x.cpu().numpy().view(np.uint32), w.view(np.uint32))
        assert np.array_equal(od.view(torch.int16).cpu().numpy().view(np.uint16), want_o)
    # the store modes that leave the state alone
    out0 = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    for stores in (gpu.PROBE_STORE_OUT, gpu.PROBE_STORE_NONE):
        for x, st in zip(sd, state):
            x.copy_(torch.from_numpy(st))
        od.copy_(torch.from_numpy(out0.view(np.int16)))
        gpu.stream_probe(rd, sd, od, n, 4, stores=stores)
        for x, st in zip(sd, state):
            assert np.array_equal(x.cpu().numpy().view(np.uint32), st.view(np.uint32))
        want_o = probe_numpy_parts(reads, state, n, stores, out0)
        assert np.array_equal(od.cpu().numpy().view(np.uint16), want_o), f"stores={stores}"
    # errors
    with pytest.raises(gpu.ZdoError) as e:
        gpu.stream_probe(rd, sd, od, n, stores=3)
    assert e.value.code == gpu.EINVAL
    with pytest.raises(gpu.ZdoError) as e:
        gpu.stream_probe(rd[:5], sd, od, n)
    assert e.value.code == gpu.EINVAL
    with pytest.raises(gpu.ZdoError) as e:
        gpu.stream_probe(rd, sd, od, n - 8)
    assert e.value.code == gpu.EINVAL
    with pytest.raises(gpu.ZdoError) as e:
        gpu.stream_probe(rd, [sd[0], sd[0], sd[2]], od, n)
    assert e.value.code == gpu.EALIAS
    free()


def test_device_copy(gpu):
    src = torch.from_numpy(np.random.default_rng(1).integers(0, 1 << 30, 1 << 18, dtype=np.int64).astype(np.int32)).to(DEV)
    dst = torch.zeros_like(src)
    gpu.device_copy(dst, src)
    assert torch.equal(dst, src)
    rc = gpu.require_library().zdo_device_copy(dst.data_ptr(), src.data_ptr(), 15, None)
    assert rc == gpu.EINVAL
    free()
