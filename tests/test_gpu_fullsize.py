"""Full-size parity of the Llama-3-8B and Llama-3-70B rank shards: every
owned element compared with the oracle.

Page "04 · 分布式优化器", §4.3: the rank steps its fp32 shard, split parameters
included, and writes the updated parameters into its owned range. Rank 1's
full-size launch runs once on the GPU. The state before the step is kept in
a second device copy; the shard is then streamed to the host in chunks of at
most 2^26 slots (D contribution slices, the state before and after, the
parameter slice), the oracle steps each chunk from the bytes the device
received, and every fp32 and bf16 output must equal it bit for bit. The
chunks follow the oracle's own range map (oracle.layout.rank_pieces): the
rank's pieces of one bucket form one run, contiguous in the shard and in the
buffer, which gives each chunk's LOCAL and WORLD offsets. Every parameter
slot the rank does not own must keep its sentinel.

Llama-3-8B runs in WORLD coordinates (D whole buffers of N = 8.03e9
elements, offsets beyond 2^32) and in LOCAL slices; Llama-3-70B (D = 32,
2.2e9 owned elements) in LOCAL slices, the configuration bench.py times.
"""

import sys
import time

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.numerics as ON
import workloads as W
from test_gpu_parity import DEV, SENTINEL, _gen_state, assert_bf16, assert_f32, free, hp_kwargs, local_stride

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


def say(msg: str) -> None:
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


def owned_runs(lay, r):
    """[shard start, world start, length] of the rank's owned elements, one
    run per bucket (its pieces there are adjacent in both coordinates)."""
    runs = []
    for pc in OL.rank_pieces(lay, r):
        if runs and runs[-1][0] + runs[-1][2] == pc.shard_offset and \
                runs[-1][1] + runs[-1][2] == pc.gbuf_world.start:
            runs[-1][2] += pc.gbuf_world.size
        else:
            runs.append([pc.shard_offset, pc.gbuf_world.start, pc.gbuf_world.size])
    return runs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,coords", [("llama3_8b", "world"), ("llama3_8b", "local"), ("llama3_70b", "local")])
def test_llama_shard_every_element(gpu, name, coords):
    w = W.get(name)
    r = w.verify_ranks[0]
    D = w.dp_size
    t0 = time.perf_counter()
    lay = OL.build_layout(w.param_numel, w.bucket_numel, D)
    plan = gpu.build_range_map(w.param_numel, w.bucket_numel, D, r)
    Ln, N = plan.shard_numel, plan.buffer_numel
    assert (Ln, N) == (OL.shard_numel(lay, r), lay.buffer_numel)
    runs = owned_runs(lay, r)
    E = sum(n for _, _, n in runs)
    assert E == plan.owned_numel
    world = coords == "world"
    C = gpu.WORLD if world else gpu.LOCAL
    n_rep = N if world else Ln
    stride = local_stride(n_rep)
    say(f"{name} {coords}: rank {r}, D={D}, E={E}, L={Ln}, N={N}, {len(runs)} runs")

    # contributions: rank-shard values drawn in LOCAL order, placed at the
    # owned elements of whole buffers in WORLD mode (other elements are never
    # read)
    bufs = torch.empty(D * stride, dtype=torch.bfloat16, device=DEV)
    reps = []
    tmp = torch.empty(Ln, dtype=torch.bfloat16, device=DEV) if world else None
    for j in range(D):
        if world:
            W.normal_bf16(Ln, w.grad_sigma, W.seed(w.cfg, 0, "grad", j), out=tmp)
            dst = bufs[j * stride: j * stride + N]
            for k0, w0, n in runs:
                dst[w0:w0 + n].copy_(tmp[k0:k0 + n])
        else:
            dst = bufs[j * stride: j * stride + Ln]
            W.normal_bf16(Ln, w.grad_sigma, W.seed(w.cfg, 0, "grad", j), out=dst)
        reps.append(dst.view(torch.int16))
    del tmp
    st = _gen_state(w, Ln)
    before = [x.clone() for x in st]
    par = torch.full((n_rep,), SENTINEL, dtype=torch.int16, device=DEV)
    torch.cuda.synchronize()
    say(f"inputs on the device in {time.perf_counter() - t0:.1f}s")

    gpu.sharded_adam_step(plan, reps, C, w.scale, *st, par, C, **hp_kwargs(w.hp, 1))
    torch.cuda.synchronize()
    assert int((par == SENTINEL).sum()) == n_rep - E, "a slot outside the owned elements was written"
    say(f"step done, sentinels intact ({time.perf_counter() - t0:.1f}s)")

    hp = ON.hp_array(w.hp, 1)
    stage_g = torch.empty((D, CHUNK), dtype=torch.int16, pin_memory=True)
    stage_b = torch.empty((3, CHUNK), dtype=torch.float32, pin_memory=True)
    stage_a = torch.empty((3, CHUNK), dtype=torch.float32, pin_memory=True)
    stage_p = torch.empty(CHUNK, dtype=torch.int16, pin_memory=True)
    done, t_oracle, last = 0, 0.0, time.perf_counter()
    for k_run, w_run, n_run in runs:
        for off in range(0, n_run, CHUNK):
            n = min(CHUNK, n_run - off)
            k0 = k_run + off
            gi = (w_run + off) if world else k0
            for j in range(D):
                stage_g[j, :n].copy_(reps[j][gi:gi + n], non_blocking=True)
            for i in range(3):
                stage_b[i, :n].copy_(before[i][k0:k0 + n], non_blocking=True)
                stage_a[i, :n].copy_(st[i][k0:k0 + n], non_blocking=True)
            stage_p[:n].copy_(par[gi:gi + n], non_blocking=True)
            torch.cuda.synchronize()
            grads = [stage_g[j, :n].numpy().view(np.uint16) for j in range(D)]
            want = [stage_b[i, :n].numpy() for i in range(3)]      # stepped in place by the oracle
            want_par = np.empty(n, np.uint16)
            a = time.perf_counter()
            ON.step(grads, w.scale, *want, hp, want_par)
            t_oracle += time.perf_counter() - a
            for i, nm in enumerate(("master", "exp_avg", "exp_avg_sq")):
                got = stage_a[i, :n].numpy()
                if not np.array_equal(got.view(np.uint32), want[i].view(np.uint32)):
                    assert_f32(got, want[i], f"{name} {coords} {nm} slots [{k0}, {k0 + n})")
            got_p = stage_p[:n].numpy().view(np.uint16)
            if not np.array_equal(got_p, want_par):
                assert_bf16(got_p, want_par, f"{name} {coords} params slots [{k0}, {k0 + n})")
            done += n
            if time.perf_counter() - last > 20:
                last = time.perf_counter()
                say(f"{done}/{E} elements equal so far ({done / E:.0%})")
    assert done == E
    say(f"all {E} owned elements bit-exact; oracle {t_oracle:.1f}s, total {time.perf_counter() - t0:.1f}s")
    del bufs, reps, st, before, par, stage_g, stage_b, stage_a, stage_p
    free()
