"""Randomised parity: seeded draws over operation (AllReduce, ReduceScatter,
AllGather, send/recv), protocol, rank count, dtype, size, placement,
workgroup size, the pipelined Sentinel's credit and the epoch source, each
checked against the oracle (bit-exact for LL and Sentinel, within the atomic
protocol's tolerance for LL128); and draws over the tuning options (chunk,
slices, LL128 kernel, staging, buffers and consumer waves, first-XCDs span)."""
import numpy as np
import pytest
import torch

import message_allreduce_amd as llar
import oracle
from oracle import models
from workloads import make_partials, random_bits

from gpu_util import CODE, TORCH_DT, assert_exact, assert_tol, run, to_device, to_host

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]
AR_PROTOCOLS = ["ll", "sentinel", "ll128", "ll128_pipelined", "sentinel_pipelined", "auto"]


def draw(rng):
    op = rng.choice(["allreduce", "allreduce", "reduce_scatter", "all_gather", "send_recv"])
    dtype = str(rng.choice(DTYPES))
    n_ranks = int(rng.integers(1, 9))
    esize = 4 if dtype == "fp32" else 2
    nbytes = int(rng.choice([rng.integers(1, 64), rng.integers(64, 4096), rng.integers(4096, 1 << 18),
                             rng.integers(1 << 18, 3 << 20)]))
    n = max(1, nbytes // esize)
    placement = int(rng.integers(0, 3))
    threads = int(rng.choice([0, 64, 128, 256, 512]))
    if op == "allreduce":
        proto = str(rng.choice(AR_PROTOCOLS))
    elif op == "reduce_scatter":
        proto = str(rng.choice(["ll", "sentinel", "ll128", "auto"]))
        n = max(1, n // n_ranks)
    elif op == "all_gather":
        proto = str(rng.choice(["ll", "sentinel", "auto"]))
        n = max(1, n // n_ranks)
    else:
        proto = str(rng.choice(["ll", "sentinel", "auto"]))
    # drawn last, so the fields above keep their values for a given seed
    credit = int(rng.integers(0, 3))      # pipelined Sentinel: workgroup, slot or owner credit
    dev_epoch = int(rng.integers(0, 2))   # 1: the device-resident epoch (per-workgroup epoch words)
    return op, dtype, n_ranks, n, proto, placement, threads, credit, dev_epoch


CASES = [draw(np.random.default_rng([7000, i])) for i in range(200)]


@pytest.mark.parametrize("index", range(len(CASES)), ids=["%s-%s-N%d-n%d-%s-p%d-t%d-c%d-e%d" % c for c in CASES])
def test_random_configuration(index):
    case = CASES[index]
    op, dtype, n_ranks, n, proto, placement, threads, credit, dev_epoch = case
    dt = CODE[dtype]
    esize = 4 if dtype == "fp32" else 2
    max_bytes = n * esize * (n_ranks if op in ("reduce_scatter", "all_gather") else 1)
    c = llar.Communicator(n_ranks, TORCH_DT[dt], max_bytes)
    try:
        c.set_option("spin_timeout_us", 100_000)
        c.set_option("placement", placement)
        c.set_option("device_epoch", dev_epoch)
        if not (threads == 64 and proto in ("sentinel_pipelined", "auto") and op == "allreduce"):
            c.set_option("threads", threads)
        if proto == "sentinel_pipelined" and threads == 0:
            # the slot and owner credits run 1024-thread workgroups by default
            c.set_option("sentinel_credit", credit)
        seed = index
        if op == "allreduce":
            bits = make_partials(7100, seed, n_ranks, dtype, n, "normal", 0.5)
            got = run(c, bits, proto, dt)
            want = oracle.allreduce(bits, dt)
            (assert_tol if proto.startswith("ll128") else assert_exact)(got, want, dt, str(case))
        elif op == "reduce_scatter":
            bits = make_partials(7200, seed, n_ranks, dtype, n_ranks * n, "normal", 0.5)
            parts = [to_device(bits[r], dt) for r in range(n_ranks)]
            outs = [torch.empty(n, dtype=TORCH_DT[dt], device="cuda") for _ in range(n_ranks)]
            c.reduce_scatter(parts, outs, proto)
            torch.cuda.synchronize()
            assert c.device_status()[0] == 0
            want = oracle.reduce_scatter(bits, dt)
            for j in range(n_ranks):
                (assert_tol if proto == "ll128" else assert_exact)(to_host(outs[j], dt), want[j], dt,
                                                                   "%s rank %d" % (case, j))
        elif op == "all_gather":
            frags = np.stack([random_bits(7300, seed + r, n, dtype) for r in range(n_ranks)])
            ins = [to_device(frags[r], dt) for r in range(n_ranks)]
            outs = [torch.empty(n_ranks * n, dtype=TORCH_DT[dt], device="cuda") for _ in range(n_ranks)]
            c.all_gather(ins, outs, proto)
            torch.cuda.synchronize()
            assert c.device_status()[0] == 0
            wire = "sentinel" if proto == "sentinel" or (proto == "auto" and n_ranks * n * esize > 64 << 10) else "ll"
            want = models.all_gather(list(frags), dt, wire)
            for j in range(n_ranks):
                assert np.array_equal(to_host(outs[j], dt), want), "%s copy %d" % (case, j)
        else:
            bits = random_bits(7400, seed, n, dtype)
            recv = torch.empty(n, dtype=TORCH_DT[dt], device="cuda")
            c.send_recv(to_device(bits, dt), recv, proto)
            torch.cuda.synchronize()
            assert c.device_status()[0] == 0
            wire = "sentinel" if proto == "sentinel" or (proto == "auto" and n * esize > 64 << 10) else "ll"
            assert np.array_equal(to_host(recv, dt), models.p2p_transfer(bits, dt, wire)), str(case)
    except llar.LlarError as e:
        if e.status == -2:  # a geometry this device cannot hold at once: a documented refusal
            pytest.skip("unsupported on this device: %s" % e)
        raise
    finally:
        c.close()


# ----------------------------------------------------------------------------- tuning options
def draw_tuning(rng):
    """An AllReduce under the kernel-selection and geometry options: chunk
    size, slices, workgroup size, LL128 kernel, staging and buffers, consumer
    waves, pipelined-Sentinel buffers and credit, and the first-XCDs span of
    the one-shot reduce."""
    dtype = str(rng.choice(DTYPES))
    n_ranks = int(rng.integers(1, 9))
    esize = 4 if dtype == "fp32" else 2
    nbytes = int(rng.choice([rng.integers(1, 4096), rng.integers(4096, 1 << 17), rng.integers(1 << 17, 2 << 20)]))
    n = max(1, nbytes // esize)
    proto = str(rng.choice(["ll", "sentinel", "ll128", "ll128_pipelined", "sentinel_pipelined"]))
    opts = {"placement": int(rng.integers(0, 3)), "slices": int(rng.choice([0, 0, rng.integers(1, 65)])),
            "chunk_bytes": int(rng.choice([0, 2048, 8192, 32768, 131072]))}
    # 16-bit LL128 staging: integer data whose partial sums the 16-bit type holds
    acc16 = dtype != "fp32" and proto.startswith("ll128") and rng.random() < 0.5
    if acc16 and dtype == "bf16":
        n_ranks = min(n_ranks, 4)  # |sum| <= 256: exact in bfloat16
    opts["ll128_acc"] = int(acc16)
    if proto in ("ll", "sentinel"):
        opts["local_xcds"] = int(rng.integers(0, 9))
        opts["threads"] = int(rng.choice([0, 64, 128, 256, 512]))
    elif proto == "ll128":
        opts["threads"] = int(rng.choice([0, 64, 128, 256, 512]))
    elif proto == "ll128_pipelined":
        kernel = int(rng.integers(0, 2))
        opts["ll128_kernel"] = kernel
        if kernel == 0:
            threads = int(rng.choice([0, 128, 256, 512, 1024]))
            waves = (threads or 1024) // 64
            opts["threads"] = threads
            opts["consumer_waves"] = int(rng.choice([0, rng.integers(1, min(waves - 1, 15) + 1)]))
            opts["ll128_buffers"] = int(rng.choice([0, 2 * rng.integers(1, 33)]))
        else:
            opts["threads"] = int(rng.choice([0, 64, 128, 256, 512]))
    else:
        credit = int(rng.integers(0, 3))
        opts["sentinel_credit"] = credit
        # the owner credit needs a credit wave beside a producer and a consumer
        opts["threads"] = int(rng.choice(([0, 128, 256, 512] if credit < 2 else [0, 256, 512])
                                         + ([1024] if credit else [])))
        if credit == 0:
            opts["pipeline_buffers"] = int(rng.choice([4, 6, 8]))
    return dtype, n_ranks, n, proto, acc16, opts


TUNING = [draw_tuning(np.random.default_rng([7500, i])) for i in range(120)]


@pytest.mark.parametrize("index", range(len(TUNING)),
                         ids=["%s-N%d-n%d-%s-a%d" % c[:5] for c in TUNING])
def test_random_tuning(index):
    dtype, n_ranks, n, proto, acc16, opts = TUNING[index]
    dt = CODE[dtype]
    esize = 4 if dtype == "fp32" else 2
    c = llar.Communicator(n_ranks, TORCH_DT[dt], n * esize)
    try:
        c.set_option("spin_timeout_us", 100_000)
        for k, v in opts.items():
            c.set_option(k, v)
        what = "%s %s N=%d n=%d %s" % (dtype, proto, n_ranks, n, opts)
        if acc16:
            bits = make_partials(7600, index, n_ranks, dtype, n, "integer", 1.0)
            assert_exact(run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, what)
        else:
            bits = make_partials(7600, index, n_ranks, dtype, n, "normal", 0.5)
            (assert_tol if proto.startswith("ll128") else assert_exact)(
                run(c, bits, proto, dt), oracle.allreduce(bits, dt), dt, what)
    except llar.LlarError as e:
        if e.status == -2:  # a geometry this device cannot hold at once: a documented refusal
            pytest.skip("unsupported on this device: %s" % e)
        raise
    finally:
        c.close()
