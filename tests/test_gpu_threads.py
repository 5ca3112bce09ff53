"""Calls from several host threads at once: each thread plans and launches its own layouts
on its own stream, repeatedly, while the others do the same.  The library keeps its plan
cache and its test pins per thread and takes no lock, so every result must still match the
oracle, and a pin set by one thread never reaches another thread's calls."""
import threading

import numpy as np
import pytest
import torch

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import DeviceProblem, check_full, oracle_full

pytestmark = pytest.mark.gpu

ROUNDS = 6


def _problems(t):
    return [synth.make_dense(200 + 17 * t, 300 + 16 * t, 512, seed=3000 + t),
            synth.make_contiguous(3, 256, 384, seed=3100 + t, counts=[70 + t, 0, 150]),
            synth.make_masked(4, 96, 208, 256, seed=3200 + t, masked_m=[5, 96, 0, 40 + t])]


def test_threads_with_their_own_streams():
    n_threads = 4
    # inputs and oracle results prepared up front (the oracle is CPU work)
    cases = [[(p, oracle_full(p)) for p in _problems(t)] for t in range(n_threads)]
    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            dps = [DeviceProblem(p) for p, _ in cases[t]]
            torch.cuda.current_stream().synchronize()     # uploads done before use
            for r in range(ROUNDS):
                with torch.cuda.stream(stream):
                    for dp in dps:
                        dp.reset()
                        dp.run(stream=stream, workspace=(r + t) % 2 == 0)
                stream.synchronize()
                for dp, (p, ref) in zip(dps, cases[t]):
                    check_full(p, dp.d.cpu().numpy().view(np.uint16), ref,
                               f"thread {t} round {r} {p.kind}")
        except BaseException as e:                     # reported by the main thread
            errors.append((t, e))

    print(f"[gpu] {n_threads} threads x {ROUNDS} rounds x 3 layouts", flush=True)
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors[0]


def test_one_thread_pins_while_the_others_plan():
    """Thread 0 pins every instance in turn (with forced split counts) and checks that its
    calls run the pinned plan; the other threads keep calling with the planner's choice at
    the same time and must see neither the pins nor wrong results."""
    n_threads = 3
    cases = [[(p, oracle_full(p)) for p in _problems(t)] for t in range(n_threads)]
    insts = fp8bs.instances()
    errors = []
    done = threading.Event()

    def pinner():
        try:
            stream = torch.cuda.Stream()
            dps = [DeviceProblem(p) for p, _ in cases[0]]
            torch.cuda.current_stream().synchronize()
            for i, info in enumerate(insts):
                for dp, (p, ref) in zip(dps, cases[0]):
                    if p.kind == "contiguous" and 128 % info["block_m"] and info["block_m"] != 256:
                        continue
                    fp8bs.force_instance(i)
                    fp8bs.force_splits(1 + i % 3 if p.kind == "dense" else 0)
                    try:
                        with torch.cuda.stream(stream):
                            dp.reset()
                            dp.run(stream=stream, workspace=True)
                    finally:
                        fp8bs.force_instance(-1)
                        fp8bs.force_splits(0)
                    stream.synchronize()
                    check_full(p, dp.d.cpu().numpy().view(np.uint16), ref,
                               f"pinning thread, instance {i}, {p.kind}")
        except BaseException as e:
            errors.append(("pinner", e))
        finally:
            done.set()

    def planner(t):
        try:
            stream = torch.cuda.Stream()
            dps = [DeviceProblem(p) for p, _ in cases[t]]
            torch.cuda.current_stream().synchronize()
            r = 0
            while not done.is_set() or r < 2:
                # this thread never pinned anything: its setters report the unpinned state
                assert fp8bs.force_instance(-1) == -1 and fp8bs.force_splits(0) == 0
                with torch.cuda.stream(stream):
                    for dp in dps:
                        dp.reset()
                        dp.run(stream=stream, workspace=r % 2 == 0)
                stream.synchronize()
                for dp, (p, ref) in zip(dps, cases[t]):
                    check_full(p, dp.d.cpu().numpy().view(np.uint16), ref,
                               f"planning thread {t} round {r} {p.kind}")
                r += 1
        except BaseException as e:
            errors.append((t, e))

    print(f"[gpu] one pinning thread over {len(insts)} instances, {n_threads - 1} planning "
          "threads", flush=True)
    threads = [threading.Thread(target=pinner)] + \
        [threading.Thread(target=planner, args=(t,)) for t in range(1, n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=110)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors[0]
