"""GPU: the split-K workspace under concurrent host threads sharing one stream.

The library's split-K scratch is per (device, stream), allocated in stream
order and grown with hipMallocAsync / hipFreeAsync on that stream; a call
holds it from lookup until its kernels are enqueued (kwkr.cn article,
troubleshooting table in section 5.1: state shared by host threads must be
thread-safe).  Two host threads here issue, on the same stream, split-K GEMMs
whose workspace needs grow from 0.5 MB to 16 MB, several rounds each, every
call into its own C.  Every result must be the oracle's within the stated
bound, and all repeats of one problem bitwise equal (one plan, fixed order).
"""
import threading

import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16 = torch.float16


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()
    return m


def test_two_threads_one_stream_through_workspace_growth(dg):
    # (M, N, K, forced K splits or 0 for the built-in plan)
    problems = [(64, 512, 4096, 0), (64, 2048, 4096, 0), (64, 4096, 4096, 0),
                (256, 256, 4100, 16), (256, 512, 4100, 16), (256, 1024, 4100, 16)]
    cases = [synth.gemm_case(M, N, K, F16, torch.float32, seed=M + N + K + S, name=f"{M}x{N}x{K}/S{S}")
             for (M, N, K, S) in problems]
    dev = [c.to(DEV) for c in cases]
    ws = []
    for (M, N, K, S), d in zip(problems, dev):
        text = dg.plan(d.A, d.B, d.C) if S == 0 else None
        if text is not None:
            assert "splits=1 " not in text, text
        ws.append(text)
    print("[workspace] plans:", [t.split(" ws=")[1].split(" ")[0] if t else "forced" for t in ws], flush=True)

    stream = torch.cuda.Stream()
    rounds, nthreads = 4, 2
    outs = [[[torch.full_like(d.C, float("nan")) for d in dev] for _ in range(rounds)] for _ in range(nthreads)]
    errors = []
    start = threading.Barrier(nthreads)

    def worker(t):
        try:
            start.wait()
            for r in range(rounds):
                # thread 0 walks the problems up (growing), thread 1 down
                order = range(len(problems)) if t == 0 else reversed(range(len(problems)))
                for i in order:
                    d, S = dev[i], problems[i][3]
                    C = outs[t][r][i]
                    if S:
                        dg.gemm_with_choice(d.A, d.B, C, (2, -1, S, -1), stream=stream)
                    else:
                        dg.gemm(d.A, d.B, C, stream=stream)
        except Exception as e:   # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    stream.synchronize()
    assert not errors, errors
    for i, c in enumerate(cases):
        ref = oracle.ref_gemm(c.A, c.B, None)
        first = outs[0][0][i].cpu()
        rep = oracle.compare(first, ref, "f32", c.rtol)
        print(f"[workspace] {c.name}: {rep}", flush=True)
        assert rep.ok, str(rep)
        for t in range(nthreads):
            for r in range(rounds):
                assert torch.equal(outs[t][r][i].cpu(), first), (c.name, t, r)
