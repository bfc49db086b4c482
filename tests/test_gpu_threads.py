"""Calls from several host threads at once, each on its own stream with its own workspace, give the same results
as the same calls made one at a time (the ABI's reentrancy contract).

Three threads run a resident fit, a streamed fit from pinned host memory and a batched fit concurrently, twice
over; each result must equal its serial run bit for bit (centroids, assignments, counts).
"""
import threading

import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _data(name, seed, **kw):
    w = synth.WORKLOADS[name].scaled(seed=seed, **kw)
    Xn = synth.points(w)
    return parity.x_from_numpy(Xn, w.dtype, DEV), torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)


def _jobs():
    Xa, Ca = _data("c2", 11, N=80_000, K=512)
    Xs, Cs = _data("c4", 12, N=120_000, K=1024)
    Xs_host = Xs.cpu().pin_memory()
    Xb = torch.stack([_data("c1", 20 + b)[0] for b in range(8)])
    Cb = torch.stack([_data("c1", 20 + b)[1] for b in range(8)])

    def resident(ws, stream):
        C, a, n, _ = km.fit(Xa, Ca, 6, ws=ws)
        return C, a, n

    def streamed(ws, stream):
        C, a, n, _ = km.fit_streamed(Xs_host, Cs, 3, 50_000, copy_stream=torch.cuda.Stream(), ws=ws)
        return C, a, n

    def batched(ws, stream):
        C, a, n, _ = km.fit_batched(Xb, Cb, 5, ws=ws)
        return C, a, n

    return [("resident", resident), ("streamed", streamed), ("batched", batched)]


def _run(fn, ws, stream):
    with torch.cuda.stream(stream):
        out = fn(ws, stream)
    stream.synchronize()
    return out


def test_concurrent_fits_equal_serial():
    jobs = _jobs()
    streams = [torch.cuda.Stream() for _ in jobs]
    workspaces = [km.Workspace(DEV) for _ in jobs]
    serial = [_run(fn, workspaces[i], streams[i]) for i, (_, fn) in enumerate(jobs)]
    torch.cuda.synchronize()
    for rep in range(2):
        results = [None] * len(jobs)
        errors = []

        def worker(i):
            try:
                results[i] = _run(jobs[i][1], workspaces[i], streams[i])
            except Exception as e:  # reported below, in the main thread
                errors.append((jobs[i][0], repr(e)))

        threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
        print(f"[threads] rep {rep}: {len(threads)} threads", flush=True)
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a thread did not finish"
        assert not errors, errors
        torch.cuda.synchronize()
        for (name, _), ref, got in zip(jobs, serial, results):
            for what, x, y in zip(("centroids", "assignment", "counts"), ref, got):
                assert torch.equal(x.cpu(), y.cpu()), f"rep {rep}: {name} {what} differ from the serial run"
