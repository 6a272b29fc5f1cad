"""GPU routing (moe_route) against the oracle's plain definition of the
expert-sorted order, on both launch paths: one workgroup when every
assignment fits one 1024-key chunk, the sort / scan / scatter passes beyond.

Sizes straddle the chunk boundary (1023, 1024, 1025) and reach several
chunks with a ragged last one; ids include values outside [0, E), which no
expert segment may hold. Offsets and the valid prefix of sorted2assign must
match the oracle bit for bit, and tile offsets must be the prefix sums of
ceil(n_e / 256)."""
import numpy as np
import pytest

import oracle
import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import host, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ids(A, E, seed, invalid_frac=0.05):
    g = synth.rng(95, 0, seed)
    ids = g.integers(0, E, size=A).astype(np.int32)
    bad = g.random(A) < invalid_frac
    ids[bad] = g.choice(np.array([-2, -1, E, E + 1], np.int32), size=int(bad.sum()))
    return ids


@pytest.mark.parametrize("A,E", [(1, 8), (5, 1), (512, 8), (1023, 384), (1024, 384), (1025, 384),
                                 (1024, 4096), (3000, 7), (5000, 4096), (2048, 1),
                                 # chunk columns split over 2-4 threads, ragged last part; one too wide for that
                                 (70000, 384), (66000, 1), (200000, 7), (100000, 600)])
def test_route_against_oracle(A, E):
    print(f"[route] A={A} E={E}", flush=True)
    ids = _ids(A, E, seed=A + E)
    offs, s2a, tiles = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    n_valid = int(o_offs[-1])
    assert np.array_equal(host(offs), o_offs)
    assert np.array_equal(host(s2a)[:n_valid], o_s2a[:n_valid])
    n_e = np.diff(o_offs)
    assert np.array_equal(host(tiles), np.concatenate([[0], np.cumsum((n_e + 255) // 256)]))


def test_route_no_assignments():
    # A = 0 through the C ABI (a valid ids pointer, no entries): empty segments
    import torch
    E = 16
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    tiles = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    s2a = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    L = nvq.lib()
    ws = torch.empty(L.moe_route_workspace_size(0, E), dtype=torch.uint8, device="cuda")
    rc = L.moe_route(ids.data_ptr(), 0, E, offs.data_ptr(), s2a.data_ptr(), tiles.data_ptr(), ws.data_ptr(),
                     ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert np.array_equal(host(offs), np.zeros(E + 1, np.int32))
    assert np.array_equal(host(tiles), np.zeros(E + 1, np.int32))
    assert host(s2a)[0] == -7


def test_route_one_chunk_all_to_one_expert_and_repeat():
    # every assignment on the last expert, then the same ids again: the
    # single-workgroup path must give the same bytes on every call
    A, E = 1000, 384
    ids = np.full(A, E - 1, np.int32)
    first = [host(t) for t in nvq.moe_route(to_dev(ids), E)]
    o_offs, o_s2a = oracle.route(ids, E)
    assert np.array_equal(first[0], o_offs) and np.array_equal(first[1], o_s2a)
    for _ in range(3):
        again = [host(t) for t in nvq.moe_route(to_dev(ids), E)]
        assert all(np.array_equal(a, b) for a, b in zip(first, again))
