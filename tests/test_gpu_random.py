"""Seeded random combinations of shape, sequences, masks, format, entry
point and chunk placement, each compared with the oracle.  Every case is
small (the oracle runs in milliseconds); together they cross the options the
hand-written cases take one at a time."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_movement_amd as kvm
from paged_kv_movement_amd import workloads as wl
from gpu_util import (say, setup_device, host_from_dev_pool, check_store, check_retrieve, cachegen_bins,
                      check_store_cachegen, check_retrieve_cachegen)

pytestmark = pytest.mark.gpu

N_CASES = 600
FORMATS = [kvm.FMT_BF16, kvm.FMT_FP8, kvm.FMT_FP8_E5M2, kvm.FMT_K16_V8, kvm.FMT_CACHEGEN]


def _case(i):
    rng = np.random.default_rng(9000 + i)
    L = int(rng.integers(1, 6))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([8, 16, 24, 64, 128]))
    P = int(rng.choice([16, 32]))
    C = P * int(rng.choice([1, 2, 8, 16]))
    n_seqs = int(rng.integers(1, 5))
    ranges, masks = [], []
    for _ in range(n_seqs):
        s = C * int(rng.integers(0, 3))
        e = s + int(rng.integers(0, 4 * C + 1))
        n_ch = -(-(e - s) // C)
        m = (rng.random(n_ch) < 0.8).astype(np.uint8)
        ranges.append((s, e))
        masks.append(m)
    pages_needed = sum(-(-e // P) for (_, e) in ranges)
    num_pages = pages_needed + int(rng.integers(1, 64))
    fmt = FORMATS[int(rng.integers(0, len(FORMATS)))]
    store_form = rng.choice(["full", "planned", "layers", "layer-range", "layer-range-2s"]) \
        if fmt != kvm.FMT_CACHEGEN \
        else "full"
    retrieve_form = rng.choice(["chunk", "ordered", "layers", "layer-range", "layer-range-2s"]) \
        if fmt != kvm.FMT_CACHEGEN else rng.choice(["chunk", "ordered"])
    where = rng.choice(["device", "device", "host"])
    cap = int(rng.choice([0, 0, 1, 3, 17]))
    w = wl.custom(f"rand{i}", 9000 + i, L, H, D, num_pages, ranges, masks=masks, page_size=P, chunk_size=C,
                  outliers=0 if fmt == kvm.FMT_BF16 else min(2, H * D))
    return w, fmt, str(store_form), str(retrieve_form), str(where), cap


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    w, fmt, store_form, retrieve_form, where, cap = _case(i)
    say("random case", i, "L H D P C", w.num_layers, w.num_kv_heads, w.head_dim, w.page_size, w.chunk_size,
        "seqs", [(s.tok_start, s.tok_end) for s in w.seqs], "fmt", fmt, store_form, retrieve_form, where, "cap", cap)
    arr = wl.host_pool(w)
    pool, paged, batch, cs = setup_device(w, arr, fmt=fmt, fill=0xCD, where=where)
    masks = [sq.hit_mask for sq in w.seqs]
    s = torch.cuda.Stream()
    if fmt == kvm.FMT_CACHEGEN:
        kb, vb = cachegen_bins(w.num_layers, 9000 + i)
        kvm.store_cachegen(paged, batch, kb, vb, stream=s)
    elif store_form == "full":
        kvm.store(paged, batch, fmt, stream=s)
    elif store_form == "planned":
        kvm.store(paged, batch, fmt, stream=s, workspace=batch.new_store_workspace(fmt))
    elif store_form.startswith("layer-range"):
        # every layer in one call, the first at full width and the rest
        # capped; with "-2s" every other layer on a second stream
        kvm.store_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=s,
                         max_workgroups=[0] + [cap] * (w.num_layers - 1),
                         alt_stream=torch.cuda.Stream() if store_form.endswith("-2s") else None)
    else:
        for l in range(w.num_layers):
            kvm.store_layer(paged, batch, l, fmt=fmt, stream=s, max_workgroups=cap)
    s.synchronize()
    assert kvm.take_faults() == 0
    if fmt == kvm.FMT_CACHEGEN:
        check_store_cachegen(w, arr, cs, kb, vb)
    else:
        check_store(w, arr, cs, fmt)
    pool.view(torch.int16).fill_(0x7E57)
    s.wait_stream(torch.cuda.current_stream())       # the fill lands before the retrieve writes
    ws = paged.new_workspace() if retrieve_form == "ordered" else None
    if fmt == kvm.FMT_CACHEGEN:
        n = kvm.retrieve_cachegen(paged, batch, kb, vb, stream=s, workspace=ws)
    elif retrieve_form == "layers":
        for l in range(w.num_layers):
            n = kvm.retrieve_layer_ex(paged, batch, l, fmt=fmt, stream=s, max_workgroups=cap)
    elif retrieve_form.startswith("layer-range"):
        n = kvm.retrieve_layers(paged, batch, 0, w.num_layers, fmt=fmt, stream=s,
                                max_workgroups=[0] + [cap] * (w.num_layers - 1),
                                alt_stream=torch.cuda.Stream() if retrieve_form.endswith("-2s") else None)
    else:
        n = kvm.retrieve(paged, batch, fmt=fmt, stream=s, workspace=ws)
    s.synchronize()
    assert kvm.take_faults() == 0
    before = np.full_like(arr, 0x7E57)
    got = host_from_dev_pool(pool)
    if fmt == kvm.FMT_CACHEGEN:
        counts = check_retrieve_cachegen(w, before, got, cs, masks, kb, vb)
    else:
        counts = check_retrieve(w, before, got, cs, fmt, masks)
    assert n == counts
