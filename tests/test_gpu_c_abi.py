"""The C ABI from plain C: tests/abi_c_example.c (built by the build step)
stores a sequence (kv_store_chunks, kv_store_chunks_ws, kv_store_layers on
two streams), clears the pool and restores it (kv_retrieve_chunks,
kv_retrieve_layer, kv_retrieve_chunks_ws, kv_retrieve_chunks_noalloc,
kv_retrieve_layers on two streams), checking the rows itself."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXAMPLE = os.path.join(ROOT, "tests", "abi_c_example")


def test_c_program_round_trip():
    if not os.path.exists(EXAMPLE):
        pytest.fail(f"{EXAMPLE} is missing: build it with __graft_entry__.build() "
                    "(paged_kv_movement_amd.build.build_c_example)")
    print("case C ABI example", flush=True)
    r = subprocess.run([EXAMPLE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "restored bit for bit" in r.stdout and "layer ranges on two streams both ways" in r.stdout
