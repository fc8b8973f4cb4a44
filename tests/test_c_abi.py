"""The C ABI from a plain C program (tests/c_abi_example.c), with no Python between the
caller and the library: the host block manager and metadata builders on the pages'
worked examples (CPU), and one KV write plus one paged decode with device memory taken
from the HIP runtime (GPU), checked against the oracle."""

from __future__ import annotations

import json
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

from paged_kv_cache_73_amd import _native
from paged_kv_cache_73_amd import workloads as W

from tests import harness as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
LIB_DIR = os.path.dirname(_native.LIB_PATH)


def _build(tmp_path, gpu: bool) -> str:
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    if not os.path.exists(_native.LIB_PATH):
        pytest.skip("libpa.so is not built")
    exe = str(tmp_path / ("c_abi_gpu" if gpu else "c_abi_host"))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include")]
    if gpu:
        cmd += ["-DPA_EXAMPLE_GPU", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]
    cmd += [SRC, "-o", exe, "-L", LIB_DIR, "-l:libpa.so", f"-Wl,-rpath,{LIB_DIR}"]
    if gpu:
        cmd += ["-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=120)
    return exe


def test_c_program_host_calls(tmp_path, golden):
    exe = _build(tmp_path, gpu=False)
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60, check=True)
    got = json.loads(r.stdout)
    assert got["abi_version"] == _native.lib().pa_abi_version()
    # block table [3, 1, 5] with block size 4: the pages print which tokens each block holds
    bt = golden("block_table_example.json")
    expect = {}
    for phys, tokens in bt["printed_layout"].items():
        for off, tok in enumerate(tokens):
            expect[tok] = int(phys) * bt["block_size"] + off
    assert got["slots_of_tokens_0_to_9"] == [expect[t] for t in range(10)]
    # varlen metadata as printed for query lengths [10, 3, 1] and key lengths [0, 1, 7]
    vx = golden("varlen_example.json")
    assert got["cu_seqlens_q"] == vx["printed_cu_seq_lens_q"]
    assert got["cu_seqlens_k"] == vx["printed_cu_seq_lens_k"]
    assert (got["max_q"], got["max_k"]) == (vx["printed_max_length_q"], vx["printed_max_length_k"])
    # free blocks are handed out 0, 1, 2, ...; sharing adds a reference; writing into the
    # shared, partly filled block copies it to a new block; releasing both rows frees all
    assert got["row_a"] == [0, 1, -1, -1]
    assert got["refs_after_share"] == [2, 2]
    assert got["row_b_after_write"] == [0, 2, -1, -1]
    assert (got["cow_src"], got["cow_dst"]) == ([1], [2])
    assert got["refs_after_cow"] == [2, 1, 1]
    assert got["free_after_release"] == 8
    assert got["alloc_9_of_8"] == "PA_ERR_OUT_OF_BLOCKS"
    assert (got["validate_bad_table"], got["bad_index"]) == ("PA_ERR_METADATA", 0)


@pytest.mark.gpu
def test_c_program_decode_on_the_gpu(tmp_path):
    exe = _build(tmp_path, gpu=True)
    w = W.tiny_decode(seed=0)
    o = H.oracle_run(w)
    p = o.plan
    table = np.asarray(p.tables, dtype=np.int32)
    hdr = [w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.batch, w.num_heads,
           table.shape[1], len(p.new_slots), max(p.seqlens_k)]
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<9i", *hdr) + struct.pack("<f", w.scale))
        for a in (o.k_pool_ctx, o.v_pool_ctx, H.storage(w.q, "f32"), H.storage(w.k_new, "f32"),
                  H.storage(w.v_new, "f32")):
            f.write(np.ascontiguousarray(a, dtype=np.float32).tobytes())
        for a in (table, p.seqlens_k, p.new_slots):
            f.write(np.ascontiguousarray(a, dtype=np.int32).tobytes())
    r = subprocess.run([exe, "gpu", str(inp), str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(out, dtype=np.float32).reshape(o.out.shape).astype(np.float64)
    H.assert_close(got, o.out, "f32", "decode from C")
