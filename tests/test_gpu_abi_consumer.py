"""The C ABI from a plain C++ program, with no Python binding and no torch.

tests/native/abi_decode.cpp (built by __graft_entry__.build() into
tests/native/abi_decode) reads one decode step's inputs from raw files,
allocates its own device buffers and stream with the HIP runtime, runs
pkv_slot_mapping, pkv_kv_append, pkv_decode_schedule and split-K
pkv_paged_decode_attention, checks that host validation refuses two bad
calls, and writes the output and both pools back. The pools must equal the
oracle's append bit for bit and the output its attention within the decode
bars (max abs 1e-2 BF16 / 3e-2 FP8, relative L2 1e-4).
"""

import os
import subprocess

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as ref

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "native", "abi_decode")
PKV_BF16, PKV_FP8 = 0, 1

CASES = [
    # lengths, n_q, n_kv, bs, dtype, partition
    ([37, 700, 1500, 1, 260], 16, 2, 16, W.BF16, 64),
    ([900, 33, 2100], 64, 8, 32, W.FP8, 128),
]


@pytest.mark.parametrize("case", CASES, ids=["bf16", "fp8"])
def test_decode_step_through_the_c_abi(case, tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.access(EXE, os.X_OK):
        # build() compiles it (and fails loudly if it cannot); a tree that was
        # not built has no library either, which every other GPU test reports
        pytest.skip(f"{EXE} is not built: run __graft_entry__.build() first")
    lens, n_q, n_kv, bs, dt, P = case
    w = W.custom("abi", lens, n_q, n_kv, 128, bs, dt, seed=2190 + CASES.index(case))
    kc, vc, ks, vs = W.make_cache(w)                   # tails and unused blocks NaN-poisoned
    q = W.make_query(w)
    k_new, v_new = W.make_new_tokens(w)
    max_ctx = int(w.context_lens.max())
    fp8 = dt == W.FP8
    header = np.array([w.B, n_q, n_kv, 128, bs, w.num_blocks, w.block_tables.shape[1],
                       PKV_FP8 if fp8 else PKV_BF16, P, max_ctx, int(fp8)], dtype=np.int32)
    with open(tmp_path / "header.bin", "wb") as f:
        f.write(header.tobytes() + np.float32(w.scale).tobytes())
    files = {"q": W.bits(q), "k": W.bits(kc), "v": W.bits(vc),
             "bt": np.ascontiguousarray(w.block_tables, dtype=np.int32),
             "cl": np.ascontiguousarray(w.context_lens, dtype=np.int32),
             "k_new": W.bits(k_new), "v_new": W.bits(v_new)}
    if fp8:
        files["k_scale"] = ks.numpy().astype(np.float32)
        files["v_scale"] = vs.numpy().astype(np.float32)
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    print(f"[abi consumer] {dt} B={w.B} P={P}", flush=True)
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "abi consumer: ok" in r.stdout

    slots = ref.slot_mapping(w.block_tables, w.context_lens - 1, bs)
    sk = None if ks is None else ks.numpy()
    sv = None if vs is None else vs.numpy()
    k_ref, v_ref = ref.kv_append(files["k"], files["v"], files["k_new"], files["v_new"], slots,
                                 dt, sk, sv)
    k_got = np.fromfile(tmp_path / "k_out.bin", dtype=k_ref.dtype).reshape(k_ref.shape)
    v_got = np.fromfile(tmp_path / "v_out.bin", dtype=v_ref.dtype).reshape(v_ref.shape)
    assert np.array_equal(k_got, k_ref) and np.array_equal(v_got, v_ref)
    expect = ref.decode_attention(files["q"], k_ref, v_ref, w.block_tables, w.context_lens,
                                  w.scale, dt, sk, sv)
    got = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(expect.shape)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - expect))
    rel = np.linalg.norm(got - expect) / np.linalg.norm(expect)
    assert err <= (3e-2 if fp8 else 1e-2) and rel <= 1e-4, (err, rel)
