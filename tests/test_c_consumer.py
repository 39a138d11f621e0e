"""The library used from plain C, with no Python or PyTorch in the process.

tests/c_consumer.c includes only include/cpattn.h (and, through it, the HIP
runtime's C API), is compiled by gcc as C11 with warnings as errors, and links
against the built libcpattn.so.  The CPU test checks that it compiles and links
(the header is valid C and every function it calls is exported); the GPU test
runs it on seeded bf16 inputs and compares what it writes with the oracle:

* attention over all keys (bf16 O and its LSE) -- the bf16 gates;
* attention over two key ranges with f32 outputs, folded by attn_merge -- the
  same gates against attention over all keys (the merge rule of Ring
  Attention's blockwise streaming, "Scaling AI inference across multiple GPUs
  using NVIDIA TensorRT with multi-device inference support", section "Ring
  Attention");
* the Ulysses pack of a [B, S_local, H, D] shard -- bit for bit against the
  oracle's relayout (same page, section "DeepSpeed Ulysses"); the program
  itself checks that the unpack restores the shard bit for bit.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

from long_sequence_bidirectional_amd import _lib, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_consumer.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libcpattn.so not built (run python -m long_sequence_bidirectional_amd.build)")
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "c_consumer")
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", libdir, "-lcpattn", f"-Wl,-rpath,{libdir}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_consumer_compiles_and_links(tmp_path):
    exe = build(tmp_path)
    assert os.path.getsize(exe) > 0


# (B, H, S, Skv, D, Skv_a): ragged query tiles and key blocks; the key split falls inside a block
SHAPES = [(1, 4, 300, 333, 128, 130), (2, 2, 257, 100, 64, 37)]


@pytest.mark.gpu
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_c_consumer_against_oracle(tmp_path, shape):
    import oracle
    from helpers import assert_bf16_parity, f64_of_bf16, log, scale_of

    B, H, S, Skv, D, Skv_a = shape
    log(f"c_consumer {shape}")
    seed = 7100 + D + S
    q = inputs.random_bf16((B, H, S, D), seed)
    k = inputs.random_bf16((B, H, Skv, D), seed + 1)
    v = inputs.random_bf16((B, H, Skv, D), seed + 2)
    scale = scale_of(D)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(struct.pack("<6qd", B, H, S, Skv, D, Skv_a, scale))
        for t in (q, k, v):
            f.write(np.ascontiguousarray(t, dtype=np.uint16).tobytes())
    exe = build(tmp_path)
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr

    n, rows = B * H * S * D, B * H * S
    raw = open(fout, "rb").read()
    assert len(raw) == n * 2 + rows * 4 + n * 4 + rows * 4 + n * 2
    off = 0

    def take(dtype, count, shape_):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off).reshape(shape_)
        off += count * np.dtype(dtype).itemsize
        return a

    o = take(np.uint16, n, (B, H, S, D))
    lse = take(np.float32, rows, (B, H, S))
    om = take(np.float32, n, (B, H, S, D))
    lm = take(np.float32, rows, (B, H, S))
    packed = take(np.uint16, n, (B, H, S, D))

    o_ref, l_ref = oracle.attention(f64_of_bf16(q), f64_of_bf16(k), f64_of_bf16(v), scale)
    assert_bf16_parity(f64_of_bf16(o), lse.astype(np.float64), o_ref, l_ref, "C program, all keys")
    assert_bf16_parity(om.astype(np.float64), lm.astype(np.float64), o_ref, l_ref,
                       f"C program, keys [0,{Skv_a}) and [{Skv_a},{Skv}) merged")
    shard = np.asarray(q).reshape(B, S, H, D)       # q's words read as a [B, S_local, H, D] shard
    ref = oracle.ulysses_pack(shard, H, oracle.SEQ_TO_HEAD)
    assert np.array_equal(packed.reshape(ref.shape), ref)
