"""Plant plausible mistakes in a scratch copy of oracle.c, build it with gcc, and check that the
pins catch each one (a dropped term, a wrong sign, a transposed operand, a wrong tie rule, a
wrong precision, misplaced copies). The committed oracle is never modified."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from bf16_ref import bf16_rne_reference_f32_bits, bf16_rne_reference_f64
from concurrent_gemm_dma_amd import workloads as wl

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "tie_rounds_up": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "drop_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        float a",
                       "for (int64_t k = 0; k < K - 1; ++k) {\n        float a"),
    "wrong_sign": ("acc = acc + a * b;", "acc = acc - a * b;"),
    "transposed_b": ("float b = f32_from_bf16(B[k * N + j]);", "float b = f32_from_bf16(B[j * N + k]);"),
    "f64_precision": ("int q = e - 8;", "int q = e - 9;"),
    "gather_reversed": ("memcpy((unsigned char*)dst + (size_t)i * shard_bytes, shards[i], shard_bytes);",
                        "memcpy((unsigned char*)dst + (size_t)i * shard_bytes, shards[n_shards - 1 - i], shard_bytes);"),
    "a2a_not_transposed": ("const size_t to = ((size_t)j * (size_t)grid + (size_t)i) * block_bytes;",
                           "const size_t to = from;"),
    "reduce_drops_last_rank": ("for (int r = 1; r < world; ++r) {", "for (int r = 1; r < world - 1; ++r) {"),
    "reduce_starts_from_plus_zero": ("float acc = f32_from_bf16(in[0][e]);",
                                     "float acc = 0.0f + f32_from_bf16(in[0][e]);"),
    "reduce_reverse_order": ("acc = acc + f32_from_bf16(in[r][e]);",
                             "acc = f32_from_bf16(in[world - 1 - r][e]) + acc;"),
    "allreduce_wrong_slot": ("const uint16_t* from = (i == rank) ? reduced : peers[i];",
                             "const uint16_t* from = (i == 0) ? reduced : peers[i];"),
}


def _decode(h):
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _pins_pass() -> bool:
    """A compact run of the pins against whatever library `oracle` currently uses."""
    try:
        # rounding: hand cases + a structured sweep
        bits = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x7F7F8000, 0x00018000], np.uint32)
        if not np.array_equal(oracle.bf16_from_f32_bits(bits), bf16_rne_reference_f32_bits(bits)):
            return False
        x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 3.14159, -2.5e-39, 1e38], dtype=np.float64)
        if not np.array_equal(oracle.bf16_from_f64(x), bf16_rne_reference_f64(x)):
            return False
        # GEMM: square inputs (so a transposed index stays in bounds) vs fp64 brute force
        for n, k in ((6, 6), (16, 16)):
            A = wl.gen_bf16((n, k), ("normal", 0.0, 1.0), 3 + n)
            B = wl.gen_bf16((k, n), ("normal", 0.0, 1.0), 4 + n)
            exact = _decode(A).astype(np.float64) @ _decode(B).astype(np.float64)
            _, acc = oracle.gemm_f32acc(A, B, want_acc=True)
            absum = np.abs(_decode(A).astype(np.float64)) @ np.abs(_decode(B).astype(np.float64))
            gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
            if not np.all(np.abs(acc - exact) <= gamma * absum):
                return False
        # copies vs per-byte definitions
        shards = [wl.gen_bytes(7, 20 + i) for i in range(4)]
        if not np.array_equal(oracle.gather(shards), np.concatenate(shards)):
            return False
        src = wl.gen_bytes(3 * 3 * 2, 30)
        want = np.zeros_like(src)
        for i in range(3):
            for j in range(3):
                want[(j * 3 + i) * 2:(j * 3 + i) * 2 + 2] = src[(i * 3 + j) * 2:(i * 3 + j) * 2 + 2]
        if not np.array_equal(oracle.all2all_block(src, 3, 2), want):
            return False
        # reduce-scatter: hand-worked cases and exact integer sums
        for contribs, want in (([[0x3F80], [0x4B80], [0xCB80]], 0x0000),
                               ([[0x3F80], [0x3B80], [0x3B80]], 0x3F81),
                               ([[0x8000], [0x8000], [0x8000]], 0x8000)):
            got = oracle.reduce_sum_bf16([np.array(c, np.uint16) for c in contribs])
            if int(got[0]) != want:
                return False
        ints = np.random.default_rng(5).integers(-16, 17, size=(8, 64))
        enc = [((ints[r].astype(np.float32).view(np.uint32)) >> np.uint32(16)).astype(np.uint16)
               for r in range(8)]
        want = (ints.sum(axis=0).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        if not np.array_equal(oracle.reduce_sum_bf16(enc), want):
            return False
        # all-reduce slot placement (every peer slot holds a real buffer, so a wrong slot reads
        # valid memory and is caught by the comparison)
        peers = [np.full(3, 0x1000 + i, np.uint16) for i in range(4)]
        reduced, dst = oracle.allreduce_local([e[:3].copy() for e in enc[:4]], peers, 2)
        for i in range(4):
            if not np.array_equal(dst[i * 3:(i + 1) * 3], reduced if i == 2 else peers[i]):
                return False
        return True
    except Exception:
        return False


def _build(tmp_path, text, name):
    c = tmp_path / f"{name}.c"
    c.write_text(text)
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), tmp_path / "oracle.h")
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    return oracle.load_library(str(so))


def test_unmutated_passes(orc):
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(orc, tmp_path, monkeypatch, name, host_only):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation anchor for {name} not unique"
    mutant = _build(tmp_path, text.replace(before, after), name)
    monkeypatch.setattr(oracle, "_lib", mutant)
    assert not _pins_pass(), f"pins did not catch mutant {name}"
