"""Seeded synthetic inputs for the routed-expert MoE decode path.

This module is shared by the CPU oracle side (tests) and the GPU side (tests,
bench).  It only draws random bytes and random normals; it holds none of the
method's arithmetic (no dequantisation, no matvec, no routing).

Weights are drawn from a counter-based SplitMix64 stream (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
64-bit word ``i`` of a stream with key ``k`` is ``mix64(k + (i+1)*GOLDEN)``.
The same definition is implemented twice, here in numpy (host twin) and in
``fill.hip`` (GPU fill for the multi-GiB expert tensors); a GPU test checks
that both produce identical bytes.

Byte recipes (one block at a time, block index ``i`` within a tensor):

* MXFP4 (17 B / 32 weights): words ``w0, w1, w2 = word(k, 3i..3i+2)``;
  byte 0 (the E8M0 exponent) ``= 118 + ((w2 >> 32) * 17 >> 32)``, i.e.
  uniform over 118..134; bytes 1..8 and 9..16 are the little-endian bytes of
  ``w0`` and ``w1`` (each 4-bit code uniform over 16 values).
* Q2_K (84 B / 256 weights): ``w_j = word(k, 12i + j)``; bytes 0..79 are the
  little-endian bytes of ``w_0..w_9`` (scale/min nibbles and 2-bit codes,
  uniform); bytes 80..81 and 82..83 are binary16 ``d`` and ``dmin``, each
  ``f16_rne(A + B*u)`` with ``u = (w >> 40) * 2**-24`` for ``w = w_10`` and
  ``w_11``, evaluated in fp32 as one multiply then one add (A, B are the fp32
  values nearest 1e-3 and 9e-3), so ``d, dmin`` ~ U(1e-3, 1e-2).
* INT4 group-32 raw tensors (codes + BF16 scales), only for stand-alone
  matvec tests: code word ``j`` is the low/high 32 bits of ``word(k, j//2)``;
  scale ``g`` has bits ``((120 + (w >> 61)) << 7) | ((w >> 54) & 0x7F)`` for
  ``w = word(k2, g)`` (positive, exponent 2^-7..2^0, random mantissa).

Router weights and activations are normals drawn on the host with numpy's
PCG64 and are uploaded; no transcendental has to agree between host and GPU.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1

TAG_MXFP4 = 1
TAG_Q2K = 2
TAG_INT4 = 3
TAG_INT4_SCALE = 4

PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2

MXFP4_BLOCK_BYTES = 17
Q2K_BLOCK_BYTES = 84

# fp32 bit patterns of the constants nearest 1e-3 and 9e-3 (given as bits so
# that host and GPU start from the very same fp32 values).
_F32_1EM3_BITS = 0x3A83126F
_F32_9EM3_BITS = 0x3C1374BC


def _mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def stream_key(seed: int, *ids: int) -> int:
    """Key of the stream named by ``ids`` under ``seed`` (all 64-bit)."""
    k = _mix64_int(seed + GOLDEN)
    for v in ids:
        k = _mix64_int(((k ^ (v & M64)) + GOLDEN) & M64)
    return k


def tensor_key(seed: int, tag: int, layer: int, expert: int, proj: int) -> int:
    return stream_key(seed, tag, layer, expert, proj)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def words(key: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of stream ``key`` as uint64."""
    i = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GOLDEN)
    return _mix64_np(z)


def _le_bytes(w: np.ndarray) -> np.ndarray:
    return w.astype("<u8").view(np.uint8).reshape(w.shape + (8,))


def mxfp4_blocks(key: int, nblocks: int, block0: int = 0) -> np.ndarray:
    """``nblocks`` MXFP4 blocks (uint8 [nblocks, 17]) starting at block ``block0``."""
    w = words(key, 3 * block0, 3 * nblocks).reshape(nblocks, 3)
    out = np.empty((nblocks, MXFP4_BLOCK_BYTES), dtype=np.uint8)
    hi = w[:, 2] >> np.uint64(32)
    with np.errstate(over="ignore"):
        out[:, 0] = (np.uint64(118) + ((hi * np.uint64(17)) >> np.uint64(32))).astype(np.uint8)
    out[:, 1:9] = _le_bytes(w[:, 0])
    out[:, 9:17] = _le_bytes(w[:, 1])
    return out


def _f32_from_bits(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def q2k_blocks(key: int, nblocks: int, block0: int = 0) -> np.ndarray:
    """``nblocks`` Q2_K blocks (uint8 [nblocks, 84]) starting at block ``block0``."""
    w = words(key, 12 * block0, 12 * nblocks).reshape(nblocks, 12)
    out = np.empty((nblocks, Q2K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:80] = _le_bytes(w[:, 0:10]).reshape(nblocks, 80)
    a = _f32_from_bits(_F32_1EM3_BITS)
    b = _f32_from_bits(_F32_9EM3_BITS)
    two_m24 = np.float32(2.0 ** -24)
    for col, off in ((10, 80), (11, 82)):
        u = (w[:, col] >> np.uint64(40)).astype(np.float32) * two_m24
        t = (b * u).astype(np.float32)
        v = (a + t).astype(np.float32)
        out[:, off:off + 2] = v.astype(np.float16).view(np.uint8).reshape(nblocks, 2)
    return out


def int4_raw(key: int, n_rows: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Random INT4 group-32 tensor: (codes int32 [n_rows, k/8], scales uint16 [n_rows, k/32])."""
    assert k % 32 == 0
    nwords = n_rows * k // 8
    w = words(key, 0, (nwords + 1) // 2)
    codes = w.view(np.uint32)[:nwords].view(np.int32).reshape(n_rows, k // 8).copy()
    ngroups = n_rows * k // 32
    ws = words(_mix64_int(key ^ TAG_INT4_SCALE), 0, ngroups)
    exp = (np.uint64(120) + (ws >> np.uint64(61))).astype(np.uint16)
    man = ((ws >> np.uint64(54)) & np.uint64(0x7F)).astype(np.uint16)
    scales = ((exp << np.uint16(7)) | man).astype(np.uint16).reshape(n_rows, k // 32)
    return codes, scales


def expert_tensor(fmt: str, seed: int, layer: int, expert: int, proj: int,
                  n_rows: int, k: int) -> np.ndarray:
    """Bytes of one expert projection ``[n_rows, k]`` in format ``fmt``."""
    if fmt == "mxfp4":
        nb = n_rows * (k // 32)
        return mxfp4_blocks(tensor_key(seed, TAG_MXFP4, layer, expert, proj), nb).reshape(-1)
    if fmt == "q2k":
        nb = n_rows * (k // 256)
        return q2k_blocks(tensor_key(seed, TAG_Q2K, layer, expert, proj), nb).reshape(-1)
    raise ValueError(fmt)


# ---------------------------------------------------------------- normals

def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape) * std).astype(np.float32)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def router_weights(seed: int, layer: int, n_experts: int, d_model: int) -> np.ndarray:
    """Router matrix fp32 [n_experts, d_model] ~ N(0, 0.02^2)."""
    return normal_f32(stream_key(seed, 0x52, layer) & 0x7FFFFFFFFFFFFFFF,
                      (n_experts, d_model), 0.02)


def tid2eid_table(seed: int, vocab: int, n_experts: int, top_k: int) -> np.ndarray:
    """A stand-in hash table for hash-routed layers: row t holds top_k distinct
    experts of token id t, drawn from a seeded permutation (the pages do not
    give the hash function)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(n_experts)[:top_k] for _ in range(vocab)]).astype(np.int32)


def token_ids(seed: int, n_tokens: int, vocab: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, vocab, size=n_tokens).astype(np.int32)


def token_bf16(token_seed: int, n_tokens: int, d_model: int) -> np.ndarray:
    """Activations bf16 bits [n_tokens, d_model] ~ N(0, 1) rounded to bfloat16."""
    return bf16_bits_from_f32(normal_f32(token_seed, (n_tokens, d_model), 1.0))


def token_f32(token_seed: int, n_tokens: int, d_model: int) -> np.ndarray:
    return normal_f32(token_seed, (n_tokens, d_model), 1.0)


# ---------------------------------------------------------------- GPU fill

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoesynth.so")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name in ("synth_fill_mxfp4", "synth_fill_q2k"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                          ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def gpu_fill(fmt: str, dst_ptr: int, seed: int, layer: int, expert0: int, n_experts: int,
             proj: int, blocks_per_expert: int, stream: int = 0) -> None:
    """Fill ``n_experts`` consecutive expert tensors at device address ``dst_ptr``.

    Expert ``expert0 + j`` occupies ``blocks_per_expert`` blocks starting at
    ``dst_ptr + j * blocks_per_expert * block_bytes``; bytes equal
    :func:`expert_tensor` for the same (seed, layer, expert, proj).
    """
    fn = {"mxfp4": _lib().synth_fill_mxfp4, "q2k": _lib().synth_fill_q2k}[fmt]
    rc = fn(ctypes.c_void_p(dst_ptr), ctypes.c_uint64(seed), layer, expert0, n_experts, proj,
            ctypes.c_int64(blocks_per_expert), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth gpu fill failed with hip error {rc}")
