"""Philox4x64-10 counter-based generator and the canvas token draw (oracle side).

Test infrastructure: only the tests, the package's smoke check and the bench's
CPU-baseline leg use this package; the GPU library never imports or links it.

Source of the generator: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 4 (the Philox
family): a 4-word, 64-bit-lane counter is permuted by 10 rounds of
multiply-high/low and xor with a 2-word key that is advanced by the Weyl
constants between rounds.  Written here from the paper's description.

Where it is used in the method: each denoising step re-randomizes the
positions of the 256-token canvas that were not accepted, and a new canvas
starts filled with random tokens ("DiffusionGemma hits ~1,500 TPS on one
H100", sections "What DiffusionGemma is" and "How the sampler actually
works"; "Google open-sources DiffusionGemma", section "Time for
Autoregressive Models to be Challenged").  The pages do not say how the
random tokens are drawn.  Reading taken: one Philox4x64-10 call per
(position, step, block) with key (seed, 0) and counter
(position, step, block, 0); the token is the high 64 bits of r0 * V, i.e.
floor(r0 * V / 2^64), using only the first output word r0.  Step 0 is the
canvas initialisation, step s >= 1 the re-draw after denoising step s.
"""
import numpy as np

MASK64 = (1 << 64) - 1
# Multipliers and Weyl key increments of Philox4x64 (SC'11, table of constants).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
ROUNDS = 10

_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a, b):
    """Full 64x64 -> 128-bit product of uint64 arrays, as (hi, lo).

    numpy has no 128-bit integers, so the product is assembled from 32-bit
    halves (schoolbook multiplication)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    a_lo, a_hi = a & _LO32, a >> _S32
    b_lo, b_hi = b & _LO32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO32) + (hl & _LO32)  # < 3 * 2^32, no overflow
    lo = (ll & _LO32) | ((mid & _LO32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(counter, key):
    """Apply Philox4x64-10 to counters.

    counter: uint64 array of shape [..., 4]; key: uint64 array of shape [..., 2]
    (broadcastable).  Returns uint64 array [..., 4].  One round maps
    (c0, c1, c2, c3) with key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
    the key gains (W0, W1) before every round after the first.
    """
    c = np.array(counter, dtype=np.uint64)
    k = np.array(key, dtype=np.uint64)
    batch = np.broadcast_shapes(c.shape[:-1], k.shape[:-1])
    c = np.broadcast_to(c, batch + (4,)).copy()
    k0 = np.broadcast_to(k[..., 0], batch).copy()
    k1 = np.broadcast_to(k[..., 1], batch).copy()
    with np.errstate(over="ignore"):
        for r in range(ROUNDS):
            if r > 0:
                k0 = k0 + np.uint64(PHILOX_W0)
                k1 = k1 + np.uint64(PHILOX_W1)
            hi0, lo0 = _mulhilo64(np.uint64(PHILOX_M0), c[..., 0])
            hi1, lo1 = _mulhilo64(np.uint64(PHILOX_M1), c[..., 2])
            c = np.stack([hi1 ^ c[..., 1] ^ k0, lo1, hi0 ^ c[..., 3] ^ k1, lo0], axis=-1)
    return c


def draw_tokens(seed, block, step, positions, vocab):
    """Uniform token ids in [0, vocab) for the given canvas positions.

    Counter (position, step, block, 0), key (seed, 0); token = hi64(r0 * vocab).
    Returns int64 array shaped like `positions`.
    """
    pos = np.asarray(positions, dtype=np.uint64)
    ctr = np.zeros(pos.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = pos
    ctr[..., 1] = np.uint64(step)
    ctr[..., 2] = np.uint64(block)
    key = np.array([seed & MASK64, 0], dtype=np.uint64)
    r = philox4x64_10(ctr, key)
    hi, _ = _mulhilo64(r[..., 0], np.uint64(vocab))
    return hi.astype(np.int64)
