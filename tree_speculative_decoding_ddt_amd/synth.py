"""Seeded synthetic inputs for the verify step.

This module only draws random numbers and lays them out; it holds none of the
step's own arithmetic (no softmax, no top-K, no tree build, no attention, no
recurrence).  Both the HIP path's tests/benchmarks and the CPU oracle's tests
take their inputs from here.

Distributions follow the workloads stated for this step (all seeded):
  * drafter logits  N(0, sigma) per entry, optionally with a planted peak of
    +8 above the row maximum at a uniformly chosen token, per (sequence, depth)
    with probability p (mixed confident and uncertain depths);
  * target logits   N(0, sigma), and with probability p per (sequence, depth d)
    every tree row at depth d gets the drafter's top-1 token of depth d+1
    raised to its row maximum + 1;
  * attention Q/K/V N(0, 1); GDN x, v, committed conv state N(0, 1); committed
    S  N(0, 1)/sqrt(dk); beta U(0, 1); g U(0.9, 1); conv weights
    U(-1/sqrt(W), 1/sqrt(W)).
bf16 arrays are returned as their uint16 bit patterns (round-to-nearest-even
from float32) so that torch can view them as bfloat16 without a copy.
"""

import numpy as np

# ---------------------------------------------------------------- bf16 bits

def to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def from_bf16_bits(b):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize(x, dtype):
    """Round float32 data to the storage dtype and return (storage, float32 view).

    dtype "f32" keeps float32; "bf16" returns uint16 bit patterns plus their
    exact float32 decoding (what a reader of the stored bytes sees)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x, x
    if dtype == "bf16":
        bits = to_bf16_bits(x)
        return bits, from_bf16_bits(bits)
    raise ValueError(dtype)


# ---------------------------------------------------------------- drafter / target

def draft_logits(rng, n, L, V, sigma, plant_p=None, plant_gap=8.0):
    """[n][L][V] float32; row d is the drafter's distribution for depth d+1."""
    z = (sigma * rng.standard_normal((n, L, V))).astype(np.float32)
    if plant_p is not None:
        hit = rng.random((n, L)) < plant_p
        where = rng.integers(0, V, size=(n, L))
        for s in range(n):
            for d in range(L):
                if hit[s, d]:
                    z[s, d, where[s, d]] = z[s, d].max() + plant_gap
    return z


def draft_top1(z):
    """Drafter top-1 token per (sequence, depth): first index of the row maximum."""
    return np.argmax(z, axis=-1)


def target_logits(rng, n, T, V, sigma, depth, top1, plant_p):
    """[n][T][V] float32 target logits with planted argmaxes.

    depth [n][T] is the depth of every tree row (-1 for unused rows) and
    top1 [n][L] the drafter's top-1 token per depth.  With probability
    plant_p per (sequence, depth d < L), every row at depth d gets
    logit[top1[d]] = row max + 1, i.e. the target agrees with the drafter's
    first choice one level further down.
    """
    y = (sigma * rng.standard_normal((n, T, V))).astype(np.float32)
    L = top1.shape[1]
    hit = rng.random((n, L)) < plant_p
    for s in range(n):
        for i in range(T):
            d = int(depth[s][i])
            if 0 <= d < L and hit[s, d]:
                y[s, i, top1[s, d]] = y[s, i].max() + 1.0
    return y


# ---------------------------------------------------------------- topologies

def lopsided_parents(L=15, side_a=25, side_b=24):
    """Parent and depth arrays of the long-context test tree: rows 1..L form a
    chain at depths 1..L, then side_a extra children of the depth-2 chain node
    (row 2, so depth 3) and side_b extra children of the depth-3 chain node
    (row 3, so depth 4).  Every parent row precedes its children."""
    parent = [-1] + [d - 1 for d in range(1, L + 1)] + [2] * side_a + [3] * side_b
    depth = [0] + list(range(1, L + 1)) + [3] * side_a + [4] * side_b
    return np.array(parent, dtype=np.int64), np.array(depth, dtype=np.int64)


def distinct_tokens(rng, T, V):
    """T distinct random token ids (row 0 included)."""
    return rng.choice(V, size=T, replace=False).astype(np.int64)


def random_parents(rng, B, L):
    """A random prefix-closed tree of B nodes (plus root) with depth <= L; rows are
    numbered so that every parent precedes its children."""
    parent = [-1]
    depth = [0]
    for i in range(1, B + 1):
        cands = [j for j in range(i) if depth[j] < L]
        p = int(cands[rng.integers(0, len(cands))])
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.array(parent, dtype=np.int64), np.array(depth, dtype=np.int64)


# ---------------------------------------------------------------- layer inputs

def attention_inputs(rng, n, T, Hq, Hkv, D, Pmax):
    """q [n][T][Hq][D], k/v_cache [n][Hkv][Pmax][D], k/v_tree [n][Hkv][T][D] (float32)."""
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(q=f(n, T, Hq, D), k_cache=f(n, Hkv, Pmax, D), v_cache=f(n, Hkv, Pmax, D),
                k_tree=f(n, Hkv, T, D), v_tree=f(n, Hkv, T, D))


def gdn_inputs(rng, n, T, H, dk, dv, W):
    """x [n][T][C], v [n][T][H][dv], beta, g [n][T][H], S [n][H][dv][dk],
    conv_state [n][W-1][C], conv_w [C][W] with C = 2*H*dk (float32)."""
    C = 2 * H * dk
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(
        x=f(n, T, C), v=f(n, T, H, dv),
        beta=rng.random((n, T, H)).astype(np.float32),
        g=(0.9 + 0.1 * rng.random((n, T, H))).astype(np.float32),
        S=(rng.standard_normal((n, H, dv, dk)) / np.sqrt(dk)).astype(np.float32),
        conv_state=f(n, W - 1, C),
        conv_w=rng.uniform(-1 / np.sqrt(W), 1 / np.sqrt(W), size=(C, W)).astype(np.float32),
    )
