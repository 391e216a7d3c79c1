"""Seeded synthetic inputs for the tensor-product convolution and the
symmetric contraction.

This module serves the tests, ``bench.py`` and ``__graft_entry__.smoke()``
alike.  It holds none of the method's arithmetic: no coupling coefficients,
paths, offsets, contractions or reductions.  What it computes is input
synthesis only: random draws, graph construction (a distance cutoff), and
the real spherical harmonics of edge vectors, which are the *values* of the
second operand (the workloads take "edge SH of random unit vectors").  Those
harmonics are a hand-written Cartesian table (textbook real basis, component
normalisation, m = -l..l, l <= 3); the tests check it against the oracle's
independently pinned harmonics.  Anything that depends on the descriptor
(the fan-in of each weight column) is passed in by the caller.

Draw order for every workload: geometry (sources, positions, edge vectors),
then node features, then weights, then species.  One ``numpy.random``
generator seeded ``1000 + workload number`` per workload.  float64 runs draw
in float64; float32 runs draw float32 normals directly.
"""

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class TPWorkload:
    number: int
    name: str
    irreps_in1: str
    irreps_in2: str
    irreps_out: str          # type filter
    layouts: tuple
    dtype: str               # "f32" or "f64"
    kind: str                # "batch", "molecules", "graph"
    n_nodes: int = 0
    n_edges: int = 0
    degree: int = 0
    batch: int = 0
    molecules: int = 0
    atoms_per_molecule: int = 0
    box: float = 0.0
    cutoff: float = 0.0
    sh_ls: tuple = ()
    fan_in_scaled: bool = True


@dataclass(frozen=True)
class SymconWorkload:
    number: int
    name: str
    irreps_in: str
    irreps_out: str
    layouts: tuple
    dtype: str
    n_atoms: int
    num_elements: int
    degrees: tuple = field(default=(1, 2, 3))


@dataclass(frozen=True)
class LinearWorkload:
    number: int
    name: str
    irreps_in: str
    irreps_out: str
    layouts: tuple
    dtype: str
    n: int
    num_classes: int = 0     # 0: shared weights; else class-indexed, classes sorted


@dataclass(frozen=True)
class FCWorkload:
    number: int
    name: str
    irreps_in1: str
    irreps_in2: str
    irreps_out: str
    layouts: tuple
    dtype: str
    n: int
    per_sample: bool = False  # one weight row per sample [n, numel] (else one shared row)


@dataclass(frozen=True)
class FCConvWorkload:
    number: int
    name: str
    irreps_in1: str
    irreps_sh: str
    irreps_out: str
    layouts: tuple
    dtype: str
    n_nodes: int
    degree: int
    sh_ls: tuple


# the output irreps of the 600k-edge convolution (13 blocks, 5,504 values per
# node), written out: the linear layer that follows the convolution mixes
# them back to 128 channels per type
CONV4_OUT = ("128x0e+128x0e+128x0e+128x1o+128x1o+128x1o+128x1o+128x1o+"
             "128x2e+128x2e+128x2e+128x2e+128x2e")

WORKLOADS = {
    1: TPWorkload(1, "single_tp_batch64_f64", "8x0e+8x1o", "0e+1o+2e",
                  "0e+0o+1e+1o+2e+2o", ("mul_ir",), "f64", "batch", batch=64,
                  sh_ls=(0, 1, 2), fan_in_scaled=False),
    2: TPWorkload(2, "molecules_64x21_cut5", "32x0e+32x1o", "0e+1o+2e",
                  "0e+1o+2e", ("mul_ir",), "f32", "molecules", molecules=64,
                  atoms_per_molecule=21, box=6.0, cutoff=5.0, sh_ls=(0, 1, 2)),
    3: TPWorkload(3, "graph_2k_nodes_32k_edges", "64x0e+64x1o+64x2e", "0e+1o+2e+3o",
                  "0e+0o+1e+1o+2e+2o", ("ir_mul",), "f32", "graph", n_nodes=2000,
                  n_edges=32000, degree=16, sh_ls=(0, 1, 2, 3)),
    4: TPWorkload(4, "graph_20k_nodes_600k_edges", "128x0e+128x1o+128x2e", "0e+1o+2e+3o",
                  "0e+1o+2e", ("mul_ir", "ir_mul"), "f32", "graph", n_nodes=20000,
                  n_edges=600000, degree=30, sh_ls=(0, 1, 2, 3)),
    5: SymconWorkload(5, "symcon_50k_atoms_10_species", "128x0e+128x1o+128x2e+128x3o",
                      "128x0e+128x1o", ("ir_mul", "mul_ir"), "f32", n_atoms=50000,
                      num_elements=10),
    6: LinearWorkload(6, "linear_after_conv_20k_nodes", CONV4_OUT, "128x0e+128x1o+128x2e",
                      ("ir_mul", "mul_ir"), "f32", n=20000),
    7: LinearWorkload(7, "species_linear_50k_atoms_10_species", "128x0e+128x1o+128x2e+128x3o",
                      "128x0e+128x1o+128x2e+128x3o", ("ir_mul", "mul_ir"), "f32", n=50000,
                      num_classes=10),
    # the fully connected product of the skill document's example (irreps x
    # irreps -> irreps) at the 32-channel scalar + vector irreps of Lesson
    # 12a's exercise 1, one row per node of a 100k-node batch
    8: FCWorkload(8, "fctp_uvw_32x0e+32x1o_100k", "32x0e+32x1o", "32x0e+32x1o", "32x0e+32x1o",
                  ("mul_ir", "ir_mul"), "f32", n=100000),
    # the fully connected product as a convolution with one weight row per
    # edge (the skill document's FullyConnectedTensorProductConv), 16-channel
    # scalar + vector features and l <= 2 harmonics on the 20k-node graph
    9: FCConvWorkload(9, "fctp_conv_20k_nodes_600k_edges", "16x0e+16x1o", "0e+1o+2e", "16x0e+16x1o",
                      ("mul_ir", "ir_mul"), "f32", n_nodes=20000, degree=30, sh_ls=(0, 1, 2)),
    # the fully connected product with external weights, one row per sample
    # (the skill document's shared_weights=False), 16-channel scalar + vector
    # features times 8-channel scalar + vector attributes over a 20k batch:
    # 8,192 weights (32 KB) per sample
    10: FCWorkload(10, "fctp_per_sample_16x0e+16x1o_x_8x0e+8x1o_20k", "16x0e+16x1o", "8x0e+8x1o",
                   "16x0e+16x1o", ("mul_ir", "ir_mul"), "f32", n=20000, per_sample=True),
}


def _np_dtype(dt):
    return {"f32": np.float32, "f64": np.float64}[dt]


def _normal(rng, shape, dt):
    if dt == "f64":
        return rng.standard_normal(shape)
    return rng.standard_normal(shape, dtype=np.float32)


# --------------------------------------------------------------------------
# real spherical harmonics of unit vectors, Cartesian table, l <= 3
# --------------------------------------------------------------------------

def edge_harmonics(vecs, ls):
    """Real harmonics (component normalisation, sum_m Y_lm^2 = 2l+1) of the
    normalised vectors, degrees ``ls`` concatenated.  Textbook table."""
    v = np.asarray(vecs, dtype=np.float64)
    v = v / np.linalg.norm(v, axis=-1, keepdims=True)
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    cols = []
    for l in ls:
        if l == 0:
            cols += [np.ones_like(x)]
        elif l == 1:
            s3 = math.sqrt(3.0)
            cols += [s3 * y, s3 * z, s3 * x]
        elif l == 2:
            s15 = math.sqrt(15.0)
            cols += [s15 * x * y, s15 * y * z, 0.5 * math.sqrt(5.0) * (3 * z * z - 1),
                     s15 * x * z, 0.5 * s15 * (x * x - y * y)]
        elif l == 3:
            a = math.sqrt(35.0 / 8.0)
            b = math.sqrt(105.0)
            c = math.sqrt(21.0 / 8.0)
            d = 0.5 * math.sqrt(7.0)
            cols += [a * y * (3 * x * x - y * y), b * x * y * z, c * y * (5 * z * z - 1),
                     d * z * (5 * z * z - 3), c * x * (5 * z * z - 1),
                     0.5 * b * z * (x * x - y * y), a * x * (x * x - 3 * y * y)]
        else:
            raise ValueError("edge harmonics are tabulated for l <= 3")
    return np.stack(cols, axis=-1)


def _irreps_dim(s):
    """Dimension of an irreps string (sum mul*(2l+1)); string arithmetic only."""
    d = 0
    for term in s.split("+"):
        term = term.strip()
        mul, rest = (term.split("x") + [None])[:2] if "x" in term else (1, term)
        d += int(mul) * (2 * int(rest[:-1]) + 1)
    return d


def fan_in_from_irreps_out(irreps_out):
    """Per weight column of a channelwise product: the number of output
    blocks of the same irrep type.  Pure string bookkeeping on the output
    irreps the descriptor reports (one weight segment per output block, in
    output order, ``mul`` wide)."""
    blocks = []
    for term in irreps_out.split("+"):
        mul, typ = term.strip().split("x")
        blocks.append((int(mul), typ))
    cnt = {}
    for _, t in blocks:
        cnt[t] = cnt.get(t, 0) + 1
    return np.concatenate([np.full(m, cnt[t], dtype=np.float64) for m, t in blocks])


# --------------------------------------------------------------------------
# graphs
# --------------------------------------------------------------------------

def molecule_graph(rng, molecules, atoms, box, cutoff):
    """Independent molecules, positions uniform in a cube of side ``box``;
    every ordered pair (src != dst) of one molecule closer than ``cutoff`` is
    an edge.  Edges are sorted by dst, then src.  Returns src, dst, vectors
    r = pos[dst] - pos[src], n_nodes."""
    pos = rng.uniform(0.0, box, size=(molecules, atoms, 3))
    src_l, dst_l, vec_l = [], [], []
    for m in range(molecules):
        p = pos[m]
        d = p[None, :, :] - p[:, None, :]          # d[s, t] = p[t] - p[s]
        dist = np.linalg.norm(d, axis=-1)
        s, t = np.nonzero((dist < cutoff) & ~np.eye(atoms, dtype=bool))
        order = np.lexsort((s, t))                   # by dst t, then src s
        s, t = s[order], t[order]
        src_l.append(s + m * atoms)
        dst_l.append(t + m * atoms)
        vec_l.append(d[s, t])
    return (np.concatenate(src_l), np.concatenate(dst_l), np.concatenate(vec_l),
            molecules * atoms)


def regular_graph(rng, n_nodes, degree):
    """dst = repeat(arange(n), degree) (sorted), src uniform with replacement
    (self-loops and repeated pairs allowed), random edge directions."""
    dst = np.repeat(np.arange(n_nodes), degree)
    src = rng.integers(0, n_nodes, size=dst.shape[0])
    vec = rng.standard_normal((dst.shape[0], 3))
    return src, dst, vec


def ragged_graph(rng, n_nodes, max_degree, n_src=None, empty_fraction=0.2):
    """A dst-sorted graph with in-degrees uniform in 0..max_degree and a
    fraction of isolated destinations (edge cases of the scatter)."""
    n_src = n_nodes if n_src is None else n_src
    deg = rng.integers(0, max_degree + 1, size=n_nodes)
    deg[rng.random(n_nodes) < empty_fraction] = 0
    dst = np.repeat(np.arange(n_nodes), deg)
    src = rng.integers(0, n_src, size=dst.shape[0])
    vec = rng.standard_normal((dst.shape[0], 3))
    return src, dst, vec


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------

def tp_inputs(wl, fan_in=None, n_nodes=None, degree=None, graph=None, seed=None):
    """Inputs of a channelwise-product workload as numpy arrays.

    ``fan_in`` (per weight column, from the descriptor) scales the weights
    by 1/sqrt(fan_in) when the workload asks for it.  ``n_nodes``/``degree``
    shrink a "graph" workload keeping its structure; ``graph="ragged"``
    replaces it by :func:`ragged_graph` with max in-degree ``degree``.
    Returns dict(x, sh, w, src, dst, n_nodes, n_src, vec); vec holds the
    edge vectors the harmonics were computed from (cast to the run dtype)."""
    rng = np.random.default_rng(1000 + wl.number if seed is None else seed)
    dt = _np_dtype(wl.dtype)
    if wl.kind == "batch":
        n = wl.batch if n_nodes is None else n_nodes
        vec = rng.standard_normal((n, 3))
        src = dst = None
        n_out, n_src = n, n
    elif wl.kind == "molecules":
        src, dst, vec, n_out = molecule_graph(rng, wl.molecules, wl.atoms_per_molecule,
                                              wl.box, wl.cutoff)
        n_src = n_out
    else:
        nn = wl.n_nodes if n_nodes is None else n_nodes
        dg = wl.degree if degree is None else degree
        if graph == "ragged":
            src, dst, vec = ragged_graph(rng, nn, dg)
        else:
            src, dst, vec = regular_graph(rng, nn, dg)
        n_out, n_src = nn, nn
    sh = edge_harmonics(vec, wl.sh_ls).astype(dt)
    x = _normal(rng, (n_src, _irreps_dim(wl.irreps_in1)), wl.dtype).astype(dt, copy=False)
    if fan_in is None:
        raise ValueError("fan_in (weight_numel values) is required")
    fan_in = np.asarray(fan_in, dtype=np.float64)
    w = _normal(rng, (sh.shape[0], fan_in.shape[0]), wl.dtype)
    if wl.fan_in_scaled:
        w = w * (1.0 / np.sqrt(fan_in)).astype(w.dtype)
    w = w.astype(dt, copy=False)
    out = dict(x=x, sh=sh, w=w, n_nodes=n_out, n_src=n_src, src=None, dst=None, vec=vec.astype(dt))
    if src is not None:
        out["src"] = src.astype(np.int32)
        out["dst"] = dst.astype(np.int32)
    return out


def symcon_inputs(wl, fan_in, n_atoms=None, seed=None):
    """Inputs of a symmetric-contraction workload: x, species (int32), w.
    ``fan_in`` per weight column is K of its (degree, output block)."""
    rng = np.random.default_rng(1000 + wl.number if seed is None else seed)
    dt = _np_dtype(wl.dtype)
    n = wl.n_atoms if n_atoms is None else n_atoms
    x = _normal(rng, (n, _irreps_dim(wl.irreps_in)), wl.dtype).astype(dt, copy=False)
    fan_in = np.asarray(fan_in, dtype=np.float64)
    w = _normal(rng, (wl.num_elements, fan_in.shape[0]), wl.dtype)
    w = (w * (1.0 / np.sqrt(fan_in)).astype(w.dtype)).astype(dt, copy=False)
    species = rng.integers(0, wl.num_elements, size=n).astype(np.int32)
    return dict(x=x, species=species, w=w)


def integer_tp_inputs(n_src, n_edges, dim1, dim2, numel, n_nodes, seed, max_degree=None):
    """Small-integer inputs for bit-exact plumbing checks: x in [-8, 8],
    harmonics and weights in [-4, 4]; with sums of at most a few dozen edges
    every partial sum is an integer far below 2**24, so float32 arithmetic is
    exact whatever the order.  Returns dict like :func:`tp_inputs` (float32,
    int32 indices, dst sorted)."""
    rng = np.random.default_rng(seed)
    dst = np.sort(rng.integers(0, n_nodes, size=n_edges))
    src = rng.integers(0, n_src, size=n_edges)
    sh = rng.integers(-4, 5, size=(n_edges, dim2)).astype(np.float32)
    x = rng.integers(-8, 9, size=(n_src, dim1)).astype(np.float32)
    w = rng.integers(-4, 5, size=(n_edges, numel)).astype(np.float32)
    return dict(x=x, sh=sh, w=w, src=src.astype(np.int32), dst=dst.astype(np.int32),
                n_nodes=n_nodes, n_src=n_src)


def output_gradient(n_nodes, dim_out, dtype, seed):
    """A seeded standard-normal gradient of the convolution's output
    [n_nodes, dim_out] (the input of the backward pass)."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (n_nodes, dim_out), dtype).astype(_np_dtype(dtype), copy=False)


def src_permutation(src):
    """Edge ids ordered by source, ties in edge order (a stable argsort):
    graph structure the backward pass takes with the sorted destinations."""
    return np.argsort(np.asarray(src), kind="stable").astype(np.asarray(src).dtype)


def species_permutation(species):
    """Atom ids ordered by element, ties in atom order (a stable argsort):
    what the symmetric contraction's backward takes with the species."""
    return np.argsort(np.asarray(species), kind="stable").astype(np.asarray(species).dtype)


def linear_inputs(wl, weight_numel, n=None, seed=None):
    """Inputs of a linear-layer workload: x [n, dim_in] N(0,1), weights
    N(0,1) ([1, numel] shared or [num_classes, numel]; the layer's own
    1/sqrt(fan-in) keeps outputs at unit scale), and for class-indexed
    weights the classes: uniform over num_classes, sorted ascending (the
    pages' indexed linear takes sorted indices), int32."""
    rng = np.random.default_rng(1000 + wl.number if seed is None else seed)
    dt = _np_dtype(wl.dtype)
    n = wl.n if n is None else n
    x = _normal(rng, (n, _irreps_dim(wl.irreps_in)), wl.dtype).astype(dt, copy=False)
    rows = wl.num_classes if wl.num_classes else 1
    w = _normal(rng, (rows, weight_numel), wl.dtype).astype(dt, copy=False)
    classes = None
    if wl.num_classes:
        classes = np.sort(rng.integers(0, wl.num_classes, size=n)).astype(np.int32)
    return dict(x=x, w=w, classes=classes)


def fc_inputs(wl, weight_numel, n=None, seed=None):
    """Inputs of a fully connected product workload: x1 [n, dim_in1] and
    x2 [n, dim_in2] N(0,1), weights N(0,1), one shared row [1, weight_numel]
    or, for a per-sample workload, one row per sample [n, weight_numel] (the
    product's own 1/sqrt(fan-in) keeps outputs at unit scale)."""
    rng = np.random.default_rng(1000 + wl.number if seed is None else seed)
    dt = _np_dtype(wl.dtype)
    n = wl.n if n is None else n
    x1 = _normal(rng, (n, _irreps_dim(wl.irreps_in1)), wl.dtype).astype(dt, copy=False)
    x2 = _normal(rng, (n, _irreps_dim(wl.irreps_in2)), wl.dtype).astype(dt, copy=False)
    w = _normal(rng, (n if wl.per_sample else 1, weight_numel), wl.dtype).astype(dt, copy=False)
    return dict(x1=x1, x2=x2, w=w)


def fcconv_inputs(wl, weight_numel, n_nodes=None, degree=None, graph=None, seed=None):
    """Inputs of the fully connected convolution workload: the regular graph
    (or the ragged one), harmonics of the edge vectors, x N(0,1), one weight
    row per edge N(0,1) (the product's 1/sqrt(fan-in) keeps outputs at unit
    scale).  Returns dict(x, sh, w, src, dst (int32), n_nodes)."""
    rng = np.random.default_rng(1000 + wl.number if seed is None else seed)
    dt = _np_dtype(wl.dtype)
    nn = wl.n_nodes if n_nodes is None else n_nodes
    dg = wl.degree if degree is None else degree
    if graph == "ragged":
        src, dst, vec = ragged_graph(rng, nn, dg)
    else:
        src, dst, vec = regular_graph(rng, nn, dg)
    sh = edge_harmonics(vec, wl.sh_ls).astype(dt)
    x = _normal(rng, (nn, _irreps_dim(wl.irreps_in1)), wl.dtype).astype(dt, copy=False)
    w = _normal(rng, (sh.shape[0], weight_numel), wl.dtype).astype(dt, copy=False)
    return dict(x=x, sh=sh, w=w, src=src.astype(np.int32), dst=dst.astype(np.int32), n_nodes=nn)
