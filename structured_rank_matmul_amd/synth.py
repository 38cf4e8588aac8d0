"""Seeded synthetic layer workloads (weights W and activations X).

This module only draws inputs.  It holds none of the DyRA arithmetic (no SVD,
no residual, no least squares): the CPU oracle side and the HIP side both take
their inputs from here and from nowhere else, so the two never share code that
computes a result.

Every draw is reproducible from ``(seed, config id, layer id, role)`` through
numpy's PCG64 seeded by a ``SeedSequence`` of those four integers.

Weights are ``W = Q1[:, :m] diag(s) Q2[:, :m]^T`` with Haar-distributed
orthogonal ``Q1``, ``Q2`` (QR of a Gaussian matrix, signs fixed by the diagonal
of R), ``m = min(c1, c2)`` and a power-law spectrum ``s_i = i^-p``.  They are
drawn in float64 and handed to the library as float32; the float32 array is
the weight (the oracle upcasts exactly that array).

BLAST-structured weights (the second static family the paper pairs with
DyRA) are drawn from factors: block (i, j) of an nb x nb grid is
``U_i diag(s_ij) V_j^T`` with Gaussian ``U_i``, ``V_j`` and couplings
``s_ij`` on a power-law decay, plus a power-law residual of a set relative
size.  The drawn factors are then known inputs for the static part; no fit
is made here.

Activations are drawn in float64 and rounded once to the compute dtype
(float32 round-to-nearest-even, then bfloat16 round-to-nearest-even for bf16
configs).  The rounded values are the input; ``exact`` returns them upcast to
float64 without further rounding.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

ROLE_W = 0
ROLE_X = 1
ROLE_CHANNELS = 2
ROLE_SCALES = 3

DTYPES = ("f32", "bf16")


def rng_for(seed: int, cfg_id: int, layer_id: int, role: int) -> np.random.Generator:
    """A PCG64 stream keyed by (seed, config, layer, role)."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(seed), int(cfg_id), int(layer_id), int(role)])))


# ---------------------------------------------------------------- rounding

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 (RNE) -> bfloat16 (RNE); return the uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Activations:
    """An activation matrix in its compute dtype.

    ``data`` is float32 (dtype "f32") or uint16 bfloat16 bit patterns ("bf16"),
    row-major [rows, cols].
    """
    data: np.ndarray
    dtype: str

    @property
    def exact(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.data.astype(np.float64)
        return bf16_bits_to_f64(self.data)

    @property
    def shape(self) -> Tuple[int, int]:
        return self.data.shape


def round_activations(x64: np.ndarray, dtype: str) -> Activations:
    if dtype == "f32":
        return Activations(np.ascontiguousarray(x64.astype(np.float32)), dtype)
    if dtype == "bf16":
        return Activations(f64_to_bf16_bits(x64), dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- weights

def haar_orthogonal(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """First `cols` columns of a Haar-distributed rows x rows orthogonal matrix."""
    g = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(g)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d


def power_spectrum(m: int, p: float) -> np.ndarray:
    return np.arange(1, m + 1, dtype=np.float64) ** (-float(p))


def draw_weight(c1: int, c2: int, p: float, kaiming: bool, rng: np.random.Generator
                ) -> Tuple[np.ndarray, np.ndarray]:
    """W (float32, [c1, c2], the X @ W orientation) and its float64 spectrum.

    With ``kaiming`` the spectrum is scaled so that ||W||_F^2 = 2*c2, the
    expected squared norm of a He-normal matrix with std sqrt(2/c1).
    """
    m = min(c1, c2)
    s = power_spectrum(m, p)
    if kaiming:
        s = s * np.sqrt(2.0 * c2 / np.sum(s * s))
    q1 = haar_orthogonal(rng, c1, m)
    q2 = haar_orthogonal(rng, c2, m)
    w = (q1 * s) @ q2.T
    return np.ascontiguousarray(w.astype(np.float32)), s


ROLE_BLAST = 4


@dataclasses.dataclass
class BlastWeight:
    """A BLAST-structured weight and its factors (all as handed to the library)."""
    W: np.ndarray    # float32 [c1, c2]
    U: np.ndarray    # float32 [c1, r]   block row i = rows i*c1/nb ..
    S: np.ndarray    # float32 [nb, nb, r] diagonal couplings s_ij
    V: np.ndarray    # float32 [c2, r]   block column j = rows j*c2/nb ..
    nb: int


def draw_blast_weight(c1: int, c2: int, nb: int, r: int, rng: np.random.Generator, p: float = 0.7,
                      residual: float = 0.35) -> BlastWeight:
    """W = [U_i diag(s_ij) V_j^T]_ij + E with ||E||_F = residual * ||structured part||_F.

    U_i [c1/nb, r] and V_j [c2/nb, r] are Gaussian with unit-norm expected
    columns; s_ij[c] = (c + 1)^-p (1 + 0.5 g), g standard normal per block and
    rank index; E has Haar singular vectors and the spectrum i^-p.  The
    factors are rounded to float32 first and the structured part is formed
    from the rounded values, so they describe the float32 W's structure up to
    W's own rounding.
    """
    if nb < 1 or c1 % nb or c2 % nb:
        raise ValueError("block count must divide both dimensions")
    pr, qr = c1 // nb, c2 // nb
    U = (rng.standard_normal((c1, r)) / np.sqrt(pr)).astype(np.float32)
    V = (rng.standard_normal((c2, r)) / np.sqrt(qr)).astype(np.float32)
    decay = power_spectrum(r, p)
    S = (decay[None, None, :] * (1.0 + 0.5 * rng.standard_normal((nb, nb, r)))).astype(np.float32)
    # block column j of the structured part: [U_1 diag(s_1j); ...; U_nb diag(s_nbj)] V_j^T
    U64, S64 = U.astype(np.float64), S.astype(np.float64)
    structured = np.empty((c1, c2))
    for j in range(nb):
        scaled = (U64.reshape(nb, pr, r) * S64[:, j, None, :]).reshape(c1, r)
        structured[:, j * qr:(j + 1) * qr] = scaled @ V[j * qr:(j + 1) * qr].astype(np.float64).T
    m = min(c1, c2)
    E = (haar_orthogonal(rng, c1, m) * power_spectrum(m, p)) @ haar_orthogonal(rng, c2, m).T
    E *= residual * np.linalg.norm(structured) / np.linalg.norm(E)
    W = np.ascontiguousarray((structured + E).astype(np.float32))
    return BlastWeight(W=W, U=U, S=S, V=V, nb=nb)


def make_blast_weight(w: "Workload", spec: "LayerSpec", nb: int, r: int, seed: int = 0) -> BlastWeight:
    """A BLAST-structured stand-in for one layer's weight (rank r, nb x nb blocks)."""
    rng = rng_for(seed, w.cfg_id, layer_index(w, spec), ROLE_BLAST + 10 * nb)
    return draw_blast_weight(spec.c1, spec.c2, nb, r, rng, p=spec.p)


def random_blast_weight(c1: int, c2: int, nb: int, r: int, seed: int, residual: float = 0.35) -> BlastWeight:
    """A small BLAST-structured weight for tests."""
    rng = rng_for(seed, 97, c1 * 100003 + c2, ROLE_BLAST + 10 * nb)
    return draw_blast_weight(c1, c2, nb, r, rng, residual=residual)


# ---------------------------------------------------------------- activations

def x_logcols(rng: np.random.Generator, rows: int, c1: int) -> np.ndarray:
    """Gaussian entries with per-column scales log-uniform in [0.1, 10]."""
    z = rng.standard_normal((rows, c1))
    d = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=c1))
    return z * d


def gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def x_layernorm_outliers(rng: np.random.Generator, rows: int, c1: int, n_out: int, factor: float,
                         ch_rng: np.random.Generator) -> np.ndarray:
    """Rows standardised to zero mean / unit variance, then `n_out` fixed channels scaled."""
    z = rng.standard_normal((rows, c1))
    z = (z - z.mean(axis=1, keepdims=True)) / z.std(axis=1, keepdims=True)
    ch = ch_rng.choice(c1, size=n_out, replace=False)
    z[:, ch] *= factor
    return z


def x_rmsnorm_massive(rng: np.random.Generator, rows: int, c1: int, n_out: int, factor: float,
                      ch_rng: np.random.Generator) -> np.ndarray:
    """Rows scaled to unit RMS, then `n_out` fixed channels scaled ("massive activations")."""
    z = rng.standard_normal((rows, c1))
    z = z / np.sqrt(np.mean(z * z, axis=1, keepdims=True))
    ch = ch_rng.choice(c1, size=n_out, replace=False)
    z[:, ch] *= factor
    return z


def x_speech_energy(rng: np.random.Generator, B: int, n: int, c1: int, rho: float = 0.99,
                    sigma: float = 0.5) -> np.ndarray:
    """Gaussian frames times a slowly varying log-normal energy exp(sigma * g_t).

    g is a unit-variance AR(1) along the frames of each clip (restarted per clip).
    """
    z = rng.standard_normal((B * n, c1))
    eps = rng.standard_normal((B, n))
    g = np.empty((B, n))
    g[:, 0] = eps[:, 0]
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, n):
        g[:, t] = rho * g[:, t - 1] + c * eps[:, t]
    e = np.exp(sigma * g).reshape(B * n, 1)
    return z * e


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    c1: int          # input features
    c2: int          # output features
    r: int           # static (weight) rank
    k: int           # correction rank
    p: float         # spectrum exponent of W
    kaiming: bool    # scale W to He-normal Frobenius norm
    x_kind: str      # activation generator


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    dtype: str
    B: int           # instances per call
    n: int           # tokens per instance
    layers: Tuple[LayerSpec, ...]
    description: str

    @property
    def tokens(self) -> int:
        return self.B * self.n

    def layer(self, name: str) -> LayerSpec:
        for s in self.layers:
            if s.name == name:
                return s
        raise KeyError(name)


def _vitl(name: str, c1: int, c2: int, x_kind: str) -> LayerSpec:
    return LayerSpec(name, c1, c2, r=min(c1, c2) // 4, k=64, p=0.7, kaiming=False, x_kind=x_kind)


WORKLOADS: Dict[str, Workload] = {
    "linear384_fp32": Workload(
        "linear384_fp32", 1, "f32", B=1, n=256,
        layers=(LayerSpec("linear", 384, 384, r=96, k=16, p=0.7, kaiming=False, x_kind="logcols"),),
        description="single fp32 linear layer, 256 tokens, 384->384, r=96, k=16"),
    "vitb_fc1": Workload(
        "vitb_fc1", 2, "bf16", B=64, n=201,
        layers=(LayerSpec("fc1", 768, 3072, r=256, k=32, p=0.5, kaiming=True, x_kind="layernorm6x20"),),
        description="ViT-B-like MLP fc1, 64 images x 201 tokens, 768->3072, r=256, k=32"),
    "vitl_block": Workload(
        "vitl_block", 3, "bf16", B=128, n=201,
        layers=(_vitl("qkv", 1024, 3072, "logcols"),
                _vitl("fc1", 1024, 4096, "logcols"),
                _vitl("fc2", 4096, 1024, "gelu_logcols")),
        description="DINOv3-ViT-L-like block, 128 images x 201 tokens, qkv/fc1/fc2, r=min/4, k=64"),
    "whisper_mlp": Workload(
        "whisper_mlp", 4, "bf16", B=16, n=1500,
        layers=(LayerSpec("fc1", 1280, 5120, r=320, k=48, p=0.6, kaiming=True, x_kind="speech"),
                LayerSpec("fc2", 5120, 1280, r=320, k=48, p=0.6, kaiming=True, x_kind="speech")),
        description="Whisper-large-shaped encoder MLP, 16 clips x 1500 frames, r=320, k=48"),
    "llama_prefill": Workload(
        "llama_prefill", 5, "bf16", B=8, n=2048,
        layers=(LayerSpec("gate", 4096, 14336, r=1024, k=64, p=0.4, kaiming=True, x_kind="rms8x50"),
                LayerSpec("up", 4096, 14336, r=1024, k=64, p=0.4, kaiming=True, x_kind="rms8x50"),
                LayerSpec("down", 14336, 4096, r=1024, k=64, p=0.4, kaiming=True, x_kind="rms8x50")),
        description="Llama-style 8B MLP prefill, 8 x 2048 tokens, r=1024, k=64"),
}

DECODE_TOKENS = (1, 16, 64)


def llama_decode(m: int) -> Workload:
    """Llama-style MLP at decode: m sequences of one token each (instances of n = 1)."""
    base = WORKLOADS["llama_prefill"]
    return Workload(f"llama_decode_m{m}", 5, "bf16", B=m, n=1, layers=base.layers,
                    description=f"Llama-style 8B MLP decode, {m} x 1 token, r=1024, k=64")


def workload(name: str) -> Workload:
    """A workload by name: one of WORKLOADS or llama_decode_m<m>."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    prefix = "llama_decode_m"
    if name.startswith(prefix) and name[len(prefix):].isdigit() and int(name[len(prefix):]) > 0:
        return llama_decode(int(name[len(prefix):]))
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)} and llama_decode_m<m>")


def layer_index(w: Workload, spec: LayerSpec) -> int:
    return w.layers.index(spec)


def make_weight(w: Workload, spec: LayerSpec, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(W float32 [c1, c2], spectrum float64) of one layer of a workload."""
    rng = rng_for(seed, w.cfg_id, layer_index(w, spec), ROLE_W)
    return draw_weight(spec.c1, spec.c2, spec.p, spec.kaiming, rng)


def make_activations(w: Workload, spec: LayerSpec, seed: int = 0, B: Optional[int] = None,
                     n: Optional[int] = None) -> Activations:
    """Activations [B*n, c1] of one layer of a workload, rounded to its dtype.

    ``B`` and ``n`` default to the workload's; smaller values give a prefix-free
    draw of the same distribution (used for bounded CPU samples).
    """
    B = w.B if B is None else int(B)
    n = w.n if n is None else int(n)
    rows = B * n
    li = layer_index(w, spec)
    # decode draws get their own stream so they never alias a prefill draw
    role_x = ROLE_X + (100 * n if n != w.n or B != w.B else 0)
    rng = rng_for(seed, w.cfg_id, li, role_x)
    ch_rng = rng_for(seed, w.cfg_id, li, ROLE_CHANNELS)
    kind = spec.x_kind
    if kind == "logcols":
        x = x_logcols(rng, rows, spec.c1)
    elif kind == "gelu_logcols":
        x = gelu_erf(x_logcols(rng, rows, spec.c1))
    elif kind == "layernorm6x20":
        x = x_layernorm_outliers(rng, rows, spec.c1, 6, 20.0, ch_rng)
    elif kind == "rms8x50":
        x = x_rmsnorm_massive(rng, rows, spec.c1, 8, 50.0, ch_rng)
    elif kind == "speech":
        x = x_speech_energy(rng, B, n, spec.c1)
    elif kind == "gaussian":
        x = rng.standard_normal((rows, spec.c1))
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    return round_activations(x, w.dtype)


def random_matrix(rows: int, cols: int, seed: int, dtype: str = "f32", scale: float = 1.0) -> Activations:
    """A plain Gaussian matrix for small tests, rounded to `dtype`."""
    rng = rng_for(seed, 99, rows * 100003 + cols, ROLE_X)
    return round_activations(scale * rng.standard_normal((rows, cols)), dtype)


def random_weight(c1: int, c2: int, seed: int, p: float = 0.7) -> np.ndarray:
    """A float32 power-law-spectrum weight for small tests."""
    rng = rng_for(seed, 98, c1 * 100003 + c2, ROLE_W)
    return draw_weight(c1, c2, p, False, rng)[0]


def all_layers() -> List[Tuple[Workload, LayerSpec]]:
    return [(w, s) for w in WORKLOADS.values() for s in w.layers]
