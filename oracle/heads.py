"""q/k preprocessing options of the KDA forward, fp64 -- TEST INFRASTRUCTURE
ONLY (see the package docstring).

L2 normalisation.  The method runs on unit-norm queries and keys: a key of
norm 1 keeps the delta-rule write (I - beta k k^T) a contraction for beta in
(0, 1].  The pages do not spell the normalisation out; the plain reading
used here divides each (token, head) row of q and of k by its Euclidean norm
with a small eps under the root: x / sqrt(sum x^2 + eps), eps = 1e-6.

Grouped key heads.  The pages' state kernel takes the number of key heads Hg
as a parameter separately from the number of heads H (page "spike(kimi-linear):
chunk_kda prefill AOT port", commit message: the chunk_delta_h pin with
Hg = 32), which reads as Hg key/query heads shared by groups of value heads;
the only value pinned there is Hg = H = 32.  Reading used here: value head h
uses key head h // (H // Hg), i.e. each key head serves H // Hg consecutive
value heads.
"""
import numpy as np

L2NORM_EPS = 1e-6


def l2norm(x, eps: float = L2NORM_EPS) -> np.ndarray:
    """Each row (last axis) divided by sqrt(sum of squares + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def expand_key_heads(x, H: int) -> np.ndarray:
    """[T, Hg, d] key/query rows -> [T, H, d]: value head h gets key head
    h // (H // Hg)."""
    x = np.asarray(x, dtype=np.float64)
    Hg = x.shape[1]
    if H % Hg:
        raise ValueError(f"Hg = {Hg} does not divide H = {H}")
    return np.repeat(x, H // Hg, axis=1)
