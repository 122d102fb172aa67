"""Float64 NumPy oracle of the offline item-vector export.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Citation keys (page title, then the section):
  [digest]  "DuoLM: Fast and Effective Personalized Recommendation with
            Language Models" (paper.rainbus.top structured digest)
  [onedev]  "DuoLM은 아이템 벡터 재사용과 공유 프리픽스로 LLM 추천 서빙을
            가속한다" (onedev.kr digest)

What is computed.  The encoder's representation a_i of an item is turned into
the ranker input vector z_i by the continuous-input interface: RMS
normalisation of a_i, calibration by a reference scale rho estimated from the
ranker's native word embeddings, and a learnable gain e^gamma ([digest] 一句话
总结 and 核心方法; [onedev] 어떻게 동작하나).  After training, every z_i is
written once, as FP16, into the GPU-resident table D whose row iota(i) answers
the virtual id V + iota(i) ([digest] 方法步骤详情 step 3).

Readings where the pages leave a step open:
  - RMS(a) = sqrt(mean_k a_k^2 + eps) with the caller's eps >= 0 (the pages
    name only "RMS normalisation"; eps = 0 is the bare definition).  A row
    whose mean square plus eps is zero is exported as zeros.
  - rho is the root mean square over every entry of the ranker's native
    embedding matrix E ([digest] 复现评估 quotes rho = 0.0280669 for the real
    model; that number is not used here).
  - FP16 is IEEE binary16 with round-half-to-even; a magnitude that rounds
    past the largest finite value becomes +-inf, tiny values become
    subnormals or zero, as IEEE rounding defines.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def rms(a: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """Per-row root mean square sqrt(mean_k a_k^2 + eps), float64, shape [n]."""
    a = np.asarray(a, dtype=F64)
    return np.sqrt(np.mean(a * a, axis=-1) + F64(eps))


def interface_vectors(a: np.ndarray, rho: float, gamma: float, eps: float = 0.0) -> np.ndarray:
    """z = e^gamma * rho * a / RMS(a), row by row, in float64 ([digest] 核心方法).

    a: [n, d] encoder outputs (any float dtype; widened exactly to float64).
    Rows with RMS(a) = 0 give zeros (reading above).
    """
    a = np.asarray(a, dtype=F64)
    r = rms(a, eps)[:, None]
    safe = np.where(r > 0, r, F64(1.0))
    normalised = np.where(r > 0, a / safe, F64(0.0))  # RMS normalisation
    calibrated = F64(rho) * normalised  # reference scale of the native embeddings
    return np.exp(F64(gamma)) * calibrated  # learnable gain e^gamma


def to_fp16_bits(z: np.ndarray) -> np.ndarray:
    """IEEE binary16 round-half-to-even of float64 values, as uint16 bit patterns."""
    with np.errstate(over="ignore"):  # overflow to +-inf is the defined result
        return np.asarray(z, dtype=F64).astype(np.float16).view(np.uint16)


def export_table(a: np.ndarray, rho: float, gamma: float, eps: float = 0.0) -> np.ndarray:
    """The FP16 table rows written for encoder outputs a ([digest] 方法步骤详情 step 3)."""
    return to_fp16_bits(interface_vectors(a, rho, gamma, eps))


def reference_scale(E: np.ndarray) -> float:
    """rho: root mean square over all entries of the native embedding matrix E."""
    e = np.asarray(E, dtype=F64)
    return float(np.sqrt(np.mean(e * e)))


def midpoint_distance(z: np.ndarray) -> np.ndarray:
    """Relative distance of each float64 value to the midpoint of the binary16
    cell holding it (the point where round-to-nearest changes its answer; for
    the top cell [65504, 65536) that is the overflow threshold 65520).  A value
    far from it has one FP16 code under any accurate evaluation; one within a
    few float64 ulps of it sits on a knife edge.  Other midpoints are at least a
    quarter cell away, so this is the nearest one whenever it matters."""
    z = np.abs(np.asarray(z, dtype=F64))
    e = np.floor(np.log2(np.maximum(z, 2.0 ** -14)))  # subnormals share 2^-14's spacing
    ulp = 2.0 ** (e - 10)
    mid = np.floor(z / ulp) * ulp + ulp / 2
    return np.abs(z - mid) / np.maximum(z, 2.0 ** -24)
