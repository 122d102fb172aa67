"""Plain-Python oracle of the ranker input assembly (the host packer).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Citation keys (page title, then the section):
  [onedev]  "DuoLM은 아이템 벡터 재사용과 공유 프리픽스로 LLM 추천 서빙을
            가속한다" (onedev.kr digest)
  [digest]  "DuoLM: Fast and Effective Personalized Recommendation with
            Language Models" (paper.rainbus.top structured digest)

What is assembled.  The ranker reads, in order, the instruction, then for
every history item a marker embedding, the item's vector and its feedback
text, then the candidate header, then the candidate item vectors ([onedev]
어떻게 동작하나).  A request carries only item ids and feedback; the runtime
assembles the shared prefix from them ([digest] 方法步骤详情 step 4) and packs
the candidates after it ([onedev] 어떻게 쓰나).  An item spread over m vectors
contributes m consecutive VIDs where a single-vector item contributes one
([digest] 实验结果, FIR m = 8).

Reading: the instruction, the marker id and the candidate header are shared
by every request of a call (one template); feedback text arrives already as
token ids (no tokenizer is involved).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def assemble_prefix(instruction: Sequence[int], marker: int, items: Sequence[Sequence[int]],
                    feedbacks: Sequence[Sequence[int]], cand_header: Sequence[int] = ()) -> np.ndarray:
    """instruction, then (marker, item VIDs, feedback ids) per history item, then the header."""
    assert len(items) == len(feedbacks)
    out = list(instruction)
    for vids, fb in zip(items, feedbacks):
        out.append(marker)
        out.extend(vids)
        out.extend(fb)
    out.extend(cand_header)
    return np.array(out, dtype=np.int32)


def pack_batch(requests: Sequence[Tuple[np.ndarray, np.ndarray, int]]):
    """Concatenate (prefix, candidate ids, m) requests as [prefix_0, cands_0,
    prefix_1, cands_1, ...] with per-request prefix length, candidate count and
    ids per candidate: the layout the device entry point reads."""
    ids, L, K, M = [], [], [], []
    for prefix, cands, m in requests:
        m = max(int(m), 1)
        assert len(cands) % m == 0
        ids.append(np.asarray(prefix, dtype=np.int32))
        ids.append(np.asarray(cands, dtype=np.int32))
        L.append(len(prefix))
        K.append(len(cands) // m)
        M.append(m)
    return (np.concatenate(ids) if ids else np.zeros(0, np.int32), np.array(L, np.int32),
            np.array(K, np.int32), np.array(M, np.int32))
