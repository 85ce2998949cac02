"""Helpers of the GPU parity tests: device buffers, metrics, the teacher-forcing rule."""
from __future__ import annotations

import sys

import numpy as np
import torch

import kv_cached_gqa_decoder_amd as vla
from oracle import decoder as D

# tolerances of the workloads: bf16 configs and the fp32 config
TOL = {"bf16": dict(cos=0.9995, rel=2e-2), "f32": dict(cos=0.9995, rel=1e-4)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_from_storage(arr: np.ndarray, storage: str) -> torch.Tensor:
    """Device tensor holding a synth storage array (uint16 bf16 bits or float32)."""
    if storage == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def logits_of(model: vla.Model) -> np.ndarray:
    out = np.zeros(model.cfg.vocab, dtype=np.float32)
    model.logits_out(out)
    return out.astype(np.float64)


def metrics(a: np.ndarray, b: np.ndarray):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel = float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
    return cos, rel


WORST = {}


def check_logits(gpu, ref, kind: str, what: str = ""):
    cos, rel = metrics(gpu, ref)
    t = TOL[kind]
    w = WORST.setdefault(kind, [1.0, 0.0])
    w[0], w[1] = min(w[0], cos), max(w[1], rel)
    if rel > 0.5 * t["rel"] or cos < 1 - 0.5 * (1 - t["cos"]):
        log(f"  {what}: cos {cos:.6f} rel {rel:.3e} (within half the tolerance: no)")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite logits"
    assert cos >= t["cos"] and rel <= t["rel"], f"{what}: cos {cos:.6f} rel {rel:.3e}"
    return cos, rel


def check_argmax(gpu_tok: int, ref_logits: np.ndarray, kind: str, what: str = ""):
    """Greedy token parity: equal to the oracle's argmax unless the oracle's top-2 gap is
    below twice the tolerance band, in which case any token within that band is correct."""
    ref = np.asarray(ref_logits, dtype=np.float64)
    top = int(np.argmax(ref))
    if gpu_tok == top:
        return
    band = 2 * TOL[kind]["rel"] * np.max(np.abs(ref))
    srt = np.sort(ref)
    assert srt[-1] - srt[-2] < band and ref[gpu_tok] >= srt[-1] - band, \
        f"{what}: gpu token {gpu_tok} vs oracle {top} (gap {srt[-1] - srt[-2]:.3e})"


def oracle_config(preset: dict, name="custom", init_std=0.02) -> D.Config:
    wd = {vla.VLA_F32: "f32", vla.VLA_BF16: "bf16", vla.VLA_INT4_G128: "int4"}[preset["wdtype"]]
    act = "bf16" if wd == "int4" else wd
    return D.Config(name, preset["n_layers"], preset["hidden"], preset["n_heads"],
                    preset["n_kv_heads"], preset["head_dim"], preset["ffn"], preset["vocab"],
                    rms_eps=preset.get("rms_eps", 1e-6), rope_theta=preset["rope_theta"],
                    wdtype=wd, act=act, num_blocks=preset["num_blocks"],
                    max_frames=preset["max_frames"], seed=preset["seed"], init_std=init_std)


def eviction_margin(vectors: np.ndarray):
    """The oracle's redundancy scoring of mean-key rows [F, D]: (winner index, the gap
    between the winner's score and the best score of any frame outside the winning
    pair, the pair matrix).

    The winning pair is the winner and its most similar partner; both carry the
    same score, so only frames outside the pair can compete with it.
    """
    from oracle.scoring import pair_matrix
    s = pair_matrix(np.asarray(vectors, dtype=np.float64))
    m = s.max(axis=1)
    win = int(np.argmax(m))
    partner = int(np.argmax(s[win]))
    rest = [m[i] for i in range(len(m)) if i not in (win, partner)]
    gap = float(m[win] - max(rest)) if rest else float("inf")
    return win, gap, s


# Eviction decisions that depend on keys the model computed (bf16-rounded on the
# device, fp64 in the oracle) are only compared when the oracle's margin is outside
# this band of cosine similarity.
KEY_BAND = 1e-2
