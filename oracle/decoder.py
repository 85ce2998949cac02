"""The oracle's KV-cached pre-norm GQA decoder (fp64, numpy).

What is computed, step by step, per layer l for a chunk of n tokens at
absolute positions P .. P+n-1 (the plain definition; no blocking or fusion):

  1. u = RMSNorm(x)                         x * (mean(x^2) + eps)^(-1/2) * g
  2. q = u Wq^T, k = u Wk^T, v = u Wv^T     ("CSR ...", §III-A: q, k, v are
                                              linear maps of the hidden state)
  3. q, k rotated by RoPE at the absolute positions ("Rebuilding Kshipra
     Around Memory", §4: a chunk after P cached tokens starts at P)
  4. k, v appended to layer l's cache (paged, see kvpool)
  5. o_h = softmax(q_h K^T / sqrt(d)) V over every visible key: all resident
     cached tokens plus the chunk's own tokens up to and including itself
     ("CSR ...", §III-A scaled softmax; "Rebuilding Kshipra ...", §4 causal
     mask covers the chunk); q head h reads KV head floor(h / g), g = Hq/Hkv
  6. x += concat_h(o_h) Wo^T
  7. x += Wdown^T-map of silu(u2 Wgate^T) * (u2 Wup^T) with u2 = RMSNorm(x)
     (SwiGLU, named by "Can an LLM Forget the Right Things?", §6; the gated
     pair is fused on the GPU as in "Running VLAs at Real-time Speed", §4.2)

Final: logits = W_Y RMSNorm(x_last) ("CSR ...", §III-A output head W_Y; the
final norm is the pre-norm reading), greedy next token = argmax, ties to the
lowest id.

Variants used by the pi0-style prefix model ("Running VLAs at Real-time
Speed", §2 and §4.1-4.2): GeGLU instead of SwiGLU (exact-erf GELU on the gate
branch); the last layer reduced to its input norm and K/V projection (its K/V
are all the action expert reads); no vocabulary (vocab 0: caller embeddings
only, no output head).

Readings where the pages are silent (each listed in the design notes): pre-norm
RMSNorm with weight 1 and eps 1e-6; HF-style rotate-half RoPE pairing
(j, j + d/2) with inv_freq_j = theta^(-2j/d), angles in fp64; scale 1/sqrt(d);
consecutive GQA grouping; no biases; untied W_Y; logits for the last row of a
prefill chunk; the cache stores post-RoPE keys and a frame's keys keep their
rotation after other frames are evicted.

The oracle keeps every activation in fp64; it does not mimic the GPU's bf16
rounding of activations (the tolerance absorbs it).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

from . import rng
from .kvpool import BlockPool, NoBlocks, NothingToEvict, Segment


# ----------------------------------------------------------------------------
# configuration
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e4
    wdtype: str = "bf16"        # storage of the projection weights: f32 | bf16 | int4
    act: str = "bf16"           # activation / KV storage on the GPU: f32 | bf16
    block_tokens: int = 16
    num_blocks: int = 64
    max_frames: int = 64
    seed: int = 1234
    init_std: float = 0.02
    ffn_kind: str = "swiglu"    # swiglu | geglu
    kv_only_last: bool = False  # last layer: input norm + K/V only
    stream_base: int = 0        # added to the per-layer weight streams

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def embed_storage(self) -> str:
        return "f32" if self.act == "f32" else "bf16"

    @property
    def weight_storage(self) -> str:
        # INT4 master weights are drawn fp64 -> rounded to fp32 -> quantised
        return {"f32": "f32", "bf16": "bf16", "int4": "f32"}[self.wdtype]

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The workloads' model shapes (batch 1 everywhere).
C1 = Config("c1_tiny_f32", 2, 256, 4, 2, 64, 688, 1024, rope_theta=1e4, wdtype="f32",
            act="f32", num_blocks=8, max_frames=8, seed=1235)
C2 = Config("c2_qwen1p5b_bf16", 28, 1536, 12, 2, 128, 8960, 151936, rope_theta=1e6,
            wdtype="bf16", act="bf16", num_blocks=96, max_frames=16, seed=1236)
C3 = C2.with_(name="c3_semantic_eviction", num_blocks=512, max_frames=128, seed=1237)
C5 = Config("c5_llama3_8b_int4", 32, 4096, 32, 8, 128, 14336, 128256, rope_theta=5e5,
            wdtype="int4", act="bf16", num_blocks=7534, max_frames=256, seed=1239)
CONFIGS = {c.name: c for c in (C1, C2, C3, C5)}


def kv_bytes_per_token(cfg: Config, bytes_per_elem: int) -> int:
    """KV bytes per token = 2 x layers x KV heads x head dim x bytes per element.

    "Rebuilding Kshipra Around Memory", §1 (GQA-aware sizing).
    """
    return 2 * cfg.n_layers * cfg.n_kv_heads * cfg.head_dim * bytes_per_elem


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
class Weights:
    """Seeded random-init weights, logical (out, in) row-major, regenerated from the seed.

    Values are rounded into the configuration's storage type and held as fp32
    (exact for fp32 and bf16 values, and for INT4 q*s products); fp64 copies
    are made on first use and cached (``f64``).
    """

    def __init__(self, cfg: Config, cache_f64: bool = True, layers=None):
        self.cfg = cfg
        self.cache_f64 = cache_f64
        self._f32 = {}
        self._f64 = {}
        self.layers = range(cfg.n_layers) if layers is None else layers

    # shapes of the logical tensors
    def shape(self, name: str):
        c = self.cfg
        qd, kd = c.n_heads * c.head_dim, c.n_kv_heads * c.head_dim
        return {"q": (qd, c.hidden), "k": (kd, c.hidden), "v": (kd, c.hidden),
                "o": (c.hidden, qd), "gate": (c.ffn, c.hidden), "up": (c.ffn, c.hidden),
                "down": (c.hidden, c.ffn), "embed": (c.vocab, c.hidden),
                "head": (c.vocab, c.hidden)}[name]

    _KIND = {"q": rng.KIND_Q, "k": rng.KIND_K, "v": rng.KIND_V, "o": rng.KIND_O,
             "gate": rng.KIND_GATE, "up": rng.KIND_UP, "down": rng.KIND_DOWN}

    def stream(self, name: str, layer: int = -1) -> int:
        if name == "embed":
            return rng.STREAM_EMBED
        if name == "head":
            return rng.STREAM_HEAD
        return self.cfg.stream_base + rng.layer_stream(layer, self._KIND[name])

    def _make(self, name: str, layer: int) -> np.ndarray:
        c = self.cfg
        if name == "embed":
            return rng.tensor(c.seed, self.stream(name), self.shape(name), c.init_std,
                              c.embed_storage, out_f32=True)
        w = rng.tensor(c.seed, self.stream(name, layer), self.shape(name), c.init_std,
                       c.weight_storage, out_f32=True)
        if c.wdtype == "int4":
            from .int4 import quantize_g128
            w = quantize_g128(w)[2]
        return w

    def f32(self, name: str, layer: int = -1) -> np.ndarray:
        key = (name, layer)
        if key not in self._f32:
            self._f32[key] = self._make(name, layer)
        return self._f32[key]

    def f64(self, name: str, layer: int = -1) -> np.ndarray:
        key = (name, layer)
        if key in self._f64:
            return self._f64[key]
        w = self.f32(name, layer).astype(np.float64)
        if self.cache_f64:
            self._f64[key] = w
        return w

    def norm(self, layer: int = -1) -> np.ndarray:
        """RMSNorm weight: 1.0 everywhere (the configs state weights 1.0)."""
        return np.ones(self.cfg.hidden, dtype=np.float64)

    def set(self, name: str, layer: int, value: np.ndarray) -> None:
        """Override a tensor (oracle self-tests only)."""
        self._f32[(name, layer)] = np.asarray(value, dtype=np.float32)
        self._f64.pop((name, layer), None)
        if np.asarray(value).dtype == np.float64:
            self._f64[(name, layer)] = np.asarray(value)


# ----------------------------------------------------------------------------
# the operations
# ----------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """fp64 angles pos * theta^(-2j/d), j = 0 .. d/2-1; shape [n, d/2]."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / head_dim)
    return np.outer(np.asarray(positions, dtype=np.float64), inv_freq)


def apply_rope(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE: pair (j, j + d/2) rotated by ang[:, j]. x: [n, heads, d]."""
    h = x.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with masked entries given as -inf (two-pass: max, then normalised exp)."""
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """o[t, h] = softmax_tau(q[t,h] . k[tau, h//g] / sqrt(d) | visible[t, tau]) @ v[:, h//g].

    q [n, Hq, d]; k, v [T, Hkv, d] in logical order; visible [n, T] bool.
    """
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.empty((n, hq, v.shape[-1]), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for h in range(hq):
        kh = h // g
        s = (q[:, h, :] @ k[:, kh, :].T) * scale
        s = np.where(visible, s, -np.inf)
        out[:, h, :] = softmax_rows(s) @ v[:, kh, :]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(u: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Wdown-map of silu(u Wgate^T) * (u Wup^T)."""
    return (silu(u @ wg.T) * (u @ wu.T)) @ wd.T


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def geglu_ffn(u: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Wdown-map of gelu(u Wgate^T) * (u Wup^T)."""
    return (gelu_erf(u @ wg.T) * (u @ wu.T)) @ wd.T


def ffn(cfg: "Config", u: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    return (geglu_ffn if cfg.ffn_kind == "geglu" else swiglu_ffn)(u, wg, wu, wd)


# ----------------------------------------------------------------------------
# KV stores: a contiguous one and a paged one (physical pool + block tables)
# ----------------------------------------------------------------------------
class ContiguousKV:
    """Per-segment K/V arrays, gathered in logical (creation) order."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.k = {}   # (segment id, layer) -> [ntok, Hkv, d]
        self.v = {}

    def write(self, seg_id, seg: Segment, layer, offset, k, v):
        kk = self.k.setdefault((seg_id, layer), np.zeros((0,) + k.shape[1:]))
        vv = self.v.setdefault((seg_id, layer), np.zeros((0,) + v.shape[1:]))
        assert kk.shape[0] == offset
        self.k[(seg_id, layer)] = np.concatenate([kk, k.astype(np.float64)])
        self.v[(seg_id, layer)] = np.concatenate([vv, v.astype(np.float64)])

    def read(self, seg_id, seg: Segment, layer):
        return self.k[(seg_id, layer)], self.v[(seg_id, layer)]

    def drop(self, seg_id):
        for key in [k for k in self.k if k[0] == seg_id]:
            del self.k[key]
            del self.v[key]


class PagedKV:
    """Physical pool K,V[L][num_blocks][block_tokens][Hkv][d] addressed through block tables."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        shape = (cfg.n_layers, cfg.num_blocks, cfg.block_tokens, cfg.n_kv_heads, cfg.head_dim)
        self.k = np.full(shape, np.nan)
        self.v = np.full(shape, np.nan)

    def write(self, seg_id, seg: Segment, layer, offset, k, v):
        bt = self.cfg.block_tokens
        for i in range(k.shape[0]):
            t = offset + i
            b = seg.blocks[t // bt]
            self.k[layer, b, t % bt] = k[i]
            self.v[layer, b, t % bt] = v[i]

    def read(self, seg_id, seg: Segment, layer):
        bt = self.cfg.block_tokens
        idx_b = [seg.blocks[t // bt] for t in range(seg.ntok)]
        idx_t = [t % bt for t in range(seg.ntok)]
        return self.k[layer, idx_b, idx_t], self.v[layer, idx_b, idx_t]

    def drop(self, seg_id):
        pass


# ----------------------------------------------------------------------------
# the cached decoder session
# ----------------------------------------------------------------------------
class Session:
    """State of one model instance: weights, block pool, segments, KV, position counter.

    Mirrors what the GPU library keeps behind its handle, in fp64.
    """

    def __init__(self, cfg: Config, weights: Weights | None = None, paged: bool = False,
                 initial_free=None):
        self.cfg = cfg
        self.w = weights if weights is not None else Weights(cfg)
        self.pool = BlockPool(cfg.num_blocks, initial_free)
        self.kv = PagedKV(cfg) if paged else ContiguousKV(cfg)
        self.segments: list[tuple[int, Segment]] = []   # (segment id, segment) in logical order
        self._next_seg = 0
        self.next_pos = 0
        self.next_frame_id = 0
        self.last_logits = None

    # -- bookkeeping ---------------------------------------------------------
    def frames(self):
        return [s for _, s in self.segments if s.kind == "frame"]

    def resident_tokens(self) -> int:
        return sum(s.ntok for _, s in self.segments)

    def block_table(self):
        """Logical block list with valid-token counts: [(block, ntok_in_block), ...]."""
        bt = self.cfg.block_tokens
        out = []
        for _, s in self.segments:
            for i, b in enumerate(s.blocks):
                out.append((b, min(bt, s.ntok - i * bt)))
        return out

    def _new_frame(self, n: int) -> tuple[int, Segment]:
        bt = self.cfg.block_tokens
        if len(self.frames()) >= self.cfg.max_frames:
            raise NoBlocks("frame registry full")
        blocks = self.pool.alloc(-(-n // bt))
        seg = Segment("frame", self.next_frame_id, self.next_pos, n, blocks)
        sid = self._next_seg
        self._next_seg += 1
        self.segments.append((sid, seg))
        self.next_frame_id += 1
        self.next_pos += n
        return sid, seg

    def _tail_slot(self) -> tuple[int, Segment, int]:
        """Segment and offset that receive one decode token (allocating a block if needed)."""
        bt = self.cfg.block_tokens
        if self.segments and self.segments[-1][1].kind == "tail":
            sid, seg = self.segments[-1]
            if seg.ntok == len(seg.blocks) * bt:
                seg.blocks.extend(self.pool.alloc(1))
        else:
            blocks = self.pool.alloc(1)
            seg = Segment("tail", -1, self.next_pos, 0, blocks)
            sid = self._next_seg
            self._next_seg += 1
            self.segments.append((sid, seg))
        off = seg.ntok
        seg.ntok += 1
        self.next_pos += 1
        return sid, seg, off

    def gather(self, layer: int):
        """All resident K, V of a layer in logical order (fp64)."""
        ks, vs = [], []
        for sid, seg in self.segments:
            if seg.ntok == 0:
                continue
            k, v = self.kv.read(sid, seg, layer)
            ks.append(np.asarray(k, dtype=np.float64)[: seg.ntok])
            vs.append(np.asarray(v, dtype=np.float64)[: seg.ntok])
        c = self.cfg
        if not ks:
            z = np.zeros((0, c.n_kv_heads, c.head_dim))
            return z, z
        return np.concatenate(ks), np.concatenate(vs)

    # -- the forward ---------------------------------------------------------
    def _forward(self, x: np.ndarray, positions, place) -> np.ndarray:
        """Run every layer over n new rows; ``place(layer, k, v)`` stores their K/V.

        Returns the final hidden rows [n, H] (before the final norm).
        """
        c = self.cfg
        n = x.shape[0]
        ang = rope_angles(positions, c.head_dim, c.rope_theta)
        for l in range(c.n_layers):
            t_before = self.resident_tokens() - n   # resident tokens before this chunk
            u = rmsnorm(x, self.w.norm(l), c.rms_eps)
            q = (u @ self.w.f64("q", l).T).reshape(n, c.n_heads, c.head_dim)
            k = (u @ self.w.f64("k", l).T).reshape(n, c.n_kv_heads, c.head_dim)
            v = (u @ self.w.f64("v", l).T).reshape(n, c.n_kv_heads, c.head_dim)
            q = apply_rope(q, ang)
            k = apply_rope(k, ang)
            place(l, k, v)
            if c.kv_only_last and l == c.n_layers - 1:
                break                               # only this layer's K/V are used
            K, V = self.gather(l)
            T = K.shape[0]
            visible = np.ones((n, T), dtype=bool)
            # causal inside the chunk: the chunk is the last n resident rows
            tri = np.tril(np.ones((n, n), dtype=bool))
            visible[:, t_before:] = tri
            o = gqa_attention(q, K, V, visible)
            x = x + o.reshape(n, -1) @ self.w.f64("o", l).T
            u2 = rmsnorm(x, self.w.norm(l), c.rms_eps)
            x = x + ffn(c, u2, self.w.f64("gate", l), self.w.f64("up", l),
                        self.w.f64("down", l))
        return x

    def _logits(self, h_last: np.ndarray):
        if self.cfg.vocab == 0:
            return None                             # no output head
        u = rmsnorm(h_last, self.w.norm(), self.cfg.rms_eps)
        return self.w.f64("head") @ u

    def embed(self, tokens) -> np.ndarray:
        return self.w.f32("embed")[np.asarray(tokens, dtype=np.int64)].astype(np.float64)

    def prefill_chunk(self, tokens=None, embeds=None):
        """Append one frame (token ids or caller embeddings); returns (frame id, last-row logits)."""
        if (tokens is None) == (embeds is None):
            raise ValueError("exactly one of tokens / embeds")
        x = self.embed(tokens) if tokens is not None else np.asarray(embeds, dtype=np.float64)
        n = x.shape[0]
        if n <= 0:
            raise ValueError("empty chunk")
        sid, seg = self._new_frame(n)

        def place(l, k, v):
            self.kv.write(sid, seg, l, 0, k, v)

        h = self._forward(x, seg.positions, place)
        self.last_logits = self._logits(h[-1])
        return seg.frame_id, self.last_logits

    def decode_step(self, token: int):
        """One token at the next position; returns (greedy next token, logits)."""
        x = self.embed([token])
        sid, seg, off = self._tail_slot()

        def place(l, k, v):
            self.kv.write(sid, seg, l, off, k, v)

        h = self._forward(x, [seg.start_pos + off], place)
        self.last_logits = self._logits(h[-1])
        return int(np.argmax(self.last_logits)), self.last_logits

    def append_raw(self, k: np.ndarray, v: np.ndarray) -> int:
        """Append a frame whose stored K/V ([L][n][Hkv][d], post-RoPE) are given as is."""
        n = k.shape[1]
        sid, seg = self._new_frame(n)
        for l in range(self.cfg.n_layers):
            self.kv.write(sid, seg, l, 0, k[l], v[l])
        return seg.frame_id

    # -- scoring / eviction --------------------------------------------------
    def mean_keys(self, layer: int):
        """[(frame id, fp64 mean over the frame's tokens of its stored keys, flattened Hkv*d)]."""
        out = []
        for sid, seg in self.segments:
            if seg.kind != "frame":
                continue
            k, _ = self.kv.read(sid, seg, layer)
            out.append((seg.frame_id, np.mean(np.asarray(k, dtype=np.float64)[: seg.ntok],
                                              axis=0).reshape(-1)))
        return out

    def score(self, layer: int = 0):
        """Winner of the redundancy scoring on ``layer``: (frame id, its max cosine, m vector)."""
        from .scoring import pick_redundant
        mk = self.mean_keys(layer)
        if len(mk) < 2:
            raise NothingToEvict("fewer than 2 frames")
        ids = [f for f, _ in mk]
        idx, score, m = pick_redundant(np.stack([v for _, v in mk]))
        return ids[idx], score, m

    def evict(self, frame_id: int) -> None:
        for i, (sid, seg) in enumerate(self.segments):
            if seg.kind == "frame" and seg.frame_id == frame_id:
                self.pool.release(seg.blocks)      # pushed in logical order
                self.kv.drop(sid)
                del self.segments[i]
                return
        raise KeyError(frame_id)

    def score_and_evict(self, layer: int = 0):
        fid, score, _ = self.score(layer)
        self.evict(fid)
        return fid, score

    # -- baseline eviction policies ("Can an LLM Forget the Right Things?", section 5) --
    def pick(self, policy: str, layer: int = 0):
        """The frame a policy evicts next and its score: (frame id, score).

        semantic: the all-pairs redundancy winner (``score``);
        fifo:     the oldest resident frame (score 0);
        adjacent: the older frame of the most similar pair of frames adjacent in
                  arrival order (strict greater-than keeps the first pair on ties),
                  scored by that pair's cosine.
        """
        from .scoring import adjacent_pair_pick, cosine
        frames = self.frames()
        if not frames:
            raise NothingToEvict("no frame resident")
        if policy == "fifo":
            return frames[0].frame_id, 0.0
        if policy == "semantic":
            fid, score, _ = self.score(layer)
            return fid, score
        if policy == "adjacent":
            mk = self.mean_keys(layer)
            if len(mk) < 2:
                raise NothingToEvict("fewer than 2 frames")
            vecs = np.stack([v for _, v in mk])
            i = adjacent_pair_pick(vecs)
            return mk[i][0], cosine(vecs[i], vecs[i + 1])
        raise ValueError(policy)

    def make_room(self, policy: str, n_tokens: int, window: int = 0, layer: int = 0):
        """Evict frames chosen by ``policy`` until a frame of n_tokens fits (its blocks and
        a frame slot are free) and, with window > 0, fewer than ``window`` frames are
        resident (a sliding window of at most ``window`` frames after the insert). With
        one frame left every policy takes it. Returns the evicted frame ids; raises
        NoBlocks (state unchanged) when even an empty cache would not make room."""
        bt = self.cfg.block_tokens
        need = -(-n_tokens // bt)
        evictable = sum(len(s.blocks) for s in self.frames())
        if need > len(self.pool.free) + evictable:
            raise NoBlocks(f"need {need} blocks, at most {len(self.pool.free) + evictable}")
        out = []
        while (len(self.pool.free) < need or len(self.frames()) >= self.cfg.max_frames
               or (window > 0 and len(self.frames()) >= window)):
            frames = self.frames()
            fid = frames[0].frame_id if len(frames) == 1 else self.pick(policy, layer)[0]
            self.evict(fid)
            out.append(fid)
        return out

    def rollback(self, keep_frame_id: int) -> None:
        """Drop every segment created after frame ``keep_frame_id`` (newest first).

        Blocks go back in reverse allocation order, which restores the free-list
        exactly when nothing was evicted in between; the position and frame-id
        counters return to their values right after that frame.
        """
        idx = [i for i, (_, s) in enumerate(self.segments)
               if s.kind == "frame" and s.frame_id == keep_frame_id]
        if not idx:
            raise KeyError(keep_frame_id)
        keep = idx[0]
        for sid, seg in reversed(self.segments[keep + 1:]):
            self.pool.release(list(reversed(seg.blocks)))
            self.kv.drop(sid)
        self.segments = self.segments[: keep + 1]
        kept = self.segments[keep][1]
        self.next_pos = kept.start_pos + kept.ntok
        self.next_frame_id = keep_frame_id + 1


# ----------------------------------------------------------------------------
# the dense, uncached definition (no KV cache): used to pin the cached session
# ----------------------------------------------------------------------------
def dense_forward(cfg: Config, w: Weights, x: np.ndarray, positions) -> np.ndarray:
    """Causal forward over the whole sequence at once; returns logits for every row [T, V]."""
    T = x.shape[0]
    ang = rope_angles(positions, cfg.head_dim, cfg.rope_theta)
    causal = np.tril(np.ones((T, T), dtype=bool))
    for l in range(cfg.n_layers):
        u = rmsnorm(x, w.norm(l), cfg.rms_eps)
        q = apply_rope((u @ w.f64("q", l).T).reshape(T, cfg.n_heads, cfg.head_dim), ang)
        k = apply_rope((u @ w.f64("k", l).T).reshape(T, cfg.n_kv_heads, cfg.head_dim), ang)
        v = (u @ w.f64("v", l).T).reshape(T, cfg.n_kv_heads, cfg.head_dim)
        o = gqa_attention(q, k, v, causal)
        x = x + o.reshape(T, -1) @ w.f64("o", l).T
        u2 = rmsnorm(x, w.norm(l), cfg.rms_eps)
        x = x + ffn(cfg, u2, w.f64("gate", l), w.f64("up", l), w.f64("down", l))
    u = rmsnorm(x, w.norm(), cfg.rms_eps)
    return u @ w.f64("head").T
