"""GPU parity of the INT4 group-128 path (bf16 activations) against the CPU oracle.

The oracle runs the same decoder in fp64 on the dequantised weights w_hat = q * s
("Rebuilding Kshipra Around Memory", section 2: INT4 per group of 128, one fp16
scale per group, the same scale to encode and decode). Inputs from synth.py,
expected values from oracle/ only.
"""
import numpy as np
import pytest

import kv_cached_gqa_decoder_amd as vla
import synth
from oracle import decoder as D
from tests.gpu_util import (check_argmax, check_logits, dev_from_storage, log, logits_of,
                            metrics, oracle_config)
from tests.test_gpu_parity import TINY_INT4

pytestmark = pytest.mark.gpu


class _Pair:
    """One model on each side, driven in lock step."""

    def __init__(self, p, init_std):
        self.p = p
        self.sess = D.Session(oracle_config(p, init_std=init_std))
        self.m = vla.Model(vla.make_config(**p, init_std=init_std))
        self.call = 0

    def raw(self, seed, f, n):
        p = self.p
        (k32, v32), (ks, vs) = synth.raw_kv_frame(seed, f, p["n_layers"], n, p["n_kv_heads"],
                                                  p["head_dim"], "bf16")
        fid = self.m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), n)
        assert fid == self.sess.append_raw(k32, v32)

    def embeds(self, n, what):
        x32, xs = synth.embeddings(self.p["seed"], self.call, n, self.p["hidden"], "bf16")
        self.call += 1
        fid = self.m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n)
        ofid, ref = self.sess.prefill_chunk(embeds=x32)
        assert fid == ofid
        check_logits(logits_of(self.m), ref, "bf16", what)
        return ref

    def ids(self, n, what):
        ids = synth.token_ids(self.p["seed"], self.call, n, self.p["vocab"])
        self.call += 1
        fid = self.m.prefill_chunk(tokens=ids)
        ofid, ref = self.sess.prefill_chunk(tokens=ids)
        assert fid == ofid
        check_logits(logits_of(self.m), ref, "bf16", what)
        return ref

    def decode(self, ref, k, what):
        tok = int(np.argmax(ref))
        for i in range(k):
            g = self.m.decode_step(tok)
            nxt, ref = self.sess.decode_step(tok)
            check_logits(logits_of(self.m), ref, "bf16", f"{what} decode {i}")
            check_argmax(g, ref, "bf16", f"{what} decode {i}")
            tok = nxt
        return ref


def test_int4_ragged_chunks_and_decodes():
    """Tiny INT4 decoder: chunks of 37, 100, 16 and 1 rows (partial 64-row GEMM
    tiles), decode tails inside and across blocks."""
    t = _Pair(TINY_INT4, 0.08)
    ref = t.embeds(37, "int4 prefill 37")
    ref = t.ids(100, "int4 prefill ids 100")
    ref = t.decode(ref, 3, "int4")
    ref = t.embeds(16, "int4 prefill 16")
    ref = t.embeds(1, "int4 prefill 1")
    ref = t.decode(ref, 18, "int4")
    blocks, ntok = t.m.block_table()
    assert [(int(b), int(n)) for b, n in zip(blocks, ntok)] == t.sess.block_table()
    t.m.close()


def test_int4_llama3_8b_shape_one_layer():
    """The Llama-3-8B layer shape (hidden 4096, 32/8 heads, FFN 14336) with one layer
    and a 4,096-entry vocabulary: a 2,000-token raw cached context, a 512-token chunk
    (64-row tiles, no K split), a 40-token chunk (the residual projections split
    their 32 or 112 groups, with a short last split) and 3 decodes."""
    p = dict(vla.PRESETS["c5_llama3_8b_int4"], n_layers=1, vocab=4096, num_blocks=200,
             max_frames=16)
    t = _Pair(p, 0.02)
    for f in range(4):
        t.raw(21, f, 500)
    ref = t.ids(512, "llama3-8b-shape prefill 512")
    ref = t.embeds(40, "llama3-8b-shape prefill 40")
    ref = t.decode(ref, 3, "llama3-8b-shape")
    log("llama3-8b shape: last logits cos %.6f rel %.2e" % metrics(logits_of(t.m), ref))
    t.m.close()


def test_int4_wide_rows_one_layer():
    """Rows wider than 4096 on one layer (hidden 5120, 40/8 heads, FFN 13824): the
    q/k/v projection takes whole 5120-wide rows per wavefront (4 blocks of 64
    chunks), the gated projection the grid-stride loop over 8-row groups, the O
    projection (K 5120) and the down projection (K 13824) the 2-row streaming loop
    with a short last block; chunks of 70 and 1 rows, then 3 decodes."""
    p = dict(vla.PRESETS["c5_llama3_8b_int4"], n_layers=1, hidden=5120, n_heads=40, n_kv_heads=8,
             ffn=13824, vocab=4096, num_blocks=40, max_frames=8, max_chunk=128)
    t = _Pair(p, 0.02)
    ref = t.embeds(70, "wide-rows prefill 70")
    ref = t.embeds(1, "wide-rows prefill 1")
    ref = t.decode(ref, 3, "wide-rows")
    log("wide rows: last logits cos %.6f rel %.2e" % metrics(logits_of(t.m), ref))
    t.m.close()


def test_int4_llama3_8b_shape_full_120k_context_one_layer():
    """The long-context workload at its full size on one layer: a 120,000-token raw
    prefix (235 frames of up to 512 tokens, 7,500 blocks), the 512-token chunk of ids
    and 2 decodes, in the launch configuration the benchmark times (the output head
    aside, every kernel shape depends on the context and the layer width, not on the
    layer count)."""
    p = dict(vla.PRESETS["c5_llama3_8b_int4"], n_layers=1, vocab=4096)
    t = _Pair(p, 0.02)
    done, f = 0, 0
    while done < 120000:
        n = min(512, 120000 - done)
        t.raw(31, f, n)
        done += n
        f += 1
    ref = t.ids(512, "120K-context prefill 512")
    ref = t.decode(ref, 2, "120K-context")
    t.m.close()
