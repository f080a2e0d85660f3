"""dl_check_indices: the validation kernel over the paged-cache index inputs
reports exactly the violated preconditions as bits of its device word (and
0 for valid inputs).  Only the validation kernel runs on the planted bad
arrays; no compute kernel is given them."""
import numpy as np
import pytest
import torch

from transformer_decoder_layer_residual_amd import binding as dl
from transformer_decoder_layer_residual_amd import inputs as gen

from _util import DEV, dev_i32

pytestmark = pytest.mark.gpu


def run(**kw):
    word = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    dev = {k: (dev_i32(v) if isinstance(v, np.ndarray) else v) for k, v in kw.items()}
    dl.dl_check_indices(word, **dev)
    torch.cuda.synchronize()
    return int(word.item())


def prefill_case():
    cfg = gen.CONFIGS[4]
    pb = gen.packed([300, 17, 129, 1])
    bt = gen.block_table(cfg, pb.lens + 8)
    return cfg, pb, bt


def test_valid_prefill_and_decode_inputs_give_zero():
    cfg, pb, bt = prefill_case()
    kw = dict(block_table=bt.table, num_blocks=bt.num_blocks, block_size=cfg.block_size,
              positions=pb.positions, seq_of_token=pb.seq_of_token, cu_seqlens=pb.cu_seqlens,
              max_seqlen=pb.max_seqlen)
    assert run(**kw) == 0
    ctx = (pb.lens + 8).astype(np.int32)
    assert run(block_table=bt.table, num_blocks=bt.num_blocks, block_size=cfg.block_size,
               positions=ctx - 1, context_lens=ctx, max_context_len=int(ctx.max())) == 0


@pytest.mark.parametrize("plant,bit", [
    ("seq", dl.DL_CHECK_BIT_SEQ),
    ("seq_negative", dl.DL_CHECK_BIT_SEQ),
    ("position", dl.DL_CHECK_BIT_POSITION),
    ("position_past_table", dl.DL_CHECK_BIT_POSITION),
    ("block_written", dl.DL_CHECK_BIT_BLOCK),
    ("cu_decreasing", dl.DL_CHECK_BIT_CU),
    ("cu_end", dl.DL_CHECK_BIT_CU),
    ("cu_too_long", dl.DL_CHECK_BIT_CU),
])
def test_planted_prefill_violation_sets_its_bit(plant, bit):
    cfg, pb, bt = prefill_case()
    table, pos, seq, cu = bt.table.copy(), pb.positions.copy(), pb.seq_of_token.copy(), \
        pb.cu_seqlens.copy()
    max_seqlen = pb.max_seqlen
    if plant == "seq":
        seq[5] = pb.B
    elif plant == "seq_negative":
        seq[-1] = -1
    elif plant == "position":
        pos[7] = -3
    elif plant == "position_past_table":
        pos[2] = table.shape[1] * cfg.block_size
    elif plant == "block_written":
        t = int(pb.cu_seqlens[2]) + 3                 # a token of sequence 2
        table[2, pos[t] // cfg.block_size] = bt.num_blocks
    elif plant == "cu_decreasing":
        cu[2] = cu[1] - 1
    elif plant == "cu_end":
        cu[-1] = pb.T + 1
    elif plant == "cu_too_long":
        max_seqlen = pb.max_seqlen - 1
    got = run(block_table=table, num_blocks=bt.num_blocks, block_size=cfg.block_size,
              positions=pos, seq_of_token=seq, cu_seqlens=cu, max_seqlen=max_seqlen,
              T=pb.T)
    assert got == bit, (plant, got)


@pytest.mark.parametrize("plant", ["zero", "above_max", "past_table", "read_block"])
def test_planted_decode_violation_sets_its_bit(plant):
    cfg = gen.CONFIGS[3]
    ctx = np.array([130, 4000, 1, 257], np.int32)
    bt = gen.block_table(cfg, ctx)
    table = bt.table.copy()
    max_ctx = int(ctx.max())
    c = ctx.copy()
    bit = dl.DL_CHECK_BIT_CONTEXT
    if plant == "zero":
        c[2] = 0
    elif plant == "above_max":
        c[0] = max_ctx + 1
    elif plant == "past_table":
        max_ctx = table.shape[1] * cfg.block_size + 5
        c[1] = max_ctx
    else:
        table[1, 3] = -7                                 # read by context 4000, not written
        bit = dl.DL_CHECK_BIT_BLOCK
    got = run(block_table=table, num_blocks=bt.num_blocks, block_size=cfg.block_size,
              context_lens=c, max_context_len=max_ctx)
    assert got == bit, (plant, got)
