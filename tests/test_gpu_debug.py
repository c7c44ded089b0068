"""The debug build (libeagle3_debug.so): the same kernels, with each call's
device-resident indices checked on the host before anything is enqueued.

On valid inputs it must give the release library's results bit for bit.  On
inputs that break the range contract (a page id outside the cache, a token id
outside the vocabulary, a d2t target outside the vocabulary, a context past
max_ctx, inconsistent extend boundaries) it must return
EAGLE3_ERR_INVALID_ARG -- found on the host, so no kernel ever sees them."""
import pytest
import torch

import workloads as W
from eagle_draft_head_step_amd import binding
from gpu_util import DEV, clone, dev_state, gpu_chain, to_dev

pytestmark = pytest.mark.gpu

INVALID = -1


def _heads(cfg, Wt):
    return binding.DraftHead(cfg, to_dev(Wt)), binding.DraftHead(cfg, to_dev(Wt), debug=True)


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_debug_build_matches_release(name):
    cfg = W.get_config(name)
    print(f"[debug] {name}: release vs debug", flush=True)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    rel, dbg = _heads(cfg, Wt)
    d = dev_state(cfg, st)
    out = []
    for head in (rel, dbg):
        dd = clone(d)
        ws = head.workspace(cfg.batch, cfg.max_ctx, cfg.gamma)
        out.append(gpu_chain(head, cfg, dd, ws, cfg.gamma) + tuple(dd[k] for k in W.cache_keys(cfg)))
    torch.cuda.synchronize()
    for a, b in zip(*out):
        assert torch.equal(a, b)


def _expect(code, fn):
    with pytest.raises(binding.Eagle3Error) as e:
        fn()
    assert e.value.code == code


@pytest.mark.parametrize("name", ["mha_small", "mla_small"])
def test_debug_build_rejects_out_of_range(name):
    cfg = W.get_config(name)
    print(f"[debug] {name}: range checks", flush=True)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    _, dbg = _heads(cfg, Wt)
    d = dev_state(cfg, st)
    g = cfg.gamma
    ws = dbg.workspace(cfg.batch, cfg.max_ctx, g)
    kc = d["k_cache"] if cfg.attn_kind == 0 else d["kv_cache"]
    num_pages = int(kc.shape[0])

    def chain(dd, head=dbg):
        return gpu_chain(head, cfg, dd, ws, g)

    # a page id past the cache, in a page the chain reads
    dd = clone(d)
    dd["block_table"][0, 0] = num_pages
    _expect(INVALID, lambda: chain(dd))
    # a negative page id in the page the chain's last step writes
    dd = clone(d)
    last = (int(st["ctx_len"][1]) + g - 1) // cfg.page_size
    dd["block_table"][1, last] = -1
    _expect(INVALID, lambda: chain(dd))
    # a token id outside the target vocabulary
    dd = clone(d)
    dd["token_in"][0] = cfg.target_vocab
    _expect(INVALID, lambda: chain(dd))
    # a context past max_ctx
    dd = clone(d)
    _expect(INVALID, lambda: gpu_chain(dbg, cfg, dd, ws, g, max_ctx=int(st["ctx_len"].max()) - 1))
    # a d2t target outside the target vocabulary
    bad = dict(Wt)
    bad["d2t"] = Wt["d2t"].clone()
    bad["d2t"][3] = cfg.target_vocab - 3
    bad_head = binding.DraftHead(cfg, to_dev(bad), debug=True)
    _expect(INVALID, lambda: chain(clone(d), bad_head))
    torch.cuda.synchronize()


def test_debug_build_extend_boundaries():
    cfg = W.get_config("mha_small")
    print("[debug] mha_small: extend boundaries", flush=True)
    Wt, st = W.make_weights(cfg), W.make_inputs(cfg)
    _, dbg = _heads(cfg, Wt)
    q = [2] * cfg.batch
    ex = to_dev(W.make_extend_inputs(cfg, q))
    d = dev_state(cfg, st)
    T = int(ex["token_in"].shape[0])
    ws = dbg.extend_workspace(T, cfg.batch, cfg.max_ctx, 2)
    common = dict(max_q_len=2, aux=ex["aux"].reshape(T, -1), token_in=ex["token_in"], k_cache=d["k_cache"],
                  v_cache=d["v_cache"], block_table=d["block_table"], ctx_len=d["ctx_len"],
                  max_ctx=cfg.max_ctx, hidden_out=torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV),
                  token_out=torch.empty(T, dtype=torch.int32, device=DEV), workspace=ws)
    dbg.draft_extend(cu_seqlens=ex["cu_seqlens"], **common)       # valid
    bad = ex["cu_seqlens"].clone()
    bad[-1] = T - 1                                                # cu[B] != T
    _expect(INVALID, lambda: dbg.draft_extend(cu_seqlens=bad, **common))
    bad = ex["cu_seqlens"].clone()
    bad[1] = 3                                                     # a sequence with 3 > max_q_len new tokens
    _expect(INVALID, lambda: dbg.draft_extend(cu_seqlens=bad, **common))
    torch.cuda.synchronize()
