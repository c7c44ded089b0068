"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before any launch."""
import ctypes

import pytest

import workloads as W
from eagle_draft_head_step_amd import binding


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_header_symbol(L):
    names = binding.header_symbols()
    assert {"eagle3_draft_step", "eagle3_draft_chain", "eagle3_greedy_accept"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert L.eagle3_status_string(code).decode() == binding.STATUS[code]


def _cfg(name, **kw):
    return binding.make_config(W.get_config(name).replace(**kw))


def test_sizes_host_only(L):
    for name in ("tiny_mha_b1", "mha_small", "mla_small"):
        c = W.get_config(name)
        assert binding.packed_weights_size(c) > 0
        assert binding.workspace_size(c, c.batch, c.max_ctx, c.gamma) > 0
    c = W.get_config("llama3_8b_gqa_b32")
    # packed weights: every GEMM matrix once, in bf16 (tiles pad only the edges)
    H, I = c.hidden, c.intermediate
    n = (H * 3 * H + (c.n_heads + 2 * c.n_kv_heads) * c.head_dim * 2 * H + H * c.n_heads * c.head_dim
         + 2 * I * H + H * I + c.draft_vocab * H) * 2
    assert n <= binding.packed_weights_size(c) <= n + 64 * 1024


def _status(L, fn, *args):
    return getattr(L, fn)(*args)


def test_config_errors(L):
    n = ctypes.c_size_t()
    c = _cfg("mha_small")
    c.fc_in_features = 2 * c.hidden                       # fc width vs fused layers
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -2
    c = _cfg("mla_small")
    c.yarn_factor = 0.0                                    # MLA head without YaRN
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -3
    c = _cfg("mla_small")
    c.yarn_beta_fast, c.yarn_beta_slow = 1.0, 32.0         # inverted ramp
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -3
    c.yarn_beta_fast, c.yarn_beta_slow = 1.0, 1.0          # equal betas: a one-pair ramp, accepted
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == 0
    c = _cfg("mha_small")
    c.draft_vocab = c.target_vocab + 1
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -1
    c = _cfg("mha_small")
    c.n_kv_heads = 4                                       # 6 q heads over 4 kv heads
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -2
    c = _cfg("mha_small")
    c.head_dim = 48
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -3
    assert L.eagle3_packed_weights_size(None, ctypes.byref(n)) == -1
    c = _cfg("mha_small")
    assert L.eagle3_workspace_size(ctypes.byref(c), 0, 10, 1, ctypes.byref(n)) == -1
    assert L.eagle3_workspace_size(ctypes.byref(c), 4, 10, 0, ctypes.byref(n)) == -1


def _args(batch=4, **kw):
    a = binding.StepArgs()
    a.batch = batch
    fake = 0x100000          # never dereferenced: validation fails first
    for f in ("aux", "token_in", "k_cache", "v_cache", "block_table", "ctx_len", "hidden_out",
              "token_out", "workspace"):
        setattr(a, f, fake)
    a.max_pages = 4
    a.max_ctx = 100
    a.workspace_bytes = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _weights():
    w = binding.Weights()
    for n in binding.WEIGHT_NAMES:
        setattr(w, n, 0x200000)
    return w


def test_step_argument_errors(L):
    c = _cfg("mha_small")
    w = _weights()
    P = ctypes.c_void_p(0x300000)
    call = lambda a, k=0: L.eagle3_draft_step(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), k, None)
    assert call(_args(batch=0)) == -1                      # empty batch
    assert call(_args(token_in=None)) == -1
    assert call(_args(aux=None, hidden_in=None)) == -1
    assert call(_args(max_pages=1)) == -1                  # 64 slots < ctx 100 + 1
    assert call(_args(), k=-1) == -1
    assert call(_args(aux=0x100001)) == -1                 # misaligned activations
    assert call(_args()) == -4                             # workspace too small
    chain = lambda a, g: L.eagle3_draft_chain(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), g, None)
    assert chain(_args(), 0) == -1                         # gamma < 1
    assert chain(_args(max_pages=2, max_ctx=126), 3) == -1 # 128 slots < 126 + 3
    assert L.eagle3_greedy_accept(None, None, 4, 2, None, None, None) == -1
    assert L.eagle3_greedy_accept(0x1000, 0x1000, 0, 2, 0x1000, 0x1000, None) == -1
    assert L.eagle3_greedy_accept(0x1000, 0x1000, 4, 0, 0x1000, 0x1000, None) == -1


def test_target_lm_head_needs_matching_vocab(L):
    """No d2t is allowed only when the head scores over the target vocabulary."""
    P = ctypes.c_void_p(0x300000)
    c = _cfg("mha_small")                                  # draft 1000 < target 3000
    w = _weights()
    w.d2t = None
    a = _args()
    assert L.eagle3_draft_step(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), 0, None) == -1
    c = _cfg("mha_small_aux2_tgt_head")                    # draft == target vocabulary
    a = _args()
    assert L.eagle3_draft_step(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), 0, None) == -4


def _ext_args(**kw):
    a = binding.ExtendArgs()
    a.num_tokens, a.batch, a.max_q_len = 6, 3, 3
    fake = 0x100000
    for f in ("cu_seqlens", "aux", "token_in", "k_cache", "v_cache", "block_table", "ctx_len", "hidden_out",
              "token_out", "workspace"):
        setattr(a, f, fake)
    a.max_pages = 4
    a.max_ctx = 100
    a.workspace_bytes = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_extend_argument_errors(L):
    c = _cfg("mha_small")
    w = _weights()
    P = ctypes.c_void_p(0x300000)
    call = lambda a: L.eagle3_draft_extend(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), None)
    assert call(_ext_args(num_tokens=0)) == -1
    assert call(_ext_args(cu_seqlens=None)) == -1
    assert call(_ext_args(aux=None)) == -1                 # the extend always fuses aux states
    assert call(_ext_args(max_q_len=0)) == -1
    assert call(_ext_args(max_pages=1)) == -1              # 64 slots < ctx 100 + 3
    assert call(_ext_args(hidden_out=0x100001)) == -1      # misaligned
    assert call(_ext_args()) == -4                         # workspace too small
    n = ctypes.c_size_t(0)
    assert L.eagle3_extend_workspace_size(ctypes.byref(c), 8, 3, 100, 3, ctypes.byref(n)) == 0 and n.value > 0
    assert L.eagle3_extend_workspace_size(ctypes.byref(c), 0, 3, 100, 3, ctypes.byref(n)) == -1


def test_relaxed_accept_argument_errors(L):
    n = ctypes.c_size_t(0)
    assert L.eagle3_relaxed_accept_workspace_size(16, 3, 129280, ctypes.byref(n)) == 0 and n.value > 0
    assert n.value % 16 == 0
    assert L.eagle3_relaxed_accept_workspace_size(0, 3, 100, ctypes.byref(n)) == -1
    assert L.eagle3_relaxed_accept_workspace_size(4, 0, 100, ctypes.byref(n)) == -1
    assert L.eagle3_relaxed_accept_workspace_size(4, 3, 0, ctypes.byref(n)) == -1
    assert L.eagle3_relaxed_accept_workspace_size(4, 3, 100, None) == -1
    L.eagle3_relaxed_accept_workspace_size(4, 3, 100, ctypes.byref(n))
    f = 0x100000
    ok = dict(draft=f, logits=f, relaxed=None, batch=4, gamma=3, vocab=100, topk=10, delta=0.6,
              accept_len=f, bonus=f, workspace=f, workspace_bytes=n.value, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return L.eagle3_relaxed_accept(*a.values())

    assert call(draft=None) == -1
    assert call(logits=None) == -1
    assert call(workspace=None) == -1
    assert call(topk=0) == -1
    assert call(delta=-0.1) == -1
    assert call(delta=float("nan")) == -1
    assert call(delta=float("inf")) == -1
    assert call(logits=f + 2) == -1                      # misaligned
    assert call(workspace=f + 8) == -1
    assert call(batch=70000) == -1
    assert call(workspace_bytes=n.value - 1) == -4


def test_weight_format_errors(L):
    P = ctypes.c_void_p(0x300000)
    n = ctypes.c_size_t(0)
    for bad in (-1, 3):
        c = _cfg("mha_small")
        c.weight_format = bad
        assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -1
    # NVFP4 needs every GEMM input width to be a multiple of 16 (mha_small's MLP is 344 wide)
    c = _cfg("mha_small", weight_format="nvfp4")
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -3
    c = _cfg("mha_small_nvfp4")
    assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == 0
    nv = n.value
    L.eagle3_packed_weights_size(ctypes.byref(_cfg("mha_small_fp8")), ctypes.byref(n))
    f8 = n.value
    L.eagle3_packed_weights_size(ctypes.byref(_cfg("mha_small")), ctypes.byref(n))
    assert nv < f8 < n.value                         # fewer weight bytes per format
    # a quantized head without its scales is rejected before any launch
    w = _weights()
    for cname in ("mha_small_fp8", "mha_small_nvfp4"):
        c = _cfg(cname)
        assert L.eagle3_pack_weights(ctypes.byref(c), ctypes.byref(w), P, 1 << 40, None) == -1
        for i in range(len(binding.GEMM_MATS)):
            w.row_scale[i] = 0x400000
        if cname.endswith("nvfp4"):
            assert L.eagle3_pack_weights(ctypes.byref(c), ctypes.byref(w), P, 1 << 40, None) == -1
        w.row_scale[binding.GEMM_MATS.index("w_o")] = None
        assert L.eagle3_pack_weights(ctypes.byref(c), ctypes.byref(w), P, 1 << 40, None) == -1
        w = _weights()


def test_cache_dtype_and_page_count(L):
    """Only a bf16 cache matches the head's bf16 attention; a negative cache
    page count is an argument error."""
    n = ctypes.c_size_t()
    for name in ("mha_small", "mla_small"):
        c = _cfg(name)
        assert c.cache_dtype == 0
        c.cache_dtype = 1
        assert L.eagle3_packed_weights_size(ctypes.byref(c), ctypes.byref(n)) == -3
        assert L.eagle3_workspace_size(ctypes.byref(c), 4, 10, 1, ctypes.byref(n)) == -3
    c = _cfg("mha_small")
    w = _weights()
    P = ctypes.c_void_p(0x300000)
    assert L.eagle3_draft_step(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(_args(num_pages=-1)), 0,
                               None) == -1
    assert L.eagle3_draft_extend(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(_ext_args(num_pages=-1)),
                                 None) == -1


def test_debug_library_same_abi():
    """The debug build exports the same symbols and validates arguments the
    same way before its host-side range checks (which need a GPU)."""
    D = binding.lib(debug=True)
    for name in binding.header_symbols():
        assert hasattr(D, name), name
    c = _cfg("mha_small")
    w = _weights()
    P = ctypes.c_void_p(0x300000)
    call = lambda a: D.eagle3_draft_step(ctypes.byref(c), ctypes.byref(w), P, ctypes.byref(a), 0, None)
    assert call(_args(batch=0)) == -1
    assert call(_args()) == -4                             # workspace too small, found before any copy
    c.cache_dtype = 1
    n = ctypes.c_size_t()
    assert D.eagle3_workspace_size(ctypes.byref(c), 4, 10, 1, ctypes.byref(n)) == -3
