"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before anything reaches the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pf():
    import bounded_kv_cache_pf_amd as pf
    return pf


def _declared():
    text = open(os.path.join(ROOT, "include", "pf.h")).read()
    return sorted(set(re.findall(r"^[a-z_0-9 ]+\**\s*\**(pf_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_path():
    names = _declared()
    for n in ("pf_score_select", "pf_selection_deltas", "pf_rope_shift", "pf_partition_attn",
              "pf_score_select_workspace_bytes", "pf_partition_attn_workspace_bytes", "pf_abi_version",
              "pf_status_name", "pf_last_error_message"):
        assert n in names


def test_every_declared_symbol_is_exported(pf):
    for n in _declared():
        assert hasattr(pf.lib, n), n
    assert pf.lib.pf_abi_version() == 1


def test_status_names(pf):
    assert pf.lib.pf_status_name(0) == b"PF_OK"
    assert pf.lib.pf_status_name(6) == b"PF_ERR_WORKSPACE"
    assert pf.lib.pf_status_name(99) == b"PF_UNKNOWN"


A = 0x10000   # fake, aligned device addresses: validation fails before any use
B = 0x20000
C = 0x30000


def _err(pf, st):
    return pf.lib.pf_status_name(st).decode(), pf.lib.pf_last_error_message().decode()


def test_score_select_validation(pf):
    L = pf.lib
    ws = L.pf_score_select_workspace_bytes(6240, 12, 40, 182)
    assert ws > 40 * 182 // 64 * 4
    assert L.pf_score_select_workspace_bytes(0, 12, 40, 182) == 0
    assert _err(pf, L.pf_score_select(None, 6240, 12, B, 40, 182, 16, C, None, A, ws, None))[0] == "PF_ERR_NULL"
    name, msg = _err(pf, L.pf_score_select(A, 6240, 12, B, 40, 182, 41, C, None, A, ws, None))
    assert name == "PF_ERR_RANGE" and "top_k" in msg
    assert _err(pf, L.pf_score_select(A, 6240, 12, B, 40, 182, 0, C, None, A, ws, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_score_select(A, 6240, 12, B, 40, 182, 257, C, None, A, ws, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_score_select(A, 6240, 33, B, 40, 182, 16, C, None, A, ws, None))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, L.pf_score_select(A, 6240, 12, B, 5000, 182, 16, C, None, A, ws, None))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, L.pf_score_select(A + 2, 6240, 12, B, 40, 182, 16, C, None, A, ws, None))[0] == "PF_ERR_MISALIGNED"
    name, msg = _err(pf, L.pf_score_select(A, 6240, 12, B, 40, 182, 16, C, None, A, ws - 1, None))
    assert name == "PF_ERR_WORKSPACE" and str(ws) in msg
    assert _err(pf, L.pf_score_select(A, 6240, 12, B, 40, 182, 16, C, None, None, ws, None))[0] == "PF_ERR_WORKSPACE"
    assert _err(pf, L.pf_score_select(A, 0, 12, B, 40, 182, 16, C, None, A, ws, None))[0] == "PF_ERR_SHAPE"


def test_random_select_validation(pf):
    L = pf.lib
    assert _err(pf, L.pf_select_random(40, 16, 1, 0, 1, None, None))[0] == "PF_ERR_NULL"
    assert _err(pf, L.pf_select_random(40, 41, 1, 0, 1, A, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_select_random(40, 0, 1, 0, 1, A, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_select_random(5000, 16, 1, 0, 1, A, None))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, L.pf_select_random(40, 16, 1, 0, 0, A, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_select_random(40, 16, 1, 0, 1, A + 2, None))[0] == "PF_ERR_MISALIGNED"


def test_deltas_validation(pf):
    L = pf.lib
    assert _err(pf, L.pf_selection_deltas(None, 16, B, 40, 168, 4, C, None))[0] == "PF_ERR_NULL"
    assert _err(pf, L.pf_selection_deltas(A, 41, B, 40, 168, 4, C, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_selection_deltas(A, 16, B, 40, 168, 0, C, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_selection_deltas(A + 1, 16, B, 40, 168, 4, C, None))[0] == "PF_ERR_MISALIGNED"


def test_rope_validation(pf):
    L = pf.lib
    assert L.pf_rope_shift(None, 12, 182, 40, None, None, 0, 1e4, None) == 0     # nothing to do
    assert L.pf_last_error_message() == b""
    assert _err(pf, L.pf_rope_shift(None, 12, 182, 40, B, C, 16, 1e4, None))[0] == "PF_ERR_NULL"
    assert _err(pf, L.pf_rope_shift(A, 12, 182, 40, B, None, 16, 1e4, None))[0] == "PF_ERR_NULL"
    assert _err(pf, L.pf_rope_shift(A, 40, 182, 40, B, C, 16, 1e4, None))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, L.pf_rope_shift(A, 12, 182, 40, None, C, 41, 1e4, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_rope_shift(A, 12, 182, 40, B, C, -1, 1e4, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_rope_shift(A, 12, 182, 40, B, C, 16, 1.0, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_rope_shift(A + 8, 12, 182, 40, B, C, 16, 1e4, None))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, L.pf_rope_shift(A, 12, 0, 40, B, C, 16, 1e4, None))[0] == "PF_ERR_SHAPE"


def test_batched_validation(pf):
    L = pf.lib
    one = L.pf_score_select_workspace_bytes(6240, 12, 116, 182)
    ws30 = L.pf_score_select_batched_workspace_bytes(6240, 12, 116, 182, 30)
    assert ws30 == 30 * one and one % 256 == 0
    assert L.pf_score_select_batched_workspace_bytes(6240, 12, 116, 182, 0) == 0
    qs, ps = 6240 * 12 * 128, 116 * 182 * 12 * 128
    assert _err(pf, L.pf_score_select_batched(A, qs, 6240, 12, B, ps, 116, 182, 16, 0, C, None, A, ws30,
                                              None))[0] == "PF_ERR_RANGE"
    name, msg = _err(pf, L.pf_score_select_batched(A, qs - 8, 6240, 12, B, ps, 116, 182, 16, 30, C, None, A,
                                                   ws30, None))
    assert name == "PF_ERR_SHAPE" and "q_batch_stride" in msg
    assert _err(pf, L.pf_score_select_batched(A, qs + 4, 6240, 12, B, ps, 116, 182, 16, 30, C, None, A, ws30,
                                              None))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, L.pf_score_select_batched(A, qs, 6240, 12, B, ps, 116, 182, 16, 30, C, None, A, ws30 - 1,
                                              None))[0] == "PF_ERR_WORKSPACE"
    assert _err(pf, L.pf_selection_deltas_batched(A, 16, B, 116, 480, 4, 0, C, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_rope_shift_batched(A, ps, 12, 182, 116, B, C, 16, 70000, 1e4, None))[0] == "PF_ERR_RANGE"
    name, msg = _err(pf, L.pf_rope_shift_batched(A, ps - 8, 12, 182, 116, B, C, 16, 30, 1e4, None))
    assert name == "PF_ERR_SHAPE" and "k_batch_stride" in msg


def test_rollin_validation(pf):
    L = pf.lib
    assert _err(pf, L.pf_rollin(None, B, C, 12, 182, 40, A, B, 0, None))[0] == "PF_ERR_NULL"
    assert _err(pf, L.pf_rollin(A, B, C, 40, 182, 40, A, B, 0, None))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, L.pf_rollin(A, B, C, 12, 182, -1, A, B, 0, None))[0] == "PF_ERR_RANGE"
    assert _err(pf, L.pf_rollin(A + 8, B, C, 12, 182, 4, A, B, 0, None))[0] == "PF_ERR_MISALIGNED"
    blk = 182 * 12 * 128
    name, msg = _err(pf, L.pf_rollin_batched(A, B, 40 * blk, C, 41, 12, 182, 40, A, B, blk, 0, 30, None))
    assert name == "PF_ERR_SHAPE" and "slot" in msg


def _attn(pf, **kw):
    args = dict(q=A, n_q=6240, H=12, sk=B, sv=C, ns=12480, pk=B, pv=C, nb=40, nc=182, ids=A, nsel=16,
                rk=B, rv=C, nr=6240, ck=B, cv=C, ncur=6240, scale=0.0, o=A, lse=None, ws=None, wsb=0)
    args.update(kw)
    a = args
    return pf.lib.pf_partition_attn(a["q"], a["n_q"], a["H"], a["sk"], a["sv"], a["ns"], a["pk"], a["pv"],
                                    a["nb"], a["nc"], a["ids"], a["nsel"], a["rk"], a["rv"], a["nr"],
                                    a["ck"], a["cv"], a["ncur"], a["scale"], a["o"], a["lse"], a["ws"],
                                    a["wsb"], None)


def test_attn_validation(pf):
    assert _err(pf, _attn(pf, q=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _attn(pf, o=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _attn(pf, sk=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _attn(pf, ids=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _attn(pf, nsel=41))[0] == "PF_ERR_RANGE"
    assert _err(pf, _attn(pf, nsel=1025, nb=2000))[0] == "PF_ERR_RANGE"
    assert _err(pf, _attn(pf, H=0))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, _attn(pf, n_q=0))[0] == "PF_ERR_SHAPE"
    assert _err(pf, _attn(pf, nc=0))[0] == "PF_ERR_SHAPE"
    assert _err(pf, _attn(pf, ns=-1))[0] == "PF_ERR_SHAPE"
    assert _err(pf, _attn(pf, ns=0, nsel=0, nr=0, ncur=0))[0] == "PF_ERR_SHAPE"
    assert _err(pf, _attn(pf, rk=B + 4))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, _attn(pf, lse=A + 2))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, _attn(pf, ns=1 << 31))[0] == "PF_ERR_UNSUPPORTED"
    # the pool is addressed with 32-bit byte offsets: under 2 GiB of K (or V)
    rows_2gib = (1 << 31) // (12 * 128 * 2)
    name, msg = _err(pf, _attn(pf, nb=rows_2gib // 182 + 1))
    assert name == "PF_ERR_UNSUPPORTED" and "pool" in msg
    assert _err(pf, _attn(pf, nb=rows_2gib // 182 - 1, ws=None))[0] == "PF_ERR_WORKSPACE"   # passes the pool check
    # contiguous partitions of 2 GiB or more are accepted (their tiles are
    # addressed from each tile's first row): the call gets past every shape
    # check and stops at the missing workspace, before any launch
    for part in ("ns", "nr", "ncur"):
        big = dict(ns=12480, nr=6240, ncur=6240)
        big[part] = rows_2gib + 1000
        n_keys = big["ns"] + 16 * 182 + big["nr"] + big["ncur"]
        assert pf.lib.pf_partition_attn_workspace_bytes(6240, 12, n_keys) > 0
        assert _err(pf, _attn(pf, ws=None, wsb=0, **big))[0] == "PF_ERR_WORKSPACE", part
    need = pf.lib.pf_partition_attn_workspace_bytes(6240, 12, 27872)
    assert need > 0
    name, msg = _err(pf, _attn(pf, ws=None, wsb=0))
    assert name == "PF_ERR_WORKSPACE" and str(need) in msg
    assert _err(pf, _attn(pf, ws=C, wsb=need - 1))[0] == "PF_ERR_WORKSPACE"
    assert _err(pf, _attn(pf, ws=C + 8, wsb=need))[0] == "PF_ERR_MISALIGNED"


def test_attention_tail_plan_sizes(pf):
    # The workspace holds one partial slot (256 x 128 fp32 U, then m and l) per
    # key segment of the tail units. Without a GPU the library plans for 256
    # resident workgroups (one per CU of an MI355X). After floor(U / 256) whole
    # rounds, full tail units and the heads' partial last units (n_q % 256
    # queries) each get one segment count; a partial unit with at most four
    # live waves counts 3/4 of a full unit per key tile, and segments hold at
    # least 16 key tiles.
    slot = (256 * 128 + 2 * 256) * 4
    ws = pf.lib.pf_partition_attn_workspace_bytes
    # 6240 q x 12 heads: 24 full + 1 partial (96 q, 3 live waves) units per head,
    # 300 units: 256 whole, then 32 full x 6 segments + 12 partial x 5
    assert ws(6240, 12, 27872) == (32 * 6 + 12 * 5) * slot
    # 1100 q x 7 heads: 28 full units x 7 segments + 7 partial (76 q) x 6
    assert ws(1100, 7, 20000) == (28 * 7 + 7 * 6) * slot
    # 6300 q: partial units with 156 q (five live waves) cost as much as full
    # ones; 47 key tiles allow two segments of each
    assert ws(6300, 12, 6000) == (32 * 2 + 12 * 2) * slot
    # 6144 q: no partial units; 32 tail units x 8 segments
    assert ws(6144, 12, 27872) == 32 * 8 * slot
    # 24 key tiles: too short to cut, the tail units run whole (no workspace)
    assert ws(6300, 12, 3000) == 0


def test_binding_rejects_cpu_tensors(pf):
    import torch
    q = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pf.pf_partition_attn(q, q, q, None, None, 8, None, None, None, q, q)


def _conv(pf, **kw):
    a = dict(x=A, nb=1, T=4, H=60, W=104, ci=16, kt=2, kh=1, kw=1, w=B, b=None, co=256, act=1, y=C, ws=None, wsb=0)
    a.update(kw)
    return pf.lib.pf_hr_conv(a["x"], a["nb"], a["T"], a["H"], a["W"], a["ci"], a["kt"], a["kh"], a["kw"], a["w"],
                             a["b"], a["co"], a["act"], a["y"], a["ws"], a["wsb"], None)


def test_hr_conv_validation(pf):
    assert _err(pf, _conv(pf, x=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _conv(pf, w=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _conv(pf, y=None))[0] == "PF_ERR_NULL"
    assert _err(pf, _conv(pf, x=A + 8))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, _conv(pf, b=B + 2))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, _conv(pf, nb=0))[0] == "PF_ERR_SHAPE"
    assert _err(pf, _conv(pf, T=1))[0] == "PF_ERR_SHAPE"            # smaller than the kernel
    assert _err(pf, _conv(pf, ci=8))[0] == "PF_ERR_UNSUPPORTED"     # not a multiple of 16
    assert _err(pf, _conv(pf, co=40))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, _conv(pf, kt=0))[0] == "PF_ERR_UNSUPPORTED"
    assert _err(pf, _conv(pf, kt=4, kh=4, kw=8, T=8, H=8, W=8))[0] == "PF_ERR_UNSUPPORTED"   # 128 taps
    # a deep, narrow stage asks for a split-K workspace and refuses to run without it
    need = pf.lib.pf_hr_conv_workspace_bytes(1, 2, 14, 26, 1024, 1, 2, 2, 2048)
    assert need > 0
    name, msg = _err(pf, _conv(pf, T=2, H=14, W=26, ci=1024, kt=1, kh=2, kw=2, co=2048))
    assert name == "PF_ERR_WORKSPACE" and str(need) in msg
    # a shallow stage needs none
    assert pf.lib.pf_hr_conv_workspace_bytes(1, 4, 60, 104, 16, 2, 1, 1, 256) == 0


def test_hr_branch_validation(pf):
    L = pf.lib
    widths = (ctypes.c_int * 4)(256, 512, 1024, 2048)
    ws = (ctypes.c_void_p * 4)(B, B, B, B)
    bs = (ctypes.c_void_p * 4)(None, None, None, None)
    need = L.pf_hr_branch_workspace_bytes(1, 4, 60, 104, 16, widths, 1536)
    assert need > 0
    call = lambda **k: L.pf_hr_branch(k.get("z", A), 1, k.get("T", 4), k.get("H", 60), k.get("W", 104), 16,
                                      k.get("ws_", ws), bs, k.get("widths", widths), B, None, 1536, C,
                                      k.get("wsp", A), k.get("wsb", need), None)
    assert _err(pf, call(z=None))[0] == "PF_ERR_NULL"
    assert _err(pf, call(ws_=None))[0] == "PF_ERR_NULL"
    assert _err(pf, call(T=1))[0] == "PF_ERR_SHAPE"
    assert _err(pf, call(H=7))[0] == "PF_ERR_SHAPE"
    bad = (ctypes.c_int * 4)(256, 500, 1024, 2048)
    assert _err(pf, call(widths=bad))[0] == "PF_ERR_UNSUPPORTED"
    name, msg = _err(pf, call(wsb=need - 1))
    assert name == "PF_ERR_WORKSPACE" and str(need) in msg
    assert _err(pf, call(wsp=None))[0] == "PF_ERR_WORKSPACE"
    # the output size the binding allocates comes from the library: the
    # default block gives the pages' 182 tokens
    assert L.pf_hr_branch_out_tokens(4, 60, 104) == 182
    assert L.pf_hr_branch_out_tokens(5, 63, 111) == 2 * 7 * 13
    assert L.pf_hr_branch_out_tokens(1, 60, 104) == 0


def test_select_place_validation(pf):
    L = pf.lib
    need = L.pf_score_select_workspace_bytes(6240, 12, 40, 182)
    call = lambda **k: L.pf_select_place(A, 6240, 12, B, 40, 182, k.get("top_k", 16), k.get("tags", C), 176, 4,
                                         A, k.get("deltas", B), None, k.get("ws", C), need, None)
    assert _err(pf, call(tags=None))[0] == "PF_ERR_NULL"
    assert _err(pf, call(deltas=None))[0] == "PF_ERR_NULL"
    assert _err(pf, call(tags=C + 2))[0] == "PF_ERR_MISALIGNED"
    assert _err(pf, call(top_k=41))[0] == "PF_ERR_RANGE"
    assert _err(pf, call(ws=None))[0] == "PF_ERR_WORKSPACE"


class _FakeDev:
    """Stands in for a device tensor in the binding's host-side checks: the
    attributes those checks read, backed by a CPU tensor. No call gets as far
    as the library, so nothing is ever dereferenced."""

    def __init__(self, t, device="cuda:0"):
        import torch
        self._t = t
        self.is_cuda = True
        self.device = torch.device(device)
        self.dtype = t.dtype
        self.shape = t.shape

    def dim(self):
        return self._t.dim()

    def numel(self):
        return self._t.numel()

    def element_size(self):
        return self._t.element_size()

    def is_contiguous(self):
        return self._t.is_contiguous()

    def stride(self, *a):
        return self._t.stride(*a)

    def __getitem__(self, i):
        return _FakeDev(self._t[i], str(self.device))

    def data_ptr(self):
        raise AssertionError("the binding must reject this call before passing pointers")


def _fake(shape, dtype=None, device="cuda:0"):
    import torch
    return _FakeDev(torch.zeros(shape, dtype=dtype or torch.bfloat16), device)


def test_binding_checks_attention_outputs(pf):
    import torch
    H, n = 2, 64
    q = _fake((n, H, 128))
    kv = _fake((32, H, 128))
    call = lambda **k: pf.pf_partition_attn(q, kv, kv, None, None, 8, None, kv, kv, kv, kv, **k)
    with pytest.raises(ValueError, match="shape"):
        call(o=_fake((n - 1, H, 128)))                         # one row short
    with pytest.raises(TypeError):
        call(o=_fake((n, H, 128), torch.float32))              # wrong dtype
    with pytest.raises(ValueError, match="CUDA"):
        call(o=torch.zeros((n, H, 128), dtype=torch.bfloat16))  # host buffer
    with pytest.raises(ValueError, match="cuda:1"):
        call(o=_fake((n, H, 128), device="cuda:1"))            # another device
    with pytest.raises(ValueError, match="lse"):
        call(o=_fake((n, H, 128)), lse=_fake((H, n - 1), torch.float32))
    with pytest.raises(TypeError, match="lse"):
        call(o=_fake((n, H, 128)), lse=_fake((H, n), torch.float16))
    with pytest.raises(TypeError, match="workspace"):
        call(o=_fake((n, H, 128)), workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="recent_k"):
        pf.pf_partition_attn(q, kv, kv, None, None, 8, None, _fake((32, H, 128), device="cuda:1"), kv, kv, kv)


def test_binding_checks_selection_outputs(pf):
    import torch
    H, n, n_c, M, k = 2, 64, 8, 10, 4
    q = _fake((n, H, 128))
    pool = _fake((M * n_c, H, 128))
    tags = _fake((M,), torch.int32)
    with pytest.raises(ValueError, match="ids_out"):
        pf.pf_score_select(q, pool, n_c, k, ids_out=_fake((k - 1,), torch.int32))
    with pytest.raises(ValueError, match="scores_out"):
        pf.pf_score_select(q, pool, n_c, k, ids_out=_fake((k,), torch.int32),
                           scores_out=_fake((M - 1,), torch.float32))
    with pytest.raises(TypeError, match="scores_out"):
        pf.pf_score_select(q, pool, n_c, k, ids_out=_fake((k,), torch.int32), scores_out=_fake((M,), torch.int32))
    with pytest.raises(TypeError, match="ids_out"):
        pf.pf_select_place(q, pool, n_c, k, tags, 48, 4, ids_out=torch.zeros(k, dtype=torch.int32))
    with pytest.raises(ValueError, match="deltas_out"):
        pf.pf_select_place(q, pool, n_c, k, tags, 48, 4, ids_out=_fake((k,), torch.int32),
                           deltas_out=_fake((k - 1,), torch.int32))
    with pytest.raises(ValueError, match="pos_tags"):
        pf.pf_select_place(q, pool, n_c, k, _fake((M,), torch.int32, "cuda:1"), 48, 4)
    qb = _fake((3, n, H, 128))
    pb = _fake((3, M * n_c, H, 128))
    with pytest.raises(ValueError, match="ids_out"):
        pf.pf_score_select_batched(qb, pb, n_c, k, ids_out=_fake((3, k - 1), torch.int32))
    with pytest.raises(ValueError, match="deltas_out"):
        pf.pf_selection_deltas(_fake((k,), torch.int32), tags, 48, 4, deltas_out=_fake((k - 1,), torch.int32))


def test_bench_calls_only_bound_functions(pf):
    # every binding function bench.py calls exists (a missing one fails the
    # GPU run only after minutes of work)
    src = open(os.path.join(ROOT, "bench.py")).read()
    for name in sorted(set(re.findall(r"pf\.(pf_[a-z_0-9]+)", src))):
        assert hasattr(pf, name), name
