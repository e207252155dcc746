"""Host-side checks of the C ABI (no GPU work is launched): the library loads, exports
every function include/sparse_attn.h declares, sizes and counts agree with their
definitions, and invalid arguments are rejected before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def sa():
    import dynamic_block_sparse_mean_amd as m

    if not os.path.exists(m.library_path):
        pytest.fail("libsparse_attn.so is not built (python -m dynamic_block_sparse_mean_amd.build)")
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(sa_\w+|sparse_attn_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_method_calls():
    names = declared_functions()
    for required in ("sparse_attn_plan", "sparse_attn_forward", "sparse_attn_pool", "sparse_attn_select",
                     "sparse_attn_prepare", "sparse_attn_attend", "sparse_attn_debug_qk_tile"):
        assert required in names


def test_library_exports_every_declared_symbol(sa):
    lib = ctypes.CDLL(sa.library_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_n_keep_matches_oracle(sa):
    for nK in (1, 3, 16, 64, 512, 591, 1182, 1920, 4096):
        for keep in (1e-9, 0.01, 0.05, 0.1, 0.15, 0.2, 0.25, 0.3, 1 / 3, 0.5, 0.7, 0.999, 1.0):
            assert sa.n_keep(nK, keep) == oracle.n_keep(nK, keep), (nK, keep)
    for bad in (0.0, -1.0, 1.0001, float("nan")):
        with pytest.raises(ValueError):
            sa.n_keep(10, bad)


def test_num_blocks(sa):
    assert sa.num_blocks(75600, 128) == 591 and sa.num_blocks(75600, 64) == 1182
    assert sa.num_blocks(32760, 128) == 256 and sa.num_blocks(32760, 64) == 512
    assert sa.num_blocks(1, 64) == 1 and sa.num_blocks(0, 64) == -1


def test_forward_layout_sizes(sa):
    B, H, L = 1, 40, 75600
    lay = sa.forward_layout(B, H, L, 128, 128, 64, "int8fp8")
    nQ, nK = 591, 1182
    assert (lay["nQ"], lay["nK"]) == (nQ, nK)
    assert lay["k_off"] - lay["q_off"] >= B * H * nQ * 128 * 128
    assert lay["v_off"] - lay["k_off"] >= B * H * nK * 64 * 128
    assert lay["sq_off"] - lay["v_off"] >= B * H * nK * 64 * 128
    assert lay["total"] >= lay["sv_off"] + 4 * B * H * nK
    for k in ("q_off", "k_off", "v_off", "sq_off", "sk_off", "sv_off"):
        assert lay[k] % 256 == 0
    bf = sa.forward_layout(B, H, L, 128, 128, 64, "bf16")
    assert bf["k_off"] - bf["q_off"] >= B * H * nQ * 128 * 128 * 2  # the prologue's bf16 Q
    assert bf["v_off"] - bf["k_off"] >= B * H * nK * 64 * 128 * 2
    assert bf["sq_off"] - bf["v_off"] >= B * H * nK * 64 * 128 * 2 and bf["total"] >= bf["sq_off"] + 4
    assert sa.forward_workspace_bytes(B, H, L, 128, 128, 64, "int8fp8") == lay["total"]
    # plan workspace: fp64 means + fp64 score matrix
    assert sa.plan_workspace_bytes(B, H, L, 128, 128, 64) >= 8 * B * H * (nQ * 128 + nK * 128 + nQ * nK)


def _tensor(sa, B=1, H=2, L=256, D=128, dtype=1, ptr=0x1000, strides=None):
    sb, sh, sl = strides or (H * L * D, L * D, D)
    return sa.SaTensor(ptr, dtype, 0, B, H, L, D, sb, sh, sl)


def _plan_call(sa, q, k, bq=64, bk=64, keep=0.25, nk=None, ws_bytes=1 << 30, plan_ptr=0x2000):
    L = q.L
    nK = -(-L // bk)
    nk = sa.n_keep(nK, keep) if nk is None else nk
    return sa.lib().sparse_attn_plan(ctypes.byref(q), ctypes.byref(k), bq, bk, keep, plan_ptr, nk,
                                     0x3000, ws_bytes, None)


def test_plan_rejects_bad_arguments_without_launching(sa):
    E = {"inv": -1, "uns": -2, "ws": -3, "shape": -4}
    ok_q, ok_k = _tensor(sa), _tensor(sa)
    assert _plan_call(sa, _tensor(sa, D=64), ok_k) == E["uns"]
    assert _plan_call(sa, ok_q, _tensor(sa, L=300)) == E["shape"]
    assert _plan_call(sa, ok_q, ok_k, bq=96) == E["uns"]
    assert _plan_call(sa, ok_q, ok_k, bk=32) == E["uns"]
    assert _plan_call(sa, ok_q, ok_k, keep=1.5, nk=1) == E["inv"]
    assert _plan_call(sa, ok_q, ok_k, nk=3) == E["shape"]  # keep 0.25 of 4 blocks is 1
    assert _plan_call(sa, ok_q, ok_k, ws_bytes=16) == E["ws"]
    assert _plan_call(sa, _tensor(sa, ptr=0), ok_k) == E["inv"]
    assert _plan_call(sa, _tensor(sa, ptr=0x1008), ok_k) == E["uns"]  # not 16-byte aligned
    assert _plan_call(sa, _tensor(sa, strides=(1, 1, 64)), ok_k) == E["uns"]  # rows overlap
    assert _plan_call(sa, _tensor(sa, dtype=7), ok_k) == E["uns"]
    assert _plan_call(sa, ok_q, ok_k, plan_ptr=0) == E["inv"]
    msg = sa.lib().sa_last_error().decode()
    assert "plan_idx" in msg
    # empty inputs: a size of zero is an invalid argument, rejected before any launch
    for empty in ({"L": 0}, {"B": 0}, {"H": 0}):
        assert _plan_call(sa, _tensor(sa, **empty), _tensor(sa, **empty), nk=1) == E["inv"]
        assert "positive" in sa.lib().sa_last_error().decode()
    # beyond one launch: B*H above 65535 (grid z of the score kernel), or B*H*(nQ + 2 nK)
    # workgroups above 2^24 - 1 (the quantization pass's 256-thread grid)
    for big in ({"B": 70000, "H": 1}, {"B": 2, "H": 40000}, {"B": 1 << 40, "H": 1 << 40},
                {"B": 1, "H": 4096, "L": 524288}):
        assert _plan_call(sa, _tensor(sa, **big), _tensor(sa, **big), bq=128, bk=128, keep=0.1) == E["uns"]
        assert "too large for one launch" in sa.lib().sa_last_error().decode()
    assert sa.plan_workspace_bytes(1, 1024, 524288, 128, 128, 128) > 0  # 1024 * 12288 fits


def test_forward_rejects_bad_arguments_without_launching(sa):
    lib = sa.lib()
    q, k, v = _tensor(sa, ptr=0x1000), _tensor(sa, ptr=0x2000), _tensor(sa, ptr=0x3000)
    out = _tensor(sa, ptr=0x4000)

    def call(q=q, k=k, v=v, out=out, nk=2, mode=1, ws=1 << 30, bq=64, bk=64, plan=0x5000):
        return lib.sparse_attn_forward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), plan, bq, bk,
                                       nk, mode, 0.0, ctypes.byref(out), 0x6000, ws, None)

    assert call(nk=0) == -1
    assert call(nk=5) == -1  # only 4 key blocks
    assert call(mode=9) == -2
    assert call(ws=100) == -3
    assert call(out=_tensor(sa, ptr=0x1000)) == -1  # aliases q
    assert call(v=_tensor(sa, L=128, ptr=0x3000)) == -4
    assert call(q=_tensor(sa, dtype=0, ptr=0x1000)) == -2  # fp32 not accepted by forward
    assert call(plan=0) == -1
    for empty in ({"L": 0}, {"B": 0}, {"H": 0}):  # empty inputs
        assert call(q=_tensor(sa, ptr=0x1000, **empty), k=_tensor(sa, ptr=0x2000, **empty),
                    v=_tensor(sa, ptr=0x3000, **empty), out=_tensor(sa, ptr=0x4000, **empty), nk=1) == -1
    big = {"B": 1, "H": 70000}  # beyond one launch
    assert call(q=_tensor(sa, ptr=0x1000, **big), k=_tensor(sa, ptr=0x2000, **big),
                v=_tensor(sa, ptr=0x3000, **big), out=_tensor(sa, ptr=0x4000, **big), nk=1) == -2
    with pytest.raises(RuntimeError, match="too large for one launch"):
        sa.forward_workspace_bytes(1, 70000, 256, 128, 64, 64)


def test_plan_prepare_rejects_bad_arguments_without_launching(sa):
    lib = sa.lib()
    q, k, v = _tensor(sa, ptr=0x1000), _tensor(sa, ptr=0x2000), _tensor(sa, ptr=0x3000)

    def call(q=q, k=k, v=v, keep=0.25, nk=1, mode=1, pws=1 << 30, fws=1 << 30, bq=64, bk=64, plan=0x5000):
        return lib.sparse_attn_plan_prepare(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), bq, bk, keep,
                                            mode, plan, nk, 0x6000, pws, 0x7000, fws, None)

    assert call(nk=2) == -4  # keep 0.25 of 4 blocks is 1
    assert call(keep=0.0) == -1
    assert call(mode=9) == -2
    assert call(pws=16) == -3
    assert call(fws=100) == -3
    assert call(v=_tensor(sa, L=128, ptr=0x3000)) == -4
    assert call(q=_tensor(sa, dtype=0, ptr=0x1000), k=_tensor(sa, dtype=0, ptr=0x2000)) == -2  # fp32
    assert call(bk=32) == -2
    assert call(plan=0) == -1
    for empty in ({"L": 0}, {"B": 0}, {"H": 0}):  # empty inputs
        assert call(q=_tensor(sa, ptr=0x1000, **empty), k=_tensor(sa, ptr=0x2000, **empty),
                    v=_tensor(sa, ptr=0x3000, **empty)) == -1


def test_debug_tile_calls_reject_bad_arguments_without_launching(sa):
    lib = sa.lib()
    B, H, L, D, bq, bk = 1, 2, 1024, 128, 64, 64
    ws_bytes = {m: sa.forward_workspace_bytes(B, H, L, D, bq, bk, m) for m in ("int8fp8", "fp8")}
    for fn, mode in ((lib.sparse_attn_debug_qk_tile, "int8fp8"), (lib.sparse_attn_debug_qk_tile_fp8, "fp8")):
        ok = dict(ws=0x10000, wsb=ws_bytes[mode], plan=0x2000, nk=4, b=0, h=0, i=0, t=0, out=0x3000, D=D, bq=bq)
        def call(**kw):
            a = dict(ok, **kw)
            return fn(a["ws"], a["wsb"], B, H, L, a["D"], a["bq"], bk, a["plan"], a["nk"], a["b"], a["h"],
                      a["i"], a["t"], a["out"], None)
        assert call(wsb=16) == -3
        assert call(out=0) == -1 and call(plan=0) == -1
        assert call(t=4) == -1 and call(h=2) == -1 and call(i=16) == -1 and call(b=-1) == -1
        assert call(D=64) == -2 and call(bq=96) == -2


def test_plan_noalloc_rejects_bad_arguments_and_large_shapes_without_launching(sa):
    lib = sa.lib()
    E = {"inv": -1, "uns": -2, "ws": -3, "shape": -4}
    assert lib.sa_plan_noalloc_max_bytes() == 64 << 20
    def call(q, k, bq=64, bk=64, keep=0.25, nk=None, plan_ptr=0x2000):
        nK = -(-q.L // bk)
        nk = sa.n_keep(nK, keep) if nk is None else nk
        return lib.sparse_attn_plan_noalloc(ctypes.byref(q), ctypes.byref(k), bq, bk, keep, plan_ptr, nk, None)
    ok_q, ok_k = _tensor(sa), _tensor(sa)
    assert call(_tensor(sa, D=64), ok_k) == E["uns"]
    assert call(ok_q, _tensor(sa, L=300)) == E["shape"]
    assert call(ok_q, ok_k, bq=96) == E["uns"]
    assert call(ok_q, ok_k, nk=3) == E["shape"]
    assert call(ok_q, ok_k, plan_ptr=0) == E["inv"]
    assert call(_tensor(sa, ptr=0), ok_k) == E["inv"]
    # 480p with 40 heads needs 73 MiB of scratch: refused with the limit named, before any launch
    big = dict(B=1, H=40, L=32760)
    assert sa.plan_workspace_bytes(1, 40, 32760, 128, 128, 64) > 64 << 20
    assert call(_tensor(sa, **big), _tensor(sa, **big), bq=128, bk=64, keep=0.2) == E["ws"]
    assert "noalloc" in lib.sa_last_error().decode() and str(64 << 20) in lib.sa_last_error().decode()
    # one GPU's 5-head share of the 720p shape fits
    assert sa.plan_workspace_bytes(1, 5, 75600, 128, 128, 64) <= 64 << 20


def test_ulysses_payload_sizes(sa):
    # 720p over 8 peers, Q, K, V: Lmax = 9450 tokens, 5 heads per group, 3 tensors, 129 bytes a row
    chunk, total = sa.ulysses_payload_bytes(1, 5, 75600, 8, 3)
    rows = 9450 * 5 * 3
    assert chunk == -(-rows * 129 // 256) * 256 and total == 8 * chunk
    chunk, total = sa.ulysses_payload_bytes(2, 1, 10, 4, 1)  # Lmax = 3, the last shard holds 1 token
    assert chunk == 1024 and total == 4096  # 2 * 3 rows of 129 bytes, rounded up to 256
    with pytest.raises(RuntimeError):
        sa.ulysses_payload_bytes(1, 1, 10, 8, 1)  # Lmax = 2: 7 * 2 >= 10 leaves the last peer empty
    with pytest.raises(RuntimeError):
        sa.ulysses_payload_bytes(1, 1, 100, 8, 4)  # at most 3 tensors


def test_ulysses_calls_reject_bad_arguments_without_launching(sa):
    lib = sa.lib()
    L, P = 1000, 4  # shards of 250 tokens
    seq = (sa.SaTensor * 3)(*[_tensor(sa, H=8, L=250, ptr=0x1000 * (i + 1)) for i in range(3)])
    heads = (sa.SaTensor * 3)(*[_tensor(sa, H=2, L=L, ptr=0x10000 * (i + 1)) for i in range(3)])
    _, need = sa.ulysses_payload_bytes(1, 2, L, P, 3)

    def pack_seq(x=seq, n=3, L=L, P=P, rank=1, h0=0, hc=2, pay=0x100000, nbytes=need):
        return lib.sa_ulysses_pack_seq(x, n, L, P, rank, h0, hc, pay, nbytes, None)

    def unpack_seq(y=seq, n=3, L=L, P=P, rank=1, h0=0, hc=2, pay=0x100000, nbytes=need):
        return lib.sa_ulysses_unpack_seq(pay, nbytes, L, P, rank, h0, hc, y, n, None)

    for call in (pack_seq, unpack_seq):
        assert call(nbytes=need - 1) == -3
        assert call(pay=0) == -1
        assert call(pay=0x100008) == -2  # not 16-byte aligned
        assert call(rank=4) == -1
        assert call(L=1001) == -4  # shard 1 of 1001 tokens over 4 peers holds 251
        assert call(h0=1, hc=2) == -1  # the chunk runs past a group of 2 heads
        assert call(hc=0) == -1
        assert call(n=4) == -1
        assert call(P=3) == -2  # 8 heads do not split into 3 groups
        bad = (sa.SaTensor * 3)(seq[0], _tensor(sa, H=8, L=249, ptr=0x2000), seq[2])
        assert call(bad) == -4
    # head side: the payload size follows from the tensors
    assert lib.sa_ulysses_pack_head(heads, 3, P, 0x100000, need - 1, None) == -3
    assert lib.sa_ulysses_unpack_head(0x100000, need - 1, P, heads, 3, None) == -3
    assert lib.sa_ulysses_unpack_head(0, need, P, heads, 3, None) == -1
    fp32 = (sa.SaTensor * 1)(_tensor(sa, H=2, L=L, dtype=0))
    assert lib.sa_ulysses_pack_head(fp32, 1, P, 0x100000, need, None) == -2


def test_prologue_rejects_bad_arguments_without_launching(sa):
    lib = sa.lib()
    q, k, v = _tensor(sa, ptr=0x1000), _tensor(sa, ptr=0x2000), _tensor(sa, ptr=0x3000)  # L = 256
    big = 1 << 30

    def call(mode=1, eps=1e-6, theta=1e4, grid=(4, 8, 8), qg=0x8000, kg=0x9000, pws=big, q=q):
        pro = sa.SaQkPrologue(qg, kg, eps, *grid, theta)
        return lib.sparse_attn_plan_prepare_prologue(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 64, 64,
                                                     0.25, mode, ctypes.byref(pro), 0x5000, 1, 0x6000, pws,
                                                     0x7000, big, None)

    assert call(mode=0, eps=0.0) == -1 and call(mode=0, grid=(4, 8, 9)) == -4  # bf16 mode: same checks
    assert call(mode=3) == -2  # no such mode
    assert call(eps=0.0) == -1 and call(eps=float("nan")) == -1
    assert call(theta=1.0) == -1
    assert call(grid=(4, 8, 9)) == -4  # 288 tokens, L = 256
    assert call(grid=(0, 8, 8)) == -1
    assert call(qg=0) == -1 and call(kg=0) == -1
    assert call(qg=0x8004) == -2  # not 16-byte aligned
    need = sa.plan_prologue_workspace_bytes(1, 2, 256, 128, 64, 64, (4, 8, 8))
    plain = sa.plan_workspace_bytes(1, 2, 256, 128, 64, 64)
    assert need == plain + 3584  # (4*22 + 8*21 + 8*21) pairs x 8 bytes = 3392, rounded up to 256
    assert call(pws=plain + 3391) == -3  # one byte short of the table itself
    assert lib.sparse_attn_plan_prepare_prologue(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 64, 64,
                                                 0.25, 1, None, 0x5000, 1, 0x6000, big, 0x7000, big, None) == -1


def test_nvfp4_calls_reject_bad_arguments_without_launching(sa):
    lib = sa.lib()
    nbytes = ctypes.c_size_t(0)
    assert lib.sa_nvfp4_quantize_workspace_bytes(4, 64, ctypes.byref(nbytes)) == 0 and nbytes.value == 4096
    assert lib.sa_nvfp4_quantize_workspace_bytes(0, 64, ctypes.byref(nbytes)) == -1

    def quant(x=0x1000, rows=4, K=64, ld=64, codes=0x2000, scales=0x3000, S=0x4000, ws=0x5000, wsb=4096):
        return lib.sa_nvfp4_quantize(x, rows, K, ld, codes, scales, S, ws, wsb, None)

    assert quant(rows=0) == -1 and "positive" in lib.sa_last_error().decode()
    assert quant(x=0) == -1
    assert quant(K=32, ld=32) == -2  # blocks of 16 are read four at a time
    assert quant(ld=56) == -2 and quant(ld=68) == -2  # ld below K, ld not a multiple of 8
    assert quant(x=0x1008) == -2 and quant(scales=0x3002) == -2  # alignment
    assert quant(wsb=4092) == -3 and quant(ws=0) == -3

    def gemm(M=256, N=256, K=256, ldy=256, y=0x7000, bias=0x8000, a=0x1000):
        return lib.sa_nvfp4_gemm(a, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, bias, y, M, N, K, ldy, None)

    assert gemm(M=0) == -1 and gemm(a=0) == -1
    assert gemm(K=128) == -2 and "multiple of 256" in lib.sa_last_error().decode()
    assert gemm(N=252, ldy=252) == -2  # N a multiple of 8
    assert gemm(ldy=252) == -2 and gemm(ldy=258) == -2  # ldy below N, not a multiple of 4
    assert gemm(y=0x7004) == -2 and gemm(bias=0x8001) == -2  # alignment
    assert gemm(M=1 << 22, K=1 << 12, ldy=256) == -2 and "4 GiB" in lib.sa_last_error().decode()


def test_status_strings(sa):
    lib = sa.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.sa_status_string(code).decode() != "unknown status"
    assert lib.sa_status_string(-99).decode() == "unknown status"


def test_python_binding_has_no_cpu_path(sa, monkeypatch):
    # Without the library every call must raise instead of computing something else.
    import dynamic_block_sparse_mean_amd as m

    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "library_path", "/nonexistent/libsparse_attn.so")
    with pytest.raises(RuntimeError):
        m.n_keep(10, 0.5)


def test_synthetic_generator_is_seeded_and_shaped():
    from synth import CONFIGS, make_qkv

    cfg = CONFIGS["tiny"]
    q1, k1, v1 = make_qkv(cfg)
    q2, k2, v2 = make_qkv(cfg)
    assert q1.shape == (1, 2, 1024, 128) and q1.dtype == np.float32
    assert np.array_equal(q1, q2) and np.array_equal(v1, v2)
    # a head drawn alone equals the same head drawn with the others
    qh, _, _ = make_qkv(cfg, heads=[1])
    assert np.array_equal(qh[0, 0], q1[0, 1])
    # Q and K share their smooth part: strongly correlated, V is independent noise
    c = np.corrcoef(q1[0, 0].ravel(), k1[0, 0].ravel())[0, 1]
    assert c > 0.8
    assert abs(v1.mean()) < 0.02 and abs(v1.std() - 1) < 0.02
    assert {c.L for c in CONFIGS.values()} == {1024, 32760, 75600, 122880}
