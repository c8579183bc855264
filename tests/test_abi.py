"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/verify_attn.h, and rejects malformed arguments on the host
with the documented status codes (before any HIP call is made)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_attn.h")


@pytest.fixture(scope="module")
def ops():
    from long_context_verify_tree_amd import ops as o
    if not os.path.exists(o.LIB_PATH):
        pytest.fail("libverify_attn.so is not built (run __graft_entry__.build())")
    o.load()
    return o


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("verify_attn_dense", "verify_attn_sparse", "select_verify_set", "verify_attn_partials",
                 "verify_attn_merge", "va_attn_workspace_size", "va_select_workspace_size", "va_status_str",
                 "va_last_error", "va_version"):
        assert want in names


def test_library_exports_every_declared_symbol(ops):
    lib = ctypes.CDLL(ops.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_single_hip_runtime_in_process(ops):
    maps = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
    assert len(set(maps)) == 1, set(maps)


def test_status_strings(ops):
    lib = ops._lib
    assert lib.va_status_str(0) == b"ok"
    assert b"workspace" in lib.va_status_str(3)
    assert lib.va_version() >= 100


def good_desc(ops, B=2, Hq=8, Hkv=2, D=128, L=1000, N=8, dtype=1):
    d = ops.AttnDesc()
    d.B, d.Hq, d.Hkv, d.D, d.L, d.N, d.dtype, d.scale = B, Hq, Hkv, D, L, N, dtype, 0.0
    d.q_stride = (ctypes.c_int64 * 3)(Hq * N * D, N * D, D)
    d.kc_stride = (ctypes.c_int64 * 3)(Hkv * L * D, L * D, D)
    d.vc_stride = (ctypes.c_int64 * 3)(Hkv * L * D, L * D, D)
    d.kd_stride = (ctypes.c_int64 * 3)(Hkv * N * D, N * D, D)
    d.vd_stride = (ctypes.c_int64 * 3)(Hkv * N * D, N * D, D)
    d.o_stride = (ctypes.c_int64 * 3)(Hq * N * D, N * D, D)
    return d


def ws_size(ops, d, n):
    out = ctypes.c_size_t()
    st = ops._lib.va_attn_workspace_size(ctypes.byref(d) if d is not None else None, n, ctypes.byref(out))
    return st, out.value


def test_workspace_size_and_validation(ops):
    d = good_desc(ops)
    st, n = ws_size(ops, d, d.L)
    assert st == ops.VA_OK and n > 0
    st0, n0 = ws_size(ops, d, 0)
    assert st0 == ops.VA_OK and 0 < n0 < n
    assert ws_size(ops, None, 10)[0] == ops.VA_EINVAL
    assert ws_size(ops, d, d.L + 1)[0] == ops.VA_EINVAL
    for field, val, code in (("Hkv", 3, ops.VA_EINVAL), ("D", 96, ops.VA_EUNSUPPORTED), ("N", 0, ops.VA_EINVAL),
                             ("N", 257, ops.VA_EUNSUPPORTED), ("L", -1, ops.VA_EINVAL), ("B", 0, ops.VA_EINVAL),
                             ("dtype", 7, ops.VA_EINVAL), ("scale", float("nan"), ops.VA_EINVAL)):
        bad = good_desc(ops)
        setattr(bad, field, val)
        assert ws_size(ops, bad, 0)[0] == code, field
        assert ops._lib.va_last_error() != b""
    bad = good_desc(ops)
    bad.kc_stride = (ctypes.c_int64 * 3)(2 * 1000 * 128, 1000 * 128, 100)   # rows not 16-byte aligned
    assert ws_size(ops, bad, 0)[0] == ops.VA_EINVAL
    # keys are addressed with 32-bit byte offsets inside one (sequence, kv head) region
    for attr in ("kc_stride", "vc_stride", "kd_stride", "vd_stride"):
        for key_stride in (0, -128):
            bad = good_desc(ops)
            setattr(bad, attr, (ctypes.c_int64 * 3)(0, 0, key_stride))
            assert ws_size(ops, bad, 0)[0] == ops.VA_EUNSUPPORTED, (attr, key_stride)
    big = good_desc(ops, L=(1 << 23) - 64)         # (L + 64) * 256 B = 2 GiB: the largest accepted region
    assert ws_size(ops, big, 0)[0] == ops.VA_OK
    big = good_desc(ops, L=(1 << 23) - 63)
    assert ws_size(ops, big, 0)[0] == ops.VA_EUNSUPPORTED
    wide = good_desc(ops, L=1 << 20)               # token-major cache: 8 heads x 128 per key -> 2 KiB stride
    wide.kc_stride = (ctypes.c_int64 * 3)(1 << 30, 128, 1024)
    assert ws_size(ops, wide, 0)[0] == ops.VA_EUNSUPPORTED


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every call below fails validation first


def dense(ops, d, ws_bytes, **over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kd=FAKE, vd=FAKE, parent=FAKE, out=FAKE, lse=None, ws=FAKE)
    a.update(over)
    return ops._lib.verify_attn_dense(ctypes.byref(d) if d is not None else None, a["q"], a["kc"], a["vc"], a["kd"],
                                      a["vd"], a["parent"], a["out"], a["lse"], a["ws"], ws_bytes, None)


def test_dense_rejects_before_launch(ops):
    d = good_desc(ops)
    _, need = ws_size(ops, d, d.L)
    assert dense(ops, None, need) == ops.VA_EINVAL
    assert dense(ops, d, need - 1) == ops.VA_EWORKSPACE
    assert dense(ops, d, need, ws=None) == ops.VA_EWORKSPACE
    assert dense(ops, d, need, q=None) == ops.VA_EINVAL
    assert dense(ops, d, need, out=None) == ops.VA_EINVAL
    assert dense(ops, d, need, parent=None) == ops.VA_EINVAL
    assert dense(ops, d, need, kc=None) == ops.VA_EINVAL
    assert dense(ops, d, need, q=ctypes.c_void_p(0x100002)) == ops.VA_EINVAL   # misaligned base
    d.D = 80
    assert dense(ops, d, need) == ops.VA_EUNSUPPORTED


def test_sparse_rejects_before_launch(ops):
    d = good_desc(ops)
    lib = ops._lib

    def sparse(K, stride, idx=FAKE, ws_bytes=1 << 30):
        return lib.verify_attn_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, idx, K, stride, FAKE, None,
                                      FAKE, ws_bytes, None)
    assert sparse(d.L + 1, d.L + 1) == ops.VA_EINVAL
    assert sparse(-1, 10) == ops.VA_EINVAL
    assert sparse(100, 99) == ops.VA_EINVAL
    assert sparse(100, 100, idx=None) == ops.VA_EINVAL
    assert sparse(100, 100, ws_bytes=16) == ops.VA_EWORKSPACE


def test_staged_partials_binding_checks_the_index_list(ops):
    # the binding rejects a malformed verify list before any library call
    # (CPU tensors: nothing reaches a device)
    import torch
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    kc = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16)
    kd = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    parent = torch.zeros(1, 8, dtype=torch.int32)
    desc = ops.make_desc(q, kc, kc, kd, kd, q)
    ws = torch.zeros(16, dtype=torch.uint8)
    for bad in (torch.zeros(1, 10, dtype=torch.int64), torch.zeros(10, dtype=torch.int32),
                torch.zeros(1, 20, dtype=torch.int32)[:, ::2]):
        with pytest.raises(ValueError):
            ops.verify_attn_partials(desc, q, kc, kc, kd, kd, parent, ws, verify_idx=bad)


def select(ops, B, L, ld, sink, window, m, budget, out=FAKE, ds=FAKE, ws=None, ws_bytes=0):
    return ops._lib.select_verify_set(ds, FAKE, B, L, ld, sink, window, m, budget, out, ws, ws_bytes, None)


def test_select_rejects_before_launch(ops):
    assert select(ops, 2, 1000, 999, 4, 16, 10, 100) == ops.VA_EINVAL            # ld < L
    assert select(ops, 2, 1000, 1000, 4, 16, 10, 19) == ops.VA_EINVAL            # budget < sink + window
    assert select(ops, 2, 1000, 1000, -1, 16, 10, 100) == ops.VA_EINVAL
    assert select(ops, 2, 1000, 1000, 4, 16, 10, 100, out=None) == ops.VA_EINVAL
    assert select(ops, 2, 1000, 1000, 4, 16, 10, 100, ds=None) == ops.VA_EINVAL
    longest = 24 * 32768                                                          # longest selector row
    assert select(ops, 1, longest + 1, longest + 1, 4, 16, 10, 100) == ops.VA_EUNSUPPORTED
    assert select(ops, 1, longest + 1, longest + 1, 4, 16, 10, longest + 1, out=None) == ops.VA_EINVAL  # all taken: no limit
    # nothing to do: OK without a launch
    assert select(ops, 0, 1000, 1000, 4, 16, 10, 100) == ops.VA_OK
    assert select(ops, 2, 1000, 1000, 4, 16, 10, 0, out=None) != ops.VA_EHIP
    n = ctypes.c_size_t(99)
    assert ops._lib.va_select_workspace_size(4, 131072, ctypes.byref(n)) == ops.VA_OK


def test_product_path_does_not_touch_the_oracle():
    """The binding and the HIP sources never import or include the oracle."""
    pkg = os.path.join(ROOT, "long_context_verify_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                bad = re.findall(r"^\s*(?:import\s+oracle|from\s+oracle|#\s*include\s*[<\"].*oracle)", text,
                                 flags=re.M)
                assert not bad, (os.path.join(dirpath, f), bad)


def test_commit_rejects_before_launch(ops):
    d = good_desc(ops)
    f = ops._lib.accept_commit
    args = [FAKE] * 8
    assert f(None, *args, None) == ops.VA_EINVAL
    for k in range(8):
        a = list(args)
        a[k] = None
        assert f(ctypes.byref(d), *a, None) == ops.VA_EINVAL, k
    a = list(args)
    a[0] = ctypes.c_void_p(0x100004)   # misaligned cache
    assert f(ctypes.byref(d), *a, None) == ops.VA_EINVAL
    d.D = 96
    assert f(ctypes.byref(d), *args, None) == ops.VA_EUNSUPPORTED


def test_commit_rejects_aliased_lengths(ops):
    # new_len written in place of cache_len, accepted or the parent rows would
    # race with the other KV heads' reads: rejected on the host
    d = good_desc(ops)                      # B = 2, N = 8
    f = ops._lib.accept_commit
    base = 0x200000
    P = lambda off: ctypes.c_void_p(base + off)
    kc, vc, kd, vd = P(0x10000), P(0x20000), P(0x30000), P(0x40000)
    parent, accepted, cache_len = P(0x1000), P(0x2000), P(0x3000)
    ok_new = P(0x4000)
    for new in (cache_len, P(0x3000 + 4), P(0x3000 - 4), accepted, P(0x1000 + 60)):
        assert f(ctypes.byref(d), kc, vc, kd, vd, parent, accepted, cache_len, new, None) == ops.VA_EINVAL
        assert b"overlap" in ops._lib.va_last_error()
    # adjacent but disjoint ranges pass the overlap check; a misaligned cache
    # (checked after it) stops the call before any launch
    bad_kc = P(0x10004)
    for new in (P(0x3000 + 8), P(0x3000 - 8), ok_new):
        assert f(ctypes.byref(d), bad_kc, vc, kd, vd, parent, accepted, cache_len, new, None) == ops.VA_EINVAL
        assert b"aligned" in ops._lib.va_last_error()


def test_tree_rejects_before_launch(ops):
    f = ops._lib.build_draft_tree
    ok_args = (FAKE, FAKE, 2, 4, 3, 10, FAKE, FAKE, FAKE, FAKE, None)
    assert f(*ok_args[:2], 2, 4, 3, 0, *ok_args[6:]) == ops.VA_EINVAL          # N < 1
    assert f(*ok_args[:2], 2, 4, 3, 257, *ok_args[6:]) == ops.VA_EUNSUPPORTED  # N > 256
    assert f(*ok_args[:2], 2, 64, 128, 10, *ok_args[6:]) == ops.VA_EUNSUPPORTED  # K x T > 4096
    assert f(*ok_args[:2], 2, 2, 2, 7, *ok_args[6:]) == ops.VA_EINVAL          # only 2 + 4 prefixes
    assert f(None, *ok_args[1:]) == ops.VA_EINVAL
    assert f(*ok_args[:6], None, *ok_args[7:]) == ops.VA_EINVAL


def test_controller_host_functions_match_the_oracle(ops):
    # host functions of the library: no GPU involved
    from oracle import verify_oracle as vo
    rng = np.random.default_rng(3)
    for shape in (dict(B=8, Hq=32, Hkv=8, D=128, L=32768), dict(B=4, Hq=64, Hkv=8, D=128, L=131072),
                  dict(B=16, Hq=28, Hkv=4, D=128, L=32768), dict(B=1, Hq=4, Hkv=1, D=64, L=256, dtype=0),
                  dict(B=2, Hq=8, Hkv=1, D=64, L=5000, dtype=0)):
        d = good_desc(ops, N=8, **shape)
        e = 4 if shape.get("dtype", 1) == 0 else 2
        for _ in range(40):
            bw, cs, ct, c0 = rng.uniform(1e12, 8e12), rng.uniform(5e14, 2.5e15), rng.uniform(1e14, 1e15), \
                rng.uniform(0, 1e-5)
            n_ctx, N = int(rng.integers(0, shape["L"] + 1)), int(rng.integers(1, 257))
            got = ops.verify_time_model(d, n_ctx, bw, cs, ct, c0, N)
            want = vo.verify_time_plan(shape["B"], shape["Hq"], shape["Hkv"], shape["D"], n_ctx, N, e, bw, cs, ct, c0)
            assert got == pytest.approx(want, rel=1e-12), (shape, n_ctx, N)
            # and the parts of the plans are the library's (its workspace size:
            # slots for the larger of the dense and sparse part counts, then a
            # 256-byte header)
            d.N = N
            _, ws = ws_size(ops, d, n_ctx)
            rows = shape["B"] * shape["Hq"] * N
            parts = max(vo.kernel_plan(shape["B"], shape["Hq"], shape["Hkv"], n_ctx, N, e, sparse=sp)[4]
                        for sp in (False, True))
            assert ws == -(-rows * parts * shape["D"] * 4 // 256) * 256 + -(-rows * parts * 4 // 256) * 256 + 256
            d.N = 8
    for _ in range(50):
        n = int(rng.integers(1, 40))
        a = np.cumsum(rng.random(n) ** 2).astype(np.float32)
        t = np.sort(rng.uniform(1e-4, 3e-4, n))
        t_draft, l_ar = float(rng.uniform(0, 1e-4)), float(rng.uniform(1e-4, 2e-4))
        assert ops.choose_tree_size(a, t, t_draft, l_ar) == vo.choose_tree_size(a, t, t_draft, l_ar)[0]
    with pytest.raises(ops.VerifyAttnError):
        ops.verify_time_model(d, 100, 0.0, 1e15, 1e15, 0.0, 4)
    with pytest.raises(ops.VerifyAttnError):
        ops.choose_tree_size(np.ones(3), np.ones(3), 0.0, 0.0)


def test_error_messages_are_per_thread(ops):
    # two host threads fail different calls, then each reads the message of
    # its own call (the library keeps the last message per thread)
    import threading
    bar = threading.Barrier(2)
    got = {}

    def worker(name, over):
        d = good_desc(ops)
        for k, v in over.items():
            setattr(d, k, v)
        st = ws_size(ops, d, 100)[0]
        bar.wait()   # both calls have failed before either message is read
        got[name] = (st, ops._lib.va_last_error().decode())

    ts = [threading.Thread(target=worker, args=("d", {"D": 96})),
          threading.Thread(target=worker, args=("h", {"Hq": 6, "Hkv": 4}))]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert got["d"][0] == 2 and "D = 96" in got["d"][1]
    assert got["h"][0] == 1 and "multiple of Hkv" in got["h"][1]
