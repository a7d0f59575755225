"""The C ABI without a GPU: header, exports, argument checks, status text.

Calls here pass invalid arguments (rejected on the host before any HIP call)
or run only where no GPU is present (then valid calls return KVS_ENODEV)."""
import ctypes
import os
import re
import subprocess

import pytest

import kv_cache_eviction_lse_amd as kvs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvscore.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvs.LIB_PATH):
        from kv_cache_eviction_lse_amd import build

        build.build()
    return kvs.lib()


def _no_gpu():
    try:
        import torch

        return torch.cuda.device_count() == 0
    except Exception:
        return True


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kv[a-z_]+)\s*\(", src)))


@pytest.mark.parametrize("std,cc", [("c99", "gcc"), ("c++17", "g++")])
def test_header_compiles(tmp_path, std, cc):
    src = tmp_path / ("t.c" if cc == "gcc" else "t.cpp")
    src.write_text('#include "kvscore.h"\nint main(void){ kvs_attn_desc d; kvs_evict_desc e; (void)d; (void)e;'
                   ' return (int)sizeof(d) + (int)sizeof(e) > 0 ? 0 : 1; }\n')
    subprocess.run([cc, f"-std={std}", "-Wall", "-Werror", "-pedantic", "-I", os.path.dirname(HEADER),
                    "-fsyntax-only", str(src)], check=True)


def test_exports_match_header(L):
    declared = _declared_functions()
    assert set(declared) == set(kvs.EXPORTED_SYMBOLS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", kvs.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared), exported ^ set(declared)


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvscore.h"\nint main(void){'
                   'printf("%zu %zu %zu %zu\\n", sizeof(kvs_attn_desc), offsetof(kvs_attn_desc, scale),'
                   ' sizeof(kvs_evict_desc), offsetof(kvs_evict_desc, score_head_stride)); return 0; }\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()))
    want = [ctypes.sizeof(kvs.AttnDesc), kvs.AttnDesc.scale.offset, ctypes.sizeof(kvs.EvictDesc),
            kvs.EvictDesc.score_head_stride.offset]
    assert got == want


def test_strerror_covers_codes(L):
    texts = [L.kvs_strerror(c).decode() for c in range(7)]
    assert len(set(texts)) == 7 and "unknown" not in " ".join(texts)
    assert L.kvs_strerror(99).decode() == "unknown status"
    assert L.kvs_version() >= 100


FAKE = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced: rejected or no device


def _desc(**kw):
    d = kvs.AttnDesc()
    d.n_qheads, d.n_kvheads, d.head_dim, d.mask = 4, 2, 128, kvs.MASK_REPEAT
    d.n_ctx, d.n_q, d.chunk = 64, 32, 32
    d.q_head_stride, d.q_tok_stride = 32 * 128, 128
    d.k_head_stride, d.k_tok_stride = 64 * 128, 128
    d.ks_head_stride, d.ks_tok_stride = 32 * 128, 128
    d.scale, d.reserved = 0.088, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


ATTN_BAD = [
    (dict(n_qheads=5), kvs.KVS_EINVAL),
    (dict(n_kvheads=0), kvs.KVS_EINVAL),
    (dict(head_dim=96), kvs.KVS_EUNSUPPORTED),
    (dict(mask=7), kvs.KVS_EINVAL),
    (dict(n_q=-1), kvs.KVS_EINVAL),
    (dict(chunk=0), kvs.KVS_EINVAL),
    (dict(scale=0.0), kvs.KVS_EINVAL),
    (dict(scale=float("nan")), kvs.KVS_EINVAL),
    (dict(q_tok_stride=100), kvs.KVS_EUNSUPPORTED),
    (dict(k_tok_stride=64), kvs.KVS_EINVAL),
    (dict(k_tok_stride=(1 << 22) + 8), kvs.KVS_EUNSUPPORTED),  # tile offsets are 32-bit
    (dict(reserved=1), kvs.KVS_EINVAL),
    (dict(mask=kvs.MASK_CAUSAL), kvs.KVS_EINVAL),  # CAUSAL needs n_q == n_ctx
    (dict(n_ctx=1 << 31), kvs.KVS_EUNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", ATTN_BAD)
def test_lse_rejects(L, kw, code):
    d = _desc(**kw)
    assert L.kvscore_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == code
    assert L.kvs_last_error().decode()


def test_null_and_misaligned_pointers(L):
    d = _desc()
    assert L.kvscore_lse(None, FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_lse(ctypes.byref(d), None, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_lse(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == kvs.KVS_EINVAL  # Kself for REPEAT
    assert L.kvscore_lse(ctypes.byref(d), FAKE, FAKE, FAKE, None, None) == kvs.KVS_EINVAL
    assert L.kvscore_lse(ctypes.byref(d), ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, None) == kvs.KVS_EUNSUPPORTED


@pytest.mark.parametrize("kw,code", ATTN_BAD)
def test_attention_rejects_bad_desc(L, kw, code):
    d = _desc(**kw)
    assert L.kvscore_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code


def test_attention_rejects_pointers(L):
    d = _desc()
    A = L.kvscore_attention
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL  # V
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == kvs.KVS_EINVAL  # Vself (REPEAT)
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == kvs.KVS_EINVAL  # O
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == kvs.KVS_EINVAL  # lse
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x100008), FAKE,
             None) == kvs.KVS_EUNSUPPORTED
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), FAKE, FAKE, FAKE,
             None) == kvs.KVS_EUNSUPPORTED


def _vdesc(**kw):
    d = kvs.VnormDesc()
    d.n_kvheads, d.head_dim, d.n_tok, d.d_model, d.reserved = 2, 128, 100, 512, 0
    d.v_head_stride, d.v_tok_stride, d.wo_row_stride = 100 * 128, 128, 256
    for k, v in kw.items():
        setattr(d, k, v)
    return d


VNORM_BAD = [
    (dict(reserved=3), kvs.KVS_EINVAL),
    (dict(n_kvheads=0), kvs.KVS_EINVAL),
    (dict(head_dim=80), kvs.KVS_EUNSUPPORTED),
    (dict(n_tok=-1), kvs.KVS_EINVAL),
    (dict(d_model=-5), kvs.KVS_EINVAL),
    (dict(v_tok_stride=64), kvs.KVS_EINVAL),
    (dict(v_tok_stride=132), kvs.KVS_EUNSUPPORTED),
    (dict(wo_row_stride=248), kvs.KVS_EINVAL),
    (dict(wo_row_stride=(1 << 22) + 8), kvs.KVS_EUNSUPPORTED),
    (dict(n_tok=(1 << 30) + 1), kvs.KVS_EUNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", VNORM_BAD)
def test_vnorm_rejects(L, kw, code):
    d = _vdesc(**kw)
    assert L.kvscore_vnorm(ctypes.byref(d), FAKE, FAKE, FAKE, None) == code


def test_vnorm_rejects_pointers(L):
    d = _vdesc()
    assert L.kvscore_vnorm(None, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_vnorm(ctypes.byref(d), None, FAKE, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_vnorm(ctypes.byref(d), FAKE, None, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_vnorm(ctypes.byref(d), FAKE, FAKE, None, None) == kvs.KVS_EINVAL
    assert L.kvscore_vnorm(ctypes.byref(d), FAKE, ctypes.c_void_p(0x100008), FAKE, None) == kvs.KVS_EUNSUPPORTED


def _ddesc(**kw):
    d = kvs.DecodeDesc()
    d.n_qheads, d.n_kvheads, d.head_dim, d.n_q = 8, 2, 128, 1
    d.q_head_stride, d.q_tok_stride, d.capacity = 128, 128, 1000
    d.scale, d.reserved = 0.088, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


DECODE_BAD = [
    (dict(reserved=1), kvs.KVS_EINVAL),
    (dict(n_qheads=7), kvs.KVS_EINVAL),
    (dict(head_dim=96), kvs.KVS_EUNSUPPORTED),
    (dict(n_q=0), kvs.KVS_EINVAL),
    (dict(capacity=-1), kvs.KVS_EINVAL),
    (dict(scale=float("inf")), kvs.KVS_EINVAL),
    (dict(q_head_stride=100), kvs.KVS_EUNSUPPORTED),
    (dict(n_q=2, q_tok_stride=64), kvs.KVS_EINVAL),
    (dict(head_stride_rows=-1), kvs.KVS_EINVAL),
    (dict(head_stride_rows=501), kvs.KVS_EINVAL),  # 2 heads x 501 rows > capacity 1000
]


@pytest.mark.parametrize("kw,code", DECODE_BAD)
def test_decode_rejects(L, kw, code):
    d = _ddesc(**kw)
    assert L.kvscore_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == code
    assert L.kvscore_decode_workspace_bytes(ctypes.byref(d)) == 0


def test_decode_workspace_and_pointers(L):
    d = _ddesc()
    need = L.kvscore_decode_workspace_bytes(ctypes.byref(d))
    # chunks of 32 rows under 98,304 rows of cache, 64 under 196,608, else 128
    # (with 4 or 8 queries per wave alike):
    # (capacity // rows + heads) chunks x queries per KV head x (4 + 128) floats
    assert need == (1000 // 32 + 2) * 4 * 132 * 4
    for cap, rows in ((8192, 32), (98303, 32), (98304, 64), (196607, 64), (196608, 128), (244110, 128)):
        assert L.kvscore_decode_workspace_bytes(ctypes.byref(_ddesc(capacity=cap))) == (cap // rows + 2) * 4 * 132 * 4
    for cap, rows in ((65536, 32), (98304, 64), (241024, 128)):  # G = 5: 8 queries per wave
        d5 = _ddesc(capacity=cap, n_qheads=10)
        assert L.kvscore_decode_workspace_bytes(ctypes.byref(d5)) == (cap // rows + 2) * 5 * 132 * 4
    D = L.kvscore_decode
    assert D(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == kvs.KVS_EWORKSPACE
    assert D(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == kvs.KVS_EWORKSPACE
    assert D(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == kvs.KVS_EINVAL
    assert D(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None) == kvs.KVS_EINVAL
    assert D(ctypes.byref(d), ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
             None) == kvs.KVS_EUNSUPPORTED


def test_decode_head_stride_workspace(L):
    """Per-head regions of S rows with live counts: the workspace bound is the
    offsets form's (every region's chunks fit in capacity / 128 + heads)."""
    d = _ddesc(head_stride_rows=500)
    assert L.kvscore_decode_workspace_bytes(ctypes.byref(d)) == (1000 // 32 + 2) * 4 * 132 * 4


def _sdesc(**kw):
    d = kvs.StreamDesc()
    d.n_kvheads, d.head_dim, d.n_seen, d.n_new, d.window = 2, 128, 100, 3, 16
    d.tau, d.reserved, d.capacity = 0.5, 0, 200
    d.new_head_stride, d.new_tok_stride, d.score_head_stride = 3 * 128, 128, 3
    for k, v in kw.items():
        setattr(d, k, v)
    return d


STREAM_BAD = [
    (dict(reserved=1), kvs.KVS_EINVAL),
    (dict(n_kvheads=0), kvs.KVS_EINVAL),
    (dict(head_dim=96), kvs.KVS_EUNSUPPORTED),
    (dict(n_seen=-1), kvs.KVS_EINVAL),
    (dict(n_new=-1), kvs.KVS_EINVAL),
    (dict(window=-1), kvs.KVS_EINVAL),
    (dict(capacity=102), kvs.KVS_ECAPACITY),            # 103 tokens could all be kept
    (dict(n_seen=0, n_new=1, window=300, capacity=299), kvs.KVS_ECAPACITY),  # the window ring needs 300 rows
    (dict(n_seen=1 << 30, capacity=(1 << 30) + 8), kvs.KVS_EUNSUPPORTED),
    (dict(new_tok_stride=100), kvs.KVS_EUNSUPPORTED),
    (dict(new_tok_stride=64), kvs.KVS_EINVAL),
    (dict(score_head_stride=2), kvs.KVS_EINVAL),
    (dict(new_head_stride=-8), kvs.KVS_EINVAL),
]


@pytest.mark.parametrize("kw,code", STREAM_BAD)
def test_stream_rejects(L, kw, code):
    d = _sdesc(**kw)
    assert L.kv_stream_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code


def test_stream_pointers(L):
    d = _sdesc()
    A = L.kv_stream_append
    assert A(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == kvs.KVS_EINVAL
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == kvs.KVS_EINVAL
    assert A(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, FAKE,
             None) == kvs.KVS_EUNSUPPORTED
    assert A(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_EINVAL


def test_max_and_futuremass_reject(L):
    d = _desc()
    assert L.kvscore_max(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, 2, None) == kvs.KVS_EINVAL
    assert L.kvscore_max(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, 0, None) == kvs.KVS_EINVAL
    dc = _desc(mask=kvs.MASK_CAUSAL, n_q=64, q_head_stride=64 * 128)
    assert L.kvscore_max(ctypes.byref(dc), FAKE, FAKE, FAKE, None, None, FAKE, 0, None) == kvs.KVS_EINVAL
    assert L.kvscore_futuremass(ctypes.byref(d), FAKE, FAKE, FAKE, 0, None, None, FAKE, None) == kvs.KVS_EINVAL
    assert L.kvscore_futuremass(ctypes.byref(dc), FAKE, FAKE, FAKE, -1, None, None, FAKE, None) == kvs.KVS_EINVAL


def _edesc(**kw):
    e = kvs.EvictDesc()
    e.n_kvheads, e.head_dim, e.n_tok, e.k, e.tau, e.scope = 2, 128, 1000, 100, 0.0, kvs.SCOPE_HEAD
    e.window, e.capacity = 32, 2 * 132
    e.kv_head_stride, e.kv_tok_stride, e.score_head_stride = 1000 * 128, 128, 1000
    for k, v in kw.items():
        setattr(e, k, v)
    return e


EVICT_BAD = [
    (dict(n_kvheads=0), kvs.KVS_EINVAL),
    (dict(head_dim=80), kvs.KVS_EUNSUPPORTED),
    (dict(n_tok=-5), kvs.KVS_EINVAL),
    (dict(window=-1), kvs.KVS_EINVAL),
    (dict(capacity=2 * 131), kvs.KVS_ECAPACITY),
    (dict(k=-1, capacity=1999), kvs.KVS_ECAPACITY),  # threshold mode needs Hkv * n
    (dict(kv_tok_stride=132), kvs.KVS_EUNSUPPORTED),
    (dict(kv_tok_stride=120), kvs.KVS_EINVAL),
    (dict(score_head_stride=999), kvs.KVS_EINVAL),
    (dict(scope=3), kvs.KVS_EINVAL),
    # layer budget: 2 windows of 32 + min(100, 2 * 968) = 164 rows
    (dict(scope=kvs.SCOPE_LAYER, capacity=163), kvs.KVS_ECAPACITY),
    (dict(scope=kvs.SCOPE_LAYER, n_kvheads=4096, n_tok=1 << 20, kv_head_stride=(1 << 20) * 128,
          score_head_stride=1 << 20, capacity=1 << 40), kvs.KVS_EUNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", EVICT_BAD)
def test_evict_rejects(L, kw, code):
    e = _edesc(**kw)
    ws = L.kv_evict_workspace_bytes(ctypes.byref(_edesc()))
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == code


def test_evict_workspace_checks(L):
    e = _edesc()
    ws = L.kv_evict_workspace_bytes(ctypes.byref(e))
    assert ws > 0 and ws % 256 == 0
    assert L.kv_evict_workspace_bytes(ctypes.byref(_edesc(n_kvheads=0))) == 0
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, None) == kvs.KVS_EWORKSPACE
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == kvs.KVS_EWORKSPACE
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x100010), ws,
                      None) == kvs.KVS_EWORKSPACE
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == kvs.KVS_EINVAL


def test_evict_noalloc_rejects(L):
    """Host checks of kv_evict_noalloc: kv_evict's argument checks, and the
    layer's workspace must fit the built-in scratch (KVS_EWORKSPACE)."""
    for kw, code in EVICT_BAD:
        e = _edesc(**kw)
        assert L.kv_evict_noalloc(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code, kw
    e = _edesc()
    assert L.kv_evict_noalloc(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == kvs.KVS_EINVAL
    # (threshold mode takes the grid path, whose histograms need 24 KiB per head)
    big = _edesc(n_kvheads=300, k=-1, capacity=300 * 1000, kv_head_stride=1000 * 128)
    assert L.kv_evict_workspace_bytes(ctypes.byref(big)) > kvs.EVICT_NOALLOC_MAX_WORKSPACE
    assert L.kv_evict_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_EWORKSPACE
    assert "scratch" in L.kvs_last_error().decode()


def test_noalloc_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define KVS_EVICT_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kvs.EVICT_NOALLOC_MAX_WORKSPACE


@pytest.mark.skipif(not _no_gpu(), reason="valid calls would launch on a GPU host")
def test_valid_calls_without_gpu_return_enodev(L):
    d = _desc()
    assert L.kvscore_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_ENODEV
    assert L.kvscore_max(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, 0, None) == kvs.KVS_ENODEV
    dc = _desc(mask=kvs.MASK_CAUSAL, n_q=64, q_head_stride=64 * 128)
    assert L.kvscore_futuremass(ctypes.byref(dc), FAKE, FAKE, FAKE, 8, None, None, FAKE, None) == kvs.KVS_ENODEV
    e = _edesc()
    ws = L.kv_evict_workspace_bytes(ctypes.byref(e))
    assert L.kv_evict(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == kvs.KVS_ENODEV
    assert L.kv_evict_noalloc(ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvs.KVS_ENODEV
    assert L.kv_stream_append(ctypes.byref(_sdesc()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              None) == kvs.KVS_ENODEV
    assert "device" in L.kvs_last_error().decode()


def test_binding_requires_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvs, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kvs, "_lib", None)
    with pytest.raises(ImportError):
        kvs.lib()


def test_last_error_is_per_thread(L):
    """kvs_last_error keeps each calling thread's own message."""
    import threading

    results = {}

    def worker(name, kw, expect):
        d = _desc(**kw)
        got = []
        for _ in range(200):
            code = L.kvscore_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None)
            got.append((code, L.kvs_last_error().decode()))
        results[name] = (got, expect)

    threads = [threading.Thread(target=worker, args=("dim", dict(head_dim=96), "head_dim 96")),
               threading.Thread(target=worker, args=("mask", dict(mask=7), "unknown mask 7"))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for name, (got, expect) in results.items():
        assert all(expect in msg for _, msg in got), name



# ---------------------------------------------------------------- binding checks
# Shapes the C ABI cannot see (it gets pointers and a descriptor) are checked
# by the Python binding before the device is; these run on host tensors.

def _t(shape, dtype):
    import torch

    return torch.zeros(shape, dtype=dtype)


def test_binding_rejects_scores_of_wrong_shape():
    import torch

    K = _t((2, 100, 128), torch.bfloat16)
    for bad in ((1, 100), (2, 99), (3, 100)):
        with pytest.raises(ValueError, match="scores must be"):
            kvs.evict(_t(bad, torch.float32), K, K, window=8, k=10)


def test_binding_rejects_small_or_mistyped_outputs():
    import torch

    K = _t((2, 100, 128), torch.bfloat16)
    s = _t((2, 100), torch.float32)
    cap = 2 * (8 + 10)
    good = (_t(cap, torch.int32), _t(3, torch.int64), _t((cap, 128), torch.bfloat16), _t((cap, 128), torch.bfloat16))
    bad_sets = {
        "kept_idx": (_t(cap - 1, torch.int32),) + good[1:],
        "head_offsets": (good[0], _t(2, torch.int64)) + good[2:],
        "K_out": good[:2] + (_t((cap - 1, 128), torch.bfloat16), good[3]),
        "V_out": good[:3] + (_t((cap, 64), torch.bfloat16),),
    }
    for name, outs in bad_sets.items():
        with pytest.raises(ValueError, match=name):
            kvs.evict(s, K, K, window=8, k=10, outputs=outs)
    with pytest.raises(ValueError, match="kept_idx"):
        kvs.evict(s, K, K, window=8, k=10, outputs=(_t(cap, torch.int64),) + good[1:])
    # right shapes on the host: the device check is what fails
    with pytest.raises(ValueError, match="GPU tensor"):
        kvs.evict(s, K, K, window=8, k=10, outputs=good)


def test_binding_rejects_self_keys_of_wrong_shape():
    import torch

    Q = _t((8, 64, 128), torch.bfloat16)
    K = _t((2, 300, 128), torch.bfloat16)
    for bad in ((2, 63, 128), (1, 64, 128), (2, 64, 64)):
        with pytest.raises(ValueError, match="Kself must be"):
            kvs.lse(Q, K, _t(bad, torch.bfloat16), scale=0.1, mask="repeat", chunk=64)
        with pytest.raises(ValueError, match="Kself must be"):
            kvs.attention(Q, K, K, _t(bad, torch.bfloat16), _t(bad, torch.bfloat16), scale=0.1, mask="repeat",
                          chunk=64)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvs.lse(Q, K, _t((2, 64, 128), torch.bfloat16), scale=0.1, mask="repeat", chunk=64)
