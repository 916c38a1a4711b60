"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, answers host-only queries, rejects bad arguments before any
launch, and links no device allocator."""

import ctypes
import os
import subprocess

import pytest

import paged_kv_split_attn_amd as pkv

LIB = pkv.library_path()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libpkv.so is not built (python -m paged_kv_split_attn_amd.build)")
    return pkv.load_library()


# Bytes of a workgroup's merge record: its first and last segment with the
# workgroups each spans (8 words), then the segment of each wave's two slots.
REC = 32 + 8 * pkv.WAVES_PER_GROUP


def test_header_declares_expected_entry_points():
    names = pkv.declared_functions()
    assert set(names) == {
        "pkv_status_str", "pkv_version", "pkv_workspace_bytes", "pkv_build_metadata",
        "pkv_append_kv", "pkv_append_kv_ragged", "pkv_decode", "pkv_decode_append", "pkv_decode_plan",
        "pkv_decode_masked",
        "pkv_decode_tokens", "pkv_prefill", "pkv_decode_scratch", "pkv_debug_validate", "pkv_debug_read_ceiling"}


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in pkv.declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_no_device_allocation_linked():
    out = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    undefined = {ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()}
    for bad in ("hipMalloc", "hipFree", "hipMallocAsync", "hipFreeAsync", "hipMallocManaged",
                "hipHostMalloc", "hipExtMallocWithFlags", "hipMallocPitch"):
        assert bad not in undefined, bad


def test_status_strings_and_version(lib):
    assert pkv.pkv_status_str(pkv.PKV_OK) == "ok"
    for st in range(1, 7):
        assert pkv.pkv_status_str(st) not in ("ok", "unknown status")
    assert pkv.pkv_status_str(99) == "unknown status"
    assert pkv.pkv_version() >> 16 == 2 and pkv.pkv_version() & 0xffff >= 6


def _desc(**kw):
    base = dict(max_batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                num_workgroups=256, min_tiles_per_group=0)
    base.update(kw)
    return pkv.Desc(**base)


def test_workspace_bytes(lib):
    d = _desc()
    n = pkv.pkv_workspace_bytes(d)
    groups, hg, segs = 256, 4, 16 * 8
    expect = 256  # header
    for sz in (32 * groups * pkv.WAVES_PER_GROUP, REC * groups, 4 * segs, 4 * 2 * groups * hg,
               4 * 2 * groups * hg * 128):
        expect += (sz + 255) // 256 * 256
    assert n == expect
    assert pkv.pkv_workspace_bytes(_desc(num_workgroups=16)) < n
    for bad in (dict(num_q_heads=30), dict(max_batch=0), dict(num_workgroups=-1),
                dict(num_workgroups=70000), dict(min_tiles_per_group=-1)):
        with pytest.raises(pkv.PkvError):
            pkv.pkv_workspace_bytes(_desc(**bad))


def _raw(lib, name, *args):
    return getattr(lib, name)(*args)


def test_host_checks_reject_before_launch(lib):
    d = _desc().c()
    pool = pkv._CPool(100, 16, 8, 128, 0x1000, 0x2000)
    ws_bytes = pkv.pkv_workspace_bytes(_desc())
    fake = 0x10000  # never dereferenced: every call below fails a host check first
    B = ctypes.byref
    # null pointers
    assert _raw(lib, "pkv_build_metadata", B(d), None, 4, 0, fake, fake, ws_bytes, None) == 1
    assert _raw(lib, "pkv_decode", B(pool), B(d), None, fake, fake, 10, fake, 4, 0.1, fake,
                ws_bytes, fake, None) == 1
    # batch above capacity
    assert _raw(lib, "pkv_build_metadata", B(d), fake, 17, 0, fake, fake, ws_bytes, None) == 4
    # workspace too small
    assert _raw(lib, "pkv_build_metadata", B(d), fake, 4, 0, fake, fake, ws_bytes - 1, None) == 3
    assert _raw(lib, "pkv_decode", B(pool), B(d), fake, fake, fake, 10, fake, 4, 0.1, fake,
                ws_bytes - 1, fake, None) == 3
    # negative forced workgroup count
    assert _raw(lib, "pkv_build_metadata", B(d), fake, 4, -1, fake, fake, ws_bytes, None) == 1
    # unsupported head_dim / page_size (every group size G is supported)
    for bad in (dict(head_dim=96), dict(page_size=12), dict(page_size=24)):
        db = _desc(**bad)
        assert _raw(lib, "pkv_build_metadata", B(db.c()), fake, 4, 0, fake, fake, 1 << 30,
                    None) == 2
    # pool that disagrees with the descriptor
    pool_bad = pkv._CPool(100, 16, 4, 128, 0x1000, 0x2000)
    assert _raw(lib, "pkv_decode", B(pool_bad), B(d), fake, fake, fake, 10, fake, 4, 0.1, fake,
                ws_bytes, fake, None) == 1
    # fused append without its rows
    assert _raw(lib, "pkv_decode_append", B(pool), B(d), fake, None, fake, fake, fake, 10, fake, 4,
                0.1, fake, ws_bytes, fake, None) == 1
    # masked decode: no mask, or a stride that is not a multiple of 4
    assert _raw(lib, "pkv_decode_masked", B(pool), B(d), fake, None, 16, fake, fake, 10, fake, 4,
                0.1, fake, ws_bytes, fake, None) == 1
    assert _raw(lib, "pkv_decode_masked", B(pool), B(d), fake, fake, 18, fake, fake, 10, fake, 4,
                0.1, fake, ws_bytes, fake, None) == 1
    # prefill: null query offsets, negative max_q_len, batch above capacity
    assert _raw(lib, "pkv_prefill", B(pool), B(d), fake, None, fake, fake, 10, fake, 4, 8, 1, 0.1,
                fake, None) == 1
    assert _raw(lib, "pkv_prefill", B(pool), B(d), fake, fake, fake, fake, 10, fake, 4, -1, 1, 0.1,
                fake, None) == 1
    assert _raw(lib, "pkv_prefill", B(pool), B(d), fake, fake, fake, fake, 10, fake, 17, 8, 1, 0.1,
                fake, None) == 4
    # token-major decode: page size other than 16, no slots, a contiguous layout
    # larger than the caches, a table of 2^31 entries or more, a small workspace
    d32 = _desc(page_size=32).c()
    assert _raw(lib, "pkv_decode_tokens", B(d32), fake, fake, 100, fake, 8, fake, fake, fake, 4,
                0.1, fake, ws_bytes, fake, None) == 1
    assert _raw(lib, "pkv_decode_tokens", B(d), fake, fake, 0, fake, 8, fake, fake, fake, 4, 0.1,
                fake, ws_bytes, fake, None) == 1
    assert _raw(lib, "pkv_decode_tokens", B(d), fake, fake, 31, None, 8, fake, fake, fake, 4, 0.1,
                fake, ws_bytes, fake, None) == 1
    assert _raw(lib, "pkv_decode_tokens", B(d), fake, fake, 100, fake, 1 << 30, fake, fake, fake,
                4, 0.1, fake, ws_bytes, fake, None) == 4
    assert _raw(lib, "pkv_decode_tokens", B(d), fake, fake, 100, fake, 8, fake, fake, fake, 4, 0.1,
                fake, 16, fake, None) == 3
    # read-ceiling probe: size not a multiple of 16, sink too small
    assert _raw(lib, "pkv_debug_read_ceiling", fake, 100, fake, 1 << 20, None) == 1
    assert _raw(lib, "pkv_debug_read_ceiling", fake, 1 << 20, fake, 1000, None) == 1
    # NaN scale
    assert _raw(lib, "pkv_decode", B(pool), B(d), fake, fake, fake, 10, fake, 4, float("nan"),
                fake, ws_bytes, fake, None) == 1
    # append with a head_dim that is not a multiple of 8 channels
    pool_odd = pkv._CPool(100, 16, 8, 60, 0x1000, 0x2000)
    assert _raw(lib, "pkv_append_kv", B(pool_odd), fake, fake, fake, fake, 10, fake, 4, None) == 2
    # static-scratch decode: a descriptor whose workspace exceeds the scratch,
    # and null arguments, are refused before anything is looked up or launched
    big = _desc(num_workgroups=65536).c()
    assert pkv.pkv_workspace_bytes(_desc(num_workgroups=65536)) > pkv.SCRATCH_BYTES
    assert _raw(lib, "pkv_decode_scratch", B(pool), B(big), fake, fake, fake, 10, 4, 0.1, fake,
                fake, None) == pkv.PKV_ERR_SCRATCH_TOO_SMALL
    assert _raw(lib, "pkv_decode_scratch", B(pool), B(d), None, fake, fake, 10, 4, 0.1, fake,
                fake, None) == 1
    assert _raw(lib, "pkv_decode_scratch", B(pool), B(d), fake, fake, fake, 10, 17, 0.1, fake,
                fake, None) == 4
    assert pkv.pkv_status_str(pkv.PKV_ERR_SCRATCH_TOO_SMALL).startswith("the descriptor needs")
    # planning decode: no lengths, no kv_indptr, one of k_new / v_new, a
    # negative forced count, batch above capacity, a small workspace
    args = lambda **kw: [B(pool), B(d), kw.get("q", fake), kw.get("kn", fake), kw.get("vn", fake),
                         kw.get("sl", fake), kw.get("b", 4), kw.get("f", 0), kw.get("ip", fake),
                         fake, 10, 0.1, fake, kw.get("ws", ws_bytes), fake, None]
    assert _raw(lib, "pkv_decode_plan", *args(sl=None)) == 1
    assert _raw(lib, "pkv_decode_plan", *args(ip=None)) == 1
    assert _raw(lib, "pkv_decode_plan", *args(vn=None)) == 1
    assert _raw(lib, "pkv_decode_plan", *args(f=-1)) == 1
    assert _raw(lib, "pkv_decode_plan", *args(b=17)) == 4
    assert _raw(lib, "pkv_decode_plan", *args(ws=ws_bytes - 1)) == 3
    assert _raw(lib, "pkv_decode_plan", *args(q=None)) == 1
    # extend append: no query offsets, negative row bound, odd head_dim, a grid
    # of 2^31 workgroups or more
    assert _raw(lib, "pkv_append_kv_ragged", B(pool), fake, fake, None, fake, fake, 10, fake, 4,
                8, None) == 1
    assert _raw(lib, "pkv_append_kv_ragged", B(pool), fake, fake, fake, fake, fake, 10, fake, 4,
                -1, None) == 1
    assert _raw(lib, "pkv_append_kv_ragged", B(pool_odd), fake, fake, fake, fake, fake, 10, fake,
                4, 8, None) == 2
    assert _raw(lib, "pkv_append_kv_ragged", B(pool), fake, fake, fake, fake, fake, 10, fake,
                65536, 1 << 20, None) == 4


def test_binding_requires_gpu_tensors(lib):
    import torch
    d = _desc()
    with pytest.raises(ValueError):
        pkv.pkv_build_metadata(d, torch.zeros(4, dtype=torch.int32), 0,
                               torch.zeros(5, dtype=torch.int32), torch.zeros(10, dtype=torch.uint8))


def test_missing_library_fails_loudly(tmp_path):
    # no fallback: every entry point needs the HIP library and says so when it is absent
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import paged_kv_split_attn_amd as p\n"
            "try:\n"
            "    p.pkv_version()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    env = dict(os.environ, PKV_LIBRARY=str(tmp_path / "absent" / "libpkv.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised: libpkv.so not found" in r.stdout


def test_header_wave_count_matches_library(lib):
    # the workspace holds one 32-byte range per wave and one merge record per workgroup
    one = pkv.pkv_workspace_bytes(_desc(num_workgroups=1024))
    two = pkv.pkv_workspace_bytes(_desc(num_workgroups=2048))
    per_group = 32 * pkv.WAVES_PER_GROUP + REC + 4 * 2 * 4 * (1 + 128)
    assert two - one == 1024 * per_group
