"""The C ABI without a device: exports, error codes, refcounts (CPU only)."""
from __future__ import annotations

import ctypes
import re
import subprocess

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from position_independent_kv_legolink_amd import binding
from tests.conftest import ROOT

HEADER = f"{ROOT}/include/piclink.h"


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:pic_status|const char \*)\s*(pic_[a-z_]+)\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 16
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (pic_[a-z_]+)$", out, re.M))
    assert set(names) <= exported, set(names) - exported
    L = pic.lib()
    for n in names:
        assert hasattr(L, n)
    assert sorted(binding.EXPORTS) == names


def meta(**over):
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, num_pages=64, dtype="bf16",
              rope_theta=5e5, max_position=4096, device=None)
    kw.update(over)
    return pic.Store(**kw)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(page_size=8), dict(num_q_heads=6),
                                 dict(num_q_heads=32, num_kv_heads=2), dict(num_pages=0), dict(rope_theta=0.0),
                                 dict(max_position=0), dict(max_position=(1 << 22) + 1)])
def test_store_config_validation(bad):
    with pytest.raises(pic.PicError) as e:
        meta(**bad)
    assert e.value.status == -1


def test_store_accepts_the_largest_max_position():
    meta(max_position=1 << 22).close()


def test_key_layout_is_validated():
    """The binding names the two key forms; the C ABI rejects any other value."""
    meta(key_layout="segment_rope").close()
    with pytest.raises(ValueError):
        meta(key_layout="rotated")
    cfg = pic.binding.StoreConfig(8, 2, 128, 16, 64, 0, 5e5, 4096, 2)
    h = ctypes.c_void_p()
    assert pic.lib().pic_store_create(ctypes.byref(cfg), None, None, None, None, ctypes.byref(h)) == -1
    assert b"key_layout" in pic.lib().pic_last_error()


def test_plans_of_both_key_layouts_are_identical():
    """The key form changes only how keys are rotated, not the plan."""
    ex = []
    for layout in ("position_free", "segment_rope"):
        st = meta(key_layout=layout)
        for c in range(3):
            st.store_chunk(c, None, None, n_tokens=50)
        plan = st.link_plan([pic.LinkRequest(chunk_ids=[2, 0, 1], suffix_len=9)], k=5)
        ex.append(plan.export())
        plan.free()
        st.close()
    for key in ex[0]:
        assert np.array_equal(ex[0][key], ex[1][key]), key


def test_store_and_plan_errors():
    s = meta()
    s.store_chunk(1, n_tokens=40)               # 3 pages
    with pytest.raises(pic.PicError) as e:
        s.store_chunk(1, n_tokens=5)
    assert e.value.status == -4                 # exists
    with pytest.raises(pic.PicError) as e:
        s.store_chunk(2, n_tokens=0)
    assert e.value.status == -1
    with pytest.raises(pic.PicError) as e:
        s.store_chunk(3, n_tokens=16 * 62)       # 62 pages > 61 free
    assert e.value.status == -2
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([7], 4)], k=2)
    assert e.value.status == -3                 # unknown chunk
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([1], 4)], k=-1)
    assert e.value.status == -1
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([1], 4)], k=2, pos_offset=4096 - 40)   # beyond the RoPE table
    assert e.value.status == -1
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([1] * 62, 0)], k=16)   # one private page per chunk: 62 > 61 free
    assert e.value.status == -2
    assert s.stats() == dict(free_pages=61, chunks=1, plans=0)   # a failed plan takes nothing


def test_refcounts_keep_pages_of_released_chunks_alive():
    s = meta()
    s.store_chunk(1, n_tokens=40)
    s.store_chunk(2, n_tokens=16)
    free0 = s.stats()["free_pages"]
    plan = s.link_plan([pic.LinkRequest([1, 2], 5)], k=2)
    # private: first page of each chunk + 1 suffix page
    assert s.stats()["free_pages"] == free0 - 3
    s.release(1)
    assert s.stats()["free_pages"] == free0 - 3          # still referenced by the plan
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([1], 5)], k=2)
    assert e.value.status == -3
    with pytest.raises(pic.PicError) as e:
        s.close()
    assert e.value.status == -7                          # live plan
    plan.free()
    assert s.stats()["free_pages"] == free0 + 3          # chunk 1's pages came back too
    s.release(2)
    assert s.stats() == dict(free_pages=64, chunks=0, plans=0)
    s.close()


def test_device_calls_on_metadata_store_fail_cleanly():
    s = meta()
    s.store_chunk(1, n_tokens=40)
    plan = s.link_plan([pic.LinkRequest([1], 5)], k=2)
    L = pic.lib()
    st = L.pic_plan_upload(s.handle, plan.handle, None, 0, None)
    assert st == -7
    st = L.pic_link_attend(s.handle, plan.handle, None, None, None, None, None, None, 0, None)
    assert st == -7
    assert b"metadata-only" in L.pic_last_error()
    plan.free()


def test_null_arguments_are_rejected():
    L = pic.lib()
    assert L.pic_store_create(None, None, None, None, None, None) == -1
    assert L.pic_store_stats(None, None, None, None) == -1
    assert L.pic_plan_info(None, None) == -1
    assert L.pic_store_destroy(None) == 0


def test_plan_sizes_report_workspace():
    s = meta()
    s.store_chunk(1, n_tokens=512)
    plan = s.link_plan([pic.LinkRequest([1], 64)], k=2)
    z = plan.sizes
    assert z["rows"] == 66 and z["pages"] == 36 and z["private_pages"] == 5 and z["cow_pages"] == 1
    assert z["workspace_bytes"] % 256 == 0 and z["workspace_bytes"] >= 36 * 16
    plan.free()


def test_workspace_breakdown_adds_up():
    """table_bytes + max(partial_bytes + rotated_key_bytes, decode_partial_bytes) (+ 256-byte
    alignment) = workspace_bytes: the link call's scratch and decode's partials share one region,
    except when the keys are rotated ahead (decode then reads them and its partials follow).
    The rotated keys are one page of keys per logical page, the link partials one float32 row per
    split slot, the decode partials one per decode item and query head."""
    s = meta(num_pages=400)
    for c in range(6):
        s.store_chunk(c, n_tokens=300)
    req = [pic.LinkRequest(list(range(6)), 40)]
    page_bytes = 2 * 16 * 128 * 2          # Hkv 2, page 16, d 128, bf16
    for kw in (dict(rope_keys=1), dict(rope_keys=2), dict(rope_keys=1, split_pages=4), dict(decode=3),
               dict(decode=3, rope_keys=2), dict(decode=3, rope_keys=1, split_pages=4)):
        plan = s.link_plan(req, k=3, **kw)
        z = plan.sizes
        link = z["partial_bytes"] + z["rotated_key_bytes"]
        if z["rotated_pages"]:   # decode reads the rotated keys: its partials follow them
            parts = z["table_bytes"] + link + z["decode_partial_bytes"]
        else:
            parts = z["table_bytes"] + max(link, z["decode_partial_bytes"])
        assert parts <= z["workspace_bytes"] <= parts + 8 * 256, (kw, z)
        assert z["rotated_key_bytes"] >= z["rotated_pages"] * page_bytes
        assert z["rotated_key_bytes"] < z["rotated_pages"] * page_bytes + 256
        assert (z["partial_bytes"] > 0) == (z["split_items"] > 0), (kw, z)
        if kw.get("decode"):
            # 1 request, 2 KV heads, G = 4 query heads: d floats and one lse per head and item
            assert z["decode_items"] > 0
            assert z["decode_partial_bytes"] >= z["decode_items"] * 4 * (128 + 1) * 4
        else:
            assert z["decode_items"] == 0 and z["decode_partial_bytes"] == 0
        plan.free()


def test_rope_keys_option_is_validated():
    s = meta()
    s.store_chunk(1, n_tokens=40)
    for bad in (-1, 3):
        with pytest.raises(pic.PicError) as e:
            s.link_plan([pic.LinkRequest([1], 5)], k=2, rope_keys=bad)
        assert e.value.status == -1
    s.close()
    f = meta(dtype="f32", head_dim=64)
    f.store_chunk(1, n_tokens=40)
    with pytest.raises(pic.PicError) as e:
        f.link_plan([pic.LinkRequest([1], 5)], k=2, rope_keys=2)   # bf16 stores only
    assert e.value.status == -1
    for rk in (0, 1):
        plan = f.link_plan([pic.LinkRequest([1], 5)], k=2, rope_keys=rk)
        assert plan.sizes["rotated_pages"] == 0
        plan.free()
    assert f.stats()["plans"] == 0


def test_rotated_keys_take_one_page_per_logical_page_of_workspace():
    """rope_keys=2 adds the rotated keys of every logical page (Hkv x page x d bf16 each) to the
    workspace; rope_keys=1 adds nothing; a plan without rows rotates nothing."""
    s = meta()
    s.store_chunk(1, n_tokens=512)
    fused = s.link_plan([pic.LinkRequest([1], 64)], k=2, rope_keys=1)
    rot = s.link_plan([pic.LinkRequest([1], 64)], k=2, rope_keys=2)
    assert fused.sizes["rotated_pages"] == 0
    assert rot.sizes["rotated_pages"] == rot.sizes["pages"] == 36
    page_bytes = 2 * 16 * 128 * 2
    assert rot.sizes["workspace_bytes"] - fused.sizes["workspace_bytes"] == 36 * page_bytes
    empty = s.link_plan([pic.LinkRequest([1], 0)], k=0, rope_keys=2)
    assert empty.sizes["rows"] == 0 and empty.sizes["rotated_pages"] == 0
    for p in (fused, rot, empty):
        p.free()


def test_decode_option_is_validated():
    """decode=1 builds one decode item per (request, KV head) range and rotates nothing ahead for
    decode (the decode kernel rotates the keys it reads), with either rope_keys mode of the link
    call; it needs a bf16 store and a RoPE table row for the new token's position."""
    s = meta()
    s.store_chunk(1, n_tokens=40)
    plan = s.link_plan([pic.LinkRequest([1], 5)], k=2, decode=True)
    assert plan.sizes["decode_items"] == 2            # 1 request x 2 KV heads, 4 pages each
    assert plan.sizes["pages"] == 4
    plain = s.link_plan([pic.LinkRequest([1], 5)], k=2)
    assert plain.sizes["decode_items"] == 0
    # the same link choice as without decode
    assert plan.sizes["rotated_pages"] == plain.sizes["rotated_pages"]
    plan.free()
    plain.free()
    for rk in (1, 2):
        p = s.link_plan([pic.LinkRequest([1], 5)], k=2, decode=True, rope_keys=rk)
        assert p.sizes["decode_items"] == 2
        assert p.sizes["rotated_pages"] == (4 if rk == 2 else 0)
        p.free()
    # the request ends at position 4095 = the last table row: linking is fine, the decode token
    # at 4096 has no row
    s.link_plan([pic.LinkRequest([1], 5)], k=2, pos_offset=4096 - 45).free()
    with pytest.raises(pic.PicError) as e:
        s.link_plan([pic.LinkRequest([1], 5)], k=2, pos_offset=4096 - 45, decode=True)
    assert e.value.status == -1
    assert s.stats()["plans"] == 0
    s.close()
    f = meta(dtype="f32", head_dim=64)
    f.store_chunk(1, n_tokens=40)
    with pytest.raises(pic.PicError) as e:
        f.link_plan([pic.LinkRequest([1], 5)], k=2, decode=True)
    assert e.value.status == -1


def _usage_consistent(s):
    u = s.usage()
    assert u["pages_free"] + u["pages_chunks"] + u["pages_plans_only"] == u["pages_total"]
    assert u["pages_free"] == s.stats()["free_pages"] and u["chunks"] == s.stats()["chunks"]
    return u


def test_evict_releases_least_recently_used_chunks():
    """Chunks age by ingest and by the plans that link them; eviction frees the oldest first."""
    s = meta(num_pages=6)
    for cid in (1, 2, 3):
        s.store_chunk(cid, n_tokens=32)              # 2 pages each: the pool is full
    assert _usage_consistent(s)["pages_chunks"] == 6
    s.link_plan([pic.LinkRequest([1], 0)], k=0).free()   # chunk 1 is now the most recent
    assert s.evict(2) == 1                           # chunk 2: ingested before 3, never linked since
    with pytest.raises(pic.PicError) as e:
        s.chunk_pages(2)
    assert e.value.status == -3
    assert s.evict(2) == 0                           # already 2 free pages
    assert s.evict(4) == 1                           # then chunk 3
    u = _usage_consistent(s)
    assert u["chunks"] == 1 and u["evictions"] == 2 and u["pages_free"] == 4
    s.close()


def test_evict_skips_chunks_that_live_plans_hold():
    """A chunk whose pages a live plan holds frees nothing when released, so eviction passes it
    by; a target that only such chunks could meet fails without evicting anything."""
    s = meta(num_pages=8)
    for cid in (1, 2, 3):
        s.store_chunk(cid, n_tokens=32)
    plan = s.link_plan([pic.LinkRequest([1], 0)], k=0)   # holds chunk 1's pages; touches it last
    with pytest.raises(pic.PicError) as e:
        s.evict(8)                                   # 2 free + 4 of chunks 2 and 3 < 8
    assert e.value.status == -2
    assert s.stats()["chunks"] == 3 and s.usage()["evictions"] == 0
    assert s.evict(6) == 2                           # chunks 2 and 3; chunk 1 stays
    assert s.stats()["chunks"] == 1
    plan.free()
    assert s.evict(8) == 1
    assert _usage_consistent(s)["pages_free"] == 8
    with pytest.raises(pic.PicError) as e:
        s.evict(9)
    assert e.value.status == -1
    s.close()


def test_usage_counts_pages_held_only_by_plans():
    """Private pages, and the pages of a chunk released while a plan uses it, are held by plans
    only; they return to the pool with the plan."""
    s = meta(num_pages=16)
    s.store_chunk(1, n_tokens=40)                    # 3 pages
    plan = s.link_plan([pic.LinkRequest([1], 20)], k=2)   # private: chunk page 0 (copy-on-write) + 2 suffix pages
    u = _usage_consistent(s)
    assert u["pages_chunks"] == 3 and u["pages_plans_only"] == 3 and u["plans"] == 1
    s.release(1)
    u = _usage_consistent(s)
    assert u["pages_chunks"] == 0 and u["pages_plans_only"] == 6
    plan.free()
    assert _usage_consistent(s)["pages_free"] == 16
    s.close()


def test_compile_offset_is_validated():
    """A store's compile offset (keys compiled after leading tokens) must lie in [0, 4096] and below
    max_position, and no segment may reach past the RoPE table once it is added."""
    for bad in (-1, 4097):
        with pytest.raises(pic.PicError):
            meta(key_layout="segment_rope", compile_offset=bad)
    with pytest.raises(pic.PicError):
        meta(key_layout="segment_rope", compile_offset=4, max_position=4)
    s = meta(key_layout="segment_rope", compile_offset=70, max_position=130)
    s.store_chunk(1, n_tokens=64)
    s.store_chunk(2, n_tokens=60)
    with pytest.raises(pic.PicError):          # 70 + 64 > 130: the scatter would pass the table
        s.link_plan([pic.LinkRequest([1], 0)], k=2)
    plan = s.link_plan([pic.LinkRequest([2], 0)], k=2)   # 70 + 60 = 130 fits
    plan.free()
    # no effect on position-free stores beyond validation
    p = meta(compile_offset=4)
    p.store_chunk(1, n_tokens=64)
    p.link_plan([pic.LinkRequest([1], 10)], k=2).free()
