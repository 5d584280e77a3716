"""The C ABI: the built library exports every call the header declares, and
host-side validation rejects bad scalars before anything is launched.  These
run without a GPU: every call here fails validation (or has an empty batch)
and returns before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "graft.h")

G = pytest.importorskip("tree_attention_verification_graft_amd.binding")
lib = G.lib()
P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(graft_\w+)\s*\(", text, re.M)))


def test_header_declares_the_calls():
    names = header_functions()
    for n in ["graft_build_tree", "graft_tree_attention", "graft_accept",
              "graft_accept_sample", "graft_update_adjacency", "graft_update_adjacency_tree",
              "graft_append_kv", "graft_tree_attention_rope", "graft_append_kv_rope"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in header_functions() if n not in exported]
    assert not missing, missing
    assert sorted(G.EXPORTED) == header_functions()


def _cfg(**kw):
    c = dict(kmax=6, stage_depth=[0, 1, 5], stage_tau=[0.3] * 3, stage_k_ret=[4, 2, 0],
             k_ret_none=0, env_parent=[-1, -1, 0, 0, 1, 1], env_rank=[0, 1, 0, 1, 0, 1])
    c.update(kw)
    return G.make_config(c)


def _build(cfg, batch=1, n_draft_max=8, vocab=10, top_s=2):
    return lib.graft_build_tree(ctypes.byref(cfg), batch, n_draft_max, *([FAKE] * 7), vocab,
                                top_s, *([FAKE] * 6), None)


def test_build_tree_validation():
    assert _build(_cfg(kmax=0)) == -1
    assert _build(_cfg(kmax=200)) == -1
    assert _build(_cfg(stage_k_ret=[7, 2, 0])) == -1          # K_ret > kmax
    assert _build(_cfg(stage_depth=[1, 0, 5])) == -1          # not ascending
    assert _build(_cfg(env_parent=[-1, -1, 0, 3, 1, 1])) == -1  # parent after slot
    assert _build(_cfg(env_rank=[0, 1, 0, 2, 0, 1])) == -1    # rank >= top_s
    assert _build(_cfg(env_parent=[-1, -1, 0], env_rank=[0, 1, 0])) == -1  # env < kmax
    assert _build(_cfg(), n_draft_max=300) == -2
    assert _build(_cfg(), top_s=0) == -1
    assert "top_s" in G.graft_last_error()
    assert _build(_cfg(), batch=0) == 0                       # nothing to do


def _attn(dtype=1, batch=1, n_max=17, hq=4, hkv=1, D=128, block=16, max_blocks=8,
          max_prefix=128, ws=None, ws_bytes=0, scale=0.1, sum_prefix=0):
    return lib.graft_tree_attention(dtype, batch, n_max, hq, hkv, D, *([FAKE] * 5), block,
                                    FAKE, max_blocks, FAKE, max_prefix, sum_prefix, FAKE, FAKE,
                                    ctypes.c_float(scale), FAKE, ws, ws_bytes, None)


def test_attention_validation():
    assert _attn(dtype=7) == -1
    assert _attn(D=96) == -2
    assert _attn(block=32) == -2
    assert _attn(hq=6, hkv=4) == -1
    # per-node and per-page byte offsets of the KV tensors are 32-bit
    assert _attn(hq=65537, hkv=65537) == -2
    assert "hkv 65537 above 65536" in G.graft_last_error()
    assert _attn(n_max=129) == -1
    assert _attn(max_blocks=2) == -1                          # 2*16 < max_prefix
    assert _attn(scale=float("inf")) == -1
    assert _attn(scale=0.0) == -1
    assert _attn(scale=-0.1) == -1
    assert _attn(batch=0) == 0
    # a long prefix needs split partials: no workspace -> workspace error
    need = lib.graft_tree_attention_workspace_size(1, 1, 61, 32, 8, 128, 65536, 0)
    assert need > 0
    # the prefix-length sum only steers the plan; a ragged batch may split
    # more, never needs a workspace when nothing is split
    assert lib.graft_tree_attention_workspace_size(1, 16, 65, 32, 8, 128, 64, 16 * 40) == 0
    assert _attn(n_max=61, hq=32, hkv=8, max_blocks=4096, max_prefix=65536) == -3
    assert "workspace" in G.graft_last_error()


def test_accept_and_update_validation():
    acc = lambda **k: lib.graft_accept(k.get("dt", 1), k.get("b", 1), k.get("n", 17),
                                       k.get("v", 1000), *([FAKE] * 9), k.get("ws", FAKE),
                                       k.get("wsb", 1 << 20), None)
    assert acc(dt=3) == -1
    assert acc(n=200) == -1
    assert acc(v=0) == -1
    assert acc(v=2**31 - 2**16 + 1) == -2  # chunk bounds would leave int32
    assert "vocab above" in G.graft_last_error()
    assert acc(wsb=8) == -3
    assert acc(b=0) == 0
    align = lambda x: -(-x // 256) * 256
    # one packed (value, index) key per (row, vocab chunk); sized for the
    # f32 chunk of 2048 entries, the smaller of the two dtypes' chunks
    assert lib.graft_accept_workspace_size(2, 65, 151936) == align(2 * 65 * 75 * 8)
    upd = lambda **k: lib.graft_update_adjacency(FAKE, FAKE, k.get("v", 100), k.get("s", 8),
                                                 k.get("np", 4), k.get("st", 10), FAKE, FAKE,
                                                 k.get("ws", FAKE), k.get("wsb", 1 << 20),
                                                 None)
    assert upd(s=0) == -1
    assert upd(s=33) == -1
    assert upd(v=0) == -1
    assert upd(wsb=100) == -3
    assert upd(np=0) == 0                                     # no transitions
    small = lib.graft_update_adjacency_workspace_size(4, 10)
    big = lib.graft_update_adjacency_workspace_size(1, 65536)
    assert 0 < small < big


def test_version_string():
    assert "gfx950" in G.graft_version()


def test_append_kv_validation():
    def app(**k):
        return lib.graft_append_kv(k.get("dt", 1), k.get("b", 2), k.get("n", 9), k.get("hkv", 2),
                                   k.get("d", 128), k.get("kt", FAKE), FAKE, FAKE, FAKE,
                                   k.get("nblk", 64), k.get("blk", 16), FAKE, k.get("mb", 8),
                                   k.get("pl", FAKE), FAKE, FAKE, k.get("npl", FAKE), None)
    assert app(dt=7) == -1
    assert app(n=0) == -1
    assert app(n=200) == -1
    assert app(blk=0) == -1
    assert app(kt=None) == -1
    assert app(npl=ctypes.c_void_p(0x2000), pl=ctypes.c_void_p(0x2000)) == -1  # aliasing
    assert "alias" in G.graft_last_error()
    assert app(b=0) == 0


def test_update_tree_validation():
    def upd(**k):
        return lib.graft_update_adjacency_tree(FAKE, FAKE, k.get("v", 100), k.get("s", 8),
                                               k.get("b", 2), k.get("n", 9), FAKE, FAKE, FAKE,
                                               k.get("ws", FAKE), k.get("wsb", 1 << 20), None)
    assert upd(n=0) == -1
    assert upd(n=200) == -1
    assert upd(s=0) == -1
    assert upd(v=0) == -1
    assert upd(wsb=8) == -3
    assert upd(ws=None) == -3
    assert upd(b=0) == 0
    assert lib.graft_update_adjacency_tree_workspace_size(2, 9) >= 2 * 9 * 12


def test_accept_sample_validation():
    def acc(**k):
        return lib.graft_accept_sample(k.get("dt", 1), k.get("b", 2), k.get("n", 17),
                                       k.get("v", 1000), k.get("lg", FAKE),
                                       ctypes.c_float(k.get("t", 0.7)), *([FAKE] * 8),
                                       k.get("ws", FAKE), k.get("wsb", 1 << 20), None)
    assert acc(dt=3) == -1
    assert acc(n=0) == -1
    assert acc(n=129) == -1
    assert acc(v=0) == -1
    assert acc(v=2**31 - 2**16 + 1) == -2  # chunk bounds would leave int32
    assert "vocab above" in G.graft_last_error()
    assert acc(t=0.0) == -1
    assert acc(t=-1.0) == -1
    assert acc(t=float("inf")) == -1
    assert acc(t=float("nan")) == -1
    assert "temperature" in G.graft_last_error()
    assert acc(t=1e-38) == -2             # log2(e) / T beyond float range
    assert acc(lg=None) == -1
    assert acc(wsb=8) == -3
    assert acc(ws=None) == -3
    assert acc(b=0) == 0
    align = lambda x: -(-x // 256) * 256
    # staged mode while the tree's logits take at most 384 MiB and a row has
    # at most 2304 chunks of 4096 bf16 or 2048 f32 entries: a 16-byte (float
    # max, float64 sum) record per (row, chunk); else lazy mode: a 32-byte
    # record per (sequence, chunk) of the root row.  Then a float64 residual
    # mass per (sequence, chunk) and a 544-byte record per sequence.
    def want(dt, B, n, V):
        e, per = (2, 4096) if dt == 1 else (4, 2048)
        ch = -(-V // per)
        lazy = B * n * V * e > 384 << 20 or ch > 2304
        recs = B * ch * 32 if lazy else B * n * ch * 16
        return align(recs) + align(B * ch * 8) + align(B * 544)
    for dt in (1, 0):
        for B, n, V in ((2, 65, 151936), (16, 65, 151936), (32, 65, 151936), (1, 1, 151936),
                        (2, 3, 2304 * 4096), (2, 3, 2304 * 4096 + 1), (1, 2, 1)):
            assert lib.graft_accept_sample_workspace_size(dt, B, n, V) == want(dt, B, n, V)
    # staged at (8, 65, 151936) bf16, lazy at (32, 65, 151936) and past 2304 chunks
    assert want(1, 8, 65, 151936) == align(8 * 65 * 38 * 16) + align(8 * 38 * 8) + align(8 * 544)
    assert want(1, 32, 65, 151936) == align(32 * 38 * 32) + align(32 * 38 * 8) + align(32 * 544)
    assert want(1, 2, 3, 2304 * 4096 + 1) == (align(2 * 2305 * 32) + align(2 * 2305 * 8)
                                              + align(2 * 544))
    assert lib.graft_accept_sample_workspace_size(5, 2, 65, 151936) == 0


def test_rope_variants_validation():
    def att(**k):
        return lib.graft_tree_attention_rope(
            k.get("dt", 1), k.get("b", 1), k.get("n", 17), 32, 8, k.get("d", 128), *([FAKE] * 5),
            16, FAKE, 8, FAKE, 128, 0, FAKE, FAKE, k.get("tp", FAKE), k.get("rope", FAKE),
            k.get("rp", 4096), ctypes.c_float(k.get("scale", 0.088)), FAKE, FAKE, 1 << 24, None)
    assert att(rp=0) == -1
    assert att(tp=None) == -1
    assert att(rope=None) == -1
    assert att(rope=ctypes.c_void_p(0x1004)) == -1        # table not 16-byte aligned
    assert "aligned" in G.graft_last_error()
    assert att(d=96) == -2                                # head_dim outside 64 / 128
    assert att(scale=0.0) == -1
    assert att(b=0) == 0

    def app(**k):
        return lib.graft_append_kv_rope(k.get("dt", 1), k.get("b", 2), 9, 2, k.get("d", 128),
                                        FAKE, FAKE, FAKE, FAKE, 64, 16, FAKE, 8, FAKE, FAKE,
                                        FAKE, ctypes.c_void_p(0x2000), k.get("rope", FAKE),
                                        k.get("rp", 4096), None)
    assert app(d=127) == -1
    assert app(rp=0) == -1
    assert app(rope=None) == -1
    assert app(dt=9) == -1
    assert app(b=0) == 0


def test_attention_plan_query():
    """The plan query is host-only and describes the launch of each
    workload's shapes: the matrix-core kernel for bf16 with head_dim 128 and
    16 or more rows, the wavefront kernel otherwise; the plan tiles every
    prefix tile exactly once; a null plan is rejected."""
    bf = G.GRAFT_BF16
    shapes = {  # (dtype, batch, n_max, hq, hkv, D, max_prefix, sum_prefix)
        "llama3_8b_b1": (bf, 1, 61, 32, 8, 128, 2048, 2048),
        "qwen3_8b_b16": (bf, 16, 65, 32, 8, 128, 4096, 36000),
        "llama31_8b_64k": (bf, 1, 65, 32, 8, 128, 65536, 65536),
        "qwen3_235b_share": (bf, 32, 65, 64, 4, 128, 8192, 32 * 8192),
        "bf16_head_dim_64": (bf, 2, 17, 8, 2, 64, 300, 600),
        "tiny_f32": (G.GRAFT_F32, 1, 17, 4, 1, 64, 128, 128),
    }
    for name, (dt, B, n_max, hq, hkv, D, mp, sp) in shapes.items():
        pl = G.graft_tree_attention_plan(dt, B, n_max, hq, hkv, D, mp, sp)
        rows = n_max * (hq // hkv)
        assert pl["matrix_cores"] == int(dt == bf and D == 128 and rows >= 16), name
        assert pl["n_row_groups"] * pl["rows_per_group"] >= rows, name
        tiles = -(-mp // 64)
        tps, shift = pl["tiles_per_split"], pl["tree_shift"]
        # split s covers prefix tiles [s tps - shift, (s + 1) tps - shift)
        covered = [t for s in range(pl["n_splits"])
                   for t in range(max(0, s * tps - shift), min(tiles, (s + 1) * tps - shift))]
        assert covered == list(range(tiles)), name
        if pl["matrix_cores"]:
            # one item per (sequence, head, row group, split), a multiple of 8,
            # run by at most one workgroup per compute unit
            items = 8 * pl["n_row_groups"] * -(-(B * hkv * pl["n_splits"]) // 8)
            assert pl["workgroups"] == (items if pl["longest_first"] else min(items, 256)), name
        else:
            assert pl["workgroups"] >= B * hkv * pl["n_splits"] * pl["n_row_groups"], name
    assert lib.graft_tree_attention_plan(bf, 1, 17, 8, 2, 128, 100, 0, None) == -1
    assert lib.graft_tree_attention_plan(bf, 1, 17, 8, 3, 128, 100, 0,
                                         ctypes.byref(G.AttentionPlan())) == -1
    assert lib.graft_tree_attention_plan(bf, 1, 17, 65537, 65537, 128, 100, 0,
                                         ctypes.byref(G.AttentionPlan())) == -2


def test_noalloc_rejects_plans_beyond_its_scratch():
    """A plan whose split partials exceed the library's scratch is rejected
    before anything touches the device; the limit is the header's."""
    text = open(HEADER).read()
    assert "#define GRAFT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    bf = G.GRAFT_BF16
    # 8 sequences of 64k tokens with the Qwen3-235B head share (64 / 4):
    # prefix splits of 65 x 16 query rows per KV head
    shape = (bf, 8, 65, 64, 4, 128, 65536, 8 * 65536)
    need = lib.graft_tree_attention_workspace_size(*shape)
    assert need > (64 << 20)
    args = [bf, 8, 65, 64, 4, 128] + [FAKE] * 5 + [16, FAKE, 4100, FAKE, 65536, 8 * 65536,
                                                  FAKE, FAKE, ctypes.c_float(0.1), FAKE, None]
    assert lib.graft_tree_attention_noalloc(*args) == -3
    assert b"scratch" in lib.graft_last_error()
