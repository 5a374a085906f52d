"""The C ABI: the library loads, exports every declared symbol, and its
host-side logic (workspace sizes, argument checks) behaves as documented.

Nothing here launches device work: every call either touches no device or
fails its argument checks before anything is enqueued.
"""

import ctypes
import os
import re

import pytest
import torch

import newton_schulz_matrix_amd as nsa
from newton_schulz_matrix_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsortho.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libnsortho.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(ns_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_api():
    names = _declared_functions()
    for want in ["ns_orthogonalize", "ns_orthogonalize_batched",
                 "ns_muon_step", "ns_muon_workspace_size",
                 "ns_soft_threshold_split", "ns_workspace_size",
                 "ns_soft_threshold_workspace_size", "ns_status_string",
                 "ns_options_default", "ns_version", "ns_plan_kernels",
                 "ns_plan_kernels_grouped"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.ns_version() >= 300


def test_status_strings_and_word_layout():
    for code in range(6):
        assert B.status_string(code) != "unknown status"
    assert B.status_string(99) == "unknown status"
    # The status word keeps the code in its low byte and the place bits
    # above it, as the header's NS_STATUS_CODE and NS_STATUS_AT_* say.
    text = open(HEADER).read()
    assert "NS_ERR_NONFINITE = 5" in text
    for name, bit in [("NS_STATUS_AT_INPUT", B.STATUS_AT_INPUT),
                      ("NS_STATUS_AT_STATE", B.STATUS_AT_STATE),
                      ("NS_STATUS_AT_ITERATE", B.STATUS_AT_ITERATE),
                      ("NS_STATUS_AT_OUTPUT", B.STATUS_AT_OUTPUT),
                      ("NS_STATUS_AT_SPLIT", B.STATUS_AT_SPLIT),
                      ("NS_STATUS_GUARD_RESTART", B.STATUS_GUARD_RESTART)]:
        m = re.search(r"#define " + name + r" \(1 << (\d+)\)", text)
        assert m and (1 << int(m.group(1))) == bit, name
        assert bit > 0xFF
    word = B.NS_ERR_NONFINITE | B.STATUS_AT_STATE | B.STATUS_AT_OUTPUT
    assert nsa.status_code(word) == B.NS_ERR_NONFINITE
    assert nsa.status_code(B.STATUS_GUARD_RESTART) == 0


def test_options_defaults():
    opt = B.Options()
    B.lib().ns_options_default(ctypes.byref(opt))
    assert opt.restart_mask == 1 << 4
    assert abs(opt.eps - 1e-7) < 1e-12
    assert opt.internal == -1 and not opt.d_status
    assert opt.tile == 0


def test_workspace_size_layout():
    # Standard: partial sums + 2 pairs of X and X^T buffers + 2 n x n
    # buffers (fp16 internal).
    ws = nsa.workspace_size(4096, 14336, 1, torch.bfloat16, "standard",
                            tile=256)
    x = 4096 * 14336 * 2
    nn = 4096 * 4096 * 2
    assert 4 * x + 2 * nn <= ws <= 4 * x + 2 * nn + 16384
    wg = nsa.workspace_size(4096, 14336, 1, torch.bfloat16, "gram", tile=256)
    assert wg - ws == pytest.approx(2 * nn, abs=1024)
    # Tile 192: n and m are padded to multiples of 192 (4224 and 14400).
    w192 = nsa.workspace_size(4096, 14336, 1, torch.bfloat16, "standard",
                              tile=192)
    x192, nn192 = 4224 * 14400 * 2, 4224 * 4224 * 2
    assert 4 * x192 + 2 * nn192 <= w192 <= 4 * x192 + 2 * nn192 + 16384
    # Tall input has the same workspace as its transpose.
    assert nsa.workspace_size(14336, 4096) == nsa.workspace_size(4096, 14336)
    # Ragged sizes are padded to the tile edge (128 below 512 rows).
    w = nsa.workspace_size(200, 300, 1, torch.float16, "standard")
    assert w >= 4 * 256 * 384 * 2 + 2 * 256 * 256 * 2
    # fp32 doubles the buffers.
    assert nsa.workspace_size(256, 1024, 1, torch.float32) > \
        nsa.workspace_size(256, 1024, 1, torch.bfloat16)
    # Batches scale linearly.
    one = nsa.workspace_size(2048, 1408, 1, torch.bfloat16, "gram", tile=256)
    many = nsa.workspace_size(2048, 1408, 128, torch.bfloat16, "gram",
                              tile=256)
    assert 127 * one < many <= 128 * one


def _padded_n(rows, cols, batch=1, mode="gram"):
    """n_pad the automatic tile choice gives, read off the workspace size."""
    n = min(rows, cols)
    ws = nsa.workspace_size(rows, cols, batch, torch.bfloat16, mode)
    for tile in (128, 192, 256):
        if nsa.workspace_size(rows, cols, batch, torch.bfloat16, mode,
                              tile=tile) == ws:
            return tile
    raise AssertionError(f"no forced tile reproduces the automatic plan for {n}")


def test_largest_sizes_are_accepted():
    # No 2 GiB cap on one matrix: a 16384 x 65536 bf16 input needs 2 GiB X
    # buffers; n = 65536 and m = 2^24 are the limits.
    assert nsa.workspace_size(16384, 65536, 1, torch.bfloat16, "gram") > 8 << 30
    assert nsa.workspace_size(8, 1 << 24, 1, torch.bfloat16, "standard") > 0
    assert nsa.workspace_size(65536, 65536, 1, torch.bfloat16, "standard") > 0


def test_automatic_tile_choice():
    # 4096 x 4096 symmetric products: 253 tiles of 192 fill the 256 compute
    # units where 136 tiles of 256 leave half of them idle.
    assert _padded_n(4096, 14336) == 192
    # Large matrices: the 192 tile beats both others (measured on MI355X:
    # 8192 x 28672 in 19.1 ms at 192, 22.4 ms at 128, 23.8 ms at 256).
    # 192-padding differs from the other two here, so the match is unique.
    assert _padded_n(8192, 28672) == 192
    assert _padded_n(5120, 17920) == 192
    assert _padded_n(8192, 8192) == 192
    # Small matrices use 128, and so does the 128-expert MoE batch (1408 is
    # a multiple of 128, and its launches take the two-work-groups-per-CU
    # kernels).
    assert _padded_n(300, 500) == 128
    assert _padded_n(2048, 1408, 128) == 128
    # Forced tiles: fp32 products take 64 or 128, 16-bit ones 128, 192 or
    # 256; unknown edges are refused.
    lib = B.lib()
    for tile in (64, 200, 512):
        opt = B.make_options(tile=tile)
        assert lib.ns_workspace_size(512, 512, 1, B.NS_BF16, 0,
                                     ctypes.byref(opt)) == 0
    for tile in (192, 256):
        opt = B.make_options(tile=tile)
        assert lib.ns_workspace_size(512, 512, 1, B.NS_FP32, 0,
                                     ctypes.byref(opt)) == 0
    # fp32 takes 64 tiles while the n x n products would have fewer than 256
    # tiles of 128 (one wave on the chip): the 256 x 1024 matrix (3 tiles of
    # 128, 10 of 64) and a batch of 12 512 x 1000 (120), not a batch of 40
    # (400).
    for (r, c, b), want in [((256, 1024, 1), 64), ((512, 1000, 12), 64),
                            ((512, 1000, 40), 128), ((4096, 4096, 1), 128)]:
        ks = nsa.plan_kernels(r, c, b, torch.float32, "gram")
        assert ks[2].startswith(f"xxt<f32,{want},"), (r, c, b, ks)


def test_workspace_size_rejects_bad_arguments():
    lib = B.lib()
    bad = [(0, 5, 1, 0, 0), (5, 0, 1, 0, 0), (5, 5, 0, 0, 0), (5, 5, 1, 7, 0),
           (5, 5, 1, 0, 3), (5, 5, 70000, 0, 0),
           (65537, 70000, 1, 0, 0),            # n above 65536
           (5, (1 << 24) + 1, 1, 0, 0),        # m above 2^24 (16-bit)
           (5, (1 << 23) + 1, 1, 2, 0)]        # m above 2^23 (fp32)
    for rows, cols, batch, dt, mode in bad:
        assert lib.ns_workspace_size(rows, cols, batch, dt, mode, None) == 0
    # fp32 input cannot use 16-bit products; bf16 input cannot use fp32.
    opt = B.make_options(internal="fp16")
    assert lib.ns_workspace_size(8, 8, 1, B.NS_FP32, 0, ctypes.byref(opt)) == 0
    opt = B.make_options(internal="fp32")
    assert lib.ns_workspace_size(8, 8, 1, B.NS_BF16, 0, ctypes.byref(opt)) == 0


def test_bf16_products_are_refused():
    # bf16 operands keep 8 mantissa bits in every stored intermediate and
    # miss the 1e-2 bar of 16-bit input, so the option is refused for every
    # input type (the automatic choice is fp16 for 16-bit input).
    lib = B.lib()
    opt = B.make_options(internal="bf16")
    for dt in (B.NS_BF16, B.NS_FP16, B.NS_FP32):
        assert lib.ns_workspace_size(64, 96, 1, dt, 1, ctypes.byref(opt)) == 0
    assert _call(opt=opt) == 2
    assert _call(opt=opt, dtype=B.NS_FP16) == 2
    assert nsa.plan_kernels(64, 96, dtype=torch.bfloat16)[1] == "stage<bf16,f16>"


def _call(ptr=1, rows=8, cols=8, ld=8, dtype=B.NS_BF16, steps=5, abc=None,
          mode=B.NS_STANDARD, opt=None, ws=256, ws_bytes=1 << 40):
    a, b, c = B._coefficients(abc or B.TUNED_ABC, max(steps, 1))
    return B.lib().ns_orthogonalize(
        ctypes.c_void_p(ptr), rows, cols, ld, dtype, steps, a, b, c, mode,
        ctypes.byref(opt) if opt is not None else None, ctypes.c_void_p(ws),
        ws_bytes, None)


def test_orthogonalize_argument_checks():
    inv, dt, wsp = 1, 2, 3
    assert _call(ptr=0) == inv
    assert _call(rows=0) == inv
    assert _call(ld=7) == inv
    assert _call(steps=0) == inv
    assert _call(steps=17) == inv
    assert _call(dtype=9) == dt
    assert _call(mode=5) == inv
    assert _call(ws=0) == wsp
    assert _call(ws=128 + 256) == wsp                    # misaligned
    assert _call(ws_bytes=16) == wsp
    assert _call(abc=(float("nan"), 1.0, 1.0)) == inv
    opt = B.make_options(eps=-1.0)
    assert _call(opt=opt) == inv
    # Gram with fp16 state: Q reaches the product of the a_k between
    # restarts, which must stay below 2^15 (3.4445^8 < 2^15 < 3.4445^9).
    opt = B.make_options(restart_mask=0)
    assert _call(steps=9, mode=B.NS_GRAM, opt=opt) == inv
    assert _call(steps=8, mode=B.NS_GRAM, opt=opt, ws_bytes=16) == wsp
    opt = B.make_options(restart_mask=(1 << 4) | (1 << 7))
    # 3 + 3 + 3 steps between restarts: 3.4445^3 < 2^15, but the check runs
    # before the workspace check, which is what fails here.
    assert _call(steps=9, mode=B.NS_GRAM, opt=opt, ws_bytes=16) == wsp


def test_coefficient_range_check_follows_the_scalar_map():
    # Schedules whose product of |a_k| is small but whose other stored
    # quantities leave the fp16 range: Z' = b R + c R^2 reaches |c| at
    # s = 1, V = R Z and R <- R Z^2 grow with z^2, and the standard form's
    # X (held as 2^10 X) reaches p(1) = a + b + c.
    inv, wsp = 1, 3
    gram, std = B.NS_GRAM, B.NS_STANDARD
    opt0 = B.make_options(restart_mask=0)
    assert _call(steps=1, abc=(1.0, 0.0, 40000.0), mode=gram, opt=opt0) == inv
    assert _call(steps=1, abc=(1.0, 0.0, 20000.0), mode=gram, opt=opt0, ws_bytes=16) == wsp
    # R <- R z^2 after step 1 with z = 200 at s = 1: 4e4 (the product of
    # the a_k is only 200); step 2 multiplies by 1.
    assert _call(steps=2, abc=[(200.0, 0.0, 0.0), (1.0, 0.0, 0.0)], mode=gram,
                 opt=opt0) == inv
    assert _call(steps=2, abc=[(100.0, 0.0, 0.0), (1.0, 0.0, 0.0)], mode=gram,
                 opt=opt0, ws_bytes=16) == wsp
    # Standard form: the next X is p(s) <= 40; held as 2^10 X that is 4e4.
    assert _call(steps=2, abc=(40.0, 0.0, 0.0), mode=std) == inv
    assert _call(steps=2, abc=(20.0, 0.0, 0.0), mode=std, ws_bytes=16) == wsp
    # fp32 products have fp32's range.
    assert _call(steps=2, abc=(40.0, 0.0, 0.0), mode=std, dtype=B.NS_FP32,
                 ws_bytes=16) == wsp
    # The result of a one-step schedule is p(s) <= 40000: above 2^15 in fp16
    # I/O, inside bf16's and fp32's range.
    one = (40000.0, 0.0, 0.0)
    assert _call(steps=1, abc=one, mode=std, dtype=B.NS_FP16) == inv
    assert _call(steps=1, abc=one, mode=std, dtype=B.NS_BF16, ws_bytes=16) == wsp
    assert _call(steps=1, abc=one, mode=std, dtype=B.NS_FP32, ws_bytes=16) == wsp
    # The tuned and classic triples, and every per-shape ROOT schedule in
    # the coefficient table, pass in both forms.
    for abc in (B.TUNED_ABC, (2.0, -1.5, 0.5)):
        for mode in (std, gram):
            assert _call(abc=abc, mode=mode, ws_bytes=16) == wsp
    from newton_schulz_matrix_amd import coeffs
    for entry in coeffs.load_table().values():
        sched = [tuple(t) for t in entry["coefficients"]]
        for mode in (std, gram):
            assert _call(steps=len(sched), abc=sched, mode=mode, ws_bytes=16) == wsp


def test_grouped_argument_checks():
    lib = B.lib()
    a, b, c = B._coefficients(B.TUNED_ABC, 5)
    # The workspace is the batch's plus the member table.
    plain = nsa.workspace_size(300, 700, 24, torch.bfloat16, "gram")
    grouped = nsa.grouped_workspace_size(300, 700, 24, torch.bfloat16, "gram")
    assert plain + 24 * 24 <= grouped <= plain + 24 * 24 + 512
    assert nsa.grouped_workspace_size(700, 300, 24) == 0      # n > m
    need = grouped

    def call(members, n=300, m=700, wsb=None):
        arr = (B.Matrix * len(members))()
        for i, (data, ld, tr, res) in enumerate(members):
            arr[i].data, arr[i].ld, arr[i].transposed, arr[i].reserved = data, ld, tr, res
        return lib.ns_orthogonalize_grouped(arr, len(members), n, m, B.NS_BF16, 5, a, b, c, B.NS_GRAM, None,
                                            ctypes.c_void_p(256), need if wsb is None else wsb, None)
    ok = (256, 700, 0, 0)
    assert call([ok, (512, 300, 1, 0)], wsb=16) == 3          # arguments fine; workspace too small
    assert call([ok, (0, 700, 0, 0)]) == 1                     # null member
    assert call([ok, (256, 699, 0, 0)]) == 1                   # ld below the stored width
    assert call([ok, (256, 299, 1, 0)]) == 1
    assert call([ok, (256, 700, 2, 0)]) == 1                   # transposed not 0 or 1
    assert call([ok, (256, 700, 0, 5)]) == 1                   # reserved not 0
    assert call([ok], n=701, m=700) == 1                       # n > m
    assert lib.ns_orthogonalize_grouped(None, 1, 300, 700, B.NS_BF16, 5, a, b, c, B.NS_GRAM, None,
                                        ctypes.c_void_p(256), need, None) == 1


def test_guard_threshold_checks():
    inv, wsp = 1, 3
    for bad in (-1.0, float("nan"), float("inf")):
        assert _call(opt=B.make_options(guard=bad), mode=B.NS_GRAM) == inv
    assert _call(opt=B.make_options(guard=100.0), mode=B.NS_GRAM, ws_bytes=16) == wsp
    # The guarded Gram form always enqueues the (gated) restart update.
    ks = nsa.plan_kernels(300, 700, 1, torch.bfloat16, "gram", restart_mask=0)
    assert not any(k.startswith("upd<") for k in ks)
    opt = B.make_options(restart_mask=0, guard=100.0)
    buf = ctypes.create_string_buffer(512)
    B.lib().ns_plan_kernels(300, 700, 1, B.NS_BF16, B.NS_GRAM, 5, ctypes.byref(opt), buf, 512)
    assert "upd<f16,f16,128,tile,noE,x>" in buf.value.decode().split()


def test_plan_kernels_names_the_builds():
    ks = nsa.plan_kernels(4096, 14336, 1, torch.bfloat16, "gram")
    assert ks == ["sumsq<bf16>", "stage<bf16,f16>", "xxt<f16,192,tile>",
                  "nn<f16,192,tile>", "upd<f16,f16,192,tile,noE>",
                  "out<f16,bf16,192,tile,noE>"]
    # The MoE batch writes more than 256 MiB per launch: the builds with
    # non-temporal stores (",nt").
    ks = nsa.plan_kernels(2048, 1408, 128, torch.bfloat16, "standard")
    assert ks[2:] == ["xxt<f16,128,pairloop,nt>", "nn<f16,128,pairloop,nt>",
                      "upd<f16,f16,128,pair,E,nt>", "out<f16,bf16,128,pair,E,nt>"]
    ks = nsa.plan_kernels(768, 768, 48, torch.bfloat16, "gram")
    assert not any(k.endswith(",nt>") for k in ks)
    # Five 4096 x 4096 matrices: only the n x n launch that also writes the
    # fresh Q (2 x 168 MB) passes the limit.
    ks = nsa.plan_kernels(4096, 4096, 5, torch.bfloat16, "gram", tile=128)
    assert "nn<f16,128,pair,nt>" in ks and "nn<f16,128,pair>" in ks
    # The naive Gram form has no restart update; fp32
    # reads the a X term from global memory (small fp32 matrices take 64
    # tiles).
    ks = nsa.plan_kernels(300, 200, 1, torch.float32, "gram", restart_mask=0)
    assert not any(k.startswith("upd<") for k in ks)
    ks = nsa.plan_kernels(300, 200, 1, torch.float32, "standard")
    assert "upd<f32,f32,64,tile,Eg>" in ks
    assert B.lib().ns_plan_kernels(0, 5, 1, 0, 0, 5, None, None, 0) == -1
    # Builds that read extended arguments carry ",x": with the guard every
    # launch but the first step's n x n product (and never the non-temporal
    # builds); in a grouped call the final product only.
    ks = nsa.plan_kernels(4096, 14336, 1, torch.bfloat16, "gram", guard=100.0)
    assert ks == ["sumsq<bf16>", "stage<bf16,f16>", "xxt<f16,192,tile,x>",
                  "nn<f16,192,tile>", "nn<f16,192,tile,x>",
                  "upd<f16,f16,192,tile,noE,x>", "out<f16,bf16,192,tile,noE,x>"]
    ks = nsa.plan_kernels(2048, 1408, 128, torch.bfloat16, "gram", guard=100.0)
    assert ks[2:4] == ["xxt<f16,128,pairloop,x>", "nn<f16,128,pairloop,nt>"]
    for orient in ((768, 3072), (3072, 768)):
        ks = nsa.plan_kernels(*orient, 24, torch.bfloat16, "standard", grouped=True)
        assert ks[2:] == ["xxt<f16,192,tile>", "nn<f16,192,tile>",
                          "upd<f16,f16,192,loop,E>", "out<f16,bf16,192,loop,E,x>"]
    opt = B.make_options()
    assert B.lib().ns_plan_kernels_grouped(3072, 768, 24, B.NS_BF16, B.NS_GRAM, 5,
                                           ctypes.byref(opt), None, 0) == -1


def test_batched_argument_checks():
    a, b, c = B._coefficients(B.TUNED_ABC, 5)
    lib = B.lib()
    # batch stride smaller than one matrix.
    st = lib.ns_orthogonalize_batched(ctypes.c_void_p(256), 4, 8, 8, 8, 32,
                                      B.NS_BF16, 5, a, b, c, B.NS_GRAM, None,
                                      ctypes.c_void_p(256), 1 << 40, None)
    assert st == 1
    # The update's one-dimensional grid: batch * (n/128) * (m/128) < 2^31.
    assert lib.ns_workspace_size(8192, 1 << 20, 65535, B.NS_BF16, 1, None) == 0
    assert lib.ns_workspace_size(8192, 1 << 20, 255, B.NS_BF16, 1, None) > 0


def test_soft_threshold_argument_checks():
    lib = B.lib()
    assert lib.ns_soft_threshold_workspace_size(0, 0) == 0
    assert lib.ns_soft_threshold_workspace_size(10, 5) == 0
    need = lib.ns_soft_threshold_workspace_size(10, 0)
    assert need > 0
    args = dict(M=256, Bp=256, O=None, numel=10, dt=0, lam=-1.0, mult=3.0,
                ws=256, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return lib.ns_soft_threshold_split(
            ctypes.c_void_p(a["M"]), ctypes.c_void_p(a["Bp"]),
            ctypes.c_void_p(a["O"]), a["numel"], a["dt"], a["lam"], a["mult"],
            None, None, ctypes.c_void_p(a["ws"]), a["wsb"], None)
    assert call(M=0) == 1
    assert call(numel=0) == 1
    # Bin counts are 32-bit: 2^32 elements and more are refused.
    assert lib.ns_soft_threshold_workspace_size(1 << 32, 0) == 0
    assert lib.ns_soft_threshold_workspace_size((1 << 32) - 1, 0) == need
    assert call(numel=1 << 32) == 1
    assert call(lam=float("nan")) == 1
    assert call(mult=float("inf")) == 1
    assert call(dt=4) == 2
    assert call(wsb=need - 1) == 3
    assert call(ws=0) == 3


def test_muon_workspace_and_argument_checks():
    lib = B.lib()
    # The Muon workspace is the orthogonalization's plus one U buffer in the
    # I/O dtype.
    ns_ws = nsa.workspace_size(300, 700, 2, torch.bfloat16, "gram")
    mu_ws = nsa.muon_workspace_size(300, 700, 2, torch.bfloat16, "gram")
    assert ns_ws + 2 * 300 * 700 * 2 <= mu_ws <= ns_ws + 2 * 300 * 700 * 2 + 512
    assert lib.ns_muon_workspace_size(0, 5, 1, 0, 1, None) == 0
    a, b, c = B._coefficients(B.TUNED_ABC, 5)
    need = lib.ns_muon_workspace_size(8, 8, 1, B.NS_BF16, B.NS_GRAM, None)

    def call(W=256, G=256, M=256, batch=1, rows=8, cols=8, ld=8, bs=64,
             dt=B.NS_BF16, lr=0.02, mom=0.95, nest=1, steps=5, mode=B.NS_GRAM,
             ws=256, wsb=None):
        return lib.ns_muon_step(
            ctypes.c_void_p(W), ctypes.c_void_p(G), ctypes.c_void_p(M), batch,
            rows, cols, ld, bs, dt, lr, mom, nest, steps, a, b, c, mode, None,
            ctypes.c_void_p(ws), need if wsb is None else wsb, None)
    inv, dt, wsp = 1, 2, 3
    assert call(W=0) == inv
    assert call(G=0) == inv
    assert call(M=0) == inv
    assert call(ld=7) == inv
    assert call(batch=2, bs=32) == inv          # stride below one matrix
    assert call(lr=float("nan")) == inv
    assert call(lr=float("inf")) == inv
    assert call(mom=1.0) == inv
    assert call(mom=-0.1) == inv
    assert call(steps=0) == inv
    assert call(dt=7) == dt
    assert call(wsb=need - 1) == wsp
    assert call(ws=0) == wsp
