"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/vt.h declares, and rejects bad arguments with the documented status before any HIP
call.  Pointers here are fake, aligned addresses that validation never dereferences."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import draft_sampling_verification_amd as vt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(vt.LIB_PATH), reason="libvt.so not built")

OK, INV, UNS, WS, HIP = range(5)
F32, BF16 = 0, 1
P = ctypes.c_void_p
A = P(0x100000)  # 16-byte aligned fake device address
A2 = P(0x200000)
NUL = None


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(vt_\w+)\s*\(", text, re.M)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for fn in ("vt_lmhead_trimmed", "vt_softmax_temp", "vt_spec_verify", "vt_token_histogram", "vt_keep_select",
               "vt_trim_head", "vt_spec_generate_markov"):
        assert fn in names
    assert set(names) == set(vt.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = vt.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", vt.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (vt_\w+)$", out, re.M))
    for fn in declared_functions():
        assert hasattr(L, fn), fn
        assert fn in exported, fn


def test_status_strings():
    L = vt.lib()
    seen = set()
    for s in range(5):
        msg = L.vt_status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert L.vt_status_string(99) == b"unknown status"


def test_workspace_sizes():
    L = vt.lib()
    assert L.vt_softmax_temp_workspace_bytes(6, 4096) == 0  # single chunk rows need none
    assert L.vt_softmax_temp_workspace_bytes(6, 4097) > 0
    big = L.vt_softmax_temp_workspace_bytes(2304, 128256)
    assert big >= 2304 * 32 * 8
    assert L.vt_spec_verify_workspace_bytes(1, 4, 18) == 0
    assert L.vt_spec_verify_workspace_bytes(256, 8, 128256) >= 256 * 9 * 32 * 8  # greedy: per target row
    assert L.vt_spec_verify_workspace_bytes(4, 0, 128256) == 0
    assert L.vt_softmax_temp_workspace_bytes(0, 10) == 0
    assert L.vt_spec_verify_workspace_bytes(-1, 3, 10) == 0


# ------------------------------------------------------------------ vt_lmhead_trimmed

def lm(hidden=A, weight=A2, keep=NUL, M=6, H=3072, Vt=100, V=128, logits=A):
    return vt.lib().vt_lmhead_trimmed(hidden, weight, keep, M, H, Vt, V, logits, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=NUL), INV), (dict(weight=NUL), INV), (dict(logits=NUL), INV),
    (dict(M=0), INV), (dict(H=0), INV), (dict(Vt=0), INV), (dict(V=0), INV), (dict(M=-3), INV),
    (dict(Vt=200, V=128), INV),                       # untrimmed head with more columns than rows
    (dict(H=3076), UNS),                              # H % 8 != 0
    (dict(hidden=P(0x100008)), UNS),                  # misaligned hidden
    (dict(weight=P(0x200002)), UNS),                  # misaligned weight
])
def test_lmhead_rejects(kw, status):
    assert lm(**kw) == status


# ------------------------------------------------------------------ vt_softmax_temp

def sm(logits=A, dtype=F32, rows=6, n=128256, ld=None, T=1.0, lse=A, probs=NUL, u=NUL, sampled=NUL, ws=A2,
       wsb=1 << 30):
    ld = n if ld is None else ld
    return vt.lib().vt_softmax_temp(logits, dtype, rows, n, ld, T, lse, probs, u, sampled, ws, wsb, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(logits=NUL), INV), (dict(lse=NUL), INV), (dict(dtype=7), INV),
    (dict(rows=0), INV), (dict(n=0), INV), (dict(n=10, ld=9), INV),
    (dict(T=-1.0), INV), (dict(T=math.nan), INV), (dict(T=math.inf), INV), (dict(T=-0.0 - 1e-30), INV),
    (dict(u=A), INV), (dict(sampled=A), INV),            # u and sampled come together
    (dict(ws=NUL), WS), (dict(wsb=16), WS),
])
def test_softmax_rejects(kw, status):
    assert sm(**kw) == status


def test_softmax_workspace_exact_size_accepted_by_validation():
    need = vt.lib().vt_softmax_temp_workspace_bytes(6, 128256)
    assert sm(wsb=need - 1) == WS


# ------------------------------------------------------------------ vt_spec_verify

def vf(B=4, gamma=5, V=128256, Vt=32768, target=A, tdt=F32, tlse=A, Tt=1.0, draft=A, R=6, dlse=A, Td=1.0,
       ids=A, keep=A, f2t=A, ua=A, uf=A, tok=A, nacc=A, ws=A2, wsb=1 << 30):
    return vt.lib().vt_spec_verify(B, gamma, V, Vt, target, tdt, tlse, Tt, draft, R, dlse, Td, ids, keep, f2t,
                                   ua, uf, tok, nacc, ws, wsb, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(target=NUL), INV), (dict(tlse=NUL), INV), (dict(draft=NUL), INV), (dict(dlse=NUL), INV),
    (dict(ids=NUL), INV), (dict(ua=NUL), INV), (dict(uf=NUL), INV), (dict(tok=NUL), INV), (dict(nacc=NUL), INV),
    (dict(tdt=3), INV), (dict(B=0), INV), (dict(gamma=0), INV), (dict(V=0), INV), (dict(Vt=0), INV),
    (dict(Vt=200000), INV),                              # more kept ids than the vocabulary
    (dict(R=4), INV),                                    # fewer draft rows than drafts
    (dict(Tt=-1.0), INV), (dict(Td=-0.5), INV), (dict(Tt=math.nan), INV), (dict(Td=math.inf), INV),
    (dict(Tt=0.0, ids=NUL), INV),                        # greedy still needs the draft ids
    (dict(keep=NUL, f2t=NUL), INV),                      # trimmed head without the id maps
    (dict(keep=NUL), INV), (dict(f2t=NUL), INV),         # only one of the two maps
    (dict(gamma=65, R=66), UNS),
    (dict(ws=NUL), WS), (dict(wsb=8), WS),
])
def test_verify_rejects(kw, status):
    assert vf(**kw) == status


def test_missing_library_fails_loudly(tmp_path):
    # the binding has no fallback: without libvt.so every call raises
    code = ("import draft_sampling_verification_amd as vt; vt.LIB_PATH = '/nonexistent/libvt.so'\n"
            "try:\n    vt.lib()\nexcept RuntimeError as e:\n    print('raised', 'missing' in str(e))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.stdout.strip() == "raised True", out.stderr


# ------------------------------------------------------------------ vt_spec_block

def blk(hidden=A, weight=A2, wt=NUL, keep=A, f2t=A, B=4, gamma=5, R=6, H=3072, Vt=32768, V=128256, target=A,
        tdt=F32, Tt=1.0, Td=1.0, ud=A, ua=A, uf=A, dl=A, dlse=A, ids=A, tlse=A, tok=A, nacc=A, ws=A2, wsb=1 << 30):
    return vt.lib().vt_spec_block(hidden, weight, wt, keep, f2t, B, gamma, R, H, Vt, V, target, tdt, Tt, Td, ud, ua,
                                  uf, dl, dlse, ids, tlse, tok, nacc, NUL, NUL, ws, wsb, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=NUL), INV), (dict(weight=NUL), INV), (dict(target=NUL), INV), (dict(ud=NUL), INV),
    (dict(ua=NUL), INV), (dict(uf=NUL), INV), (dict(dl=NUL), INV), (dict(dlse=NUL), INV), (dict(ids=NUL), INV),
    (dict(tlse=NUL), INV), (dict(tok=NUL), INV), (dict(nacc=NUL), INV), (dict(tdt=2), INV),
    (dict(B=0), INV), (dict(gamma=0), INV), (dict(R=4), INV), (dict(H=0), INV), (dict(Vt=0), INV),
    (dict(V=1000), INV), (dict(Tt=-1.0), INV), (dict(Td=math.nan), INV),
    (dict(Td=0.0), INV),                                  # argmax drafts need greedy verification
    (dict(Tt=0.0, Td=0.0, ud=NUL, ua=NUL, uf=NUL, tlse=NUL, ids=NUL), INV),  # greedy still writes ids
    (dict(Tt=0.0, ua=NUL, uf=NUL, tlse=NUL, ud=NUL), INV),  # sampled drafts still need u_draft
    (dict(keep=NUL, f2t=NUL), INV), (dict(keep=NUL), INV), (dict(f2t=NUL), INV),
    (dict(gamma=65, R=65), UNS), (dict(H=3070), UNS), (dict(hidden=P(0x100004)), UNS),
    (dict(wt=P(0x100004)), UNS), (dict(wt=A, H=3080), UNS),  # the K-tiled head needs whole 32-column steps
    (dict(ws=NUL), WS), (dict(wsb=64), WS),
])
def test_block_rejects(kw, status):
    assert blk(**kw) == status


def test_block_workspace_sizes():
    L = vt.lib()
    small = L.vt_spec_block_workspace_bytes(1, 5, 6, 3072, 128256, 128256)
    big = L.vt_spec_block_workspace_bytes(256, 8, 9, 4096, 65536, 128256)
    assert 0 < small < big
    assert L.vt_spec_block_workspace_bytes(1, 5, 4, 3072, 100, 100) == 0  # R < gamma


# ------------------------------------------------------------------ keep-set construction

def hist(tokens=A, n=1000, V=128256, acc=0, counts=A2, ws=NUL, wsb=0):
    return vt.lib().vt_token_histogram(tokens, n, V, acc, counts, ws, wsb, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(counts=NUL), INV), (dict(tokens=NUL), INV), (dict(n=-1), INV), (dict(V=0), INV),
    (dict(V=1 << 31), UNS), (dict(tokens=P(0x100002)), UNS),
    (dict(n=1 << 24), WS), (dict(n=1 << 24, ws=A, wsb=1024), WS),
])
def test_histogram_rejects(kw, status):
    assert hist(**kw) == status


def test_histogram_workspace_sizes():
    L = vt.lib()
    assert L.vt_token_histogram_workspace_bytes(1000, 128256) == 0      # one group writes counts directly
    assert L.vt_token_histogram_workspace_bytes(1 << 26, 128256) == 64 * 128256 * 4
    assert L.vt_token_histogram_workspace_bytes(1 << 26, 1000) == 256 * 1000 * 4
    assert L.vt_token_histogram_workspace_bytes(-1, 10) == 0


def sel(counts=A, V=128256, rule=0, k=100, p=0.5, f=1, keep=A2, f2t=A2, nk=A):
    return vt.lib().vt_keep_select(counts, V, rule, k, p, f, keep, f2t, nk, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(counts=NUL), INV), (dict(keep=NUL), INV), (dict(f2t=NUL), INV), (dict(nk=NUL), INV), (dict(V=0), INV),
    (dict(rule=3), INV), (dict(k=0), INV), (dict(k=128257), INV),
    (dict(rule=1, p=0.0), INV), (dict(rule=1, p=1.5), INV), (dict(rule=1, p=math.nan), INV),
    (dict(V=1 << 31), UNS),
])
def test_keep_select_rejects(kw, status):
    assert sel(**kw) == status


def trim(w=A, V=128256, H=3072, keep=A2, k=10, out=A):
    return vt.lib().vt_trim_head(w, V, H, keep, k, out, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(w=NUL), INV), (dict(keep=NUL), INV), (dict(out=NUL), INV), (dict(V=0), INV), (dict(H=0), INV),
    (dict(k=0), INV), (dict(H=3070), UNS), (dict(w=P(0x100008)), UNS), (dict(out=P(0x100004)), UNS),
])
def test_trim_head_rejects(kw, status):
    assert trim(**kw) == status


def trim_tiled(w=A, V=128256, H=3072, keep=A2, k=10, out=A):
    return vt.lib().vt_trim_head_tiled(w, V, H, keep, k, out, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(w=NUL), INV), (dict(out=NUL), INV), (dict(V=0), INV), (dict(H=0), INV), (dict(k=0), INV),
    (dict(keep=NUL, k=128257), INV),  # rows 0..k-1 of the head need k <= V_rows
    (dict(H=3080), UNS), (dict(w=P(0x100008)), UNS), (dict(out=P(0x100004)), UNS), (dict(k=1 << 31), UNS),
])
def test_trim_head_tiled_rejects(kw, status):
    assert trim_tiled(**kw) == status


def test_trim_head_tiled_bytes():
    L = vt.lib()
    assert L.vt_trim_head_tiled_bytes(65536, 4096) == 65536 * 4096 * 2
    assert L.vt_trim_head_tiled_bytes(300, 64) == 512 * 64 * 2   # the last 256-row block is filled out
    assert L.vt_trim_head_tiled_bytes(300, 80) == 0             # H % 32 != 0
    assert L.vt_trim_head_tiled_bytes(0, 64) == 0


# ------------------------------------------------------------------ generation loop

def gen(tt=A, dt=A2, V=18, Tt=1.0, Td=1.0, g=4, B=10, L=20, u=A, tok=A2, st=NUL):
    return vt.lib().vt_spec_generate_markov(tt, dt, V, Tt, Td, g, B, L, u, tok, st, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(tt=NUL), INV), (dict(dt=NUL), INV), (dict(u=NUL), INV), (dict(tok=NUL), INV),
    (dict(V=0), INV), (dict(g=0), INV), (dict(B=0), INV), (dict(L=0), INV),
    (dict(Tt=0.0), INV), (dict(Td=-1.0), INV), (dict(Tt=math.inf), INV), (dict(Td=math.nan), INV),
    (dict(V=65), UNS), (dict(g=65), UNS), (dict(L=1 << 31), UNS),
])
def test_generate_rejects(kw, status):
    assert gen(**kw) == status
