"""The C ABI on the host: the library loads, exports every entry point include/spec.h
declares, the ctypes structs match the C layout (checked by compiling the header with gcc),
and host-side validation rejects bad configurations before any device work."""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_decoding_token_amd import binding as B
from speculative_decoding_token_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")


def declared_functions():
    return re.findall(r"^(?:int|int32_t|const char\*)\s+(\w+)\(", open(HEADER).read(), re.M)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    decl = declared_functions()
    assert sorted(decl) == sorted(B.EXPORTED)
    for name in decl:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    assert set(decl) <= exported


STRUCTS = ["spec_layer_weights", "spec_layer_scales", "spec_gdn_shape", "spec_model_desc", "spec_mtp_desc", "spec_sampler", "spec_ngram_cfg",
           "spec_config", "spec_probs", "spec_stats", "spec_gate"]


def test_ctypes_layout_matches_c(tmp_path):
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for s in STRUCTS:
        lines.append(f'  printf("{s} %zu\\n", sizeof({s}));')
        for fname, _ in getattr(B, s)._fields_:
            lines.append(f'  printf("{s}.{fname} %zu\\n", offsetof({s}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-o", str(exe), str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for s in STRUCTS:
        cls = getattr(B, s)
        assert int(got[s]) == ctypes.sizeof(cls), s
        for fname, _ in cls._fields_:
            assert int(got[f"{s}.{fname}"]) == getattr(cls, fname).offset, f"{s}.{fname}"


def host_cfg(shape, draft=None, **kw):
    cfg = B.spec_config()
    dummy = {"embed": 1, "lm_head": 1, "final_norm": 1,
             "layers": [{n: 1 for n in synth.LAYER_TENSORS} for _ in range(shape.n_layers)]}
    keep = []
    cfg.target = B.model_desc(shape, dummy, keep)
    cfg.draft_kind = B.DRAFT_NONE
    if draft is not None:
        cfg.draft_kind = B.DRAFT_MODEL
        dd = {"embed": 1, "lm_head": 1, "final_norm": 1,
              "layers": [{n: 1 for n in synth.LAYER_TENSORS} for _ in range(draft.n_layers)]}
        cfg.draft = B.model_desc(draft, dd, keep)
    cfg.sampler = B.sampler(kw.get("temperature", 1.0), kw.get("top_k", 20), kw.get("top_p", 0.95))
    cfg.seed = 0
    cfg.max_batch = kw.get("max_batch", 1)
    cfg.max_ctx = kw.get("max_ctx", 2048)
    cfg.max_k = kw.get("max_k", 8)
    return cfg, keep


def test_workspace_size_host_only():
    t, d = synth.SHAPES["qwen8b"], synth.SHAPES["qwen0p6b"]
    cfg, keep = host_cfg(t, d, max_ctx=2048, max_k=16)
    n = B.spec_workspace_size(cfg)
    # the two caches dominate: 36 layers x 8 kv heads x (2048+18) positions x 128 x 2 bytes x 2
    cache_t = 36 * 8 * (2048 + 16 + 2) * 128 * 2 * 2
    cache_d = 28 * 8 * (2048 + 16 + 2) * 128 * 2 * 2
    assert cache_t + cache_d < n < cache_t + cache_d + 256 << 20


@pytest.mark.parametrize("mut,code", [
    (lambda c: setattr(c, "max_k", 17), B.SPEC_E_INVAL),
    (lambda c: setattr(c, "max_batch", 0), B.SPEC_E_INVAL),
    (lambda c: setattr(c.sampler, "top_k", 65), B.SPEC_E_UNSUPPORTED),
    (lambda c: setattr(c.sampler, "top_p", 0.0), B.SPEC_E_INVAL),
    (lambda c: setattr(c.sampler, "top_p", 1.5), B.SPEC_E_INVAL),
    (lambda c: setattr(c.target, "head_dim", 96), B.SPEC_E_UNSUPPORTED),
    (lambda c: setattr(c.target, "n_kv_heads", 5), B.SPEC_E_INVAL),
    (lambda c: setattr(c.target, "dtype", 7), B.SPEC_E_INVAL),
    (lambda c: setattr(c.draft, "vocab", 1024), B.SPEC_E_INVAL),
    (lambda c: setattr(c, "draft_kind", 9), B.SPEC_E_INVAL),
    (lambda c: setattr(c, "max_batch", 8), B.SPEC_E_UNSUPPORTED),   # 8 x 9 rows > 64
    (lambda c: setattr(c.target, "weights", 2), B.SPEC_E_INVAL),
    (lambda c: (setattr(c.target, "weights", B.WEIGHTS_FP8_ROW), setattr(c.target, "dtype", B.DTYPE_F32)),
     B.SPEC_E_UNSUPPORTED),
    (lambda c: (setattr(c.target, "weights", B.WEIGHTS_FP8_ROW), setattr(c, "max_batch", 2)),
     B.SPEC_E_UNSUPPORTED),                                           # fp8: 2 x 9 rows > 16
    (lambda c: (setattr(c.target, "weights", B.WEIGHTS_FP8_ROW), setattr(c, "draft_kind", B.DRAFT_MTP)),
     B.SPEC_E_UNSUPPORTED),
])
def test_config_validation(mut, code):
    cfg, keep = host_cfg(synth.SHAPES["qwen8b"], synth.SHAPES["qwen0p6b"])
    mut(cfg)
    with pytest.raises(B.SpecError) as e:
        B.spec_workspace_size(cfg)
    assert e.value.code == code
    assert B.spec_last_error(None) != ""


def test_fp8_rows_cap_the_workspace():
    t = synth.SHAPES["qwen8b"]
    cfg, keep = host_cfg(t, max_k=6, max_batch=2)
    native = B.spec_workspace_size(cfg)
    cfg.target.weights = B.WEIGHTS_FP8_ROW
    fp8 = B.spec_workspace_size(cfg)
    # the same caches; activations (logits first) for 2 x 8 rows per forward instead of 2 x 16
    assert 16 * t.vocab * 4 < native - fp8 < 16 * t.vocab * 4 + (32 << 20)


@pytest.mark.parametrize("shape,nc,nf,code", [
    ((0, 128, 128), 1, 1, B.SPEC_E_INVAL),
    ((4, 64, 128), 1, 1, B.SPEC_E_UNSUPPORTED),
    ((4, 128, 48), 1, 1, B.SPEC_E_UNSUPPORTED),
    ((4, 128, 128), 40, 25, B.SPEC_E_RANGE),
    ((4, 128, 128), 2**31 - 1, 1, B.SPEC_E_RANGE),   # no wrap of the token sum
    ((4, 128, 128), -1, 1, B.SPEC_E_INVAL),
    ((4, 128, 128), 1, 1, B.SPEC_E_INVAL),   # null buffers
])
def test_gdn_argument_checks(shape, nc, nf, code):
    # every case is rejected on the host before any HIP call
    with pytest.raises(B.SpecError) as e:
        B.spec_gdn_commit_forward(*shape, None, None, None, None, None, None, nc, nf, None, stream=0)
    assert e.value.code == code


def test_gdn_nothing_to_do_is_ok():
    B.spec_gdn_commit_forward(4, 128, 128, None, None, None, None, None, None, 0, 0, None, stream=0)


def test_greedy_sampler_ignores_top_k():
    cfg, keep = host_cfg(synth.SHAPES["qwen8b"], temperature=0.0, top_k=0)
    assert B.spec_workspace_size(cfg) > 0


def test_truncate_scratch_size():
    n = B.spec_truncate_scratch_size(576, 151936)
    assert n >= 576 * 10 * 64 * 8
    with pytest.raises(B.SpecError):
        B.spec_truncate_scratch_size(1, 64 * 16384 * 2)   # too many segments for one merge


def test_mtp_and_ngram_configs():
    t = synth.SHAPES["qwen9b_mtp"]
    cfg, keep = host_cfg(t, max_ctx=8192, max_k=4)
    base = B.spec_workspace_size(cfg)
    cfg.draft_kind = B.DRAFT_MTP
    with_mtp = B.spec_workspace_size(cfg)
    # one more cache layer (8 kv heads x (8192+6) positions x 128 x 2 bytes x 2) and activations
    assert with_mtp - base > 8 * (8192 + 6) * 128 * 2 * 2
    cfg.draft_kind = B.DRAFT_NGRAM
    cfg.ngram = B.spec_ngram_cfg(3, 16)
    assert B.spec_workspace_size(cfg) == base
    cfg.ngram = B.spec_ngram_cfg(0, 16)
    with pytest.raises(B.SpecError) as e:
        B.spec_workspace_size(cfg)
    assert e.value.code == B.SPEC_E_INVAL
    cfg.ngram = B.spec_ngram_cfg(5, 4)
    with pytest.raises(B.SpecError):
        B.spec_workspace_size(cfg)
