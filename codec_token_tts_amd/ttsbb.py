"""Thin Python binding of libttsbb.so (the C ABI in include/ttsbb.h).

Argument marshalling only: every step of the forward pass runs in the library's HIP
kernels.  Tensor arguments may be torch tensors on the GPU (their data_ptr is passed),
raw integer device addresses, or None for NULL.  The library is loaded from
codec_token_tts_amd/lib/libttsbb.so; if it is missing, loading raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libttsbb.so")

OK, INVALID_ARG, UNSUPPORTED, OOM, DEVICE_ERROR = 0, -1, -2, -3, -4
F32, BF16 = 0, 1

(TAP_X_IN, TAP_H_ATTN, TAP_QKV, TAP_Q, TAP_K, TAP_V, TAP_ATTN, TAP_X_MID, TAP_H_FFN, TAP_MLP,
 TAP_X_OUT, TAP_HEAD_IN, TAP_LOGITS, TAP_LOGITS_U) = range(14)

EXPORTS = ["ttsbb_default_config", "ttsbb_create", "ttsbb_destroy", "ttsbb_status_str",
           "ttsbb_sync", "ttsbb_codebook_embed", "ttsbb_decode_step", "ttsbb_decode_step_noalloc", "ttsbb_prefill", "ttsbb_maskgit_pass",
           "ttsbb_maskgit_pass_cfg", "ttsbb_maskgit_step", "ttsbb_rvq_decode", "ttsbb_philox_words", "ttsbb_unmask_schedule", "ttsbb_set_tap_layer", "ttsbb_read_tap", "ttsbb_profile_start",
           "ttsbb_profile_stop"]

(K_EMBED, K_RMSNORM, K_GEMM_QKV, K_ROPE_KV, K_DECODE_ATTN, K_DECODE_COMBINE, K_FLASH_ATTN, K_GEMM_O,
 K_GEMM_GATE_UP, K_GEMM_DOWN, K_GEMM_HEAD, K_ARGMAX, K_SCORES, K_SELECT) = range(14)
K_COUNT = 15
K_NAMES = ["embed", "rmsnorm", "gemm_qkv", "rope_kv", "decode_attn", "decode_combine", "flash_attn",
           "gemm_o", "gemm_gate_up", "gemm_down", "gemm_head", "argmax", "scores", "select", "rvq"]


class ttsbb_maskgit_step_args(C.Structure):
    _fields_ = [("n_text", C.c_int32), ("text_ids", C.c_void_p), ("text_table", C.c_void_p),
                ("text_vocab", C.c_int32), ("n_frames", C.c_int32), ("n_target", C.c_int32),
                ("n_cb", C.c_int32), ("cb_vocab", C.c_int32), ("mask_id", C.c_int32),
                ("audio_tables", C.c_void_p), ("audio_heads", C.c_void_p), ("codes", C.c_void_p),
                ("n_unmask", C.c_int32), ("layer_penalty", C.c_float), ("cfg_scale", C.c_float),
                ("class_temp", C.c_float), ("pos_temp", C.c_float), ("top_k_ratio", C.c_float),
                ("u_class", C.c_void_p), ("u_pos", C.c_void_p), ("pred", C.c_void_p), ("conf", C.c_void_p),
                ("picked", C.c_void_p), ("rng_seed", C.c_uint64), ("rng_counter", C.c_void_p)]


class TtsbbError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, ttsbb_status_str(status), status))
        self.status = status


class ttsbb_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_double), ("dtype", C.c_int32),
                ("kv_page", C.c_int32), ("max_rows", C.c_int32), ("max_pos", C.c_int32),
                ("max_head_cols", C.c_int32)]


class ttsbb_layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "q_norm", "k_norm", "ffn_norm", "wq", "wk",
                                          "wv", "wo", "w_gate", "w_up", "w_down")]


_lib = None


def lib() -> C.CDLL:
    """Load libttsbb.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libttsbb.so is not built (%s); run python -m codec_token_tts_amd.build"
                           % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    sig = {
        "ttsbb_default_config": (None, [C.POINTER(ttsbb_config)]),
        "ttsbb_create": (i32, [C.POINTER(ttsbb_config), C.POINTER(ttsbb_layer), vp, vp,
                               C.POINTER(vp)]),
        "ttsbb_destroy": (None, [vp]),
        "ttsbb_status_str": (C.c_char_p, [i32]),
        "ttsbb_sync": (i32, [vp]),
        "ttsbb_codebook_embed": (i32, [vp, i32, i32, vp, vp, i32, vp, vp, vp, i32, vp]),
        "ttsbb_decode_step": (i32, [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp]),
        "ttsbb_decode_step_noalloc": (i32, [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp]),
        "ttsbb_prefill": (i32, [vp, i32, vp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp]),
        "ttsbb_maskgit_pass": (i32, [vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, f32,
                                     vp, vp, vp]),
        "ttsbb_maskgit_pass_cfg": (i32, [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, f32,
                                         f32, vp, vp, vp]),
        "ttsbb_maskgit_step": (i32, [vp, C.POINTER(ttsbb_maskgit_step_args)]),
        "ttsbb_rvq_decode": (i32, [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "ttsbb_philox_words": (i32, [vp, C.c_uint64, C.c_uint64, C.c_uint32, C.c_uint32, i32, vp]),
        "ttsbb_unmask_schedule": (i32, [i32, i32, C.POINTER(i32)]),
        "ttsbb_set_tap_layer": (i32, [vp, i32]),
        "ttsbb_read_tap": (i32, [vp, i32, vp, i64, C.POINTER(i32), C.POINTER(i32)]),
        "ttsbb_profile_start": (i32, [vp, C.c_uint32, i32]),
        "ttsbb_profile_stop": (i32, [vp, C.POINTER(f32), C.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def ptr(t):
    """Device address of a torch tensor (must live on the GPU), an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("ttsbb needs device tensors; got a tensor on %s" % t.device)
    return t.data_ptr()


def _check(status: int, where: str):
    if status != OK:
        raise TtsbbError(status, where)


def ttsbb_status_str(status: int) -> str:
    return lib().ttsbb_status_str(status).decode()


def ttsbb_default_config() -> ttsbb_config:
    cfg = ttsbb_config()
    lib().ttsbb_default_config(C.byref(cfg))
    return cfg


def make_layer(attn_norm, q_norm, k_norm, ffn_norm, wq, wk, wv, wo, w_gate, w_up, w_down):
    return ttsbb_layer(*[ptr(t) for t in (attn_norm, q_norm, k_norm, ffn_norm, wq, wk, wv, wo,
                                          w_gate, w_up, w_down)])


def ttsbb_create(cfg: ttsbb_config, layers, final_norm, stream=None, raw_status: bool = False):
    """Returns a context handle (int).  `layers` is a sequence of ttsbb_layer."""
    arr = (ttsbb_layer * max(1, len(layers)))(*layers)
    out = C.c_void_p()
    st = lib().ttsbb_create(C.byref(cfg), arr if len(layers) else None, ptr(final_norm),
                            ptr(stream) if stream is not None else None, C.byref(out))
    if raw_status:
        return st, out.value
    _check(st, "ttsbb_create")
    return out.value


def ttsbb_destroy(ctx):
    lib().ttsbb_destroy(ctx)


def ttsbb_sync(ctx) -> int:
    return lib().ttsbb_sync(ctx)


def ttsbb_codebook_embed(ctx, n_rows, n_cb, codes, tables, cb_vocab, is_text, text_ids,
                         text_table, text_vocab, out, check: bool = True) -> int:
    st = lib().ttsbb_codebook_embed(ctx, n_rows, n_cb, ptr(codes), ptr(tables), cb_vocab,
                                    ptr(is_text), ptr(text_ids), ptr(text_table), text_vocab,
                                    ptr(out))
    if check:
        _check(st, "ttsbb_codebook_embed")
    return st


def ttsbb_decode_step(ctx, batch, x, positions, page_table, max_pages, kv_pool, n_pages,
                      head=None, n_groups=0, group_vocab=0, argmax=None, logits=None,
                      check: bool = True) -> int:
    st = lib().ttsbb_decode_step(ctx, batch, ptr(x), ptr(positions), ptr(page_table), max_pages,
                                 ptr(kv_pool), n_pages, ptr(head), n_groups, group_vocab,
                                 ptr(argmax), ptr(logits))
    if check:
        _check(st, "ttsbb_decode_step")
    return st


def ttsbb_decode_step_noalloc(ctx, batch, x, positions, page_table, max_pages, kv_pool, n_pages,
                              head=None, n_groups=0, group_vocab=0, argmax=None, logits=None,
                              check: bool = True) -> int:
    st = lib().ttsbb_decode_step_noalloc(ctx, batch, ptr(x), ptr(positions), ptr(page_table), max_pages,
                                         ptr(kv_pool), n_pages, ptr(head), n_groups, group_vocab,
                                         ptr(argmax), ptr(logits))
    if check:
        _check(st, "ttsbb_decode_step_noalloc")
    return st


def ttsbb_maskgit_pass(ctx, n_text, text_ids, text_table, text_vocab, n_frames, n_cb, cb_vocab,
                       mask_id, audio_tables, audio_heads, codes, n_unmask, layer_penalty, pred,
                       conf, picked, check: bool = True) -> int:
    st = lib().ttsbb_maskgit_pass(ctx, n_text, ptr(text_ids), ptr(text_table), text_vocab,
                                  n_frames, n_cb, cb_vocab, mask_id, ptr(audio_tables),
                                  ptr(audio_heads), ptr(codes), n_unmask, float(layer_penalty),
                                  ptr(pred), ptr(conf), ptr(picked))
    if check:
        _check(st, "ttsbb_maskgit_pass")
    return st


def ttsbb_unmask_schedule(n_total: int, n_steps: int):
    out = (C.c_int32 * max(1, n_steps))()
    _check(lib().ttsbb_unmask_schedule(n_total, n_steps, out), "ttsbb_unmask_schedule")
    return [int(out[i]) for i in range(n_steps)]


def ttsbb_set_tap_layer(ctx, layer: int):
    _check(lib().ttsbb_set_tap_layer(ctx, layer), "ttsbb_set_tap_layer")


def ttsbb_maskgit_pass_cfg(ctx, n_text, text_ids, text_table, text_vocab, n_frames, n_target, n_cb,
                           cb_vocab, mask_id, audio_tables, audio_heads, codes, n_unmask, layer_penalty,
                           cfg_scale, pred, conf, picked, check: bool = True) -> int:
    st = lib().ttsbb_maskgit_pass_cfg(ctx, n_text, ptr(text_ids), ptr(text_table), text_vocab,
                                      n_frames, n_target, n_cb, cb_vocab, mask_id, ptr(audio_tables),
                                      ptr(audio_heads), ptr(codes), n_unmask, float(layer_penalty),
                                      float(cfg_scale), ptr(pred), ptr(conf), ptr(picked))
    if check:
        _check(st, "ttsbb_maskgit_pass_cfg")
    return st


def ttsbb_maskgit_step(ctx, n_text, text_ids, text_table, text_vocab, n_frames, n_target, n_cb, cb_vocab,
                       mask_id, audio_tables, audio_heads, codes, n_unmask, layer_penalty, pred, conf, picked,
                       cfg_scale=0.0, class_temp=0.0, pos_temp=0.0, top_k_ratio=0.1, u_class=None, u_pos=None,
                       rng_seed=0, rng_counter=None, check: bool = True) -> int:
    a = ttsbb_maskgit_step_args(n_text, ptr(text_ids), ptr(text_table), text_vocab, n_frames, n_target, n_cb,
                                cb_vocab, mask_id, ptr(audio_tables), ptr(audio_heads), ptr(codes), n_unmask,
                                float(layer_penalty), float(cfg_scale), float(class_temp), float(pos_temp),
                                float(top_k_ratio), ptr(u_class), ptr(u_pos), ptr(pred), ptr(conf), ptr(picked),
                                int(rng_seed) & 0xFFFFFFFFFFFFFFFF, ptr(rng_counter))
    st = lib().ttsbb_maskgit_step(ctx, C.byref(a))
    if check:
        _check(st, "ttsbb_maskgit_step")
    return st


def ttsbb_rvq_decode(ctx, n_frames, n_q, codebook_size, codebook_dim, out_dim, codes, embed, proj_w, proj_b, out,
                     check: bool = True) -> int:
    st = lib().ttsbb_rvq_decode(ctx, n_frames, n_q, codebook_size, codebook_dim, out_dim, ptr(codes), ptr(embed),
                                ptr(proj_w), ptr(proj_b), ptr(out))
    if check:
        _check(st, "ttsbb_rvq_decode")
    return st


def ttsbb_philox_words(ctx, seed, block0, word2, word3, n_blocks, out, check: bool = True) -> int:
    st = lib().ttsbb_philox_words(ctx, int(seed) & 0xFFFFFFFFFFFFFFFF, int(block0) & 0xFFFFFFFFFFFFFFFF,
                                  int(word2) & 0xFFFFFFFF, int(word3) & 0xFFFFFFFF, n_blocks, ptr(out))
    if check:
        _check(st, "ttsbb_philox_words")
    return st


def ttsbb_prefill(ctx, n_tokens, x, cache_len, page_table, max_pages, kv_pool, n_pages, head=None, n_groups=0,
                  group_vocab=0, argmax=None, logits=None, check: bool = True) -> int:
    st = lib().ttsbb_prefill(ctx, n_tokens, ptr(x), ptr(cache_len), ptr(page_table), max_pages, ptr(kv_pool),
                             n_pages, ptr(head), n_groups, group_vocab, ptr(argmax), ptr(logits))
    if check:
        _check(st, "ttsbb_prefill")
    return st


def ttsbb_read_tap(ctx, tap: int, dst, n_floats: int):
    rows, cols = C.c_int32(0), C.c_int32(0)
    _check(lib().ttsbb_read_tap(ctx, tap, ptr(dst), n_floats, C.byref(rows), C.byref(cols)),
           "ttsbb_read_tap")
    return rows.value, cols.value


def ttsbb_profile_start(ctx, mask: int = (1 << 14) - 1, max_launches: int = 65536):
    _check(lib().ttsbb_profile_start(ctx, mask, max_launches), "ttsbb_profile_start")


def ttsbb_profile_stop(ctx):
    """Returns {kernel class name: (total ms, launches)}."""
    ms = (C.c_float * K_COUNT)()
    n = (C.c_int32 * K_COUNT)()
    _check(lib().ttsbb_profile_stop(ctx, ms, n), "ttsbb_profile_stop")
    return {K_NAMES[k]: (float(ms[k]), int(n[k])) for k in range(K_COUNT)}
