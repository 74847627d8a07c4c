"""K8/V4 codec and paged-cache layout, CPU reference in plain numpy.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

What the pages fix
------------------
* Keys are stored with 8 bits and values with 4 bits (Launch HN digest,
  trawling.dev/post/1715, section "per-device kernel tuning and performance
  claims"; and the author's replies further down the same page).
* The engine's decode unit for that cache is ``attention_decode_k8v4``; its
  value codec works on groups of 32 and stores an fp16 scale
  (blog.123qwe.co.kr/?p=3927, section 5, the paragraph on the load log).

Readings taken where the pages are silent (the plainest ones that the rest
supports)
------------------------------------------------------------------------
* Symmetric codes, no zero point.  The blog's log line calls the codec
  "affine"; the workload specification this library is built for says
  symmetric, and a symmetric code is the affine code with zero offset.
* Keys: one scale per (token, kv head) over the head dimension.
  ``a = max|x|``; ``s = fp16(a / 127)`` (fp32 IEEE division, then round to
  nearest even into fp16; an fp16 overflow saturates to 65504);
  ``code = clamp(rint_half_even(x / s), -127, 127)`` with an fp32 IEEE
  division; ``s == 0`` gives all-zero codes.  -128 is never produced.
* Values: the same rule per (token, kv head, group of 32 consecutive
  dimensions) with 7 in place of 127 (codes -7..7; nibble 0x8 is never
  produced, a reader decodes it as -8).
* The scale of the keys is fp16 as well (the log line names a single fp16
  scale for the codec).
* Dequantized value = code * scale, exact in fp32 and fp64.

Paged byte layout (the library's own layout; both sides implement it)
---------------------------------------------------------------------
Page size 16 tokens.  For a pool of P physical pages, H kv heads, head
dimension D (64 or 128):

* ``k_codes  [P][H][16][D]``   int8, two's complement, token-major rows.
* ``k_scales [P][H][16]``      fp16 bit patterns (uint16).
* ``v_codes  [P][H][D][8]``    uint8; row d holds the 16 tokens of dimension
  d as nibbles: byte j = (code of slot 2j) & 0xF | ((code of slot 2j+1) & 0xF) << 4,
  two's complement nibbles.
* ``v_scales [P][H][16][D/32]`` fp16 bit patterns (uint16).

Token p of a sequence lives at physical page ``page_table[p // 16]``,
slot ``p % 16``.

Affine variant (the blog's log line calls the codec affine, with 32-wide
groups and an fp16 scale; it gives no formula, so these readings are taken)
-------------------------------------------------------------------------
* Unsigned codes with a zero point: keys 0..255 per (token, kv head), values
  0..15 per (token, kv head, group of 32).
* The block's range is widened to include zero: ``lo = min(min x, 0)``,
  ``hi = max(max x, 0)`` -- zero is then exact and the scale is 0 only for
  an all-zero block.
* ``s = fp16((hi - lo) / qmax)``: fp32 subtraction, fp32 IEEE division, RNE
  into fp16 (65504 on overflow).
* zero point ``z = clamp(rint_half_even(-lo / s), 0, qmax)`` (fp32 division);
  ``code = clamp(rint_half_even(x / s) + z, 0, qmax)``; ``s == 0`` gives
  code 0 and zero point 0.
* Dequantized value = ``(code - z) * s``.
* Stored bytes: key codes ``code XOR 0x80`` (the code minus 128 as int8) in
  ``k_codes``; key zero points ``z XOR 0x80`` in ``k_zeros [P][H][16]``
  (int8); value nibbles hold the unsigned codes; value zero points one byte
  per (token, group) in ``v_zeros [P][H][16][D/32]`` (uint8, 0..15).
"""

from __future__ import annotations

import numpy as np

PAGE_SIZE = 16
K_QMAX = 127
V_QMAX = 7
V_GROUP = 32
FP16_MAX = np.float16(65504.0)


# ---------------------------------------------------------------------------
# input widening
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Inputs arrive either as float32 values or as bfloat16 bit patterns."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# the quantizer
# ---------------------------------------------------------------------------

def fp16_scale(absmax: np.ndarray, qmax: int) -> np.ndarray:
    """fp16 scale for an absmax: fp32 division by qmax, then RNE into fp16,
    saturating an overflow to 65504.  Returns float16 values."""
    a = np.asarray(absmax, dtype=np.float32)
    s32 = (a / np.float32(qmax)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    return np.where(np.isinf(s16), FP16_MAX, s16).astype(np.float16)


def quantize_block(x: np.ndarray, qmax: int):
    """Symmetric absmax quantization of the last axis of ``x`` (float32).

    Returns (codes int8 with the shape of x, scale bits uint16 with the shape
    of x without its last axis)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s16 = fp16_scale(a, qmax)
    s = s16.astype(np.float32)[..., None]
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    r = (x / safe).astype(np.float32)            # fp32 IEEE division
    c = np.clip(np.rint(r), -qmax, qmax)          # numpy rint: half to even
    c = np.where(s == 0, 0, c)
    return c.astype(np.int8), s16.view(np.uint16)


def quantize_k(x: np.ndarray):
    """Key rows ``[..., D]`` -> (int8 codes ``[..., D]``, fp16 scale bits ``[...]``)."""
    return quantize_block(x, K_QMAX)


def quantize_v(x: np.ndarray):
    """Value rows ``[..., D]`` -> (int4 codes as int8 ``[..., D]``,
    fp16 scale bits ``[..., D/32]``)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    if d % V_GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (d // V_GROUP, V_GROUP))
    c, s = quantize_block(g, V_QMAX)
    return c.reshape(x.shape), s


AFFINE_K_QMAX = 255
AFFINE_V_QMAX = 15


def quantize_block_affine(x: np.ndarray, qmax: int):
    """Affine quantization of the last axis of ``x`` (float32), range widened
    to include zero.  Returns (codes uint8 0..qmax with the shape of x, zero
    points uint8 and scale bits uint16 with the shape of x without its last
    axis)."""
    x = np.asarray(x, dtype=np.float32)
    lo = np.minimum(np.min(x, axis=-1), np.float32(0)).astype(np.float32)
    hi = np.maximum(np.max(x, axis=-1), np.float32(0)).astype(np.float32)
    with np.errstate(over="ignore"):
        rng = (hi - lo).astype(np.float32)          # fp32 subtraction
    s16 = fp16_scale(rng, qmax)
    s = s16.astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    z = np.clip(np.rint((-lo / safe).astype(np.float32)), 0, qmax)
    z = np.where(s == 0, 0, z)
    r = (x / safe[..., None]).astype(np.float32)    # fp32 IEEE division
    c = np.clip(np.rint(r) + z[..., None], 0, qmax)
    c = np.where(s[..., None] == 0, 0, c)
    return c.astype(np.uint8), z.astype(np.uint8), s16.view(np.uint16)


def quantize_k_affine(x: np.ndarray):
    """Key rows ``[..., D]`` -> (codes uint8 ``[..., D]``, zero points uint8
    ``[...]``, fp16 scale bits ``[...]``)."""
    return quantize_block_affine(x, AFFINE_K_QMAX)


def quantize_v_affine(x: np.ndarray):
    """Value rows ``[..., D]`` -> (codes uint8 0..15 ``[..., D]``, zero points
    ``[..., D/32]``, fp16 scale bits ``[..., D/32]``)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    if d % V_GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (d // V_GROUP, V_GROUP))
    c, z, s = quantize_block_affine(g, AFFINE_V_QMAX)
    return c.reshape(x.shape), z, s


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequantize_k(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    return codes.astype(np.float64) * fp16_bits_to_f64(scale_bits)[..., None]


def dequantize_v(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    d = codes.shape[-1]
    s = np.repeat(fp16_bits_to_f64(scale_bits), V_GROUP, axis=-1)
    assert s.shape[-1] == d
    return codes.astype(np.float64) * s


def dequantize_k_affine(codes: np.ndarray, zeros: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """(code - z) * s for unsigned key codes ``[..., D]``."""
    return (codes.astype(np.float64) - zeros.astype(np.float64)[..., None]) * fp16_bits_to_f64(scale_bits)[..., None]


def dequantize_v_affine(codes: np.ndarray, zeros: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """(code - z) * s for unsigned value codes ``[..., D]``, per group of 32."""
    z = np.repeat(zeros.astype(np.float64), V_GROUP, axis=-1)
    s = np.repeat(fp16_bits_to_f64(scale_bits), V_GROUP, axis=-1)
    return (codes.astype(np.float64) - z) * s


# ---------------------------------------------------------------------------
# paged cache
# ---------------------------------------------------------------------------

class PagedCache:
    """Four host arrays in the library's byte layout (see module docstring)."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, codec: str = "symmetric"):
        if head_dim not in (64, 128):
            raise ValueError("head_dim must be 64 or 128")
        if codec not in ("symmetric", "affine"):
            raise ValueError("codec must be 'symmetric' or 'affine'")
        P, H, D = num_pages, num_kv_heads, head_dim
        self.num_pages, self.num_kv_heads, self.head_dim = P, H, D
        self.codec = codec
        self.k_codes = np.zeros((P, H, PAGE_SIZE, D), np.int8)
        self.k_scales = np.zeros((P, H, PAGE_SIZE), np.uint16)
        self.v_codes = np.zeros((P, H, D, PAGE_SIZE // 2), np.uint8)
        self.v_scales = np.zeros((P, H, PAGE_SIZE, D // V_GROUP), np.uint16)
        if codec == "affine":
            self.k_zeros = np.zeros((P, H, PAGE_SIZE), np.int8)
            self.v_zeros = np.zeros((P, H, PAGE_SIZE, D // V_GROUP), np.uint8)

    def _arrays(self):
        extra = ("k_zeros", "v_zeros") if self.codec == "affine" else ()
        return ("k_codes", "k_scales", "v_codes", "v_scales") + extra

    def copy(self) -> "PagedCache":
        c = PagedCache.__new__(PagedCache)
        c.num_pages, c.num_kv_heads, c.head_dim = self.num_pages, self.num_kv_heads, self.head_dim
        c.codec = self.codec
        for n in self._arrays():
            setattr(c, n, getattr(self, n).copy())
        return c

    # -- writing -----------------------------------------------------------
    def write_tokens(self, pages: np.ndarray, slots: np.ndarray,
                     k_f32: np.ndarray, v_f32: np.ndarray) -> None:
        """Quantize tokens (``k_f32``/``v_f32`` shaped ``[N][H][D]``) and
        store them at (pages[i], slots[i]).  Every (page, slot) must be
        distinct."""
        pages = np.asarray(pages, np.int64)
        slots = np.asarray(slots, np.int64)
        if self.codec == "affine":
            kc, kz, ks = quantize_k_affine(k_f32)       # [N][H][D], [N][H], [N][H]
            vc, vz, vs = quantize_v_affine(v_f32)       # [N][H][D], [N][H][D/32] x2
            self.k_codes[pages, :, slots, :] = (kc ^ np.uint8(0x80)).view(np.int8)
            self.k_zeros[pages, :, slots] = (kz ^ np.uint8(0x80)).view(np.int8)
            self.v_zeros[pages, :, slots, :] = vz
        else:
            kc, ks = quantize_k(k_f32)          # [N][H][D], [N][H]
            vc, vs = quantize_v(v_f32)          # [N][H][D], [N][H][D/32]
            self.k_codes[pages, :, slots, :] = kc
        self.k_scales[pages, :, slots] = ks
        self.v_scales[pages, :, slots, :] = vs
        nib = (vc.astype(np.int16) & 0xF).astype(np.uint8)   # [N][H][D]
        byte = slots // 2
        for parity in (0, 1):
            sel = (slots % 2) == parity
            if not np.any(sel):
                continue
            p, b, n = pages[sel], byte[sel], nib[sel]          # n: [M][H][D]
            old = self.v_codes[p, :, :, b]                      # [M][H][D]
            if parity == 0:
                new = (old & 0xF0) | n
            else:
                new = (old & 0x0F) | (n << 4)
            self.v_codes[p, :, :, b] = new

    # -- reading -----------------------------------------------------------
    def k_codes_at(self, pages, slots, h):
        return self.k_codes[pages, h, slots, :]

    def v_codes_at(self, pages, slots, h):
        """Value codes ``[N][D]``: two's complement nibbles (symmetric) or
        unsigned 0..15 (affine)."""
        b = self.v_codes[pages, h, :, slots // 2]               # [N][D]
        n = np.where((slots % 2)[:, None] == 0, b & 0xF, b >> 4).astype(np.int16)
        if self.codec == "affine":
            return n.astype(np.uint8)
        return np.where(n >= 8, n - 16, n).astype(np.int8)

    def dequant_tokens(self, pages, slots, h):
        """fp64 K-hat and V-hat rows ``[N][D]`` of kv head h."""
        pages = np.asarray(pages, np.int64)
        slots = np.asarray(slots, np.int64)
        if self.codec == "affine":
            kc = (self.k_codes_at(pages, slots, h).view(np.uint8) ^ np.uint8(0x80))
            kz = (self.k_zeros[pages, h, slots].view(np.uint8) ^ np.uint8(0x80))
            kh = dequantize_k_affine(kc, kz, self.k_scales[pages, h, slots])
            vh = dequantize_v_affine(self.v_codes_at(pages, slots, h), self.v_zeros[pages, h, slots, :],
                                     self.v_scales[pages, h, slots, :])
            return kh, vh
        kh = dequantize_k(self.k_codes_at(pages, slots, h), self.k_scales[pages, h, slots])
        vh = dequantize_v(self.v_codes_at(pages, slots, h), self.v_scales[pages, h, slots, :])
        return kh, vh


def token_locations(page_table_row: np.ndarray, positions: np.ndarray):
    """(physical page, slot) of logical token positions of one sequence."""
    positions = np.asarray(positions, np.int64)
    pages = np.asarray(page_table_row, np.int64)[positions // PAGE_SIZE]
    return pages, positions % PAGE_SIZE


def append(cache: PagedCache, k_new: np.ndarray, v_new: np.ndarray, dtype: str,
           cu_new: np.ndarray, start_pos: np.ndarray, page_table: np.ndarray) -> None:
    """Quantize-and-append: new tokens of sequence b are rows
    ``cu_new[b]:cu_new[b+1]`` of ``k_new``/``v_new`` (``[N][H][D]``) and go to
    logical positions ``start_pos[b] ...`` of that sequence."""
    kf = as_f32(k_new, dtype)
    vf = as_f32(v_new, dtype)
    all_pages, all_slots = [], []
    for b in range(len(start_pos)):
        n = int(cu_new[b + 1] - cu_new[b])
        if n == 0:
            continue
        pos = int(start_pos[b]) + np.arange(n)
        p, s = token_locations(page_table[b], pos)
        all_pages.append(p)
        all_slots.append(s)
    if not all_pages:
        return
    pages = np.concatenate(all_pages)
    slots = np.concatenate(all_slots)
    rows = np.concatenate([np.arange(cu_new[b], cu_new[b + 1]) for b in range(len(start_pos))])
    cache.write_tokens(pages, slots, kf[rows], vf[rows])
