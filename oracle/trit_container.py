""".trit v1 container reader and writer of the oracle - TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the product path never does and shares no code with it.

Written from "The .trit format, version 1": section 2 "File layout" (header fields, 2.1), 2.2
"Tensor record", 2.3 "Ternary payload", 2.4 "Dense payload", section 4 "Validation" (checks 1-19)
and section 6 "What a reader is allowed to assume". Plain Python, one field at a time.

Readings where the page leaves a step open (each is also listed in the design notes):
  - Order. Fields are read in file order and each is checked as soon as it has been read; a field
    that would extend past the end of the file is check 5. So the first failure in file order is
    the one reported. Within a record: name_len, name (+ duplicate), dtype, ndim, reserved0,
    reserved1, dims, shape product, scale, flags, offset, byte_len, then checks 14, 15/16. After
    all records the payload start is the next multiple of 64 (past the end: check 5); then check 12
    per record in record order, then check 13 over the extents sorted by offset.
  - tensor_count above 1,048,576 and a name that is not valid UTF-8 are reported as check 7 (the
    tensor-table limits); the page lists the limit and the encoding but gives them no number.
  - The padding between the last record and payload_start is not checked.
  - The shape product (check 9) is the product of the dims in 64 bits, and for the byte count also
    the product times the element size (dense) or rows * beats_per_row * 16 (ternary).
  - A scale is any float32 bit pattern that is finite and > 0; dense tensors are not required to
    store exactly 1.0.
  - Verification: for each ternary tensor in record order, beats in row-major order, P1 before P2
    within a beat (check 17 names tensor, row, beat, column; check 18 tensor, row, beat and the
    first set padding column); then check 19: FNV-1a-64 over every byte from payload_start to the
    end of the file, compared when the stored hash is not 0.
"""
from __future__ import annotations

import math
import struct

MAGIC = b"TRIT"
MAX_CONFIG = 16 * 1024 * 1024
MAX_TENSORS = 1048576
MAX_NAME = 1024
F32, TRIT, BF16 = 0, 1, 2
ELEM_SIZE = {F32: 4, BF16: 2}
U64 = (1 << 64) - 1

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit (Fowler, Noll, Vo): h = offset basis; per byte: h ^= byte, h *= prime."""
    h = FNV_OFFSET
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & U64
    return h


class TritError(Exception):
    """A failed check of section 4, numbered as there (1..19)."""

    def __init__(self, check: int, offset: int = -1, tensor: int = -1, row: int = -1, beat: int = -1,
                 col: int = -1):
        super().__init__(f"check {check} (offset {offset}, tensor {tensor}, row {row}, beat {beat}, col {col})")
        self.check, self.offset, self.tensor = check, offset, tensor
        self.row, self.beat, self.col = row, beat, col


class Tensor:
    def __init__(self, name, dtype, dims, scale, offset, byte_len):
        self.name, self.dtype, self.dims, self.scale = name, dtype, dims, scale
        self.offset, self.byte_len = offset, byte_len


class _Reader:
    def __init__(self, data: bytes):
        self.data, self.pos = data, 0

    def take(self, n: int) -> bytes:
        if self.pos + n > len(self.data):
            raise TritError(5, offset=self.pos)
        b = self.data[self.pos:self.pos + n]
        self.pos += n
        return b

    def u8(self):
        return self.take(1)[0]

    def u16(self):
        return struct.unpack("<H", self.take(2))[0]

    def u32(self):
        return struct.unpack("<I", self.take(4))[0]

    def u64(self):
        return struct.unpack("<Q", self.take(8))[0]

    def f32(self):
        return struct.unpack("<f", self.take(4))[0]


def _utf8_ok(b: bytes) -> bool:
    try:
        b.decode("utf-8", errors="strict")
        return True
    except UnicodeDecodeError:
        return False


class TritFile:
    """A container that passed checks 1-16."""

    def __init__(self, data: bytes):
        self.data = bytes(data)
        r = _Reader(self.data)
        if r.take(4) != MAGIC:
            raise TritError(1, offset=0)
        at = r.pos
        version = r.u32()
        if version == 0:
            raise TritError(2, offset=at)
        if version > 1:
            raise TritError(3, offset=at)
        at = r.pos
        if r.u32() != 0:
            raise TritError(4, offset=at)
        self.payload_hash = r.u64()
        at = r.pos
        config_len = r.u32()
        if config_len > MAX_CONFIG:
            raise TritError(6, offset=at)
        at = r.pos
        self.config = r.take(config_len)
        if not _utf8_ok(self.config):
            raise TritError(6, offset=at)
        at = r.pos
        count = r.u32()
        if count > MAX_TENSORS:
            raise TritError(7, offset=at)
        self.tensors: list[Tensor] = []
        names = set()
        for i in range(count):
            at = r.pos
            name_len = r.u16()
            if name_len == 0 or name_len > MAX_NAME:
                raise TritError(7, offset=at, tensor=i)
            at = r.pos
            name = r.take(name_len)
            if not _utf8_ok(name) or name in names:
                raise TritError(7, offset=at, tensor=i)
            names.add(name)
            at = r.pos
            dtype = r.u8()
            if dtype not in (F32, TRIT, BF16):
                raise TritError(8, offset=at, tensor=i)
            at = r.pos
            ndim = r.u8()
            if ndim < 1 or ndim > 4:
                raise TritError(8, offset=at, tensor=i)
            for _ in range(2):
                at = r.pos
                if r.u8() != 0:
                    raise TritError(8, offset=at, tensor=i)
            at = r.pos
            dims = [r.u32() for _ in range(ndim)]
            prod = 1
            for d in dims:
                prod *= d
            if prod > U64:
                raise TritError(9, offset=at, tensor=i)
            at = r.pos
            scale = r.f32()
            if not math.isfinite(scale) or not scale > 0.0:
                raise TritError(10, offset=at, tensor=i)
            at = r.pos
            if r.u32() != 0:
                raise TritError(8, offset=at, tensor=i)
            at = r.pos
            offset = r.u64()
            if offset % 64 != 0:
                raise TritError(11, offset=at, tensor=i)
            at = r.pos
            byte_len = r.u64()
            if dtype == TRIT:
                if ndim != 2:
                    raise TritError(14, offset=at, tensor=i)
                rows, cols = dims
                expect = rows * ((cols + 63) // 64) * 16
                if expect > U64:
                    raise TritError(9, offset=at, tensor=i)
                if byte_len != expect:
                    raise TritError(15, offset=at, tensor=i)
            else:
                expect = prod * ELEM_SIZE[dtype]
                if expect > U64:
                    raise TritError(9, offset=at, tensor=i)
                if byte_len != expect:
                    raise TritError(16, offset=at, tensor=i)
            self.tensors.append(Tensor(name, dtype, dims, scale, offset, byte_len))
        self.payload_start = (r.pos + 63) // 64 * 64
        if self.payload_start > len(self.data):
            raise TritError(5, offset=r.pos)
        payload_len = len(self.data) - self.payload_start
        for i, t in enumerate(self.tensors):
            if t.offset + t.byte_len > payload_len:
                raise TritError(12, tensor=i)
        order = sorted(range(len(self.tensors)), key=lambda i: (self.tensors[i].offset, i))
        end, last = 0, -1
        for i in order:
            t = self.tensors[i]
            if t.byte_len == 0:
                continue
            if last >= 0 and t.offset < end:
                raise TritError(13, tensor=i)
            end, last = t.offset + t.byte_len, i

    def payload(self, i: int) -> bytes:
        t = self.tensors[i]
        return self.data[self.payload_start + t.offset:self.payload_start + t.offset + t.byte_len]

    def verify(self, check_hash: bool = True) -> None:
        for i, t in enumerate(self.tensors):
            if t.dtype != TRIT:
                continue
            rows, cols = t.dims
            bpr = (cols + 63) // 64
            p = self.payload(i)
            tail = (1 << 64) - 1 if cols % 64 == 0 else (1 << (cols % 64)) - 1
            for r in range(rows):
                for b in range(bpr):
                    o = (r * bpr + b) * 16
                    pos = int.from_bytes(p[o:o + 8], "little")
                    neg = int.from_bytes(p[o + 8:o + 16], "little")
                    both = pos & neg
                    if both:
                        k = (both & -both).bit_length() - 1
                        raise TritError(17, tensor=i, row=r, beat=b, col=64 * b + k)
                    if b == bpr - 1:
                        pad = (pos | neg) & ~tail & ((1 << 64) - 1)
                        if pad:
                            k = (pad & -pad).bit_length() - 1
                            raise TritError(18, tensor=i, row=r, beat=b, col=64 * b + k)
        if check_hash and self.payload_hash != 0:
            if fnv1a64(self.data[self.payload_start:]) != self.payload_hash:
                raise TritError(19)


def write(config: bytes, tensors: list[tuple], with_hash: bool = True) -> bytes:
    """A valid container: tensors = [(name (str), dtype, dims, scale, payload bytes)], written sorted by
    name, each payload at the next multiple of 64 after the previous one and the file ending with the
    last payload (section 2.2: sorted names; section 2: aligned payload_start and offsets)."""
    tensors = sorted(tensors, key=lambda t: t[0].encode("utf-8"))
    offs, off, end = [], 0, 0
    for name, dtype, dims, scale, data in tensors:
        offs.append(off)
        end = off + len(data)
        off = (end + 63) // 64 * 64
    head = bytearray()
    for (name, dtype, dims, scale, data), o in zip(tensors, offs):
        nb = name.encode("utf-8")
        head += struct.pack("<H", len(nb)) + nb + bytes([dtype, len(dims), 0, 0])
        head += b"".join(struct.pack("<I", d) for d in dims)
        head += struct.pack("<fIQQ", scale, 0, o, len(data))
    body = bytearray(end)  # the file ends with the last tensor's bytes
    for (name, dtype, dims, scale, data), o in zip(tensors, offs):
        body[o:o + len(data)] = data
    pre = MAGIC + struct.pack("<II", 1, 0)
    cfg = struct.pack("<I", len(config)) + config + struct.pack("<I", len(tensors))
    start = len(pre) + 8 + len(cfg) + len(head)
    pad = (-start) % 64
    h = fnv1a64(bytes(body)) if with_hash else 0
    return bytes(pre + struct.pack("<Q", h) + cfg + head + bytes(pad) + body)
