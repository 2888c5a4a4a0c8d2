"""Re-encoding of packed weight codes between the int2, int4 and int8 layouts
(test helpers, numpy and torch).

Layouts (two's-complement codes, row-major rows of in_dim codes):
  int8  one code per byte;
  int4  two per byte, element 2m in the low nibble of byte m;
  int2  four per byte, element 4m+i in bits 2i..2i+1 of byte m.
The same code values in two layouts must give identical integer block dots,
so the layer computes the same result from either encoding."""
import numpy as np


def unpack(packed, wbits):
    """[..., in_dim * wbits / 8] uint8 -> [..., in_dim] int8 codes."""
    b = np.asarray(packed, np.uint8)
    if wbits == 8:
        return b.view(np.int8)
    per = 8 // wbits
    mask, sign = (1 << wbits) - 1, 1 << (wbits - 1)
    fields = [((b >> (wbits * i)) & mask).astype(np.int16) for i in range(per)]
    c = np.stack([(f ^ sign) - sign for f in fields], axis=-1)
    return c.reshape(*b.shape[:-1], b.shape[-1] * per).astype(np.int8)


def pack(codes, wbits):
    """[..., in_dim] int8 codes (in range for wbits) -> packed uint8 rows."""
    c = np.asarray(codes, np.int8)
    lo, hi = -(1 << (wbits - 1)), (1 << (wbits - 1)) - 1
    assert c.min() >= lo and c.max() <= hi, "codes out of range for int%d" % wbits
    if wbits == 8:
        return c.view(np.uint8)
    per = 8 // wbits
    mask = (1 << wbits) - 1
    f = (c.astype(np.int16) & mask).reshape(*c.shape[:-1], c.shape[-1] // per, per)
    out = np.zeros(f.shape[:-1], np.uint8)
    for i in range(per):
        out |= (f[..., i] << (wbits * i)).astype(np.uint8)
    return out


def reencode(packed, wfrom, wto):
    return pack(unpack(packed, wfrom), wto)


def unpack_torch(packed, wbits):
    """torch version of unpack (on any device)."""
    import torch
    if wbits == 8:
        return packed.view(torch.int8)
    per = 8 // wbits
    mask, sign = (1 << wbits) - 1, 1 << (wbits - 1)
    b = packed.to(torch.int16)
    c = torch.stack([(((b >> (wbits * i)) & mask) ^ sign) - sign for i in range(per)], dim=-1)
    return c.reshape(*packed.shape[:-1], packed.shape[-1] * per).to(torch.int8)


def pack_torch(codes, wbits):
    import torch
    if wbits == 8:
        return codes.contiguous().view(torch.uint8)
    per = 8 // wbits
    mask = (1 << wbits) - 1
    f = (codes.to(torch.int16) & mask).reshape(*codes.shape[:-1], codes.shape[-1] // per, per)
    out = torch.zeros(f.shape[:-1], dtype=torch.int16, device=codes.device)
    for i in range(per):
        out |= f[..., i] << (wbits * i)
    return out.to(torch.uint8)


def reencode_torch(packed, wfrom, wto):
    return pack_torch(unpack_torch(packed, wfrom), wto)
