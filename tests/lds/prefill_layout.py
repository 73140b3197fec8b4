"""The LDS accesses of the chunked prefill kernels, restated from the address
arithmetic of csrc/gdn_prefill.hip, csrc/kda_prefill.hip and
csrc/prefill_common.hpp (d_k = 128: rows of 256 bytes, 16-byte chunks),
for the bank model in bank_model.py.  Each generator yields the 64 lane byte
addresses of one access, relative to its plane."""
from .bank_model import RD16, RDTR, WR16


def slot(i):
    """Storage slot of contraction index i (index 16h + 4g + j of each block
    of 32 sits at 8g + 4h + j)."""
    return (i & ~31) | (((i >> 2) & 3) << 3) | (((i >> 4) & 1) << 2) | (i & 3)


def swz_rows(r):
    """Chunk swizzle of K / Q rows (QkRow<128>)."""
    return ((r & 3) << 2) | (((r >> 3) & 1) << 1)


def qk_byte(r, sl, swz=swz_rows, dk=128):
    return 2 * (r * dk + (((sl >> 3) ^ swz(r % 16)) << 3) + (sl & 7))


def operand_reads(swz=swz_rows):
    """MFMA operand reads of K / Q rows: lane 16 g + r reads row 16 tb + r,
    slots 32 s + 8 g (16 bytes)."""
    for tb in range(2):
        for s in range(4):
            yield RD16, [qk_byte(16 * tb + (l & 15), 32 * s + 8 * (l >> 4), swz) for l in range(64)]


def transposing_reads(swz=swz_rows):
    """Transposing reads of K rows for the state update: lane 16 g + r reads
    row 16 hf + 4 g + r / 4, slots 32 (d / 2) + 8 (r % 4) + 4 (d % 2)."""
    for d in range(8):
        for hf in range(2):
            yield RDTR, [qk_byte(16 * hf + 4 * (l >> 4) + ((l & 15) >> 2),
                                 32 * (d >> 1) + 8 * (l & 3) + 4 * (d & 1), swz) for l in range(64)]


def scalar_piece_stores(swz=swz_rows):
    """Producers' 16-byte copies of prepared rows (scalar decay): lane l of
    wave w writes chunk l % 16 of row w + 4 i (one plane per 16 lanes)."""
    plane = 2 * 32 * 128 + 64
    for w in range(4):
        for i in range(8):
            yield WR16, [((l >> 4) ^ 2) * plane + qk_byte(w + 4 * i, 8 * (l & 15), swz) for l in range(64)]


def kda_row_stores(swz=swz_rows):
    """Per-channel-decay producers' row stores: thread t = 64 w + l holds
    octet (t % 32) % 16 (the channels of storage chunk oc) of q (t % 32 < 16)
    or k, tokens 8 (t / 32) + tt."""
    plane = 2 * 64 * 128 + 64
    for w in range(4):
        for tt in range(8):
            ad = []
            for l in range(64):
                t = 64 * w + l
                co, tau = t % 32, t // 32
                ad.append((0 if co >= 16 else 2) * plane + qk_byte(8 * tau + tt, 8 * (co % 16), swz))
            yield WR16, ad
