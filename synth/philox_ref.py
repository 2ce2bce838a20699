"""Pure-Python Philox4x32-10 (Salmon et al., SC'11), a twin of the C generator.

Used only to check that the C implementation and an independent transcription
agree bit for bit on small streams.
"""
M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    c = [int(x) & MASK for x in ctr]
    k0, k1 = int(key[0]) & MASK, int(key[1]) & MASK
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c[3] ^ k1) & MASK, p0 & MASK]
    return c


def uniform_u24(seed, i):
    """Verifier uniform number i of a seed: (2k+1) 2^-24, k = word >> 9."""
    w = philox4x32_10((i // 4, 0, 0, 0), (seed, 0))[i % 4]
    return (2 * (w >> 9) + 1) * 2.0 ** -24
