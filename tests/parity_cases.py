"""Small GPU parity cases (shapes only; the tests draw the values).

Together they reach every kernel instantiation the library builds: bf16 with
head dim 64 and 128, fp32 with head dim 64, each at GQA group sizes 1, 2, 4
and 8.  Each case spans several prefill tiles and ragged tails; decode
lengths hit page and split boundaries (1, 15, 16, 17, ...)."""


def spec(dtype, hq, hkv, d, C, P0, lens, outliers=0.0, contiguous=False):
    return dict(name=f"{dtype}_h{hq}x{hkv}_d{d}_C{C}_P{P0}", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                head_dim=d, chunk_len=C, chunk_offset=P0, decode_lens=list(lens), contiguous=contiguous,
                k_outlier_frac=outliers)


SMALL = [
    spec("bf16", 8, 2, 128, 77, 300, [1, 15, 16, 17, 300, 1023, 1025, 2100]),
    spec("bf16", 16, 2, 128, 40, 0, [5, 64, 2000], outliers=0.02),
    spec("bf16", 4, 4, 128, 100, 45, [2, 33, 511, 3000]),
    spec("bf16", 4, 2, 128, 129, 1000, [16, 17, 4097, 260]),
    spec("bf16", 4, 4, 64, 130, 17, [33, 700]),
    spec("bf16", 8, 4, 64, 1, 5000, [1, 4096]),
    spec("bf16", 8, 2, 64, 95, 2047, [1, 31, 32, 1500, 6000], outliers=0.01),
    spec("bf16", 16, 2, 64, 33, 7, [3, 257, 999]),
    spec("bf16", 8, 2, 128, 64, 12000, [20000]),           # prefill and decode splits + merges
    spec("f32", 8, 2, 64, 100, 29, [3, 999]),
    spec("f32", 2, 2, 64, 64, 2000, [1500, 1]),
    spec("f32", 4, 2, 64, 67, 500, [2, 64, 65, 1300]),
    spec("f32", 16, 2, 64, 70, 3000, [4000, 17]),
]


def instantiation(sp):
    """(dtype, head dim, group size) of a case."""
    return sp["dtype"], sp["head_dim"], sp["num_q_heads"] // sp["num_kv_heads"]
