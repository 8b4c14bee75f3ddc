"""The byte models behind bench.py's roofline figures (CPU only), pinned to
hand-counted values for the gene workload: the compulsory bytes that
roofline.achieved divides by the edge kernel's time, and the gather model
reported beside it."""
import bench


def test_compulsory_bytes_of_the_gene_edge_launch():
    # B = 32, L = 20,000, E = 64, bf16 (2 bytes); 8,096 read sources,
    # 196,614 edges, 20,033 pieces:
    #   query rows in + output rows out: 32 * 20,000 * 2 * 64 * 2 = 163,840,000
    #   key and value rows of read sources: 32 * 8,096 * 2 * 64 * 2 = 66,322,432
    #   gather index: 196,614 * 4 = 786,456; pieces: 20,033 * 16 = 320,528
    assert bench.edge_kernel_bytes(32, 20000, 8096, 196614, 20033, 64, 2) == \
        163_840_000 + 66_322_432 + 786_456 + 320_528


def test_compulsory_bytes_with_weights():
    # per (edge, sample, head) a 4-byte score, per (target, sample, head) 8
    # bytes of (max, sum): bipartite B = 16, L = 2,000, H = 8, fp32
    base = bench.edge_kernel_bytes(16, 2000, 20000, 215596, 2000, 128, 4)
    full = bench.edge_kernel_bytes(16, 2000, 20000, 215596, 2000, 128, 4, weights=True, H=8)
    assert full - base == 4 * 16 * 215596 * 8 + 8 * 16 * 2000 * 8


def test_gather_model_of_the_gene_workload():
    # every edge's key and value rows per sample, plus query and output rows
    # and the index: the survey's model, 1,775,368,348 bytes for gene
    g = bench.edge_gather_bytes(32, 20000, 196614, 64, 2)
    assert g == 32 * (20000 * 128 + 196614 * 256 + 20000 * 128) + 4 * 20001 + 4 * 196614
    assert g == 1_775_368_348


def test_compulsory_bytes_with_a_key_padding_mask():
    # one 32-bit mask word per edge position and 32 samples: gene B = 32
    # needs one word per edge, 70 samples three
    base = bench.edge_kernel_bytes(32, 20000, 8096, 196614, 20033, 64, 2)
    masked = bench.edge_kernel_bytes(32, 20000, 8096, 196614, 20033, 64, 2, masked=True)
    assert masked - base == 196614 * 4
    b70 = bench.edge_kernel_bytes(70, 10, 10, 100, 10, 64, 2, masked=True) - \
        bench.edge_kernel_bytes(70, 10, 10, 100, 10, 64, 2)
    assert b70 == 100 * 4 * 3
