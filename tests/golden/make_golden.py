"""Writes the hand-derived golden fixtures in this folder.

Every value below is a closed form worked out by hand from the definitions on
the pages (the derivation is stored with each fixture); nothing is computed by
the oracle or by the HIP library. Run: python tests/golden/make_golden.py
"""
import json
import math
import os

LN2, LN3, LN4 = math.log(2.0), math.log(3.0), math.log(4.0)

FIXTURES = {
    "attend_basic.json": {
        "citation": "memra-engine 0.124.1 tests/mla_gpu_forward.rs, gate 1 (absorbed oracle): "
                    "softmax attention of the folded query over latent rows; hand-derived",
        "derivation": "scale 1, one head, L=2, R=1. scores = q.kv_j = [ln 3, 0]; softmax = "
                      "[3/4, 1/4]; o_lat = 3/4*[1,0] + 1/4*[0,1]; lse = ln(3+1) = ln 4",
        "L": 2, "scale": 1.0, "causal": False,
        "q": [[[LN3, 0.0, 0.0]]], "pos": [1],
        "kv": [[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]],
        "o_lat": [[[0.75, 0.25]]], "lse": [[LN4]]},
    "attend_rope.json": {
        "citation": "vLLM test_mla_cross_layer_kernel_equivalence.py, "
                    "test_flashattn_mla_dense_decode_unified_slot_view: the score is "
                    "q_pe.k_pe + q_nope.kv_c and the output is P.kv_c; hand-derived",
        "derivation": "q = [0,0 | 1]: only the rope column scores. scores = [ln 2, 0]; softmax = "
                      "[2/3, 1/3]; o_lat = 2/3*[2,4] + 1/3*[6,8] = [10/3, 16/3] (k_pe is not "
                      "part of the value); lse = ln 3",
        "L": 2, "scale": 1.0, "causal": False,
        "q": [[[0.0, 0.0, 1.0]]], "pos": [1],
        "kv": [[2.0, 4.0, LN2], [6.0, 8.0, 0.0]],
        "o_lat": [[[10.0 / 3.0, 16.0 / 3.0]]], "lse": [[LN3]]},
    "attend_causal.json": {
        "citation": "memra-engine 0.124.1 tests/mla_gpu_forward.rs, gate 1 chunked shape and "
                    "gate 2: queries are a suffix of the cache, query i at position "
                    "t_kv - t_q + i sees keys 0..pos; hand-derived",
        "derivation": "q = 0 so every visible key scores 0 and the output is the mean of the "
                      "visible rows. t_kv=3, t_q=2: query 0 at pos 1 sees rows 0,1 -> [1.5,1.5], "
                      "lse ln 2; query 1 at pos 2 sees rows 0..2 -> [3,3], lse ln 3",
        "L": 2, "scale": 0.5, "causal": True,
        "q": [[[0.0, 0.0]], [[0.0, 0.0]]], "pos": [1, 2],
        "kv": [[3.0, 0.0], [0.0, 3.0], [6.0, 6.0]],
        "o_lat": [[[1.5, 1.5]], [[3.0, 3.0]]], "lse": [[LN2], [LN3]]},
    "naive.json": {
        "citation": "memra-engine 0.124.1 tests/mla_gpu_forward.rs, naive oracle (decompress K "
                    "and V per head from c_kv); vllm.cpp test_ops_mla_absorb.cpp W_UK_T [N,P,L] "
                    "and W_UV [N,L,V] shapes; hand-derived",
        "derivation": "N=1, P=1, L=2, R=0, V=1, scale 1. k_nope_j = W_UK_T[0,0,:].c_kv_j = "
                      "[ln 3, 0]; scores = q_nope*k_nope = [ln 3, 0]; p = [3/4, 1/4]; v_j = "
                      "c_kv_j.W_UV[0,:,0] = [4, 8]; out = 3/4*4 + 1/4*8 = 5",
        "scale": 1.0, "causal": False, "pos": [1],
        "q_nope": [[[1.0]]], "c_kv": [[1.0, 0.0], [0.0, 1.0]],
        "w_uk_t": [[[LN3, 0.0]]], "w_uv": [[[4.0], [8.0]]],
        "out": [[[5.0]]]},
    "merge.json": {
        "citation": "vLLM test_mla_cross_layer_kernel_equivalence.py, "
                    "test_flashmla_dense_decode_unified_slot_view: split-KV decode (num_splits) "
                    "returning (out, lse); merge by log-sum-exp weights; hand-derived",
        "derivation": "split 0 = key 0 alone: o0 = [1,0], lse0 = ln 3; split 1 = key 1: "
                      "o1 = [0,1], lse1 = 0. lse = ln(3+1); o = 3/4*o0 + 1/4*o1 = [0.75, 0.25]",
        "L": 2, "scale": 1.0, "causal": False,
        "q": [[[LN3, 0.0]]], "pos": [1], "bounds": [0, 1, 2],
        "kv": [[1.0, 0.0], [0.0, 1.0]],
        "o_lat": [[[0.75, 0.25]]], "lse": [[LN4]]},
    "bmm.json": {
        "citation": "vllm.cpp test_ops_mla_absorb.cpp, the double-precision bmm reference: "
                    "out[g,m,n] = sum_k a[g,m,k] b[g,k,n]; hand-computed products",
        "derivation": "[[1,2],[3,4]] x [[5,6],[7,8]] = [[19,22],[43,50]]; identity x B = B",
        "a": [[[1.0, 2.0], [3.0, 4.0]], [[1.0, 0.0], [0.0, 1.0]]],
        "b": [[[5.0, 6.0], [7.0, 8.0]], [[2.0, 3.0], [4.0, 5.0]]],
        "out": [[[19.0, 22.0], [43.0, 50.0]], [[2.0, 3.0], [4.0, 5.0]]]},
    "cache_write.json": {
        "citation": "vLLM test_mla_cross_layer_kernel_equivalence.py, "
                    "test_concat_and_cache_mla_into_unified_slot_view: row [kv_c | k_pe] lands "
                    "at slot = block*page + offset of a strided per-layer view, neighbours "
                    "untouched; hand-derived image",
        "derivation": "NB=2, page=2, L=2, R=1 (entry 3), 2 layers per block, layer 1 viewed: "
                      "s0 = 2*2*3 = 12, s1 = 3, offset = 6. slot 3 -> block 1 row 1 -> elements "
                      "6+12+3..6+12+5 = 21..23 <- [1,2,7]; slot 0 -> elements 6..8 <- [3,4,8]; "
                      "slot -1 skipped",
        "num_blocks": 2, "page": 2, "s0": 12, "s1": 3, "offset": 6, "buf_elems": 24,
        "kv_c": [[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]], "k_pe": [[7.0], [8.0], [9.0]],
        "slots": [3, 0, -1],
        "buf": [0, 0, 0, 0, 0, 0, 3, 4, 8, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 2, 7]},
}

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for name, d in FIXTURES.items():
        with open(os.path.join(here, name), "w") as f:
            json.dump(d, f, indent=1)
    print("wrote", len(FIXTURES), "fixtures")
