"""Writes worked_examples.json: hand-derived closed-form attention examples.

The pages print no attention input/output values, so these fixtures pin the
oracle to closed forms instead.  Each expected value below is derived by
hand from softmax(scale * q.k + mask) . v with the causal bound
kv_end = min(q_pos + 1, seq_len) (atlas PR #69, fused MLA prefill re-audit
commits) and a window of the W most recent keys (m40-llm AGENTS.md,
"Current Progress", exact recent ring; 0 = off per the atlas PR #69
cache-skip MLA fix).  Only the math module computes them; the oracle is not
called.  Run:  python tests/golden/make_golden.py
"""
import json
import math
import os

LN2, LN3, LN4, LN5, LN9 = (math.log(x) for x in (2, 3, 4, 5, 9))
E7 = math.exp(7.0)


def ex(name, why, cu, hq, hkv, scale, window, q, k, v, out):
    return {"name": name, "derivation": why, "cu_seqlens": cu,
            "n_q_heads": hq, "n_kv_heads": hkv, "scale": scale,
            "window": window, "q": q, "k": k, "v": v, "out": out}


EXAMPLES = [
    ex("two_token",
       "row 0 sees key 0 only -> v0 = 0; row 1 scores [0, ln3] -> "
       "weights [1/4, 3/4] -> 3/4",
       [0, 2], 1, 1, 1.0, 0,
       [[[0.0]], [[1.0]]], [[[0.0]], [[LN3]]], [[[0.0]], [[1.0]]],
       [[[0.0]], [[0.75]]]),
    ex("two_token_negative_scale",
       "scale -1: row 1 scores [0, -ln3] -> weights [3/4, 1/4] -> 1/4",
       [0, 2], 1, 1, -1.0, 0,
       [[[0.0]], [[1.0]]], [[[0.0]], [[LN3]]], [[[0.0]], [[1.0]]],
       [[[0.0]], [[0.25]]]),
    ex("scale_half",
       "scale 1/2, q1 = 2: row 1 scores [0, ln9] -> [1/10, 9/10] -> "
       "0.3 + 6.3 = 6.6",
       [0, 2], 1, 1, 0.5, 0,
       [[[0.0]], [[2.0]]], [[[0.0]], [[LN9]]], [[[3.0]], [[7.0]]],
       [[[3.0]], [[6.6]]]),
    ex("three_token_window2",
       "W=2: row 0 -> v0 = 10; row 1 keys {0,1} scores [7, 0] -> "
       "(10 e^7 + 20)/(e^7 + 1); row 2 keys {1,2} scores [0, ln2] -> "
       "(20 + 2*50)/3 = 40",
       [0, 3], 1, 1, 1.0, 2,
       [[[1.0]], [[1.0]], [[1.0]]], [[[7.0]], [[0.0]], [[LN2]]],
       [[[10.0]], [[20.0]], [[50.0]]],
       [[[10.0]], [[(10 * E7 + 20) / (E7 + 1)]], [[40.0]]]),
    ex("three_token_full",
       "W=0: row 2 keys {0,1,2} scores [7, 0, ln2] -> "
       "(10 e^7 + 20 + 100)/(e^7 + 3)",
       [0, 3], 1, 1, 1.0, 0,
       [[[1.0]], [[1.0]], [[1.0]]], [[[7.0]], [[0.0]], [[LN2]]],
       [[[10.0]], [[20.0]], [[50.0]]],
       [[[10.0]], [[(10 * E7 + 20) / (E7 + 1)]],
        [[(10 * E7 + 20 + 100) / (E7 + 3)]]]),
    ex("gqa_two_heads_d2",
       "one KV head, 2 Q heads, d=2, k rows e0 and e1, v = k: head 0 row 1 "
       "scores [ln2, 0] -> [2/3, 1/3]; head 1 row 1 scores [0, ln5] -> "
       "[1/6, 5/6]; row 0 -> v0 for both heads",
       [0, 2], 2, 1, 1.0, 0,
       [[[3.0, -1.0], [0.5, 0.25]], [[LN2, 0.0], [0.0, LN5]]],
       [[[1.0, 0.0]], [[0.0, 1.0]]],
       [[[1.0, 0.0]], [[0.0, 1.0]]],
       [[[1.0, 0.0], [1.0, 0.0]], [[2 / 3, 1 / 3], [1 / 6, 5 / 6]]]),
    ex("gqa_grouping_4q2kv",
       "4 Q heads over 2 KV heads, one token: heads 0,1 read KV head 0 "
       "(v = 1), heads 2,3 read KV head 1 (v = 2)",
       [0, 1], 4, 2, 1.0, 0,
       [[[0.3], [-0.2], [0.9], [1.7]]], [[[0.5], [-4.0]]], [[[1.0], [2.0]]],
       [[[1.0], [1.0], [2.0], [2.0]]]),
    ex("two_sequences_isolated",
       "cu = [0,1,3]: sequence 0 is one token -> v = 9; sequence 1 row 0 "
       "sees only its own key -> 2 (the score-100 key of sequence 0 is not "
       "visible); row 1 scores [0, ln4] -> (2 + 4*7)/5 = 6",
       [0, 1, 3], 1, 1, 1.0, 0,
       [[[5.0]], [[1.0]], [[1.0]]], [[[100.0]], [[0.0]], [[LN4]]],
       [[[9.0]], [[2.0]], [[7.0]]],
       [[[9.0]], [[2.0]], [[6.0]]]),
    ex("empty_sequence_between",
       "cu = [0,2,2,3]: an empty sequence contributes nothing; the last "
       "token is a one-token sequence -> its own v = -3",
       [0, 2, 2, 3], 1, 1, 1.0, 0,
       [[[0.0]], [[1.0]], [[2.0]]], [[[0.0]], [[LN3]], [[50.0]]],
       [[[0.0]], [[1.0]], [[-3.0]]],
       [[[0.0]], [[0.75]], [[-3.0]]]),
]

# Chunked prefill against a KV history: the queries are the last Lq of the
# sequence's Lk positions, so a later chunk sees every earlier token (the
# multi-chunk fix of atlas PR #69: kv_len = seq_len_start + n).


def exk(name, why, cu_q, cu_k, hq, hkv, scale, window, q, k, v, out):
    e = ex(name, why, cu_q, hq, hkv, scale, window, q, k, v, out)
    e["cu_seqlens_k"] = cu_k
    return e


EXAMPLES += [
    exk("history2_one_query",
        "Lk=3, Lq=1: the query sits at position 2 and sees keys {0,1,2}, "
        "scores [7, 0, ln2] -> (10 e^7 + 20 + 100)/(e^7 + 3)",
        [0, 1], [0, 3], 1, 1, 1.0, 0,
        [[[1.0]]], [[[7.0]], [[0.0]], [[LN2]]],
        [[[10.0]], [[20.0]], [[50.0]]],
        [[[(10 * E7 + 20 + 100) / (E7 + 3)]]]),
    exk("history2_one_query_window2",
        "Lk=3, Lq=1, W=2: position 2 sees keys {1,2}, scores [0, ln2] -> "
        "(20 + 2*50)/3 = 40",
        [0, 1], [0, 3], 1, 1, 1.0, 2,
        [[[1.0]]], [[[7.0]], [[0.0]], [[LN2]]],
        [[[10.0]], [[20.0]], [[50.0]]],
        [[[40.0]]]),
    exk("history1_chunk2",
        "Lk=3, Lq=2: queries at positions 1 and 2; row 0 keys {0,1} scores "
        "[7, 0] -> (10 e^7 + 20)/(e^7 + 1); row 1 keys {0,1,2} -> "
        "(10 e^7 + 120)/(e^7 + 3)",
        [0, 2], [0, 3], 1, 1, 1.0, 0,
        [[[1.0]], [[1.0]]], [[[7.0]], [[0.0]], [[LN2]]],
        [[[10.0]], [[20.0]], [[50.0]]],
        [[[(10 * E7 + 20) / (E7 + 1)]], [[(10 * E7 + 120) / (E7 + 3)]]]),
    exk("two_sequences_with_history",
        "cu_q = [0,1,2], cu_k = [0,2,3]: sequence 0's query is position 1 "
        "with scores [0, ln3] -> 3/4; sequence 1 has no history, its query "
        "sees only its own key -> 2 (the score-100 key of sequence 0 is not "
        "visible)",
        [0, 1, 2], [0, 2, 3], 1, 1, 1.0, 0,
        [[[1.0]], [[1.0]]], [[[0.0]], [[LN3]], [[0.0]]],
        [[[0.0]], [[1.0]], [[2.0]]],
        [[[0.75]], [[2.0]]]),
]

# Separate q/k and v head sizes (the absorbed MLA prefill of the atlas PR #69
# page: 320-wide q/k rows, 256-wide values): the scores use the d_qk columns
# of q and k, the output has the d_v columns of v.

EXAMPLES += [
    ex("split_head_sizes_dqk2_dv3",
       "d_qk = 2, d_v = 3: row 0 sees key 0 only -> v0 = [4, 0, -8]; row 1 "
       "scores [q1.k0, q1.k1] = [0, (ln3 - 1) + 0.5*2] = [0, ln3] -> "
       "weights [1/4, 3/4] -> [1, 3, 4]",
       [0, 2], 1, 1, 1.0, 0,
       [[[2.0, -7.0]], [[1.0, 0.5]]], [[[0.0, 0.0]], [[LN3 - 1.0, 2.0]]],
       [[[4.0, 0.0, -8.0]], [[0.0, 4.0, 8.0]]],
       [[[4.0, 0.0, -8.0]], [[1.0, 3.0, 4.0]]]),
    ex("split_head_sizes_dqk3_dv1_gqa",
       "d_qk = 3, d_v = 1, 2 Q heads on 1 KV head: head 0 row 1 scores "
       "[0, ln2] -> [1/3, 2/3] -> (6 + 2*9)/3 = 8; head 1 row 1 scores "
       "[0, -ln2] -> [2/3, 1/3] -> (2*6 + 9)/3 = 7; row 0 -> v0 = 6",
       [0, 2], 2, 1, 1.0, 0,
       [[[1.0, 1.0, 1.0], [3.0, 3.0, 3.0]], [[1.0, 0.0, 0.0], [0.0, -1.0, 0.0]]],
       [[[0.0, 0.0, -5.0]], [[LN2, LN2, 0.0]]],
       [[[6.0]], [[9.0]]],
       [[[6.0], [6.0]], [[8.0], [7.0]]]),
]

# Paged KV: key position j of sequence s is slot j % page_size of page
# block_table[s][j // page_size] (atlas PR #69, paged MLA prefill: a page
# table lookup per position).


def exp_(name, why, cu_q, table, seqlens_k, page_size, hq, hkv, scale, window,
         q, k_pool, v_pool, out):
    e = ex(name, why, cu_q, hq, hkv, scale, window, q, k_pool, v_pool, out)
    e.update(block_table=table, seqlens_k=seqlens_k, page_size=page_size)
    return e


EXAMPLES += [
    exp_("paged_reversed_pages",
         "page_size 1, table [2,1,0]: the pool holds the keys in reverse "
         "order, so positions 0,1,2 read slots 2,1,0 -> the same scores "
         "[7, 0, ln2] and values [10, 20, 50] as history2_one_query -> "
         "(10 e^7 + 120)/(e^7 + 3)",
         [0, 1], [[2, 1, 0]], [3], 1, 1, 1, 1.0, 0,
         [[[1.0]]], [[[LN2]], [[0.0]], [[7.0]]],
         [[[50.0]], [[20.0]], [[10.0]]],
         [[[(10 * E7 + 120) / (E7 + 3)]]]),
    exp_("paged_two_slot_pages_window2",
         "page_size 2, table [[1, 0]] over a 4-slot pool: positions 0,1 are "
         "slots 2,3 and position 2 is slot 0; the query at position 2 with "
         "W=2 sees positions {1,2} = slots {3,0}, scores [0, ln2] -> "
         "(20 + 2*50)/3 = 40",
         [0, 1], [[1, 0]], [3], 2, 1, 1, 1.0, 2,
         [[[1.0]]], [[[LN2]], [[-9.0]], [[7.0]], [[0.0]]],
         [[[50.0]], [[-1.0]], [[10.0]], [[20.0]]],
         [[[40.0]]]),
]

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "worked_examples.json")
    with open(path, "w") as f:
        json.dump({"source": __doc__.strip().splitlines()[0],
                   "examples": EXAMPLES}, f, indent=1)
        f.write("\n")
    print("wrote", path)
