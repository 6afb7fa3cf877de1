"""Named small GPU test cases (seeded synthetic inputs) shared by the parity tests.

Sizes span several tiles with ragged tails; each case names what it exercises.
"""
import numpy as np

import synth


def case(name):
    mk = synth.make_case
    cases = {
        "config1": lambda: synth.config(1),
        # several 128x128 tiles with ragged tails on both axes, GQA 4/2
        "bnsd_bf16_d128_b128x128_ragged": lambda: mk(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=128,
                                                     Sq=300, Skv=270, bx=128, by=128, p=0.5, seed=101),
        # padded BNSD (actual lengths), D=64, 64x128 blocks
        "bnsd_fp16_d64_b64x128_padded": lambda: mk(layout="BNSD", dtype="fp16", B=2, N=2, Nkv=1, D=64,
                                                   Sq=256, Skv=320, bx=64, by=128, p=0.5,
                                                   lengths_q=[256, 150], lengths_kv=[320, 97], seed=102),
        # varlen TND, GQA 4/1
        "tnd_fp16_d128_b64x128_gqa": lambda: mk(layout="TND", dtype="fp16", B=3, N=4, Nkv=1, D=128,
                                                bx=64, by=128, p=0.4, lengths_q=[200, 77, 333],
                                                lengths_kv=[260, 129, 190], seed=103),
        "bnsd_bf16_d128_b128x64": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=2, D=128,
                                             Sq=256, Skv=520, bx=128, by=64, p=0.3, seed=104),
        # block sizes that are not multiples of the 32-row MFMA tile
        "bnsd_bf16_d64_b48x80": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=64,
                                           Sq=200, Skv=230, bx=48, by=80, p=0.5, seed=105),
        # blocks larger than the 128-row workgroup part
        "bnsd_fp16_d128_b256x256": lambda: mk(layout="BNSD", dtype="fp16", B=1, N=2, Nkv=2, D=128,
                                              Sq=600, Skv=530, bx=256, by=256, p=0.6, seed=106),
        # element-level mask (1x1 blocks), some rows select nothing
        "bnsd_bf16_d64_b1x1": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=64,
                                         Sq=40, Skv=37, bx=1, by=1, mask_rule="bernoulli", p=0.3, seed=107),
        # null mask = dense
        "bnsd_bf16_d128_nullmask": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=128,
                                              Sq=200, Skv=300, mask_rule="dense", seed=108),
        # a sequence with no queries and one with no keys
        "tnd_bf16_d64_empty_seqs": lambda: mk(layout="TND", dtype="bf16", B=3, N=2, Nkv=2, D=64,
                                              bx=64, by=64, p=0.5, lengths_q=[100, 0, 60],
                                              lengths_kv=[50, 70, 0], seed=109),
        # rows without the diagonal: empty Q-block rows and unselected KV blocks
        "bnsd_fp16_d128_sparse_rows": lambda: mk(layout="BNSD", dtype="fp16", B=1, N=2, Nkv=1, D=128,
                                                 Sq=512, Skv=512, bx=64, by=64, mask_rule="bernoulli",
                                                 p=0.15, seed=110),
        # local window + 2 sink blocks: sink columns are selected by every Q block of every head,
        # so the dK/dV work of most units is split into pieces and reduced in piece order
        "bnsd_bf16_d128_local_sink_split": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=1,
                                                      D=128, Sq=1024, Skv=1024, bx=64, by=64,
                                                      mask_rule="local8_sink2", seed=111),
        # the same with 256-row KV blocks (two 128-row parts per unit) and ragged lengths
        "bnsd_fp16_d64_sink_split_parts": lambda: mk(layout="BNSD", dtype="fp16", B=2, N=4, Nkv=2,
                                                     D=64, Sq=1000, Skv=1000, bx=32, by=256,
                                                     mask_rule="local8_sink2",
                                                     lengths_q=[1000, 700], lengths_kv=[1000, 650],
                                                     seed=112),
        # sliding windows (preTokens, nextTokens): a band wider than a block, GQA, ragged
        "bnsd_bf16_d128_window": lambda: mk(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=128, Sq=384,
                                            Skv=320, bx=64, by=64, p=0.6, window=(100, 20), seed=116),
        # a band that excludes the diagonal (rows past the last keys are left empty), TND
        "tnd_fp16_d64_window_ahead": lambda: mk(layout="TND", dtype="fp16", B=2, N=4, Nkv=1, D=64, bx=32,
                                                by=64, p=0.7, lengths_q=[150, 97], lengths_kv=[130, 200],
                                                window=(-3, 60), seed=117),
        # zero-width window (each row sees its own key only), 128-row blocks
        "bnsd_fp16_d128_window_zero": lambda: mk(layout="BNSD", dtype="fp16", B=1, N=2, Nkv=1, D=128,
                                                 Sq=256, Skv=256, bx=128, by=128, mask_rule="ones",
                                                 window=(0, 0), seed=118),
        # an empty window (pre + next < 0 admits no pair): no block is listed, every output is 0
        "bnsd_bf16_d64_window_empty": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=64, Sq=160,
                                                 Skv=96, bx=32, by=32, mask_rule="ones", window=(2, -4),
                                                 seed=119),
        # attenMask (30% of pairs removed, one row emptied), GQA, ragged
        "bnsd_bf16_d128_attenmask": lambda: mk(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=128, Sq=200,
                                               Skv=260, bx=64, by=64, p=0.7, seed=124),
        # attenMask with a window, TND
        "tnd_fp16_d64_attenmask_window": lambda: mk(layout="TND", dtype="fp16", B=2, N=2, Nkv=1, D=64,
                                                    bx=32, by=64, p=0.8, lengths_q=[120, 77],
                                                    lengths_kv=[100, 150], window=(50, 10), seed=125),
        # local window on top of the sink pattern: split units and element masks together
        "bnsd_bf16_d128_window_sink_split": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=1,
                                                       D=128, Sq=1024, Skv=1024, bx=64, by=64,
                                                       mask_rule="local8_sink2", window=(300, 0),
                                                       seed=119),
        # head dim 256 (two dK/dV passes per work item): ragged 128x128 tiles, GQA
        "bnsd_bf16_d256_b128x128_ragged": lambda: mk(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=256,
                                                     Sq=300, Skv=270, bx=128, by=128, p=0.5, seed=130),
        # head dim 256, varlen TND with 64-row blocks (a 4-wave dK/dV workgroup on 64 KV rows)
        "tnd_fp16_d256_b64x64_gqa": lambda: mk(layout="TND", dtype="fp16", B=2, N=4, Nkv=1, D=256, bx=64,
                                               by=64, p=0.5, lengths_q=[190, 77], lengths_kv=[150, 201],
                                               seed=131),
        # head dim 256 with split dK/dV units reduced in piece order
        "bnsd_fp16_d256_sink_split": lambda: mk(layout="BNSD", dtype="fp16", B=1, N=4, Nkv=1, D=256,
                                                Sq=768, Skv=768, bx=64, by=64, mask_rule="local8_sink2",
                                                seed=132),
        # head dim 256 with a window and an attenMask, 32-row Q blocks
        "bnsd_bf16_d256_window_attenmask": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=256,
                                                      Sq=200, Skv=260, bx=32, by=128, p=0.7,
                                                      window=(90, 30), seed=133),
        # 128-row KV blocks at head dim 128 (the 16-rows-per-wave dK/dV kernel) with an attenMask and a window
        "bnsd_fp16_d128_b64x128_attenmask_window": lambda: mk(layout="BNSD", dtype="fp16", B=2, N=4, Nkv=2,
                                                              D=128, Sq=300, Skv=270, bx=64, by=128, p=0.7,
                                                              window=(150, 40), seed=134),
        # the same kernel on split units (sink columns), ragged
        "bnsd_bf16_d128_b64x128_sink_split": lambda: mk(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=1, D=128,
                                                        Sq=2000, Skv=2000, bx=64, by=128,
                                                        mask_rule="local8_sink2", seed=135),
        # more sequences than one copy launch of the sequence table takes (two launches)
        "tnd_bf16_d64_70_seqs": lambda: mk(layout="TND", dtype="bf16", B=70, N=2, Nkv=1, D=64, bx=16, by=16,
                                           p=0.6, lengths_q=[(7 * b) % 41 for b in range(70)],
                                           lengths_kv=[(11 * b + 3) % 37 for b in range(70)], seed=136),
    }
    c = cases[name]()
    if name in ATTEN:  # an attenMask over [maxSq, maxSkv], drawn after the case
        rng = np.random.default_rng(c.seed + 7)
        sq, sk = int(c.len_q.max()), int(c.len_kv.max())
        if c.layout == "BNSD":
            sq, sk = c.Sq, c.Skv
        am = (rng.random((sq, sk)) < ATTEN[name]).astype(np.uint8)
        am[:, : min(8, sk)] = 0   # the first keys stay in, so most rows keep some key ...
        am[min(5, sq - 1), :] = 1  # ... but one row loses all of them
        c.atten_mask = am
    return c


# fraction of pairs an attenMask removes, for the cases that carry one
ATTEN = {"bnsd_bf16_d128_attenmask": 0.3, "tnd_fp16_d64_attenmask_window": 0.5,
         "bnsd_bf16_d256_window_attenmask": 0.2, "bnsd_fp16_d128_b64x128_attenmask_window": 0.25}


SMALL = ["config1", "bnsd_bf16_d128_b128x128_ragged", "bnsd_fp16_d64_b64x128_padded",
         "tnd_fp16_d128_b64x128_gqa", "bnsd_bf16_d128_b128x64", "bnsd_bf16_d64_b48x80",
         "bnsd_fp16_d128_b256x256", "bnsd_bf16_d64_b1x1", "bnsd_bf16_d128_nullmask",
         "tnd_bf16_d64_empty_seqs", "bnsd_fp16_d128_sparse_rows", "bnsd_bf16_d128_local_sink_split",
         "bnsd_fp16_d64_sink_split_parts", "bnsd_bf16_d128_window", "tnd_fp16_d64_window_ahead",
         "bnsd_fp16_d128_window_zero", "bnsd_bf16_d64_window_empty", "bnsd_bf16_d128_window_sink_split", "bnsd_bf16_d128_attenmask",
         "tnd_fp16_d64_attenmask_window", "bnsd_bf16_d256_b128x128_ragged", "tnd_fp16_d256_b64x64_gqa",
         "bnsd_fp16_d256_sink_split", "bnsd_bf16_d256_window_attenmask", "bnsd_fp16_d128_b64x128_attenmask_window",
         "bnsd_bf16_d128_b64x128_sink_split", "tnd_bf16_d64_70_seqs"]

