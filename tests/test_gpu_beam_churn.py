"""Beam-search churn end to end: the host block manager (libpabm.so) drives
the device operations through many fork / prune / copy-on-write steps.

Each step prunes the live beams to a few seeded survivors, forks each back up
to the beam width, asks the manager for every beam's next slot and the
copy-on-write pairs, runs the layer-batched copy and append (or the fused
append inside pa_decode) and decodes every layer -- layer 1 with
pa_decode_shared, the beams grouped by the blocks they share (the manager's
pa_bm_shared_prefix).  Checked each step:
  * every layer's pools are bit-identical to pools the oracle maintains with
    the same copies and appends;
  * every beam's attention output matches attention (oracle, fp64) over that
    beam's own token history, kept as plain per-beam arrays that never look
    at a block table -- so a copy-on-write that went to the wrong block or
    was skipped shows up as a wrong output;
  * the manager's invariants hold (pa_bm_check) and every block a beam holds
    has the reference count the live tables imply.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_310_amd import workloads as wl
from _gpu_util import assert_attention_close, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _history_attention(q_bits, hist_k, hist_v, scale, dtype, hq, hkv):
    """[hq, d] fp64 attention of one beam over its own token history."""
    import oracle
    group = hq // hkv
    out = np.zeros((hq, q_bits.shape[-1]))
    for h in range(hq):
        k = oracle.bits_to_f64(hist_k[:, h // group, :], dtype)
        v = oracle.bits_to_f64(hist_v[:, h // group, :], dtype)
        out[h] = oracle.attention_rows(oracle.bits_to_f64(q_bits[h], dtype), k, v,
                                       np.float64(np.float32(scale)))
    return out


@pytest.mark.parametrize("hq,hkv,bs", [(8, 2, 16), (4, 4, 16), (8, 8, 32)],
                         ids=["gqa-bs16", "mha-bs16", "mha-bs32"])
def test_beam_churn_matches_oracle(hq, hkv, bs):
    import oracle
    import paged_kv_cache_310_amd as pa
    from paged_kv_cache_310_amd.kv_block_manager import KVBlockManager
    dtype, d, layers, nb = wl.BF16, 128, 2, 96
    width, keep, steps, prompt = 8, 2, 24, 45
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(1000 + hq + bs)
    say("beam churn", hq, hkv, bs)

    # pools start as noise: a read of a block the beam does not own is visible
    host_k = [wl.normal_bits(rng, (nb, hkv, bs, d), dtype) for _ in range(layers)]
    host_v = [wl.normal_bits(rng, (nb, hkv, bs, d), dtype) for _ in range(layers)]
    dev_k = [to_dev(x) for x in host_k]
    dev_v = [to_dev(x) for x in host_v]

    mgr = KVBlockManager(nb, bs, free_order=rng.permutation(nb))
    mgr.add_sequence(0, prompt)
    table, _ = mgr.block_tables([0], max_blocks=nb)
    pos = np.arange(prompt)
    prompt_slots = table[0][pos // bs].astype(np.int64) * bs + pos % bs
    pk = [wl.normal_bits(rng, (prompt, hkv, d), dtype) for _ in range(layers)]
    pv = [wl.normal_bits(rng, (prompt, hkv, d), dtype) for _ in range(layers)]
    pa.pa_append_kv_layers(dev_k, dev_v, [to_dev(x) for x in pk], [to_dev(x) for x in pv],
                           to_dev(prompt_slots))
    for l in range(layers):
        host_k[l], host_v[l] = oracle.append_kv(host_k[l], host_v[l], pk[l], pv[l],
                                                prompt_slots, bs)
    history = {0: ([x.copy() for x in pk], [x.copy() for x in pv])}
    live, next_id = [0], 1
    for child in range(1, width):
        mgr.fork(0, next_id)
        history[next_id] = tuple([x.copy() for x in h] for h in history[0])
        live.append(next_id)
        next_id += 1

    ws = None
    total_copies = 0
    for step in range(steps):
        # prune to `keep` seeded survivors, fork each back to the beam width
        survivors = sorted(rng.choice(live, size=keep, replace=False).tolist())
        for s in live:
            if s not in survivors:
                mgr.free_sequence(s)
                del history[s]
        live = []
        for s in survivors:
            live.append(s)
            for _ in range(width // keep - 1):
                mgr.fork(s, next_id)
                history[next_id] = tuple([x.copy() for x in h] for h in history[s])
                live.append(next_id)
                next_id += 1
        slots, copies = mgr.append_slots(live)
        total_copies += len(copies)
        mgr.check()

        kn = [wl.normal_bits(rng, (len(live), hkv, d), dtype) for _ in range(layers)]
        vn = [wl.normal_bits(rng, (len(live), hkv, d), dtype) for _ in range(layers)]
        q = [wl.normal_bits(rng, (len(live), hq, d), dtype) for _ in range(layers)]
        for i, s in enumerate(live):
            for l in range(layers):
                history[s][0][l] = np.concatenate([history[s][0][l], kn[l][i:i + 1]])
                history[s][1][l] = np.concatenate([history[s][1][l], vn[l][i:i + 1]])

        if len(copies):
            pa.pa_copy_blocks_layers(dev_k, dev_v, to_dev(copies))
            for l in range(layers):
                host_k[l], host_v[l] = oracle.copy_blocks(host_k[l], host_v[l], copies)
        kn_d, vn_d, slots_d = [to_dev(x) for x in kn], [to_dev(x) for x in vn], to_dev(slots)
        fused0 = step % 2 == 1      # odd steps: layer 0's append runs inside pa_decode
        first = 1 if fused0 else 0
        pa.pa_append_kv_layers(dev_k[first:], dev_v[first:], kn_d[first:], vn_d[first:],
                               slots_d)
        for l in range(layers):
            host_k[l], host_v[l] = oracle.append_kv(host_k[l], host_v[l], kn[l], vn[l], slots, bs)

        max_blocks = max(-(-len(history[s][0][0]) // bs) for s in live)
        tables, lens = mgr.block_tables(live, max_blocks=max_blocks)
        tables_d, lens_d = to_dev(tables), to_dev(lens)
        # Layer 1 decodes with the beams grouped by what they share (the
        # manager's shared prefix): all beams as one group on even steps, each
        # survivor's family as a group on odd steps.
        starts = [0, len(live)] if step % 2 == 0 else list(range(0, len(live) + 1, width // keep))
        prefix = mgr.shared_prefix(live, starts)
        assert prefix.max() > 0 and (prefix < lens).all()
        for l in range(layers):
            fused = fused0 and l == 0
            if l == 1:
                out = pa.pa_decode_shared(to_dev(q[l]), dev_k[l], dev_v[l], tables_d, lens_d,
                                          float(scale), to_dev(np.asarray(starts, np.int32)),
                                          to_dev(prefix))
            else:
                out = pa.pa_decode(to_dev(q[l]), dev_k[l], dev_v[l], tables_d, lens_d,
                                   float(scale), k_new=kn_d[l] if fused else None,
                                   v_new=vn_d[l] if fused else None,
                                   slot_mapping=slots_d if fused else None)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(dev_k[l]), host_k[l]), f"step {step} K pool layer {l}"
            assert np.array_equal(to_host(dev_v[l]), host_v[l]), f"step {step} V pool layer {l}"
            ref = np.stack([_history_attention(q[l][i], history[s][0][l], history[s][1][l],
                                               scale, dtype, hq, hkv)
                            for i, s in enumerate(live)])
            assert_attention_close(out_f64(out), ref, dtype)

        # reference counts equal the number of live tables that hold the block
        held = {}
        for row, n in zip(tables, lens):
            for b in row[: -(-int(n) // bs)]:
                held[int(b)] = held.get(int(b), 0) + 1
        for b, c in held.items():
            assert mgr.refcount(b) == c
    st = mgr.stats()
    say("copies", total_copies, "shared blocks", st["shared_blocks"], "free", st["free_blocks"])
    assert total_copies > 0 and st["copies"] == total_copies
    assert st["sequences"] == width
