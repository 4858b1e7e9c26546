"""Integer reference of the Assign work split — oracle side, test infrastructure.

Parity status: pinned by invariants (tests/test_oracle_taskmap.py: every
active unit is owned by exactly one worker, no worker exceeds L units, the
split counts match a direct per-worker walk, slots never exceed twice the
number of workers, and unit counts match a brute-force count of visible
keys per tile).  The pages fix only the idea, not the constants, so the
constants below are this library's own specification; the HIP Assign kernel
must reproduce this map bit for bit.

Pages followed:
* "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: Assign cuts every
  KV sequence into tiles and builds a load-balanced task map from the work per
  CTA; §3.3: choose the chunk length from the total load first, then cut each
  request by its real KV length, and let a task owned by one CTA write its
  result directly.
* "vLLM Triton Attention Backend Deep Dive", §3: Q blocks pack all query heads
  of one KV head (and several query tokens) into one work item; a persistent
  grid of fixed size reads its work from metadata in GPU memory.

Specification
-------------
* Q-blocks, in (sequence b, kv head g) order.  With G = Hq / Hkv and
  q_len = query tokens of b: if q_len * G <= 16 the single Q-block
  (b, g, 0, q_len) holds every query token of (b, g) ("small",
  decode-like); otherwise Q-blocks hold nt = 128 / G tokens,
  (b, g, t0, min(nt, q_len - t0)), and the n = ceil(q_len / nt) token blocks
  i = t0 / nt of one (b, g) are listed zig-zag: i = 0, n - 1, 1, n - 2, ...
  ("large").  Under causal masking a token block's unit count grows with i,
  so the zig-zag spreads short and long Q-blocks (and with them the fixed
  cost each Q-block adds) evenly over the contiguous worker ranges below.
  Row r of a Q-block is token t0 + r // G, query head g * G + r % G.
* A unit is one 64-key tile of one Q-block that holds at least one key some
  row of the Q-block may see (in the coarse sense below).  With
  pos_lo = seq_len - q_len + t0 and pos_hi = pos_lo + nt - 1:
  hi = min(seq_len - 1, pos_hi) if causal else seq_len - 1;
  lo = window_left(pos_lo) if window > 0 else 0;  no units if hi < lo;
  tiles tile_lo = lo // 64 .. tile_hi = hi // 64.  With a block mask, a tile
  t counts only if mask[b, hm, qt, (64 t) // tile] is 1 for some query tile
  qt in [pos_lo // tile, pos_hi // tile] and some head hm of the Q-block
  (hm = 0 when the mask is shared across heads).
* U = total units; the units of Q-block q are S_q .. S_q + n_q - 1 in the
  order above (S = exclusive prefix sum of n).
* L = force_split_units if it is > 0, else max(split_min_units, ceil(U / P)).
  Workers come in pairs (2k, 2k + 1), the two workgroups that share one
  compute unit, and a pair owns the 2L units [2kL, 2kL + 2L): with
  L0 = min(max(floor((2L w + 50) / 100), 1), 2L - 1) for the pair weight w
  (percent; 50 gives L0 = L, the even split), worker 2k owns [2kL, 2kL + L0)
  and worker 2k + 1 owns [2kL + L0, 2kL + 2L), each clipped to U.  Unit u
  belongs to worker_of(u) = 2 floor(u / 2L) + (u mod 2L >= L0); there are
  worker_of(U - 1) + 1 workers.  (The second workgroup on a compute unit is
  issued after the first when both are ready, so it runs slower; a weight
  above 50 gives the first one more units.)
* n_splits(q) = 0 if n_q == 0, else worker_of(S_q + n_q - 1) - worker_of(S_q) + 1.
  Q-blocks with n_splits != 1 go, in order, into the combine list.
  Q-blocks with n_splits >= 2 get partial slots slot_base(q) = running sum of
  n_splits over earlier such Q-blocks (-1 for the others); n_slots = total.

Sequence Q-blocks (heads interleaved)
-------------------------------------
* A decode batch may instead be cut into one Q-block per sequence holding all
  of its query heads: (b, 0, 0, q_len) for every b with q_len > 0, row r =
  token r // Hq, query head r % Hq.  Its units are the (tile, kv head)
  pairs, kv head fastest: unit k is tile tile_lo + k // Hkv of kv head
  k % Hkv, so n = Hkv * (tile_hi - tile_lo + 1) with the tile range above
  (no block mask).  Everything after the unit counts (prefix, L, workers,
  splits, slots) is unchanged.  (The four waves of a workgroup then read the
  same keys of different kv heads at the same time.)

Static split (no task map)
--------------------------
* The static variant of the same page's Split-K (a fixed number of splits
  per request, no Assign): every sequence must fit one small Q-block
  (q_len * G <= 16), Q-block q = (b = q // Hkv, g = q % Hkv).  Its tiles
  tile_lo .. tile_lo + n - 1 (the range above; no block mask) are cut into
  runs of c = ceil(n / S); split s owns [s c, min(n, (s + 1) c)); the
  ns = ceil(n / c) non-empty splits come first.  Item i = q S + s is split
  s of Q-block q, and writes partial slot i when ns >= 2.
"""
import numpy as np

UNIT_KEYS = 64
SMALL_MAX_ROWS = 16
LARGE_ROWS = 128


def _window_left(pos, window, expand, chunk):
    left = max(0, pos - window + 1)
    if expand and chunk > 0:
        left = (left // chunk) * chunk
    return left


def q_blocks(seq_lens, query_start_loc, Hq, Hkv, heads_interleaved=False):
    G = Hq // Hkv
    out = []
    for b in range(len(seq_lens)):
        ql = int(query_start_loc[b + 1]) - int(query_start_loc[b])
        if ql <= 0:
            continue
        if heads_interleaved:
            out.append((b, 0, 0, ql))
        elif ql * G <= SMALL_MAX_ROWS:
            for g in range(Hkv):
                out.append((b, g, 0, ql))
        else:
            nt = LARGE_ROWS // G
            n = -(-ql // nt)
            for g in range(Hkv):
                for k in range(n):
                    i = k // 2 if k % 2 == 0 else n - 1 - k // 2      # zig-zag over the token blocks
                    t0 = i * nt
                    out.append((b, g, t0, min(nt, ql - t0)))
    return out


def unit_count(desc, seq_lens, query_start_loc, Hq, Hkv, *, causal, window, expand_to_chunk,
               landmark_chunk, block_mask=None, block_mask_tile=128, heads_interleaved=False):
    b, g, t0, nt = desc
    G = Hq // Hkv
    ctx = int(seq_lens[b])
    ql = int(query_start_loc[b + 1]) - int(query_start_loc[b])
    pos_lo = ctx - ql + t0
    pos_hi = pos_lo + nt - 1
    hi = min(ctx - 1, pos_hi) if causal else ctx - 1
    lo = _window_left(pos_lo, window, expand_to_chunk, landmark_chunk) if window > 0 else 0
    if hi < lo:
        return 0
    t_lo, t_hi = lo // UNIT_KEYS, hi // UNIT_KEYS
    if heads_interleaved:
        if block_mask is not None:
            raise ValueError("sequence Q-blocks take no block mask")
        return Hkv * (t_hi - t_lo + 1)
    if block_mask is None:
        return t_hi - t_lo + 1
    heads = [0] if block_mask.shape[1] == 1 else list(range(g * G, (g + 1) * G))
    qts = range(pos_lo // block_mask_tile, pos_hi // block_mask_tile + 1)
    n = 0
    for t in range(t_lo, t_hi + 1):
        kt = (t * UNIT_KEYS) // block_mask_tile
        if any(block_mask[b, hm, qt, kt] for hm in heads for qt in qts):
            n += 1
    return n


def pair_split(L, pair_weight):
    """(L0, worker_of): the pair cut of 2L units and the unit -> worker map."""
    Lp = 2 * L
    L0 = min(max((Lp * int(pair_weight) + 50) // 100, 1), Lp - 1)
    return L0, (lambda u: 2 * (u // Lp) + (1 if u % Lp >= L0 else 0))


def worker_range(w, L, L0, U):
    """[a, b) of worker w."""
    a = (w // 2) * 2 * L + (w % 2) * L0
    return a, min(U, a + (2 * L - L0 if w % 2 else L0))


def build(seq_lens, query_start_loc, *, Hq, Hkv, num_workers, split_min_units=8,
          force_split_units=0, causal=True, window=0, window_expand_to_chunk=True,
          landmark_chunk=0, block_mask=None, block_mask_tile=128, pair_weight=50,
          heads_interleaved=False):
    seq_lens = [int(x) for x in seq_lens]
    qsl = [int(x) for x in query_start_loc]
    descs = q_blocks(seq_lens, qsl, Hq, Hkv, heads_interleaved)
    n = [unit_count(dsc, seq_lens, qsl, Hq, Hkv, causal=causal, window=window,
                    expand_to_chunk=window_expand_to_chunk, landmark_chunk=landmark_chunk,
                    block_mask=block_mask, block_mask_tile=block_mask_tile,
                    heads_interleaved=heads_interleaved) for dsc in descs]
    prefix = [0]
    for x in n:
        prefix.append(prefix[-1] + x)
    U = prefix[-1]
    P = int(num_workers)
    if force_split_units > 0:
        L = int(force_split_units)
    else:
        L = max(int(split_min_units), -(-U // P))
    L0, worker_of = pair_split(L, pair_weight)
    n_splits, slot_base, combine_list = [], [], []
    slots = 0
    for q, x in enumerate(n):
        S = prefix[q]
        ns = 0 if x == 0 else worker_of(S + x - 1) - worker_of(S) + 1
        n_splits.append(ns)
        if ns != 1:
            combine_list.append(q)
        if ns >= 2:
            slot_base.append(slots)
            slots += ns
        else:
            slot_base.append(-1)
    return {
        "desc": np.array(descs, dtype=np.int32).reshape(-1, 4),
        "n_units": np.array(n, dtype=np.int32),
        "unit_prefix": np.array(prefix, dtype=np.int32),
        "n_splits": np.array(n_splits, dtype=np.int32),
        "slot_base": np.array(slot_base, dtype=np.int32),
        "combine_list": np.array(combine_list, dtype=np.int32),
        "U": U, "P": P, "L": L, "L0": L0, "n_qb": len(descs), "n_slots": slots,
        "n_workers": worker_of(U - 1) + 1 if U else 0,
    }


def static_map(seq_lens, query_start_loc, *, Hq, Hkv, S, causal=True, window=0,
               window_expand_to_chunk=True, landmark_chunk=0):
    """Per item (q, s): (b, g, first tile, tile count) of the static split; raises
    when a sequence does not fit one small Q-block."""
    G = Hq // Hkv
    seq_lens = [int(x) for x in seq_lens]
    qsl = [int(x) for x in query_start_loc]
    items = []
    for b in range(len(seq_lens)):
        ql, ctx = qsl[b + 1] - qsl[b], seq_lens[b]
        if ql * G > SMALL_MAX_ROWS:
            raise ValueError(f"sequence {b}: q_len {ql} does not fit one small Q-block")
        for g in range(Hkv):
            n, t_lo = 0, 0
            if ql > 0:
                pos_lo, pos_hi = ctx - ql, ctx - 1
                hi = min(ctx - 1, pos_hi) if causal else ctx - 1
                lo = _window_left(pos_lo, window, window_expand_to_chunk, landmark_chunk) if window > 0 else 0
                if hi >= lo:
                    t_lo, n = lo // UNIT_KEYS, hi // UNIT_KEYS - lo // UNIT_KEYS + 1
            c = -(-n // S) if n else 1
            for s in range(S):
                a = min(n, s * c)
                items.append((b, g, t_lo + a, min(n, a + c) - a if s * c < n else 0))
    return items
