"""Oracle: the blocks of the Q-KV interaction matrix that one mesh GPU owns.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (pages of the Mesh-Attention write-ups):

* Mesh-Attention tutorial page, section "From 1-D ring to 2-D mesh": attention
  is viewed as a matrix whose rows are Q partitions and whose columns are KV
  partitions; Ring-Attention hands each GPU a row, Mesh-Attention hands each
  GPU a 2-D tile, and a GPU only exchanges data with the GPUs of its own mesh
  row and mesh column.  Panel (c) of the (missing) figure introduces an index
  rotation of the KV blocks so that each GPU works on local data.
* mlsanity page for arXiv 2512.20968, section "Abstract (arXiv)": a tile
  collects only subsets of the Q and KV partitions; KV Partition Rotation
  (KVR) balances traffic.

Readings (the figure and the rotation formula are not on the pages):

* GPU (r, c) of an R x C mesh has id g = r*C + c and holds sequence partition
  g (its Q, K and V).
* Its Q set is the Q partitions of its mesh row: r*C + t, t = 0..C-1.
* Its KV set is R partitions of its mesh column.  Rotated order: partition
  ((r + k) mod R)*C + c for k = 0..R-1, i.e. its own partition first, then
  stepping down the column cyclically.  Contiguous order: c*R + k.
* Causal rule: a key is visible to a query when its global position is not
  after the query's.  A block's class is decided by brute force over the
  token positions of both partitions: FULL when every key is visible to every
  query, SKIP when no key is visible to any query, DIAG otherwise.  With
  equal-length partitions of at least two tokens this gives FULL for
  kv_part < q_part, DIAG for equality and SKIP above; a non-causal tile is
  all FULL.
* Entries are ordered KV-slot major, then Q slot.
"""

FULL = 0
DIAG = 1
SKIP = 2


def mesh_tile_sets_ref(mesh_rows, mesh_cols, row, col, kv_rotate):
    """Q-partition set and KV-partition set (in slot order) of GPU (row, col)."""
    if mesh_rows < 1 or mesh_cols < 1:
        raise ValueError("mesh dimensions must be positive")
    if not (0 <= row < mesh_rows and 0 <= col < mesh_cols):
        raise ValueError("tile position outside the mesh")
    q_set = [row * mesh_cols + t for t in range(mesh_cols)]
    if kv_rotate:
        kv_set = [((row + k) % mesh_rows) * mesh_cols + col for k in range(mesh_rows)]
    else:
        kv_set = [col * mesh_rows + k for k in range(mesh_rows)]
    return q_set, kv_set


def _block_kind(q_part, kv_part, causal, part_len):
    """Classify one block by looking at every (query, key) position pair."""
    if not causal:
        return FULL
    q_positions = range(q_part * part_len, (q_part + 1) * part_len)
    k_positions = range(kv_part * part_len, (kv_part + 1) * part_len)
    visible = [kp <= qp for qp in q_positions for kp in k_positions]
    if all(visible):
        return FULL
    if not any(visible):
        return SKIP
    return DIAG


def block_list_ref(mesh_rows, mesh_cols, row, col, causal, kv_rotate, part_len=2):
    """All C*R blocks of tile (row, col) as (q_slot, kv_slot, q_part, kv_part, kind).

    ``part_len`` only feeds the brute-force classification; any length of two
    or more gives the same classes (a one-token partition has no diagonal).
    """
    q_set, kv_set = mesh_tile_sets_ref(mesh_rows, mesh_cols, row, col, kv_rotate)
    out = []
    for kv_slot, kv_part in enumerate(kv_set):
        for q_slot, q_part in enumerate(q_set):
            out.append((q_slot, kv_slot, q_part, kv_part,
                        _block_kind(q_part, kv_part, causal, part_len)))
    return out
