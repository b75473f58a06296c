"""Layout of the blocked KV cache (test infrastructure).

The pages give no layout for the paged cache (DeepSpeed-FastGen paper card by Holmes et al.
2024, "Key points": a blocked KV cache as in PagedAttention), so it is a design reading, and
bit-exactness of the append is defined on it:

    K pool: [num_blocks][Hkv][bs][D]           key-major inside a block
    V pool: [num_blocks][Hkv][bs/g][D][g]      g = min(8, bs): keys in groups of g, each
                                                group feature-major with its g keys adjacent

Slot s of a block holds key row s of K at k_pool[b, h, s, :] and of V at
v_pool[b, h, s // g, :, s % g].
"""
V_GROUP_MAX = 8


def v_group(block_size: int) -> int:
    return min(V_GROUP_MAX, int(block_size))


def k_pool_shape(num_blocks, num_kv_heads, head_dim, block_size):
    return (int(num_blocks), int(num_kv_heads), int(block_size), int(head_dim))


def v_pool_shape(num_blocks, num_kv_heads, head_dim, block_size):
    g = v_group(block_size)
    return (int(num_blocks), int(num_kv_heads), int(block_size) // g, int(head_dim), g)


def v_slot(block_size: int, slot: int):
    """(group, index in group) of a block slot in the V pool."""
    g = v_group(block_size)
    return slot // g, slot % g
