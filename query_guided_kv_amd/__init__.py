"""query_guided_kv_amd: query-guided KV selection on MI355X (gfx950)."""
