"""MI355X (gfx950) lightning-indexer logits: C-ABI HIP library + thin binding."""
