"""MoL (multi-LoRA MoE, virtual experts) delta path for MI355X (gfx950)."""
