"""libtilepipe: software-pipelined global->LDS tile streaming for MI355X (gfx950)."""
