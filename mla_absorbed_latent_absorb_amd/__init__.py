"""HIP (gfx950) absorbed-MLA decode library: Python binding and input generators."""
