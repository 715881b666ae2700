"""MI355X-native CacheGen KV-cache codec: a C-ABI HIP library (libcachegen.so,
declared in include/cachegen.h) and its thin Python binding."""
from ._binding import (CG_GROUP_CHANNEL, CG_GROUP_GLOBAL, CG_GROUP_LAYER,  # noqa: F401
                       CG_GROUP_LAYER_CHANNEL, CG_E_CAPACITY, CG_E_CORRUPT, CG_E_HIP, CG_E_INVAL, CG_E_MISMATCH,  # noqa: F401
                       CG_E_NOMEM, CG_OK, CG_Q_H, CG_Q_L, CG_Q_M, EXPORTS, LIB_PATH, CgError,
                       Tables, cg_build_tables, cg_build_tables_grouped, cg_chunk_info, cg_chunk_info_parse, cg_decode,
                       cg_decode_async, cg_decode_paged_async, cg_decode_streamed, cg_encode,
                       cg_encode_batch, cg_encode_batch_noalloc,
                       cg_encode_bound,
                       cg_chunk_plan_in, cg_last_error, cg_num_chunks, cg_params,
                       cg_plan_chunk, cg_release_cached, cg_tables_deserialize,
                       cg_tables_free, cg_tables_id, cg_tables_params, cg_tables_serialize, lib,
                       make_params)

__all__ = [n for n in dir() if n.startswith("cg_") or n.startswith("CG_")] + [
    "CgError", "Tables", "lib", "make_params", "EXPORTS", "LIB_PATH"]
