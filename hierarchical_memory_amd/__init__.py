"""HiSparse swap-in path for MI355X (gfx950): HIP kernels behind a C ABI, with a thin Python binding.

Importing the package loads the built HIP library and raises ImportError if it is missing; nothing here
falls back to another implementation.
"""
from .hisparse import (EXPORTED, HS_EVICT_FIFO, HS_EVICT_LRU, HS_E_HIP, HS_E_INVALID, HS_E_NOMEM, HS_E_STATE, HS_OK, HS_STATUS_BAD_ID,
                       HS_STATUS_BAD_STATE, HS_STATUS_DUP_ID, HS_STATUS_STALE, HiSparseError, HsConfig, HsDeviceViews, HsSizes, SwapIn,
                       config, config_from_hisparse_json, hs_bind_device, hs_create, hs_destroy, hs_gather,
                       hs_host_pool, hs_last_error, hs_plan, hs_step_static, HS_STATIC_PLAN_BYTES, hs_export_state, hs_import_state, HS_STATE_TABLES, HS_STATE_ROWS, hs_copy, hs_trial, hs_commit, hs_offload, hs_advance_tail, hs_rebuild_order, hs_required_sizes, hs_reset, hs_resolve, lib,
                       library_path)

lib()
