// C ABI of libfva: argument checks, buffer sizes, error reporting, launches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fva_common.h"

namespace fva {

int launch_route(const fva_problem& p, int nb, const void* q, const void* k, const void* v,
                 float* scores, int16_t* ranked, int32_t* row_count,
                 int32_t* head_count, int32_t* order, void* kv, float* qbar, float* kbar,
                 float sm_scale, hipStream_t stream);
int launch_plan(const fva_problem& p, int nb, int split_s, const int16_t* ranked,
                const int32_t* row_count, const int32_t* head_refill, int32_t* row_ptr, int32_t* col_idx,
                int32_t* head_count_final, int32_t* work_order, int32_t* plan_meta,
                uint32_t* tile_counter, hipStream_t stream);
int launch_kv_layout(const fva_problem& p, int nb, const void* k, const void* v, int32_t* order,
                     void* kv, hipStream_t stream);
int launch_schedule(const fva_problem& p, int nb, int split_s, const int32_t* row_ptr,
                    int32_t* work_order, int32_t* plan_meta, uint32_t* tile_counter,
                    hipStream_t stream);
int launch_attn(const fva_problem& p, int nb, int grid, const void* q, const void* kv,
                const int32_t* order, const int32_t* row_ptr, const int32_t* col_idx,
                const int32_t* work_order, const int32_t* plan_meta, uint32_t* tile_counter,
                void* o, float* lse, float* block_lse, void* workspace, float sm_scale,
                int64_t* item_trace, hipStream_t stream);
int launch_block_importance(const fva_problem& p, int nb, const int32_t* order, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* lse, const float* block_lse,
                            float* importance, hipStream_t stream);
int launch_reselect(const fva_problem& p, int nb, const int32_t* row_ptr, const int32_t* col_idx,
                    const float* importance, int16_t* ranked, int32_t* row_count,
                    int32_t* head_count, hipStream_t stream);
int attn_blocks_per_cu(int d, int block);

static thread_local char g_last_error[256] = "";

int record_hip_error(hipError_t e, const char* what) {
  if (e == hipSuccess) return FVA_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return FVA_ERR_HIP;
}

// Per-device launch facts, filled on first use.
struct DeviceInfo {
  int cus = 0;
  int blocks_per_cu[4] = {0, 0, 0, 0};  // (d, B) = (64,64) (64,128) (128,64) (128,128)
};
static std::mutex g_dev_mutex;
static DeviceInfo g_dev[64];

static int variant_index(int d, int block) { return (d == 128 ? 2 : 0) + (block == 128 ? 1 : 0); }

// Compute units of the current device (cached), 0 on error.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& info = g_dev[dev];
  if (info.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    info.cus = cus > 0 ? cus : 1;
  }
  return info.cus;
}

static int attn_grid(const fva_problem& p, int nb, int* grid) {
  int dev = 0;
  int st = record_hip_error(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  if (dev < 0 || dev >= 64) return FVA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& info = g_dev[dev];
  if (info.cus == 0) {
    int cus = 0;
    st = record_hip_error(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                          "hipDeviceGetAttribute");
    if (st) return st;
    info.cus = cus > 0 ? cus : 1;
  }
  const int vi = variant_index(p.head_dim, p.block);
  if (info.blocks_per_cu[vi] == 0) {
    const int b = attn_blocks_per_cu(p.head_dim, p.block);
    if (b < 0) return record_hip_error(hipErrorInvalidValue, "occupancy query");
    info.blocks_per_cu[vi] = b;
  }
  const int64_t want = (int64_t)info.cus * info.blocks_per_cu[vi];
  const int64_t tiles = (int64_t)p.num_heads * nb;
  *grid = (int)(want < tiles ? want : tiles);
  if (*grid < 1) *grid = 1;
  return FVA_OK;
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Checks shared by every entry point.  Returns the status and fills nb.
static int check_problem(const fva_problem* p, int* nb_out) {
  if (p == nullptr) return FVA_ERR_ARG;
  if (p->num_heads < 1 || p->seq_len < 1) return FVA_ERR_ARG;
  if (p->grid_t < 1 || p->grid_h < 1 || p->grid_w < 1) return FVA_ERR_ARG;
  if ((int64_t)p->grid_t * p->grid_h * p->grid_w != (int64_t)p->seq_len) return FVA_ERR_ARG;
  if (p->tile_h < 0 || p->tile_w < 0) return FVA_ERR_ARG;
  if (p->order_kind != FVA_ORDER_TILES && p->order_kind != FVA_ORDER_HILBERT) return FVA_ERR_ARG;
  if (p->reserved != 0) return FVA_ERR_ARG;
  if ((p->tile_h == 0) != (p->tile_w == 0)) return FVA_ERR_ARG;
  if (isnan(p->top_p)) return FVA_ERR_ARG;
  if (p->k_min < 1) return FVA_ERR_ARG;
  if (p->refill_per_mille < 0 || p->refill_per_mille > 1000) return FVA_ERR_ARG;
  if (!isfinite(p->sm_scale) || p->sm_scale < 0.f) return FVA_ERR_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return FVA_ERR_UNSUPPORTED;
  if (p->block != 64 && p->block != 128) return FVA_ERR_UNSUPPORTED;
  if (p->stride_token < p->head_dim || p->stride_head < p->head_dim) return FVA_ERR_ARG;
  if ((p->stride_token & 7) != 0 || (p->stride_head & 7) != 0) return FVA_ERR_ARG;
  const int64_t nb = ((int64_t)p->seq_len + p->block - 1) / p->block;
  if (nb > FVA_MAX_BLOCKS) return FVA_ERR_UNSUPPORTED;
  if (nb * p->num_heads > FVA_MAX_TILES) return FVA_ERR_UNSUPPORTED;
  // largest element offset must fit the 64-bit index arithmetic comfortably
  if ((int64_t)(p->num_heads - 1) * p->stride_head + (int64_t)(p->seq_len - 1) * p->stride_token >
      ((int64_t)1 << 40))
    return FVA_ERR_UNSUPPORTED;
  *nb_out = (int)nb;
  return FVA_OK;
}

// Routing workspace: the pooled block means (2 x H x nb x d floats), then
// room for the scores (H x nb x nb floats) for callers that do not want them.
static int64_t pooled_bytes(const fva_problem* p, int nb) {
  return 2 * (int64_t)p->num_heads * nb * p->head_dim * (int64_t)sizeof(float);
}
static int64_t workspace_need(const fva_problem* p, int nb) {
  return pooled_bytes(p, nb) + (int64_t)p->num_heads * nb * nb * (int64_t)sizeof(float);
}

// K and V of every head re-laid out in position order: 2 x H x nb*B x d bf16.
static int64_t kv_elems(const fva_problem* p, int nb) {
  return 2 * (int64_t)p->num_heads * nb * p->block * p->head_dim;
}

// Split tiles one call can produce (fewer than 2 * FVA_MAX_SPLITS / 2).
static int64_t max_splits(const fva_problem* p, int nb) {
  const int64_t rows = (int64_t)p->num_heads * nb;
  return rows < FVA_MAX_SPLITS ? rows : FVA_MAX_SPLITS;
}

// Partial results of split tiles: per slot and part, B x d floats of
// unnormalised output plus B maxima and B denominators.
static int64_t attn_workspace_need(const fva_problem* p, int nb) {
  return max_splits(p, nb) * 2 * ((int64_t)p->block * p->head_dim + 2 * p->block) * 4;
}

// The split rule's S: a tile is cut when it is heavier than about the mean
// load of one compute unit (the two workgroups a unit runs share its
// throughput, so anything lighter is absorbed by the heaviest-first queue).
static int split_rule(int cus) {
  const int split_s = cus / 2 < FVA_MAX_SPLITS / 2 ? cus / 2 : FVA_MAX_SPLITS / 2;
  return split_s < 1 ? 1 : split_s;
}

// Routing workspace of fva_route_noalloc: one static array per device (each
// GPU holds its own copy).  Host code never passes `scratch` itself to a
// kernel: in host code the name is a stand-in, not a device address.  The
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FVA_NOALLOC_SCRATCH_BYTES];
static void* g_scratch_ptr[64];

// Device address of the current device's scratch array, resolved on first
// use; FVA_OK or FVA_ERR_HIP.
static int scratch_address(void** out) {
  int dev = 0;
  int st = record_hip_error(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  if (dev < 0 || dev >= 64) return FVA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    st = record_hip_error(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st) return st;
    if (ptr == nullptr) return record_hip_error(hipErrorInvalidSymbol, "scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FVA_OK;
}

static float effective_scale(const fva_problem* p) {
  return p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
}

}  // namespace fva

using namespace fva;

extern "C" {

int fva_version(void) { return 400; }

const char* fva_status_string(int status) {
  switch (status) {
    case FVA_OK: return "ok";
    case FVA_ERR_ARG: return "invalid argument";
    case FVA_ERR_UNSUPPORTED: return "unsupported problem (head_dim/block/size limits)";
    case FVA_ERR_HIP: return "HIP runtime error";
    case FVA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* fva_last_error(void) { return g_last_error; }

int fva_sizes(const fva_problem* prob, fva_sizes_t* out) {
  int nb = 0;
  if (out == nullptr) return FVA_ERR_ARG;
  const int st = check_problem(prob, &nb);
  if (st) return st;
  const int64_t rows = (int64_t)prob->num_heads * nb;
  out->num_blocks = nb;
  out->num_rows = (int32_t)rows;
  out->order_elems = (int64_t)nb * prob->block;
  out->scores_elems = rows * nb;
  out->ranked_elems = rows * nb;
  out->col_idx_capacity = rows * nb;
  out->workspace_bytes = workspace_need(prob, nb);
  out->tile_counter_elems = 2;
  out->kv_elems = kv_elems(prob, nb);
  out->work_order_elems = rows + max_splits(prob, nb);
  out->plan_meta_elems = 2 + rows + FVA_MAX_SPLITS;
  out->attn_workspace_bytes = attn_workspace_need(prob, nb);
  out->block_lse_capacity = rows * nb * prob->block;
  return FVA_OK;
}

int fva_compute_units(int32_t* out) {
  if (out == nullptr) return FVA_ERR_ARG;
  const int cus = device_cu_count();
  if (cus < 1) return record_hip_error(hipErrorNoDevice, "compute unit count");
  *out = cus;
  return FVA_OK;
}

int fva_attn_workgroups(const fva_problem* prob, int32_t* out) {
  int nb = 0;
  if (out == nullptr) return FVA_ERR_ARG;
  int st = check_problem(prob, &nb);
  if (st) return st;
  int grid = 0;
  st = attn_grid(*prob, nb, &grid);
  if (st) return st;
  *out = grid;
  return FVA_OK;
}

int fva_route(const fva_problem* prob, const void* q, const void* k, const void* v,
              float* scores, int16_t* ranked, int32_t* row_count, int32_t* head_count,
              int32_t* order, void* kv, void* workspace, size_t workspace_bytes, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!q || !k || !ranked || !row_count || !head_count || !order || !workspace) return FVA_ERR_ARG;
  if ((v == nullptr) != (kv == nullptr)) return FVA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(workspace)) return FVA_ERR_ARG;
  if (kv && (!aligned16(v) || !aligned16(kv))) return FVA_ERR_ARG;
  if ((int64_t)workspace_bytes < workspace_need(prob, nb)) return FVA_ERR_WORKSPACE;
  float* qbar = (float*)workspace;
  float* kbar = qbar + (int64_t)prob->num_heads * nb * prob->head_dim;
  if (scores == nullptr) scores = (float*)((char*)workspace + pooled_bytes(prob, nb));
  return launch_route(*prob, nb, q, k, v, scores, ranked, row_count, head_count, order, kv, qbar,
                      kbar, effective_scale(prob), (hipStream_t)stream);
}

int fva_route_noalloc(const fva_problem* prob, const void* q, const void* k, const void* v,
                      float* scores, int16_t* ranked, int32_t* row_count, int32_t* head_count,
                      int32_t* order, void* kv, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!q || !k || !ranked || !row_count || !head_count || !order) return FVA_ERR_ARG;
  if ((v == nullptr) != (kv == nullptr)) return FVA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k)) return FVA_ERR_ARG;
  if (kv && (!aligned16(v) || !aligned16(kv))) return FVA_ERR_ARG;
  if (workspace_need(prob, nb) > (int64_t)FVA_NOALLOC_SCRATCH_BYTES) return FVA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  float* qbar = (float*)ws;
  float* kbar = qbar + (int64_t)prob->num_heads * nb * prob->head_dim;
  if (scores == nullptr) scores = (float*)((char*)ws + pooled_bytes(prob, nb));
  return launch_route(*prob, nb, q, k, v, scores, ranked, row_count, head_count, order, kv, qbar,
                      kbar, effective_scale(prob), (hipStream_t)stream);
}

int fva_kv_layout(const fva_problem* prob, const void* k, const void* v, int32_t* order, void* kv,
                  void* stream) {
  int nb = 0;
  const int st = check_problem(prob, &nb);
  if (st) return st;
  if (!k || !v || !order || !kv) return FVA_ERR_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kv)) return FVA_ERR_ARG;
  return launch_kv_layout(*prob, nb, k, v, order, kv, (hipStream_t)stream);
}

int fva_plan(const fva_problem* prob, const int16_t* ranked, const int32_t* row_count,
             const int32_t* head_refill, int32_t* row_ptr, int32_t* col_idx, int32_t* head_count_final,
             int32_t* work_order, int32_t* plan_meta, uint32_t* tile_counter, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!ranked || !row_count || !row_ptr || !col_idx || !head_count_final || !work_order ||
      !plan_meta || !tile_counter)
    return FVA_ERR_ARG;
  const int cus = device_cu_count();
  if (cus < 1) return record_hip_error(hipErrorNoDevice, "compute unit count");
  return launch_plan(*prob, nb, split_rule(cus), ranked, row_count, head_refill, row_ptr, col_idx,
                     head_count_final, work_order, plan_meta, tile_counter, (hipStream_t)stream);
}

int fva_schedule(const fva_problem* prob, const int32_t* row_ptr, int32_t* work_order,
                 int32_t* plan_meta, uint32_t* tile_counter, void* stream) {
  int nb = 0;
  const int st = check_problem(prob, &nb);
  if (st) return st;
  if (!row_ptr || !work_order || !plan_meta || !tile_counter) return FVA_ERR_ARG;
  const int cus = device_cu_count();
  if (cus < 1) return record_hip_error(hipErrorNoDevice, "compute unit count");
  return launch_schedule(*prob, nb, split_rule(cus), row_ptr, work_order, plan_meta, tile_counter,
                         (hipStream_t)stream);
}

static int attn_call(const fva_problem* prob, const void* q, const void* kv,
                     const int32_t* order, const int32_t* row_ptr, const int32_t* col_idx,
                     const int32_t* work_order, const int32_t* plan_meta,
                     uint32_t* tile_counter, void* o, float* lse, float* block_lse,
                     void* workspace, size_t workspace_bytes, int64_t* item_trace, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!q || !kv || !order || !row_ptr || !col_idx || !work_order || !plan_meta ||
      !tile_counter || !o || !workspace)
    return FVA_ERR_ARG;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned16(order) ||
      !aligned16(workspace))
    return FVA_ERR_ARG;
  if ((int64_t)workspace_bytes < attn_workspace_need(prob, nb)) return FVA_ERR_WORKSPACE;
  if (block_lse != nullptr && lse == nullptr) return FVA_ERR_ARG;
  int grid = 0;
  st = attn_grid(*prob, nb, &grid);
  if (st) return st;
  return launch_attn(*prob, nb, grid, q, kv, order, row_ptr, col_idx, work_order, plan_meta,
                     tile_counter, o, lse, block_lse, workspace, effective_scale(prob), item_trace,
                     (hipStream_t)stream);
}

int fva_sparse_attn_fwd(const fva_problem* prob, const void* q, const void* kv,
                        const int32_t* order, const int32_t* row_ptr, const int32_t* col_idx,
                        const int32_t* work_order, const int32_t* plan_meta,
                        uint32_t* tile_counter, void* o, float* lse, float* block_lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return attn_call(prob, q, kv, order, row_ptr, col_idx, work_order, plan_meta, tile_counter, o, lse,
                   block_lse, workspace, workspace_bytes, nullptr, stream);
}

int fva_sparse_attn_fwd_traced(const fva_problem* prob, const void* q, const void* kv,
                               const int32_t* order, const int32_t* row_ptr,
                               const int32_t* col_idx, const int32_t* work_order,
                               const int32_t* plan_meta, uint32_t* tile_counter, void* o,
                               float* lse, float* block_lse, void* workspace,
                               size_t workspace_bytes, int64_t* item_trace, void* stream) {
  if (item_trace == nullptr || ((uintptr_t)item_trace & 7u) != 0) return FVA_ERR_ARG;
  return attn_call(prob, q, kv, order, row_ptr, col_idx, work_order, plan_meta, tile_counter, o, lse,
                   block_lse, workspace, workspace_bytes, item_trace, stream);
}

int fva_block_importance(const fva_problem* prob, const int32_t* order, const int32_t* row_ptr,
                         const int32_t* col_idx, const float* lse, const float* block_lse,
                         float* importance, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!order || !row_ptr || !col_idx || !lse || !block_lse || !importance) return FVA_ERR_ARG;
  return launch_block_importance(*prob, nb, order, row_ptr, col_idx, lse, block_lse, importance,
                                 (hipStream_t)stream);
}

int fva_reselect(const fva_problem* prob, const int32_t* row_ptr, const int32_t* col_idx,
                 const float* importance, int16_t* ranked, int32_t* row_count,
                 int32_t* head_count, void* stream) {
  int nb = 0;
  int st = check_problem(prob, &nb);
  if (st) return st;
  if (!row_ptr || !col_idx || !importance || !ranked || !row_count || !head_count) return FVA_ERR_ARG;
  return launch_reselect(*prob, nb, row_ptr, col_idx, importance, ranked, row_count, head_count,
                         (hipStream_t)stream);
}

}  // extern "C"
