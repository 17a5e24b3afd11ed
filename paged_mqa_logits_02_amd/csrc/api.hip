// C ABI of libpmqa.so (declared in include/pmqa.h): host-side validation,
// per-device cached facts, and kernel launches.  No entry point allocates,
// synchronises or reads device memory.
#include <algorithm>
#include <mutex>

#include "pmqa.h"
#include "pmqa_internal.h"

namespace pmqa {
namespace {

constexpr int kMaxDevices = 64;

// Work counters for callers that cannot allocate a workspace
// (mqa_logits_fp8_no_alloc): one 1 KiB array per device, zero when the code
// object is loaded, left zero by every completed launch.  In host code this
// name is only a stand-in: the device address comes from hipGetSymbolAddress
// (DeviceInfo::scratch) and is the only form passed to kernels.
static __device__ __align__(256) WorkCounter scratch[kXcds];
static_assert(sizeof(scratch) >= kWorkspaceBytes, "scratch holds one call's work counters");

struct DeviceInfo {
  bool ready = false;
  int cus = 0;
  size_t lds_per_cu = 0;
  // workgroups per CU of each 64-head kernel instance [slots-1][kernel
  // variant][out] and of each general FP8 instance [ks-1][out], from registers
  // alone, and each instance's static LDS bytes
  int occ[kFastSlots][kKernelVariants][2] = {};
  size_t static_lds[kFastSlots][kKernelVariants][2] = {};
  int occ_any[2][2] = {};
  size_t static_lds_any[2][2] = {};
  // proxy score kernels [row tiles 1, 2, 4 -> 0, 1, 2][reduce]
  int occ_proxy[3][2] = {};
  size_t static_lds_proxy[3][2] = {};
  WorkCounter* scratch = nullptr;  // this device's copy of `scratch`
};

int proxy_nt_index(int nt) { return nt == 1 ? 0 : nt == 2 ? 1 : 2; }

// Resident workgroups per CU of a kernel whose register limit is `occ`,
// launched with `dyn_lds` bytes of dynamic LDS and `static_lds` of static LDS
// (in whole 1 KiB allocation blocks).
int limit_by_lds(const DeviceInfo& d, int occ, size_t static_lds, size_t dyn_lds) {
  if (d.lds_per_cu > 0) {
    const size_t per_block = (dyn_lds + static_lds + 1023) / 1024 * 1024;
    const int by_lds = (int)(d.lds_per_cu / per_block);
    if (by_lds >= 1 && by_lds < occ) occ = by_lds;
  }
  return occ;
}

// MXFP4 kernels keep at most 6 workgroups per CU: the token-record layout with
// bf16 output fits 7 by its registers and LDS and ran 88.8 us against 82-84 us
// at 6 (B=64, next_n 2); the trailing-code layout ran the same at 6 and 7.
constexpr int kMxMaxBlocksPerCu = 6;

int blocks_per_cu(const DeviceInfo& d, int slots, int variant, int out, size_t dyn_lds) {
  const int r = limit_by_lds(d, d.occ[slots - 1][variant][out],
                             d.static_lds[slots - 1][variant][out], dyn_lds);
  return variant != 0 && r > kMxMaxBlocksPerCu ? kMxMaxBlocksPerCu : r;
}

int blocks_per_cu_any(const DeviceInfo& d, int ks, int out, size_t dyn_lds) {
  return limit_by_lds(d, d.occ_any[ks - 1][out], d.static_lds_any[ks - 1][out], dyn_lds);
}

// Register-limited occupancy and static LDS of one kernel; also loads its
// code object.
bool query_kernel(const void* fn, int* occ, size_t* static_lds) {
  int blocks = 0;
  hipFuncAttributes attr;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kBlockThreads, 0) != hipSuccess ||
      hipFuncGetAttributes(&attr, fn) != hipSuccess)
    return false;
  *occ = blocks > 0 ? blocks : 1;
  *static_lds = attr.sharedSizeBytes;
  return true;
}

std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

int init_device(int device) {
  if (device < 0 || device >= kMaxDevices) return PMQA_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_dev[device];
  if (d.ready) return PMQA_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PMQA_ERR_HIP;
  if (cur != device && hipSetDevice(device) != hipSuccess) return PMQA_ERR_HIP;
  int rc = PMQA_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
    rc = PMQA_ERR_HIP;
  } else {
    d.cus = prop.multiProcessorCount;
    d.lds_per_cu = prop.maxSharedMemoryPerMultiProcessor;
    if (hipGetSymbolAddress(reinterpret_cast<void**>(&d.scratch), HIP_SYMBOL(scratch)) !=
            hipSuccess ||
        d.scratch == nullptr)
      rc = PMQA_ERR_HIP;
    // occupancy from registers (LDS is accounted per call: it depends on
    // the batch and the shape)
    for (int n = 1; n <= kFastSlots && rc == PMQA_OK; ++n)
      for (int v = 0; v < kKernelVariants && rc == PMQA_OK; ++v)
        for (int o = 0; o < 2 && rc == PMQA_OK; ++o)
          if (!query_kernel(mqa_kernel_symbol(n, v, o), &d.occ[n - 1][v][o],
                            &d.static_lds[n - 1][v][o]))
            rc = PMQA_ERR_HIP;
    for (int ks = 1; ks <= 2 && rc == PMQA_OK; ++ks)
      for (int o = 0; o < 2 && rc == PMQA_OK; ++o)
        if (!query_kernel(mqa_any_kernel_symbol(ks, o), &d.occ_any[ks - 1][o],
                          &d.static_lds_any[ks - 1][o]))
          rc = PMQA_ERR_HIP;
    for (int i = 0; i < 3 && rc == PMQA_OK; ++i)
      for (int red = 0; red < 2 && rc == PMQA_OK; ++red)
        if (!query_kernel(proxy_kernel_symbol(1 << i, red), &d.occ_proxy[i][red],
                          &d.static_lds_proxy[i][red]))
          rc = PMQA_ERR_HIP;
    hipFuncAttributes attr;
    if (rc == PMQA_OK && (hipFuncGetAttributes(&attr, schedule_kernel_symbol()) != hipSuccess ||
                          hipFuncGetAttributes(&attr, indexer_kernel_symbol()) != hipSuccess ||
                          hipFuncGetAttributes(&attr, indexer_nvfp4_kernel_symbol()) != hipSuccess))
      rc = PMQA_ERR_HIP;
  }
  if (cur != device && hipSetDevice(cur) != hipSuccess) rc = PMQA_ERR_HIP;
  if (rc == PMQA_OK) d.ready = true;
  return rc;
}

int current_device_info(DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PMQA_ERR_HIP;
  int rc = init_device(dev);
  if (rc != PMQA_OK) return rc;
  *out = &g_dev[dev];
  return PMQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Checks shared by both MQA variants.
int check_mqa_common(const void* q, const void* kv, int64_t page_stride, int32_t num_pages,
                     const float* w, const int32_t* seq_lens, const int32_t* bt,
                     int64_t bt_stride, int32_t bt_width, int32_t batch, int32_t next_n,
                     void* out, int64_t out_row_stride, int32_t max_context, int64_t min_stride) {
  if (batch < 0 || batch > PMQA_MAX_BATCH) return PMQA_ERR_SHAPE;
  if (next_n < 1 || next_n > 64) return PMQA_ERR_SHAPE;
  if (next_n > PMQA_MAX_NEXT_N) return PMQA_ERR_UNSUPPORTED;
  if (max_context < 0 || max_context % PMQA_PAGE_TOKENS != 0) return PMQA_ERR_SHAPE;
  if (batch == 0 || max_context == 0) return PMQA_OK;  // nothing to do (caller checks null)
  if (!q || !kv || !w || !seq_lens || !bt || !out) return PMQA_ERR_NULL;
  if (num_pages < 1) return PMQA_ERR_SHAPE;
  if (page_stride < min_stride) return PMQA_ERR_SHAPE;
  if (page_stride % 16 != 0) return PMQA_ERR_ALIGN;
  if (bt_width < 1 || bt_stride < bt_width) return PMQA_ERR_SHAPE;
  if ((int64_t)bt_width * PMQA_PAGE_TOKENS < max_context) return PMQA_ERR_SHAPE;
  if (out_row_stride < max_context) return PMQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(w)) return PMQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_lens) | reinterpret_cast<uintptr_t>(bt)) & 3)
    return PMQA_ERR_ALIGN;
  return PMQA_OK;
}

// Launches the kernels of one call on `stream`, one launch per pass over a
// group of query slots (each pass writes its own output rows).  64 heads with
// head_dim 128 take the kernels specialised for that shape, up to 4 slots a
// pass; any other FP8 shape takes the general kernel, as many slots a pass as
// its LDS budget for the query slice allows.
int run_mqa(const void* q, const void* q_sf, const void* kv, int64_t page_stride,
            int32_t num_pages, const float* w, const int32_t* seq_lens, const int32_t* bt,
            int64_t bt_stride, int32_t batch, int32_t next_n, int32_t heads, int32_t head_dim,
            int variant, void* out, int64_t out_row_stride, int32_t max_context,
            int32_t out_dtype, const int32_t* schedule, WorkCounter* work, void* stream) {
  DeviceInfo* d = nullptr;
  int rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  MqaArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.q_sf = static_cast<const uint8_t*>(q_sf);
  a.kv = static_cast<const uint8_t*>(kv);
  a.page_stride = page_stride;
  a.w = w;
  a.seq_lens = seq_lens;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.out = out;
  a.out_row_stride = out_row_stride;
  a.schedule = schedule;
  a.num_pages = num_pages;
  a.batch = batch;
  a.max_context = max_context;
  a.next_n = next_n;
  a.heads = heads;
  a.head_dim = head_dim;
  a.cus = d->cus;
  a.split_skew = 0;
  a.dyn_share = 0;
  a.dyn_chunk = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t prefix = (size_t)(batch + 1) * sizeof(int);
  if (heads == 64 && head_dim == 128) {
    for (int s0 = 0; s0 < next_n; s0 += kFastSlots) {
      a.slot0 = s0;
      a.slots = next_n - s0 < kFastSlots ? next_n - s0 : kFastSlots;
      const size_t lds = mqa_ring_bytes(variant, a.slots) + prefix;
      a.split_skew = split_skew_for(a.slots, variant);
      a.dyn_share = dyn_share_for(a.slots, variant);
      a.dyn_chunk = dyn_chunk_for(a.slots, variant);
      const int grid = d->cus * blocks_per_cu(*d, a.slots, variant, out_dtype, lds);
      // the counter serves the in-call split only; the launches of one call
      // run one after the other on the stream, each leaving it zero
      if (launch_mqa(a, a.slots, variant, out_dtype, grid, lds, schedule ? nullptr : work, s) !=
          hipSuccess)
        return PMQA_ERR_HIP;
    }
    return PMQA_OK;
  }
  if (variant != PMQA_VARIANT_FP8) return PMQA_ERR_UNSUPPORTED;
  const int ks = (head_dim + 127) / 128;
  const int hp = (heads + 31) / 32 * 32;
  int per = kAnyQueryBudget / (ks * 128 * hp);
  if (per < 1) return PMQA_ERR_UNSUPPORTED;
  for (int s0 = 0; s0 < next_n; s0 += per) {
    a.slot0 = s0;
    a.slots = next_n - s0 < per ? next_n - s0 : per;
    const size_t lds = mqa_any_lds_bytes(ks, hp, a.slots) + prefix;
    const int grid = d->cus * blocks_per_cu_any(*d, ks, out_dtype, lds);
    if (launch_mqa_any(a, ks, out_dtype, grid, lds, s) != hipSuccess) return PMQA_ERR_HIP;
  }
  return PMQA_OK;
}

}  // namespace
}  // namespace pmqa

using namespace pmqa;

extern "C" {

// A caller workspace: NULL (no work counter), or at least kWorkspaceBytes,
// 16-B aligned.
static int check_workspace(const void* workspace, size_t workspace_bytes) {
  if (!workspace) return PMQA_OK;
  if (workspace_bytes < kWorkspaceBytes) return PMQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PMQA_ERR_ALIGN;
  return PMQA_OK;
}

int mqa_logits_fp8(const void* q, const void* kv_fused, int64_t page_stride, int32_t num_pages,
                   const float* weights, const int32_t* seq_lens, const int32_t* block_table,
                   int64_t bt_stride, int32_t bt_width, int32_t batch, int32_t next_n,
                   int32_t num_heads, int32_t head_dim, void* out, int64_t out_row_stride,
                   int32_t max_context, int32_t out_dtype, int32_t acc_dtype,
                   const int32_t* schedule, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int wrc = check_workspace(workspace, workspace_bytes);
  if (wrc != PMQA_OK) return wrc;
  if (num_heads < 1 || head_dim < 1) return PMQA_ERR_SHAPE;
  if (num_heads > kAnyMaxHeads || head_dim > kAnyMaxDim || head_dim % 16 != 0)
    return PMQA_ERR_UNSUPPORTED;
  if (out_dtype != PMQA_F32 && out_dtype != PMQA_BF16) return PMQA_ERR_UNSUPPORTED;
  if (acc_dtype != PMQA_F32) return PMQA_ERR_UNSUPPORTED;
  int rc = check_mqa_common(q, kv_fused, page_stride, num_pages, weights, seq_lens, block_table,
                            bt_stride, bt_width, batch, next_n, out, out_row_stride, max_context,
                            (int64_t)PMQA_PAGE_TOKENS * (head_dim + 4));
  if (rc != PMQA_OK || batch == 0 || max_context == 0) return rc;
  return run_mqa(q, nullptr, kv_fused, page_stride, num_pages, weights, seq_lens, block_table,
                 bt_stride, batch, next_n, num_heads, head_dim, PMQA_VARIANT_FP8, out,
                 out_row_stride, max_context, out_dtype, schedule,
                 static_cast<WorkCounter*>(workspace), stream);
}

int mqa_logits_fp8_no_alloc(const void* q, const void* kv_fused, int64_t page_stride,
                            int32_t num_pages, const float* weights, const int32_t* seq_lens,
                            const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                            int32_t batch, int32_t next_n, int32_t num_heads, int32_t head_dim,
                            void* out, int64_t out_row_stride, int32_t max_context,
                            int32_t out_dtype, int32_t acc_dtype, const int32_t* schedule,
                            void* stream) {
  DeviceInfo* d = nullptr;
  int rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  if (sizeof(scratch) < kWorkspaceBytes) return PMQA_ERR_WORKSPACE;
  return mqa_logits_fp8(q, kv_fused, page_stride, num_pages, weights, seq_lens, block_table,
                        bt_stride, bt_width, batch, next_n, num_heads, head_dim, out,
                        out_row_stride, max_context, out_dtype, acc_dtype, schedule, d->scratch,
                        kWorkspaceBytes, stream);
}

int mqa_logits_mxfp4(const void* q, const void* q_sf, int32_t sf_vec_size,
                     int32_t is_kv_sf_interleaved, const void* kv_fused, int64_t page_stride,
                     int32_t num_pages, const float* weights, const int32_t* seq_lens,
                     const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                     int32_t batch, int32_t next_n, int32_t num_heads, int32_t head_dim,
                     void* out, int64_t out_row_stride, int32_t max_context, int32_t out_dtype,
                     const int32_t* schedule, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int wrc = check_workspace(workspace, workspace_bytes);
  if (wrc != PMQA_OK) return wrc;
  if (num_heads < 1 || head_dim < 1) return PMQA_ERR_SHAPE;
  if (num_heads != 64 || head_dim != 128) return PMQA_ERR_UNSUPPORTED;
  if (sf_vec_size != 16 && sf_vec_size != 32) return PMQA_ERR_UNSUPPORTED;
  if (is_kv_sf_interleaved != 0 && is_kv_sf_interleaved != 1) return PMQA_ERR_UNSUPPORTED;
  if (out_dtype != PMQA_F32 && out_dtype != PMQA_BF16) return PMQA_ERR_UNSUPPORTED;
  int rc = check_mqa_common(q, kv_fused, page_stride, num_pages, weights, seq_lens, block_table,
                            bt_stride, bt_width, batch, next_n, out, out_row_stride, max_context,
                            (int64_t)PMQA_PAGE_TOKENS * (head_dim / 2 + head_dim / sf_vec_size));
  if (rc != PMQA_OK || batch == 0 || max_context == 0) return rc;
  if (!q_sf) return PMQA_ERR_NULL;
  return run_mqa(q, q_sf, kv_fused, page_stride, num_pages, weights, seq_lens, block_table,
                 bt_stride, batch, next_n, num_heads, head_dim,
                 mx_kernel_variant(sf_vec_size, is_kv_sf_interleaved), out, out_row_stride,
                 max_context, out_dtype, schedule, static_cast<WorkCounter*>(workspace), stream);
}

// Validation shared by both indexer entry points; key_bytes is the packed size
// of one page of keys.  Returns PMQA_OK with *launch = false when there is
// nothing to do.
static int check_indexer(const void* query, int32_t rows, int32_t head_dim, const void* key_cache,
                  int64_t page_stride, int64_t key_bytes, int32_t num_pages,
                  const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                  int32_t num_requests, const int32_t* context_lengths, const int32_t* requests,
                  int32_t groups, const int32_t* group_row_offsets, float* scores,
                  int64_t scores_row_stride, int32_t max_context, int* uniform_g, bool* launch) {
  *launch = false;
  if (rows < 0 || groups < 0 || groups > 65535 || head_dim < 1) return PMQA_ERR_SHAPE;
  if (head_dim != 128) return PMQA_ERR_UNSUPPORTED;
  if (max_context < 0 || max_context % PMQA_PAGE_TOKENS != 0) return PMQA_ERR_SHAPE;
  if (max_context / PMQA_PAGE_TOKENS > 65535) return PMQA_ERR_SHAPE;  // grid.y = pages
  if (groups > 0 && rows < 1) return PMQA_ERR_SHAPE;
  *uniform_g = 0;
  if (!group_row_offsets && groups > 0) {
    if (rows % groups != 0) return PMQA_ERR_SHAPE;
    *uniform_g = rows / groups;
    if (*uniform_g < 1 || *uniform_g > 8) return PMQA_ERR_SHAPE;
  }
  if (groups == 0 || max_context == 0) return PMQA_OK;
  if (!query || !key_cache || !block_table || !context_lengths || !requests || !scores)
    return PMQA_ERR_NULL;
  if (num_pages < 1 || num_requests < 1) return PMQA_ERR_SHAPE;
  if (page_stride < key_bytes) return PMQA_ERR_SHAPE;
  if (page_stride % 16 != 0) return PMQA_ERR_ALIGN;
  if (bt_width < 1 || bt_stride < bt_width) return PMQA_ERR_SHAPE;
  if ((int64_t)bt_width * PMQA_PAGE_TOKENS < max_context) return PMQA_ERR_SHAPE;
  if (scores_row_stride < max_context) return PMQA_ERR_SHAPE;
  if (!aligned16(query) || !aligned16(key_cache)) return PMQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(block_table) |
       reinterpret_cast<uintptr_t>(context_lengths) | reinterpret_cast<uintptr_t>(requests) |
       reinterpret_cast<uintptr_t>(group_row_offsets)) & 3)
    return PMQA_ERR_ALIGN;
  *launch = true;
  return PMQA_OK;
}

int indexer_scores(const void* query, int32_t rows, int32_t head_dim, const void* key_cache,
                   int64_t page_stride, int32_t num_pages, const int32_t* block_table,
                   int64_t bt_stride, int32_t bt_width, int32_t num_requests,
                   const int32_t* context_lengths, const int32_t* requests, int32_t groups,
                   const int32_t* group_row_offsets, float* scores, int64_t scores_row_stride,
                   int32_t max_context, void* stream) {
  int uniform_g = 0;
  bool launch = false;
  int rc = check_indexer(query, rows, head_dim, key_cache, page_stride,
                         (int64_t)PMQA_PAGE_TOKENS * 128 * 2, num_pages, block_table, bt_stride,
                         bt_width, num_requests, context_lengths, requests, groups,
                         group_row_offsets, scores, scores_row_stride, max_context, &uniform_g,
                         &launch);
  if (rc != PMQA_OK || !launch) return rc;
  DeviceInfo* d = nullptr;
  rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  IdxArgs a;
  a.q = static_cast<const uint16_t*>(query);
  a.kc = static_cast<const uint8_t*>(key_cache);
  a.page_stride = page_stride;
  a.qs = nullptr;
  a.ks = nullptr;
  a.scale_page_stride = 0;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.lens = context_lengths;
  a.reqs = requests;
  a.offs = group_row_offsets;
  a.scores = scores;
  a.srs = scores_row_stride;
  a.num_pages = num_pages;
  a.num_requests = num_requests;
  a.rows = rows;
  a.groups = groups;
  a.uniform_g = uniform_g;
  a.max_context = max_context;
  if (launch_indexer(a, static_cast<hipStream_t>(stream)) != hipSuccess) return PMQA_ERR_HIP;
  return PMQA_OK;
}

int indexer_scores_nvfp4(const void* query, const void* query_scales, int32_t rows,
                         int32_t head_dim, const void* key_cache, int64_t page_stride,
                         const void* key_scales, int64_t scale_page_stride, int32_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                         int32_t num_requests, const int32_t* context_lengths,
                         const int32_t* requests, int32_t groups,
                         const int32_t* group_row_offsets, float* scores,
                         int64_t scores_row_stride, int32_t max_context, void* stream) {
  int uniform_g = 0;
  bool launch = false;
  int rc = check_indexer(query, rows, head_dim, key_cache, page_stride,
                         (int64_t)PMQA_PAGE_TOKENS * 128 / 2, num_pages, block_table, bt_stride,
                         bt_width, num_requests, context_lengths, requests, groups,
                         group_row_offsets, scores, scores_row_stride, max_context, &uniform_g,
                         &launch);
  if (rc != PMQA_OK || !launch) return rc;
  if (!query_scales || !key_scales) return PMQA_ERR_NULL;
  if (scale_page_stride < (int64_t)PMQA_PAGE_TOKENS * 8) return PMQA_ERR_SHAPE;
  if (scale_page_stride % 8 != 0) return PMQA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(query_scales) | reinterpret_cast<uintptr_t>(key_scales)) & 1)
    return PMQA_ERR_ALIGN;
  DeviceInfo* d = nullptr;
  rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  IdxArgs a;
  a.q = static_cast<const uint16_t*>(query);
  a.kc = static_cast<const uint8_t*>(key_cache);
  a.page_stride = page_stride;
  a.qs = static_cast<const uint8_t*>(query_scales);
  a.ks = static_cast<const uint8_t*>(key_scales);
  a.scale_page_stride = scale_page_stride;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.lens = context_lengths;
  a.reqs = requests;
  a.offs = group_row_offsets;
  a.scores = scores;
  a.srs = scores_row_stride;
  a.num_pages = num_pages;
  a.num_requests = num_requests;
  a.rows = rows;
  a.groups = groups;
  a.uniform_g = uniform_g;
  a.max_context = max_context;
  if (launch_indexer_nvfp4(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PMQA_ERR_HIP;
  return PMQA_OK;
}

int msa_proxy_score_fp4(const void* q_fp4, const void* q_scale, int32_t total_q,
                        int32_t num_qo_heads, const void* k_fp4, const void* k_scale,
                        int32_t num_kv_heads, int64_t page_stride, int32_t num_pages,
                        int64_t total_k, float q_global_scale, float k_global_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* page_table, int64_t pt_stride, int32_t pt_width,
                        const int32_t* seqused_k, int32_t batch, int32_t causal,
                        const int32_t* q_offset, int32_t max_seqlen_q, int32_t max_k_tiles,
                        int32_t reduce_heads, float* out, void* stream) {
  const bool paged = page_table != nullptr;
  if (total_q < 0 || batch < 0 || max_k_tiles < 0 || max_seqlen_q < 0) return PMQA_ERR_SHAPE;
  if (num_qo_heads < 1 || num_kv_heads < 1 || num_qo_heads % num_kv_heads != 0)
    return PMQA_ERR_SHAPE;
  const int group = num_qo_heads / num_kv_heads;
  if (group > 64 || batch > kProxyMaxBatch) return PMQA_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_heads * total_q * max_k_tiles >= ((int64_t)1 << 31))
    return PMQA_ERR_UNSUPPORTED;
  if (total_q == 0 || max_k_tiles == 0) return PMQA_OK;  // no output
  if (!out || !cu_seqlens_q) return PMQA_ERR_NULL;
  if (batch > 0) {
    if (!q_fp4 || !q_scale || !k_fp4 || !k_scale) return PMQA_ERR_NULL;
    if (paged) {
      if (!seqused_k) return PMQA_ERR_NULL;
      if (num_pages < 1 || pt_width < 1 || pt_stride < pt_width) return PMQA_ERR_SHAPE;
      if (pt_width > (1 << 23)) return PMQA_ERR_UNSUPPORTED;
      if (page_stride < (int64_t)num_kv_heads * 128 * 64) return PMQA_ERR_SHAPE;
      if (page_stride % 16 != 0) return PMQA_ERR_ALIGN;
    } else {
      if (!cu_seqlens_k) return PMQA_ERR_NULL;
      if (total_k < 0) return PMQA_ERR_SHAPE;
    }
  }
  if (((uintptr_t)q_fp4 | (uintptr_t)k_fp4) & 15) return PMQA_ERR_ALIGN;
  if (((uintptr_t)q_scale | (uintptr_t)k_scale) & 1) return PMQA_ERR_ALIGN;
  if (((uintptr_t)out | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k |
       (uintptr_t)page_table | (uintptr_t)seqused_k | (uintptr_t)q_offset) & 3)
    return PMQA_ERR_ALIGN;
  DeviceInfo* d = nullptr;
  int rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  // row tiles: every query head of a KV head's group for as many tokens as
  // the longest request has, up to 64 rows
  const int maxq = max_seqlen_q > 0 ? max_seqlen_q : (total_q > 0 ? total_q : 1);
  const int64_t want = std::min<int64_t>((int64_t)group * maxq, 64);
  const int nt = want <= 16 ? 1 : want <= 32 ? 2 : 4;
  int tc = 16 * nt / group;
  if (tc > maxq) tc = maxq;
  if (tc < 1) tc = 1;
  ProxyArgs a;
  a.q = static_cast<const uint8_t*>(q_fp4);
  a.qs = static_cast<const uint8_t*>(q_scale);
  a.k = static_cast<const uint8_t*>(k_fp4);
  a.ks = static_cast<const uint8_t*>(k_scale);
  a.cu_q = cu_seqlens_q;
  a.cu_k = paged ? nullptr : cu_seqlens_k;
  a.pt = paged ? page_table : nullptr;
  a.seqused = paged ? seqused_k : nullptr;
  a.q_offset = q_offset;
  a.out = out;
  a.page_stride = paged ? page_stride : 0;
  a.pt_stride = paged ? pt_stride : 0;
  a.total_k = paged ? 0 : total_k;
  a.pt_width = paged ? pt_width : 0;
  a.num_pages = paged ? num_pages : 0;
  a.total_q = total_q;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.group = group;
  a.tc = tc;
  a.batch = batch;
  a.max_k_tiles = max_k_tiles;
  a.causal = causal ? 1 : 0;
  a.paged = paged ? 1 : 0;
  a.reduce = reduce_heads ? 1 : 0;
  a.g = q_global_scale * k_global_scale;
  const int i = proxy_nt_index(nt);
  const int per_cu = limit_by_lds(*d, d->occ_proxy[i][a.reduce], d->static_lds_proxy[i][a.reduce],
                                  proxy_lds_bytes(batch));
  if (launch_proxy(a, nt, d->cus * per_cu, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PMQA_ERR_HIP;
  return PMQA_OK;
}

size_t mqa_logits_workspace_bytes(void) { return kWorkspaceBytes; }

int64_t mqa_logits_schedule_ints(int32_t num_units) {
  if (num_units < 1 || num_units > (1 << 20)) return -1;
  return kSchedHeader + 3 * ((int64_t)num_units + 1);
}

int32_t mqa_logits_num_units(int device, int32_t next_n, int32_t variant) {
  if (next_n < 1 || next_n > PMQA_MAX_NEXT_N) return PMQA_ERR_UNSUPPORTED;
  if (variant != PMQA_VARIANT_FP8 && variant != PMQA_VARIANT_MXFP4) return PMQA_ERR_UNSUPPORTED;
  int rc = init_device(device);
  if (rc != PMQA_OK) return rc;
  const DeviceInfo& d = g_dev[device];
  const int out = variant == PMQA_VARIANT_FP8 ? 0 : 1;  // the variant's default output
  // one unit per resident workgroup of the first pass of a 64-head, head_dim
  // 128 call: a workgroup pays the start-up of a range (page ids, first page
  // loads, query) once per unit
  const int slots = next_n < kFastSlots ? next_n : kFastSlots;
  const size_t lds = mqa_ring_bytes(variant, slots) + sizeof(int);
  return d.cus * blocks_per_cu(d, slots, variant, out, lds);
}

int mqa_logits_schedule(const int32_t* seq_lens, int32_t batch, int32_t next_n, int32_t variant,
                        int32_t max_context, int32_t num_units, int32_t* schedule,
                        void* stream) {
  if (batch < 0 || batch > PMQA_MAX_BATCH) return PMQA_ERR_SHAPE;
  if (next_n < 1 || next_n > 64) return PMQA_ERR_SHAPE;
  if (next_n > PMQA_MAX_NEXT_N) return PMQA_ERR_UNSUPPORTED;
  if (variant != PMQA_VARIANT_FP8 && variant != PMQA_VARIANT_MXFP4) return PMQA_ERR_UNSUPPORTED;
  if (max_context < 0 || max_context % PMQA_PAGE_TOKENS != 0) return PMQA_ERR_SHAPE;
  if (num_units < 0 || num_units > (1 << 20)) return PMQA_ERR_SHAPE;
  if (!schedule || (batch > 0 && !seq_lens)) return PMQA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(schedule) | reinterpret_cast<uintptr_t>(seq_lens)) & 3)
    return PMQA_ERR_ALIGN;
  DeviceInfo* d = nullptr;
  int rc = current_device_info(&d);
  if (rc != PMQA_OK) return rc;
  if (num_units == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PMQA_ERR_HIP;
    num_units = mqa_logits_num_units(dev, next_n, variant);
    if (num_units < 0) return num_units;
  }
  // the split of the call's first launch (64 heads x 128): the units are the
  // workgroups of that launch when num_units is the default
  const int skew = split_skew_for(next_n < kFastSlots ? next_n : kFastSlots, variant);
  if (launch_schedule(seq_lens, batch, next_n, variant, max_context, num_units, d->cus, skew,
                      schedule, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PMQA_ERR_HIP;
  return PMQA_OK;
}

int32_t mqa_logits_padded_seq_len(int32_t seq_len, int32_t next_n, int32_t variant) {
  (void)next_n;
  (void)variant;
  if (seq_len <= 0) return 0;
  return (int32_t)(((int64_t)seq_len + PMQA_PAGE_TOKENS - 1) / PMQA_PAGE_TOKENS *
                   PMQA_PAGE_TOKENS);
}

int32_t mqa_logits_min_block_table_width(int32_t max_seq_len, int32_t next_n, int32_t variant) {
  (void)next_n;
  (void)variant;
  if (max_seq_len <= 0) return 0;
  return (int32_t)(((int64_t)max_seq_len + PMQA_PAGE_TOKENS - 1) / PMQA_PAGE_TOKENS);
}

int mqa_logits_init(int device) { return init_device(device); }

const char* mqa_logits_status_string(int status) {
  switch (status) {
    case PMQA_OK: return "PMQA_OK";
    case PMQA_ERR_NULL: return "PMQA_ERR_NULL: a required pointer is NULL";
    case PMQA_ERR_SHAPE: return "PMQA_ERR_SHAPE: a size or stride is out of range";
    case PMQA_ERR_UNSUPPORTED: return "PMQA_ERR_UNSUPPORTED: option not implemented";
    case PMQA_ERR_ALIGN: return "PMQA_ERR_ALIGN: pointer or stride misaligned";
    case PMQA_ERR_WORKSPACE: return "PMQA_ERR_WORKSPACE: workspace smaller than mqa_logits_workspace_bytes()";
    case PMQA_ERR_HIP: return "PMQA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown pmqa status";
  }
}

}  // extern "C"
