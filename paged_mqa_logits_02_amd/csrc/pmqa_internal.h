// Internal interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmqa {

constexpr int kBlockThreads = 256;        // 4 wavefronts per workgroup
constexpr int kSchedMagic = 0x41514D50;   // "PMQA"
constexpr int kSchedHeader = 8;           // int32 header entries of a schedule
constexpr int kMaxBatch = 8192;           // prefix of page counts kept in LDS

// Arguments of the MQA logits kernels (FP8 and MXFP4).
struct MqaArgs {
  const uint8_t* q;        // fp8 [B,N,H,D] or packed fp4 [B,N,64,64]
  const uint8_t* q_sf;     // e8m0 [B,N,64,128/sf_vec_size] (MXFP4 only)
  const uint8_t* kv;       // pages
  long long page_stride;   // bytes between pages
  const float* w;          // [B*N, H]
  const int32_t* seq_lens; // [B]
  const int32_t* bt;       // [B, bt_stride]
  long long bt_stride;
  void* out;               // [B*N, out_row_stride] f32 or bf16
  long long out_row_stride;
  const int32_t* schedule; // nullable
  int num_pages;
  int batch;
  int max_context;
  int next_n;              // N: query slots per request (row b*N + t of q, w and out)
  int slot0;               // first slot scored by this launch (a pass over slots)
  int slots;               // slots scored by this launch
  int heads;               // H
  int head_dim;            // D (bytes of an FP8 key row)
  int cus;                 // compute units of the device (split weights)
  int split_skew;          // in-call split: extra share of early dispatch rounds, 1/1024ths
  int dyn_share;           // in-call split with a work counter: items left for dynamic
                           // chunks, 1/1024ths of the call's items
  int dyn_chunk;           // items per dynamic chunk
};

// Work counters of the in-call split (in the caller's workspace or the
// library's static scratch): one per XCD, each on its own 128-byte line,
// counting the chunk grabs of that XCD's workgroups.  Zero before a launch;
// the launch's last grab on each XCD returns its counter to zero.
constexpr int kXcds = 8;
struct WorkCounter {
  int next;
  int pad[31];
};
constexpr size_t kWorkspaceBytes = kXcds * sizeof(WorkCounter);  // 1 KiB per call

struct IdxArgs {
  const uint16_t* q;        // bf16 [rows, 128]; NVFP4: packed e2m1 [rows, 64]
  const uint8_t* kc;        // pages of bf16 [64, 128]; NVFP4: packed e2m1 [64, 64]
  long long page_stride;
  const uint8_t* qs;        // NVFP4 only: e4m3 [rows, 8]
  const uint8_t* ks;        // NVFP4 only: pages of e4m3 [64, 8]
  long long scale_page_stride;
  const int32_t* bt;        // [num_requests, bt_stride]
  long long bt_stride;
  const int32_t* lens;      // [groups]
  const int32_t* reqs;      // [groups]
  const int32_t* offs;      // [groups+1] or null
  float* scores;            // [rows, srs]
  long long srs;
  int num_pages;
  int num_requests;
  int rows;
  int groups;
  int uniform_g;            // rows per group when offs == null
  int max_context;
};

// Arguments of the block-max proxy score kernel (NVFP4 query and keys).
struct ProxyArgs {
  const uint8_t* q;         // packed e2m1 [total_q, hq, 64]
  const uint8_t* qs;        // e4m3 [total_q * hq, 8]
  const uint8_t* k;         // paged: page i at k + i*page_stride, [hkv, 128, 64]; flat: [total_k, hkv, 64]
  const uint8_t* ks;        // e4m3 rows of 8: paged (page*hkv + kv_head)*128 + token; flat token*hkv + kv_head
  const int32_t* cu_q;      // [batch+1]
  const int32_t* cu_k;      // flat: [batch+1]
  const int32_t* pt;        // paged: [batch, pt_stride]
  const int32_t* seqused;   // paged: [batch]
  const int32_t* q_offset;  // [batch] or null (Lk - Lq)
  float* out;               // [reduce ? 1 : hq, max_k_tiles, total_q]
  long long page_stride;
  long long pt_stride;
  long long total_k;        // flat: key rows per KV head
  int pt_width;
  int num_pages;
  int total_q;
  int hq, hkv, group;       // group = hq / hkv
  int tc;                   // query tokens per unit
  int batch;
  int max_k_tiles;
  int causal, paged, reduce;
  float g;                  // q_global_scale * k_global_scale
};
constexpr int kProxyMaxBatch = 4096;  // request tables kept in LDS
const void* proxy_kernel_symbol(int nt, int reduce);
size_t proxy_lds_bytes(int batch);
hipError_t launch_proxy(const ProxyArgs& a, int nt, int grid, hipStream_t stream);

// Kernels for 64 heads and head_dim 128, one instance per slot count of a
// pass (1..kFastSlots) and kernel variant: 0 is FP8; 1..4 are MXFP4 with
// one e8m0 code per sf_vec_size values (32 or 16), the key codes either
// after all packed rows of a page or right after each token's packed bytes.
constexpr int kFastSlots = 4;
constexpr int kKernelVariants = 5;
inline int mx_kernel_variant(int sf_vec_size, int kv_sf_interleaved) {
  return 1 + (sf_vec_size == 16 ? 1 : 0) + (kv_sf_interleaved ? 2 : 0);
}
// Skew of the work split toward early dispatch rounds (1/1024ths) for a
// launch of `slots` query slots of `variant` (measured: 4 FP8 slots, whose
// launches are long enough for the rounds to drift apart, gain ~4%).
inline int split_skew_for(int slots, int variant) { return slots == 4 && variant == 0 ? 300 : 0; }
// Dynamic part of the in-call split when a work counter is given: share of
// the call's items (1/1024ths) dealt in chunks of dyn_chunk_for items.
// Measured (shares 0..256/1024, chunks 2..16): every setting is within
// run-to-run noise of the static split for FP8 and slower for MXFP4 (a chunk
// pays its own page-id and first-page round trips), so FP8 keeps a small
// dynamic share and MXFP4 none.
inline int dyn_share_for(int slots, int variant) {
  return variant != 0 ? 0 : slots == 1 ? 32 : 64;
}
inline int dyn_chunk_for(int slots, int variant) { return variant == 0 && slots == 1 ? 2 : 4; }
const void* mqa_kernel_symbol(int slots, int variant, int out_dtype);
// LDS before the request prefix of a launch of `slots` query slots
size_t mqa_ring_bytes(int variant, int slots);

// FP8 kernels for any head count and head_dim: ks = head_dim planes of 128 B
// (1 or 2).  LDS: ring, query slice, weights, then the request prefix.
constexpr int kAnyMaxHeads = 128;
constexpr int kAnyMaxDim = 256;
constexpr int kAnyQueryBudget = 32768;  // bytes of query slice in LDS per pass
const void* mqa_any_kernel_symbol(int ks, int out_dtype);
size_t mqa_any_lds_bytes(int ks, int heads_padded, int slots);  // excluding the prefix
hipError_t launch_mqa_any(const MqaArgs& a, int ks, int out_dtype, int grid, size_t lds_bytes,
                          hipStream_t stream);
const void* schedule_kernel_symbol();
const void* indexer_kernel_symbol();
const void* indexer_nvfp4_kernel_symbol();

hipError_t launch_mqa(const MqaArgs& a, int slots, int variant, int out_dtype, int grid,
                      size_t lds_bytes, WorkCounter* work, hipStream_t stream);
hipError_t launch_schedule(const int32_t* seq_lens, int B, int next_n, int variant,
                           int max_context, int U, int cus, int skew, int32_t* sched,
                           hipStream_t stream);
hipError_t launch_indexer(const IdxArgs& a, hipStream_t stream);
hipError_t launch_indexer_nvfp4(const IdxArgs& a, hipStream_t stream);

}  // namespace pmqa
