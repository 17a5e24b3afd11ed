// One-head BF16 indexer scores on gfx950.
//
// scores[r, k] = query[r] . key_k for every query row r of group g and every
// key k below the group's length, keys gathered through the group's
// block-table row in pages of 64 (FlashInfer "flashinfer.sdsa.indexer_scores":
// one head, so no weight and no rectifier; only pages below the length are
// read; later entries are not written).
//
// One wavefront per (group, page): the group's 1..8 query rows form the A
// operand of 16x16x32 bf16 MFMAs (rows padded to 16 with zeros), the page's
// 64 keys the B operand in four 16-token tiles; head_dim 128 is four K steps.
#include "device.hpp"
#include "pmqa_internal.h"

namespace pmqa {

__global__ void __launch_bounds__(64) indexer_kernel(const IdxArgs a) {
  const int g = blockIdx.y;
  const int pi = blockIdx.x;
  const int lane = threadIdx.x;
  int L = a.lens[g];
  L = L < a.max_context ? L : a.max_context;
  if (L <= pi * kPage) return;  // also every group of length <= 0

  int r0, G;
  if (a.offs) {
    r0 = a.offs[g];
    G = a.offs[g + 1] - r0;
  } else {
    r0 = g * a.uniform_g;
    G = a.uniform_g;
  }
  if (G < 1 || G > 8 || r0 < 0 || r0 + G > a.rows) return;

  const int req = a.reqs[g];
  bool bad = (unsigned)req >= (unsigned)a.num_requests;
  int pg = bad ? 0 : a.bt[(long long)req * a.bt_stride + pi];
  bad = bad || (unsigned)pg >= (unsigned)a.num_pages;

  const int kg = lane >> 4, r = lane & 15;
  // A: row r of the group, d in [32ks + 8kg, 32ks + 8kg + 8)
  v8bf qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (r < G) qa[ks] = ldg<v8bf>(a.q + (long long)(r0 + r) * 128 + 32 * ks + 8 * kg);
    else qa[ks] = (v8bf){};
  }

  const uint8_t* page = a.kc + (long long)pg * a.page_stride;
  v4f acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    acc[s] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (!bad) {
      const uint16_t* key = reinterpret_cast<const uint16_t*>(page) + (16 * s + r) * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8bf kb = ldg_stream<v8bf>(key + 32 * ks + 8 * kg);
        acc[s] = mfma_bf16(qa[ks], kb, acc[s]);
      }
    }
  }
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int col = pi * kPage + 16 * s + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kg + i;
      if (row < G && col < L) a.scores[(long long)(r0 + row) * a.srs + col] = bad ? nan : acc[s][i];
    }
  }
}

hipError_t launch_indexer(const IdxArgs& a, hipStream_t stream) {
  dim3 grid(a.max_context / kPage, a.groups);
  hipLaunchKernelGGL(indexer_kernel, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

const void* indexer_kernel_symbol() { return reinterpret_cast<const void*>(&indexer_kernel); }

}  // namespace pmqa
