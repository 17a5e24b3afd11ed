// Read-stream calibration kernel (a measurement tool, not part of the paged
// MQA logits path; built into its own library, libpmqa_calib.so).
//
// Reads whole pages of `page_bytes` bytes, in the order of a list of page ids,
// from a pool of pages `page_stride` bytes apart, the way the logits and
// indexer kernels gather KV pages through a block table, and does nothing with
// the bytes but fold them into one word per thread (so that no load can be
// removed).  The rate it reaches is the page-gather read rate of the GPU for
// that page size, against which the kernels' byte rates can be read.
//
// Each workgroup takes a batch of pages at a time (pages i, i + G, i + 2G, ...
// of the list, G the grid size: 32 16-byte loads per thread in all) and issues
// every load of the batch before it folds any, so that the batch is in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 32;     // 16-byte loads in flight per thread
constexpr int kMaxPieces = 8;  // 16-byte loads per thread per page: pages up to 32 KiB

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// P = 16-byte loads per thread per page; BATCH = kSlots / P pages per round.
template <int P>
__global__ void __launch_bounds__(kThreads)
    read_pages_kernel(const uint8_t* __restrict__ pool, long long page_stride, int page_bytes,
                      const int32_t* __restrict__ ids, int n, unsigned* __restrict__ out) {
  constexpr int kBatch = kSlots / P;
  const int pieces = page_bytes / 16;
  unsigned acc = 0;
  for (int i0 = blockIdx.x; i0 < n; i0 += kBatch * gridDim.x) {
    long long idv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + b * gridDim.x;
      idv[b] = i < n ? ids[i] : -1;
    }
    v4u v[kBatch][P];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const long long id = idv[b];
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int c = threadIdx.x + k * kThreads;
        v[b][k] = (v4u){0u, 0u, 0u, 0u};
        if (id >= 0 && c < pieces)
          v[b][k] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u*>(pool + id * page_stride) + c);
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int k = 0; k < P; ++k) acc ^= v[b][k].x ^ v[b][k].y ^ v[b][k].z ^ v[b][k].w;
  }
  out[(long long)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int P>
void launch(const void* pool, long long page_stride, int page_bytes, const int32_t* ids, int n,
            unsigned* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(read_pages_kernel<P>, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(pool), page_stride, page_bytes, ids, n, out);
}

}  // namespace

// Reads the n pages ids[0..n) (each page_bytes bytes, 16 <= page_bytes <=
// 32768 and a multiple of 16, at pool + id * page_stride) with `grid`
// workgroups; writes grid * 256 words to `out` (device memory owned by the
// caller).  Every id must address a page inside the caller's pool.  Returns 0,
// -1 for bad arguments, -6 if the launch fails.  Enqueues on `stream` only.
extern "C" int pmqa_calib_read_pages(const void* pool, long long page_stride, int page_bytes,
                                     const int32_t* ids, int n, unsigned* out, int grid,
                                     hipStream_t stream) {
  if (!pool || !ids || !out || n <= 0 || grid <= 0 || page_bytes < 16 || page_bytes % 16 ||
      page_bytes > 16 * kThreads * kMaxPieces || page_stride < page_bytes || page_stride % 16)
    return -1;
  switch ((page_bytes / 16 + kThreads - 1) / kThreads) {
    case 1: launch<1>(pool, page_stride, page_bytes, ids, n, out, grid, stream); break;
    case 2: launch<2>(pool, page_stride, page_bytes, ids, n, out, grid, stream); break;
    case 3: launch<3>(pool, page_stride, page_bytes, ids, n, out, grid, stream); break;
    case 4: launch<4>(pool, page_stride, page_bytes, ids, n, out, grid, stream); break;
    default: launch<8>(pool, page_stride, page_bytes, ids, n, out, grid, stream); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
