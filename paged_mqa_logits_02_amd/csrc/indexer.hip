// One-head indexer scores on gfx950 (BF16 and NVFP4 inputs).
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
//
// The grid is page-major (x = group, y = page position): the dispatcher hands
// out every group's page p before any group's page p + 1, so groups that share
// a request read each of its pages at nearly the same time and all but the
// first find it in the caches, and the waves past a group's length (which
// exit at once) are spread over the whole launch instead of ending each
// group's run.  Measured against the group-major grid at 8192 query rows:
// BF16 181 -> 137 us, NVFP4 61 -> 51.5 us.
#include "device.hpp"
#include "pmqa_internal.h"

namespace pmqa {

// The group of wave (g, page pi): length, first row, row count and block-table
// row, read together (one round trip; every read is in bounds for g < groups,
// and the request is used only after the length check, so a length-0 group's
// request may hold any value).  The empty asm uses all four values at once, so
// the compiler cannot sink the request's read below the length check (which
// would make it a second round trip).  Returns false if the wave has nothing
// to do.
struct GroupMeta {
  int L, r0, G, req;
};
__device__ __forceinline__ bool group_meta(const IdxArgs& a, int g, int pi, GroupMeta& m) {
  int L = a.lens[g];
  int req = a.reqs[g];
  int r0 = g * a.uniform_g, r1 = r0 + a.uniform_g;
  if (a.offs) {
    r0 = a.offs[g];
    r1 = a.offs[g + 1];
  }
  asm volatile("" : "+s"(L), "+s"(req), "+s"(r0), "+s"(r1));
  m.req = req;
  m.L = L < a.max_context ? L : a.max_context;
  m.r0 = r0;
  m.G = r1 - r0;
  if (m.L <= pi * kPage) return false;  // also every group of length <= 0
  return m.G >= 1 && m.G <= 8 && r0 >= 0 && r0 + m.G <= a.rows;
}

__device__ __forceinline__ void store_scores(const IdxArgs& a, const GroupMeta& m, int pi,
                                             int lane, bool bad, const v4f (&acc)[4]) {
  const int kg = lane >> 4, r = lane & 15;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int col = pi * kPage + 16 * s + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kg + i;
      if (row < m.G && col < m.L)
        a.scores[(long long)(m.r0 + row) * a.srs + col] = bad ? nan : acc[s][i];
    }
  }
}

__global__ void __launch_bounds__(64) indexer_kernel(const IdxArgs a) {
  const int g = blockIdx.x;
  const int pi = blockIdx.y;
  const int lane = threadIdx.x;
  GroupMeta m;
  if (!group_meta(a, g, pi, m)) return;

  bool bad = (unsigned)m.req >= (unsigned)a.num_requests;
  const int pg = bad ? 0 : a.bt[(long long)m.req * a.bt_stride + pi];

  // A: row r of the group, d in [32ks + 8kg, 32ks + 8kg + 8); lanes past the
  // group's rows load its first row (so every load is issued at once, while
  // the block-table entry is in flight) and use zeros.
  const int kg = lane >> 4, r = lane & 15;
  const long long qrow = m.r0 + (r < m.G ? r : 0);
  v8bf qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = ldg<v8bf>(a.q + qrow * 128 + 32 * ks + 8 * kg);

  // B: all four 16-token tiles of the page at once; an out-of-range page id
  // reads page 0 instead and its scores are written as NaN.  Each load
  // instruction covers 64 bytes of 16 rows, so two consecutive instructions
  // read the two halves of each 128-byte line: the loads keep the default
  // (temporal) policy, under which the second finds the line the first
  // brought into L2 (with non-temporal loads L2 fetched ~1.5 lines per line).
  bad = bad || (unsigned)pg >= (unsigned)a.num_pages;
  const uint16_t* keys =
      reinterpret_cast<const uint16_t*>(a.kc + (long long)(bad ? 0 : pg) * a.page_stride);
  v8bf kb[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kb[s][ks] = ldg<v8bf>(keys + (16 * s + r) * 128 + 32 * ks + 8 * kg);
  // every key load is issued before the first product waits for one
  __builtin_amdgcn_sched_barrier(0);

  if (r >= m.G) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = (v8bf){};
  }
  v4f acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    acc[s] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc[s] = mfma_bf16(qa[ks], kb[s][ks], acc[s]);
  }
  store_scores(a, m, pi, lane, bad, acc);
}

// ------------------------------------------------------------------ NVFP4
//
// The same contraction with NVFP4 query rows and keys: packed e2m1, an e4m3
// scale per 16 values (query_scales [rows, 8]; key_scales [pages, 64, 8],
// paged like the keys).  An e2m1 value times an e4m3 scale has at most six
// significant bits, so each side is dequantised exactly into f16 registers and
// the f16 MFMA computes the products exactly, accumulating in fp32.
//
// K mapping: lane (kg = l>>4) holds, in K step ks, head_dim values
// 32kg + 8ks .. 32kg + 8ks + 7, the same for query and key, so the four K
// steps of a lane are one contiguous 16-byte slice of a packed row and two of
// its scales (blocks 2kg and 2kg+1).

// Two e2m1 values of byte B of `packed` (low nibble first) times s, as f16.
// The conversion applies only a power-of-two scale, so it runs with scale 1
// and s (the block's e4m3 scale in both halves) is applied by a packed f16
// multiply.  Exact: the product has at most six significant bits and is 0 or
// of magnitude 2^-10 .. 6 * 448, inside f16's normal range.
template <int B>
__device__ __forceinline__ v2h dequant2(uint32_t packed, v2h s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, B) * s;
}

// Eight dequantised values (one packed dword, scale s).
__device__ __forceinline__ v8h dequant8(uint32_t packed, v2h s) {
  const v2h a = dequant2<0>(packed, s), b = dequant2<1>(packed, s);
  const v2h c = dequant2<2>(packed, s), d = dequant2<3>(packed, s);
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 values of one NVFP4 row (16 packed bytes, two e4m3 scales, each
// widened exactly to f16) as the four K-step fragments.
__device__ __forceinline__ void dequant_row(const v4i& packed, uint32_t scales2, v8h out[4]) {
  const v2h sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)scales2, 1.0f, false);
  const v2h s0 = (v2h){sc[0], sc[0]}, s1 = (v2h){sc[1], sc[1]};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) out[ks] = dequant8((uint32_t)packed[ks], ks < 2 ? s0 : s1);
}

// One wavefront per (group, run of P pages): the group's length, request and
// rows are read once for P pages, then the P block-table entries, then every
// page's keys and scales at once, so a wave pays the chain of dependent
// reads (length, page id, keys) once per P pages.  Pages of the run at or
// beyond the length read page 0 instead (every load is issued the same way,
// and nothing of theirs is stored).
template <int P>
__global__ void __launch_bounds__(64) indexer_nvfp4_kernel(const IdxArgs a) {
  const int g = blockIdx.x;
  const int pi0 = blockIdx.y * P;
  const int lane = threadIdx.x;
  GroupMeta m;
  if (!group_meta(a, g, pi0, m)) return;
  // pages pi0 .. pi0 + np - 1 hold keys below the length (np >= 1)
  const int np = min(P, (m.L - pi0 * kPage + kPage - 1) / kPage);

  const bool req_bad = (unsigned)m.req >= (unsigned)a.num_requests;
  int pg[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    pg[p] = (!req_bad && p < np) ? a.bt[(long long)m.req * a.bt_stride + pi0 + p] : 0;

  // The query row (lanes past the group's rows read its first row and use
  // zeros) and, once the page ids are known, all key tiles of the run, each
  // load issued before any is waited for.
  const int kg = lane >> 4, r = lane & 15;
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q);
  const long long qrow = m.r0 + (r < m.G ? r : 0);
  const v4i qpacked = ldg<v4i>(q8 + qrow * 64 + 16 * kg);
  const uint32_t qsc = *reinterpret_cast<const uint16_t*>(a.qs + qrow * 8 + 2 * kg);

  bool bad[P];
  v4i kpacked[P][4];
  uint32_t ksc[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bad[p] = req_bad || (unsigned)pg[p] >= (unsigned)a.num_pages;
    const long long page_id = bad[p] ? 0 : pg[p];
    const uint8_t* page = a.kc + page_id * a.page_stride;
    const uint8_t* pscale = a.ks + page_id * a.scale_page_stride;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int key = 16 * s + r;
      kpacked[p][s] = ldg<v4i>(page + key * 64 + 16 * kg);
      ksc[p][s] = *reinterpret_cast<const uint16_t*>(pscale + key * 8 + 2 * kg);
    }
  }
  // every load of the run is issued before the first dequantisation waits
  __builtin_amdgcn_sched_barrier(0);

  v8h qa[4];
  dequant_row(qpacked, qsc, qa);
  if (r >= m.G) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = (v8h){};
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p >= np) break;
    v4f acc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8h kb[4];
      dequant_row(kpacked[p][s], ksc[p][s], kb);
      acc[s] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[s] = mfma_f16(qa[ks], kb[ks], acc[s]);
    }
    store_scores(a, m, pi0 + p, lane, bad[p], acc);
  }
}

// One page per wave: runs of 2 or 4 pages hold 2-4x the key registers and were
// measured slower (8192 rows, group-major grid: 77 us for both against
// 61 us), the waves per SIMD falling from 7 to 5 and 4.
constexpr int kNvfp4PagesPerWave = 1;

hipError_t launch_indexer_nvfp4(const IdxArgs& a, hipStream_t stream) {
  constexpr int P = kNvfp4PagesPerWave;
  dim3 grid(a.groups, (a.max_context / kPage + P - 1) / P);
  hipLaunchKernelGGL(indexer_nvfp4_kernel<P>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

const void* indexer_nvfp4_kernel_symbol() {
  return reinterpret_cast<const void*>(&indexer_nvfp4_kernel<kNvfp4PagesPerWave>);
}

hipError_t launch_indexer(const IdxArgs& a, hipStream_t stream) {
  dim3 grid(a.groups, a.max_context / kPage);
  hipLaunchKernelGGL(indexer_kernel, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

const void* indexer_kernel_symbol() { return reinterpret_cast<const void*>(&indexer_kernel); }

}  // namespace pmqa
