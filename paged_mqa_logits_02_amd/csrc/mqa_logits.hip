// Paged MQA logits on gfx950.
//
// Computes, per request b, query slot t and KV position p,
//   logits[b*N+t, p] = s_p * sum_h w[b*N+t, h] * relu(q[b,t,h,:] . k_p)
// (FlashInfer "flashinfer.attn_scores": introductory equation and the two
// bullets after it; MXFP4 has no s_p and folds its block scales into q and k).
//
// Work decomposition.  The work items of a call are (request, 64-token page)
// pairs in request-major order.  A wavefront is one "unit": it owns a
// contiguous range of items, keeps the request's query (all 64 heads x N
// slots) and head weights in registers, and streams the key pages of its range
// straight from HBM into MFMA operand registers (a key token is used by one
// wave only, so it never needs to be shared through LDS).  Ranges come either
// from a schedule buffer or from an in-kernel split computed from seq_lens in
// the prologue ("flashinfer.attn_scores", Scheduling and Setup: a per-call work
// assignment computed on the GPU, so the call needs no host round-trip).
//
// Per page and wave: 4 token sub-tiles x 4 head tiles x N slots of
// 16x16x128 MFMA; each lane then holds 4 heads x 1 token per tile.  The
// rectifier and the weighted head sum run on those registers, one cross-row
// transposing reduction leaves lane l with the logit of token l, which is
// scaled by s_p and stored: 64 consecutive columns per row and page.
#include "device.hpp"
#include "pmqa_internal.h"

namespace pmqa {

// --------------------------------------------------------------- schedule

__device__ __forceinline__ int tiles_of(int L, int max_tiles) {
  if (L <= 0) return 0;
  int t = (L + kPage - 1) / kPage;
  return t < max_tiles ? t : max_tiles;
}

// Exclusive prefix of per-request page counts into s_prefix[0..B]
// (s_prefix[B] = total).  Whole workgroup; ends with a barrier.
__device__ void build_prefix(const int32_t* __restrict__ seq_lens, int B, int max_tiles,
                             int* s_prefix, int* s_wsum) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwave = nthr / kWave;
  const int per = (B + nthr - 1) / nthr;
  const int lo = tid * per;
  const int hi = min(lo + per, B);
  int sum = 0;
  for (int i = lo; i < hi; ++i) {
    int t = tiles_of(seq_lens[i], max_tiles);
    s_prefix[i] = t;
    sum += t;
  }
  int incl = wave_inclusive_scan(sum, lane);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < nwave; ++w) {
    int v = s_wsum[w];
    base += (w < wave) ? v : 0;
    total += v;
  }
  int run = base + incl - sum;
  for (int i = lo; i < hi; ++i) {
    int t = s_prefix[i];
    s_prefix[i] = run;
    run += t;
  }
  if (tid == 0) s_prefix[B] = total;
  __syncthreads();
}

// Largest b in [0, B] with prefix[b] <= f.  For 0 <= f < prefix[B] the item f
// lies in request b at page f - prefix[b].
__device__ __forceinline__ int locate(const int* s_prefix, int B, long long f) {
  int lo = 0, hi = B;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256) schedule_kernel(const int32_t* __restrict__ seq_lens,
                                                       int B, int next_n, int variant,
                                                       int max_context, int U,
                                                       int32_t* __restrict__ sched) {
  extern __shared__ int s_prefix[];
  __shared__ int s_wsum[16];
  build_prefix(seq_lens, B, max_context / kPage, s_prefix, s_wsum);
  const long long P = s_prefix[B];
  if (threadIdx.x == 0) {
    sched[0] = kSchedMagic;
    sched[1] = U;
    sched[2] = next_n;
    sched[3] = variant;
    sched[4] = max_context;
    sched[5] = B;
    sched[6] = (int)P;
    sched[7] = 0;
  }
  for (int u = threadIdx.x; u <= U; u += blockDim.x) {
    long long f = (long long)u * P / U;
    int b = (u == U) ? B : locate(s_prefix, B, f);
    int j = (u == U) ? 0 : (int)(f - s_prefix[b]);
    int32_t* e = sched + kSchedHeader + 3 * u;
    e[0] = b;
    e[1] = j;
    e[2] = (int)f;
  }
}

// ------------------------------------------------------------ operands

// Per variant: the MFMA operand fragments of one 16-row tile and how they are
// loaded.  The K dimension (head_dim) is split over lanes identically for the
// query (A) and key (B) operand, so every product pairs matching d.
template <int VAR> struct Frag;

// FP8: lane l holds d in [16g, 16g+16) and [64+16g, 64+16g+16), g = l>>4.
template <> struct Frag<0> {
  v8i v;
  static constexpr int kRowBytes = 128;  // head_dim e4m3
  static constexpr int kKeyBytes = kPage * kRowBytes;
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    v4i lo = ldg<v4i>(row + 16 * g);
    v4i hi = ldg<v4i>(row + 64 + 16 * g);
    v = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ __forceinline__ void load_stream(const uint8_t* row, int g) {
    v4i lo = ldg_stream<v4i>(row + 16 * g);
    v4i hi = ldg_stream<v4i>(row + 64 + 16 * g);
    v = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ __forceinline__ void zero() { v = (v8i){0, 0, 0, 0, 0, 0, 0, 0}; }
};

// MXFP4: lane l holds the 32-element block g = l>>4 (16 packed bytes) and that
// block's e8m0 code.
template <> struct Frag<1> {
  v4i v;
  int sf;
  static constexpr int kRowBytes = 64;  // 128 e2m1 values
  static constexpr int kKeyBytes = kPage * kRowBytes;
  __device__ __forceinline__ void load(const uint8_t* row, int g) { v = ldg<v4i>(row + 16 * g); }
  __device__ __forceinline__ void load_stream(const uint8_t* row, int g) {
    v = ldg_stream<v4i>(row + 16 * g);
  }
  __device__ __forceinline__ void zero() {
    v = (v4i){0, 0, 0, 0};
    sf = kE8M0One;
  }
};

__device__ __forceinline__ v4f mma(const Frag<0>& q, const Frag<0>& k) {
  return mfma_fp8(q.v, k.v, (v4f){0.f, 0.f, 0.f, 0.f});
}
__device__ __forceinline__ v4f mma(const Frag<1>& q, const Frag<1>& k) {
  return mfma_fp4(q.v, q.sf, k.v, k.sf, (v4f){0.f, 0.f, 0.f, 0.f});
}

// One page of keys for one wave: 4 sub-tiles of 16 tokens, plus the per-lane
// FP8 scale of token l (MXFP4: 1).
template <int VAR> struct PageFrag {
  Frag<VAR> k[4];
  float sp;
};

template <int VAR>
__device__ __forceinline__ void load_page(PageFrag<VAR>& pf, const uint8_t* page, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint8_t* row = page + (16 * s + r) * Frag<VAR>::kRowBytes;
    pf.k[s].load_stream(row, g);
  }
  if constexpr (VAR == 0) {
    pf.sp = ldg_stream<float>(page + Frag<0>::kKeyBytes + 4 * lane);
  } else {
    const uint8_t* sfp = page + Frag<1>::kKeyBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) pf.k[s].sf = sfp[(16 * s + r) * 4 + g];
    pf.sp = 1.0f;
  }
}

template <int VAR>
__device__ __forceinline__ void zero_page(PageFrag<VAR>& pf) {
#pragma unroll
  for (int s = 0; s < 4; ++s) pf.k[s].zero();
  pf.sp = __builtin_nanf("");
}

// Query of request b (all heads, N slots) and its head weights.
template <int N, int VAR> struct QueryFrag {
  Frag<VAR> q[4][N];   // [head tile][slot]
  v4f w[4][N];         // w[mt][t][i] = weight of head 16mt + 4(l>>4) + i
};

template <int N, int VAR>
__device__ __forceinline__ void load_query(QueryFrag<N, VAR>& qf, const MqaArgs& a, int b,
                                           int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int t = 0; t < N; ++t) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const long long head_row = ((long long)(b * N + t) * 64 + 16 * mt + r);
      qf.q[mt][t].load(a.q + head_row * Frag<VAR>::kRowBytes, g);
      if constexpr (VAR == 1) qf.q[mt][t].sf = a.q_sf[head_row * 4 + g];
      qf.w[mt][t] = ldg<v4f>(a.w + (long long)(b * N + t) * 64 + 16 * mt + 4 * g);
    }
  }
}

// ------------------------------------------------------------- main kernel

template <int OUTT>
__device__ __forceinline__ void store_logit(void* out, long long idx, float v) {
  if constexpr (OUTT == 0) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
  }
}

// Scores one page for every slot and stores row b*N+t, columns 64j .. 64j+63.
template <int N, int VAR, int OUTT>
__device__ __forceinline__ void score_page(const QueryFrag<N, VAR>& qf, const PageFrag<VAR>& pf,
                                           const MqaArgs& a, int b, int j, int lane) {
  float part[N][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int t = 0; t < N; ++t) {
      float sum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        v4f acc = mma(qf.q[mt][t], pf.k[s]);
        const v4f w = qf.w[mt][t];
        sum = __builtin_fmaf(w[0], relu(acc[0]), sum);
        sum = __builtin_fmaf(w[1], relu(acc[1]), sum);
        sum = __builtin_fmaf(w[2], relu(acc[2]), sum);
        sum = __builtin_fmaf(w[3], relu(acc[3]), sum);
      }
      part[t][s] = sum;
    }
  }
#pragma unroll
  for (int t = 0; t < N; ++t) {
    float v = row_transpose_reduce4(part[t][0], part[t][1], part[t][2], part[t][3]);
    if constexpr (VAR == 0) v *= pf.sp;
    const long long idx = (long long)(b * N + t) * a.out_row_stride + (long long)j * kPage + lane;
    store_logit<OUTT>(a.out, idx, v);
  }
}

__device__ __forceinline__ int tiles_at(const int* s_prefix, int b) {
  return s_prefix[b + 1] - s_prefix[b];
}

__device__ __forceinline__ void advance(const int* s_prefix, int B, int& b, int& j) {
  ++j;
  while (b < B && j >= tiles_at(s_prefix, b)) {
    ++b;
    j = 0;
  }
}

__device__ __forceinline__ int page_id(const MqaArgs& a, int b, int j) {
  return a.bt[(long long)b * a.bt_stride + j];
}

__device__ __forceinline__ bool page_ok(const MqaArgs& a, int pg) {
  return (unsigned)pg < (unsigned)a.num_pages;
}

// Processes `count` items starting at (b, j).
template <int N, int VAR, int OUTT>
__device__ void process_range(const MqaArgs& a, const int* s_prefix, int b, int j, int count,
                              int lane) {
  const int B = a.batch;
  while (b < B && j >= tiles_at(s_prefix, b)) { ++b; j = 0; }
  if (count <= 0 || b >= B) return;

  QueryFrag<N, VAR> qf;
  load_query<N, VAR>(qf, a, b, lane);

  PageFrag<VAR> cur, nxt;
  int pg = page_id(a, b, j);
  if (page_ok(a, pg)) load_page<VAR>(cur, a.kv + (long long)pg * a.page_stride, lane);
  else zero_page<VAR>(cur);

  int b1 = b, j1 = j;
  advance(s_prefix, B, b1, j1);
  int pg1 = (count > 1 && b1 < B) ? page_id(a, b1, j1) : -1;

  for (int n = 0; n < count; ++n) {
    const bool more = (n + 1 < count) && (b1 < B);
    if (more) {
      if (page_ok(a, pg1)) load_page<VAR>(nxt, a.kv + (long long)pg1 * a.page_stride, lane);
      else zero_page<VAR>(nxt);
    }
    int b2 = b1, j2 = j1;
    if (more) advance(s_prefix, B, b2, j2);
    const int pg2 = (more && n + 2 < count && b2 < B) ? page_id(a, b2, j2) : -1;

    score_page<N, VAR, OUTT>(qf, cur, a, b, j, lane);
    if (!more) break;
    if (b1 != b) load_query<N, VAR>(qf, a, b1, lane);
    cur = nxt;
    b = b1; j = j1;
    b1 = b2; j1 = j2; pg1 = pg2;
  }
}

template <int N, int VAR, int OUTT>
__global__ void __launch_bounds__(256) mqa_logits_kernel(const MqaArgs a) {
  extern __shared__ int s_prefix[];
  __shared__ int s_wsum[16];
  build_prefix(a.seq_lens, a.batch, a.max_context / kPage, s_prefix, s_wsum);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves_per_block = blockDim.x / kWave;
  // Consecutive units on one XCD: workgroups are dealt to the 8 XCDs
  // round-robin, so renumber them XCD-major before splitting the work.
  const int G = gridDim.x;
  const int blk = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int my_unit = blk * waves_per_block + wave;
  const int total_waves = G * waves_per_block;

  const int32_t* sc = a.schedule;
  const bool use_sched = sc != nullptr && sc[0] == kSchedMagic && sc[2] == N &&
                         sc[3] == VAR && sc[4] == a.max_context && sc[5] == a.batch &&
                         sc[1] > 0;
  if (use_sched) {
    const int U = sc[1];
    for (int u = my_unit; u < U; u += total_waves) {
      const int32_t* e = sc + kSchedHeader + 3 * u;
      const int b = e[0], j = e[1];
      const int count = e[5] - e[2];
      if (b >= 0 && j >= 0) process_range<N, VAR, OUTT>(a, s_prefix, b, j, count, lane);
    }
  } else {
    const long long P = s_prefix[a.batch];
    const long long f0 = (long long)my_unit * P / total_waves;
    const long long f1 = (long long)(my_unit + 1) * P / total_waves;
    if (f1 > f0) {
      const int b = locate(s_prefix, a.batch, f0);
      process_range<N, VAR, OUTT>(a, s_prefix, b, (int)(f0 - s_prefix[b]), (int)(f1 - f0), lane);
    }
  }
}

// ------------------------------------------------------------- launchers

template <int N, int VAR, int OUTT>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&mqa_logits_kernel<N, VAR, OUTT>);
}

const void* mqa_kernel_symbol(int next_n, int variant, int out_dtype) {
#define PMQA_K(n)                                                                  \
  if (next_n == n) {                                                               \
    if (variant == 0) return out_dtype == 0 ? kernel_ptr<n, 0, 0>() : kernel_ptr<n, 0, 1>(); \
    return out_dtype == 0 ? kernel_ptr<n, 1, 0>() : kernel_ptr<n, 1, 1>();        \
  }
  PMQA_K(1)
  PMQA_K(2)
  PMQA_K(3)
  PMQA_K(4)
#undef PMQA_K
  return nullptr;
}

hipError_t launch_mqa(const MqaArgs& a, int next_n, int variant, int out_dtype, int grid,
                      size_t lds_bytes, hipStream_t stream) {
  const void* fn = mqa_kernel_symbol(next_n, variant, out_dtype);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<MqaArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kBlockThreads), args, lds_bytes, stream);
}

hipError_t launch_schedule(const int32_t* seq_lens, int B, int next_n, int variant,
                           int max_context, int U, int32_t* sched, hipStream_t stream) {
  const size_t lds = (size_t)(B + 1) * sizeof(int);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kBlockThreads), lds, stream, seq_lens, B,
                     next_n, variant, max_context, U, sched);
  return hipGetLastError();
}

const void* schedule_kernel_symbol() { return reinterpret_cast<const void*>(&schedule_kernel); }

}  // namespace pmqa
