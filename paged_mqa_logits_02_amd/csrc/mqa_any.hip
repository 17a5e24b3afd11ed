// FP8 paged MQA logits for any head count and head_dim.
//
// The same result and output contract as the 64-head, head_dim-128 kernels:
//   logits[b*N+t, p] = s_p * sum_h w[b*N+t, h] * relu(q[b,t,h,:] . k_p)
// (FlashInfer "flashinfer.attn_scores": the introductory equation, the s_p
// bullet, and the paragraph on how the two variants differ, where the FP8 form
// takes parametric shapes and the FP4 form exactly 64 heads of 128.)
//
// Products: the e4m3 operands are widened exactly to f16 in registers and
// multiplied with the f16 16x16x32 MFMA, which sums at fp32 precision (the
// FP8 forms truncate each run of 8 products below 2^-13 of the run's largest,
// so a cancelling dot product can lose its whole value; see device.hpp).
//
// The query slice of a request is kept in LDS rather than in registers, so
// the head count H and head_dim D are runtime values:
//  * D (a multiple of 16, at most 256) is cut into KS planes of 128 key bytes.
//    A page is staged plane by plane in the swizzled 128-byte-row layout of
//    the FP8 ring; the query slice uses the same layout with heads as rows.
//    Bytes past D in the last plane are zeroed in the key fragment, so the
//    products over the padding are exact zeros.
//  * The heads are padded to Hp, a multiple of 32.  Padded query rows repeat
//    row H-1 (finite values) and their weights are zero, so they add nothing.
//  * Wave w scores tokens 16w .. 16w+15 of every page for every query slot
//    of the launch: it loads those key rows itself, so the page loop needs no
//    workgroup barrier.  The query slice is shared by the waves and is
//    reloaded, between two barriers, when a range moves to its next request.
// A launch scores `slots` query slots of every request (starting at slot0);
// the host splits next_n into as many launches as the LDS budget for the
// slice requires.
#include "ring.hpp"

namespace pmqa {

constexpr int kPlaneBytes = kPage * 128;  // a 128-byte plane of a page's 64 key rows
constexpr int kAnyStages = kStages;  // page ring slots of this kernel

__host__ __device__ constexpr int heads_padded(int h) { return (h + 31) / 32 * 32; }

// Page layout of KS planes: plane ks holds bytes [128ks, 128ks+128) of every
// key row (rows 128 B apart, 16-byte chunks swizzled as in the FP8 ring),
// then the 64 fp32 scales.
template <int KS> struct PlaneLayout {
  static constexpr int kKeyBytes = KS * kPlaneBytes;
  static constexpr int kStageBytes = kKeyBytes + kPage * 4;
  static constexpr int kLoadsPerWave = 2 * KS + 1;
  // Wave w loads rows 16w .. 16w+15 of each plane (two 1 KB blocks of 8
  // rows) and the scales of those tokens.  A chunk past D is replaced by the
  // row's first chunk: it stays inside the page and is zeroed before use.
  struct Lanes {
    uint32_t key[KS][2];
    uint32_t scale;
  };
  __device__ static Lanes lanes(int wave, int lane, int D) {
    Lanes o;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * (2 * wave + i) + (lane >> 3);
        const int c = 8 * ks + ((lane & 7) ^ PageLayout<0>::swz(r));
        o.key[ks][i] = r * D + (16 * c < D ? 16 * c : 0);
      }
    o.scale = kPage * D + 64 * wave + 4 * (lane & 15);
    return o;
  }
  __device__ static void issue(uint8_t* stage, const uint8_t* page, Lanes& o, int wave,
                               int lane) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16_page(page, o.key[ks][i], stage + ks * kPlaneBytes + 8 * (2 * wave + i) * 128);
    if (lane < 16) dma4_page(page, o.scale, stage + kKeyBytes + 64 * wave);
  }
};

__device__ __forceinline__ float ldg_untracked_f32(const void* p) {
  float v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Loads request b's query slice (slots slot0 .. slot0+slots-1, all heads) into
// q_lds [slots][KS][Hp][128] and its weights into w_lds [slots][Hp], and waits
// for every load of this wave (pages in flight included).  The caller places
// a barrier before (no wave still reads the previous slice) and after (every
// wave's part has landed).
template <int KS>
__device__ void load_slice(const MqaArgs& a, int b, uint8_t* q_lds, float* w_lds, int Hp,
                           int wave, int lane) {
  const int H = a.heads, D = a.head_dim;
  const int row_blocks = Hp / 8;  // 1 KB blocks of 8 rows per plane
  const int blocks = a.slots * KS * row_blocks;
  for (int x = wave; x < blocks; x += kBlockThreads / kWave) {
    const int t = x / (KS * row_blocks);
    const int rem = x - t * KS * row_blocks;
    const int ks = rem / row_blocks;
    const int hb = rem - ks * row_blocks;
    const int h = 8 * hb + (lane >> 3);
    const int c = 8 * ks + ((lane & 7) ^ PageLayout<0>::swz(h));
    const int hs = h < H ? h : H - 1;
    const uint8_t* src = a.q + (row_of(a, b, t) * H + hs) * D + (16 * c < D ? 16 * c : 0);
    dma16(src, q_lds + ((t * KS + ks) * Hp + 8 * hb) * 128);
  }
  // one weight per thread (slots * Hp <= 256); every lane loads from a valid
  // address and the padding is zeroed after the wait
  const int e = threadIdx.x;
  const int t = e / Hp, h = e - t * Hp;
  const bool in_slice = e < a.slots * Hp;
  const bool real = in_slice && h < H;
  const float raw = ldg_untracked_f32(real ? a.w + row_of(a, b, t) * H + h : a.w);
  wait_vmcnt<0>();
  float wv = raw;
  settle(wv);
  if (in_slice) w_lds[e] = real ? wv : 0.0f;
}

// Scores tokens 16*wave .. 16*wave+15 of NP consecutive staged pages of one
// request (NP = 1 or 2) for every slot of the launch and stores them.  A
// plane's 32 bytes per lane (Frag<0>) feed four f16 products of 8 values
// each, in the same order for query and key.  With two pages each query
// fragment is read from LDS and widened to f16 once for both pages.
template <int KS, int OUTT, int NP>
__device__ __forceinline__ void score_pages_any(const uint8_t* const (&stage)[NP],
                                                const uint8_t* q_lds, const float* w_lds,
                                                const MqaArgs& a, int b, int j0,
                                                const bool (&valid)[NP], int Hp, int wave,
                                                int lane, bool partial, bool lo_ok, bool hi_ok,
                                                bool hi_any) {
  const int g = lane >> 4, rr = lane & 15;
  const int r = 16 * wave + rr;  // key row = token of the page
  v8h kh[NP][KS][4];
  float sp[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    Frag<0> kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks].load_stage(stage[p] + ks * kPlaneBytes, r, g);
    if (partial) {
      // the lane's two chunks of the last plane: d in [16c, 16c+16) for
      // c = 8(KS-1)+g (elements 0-3) and c = 8(KS-1)+4+g (elements 4-7)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kf[KS - 1].v[i] = lo_ok ? kf[KS - 1].v[i] : 0;
        kf[KS - 1].v[4 + i] = hi_ok ? kf[KS - 1].v[4 + i] : 0;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kh[p][ks][u] = e4m3x8_to_f16(kf[ks].v[2 * u], kf[ks].v[2 * u + 1]);
    sp[p] = *reinterpret_cast<const float*>(stage[p] + PlaneLayout<KS>::kKeyBytes + 4 * r);
  }
  const int slice = KS * Hp * 128;
  for (int t = 0; t < a.slots; ++t) {
    const uint8_t* qt = q_lds + t * slice;
    const float* wt = w_lds + t * Hp;
    float s_even[NP], s_odd[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) s_even[p] = s_odd[p] = 0.0f;
    // two 16-head tiles per step (Hp is a multiple of 32)
    for (int h0 = 0; h0 < Hp; h0 += 32) {
      v4f acc0[NP], acc1[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) acc0[p] = acc1[p] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<0> q0, q1;
        q0.load_stage(qt + ks * Hp * 128, h0 + rr, g);
        q1.load_stage(qt + ks * Hp * 128, h0 + 16 + rr, g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // the second half of the last plane is all zero when D ends in its first half
          if (u >= 2 && ks == KS - 1 && !hi_any) continue;
          const v8h qa0 = e4m3x8_to_f16(q0.v[2 * u], q0.v[2 * u + 1]);
          const v8h qa1 = e4m3x8_to_f16(q1.v[2 * u], q1.v[2 * u + 1]);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            acc0[p] = mfma_f16(qa0, kh[p][ks][u], acc0[p]);
            acc1[p] = mfma_f16(qa1, kh[p][ks][u], acc1[p]);
          }
        }
      }
      // lane l holds heads h0 + 4g + i (tile 0) and h0 + 16 + 4g + i (tile 1)
      const v4f w0 = *reinterpret_cast<const v4f*>(wt + h0 + 4 * g);
      const v4f w1 = *reinterpret_cast<const v4f*>(wt + h0 + 16 + 4 * g);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        s_even[p] = __builtin_fmaf(w0[0], relu(acc0[p][0]), s_even[p]);
        s_odd[p] = __builtin_fmaf(w0[1], relu(acc0[p][1]), s_odd[p]);
        s_even[p] = __builtin_fmaf(w0[2], relu(acc0[p][2]), s_even[p]);
        s_odd[p] = __builtin_fmaf(w0[3], relu(acc0[p][3]), s_odd[p]);
        s_even[p] = __builtin_fmaf(w1[0], relu(acc1[p][0]), s_even[p]);
        s_odd[p] = __builtin_fmaf(w1[1], relu(acc1[p][1]), s_odd[p]);
        s_even[p] = __builtin_fmaf(w1[2], relu(acc1[p][2]), s_even[p]);
        s_odd[p] = __builtin_fmaf(w1[3], relu(acc1[p][3]), s_odd[p]);
      }
    }
    float v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) v[p] = row_reduce4(s_even[p] + s_odd[p]) * sp[p];
    if (g == 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        store_logit<OUTT>(a.out, row_of(a, b, t) * a.out_row_stride + (long long)(j0 + p) * kPage + r,
                          v[p], valid[p]);
    }
  }
}

// Scores flat items f0 .. f0+count-1, the whole workgroup together.  Page
// pipeline as in the 64-head kernels when each wave scores only the rows it
// loaded: no barrier per page.
template <int KS, int OUTT>
__device__ void process_range_any(const MqaArgs& a, const int* s_prefix, int* s_pid,
                                  uint8_t* ring, uint8_t* q_lds, float* w_lds, long long f0,
                                  int count) {
  using L = PlaneLayout<KS>;
  // Pages are scored in pairs, so a pair's two ring slots are in use while
  // the next two pages load: kAnyStages - 2 pages ahead.
  constexpr int kAhead = kAnyStages - 2;
  static_assert(kAhead >= 1, "ring too short");
  const int B = a.batch;
  const int lane = threadIdx.x & (kWave - 1), wave = uniform(threadIdx.x / kWave);
  const int Hp = heads_padded(a.heads);
  typename L::Lanes dma_lanes = L::lanes(wave, lane, a.head_dim);
  const int g = lane >> 4;
  const bool partial = a.head_dim < 128 * KS;
  const bool lo_ok = 16 * (8 * (KS - 1) + g) < a.head_dim;
  const bool hi_ok = 16 * (8 * (KS - 1) + 4 + g) < a.head_dim;
  const bool hi_any = a.head_dim > 128 * (KS - 1) + 64;  // some lane's second half is in D

  const long long P = uniform(s_prefix[B]);
  if (f0 < 0 || f0 >= P) return;
  if (count > P - f0) count = (int)(P - f0);
  if (count <= 0) return;
  const long long f_end = f0 + count;
  int b = locate(s_prefix, B, f0);
  int j = (int)(f0 - uniform(s_prefix[b]));

  fill_pid_table(a, s_prefix, s_pid, f0, f_end, b, j);
  ring_barrier();

  int issued = 0;
  uint32_t valid_bits = 0;  // bit (item % 32): page id was in range
  int pid_next = uniform(s_pid[0]);
  auto issue_next = [&]() {
    if (issued < count) {
      const uint32_t ok = page_ok_bit(a, pid_next);  // an out-of-range id loads page 0
      const uint8_t* page = a.kv + (unsigned long long)((uint32_t)pid_next & (0u - ok)) *
                                       (unsigned long long)a.page_stride;
      L::issue(ring + ((unsigned)issued % kAnyStages) * L::kStageBytes, page, dma_lanes, wave, lane);
      valid_bits = (valid_bits & ~(1u << (issued & 31))) | (ok << (issued & 31));
      ++issued;
      if (issued < count) {
        if ((unsigned)issued % kPidTable == 0) {
          const long long f = f0 + issued;
          const int rb = locate(s_prefix, B, f);
          ring_barrier();
          fill_pid_table(a, s_prefix, s_pid, f, f_end, rb, (int)(f - uniform(s_prefix[rb])));
          ring_barrier();
        }
        pid_next = uniform(s_pid[(unsigned)issued % kPidTable]);
      }
    }
  };
#pragma unroll
  for (int k = 0; k < kAhead; ++k) issue_next();

  int n = 0;
  while (n < count && b < B) {
    ring_barrier();  // no wave still reads the previous request's slice
    load_slice<KS>(a, b, q_lds, w_lds, Hp, wave, lane);
    ring_barrier();  // the whole slice has landed
    const int pages = min(count - n, tiles_at(s_prefix, b) - j);
    // Pairs of pages, then a last single page.  Before a pair (n, n+1) the
    // pages up to n + kAhead - 1 are issued; the pair issues two more, into
    // the slots of pages n - 2 and n - 1, which this wave has scored (it
    // reads only the rows it loaded, so program order is enough).
    int k = 0;
    for (; k + 1 < pages; k += 2, n += 2, j += 2) {
      issue_next();
      issue_next();
      wait_page<L::kLoadsPerWave, kAhead>(issued - (n + 1) - 1);  // pages n and n+1
      const uint8_t* const st[2] = {ring + ((unsigned)n % kAnyStages) * L::kStageBytes,
                                    ring + ((unsigned)(n + 1) % kAnyStages) * L::kStageBytes};
      const bool valid[2] = {((valid_bits >> (n & 31)) & 1u) != 0,
                             ((valid_bits >> ((n + 1) & 31)) & 1u) != 0};
      score_pages_any<KS, OUTT, 2>(st, q_lds, w_lds, a, b, j, valid, Hp, wave, lane, partial,
                                   lo_ok, hi_ok, hi_any);
    }
    if (k < pages) {
      issue_next();
      wait_page<L::kLoadsPerWave, kAhead>(issued - n - 1);
      const uint8_t* const st[1] = {ring + ((unsigned)n % kAnyStages) * L::kStageBytes};
      const bool valid[1] = {((valid_bits >> (n & 31)) & 1u) != 0};
      score_pages_any<KS, OUTT, 1>(st, q_lds, w_lds, a, b, j, valid, Hp, wave, lane, partial,
                                   lo_ok, hi_ok, hi_any);
      ++n;
      ++j;
    }
    ++b;
    j = 0;
    while (b < B && tiles_at(s_prefix, b) == 0) ++b;
  }
  wait_vmcnt<0>();
}

template <int KS, int OUTT>
__global__ void __launch_bounds__(256)
    mqa_logits_any_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ kv,
                          const float* __restrict__ w, const int32_t* __restrict__ seq_lens,
                          const int32_t* __restrict__ bt, const int32_t* __restrict__ schedule,
                          void* __restrict__ out, const MqaArgs dims) {
  MqaArgs a = dims;
  a.q = q;
  a.q_sf = nullptr;
  a.kv = kv;
  a.w = w;
  a.seq_lens = seq_lens;
  a.bt = bt;
  a.schedule = schedule;
  a.out = out;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_wsum[16];
  __shared__ int s_pid[kPidTable];
  const int Hp = heads_padded(a.heads);
  uint8_t* ring = smem;
  uint8_t* q_lds = smem + kAnyStages * PlaneLayout<KS>::kStageBytes;
  float* w_lds = reinterpret_cast<float*>(q_lds + a.slots * KS * Hp * 128);
  int* s_prefix = reinterpret_cast<int*>(w_lds + a.slots * Hp);
  build_prefix(a.seq_lens, a.batch, a.max_context / kPage, s_prefix, s_wsum);

  const int G = gridDim.x;
  const int unit = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  // The schedule header is read at once (no short-circuit between its fields).
  const int32_t* sc = a.schedule;
  bool use_sched = false;
  if (sc != nullptr) {
    const int h0 = sc[0], h1 = sc[1], h2 = sc[2], h3 = sc[3], h4 = sc[4], h5 = sc[5], h6 = sc[6];
    use_sched = (h0 == kSchedMagic) & (h2 == a.next_n) & (h3 == 0) & (h4 == a.max_context) &
                (h5 == a.batch) & (h6 == s_prefix[a.batch]) & (h1 > 0);
  }
  if (use_sched) {
    const int U = sc[1];
    for (int u = unit; u < U; u += G) {
      const int32_t* e = sc + kSchedHeader + 3 * u;
      const long long f0 = e[2], f1 = e[5];
      if (f1 > f0)
        process_range_any<KS, OUTT>(a, s_prefix, s_pid, ring, q_lds, w_lds, f0, (int)(f1 - f0));
      ring_barrier();
    }
  } else {
    const long long P = uniform(s_prefix[a.batch]);
    const long long f0 = split_point(unit, G, a.cus, a.split_skew, P);
    const long long f1 = split_point(unit + 1, G, a.cus, a.split_skew, P);
    if (f1 > f0)
      process_range_any<KS, OUTT>(a, s_prefix, s_pid, ring, q_lds, w_lds, f0, (int)(f1 - f0));
  }
}

template <int KS, int OUTT>
static const void* any_ptr() {
  return reinterpret_cast<const void*>(&mqa_logits_any_kernel<KS, OUTT>);
}

const void* mqa_any_kernel_symbol(int ks, int out_dtype) {
  if (ks == 1) return out_dtype == 0 ? any_ptr<1, 0>() : any_ptr<1, 1>();
  if (ks == 2) return out_dtype == 0 ? any_ptr<2, 0>() : any_ptr<2, 1>();
  return nullptr;
}

size_t mqa_any_lds_bytes(int ks, int hp, int slots) {
  const size_t stage = (size_t)ks * kPlaneBytes + kPage * 4;
  return kAnyStages * stage + (size_t)slots * ks * hp * 128 + (size_t)slots * hp * 4;
}

hipError_t launch_mqa_any(const MqaArgs& a, int ks, int out_dtype, int grid, size_t lds_bytes,
                          hipStream_t stream) {
  const void* fn = mqa_any_kernel_symbol(ks, out_dtype);
  if (!fn) return hipErrorInvalidValue;
  const uint8_t* q = a.q;
  const uint8_t* kv = a.kv;
  const float* w = a.w;
  const int32_t* seq_lens = a.seq_lens;
  const int32_t* bt = a.bt;
  const int32_t* sched = a.schedule;
  void* out = a.out;
  void* args[] = {&q, &kv, &w, &seq_lens, &bt, &sched, &out, const_cast<MqaArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kBlockThreads), args, lds_bytes, stream);
}

}  // namespace pmqa
