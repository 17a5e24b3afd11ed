// Paged MQA logits on gfx950: the kernels for 64 heads and head_dim 128.
//
// Computes, per request b, query slot t and KV position p,
//   logits[b*N+t, p] = s_p * sum_h w[b*N+t, h] * relu(q[b,t,h,:] . k_p)
// (FlashInfer "flashinfer.attn_scores": introductory equation and the two
// bullets after it; MXFP4 has no s_p and folds its block scales into q and k).
// A launch scores `slots` (1..4) consecutive query slots, from slot0, of every
// request's next_n; larger next_n runs as several launches.
//
// Work decomposition.  The work items of a call are (request, 64-token page)
// pairs in request-major order.  A workgroup (4 wavefronts) is one "unit": it
// owns a contiguous range of items, taken either from a schedule buffer or
// from an in-kernel split computed from seq_lens in the prologue
// ("flashinfer.attn_scores", Scheduling and Setup: a per-call work assignment
// computed on the GPU, so the call needs no host round-trip).
//
// Data path per page.  The workgroup streams its pages through a ring of
// kStages LDS slots with gfx950 direct-to-LDS loads (global_load_lds), so the
// bytes in flight do not cost registers: kStages-1 pages are in flight while
// one is scored.  The global side of each load is permuted so that the LDS
// image is XOR-swizzled by row and the MFMA operand reads are free of bank
// conflicts.  Each wave scores a share of the page (a subset of query slots
// and 16-token sub-tiles) with its slice of the query and head weights held in
// registers: matrix products (heads x tokens), rectifier and weighted head
// sum in registers, a cross-row reduction with permlane swaps, s_p, and a
// coalesced store of exactly the page's 64 columns.
//
// Products.  FP8 operands are widened exactly to f16 (the query once per
// request, each key fragment once per page) and multiplied with the f16
// matrix instructions, whose sums keep fp32 precision; gfx950's FP8 matrix
// instructions truncate each run of 8 products to 2^-13 of its largest, which
// can lose the whole value of a cancelling dot product.  MXFP4 operands are
// multiplied as they are with the scaled f8f6f4 instruction: an e2m1 product
// always fits that window, so those sums are exact.
#include <type_traits>
#include <utility>

#include "ring.hpp"

namespace pmqa {

__global__ void __launch_bounds__(256) schedule_kernel(const int32_t* __restrict__ seq_lens,
                                                       int B, int next_n, int variant,
                                                       int max_context, int U, int cus,
                                                       int skew, int32_t* __restrict__ sched) {
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
    long long f = split_point(u, U, cus, skew, P);
    int b = (u == U) ? B : locate_lane(s_prefix, B, f);
    int j = (u == U) ? 0 : (int)(f - s_prefix[b]);
    int32_t* e = sched + kSchedHeader + 3 * u;
    e[0] = b;
    e[1] = j;
    e[2] = (int)f;
  }
}

// ---------------------------------------------------- MXFP4 page and operands
//
// Kernel variants: 0 is FP8; 1..4 are MXFP4 with a scale layout ("flashinfer.
// attn_scores", paragraph on how the variants differ: q_sf, sf_vec_size and
// is_kv_sf_interleaved): 1 = one e8m0 code per 32 values, codes after all
// packed rows; 2 = one code per 16 values, codes after all packed rows; 3 and
// 4 = the same with each token's codes right after its packed bytes (64
// records per page).
__host__ __device__ constexpr int mx_sfv(int var) { return var == 2 || var == 4 ? 16 : 32; }
__host__ __device__ constexpr bool mx_records(int var) { return var >= 3; }
constexpr int kMxVariants = 4;

// An MXFP4 page in LDS.  Trailing codes: 64 packed rows of 64 bytes (16-byte
// chunks XOR-permuted by row, as for FP8), then the 64 tokens' codes, kCodes
// per token; a wave loads its 16 rows as one 16-byte piece per lane and its
// tokens' codes as dwords.  Token records (68 or 72 bytes, 4-byte aligned):
// the page's bytes as they are, copied in 16-byte pieces; wave w's quarter
// is exactly records 16w .. 16w+15, so every wave still loads the rows it
// scores itself.  row_off / chunk_off / code_off locate a row's 16-byte chunk
// c and its codes in either image.
template <int SFV, bool REC> struct MxPageLayout {
  static constexpr int kRowBytes = 64;
  static constexpr int kKeyBytes = kPage * kRowBytes;  // 4096
  static constexpr int kCodes = 128 / SFV;             // e8m0 codes per token
  static constexpr int kRecBytes = kRowBytes + kCodes;  // a token record
  static constexpr int kStageBytes = REC ? kPage * kRecBytes : kKeyBytes + kPage * kCodes;
  static constexpr int kCodeDwords = 16 * kCodes / 4;   // a wave's tokens' codes
  static constexpr int kTailPieces = kRecBytes - 64;    // records: 16-byte pieces past 64 lanes
  static constexpr int kLoadsPerWave = 2;
  static constexpr int kRowStride = REC ? kRecBytes : kRowBytes;   // between rows
  static constexpr int kCodeStride = REC ? kRecBytes : kCodes;     // between rows' codes
  __device__ static int swz(int r) { return (r >> 1) & 3; }
  __device__ static int row_off(int r) { return r * kRowStride; }
  __device__ static int chunk_off(int r, int c) { return REC ? 16 * c : 16 * (c ^ swz(r)); }
  __device__ static int code_off(int r) {
    return REC ? r * kRecBytes + kRowBytes : kKeyBytes + r * kCodes;
  }
  struct Lanes {
    uint32_t off[kLoadsPerWave];
  };
  // Wave w loads rows 16w .. 16w+15 and those tokens' codes.
  __device__ static Lanes lanes(int wave, int lane) {
    Lanes o;
    if constexpr (!REC) {
      const int r = 16 * wave + (lane >> 2);
      o.off[0] = r * kRowBytes + 16 * ((lane & 3) ^ swz(r));
      o.off[1] = kKeyBytes + 16 * wave * kCodes + 4 * (lane < kCodeDwords ? lane : 0);
    } else {
      const int base = 16 * wave * kRecBytes;
      o.off[0] = base + 16 * lane;
      o.off[1] = base + 16 * (64 + (lane < kTailPieces ? lane : 0));
    }
    return o;
  }
  __device__ static void issue(uint8_t* stage, const uint8_t* page, Lanes& o, int wave,
                               int lane) {
    if constexpr (!REC) {
      dma16_page(page, o.off[0], stage + 16 * wave * kRowBytes);
      if (lane < kCodeDwords) dma4_page(page, o.off[1], stage + kKeyBytes + 16 * wave * kCodes);
    } else {
      dma16_page(page, o.off[0], stage + 16 * wave * kRecBytes);
      if (lane < kTailPieces) dma16_page(page, o.off[1], stage + 16 * wave * kRecBytes + 1024);
    }
  }
};

// 16 bytes from LDS: 16-byte aligned (one 128-bit read), or only 4-byte
// aligned in token records: four dword reads, which the compiler pairs.
// (A 4-byte aligned vector load is split without the memory information the
// compiler needs to tell it from the page loads into LDS still in flight, so
// it would wait for all of them before every page.)
template <bool A4>
__device__ __forceinline__ v4i lds16(const uint8_t* p) {
  if constexpr (A4) {
    typedef __attribute__((address_space(3))) const int* lds_int;
    const lds_int q = (lds_int)p;
    return (v4i){q[0], q[1], q[2], q[3]};
  } else {
    return *reinterpret_cast<const v4i*>(p);
  }
}

template <> struct PageLayout<1> : MxPageLayout<32, false> {};
template <> struct PageLayout<2> : MxPageLayout<16, false> {};
template <> struct PageLayout<3> : MxPageLayout<32, true> {};
template <> struct PageLayout<4> : MxPageLayout<16, true> {};

// MXFP4 operand fragment (16x16x128 tiles): lane l holds the 32-element block
// g = l>>4 of its row (16 packed bytes) and its codes: one (sf) per 32 values,
// or one per 16 (sf for the first half, sf2 for the second).
template <int SFV, bool REC = false> struct MxFrag {
  static constexpr int kCodes = 128 / SFV;
  v4i v;
  int sf, sf2;
  __device__ __forceinline__ void load_global(const uint8_t* row, int g) {
    v = ldg_untracked(row + 16 * g);
  }
  // codes of a query row (q_sf row of kCodes codes), loaded with it
  __device__ __forceinline__ void load_codes_global(const uint8_t* codes, int g) {
    sf = ldg_untracked_u8(codes + (SFV == 32 ? g : 2 * g));
    if constexpr (SFV == 16) sf2 = ldg_untracked_u8(codes + 2 * g + 1);
  }
  __device__ __forceinline__ void load_stage(const uint8_t* stage, int r, int g) {
    using L = MxPageLayout<SFV, REC>;
    v = lds16<REC>(stage + L::row_off(r) + L::chunk_off(r, g));
    const uint8_t* codes = stage + L::code_off(r);
    sf = codes[SFV == 32 ? g : 2 * g];
    if constexpr (SFV == 16) sf2 = codes[2 * g + 1];
  }
  __device__ __forceinline__ void settle_codes() {
    settle(sf);
    if constexpr (SFV == 16) settle(sf2);
  }
};
template <> struct Frag<1> : MxFrag<32, false> {};
template <> struct Frag<2> : MxFrag<16, false> {};
template <> struct Frag<3> : MxFrag<32, true> {};
template <> struct Frag<4> : MxFrag<16, true> {};

// Operands of the MXFP4 products.  A key fragment is multiplied as loaded.  A
// query fragment with one code per 32 values is too; with one code per 16
// values (the matrix unit takes one code per 32 values of a lane) it is split
// once per request into its two halves, each with the other half zeroed and
// its own code: the product is the sum of two scaled products, the whole key
// fragment with the first half's code, then with the second half's (the
// zeroed query half removes the key half that the code does not belong to).
// Both forms are exact: the scaled FP4 products sum without loss.
struct MxSplitQuery {
  v4i lo, hi;
  int sf, sf2;
};
template <class F>
__device__ __forceinline__ MxSplitQuery split_query(const F& f) {
  return MxSplitQuery{(v4i){f.v[0], f.v[1], 0, 0}, (v4i){0, 0, f.v[2], f.v[3]}, f.sf, f.sf2};
}
template <bool R>
__device__ __forceinline__ const MxFrag<32, R>& query_operand(const MxFrag<32, R>& f) {
  return f;
}
template <bool R>
__device__ __forceinline__ MxSplitQuery query_operand(const MxFrag<16, R>& f) {
  return split_query(f);
}
template <int SFV, bool R>
__device__ __forceinline__ const MxFrag<SFV, R>& key_operand(const MxFrag<SFV, R>& k) { return k; }

template <bool R>
__device__ __forceinline__ v4f mma(const MxFrag<32, R>& q, const MxFrag<32, R>& k) {
  return mfma_fp4(q.v, q.sf, k.v, k.sf, (v4f){0.f, 0.f, 0.f, 0.f});
}
template <bool R>
__device__ __forceinline__ v4f mma(const MxSplitQuery& q, const MxFrag<16, R>& k) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return mfma_fp4(q.hi, q.sf2, k.v, k.sf2, mfma_fp4(q.lo, q.sf, k.v, k.sf, z));
}

// How the 4 waves of a workgroup share one page: each wave takes TW query
// slots and SW 16-token sub-tiles (next_n = 3: three waves take a slot each
// and the fourth only loads).  FP8 scores every share with 16x16 tiles of
// f16 products.  kWide (MXFP4, fp32 output): the wave's share is scored with
// 32x32x64 tiles (32 heads x 32 tokens) instead of 16x16x128 ones; half the
// matrix instructions for the same products, and a lane then holds 16 heads
// of one token, so the head reduction is a single cross-half exchange.
template <int N> struct WaveSplit;
template <> struct WaveSplit<1> { static constexpr int TW = 1, SW = 1; static constexpr bool kWide = false; };
template <> struct WaveSplit<2> { static constexpr int TW = 1, SW = 2; static constexpr bool kWide = true; };
template <> struct WaveSplit<3> { static constexpr int TW = 1, SW = 4; static constexpr bool kWide = true; };
template <> struct WaveSplit<4> { static constexpr int TW = 1, SW = 4; static constexpr bool kWide = true; };

// 32x32x64 operand fragment of one K step (64 of the 128 head_dim values):
// lane l holds row (l & 31) and K values [32h, 32h + 32) of the step,
// h = l >> 5, in the same slots for the query and the key operand.
template <int VAR> struct WideFrag;

// MXFP4: lane l holds 32-element block c = 2ks + h of the row (16 packed bytes)
// and its code(s), as MxFrag.
template <int SFV, bool REC = false> struct MxWideFrag {
  static constexpr int kCodes = 128 / SFV;
  v4i v;
  int sf, sf2;
  __device__ __forceinline__ void load_global(const uint8_t* row, int ks, int h) {
    v = ldg_untracked(row + 16 * (2 * ks + h));
  }
  __device__ __forceinline__ void load_codes_global(const uint8_t* codes, int ks, int h) {
    const int c = 2 * ks + h;
    sf = ldg_untracked_u8(codes + (SFV == 32 ? c : 2 * c));
    if constexpr (SFV == 16) sf2 = ldg_untracked_u8(codes + 2 * c + 1);
  }
  __device__ __forceinline__ void load_stage(const uint8_t* stage, int r, int ks, int h) {
    using L = MxPageLayout<SFV, REC>;
    const int c = 2 * ks + h;
    v = lds16<REC>(stage + L::row_off(r) + L::chunk_off(r, c));
    const uint8_t* codes = stage + L::code_off(r);
    sf = codes[SFV == 32 ? c : 2 * c];
    if constexpr (SFV == 16) sf2 = codes[2 * c + 1];
  }
  __device__ __forceinline__ void settle_codes() {
    settle(sf);
    if constexpr (SFV == 16) settle(sf2);
  }
};
template <> struct WideFrag<1> : MxWideFrag<32, false> {};
template <> struct WideFrag<2> : MxWideFrag<16, false> {};
template <> struct WideFrag<3> : MxWideFrag<32, true> {};
template <> struct WideFrag<4> : MxWideFrag<16, true> {};

template <bool R>
__device__ __forceinline__ const MxWideFrag<32, R>& query_operand(const MxWideFrag<32, R>& f) {
  return f;
}
template <bool R>
__device__ __forceinline__ MxSplitQuery query_operand(const MxWideFrag<16, R>& f) {
  return split_query(f);
}
template <bool R>
__device__ __forceinline__ v16f mma_wide(const MxWideFrag<32, R>& q, const MxWideFrag<32, R>& k,
                                         const v16f& c) {
  return mfma32_fp4(q.v, q.sf, k.v, k.sf, c);
}
template <bool R>
__device__ __forceinline__ v16f mma_wide(const MxSplitQuery& q, const MxWideFrag<16, R>& k,
                                         const v16f& c) {
  return mfma32_fp4(q.hi, q.sf2, k.v, k.sf2, mfma32_fp4(q.lo, q.sf, k.v, k.sf, c));
}

// The query operand of one head tile as the products take it: an FP8
// fragment widened to f16 once per request (64 VGPRs for the 64 heads of a
// slot), an MXFP4 fragment as loaded or split (query_operand).
__device__ __forceinline__ Half32 query_operand(const Frag<0>& f) { return widen32(f.v); }
template <class F> using QOperandOf = std::decay_t<decltype(query_operand(std::declval<const F&>()))>;

// The wave's query slots of request b (all 64 heads) and their head weights.
template <int TW, int VAR> struct QueryFrag {
  Frag<VAR> q[4][TW];                               // [head tile][slot], as loaded
  QOperandOf<Frag<VAR>> op[4][TW];  // as multiplied
  v4f w[4][TW];        // w[mt][t][i] = weight of head 16mt + 4(l>>4) + i
};

template <int TW, int VAR>
__device__ __forceinline__ void settle_query(QueryFrag<TW, VAR>& qf) {
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      settle(qf.q[mt][t].v);
      if constexpr (VAR != 0) qf.q[mt][t].settle_codes();
      settle(qf.w[mt][t]);
      qf.op[mt][t] = query_operand(qf.q[mt][t]);
    }
}

template <int N, int TW, int VAR>
__device__ __forceinline__ void load_query(QueryFrag<TW, VAR>& qf, const MqaArgs& a, int b,
                                           int t0, int lane) {
  const int g = lane >> 4, r = lane & 15;
  constexpr int kQRow = VAR == 0 ? 128 : 64;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const long long head_row = (row_of(a, b, t0 + t) * 64 + 16 * mt + r);
      qf.q[mt][t].load_global(a.q + head_row * kQRow, g);
      if constexpr (VAR != 0) qf.q[mt][t].load_codes_global(a.q_sf + head_row * Frag<VAR>::kCodes, g);
      qf.w[mt][t] = __builtin_bit_cast(
          v4f, ldg_untracked(a.w + row_of(a, b, t0 + t) * 64 + 16 * mt + 4 * g));
    }
  }
}

// The wave's one query slot of request b for 32x32 tiles (MXFP4): q[mt][ks]
// covers heads 32mt + (l & 31), K step ks; w[mt][u][i] is the weight of head
// 32mt + 8u + 4(l >> 5) + i, the head of output element 4u + i of tile mt.
template <int VAR> struct WideQuery {
  WideFrag<VAR> q[2][2];                     // as loaded
  QOperandOf<WideFrag<VAR>> op[2][2];        // as multiplied
  v4f w[2][4];
};

template <int VAR>
__device__ __forceinline__ void settle_query(WideQuery<VAR>& qf) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      settle(qf.q[mt][ks].v);
      qf.q[mt][ks].settle_codes();
      qf.op[mt][ks] = query_operand(qf.q[mt][ks]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) settle(qf.w[mt][u]);
  }
}

template <int N, int VAR>
__device__ __forceinline__ void load_query(WideQuery<VAR>& qf, const MqaArgs& a, int b, int t0,
                                           int lane) {
  const int h = lane >> 5, r = lane & 31;
  constexpr int kQRow = 64;
  const long long slot = row_of(a, b, t0);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const long long head_row = slot * 64 + 32 * mt + r;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qf.q[mt][ks].load_global(a.q + head_row * kQRow, ks, h);
      qf.q[mt][ks].load_codes_global(a.q_sf + head_row * WideFrag<VAR>::kCodes, ks, h);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qf.w[mt][u] = __builtin_bit_cast(v4f, ldg_untracked(a.w + slot * 64 + 32 * mt + 8 * u + 4 * h));
  }
}

// ------------------------------------------------------------- main kernel

template <int VAR>
__device__ __forceinline__ float stage_scale(const uint8_t* stage, int token) {
  if constexpr (VAR == 0) {
    return *reinterpret_cast<const float*>(stage + PageLayout<0>::kKeyBytes + 4 * token);
  } else {
    return 1.0f;
  }
}

// Scores this wave's share of one staged page and stores it.
template <int N, int OUTT, int TW, int VAR>
__device__ __forceinline__ void score_page(const QueryFrag<TW, VAR>& qf,
                                           const uint8_t* stage, const MqaArgs& a, int b, int j,
                                           bool valid, int t0, int s0, int lane) {
  constexpr int SW = WaveSplit<N>::SW;
  static_assert(TW == WaveSplit<N>::TW, "the wave's slots");
  const int g = lane >> 4, rr = lane & 15;
  float part[TW][SW];
#pragma unroll
  for (int si = 0; si < SW; ++si) {
    Frag<VAR> kf;
    kf.load_stage(stage, 16 * (s0 + si) + rr, g);
    // The widening and the matrix products of a sub-tile run at raised wave
    // priority, the rectified head sums at the normal one: a wave that has
    // products ready is issued first and keeps the matrix pipe fed, and the
    // other waves' head sums fill the vector issue slots in between.
    __builtin_amdgcn_s_setprio(1);
    const auto kop = key_operand(kf);
    // all matrix products of the sub-tile first, then the rectified head sums
    v4f acc[TW][4];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[t][mt] = mma(qf.op[mt][t], kop);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      // two independent partial sums shorten the dependent FMA chain
      float s_even = 0.0f, s_odd = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4f w = qf.w[mt][t];
        s_even = __builtin_fmaf(w[0], relu(acc[t][mt][0]), s_even);
        s_odd = __builtin_fmaf(w[1], relu(acc[t][mt][1]), s_odd);
        s_even = __builtin_fmaf(w[2], relu(acc[t][mt][2]), s_even);
        s_odd = __builtin_fmaf(w[3], relu(acc[t][mt][3]), s_odd);
      }
      part[t][si] = s_even + s_odd;
    }
  }
  const long long col0 = (long long)j * kPage;
  if constexpr (SW == 4) {
    // lane l ends with token l of the page
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      float v = row_transpose_reduce4(part[t][0], part[t][1], part[t][2], part[t][3]);
      v *= stage_scale<VAR>(stage, lane);
      store_logit_at<OUTT>(a.out, row_of(a, b, t0 + t) * a.out_row_stride + col0, lane, v, valid);
    }
  } else if constexpr (SW == 2) {
    // rows 0-1 end with sub-tile s0, rows 2-3 with s0+1
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      float x = part[t][0], y = part[t][1];
      swap32(x, y);
      float s = x + y;
      float u = s;
      swap16(s, u);
      float v = s + u;
      const int token = 16 * (s0 + (lane >> 5)) + rr;
      v *= stage_scale<VAR>(stage, token);
      if ((g & 1) == 0)
        store_logit_at<OUTT>(a.out, row_of(a, b, t0 + t) * a.out_row_stride + col0, token, v,
                             valid);
    }
  } else {
    static_assert(TW == 1 && SW == 1, "unsupported split");
    float v = row_reduce4(part[0][0]);
    const int token = 16 * s0 + rr;
    v *= stage_scale<VAR>(stage, token);
    if (g == 0)
      store_logit_at<OUTT>(a.out, row_of(a, b, t0) * a.out_row_stride + col0, token, v, valid);
  }
}

// Scores this wave's share of one staged page with 32x32 tiles (MXFP4): one
// query slot, SW/2 32-token halves starting at half s0/2.  All key fragments
// of the share are read from LDS first so their latency overlaps the first
// products.
template <int N, int OUTT, int VAR>
__device__ __forceinline__ void score_page(const WideQuery<VAR>& qf, const uint8_t* stage,
                                           const MqaArgs& a, int b, int j, bool valid, int t0,
                                           int s0, int lane) {
  constexpr int NT = WaveSplit<N>::SW / 2;
  static_assert(NT == 1 || NT == 2, "wide split covers one or two halves");
  const int h = lane >> 5, rr = lane & 31, nt0 = s0 / 2;
  WideFrag<VAR> kf[NT][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) kf[nt][ks].load_stage(stage, 32 * (nt0 + nt) + rr, ks, h);
  const int token = NT == 2 ? lane : 32 * nt0 + rr;
  const float sp = stage_scale<VAR>(stage, token);
  float part[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // the two head tiles alternate so that no product waits on the one just issued
    v16f acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = mma_wide(qf.op[mt][0], kf[nt][0], (v16f){});
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = mma_wide(qf.op[mt][1], kf[nt][1], acc[mt]);
    float s_even = 0.0f, s_odd = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v4f w = qf.w[mt][u];
        s_even = __builtin_fmaf(w[0], relu(acc[mt][4 * u + 0]), s_even);
        s_odd = __builtin_fmaf(w[1], relu(acc[mt][4 * u + 1]), s_odd);
        s_even = __builtin_fmaf(w[2], relu(acc[mt][4 * u + 2]), s_even);
        s_odd = __builtin_fmaf(w[3], relu(acc[mt][4 * u + 3]), s_odd);
      }
    part[nt] = s_even + s_odd;
  }
  // lanes l and l ^ 32 hold the two head halves of one token
  float x = part[0], y = part[NT - 1];
  swap32(x, y);
  const float v = (x + y) * sp;  // NT == 2: lane l has token l; else lanes < 32 have it
  const long long idx = row_of(a, b, t0) * a.out_row_stride + (long long)j * kPage + token;
  if (NT == 2 || h == 0) store_logit<OUTT>(a.out, idx, v, valid);
}

// ------------------------------------------- head sum on the matrix unit

// With bf16 output the MXFP4 kernels sum the heads on the matrix unit.  The
// 16x16x128 products leave each lane 16 heads x 1 token of a slot (four head
// tiles); the rectified scores are packed to bf16 and multiplied by the
// slot's weights (bf16) with 16x16x32 bf16 products.  Slot t's weights are
// row t of the A operand and zero elsewhere, so the products of all of the
// wave's slots accumulate into one result whose row t is slot t's logits
// (lanes 0..15, element t).  One vector instruction per score (half a
// conversion, half a packed max) instead of two, and no cross-lane
// reduction.  Each rectified score and each weight is rounded to bf16 once
// (relative error <= 2^-9 each), so the head sum carries at most
// 2^-8 * sum_h |w_h| relu(S_h) of extra error, which the bf16 output's own
// rounding (2^-9) and tolerance absorb; fp32 output keeps the exact path.
// FP8 sums the heads in fp32 for both outputs: its f16 products already keep
// the matrix unit busiest, and the fp32 sum adds no error.
template <int N, int VAR, int OUTT> struct HeadSumOnMatrix {
  static constexpr bool value = OUTT == 1 && VAR != 0;
};

// The wave's TW slots of request b: each slot's query in four head tiles and
// its head weights as bf16 A operands.  Reduction K step s covers head tiles
// 2s and 2s+1; lane l (group g = l >> 4) holds K slots 8g .. 8g+7, element
// e <-> head 32s + 16(e >> 2) + 4g + (e & 3), which is where the first stage
// leaves that head's score in the B operand.
template <int TW, int VAR> struct RedQuery {
  static_assert(VAR != 0, "the matrix-unit head sum serves MXFP4");
  Frag<VAR> q[4][TW];                 // [head tile][slot], as loaded
  QOperandOf<Frag<VAR>> op[4][TW];    // as multiplied
  v4f wraw[TW][2][2];  // [slot][K step][head tile within the step]: as loaded
  v8bf wa[TW][2];      // [slot][K step]: A operand, nonzero in row `slot` only
};

template <int TW, int VAR>
__device__ __forceinline__ void settle_query(RedQuery<TW, VAR>& qf) {
  const int row = threadIdx.x & 15;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      settle(qf.q[mt][t].v);
      qf.q[mt][t].settle_codes();
      qf.op[mt][t] = query_operand(qf.q[mt][t]);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      settle(qf.wraw[t][st][0]);
      settle(qf.wraw[t][st][1]);
      v8bf w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (__bf16)(row == t ? qf.wraw[t][st][e >> 2][e & 3] : 0.0f);
      qf.wa[t][st] = w;
    }
  }
}

template <int N, int TW, int VAR>
__device__ __forceinline__ void load_red_query(RedQuery<TW, VAR>& qf, const MqaArgs& a, int b,
                                               int t0, int lane) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const long long slot = row_of(a, b, t0 + t);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const long long head_row = slot * 64 + 16 * mt + r;
      qf.q[mt][t].load_global(a.q + head_row * 64, g);
      qf.q[mt][t].load_codes_global(a.q_sf + head_row * Frag<VAR>::kCodes, g);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        qf.wraw[t][st][hh] = __builtin_bit_cast(
            v4f, ldg_untracked(a.w + slot * 64 + 32 * st + 16 * hh + 4 * g));
  }
}

// MXFP4: the lane's key and code addresses of sub-tile 0 (rows from 16 s0),
// computed once per page; sub-tile s adds 16 s rows of each (16 s * kRowStride
// / 16 s * kCodeStride bytes).  The
// empty asm makes the two bases opaque, so the compiler keeps them as bases
// with the sub-tile constant in the offset field (rather than hoisting one
// lane offset per sub-tile and adding the page base to each).
template <int VAR>
struct Fp4SubtileBase {
  using L = PageLayout<VAR>;
  static constexpr int kCodes = L::kCodes;
  typedef __attribute__((address_space(3))) const uint8_t* lds_ptr;
  lds_ptr key, scale;
  __device__ __forceinline__ Fp4SubtileBase(const uint8_t* stage, int s0, int rr, int g) {
    const lds_ptr st = (lds_ptr)stage;
    key = st + L::row_off(16 * s0 + rr) + L::chunk_off(rr, g);
    scale = st + L::code_off(16 * s0 + rr) + (kCodes == 4 ? g : 2 * g);
    asm("" : "+v"(key));
    asm("" : "+v"(scale));
  }
  typedef __attribute__((address_space(3))) const v4i* lds_v4i;
  __device__ __forceinline__ void load(Frag<VAR>& f, int s) const {
    if constexpr (L::kRowStride % 16 == 0) {
      f.v = *reinterpret_cast<lds_v4i>(key + 16 * s * L::kRowStride);
    } else {
      typedef __attribute__((address_space(3))) const int* lds_int;
      const lds_int q = (lds_int)(key + 16 * s * L::kRowStride);
      f.v = (v4i){q[0], q[1], q[2], q[3]};
    }
    f.sf = scale[16 * s * L::kCodeStride];
    if constexpr (kCodes == 8) f.sf2 = scale[16 * s * L::kCodeStride + 1];
  }
};

// Rectified bf16 pair: round to nearest even, then max with +0 as int16 (a
// bf16 bit pattern with the sign bit set is a negative int16).
__device__ __forceinline__ uint32_t relu_bf16x2(float x, float y) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2bf p = __builtin_convertvector((v2f){x, y}, v2bf);
  const v2s m = __builtin_elementwise_max(__builtin_bit_cast(v2s, p), (v2s){0, 0});
  return __builtin_bit_cast(uint32_t, m);
}

// Scores this wave's share of one staged page (TW slots, SW 16-token
// sub-tiles from s0) with the head sum on the matrix unit.
template <int N, int OUTT, int TW, int VAR>
__device__ __forceinline__ void score_page(const RedQuery<TW, VAR>& qf, const uint8_t* stage,
                                           const MqaArgs& a, int b, int j, bool valid, int t0,
                                           int s0, int lane) {
  constexpr int SW = WaveSplit<N>::SW;
  static_assert(TW == WaveSplit<N>::TW && TW <= 4, "one result row per slot");
  const int g = lane >> 4, rr = lane & 15;
  const long long col0 = (long long)j * kPage;
  Frag<VAR> kf[SW];
  const Fp4SubtileBase<VAR> base(stage, s0, rr, g);
#pragma unroll
  for (int si = 0; si < SW; ++si) base.load(kf[si], si);
  // All sub-tiles first (no store, hence no branch, in between, so the
  // products of one sub-tile overlap the packing of the previous one).
  v4f r[SW];
#pragma unroll
  for (int si = 0; si < SW; ++si) {
    r[si] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      v4f acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mma(qf.op[mt][t], kf[si]);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v4f& lo = acc[2 * st];
        const v4f& hi = acc[2 * st + 1];
        const uint32_t p0 = relu_bf16x2(lo[0], lo[1]), p1 = relu_bf16x2(lo[2], lo[3]);
        const uint32_t p2 = relu_bf16x2(hi[0], hi[1]), p3 = relu_bf16x2(hi[2], hi[3]);
        const v8bf kb = __builtin_bit_cast(v8bf, (v4i){(int)p0, (int)p1, (int)p2, (int)p3});
        r[si] = mfma_bf16(qf.wa[t][st], kb, r[si]);
      }
    }
  }
  // Row t of sub-tile si's result (lanes 0..15, element t) holds slot t's
  // logits of tokens 16(s0+si) + 0..15.  The permlane swaps gather the
  // sub-tiles into consecutive 16-lane rows: lane l then holds token 16 s0 + l.
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const long long row = row_of(a, b, t0 + t) * a.out_row_stride + col0;
    if constexpr (SW == 4) {
      float x0 = r[0][t], x1 = r[1][t], x2 = r[2][t], x3 = r[3][t];
      swap16(x0, x1);  // x0 rows: sub-tile 0, sub-tile 1, -, -
      swap16(x2, x3);  // x2 rows: sub-tile 2, sub-tile 3, -, -
      swap32(x0, x2);  // x0 rows: sub-tiles 0, 1, 2, 3
      const int token = 16 * s0 + lane;
      store_logit_at<OUTT>(a.out, row, token, x0 * stage_scale<VAR>(stage, token), valid);
    } else if constexpr (SW == 2) {
      float x0 = r[0][t], x1 = r[1][t];
      swap16(x0, x1);  // x0 rows: sub-tile 0, sub-tile 1, -, -
      const int token = 16 * s0 + lane;
      if (lane < 32)
        store_logit_at<OUTT>(a.out, row, token, x0 * stage_scale<VAR>(stage, token), valid);
    } else {
      const int token = 16 * s0 + rr;
      if (g == 0)
        store_logit_at<OUTT>(a.out, row, token, r[0][t] * stage_scale<VAR>(stage, token), valid);
    }
  }
}

template <bool Wide, int N, int VAR> struct QueryPick { using type = QueryFrag<WaveSplit<N>::TW, VAR>; };
template <int N, int VAR> struct QueryPick<true, N, VAR> { using type = WideQuery<VAR>; };
template <int N, int VAR, int OUTT, bool Red = HeadSumOnMatrix<N, VAR, OUTT>::value>
struct QueryOf : QueryPick<WaveSplit<N>::kWide && VAR != 0, N, VAR> {};
template <int N, int VAR, int OUTT> struct QueryOf<N, VAR, OUTT, true> {
  using type = RedQuery<WaveSplit<N>::TW, VAR>;
};

template <int N, int TW, int VAR>
__device__ __forceinline__ void load_query_any(QueryFrag<TW, VAR>& qf, const MqaArgs& a, int b,
                                               int t0, int lane) {
  load_query<N, TW, VAR>(qf, a, b, t0, lane);
}
template <int N, int VAR>
__device__ __forceinline__ void load_query_any(WideQuery<VAR>& qf, const MqaArgs& a, int b, int t0,
                                               int lane) {
  load_query<N, VAR>(qf, a, b, t0, lane);
}
template <int N, int TW, int VAR>
__device__ __forceinline__ void load_query_any(RedQuery<TW, VAR>& qf, const MqaArgs& a, int b,
                                               int t0, int lane) {
  load_red_query<N, TW, VAR>(qf, a, b, t0, lane);
}

// The page stream of one range of flat items f0 .. f0+count-1: issues each
// item's page into the LDS ring (this wave's share of it, direct-to-LDS),
// remembers which page ids were in range, and refills the page-id table every
// kPidTable items.  A page id out of range is replaced by page 0 for the load
// (so every item issues the same loads) and its outputs are written as NaN.
// The page id of the next item to issue is read one item ahead.  Every wave
// of the workgroup makes the same calls (the table fills have barriers).
//
// Start-up: the page ids of the first kFirst items are read straight from the
// block table with scalar loads (all in flight together), and those pages are
// issued before the page-id table is filled, so that the first pages travel
// while the table's block-table loads do.
template <int VAR>
struct PageFeed {
  using L = PageLayout<VAR>;
  static constexpr int kFirst = kStages - 1;  // at most; the pipeline issues kAhead first
  const MqaArgs& a;
  const int* s_prefix;
  int* s_pid;
  uint8_t* ring;
  long long f0, f_end;
  int count, issued, pid_next, wave, lane;
  uint32_t valid_bits;  // bit (item % 32): page id was in range
  typename L::Lanes lanes;
  int first_pid[kFirst];

  // (b, j): item f0's request and page.
  __device__ __forceinline__ PageFeed(const MqaArgs& a_, const int* s_prefix_, int* s_pid_,
                                      uint8_t* ring_, long long f0_, int count_, int b, int j,
                                      int wave_, int lane_)
      : a(a_), s_prefix(s_prefix_), s_pid(s_pid_), ring(ring_), f0(f0_), f_end(f0_ + count_),
        count(count_), issued(0), pid_next(0), wave(wave_), lane(lane_), valid_bits(0),
        lanes(L::lanes(wave_, lane_)) {
    // the (request, page) of items f0 .. f0+kFirst-1 first (LDS reads), then
    // their block-table entries (scalar loads, all in flight together)
    int bk[kFirst], jk[kFirst];
    int bb = b, jj = j, t = tiles_at(s_prefix, b);
#pragma unroll
    for (int k = 0; k < kFirst; ++k) {
      bk[k] = bb;
      jk[k] = jj;
      if (k + 1 < kFirst && ++jj == t) {
        jj = 0;
        do {
          ++bb;
          t = bb < a.batch ? tiles_at(s_prefix, bb) : 1;
        } while (t == 0);
      }
    }
#pragma unroll
    for (int k = 0; k < kFirst; ++k)
      first_pid[k] = k < count ? a.bt[(long long)bk[k] * a.bt_stride + jk[k]] : 0;
  }
  __device__ __forceinline__ uint8_t* stage(int n) const {
    return ring + ((unsigned)n % kStages) * L::kStageBytes;
  }
  __device__ __forceinline__ bool valid(int n) const { return (valid_bits >> (n & 31)) & 1u; }
  __device__ __forceinline__ void issue_page(int pid) {
    const uint32_t ok = page_ok_bit(a, pid);  // an out-of-range id loads page 0
    const uint8_t* page =
        a.kv + (unsigned long long)((uint32_t)pid & (0u - ok)) * (unsigned long long)a.page_stride;
    L::issue(stage(issued), page, lanes, wave, lane);
    valid_bits = (valid_bits & ~(1u << (issued & 31))) | (ok << (issued & 31));
    ++issued;
  }
  // Issues the first `ahead` items (ahead <= kFirst), then fills the first
  // block of the page-id table.  (b, j): item f0's request and page.
  template <int ahead>
  __device__ __forceinline__ void start(int b, int j) {
    static_assert(ahead >= 1 && ahead <= kFirst, "start-up depth");
#pragma unroll
    for (int k = 0; k < ahead; ++k)
      if (issued < count) issue_page(first_pid[k]);
    fill_pid_table(a, s_prefix, s_pid, f0, f_end, b, j);
    ring_barrier();
    if (issued < count) pid_next = uniform(s_pid[issued]);
  }
  __device__ __forceinline__ void issue_next() {
    if (issued >= count) return;
    issue_page(pid_next);
    if (issued < count) {
      if ((unsigned)issued % kPidTable == 0) {
        // next block of page ids; every wave gets here at the same item
        const long long f = f0 + issued;
        const int rb = locate(s_prefix, a.batch, f);
        ring_barrier();
        fill_pid_table(a, s_prefix, s_pid, f, f_end, rb, (int)(f - uniform(s_prefix[rb])));
        ring_barrier();
      }
      pid_next = uniform(s_pid[(unsigned)issued % kPidTable]);
    }
  }
};

// Scores flat items f0 .. f0+count-1, the whole workgroup together.
//
// Page pipeline.  Before waiting for page n, a wave issues its share of page
// n + kAhead into the ring slot that page n + kAhead - kStages used:
//  * when a wave scores only the 16-token sub-tile it loaded itself
//    (next_n = 1), that slot is its own and was consumed in program order: no
//    workgroup barrier at all, kAhead = kStages - 1;
//  * otherwise (waves read sub-tiles other waves loaded) a barrier after
//    page n has landed makes every share visible, and the slot issued into at
//    iteration n belongs to page n - 2, which every wave finished before the
//    barrier of iteration n - 1: kAhead = kStages - 2.
template <int N, int VAR, int OUTT>
__device__ void process_range(const MqaArgs& a, const int* s_prefix, int* s_pid, uint8_t* ring,
                              long long f0, int count) {
  using L = PageLayout<VAR>;
  constexpr int TW = WaveSplit<N>::TW, SW = WaveSplit<N>::SW, WS = 4 / SW;
  constexpr bool kShared = SW != 1;
  constexpr int kAhead = kShared ? kStages - 2 : kStages - 1;
  static_assert(kAhead >= 1, "ring too short");
  const int B = a.batch;
  const int lane = threadIdx.x & (kWave - 1), wave = uniform(threadIdx.x / kWave);
  const int t0 = (wave / WS) * TW, s0 = (wave % WS) * SW;
  // With next_n = 3 the fourth wave has no slot: it loads its share of every
  // page and takes part in the page barriers, but scores nothing.  (When the
  // waves' slot groups cover exactly N slots, every wave has one, known at
  // compile time.)
  const bool has_slot = (4 / WS) * TW <= N || t0 < N;

  const long long P = uniform(s_prefix[B]);
  if (f0 < 0 || f0 >= P) return;
  if (count > P - f0) count = (int)(P - f0);
  if (count <= 0) return;
  int b = locate(s_prefix, B, f0);
  int j = (int)(f0 - uniform(s_prefix[b]));
  PageFeed<VAR> feed(a, s_prefix, s_pid, ring, f0, count, b, j, wave, lane);

  // The first request's query slice is loaded before the first page loads
  // are issued, so that it is complete once page 0 is: the first wait is for
  // page 0, not for every page in flight.
  typename QueryOf<N, VAR, OUTT>::type qf;
  if (has_slot) load_query_any<N>(qf, a, b, t0, lane);
  feed.template start<kAhead>(b, j);
  wait_page<L::kLoadsPerWave, kAhead>(feed.issued - 1);
  if (has_slot) settle_query(qf);

  int n = 0;
  bool first = true;
  while (n < count && b < B) {
    // One request: its query slice is loaded once.  After the first request
    // it is the newest load, so waiting for it also waits for the pages in
    // flight; this happens once per request.
    if (!first && has_slot) {
      load_query_any<N>(qf, a, b, t0, lane);
      wait_vmcnt<0>();
      settle_query(qf);
    }
    first = false;
    const int pages = min(count - n, tiles_at(s_prefix, b) - j);
    for (int k = 0; k < pages; ++k, ++n, ++j) {
      feed.issue_next();
      // kAhead pages were issued after page n, except in the last kAhead
      // iterations of the range
      if (n + kAhead < count)
        wait_vmcnt<kAhead * L::kLoadsPerWave>();
      else
        wait_page<L::kLoadsPerWave, kAhead - 1>(feed.issued - n - 1);
      if constexpr (kShared) ring_barrier();  // every wave's share of page n has landed
      if (has_slot)
        score_page<N, OUTT>(qf, feed.stage(n), a, b, j, feed.valid(n), t0, s0, lane);
    }
    // next request with pages
    ++b;
    j = 0;
    while (b < B && tiles_at(s_prefix, b) == 0) ++b;
  }
  wait_vmcnt<0>();
}

template <int N, int VAR>
constexpr int ring_bytes() {
  return kStages * PageLayout<VAR>::kStageBytes;
}

// The tensor pointers are separate __restrict__ parameters so the compiler
// knows the kernel's stores never alias its inputs and keeps wave-uniform
// reads (block table, seq_lens, schedule) on the scalar cache.
// The next chunk of the workgroup's pool for the whole workgroup: one lane
// takes it from the pool's counter with a vector-memory atomic (never a
// scalar one) and shares it through LDS.  No load into LDS is in flight here
// (every range ends with its loads waited for), so a plain barrier is safe.
// A pool of NC chunks shared by W workgroups sees exactly NC + W grabs (each
// workgroup grabs until it draws past the pool), so the grab that draws
// NC + W - 1 is the pool's last: it returns the counter to zero, and the next
// launch (or graph replay) needs no clearing.
__device__ __forceinline__ int grab_chunk(WorkCounter* ctr, int last_grab, int* s_slot) {
  if (threadIdx.x == 0) {
    const int c = __hip_atomic_fetch_add(&ctr->next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c == last_grab) __hip_atomic_store(&ctr->next, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_slot = c;
  }
  __syncthreads();
  const int c = uniform(*s_slot);
  __syncthreads();  // every wave has read the slot before it is written again
  return c;
}

// MXFP4 with one code per 32 values and bf16 output runs at 6 waves per SIMD
// (at most 80 registers); the attribute keeps small changes elsewhere in the
// kernel from tipping it to 5.
template <int N, int VAR, int OUTT>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu((VAR == 1 || VAR == 3) && OUTT == 1 ? 6 : 1)))
    mqa_logits_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_sf,
                      const uint8_t* __restrict__ kv, const float* __restrict__ w,
                      const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ bt,
                      const int32_t* __restrict__ schedule, void* __restrict__ out,
                      WorkCounter* __restrict__ work, const MqaArgs dims) {
  MqaArgs a = dims;
  a.q = q;
  a.q_sf = q_sf;
  a.kv = kv;
  a.w = w;
  a.seq_lens = seq_lens;
  a.bt = bt;
  a.schedule = schedule;
  a.out = out;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_wsum[16];
  __shared__ int s_pid[kPidTable];
  uint8_t* ring = smem;
  int* s_prefix = reinterpret_cast<int*>(smem + ring_bytes<N, VAR>());
  // The grid size (a hidden kernel argument), the split parameters and the
  // query's address are read with the first batch of argument loads: read
  // where they are first needed, after the prefix's global loads, each batch
  // would be one more round trip to the arguments before the first page.
  const int G = gridDim.x;
  asm volatile("" ::"s"(G), "s"(q), "s"(dims.cus), "s"(dims.split_skew));
  build_prefix(a.seq_lens, a.batch, a.max_context / kPage, s_prefix, s_wsum);

  // Consecutive units on one XCD: workgroups are dealt to the 8 XCDs
  // round-robin, so renumber them XCD-major before splitting the work.
  const int unit = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  // The schedule header is read at once (no short-circuit between its
  // fields, which would make each read wait for the previous one).
  const int32_t* sc = a.schedule;
  bool use_sched = false;
  if (sc != nullptr) {
    const int h0 = sc[0], h1 = sc[1], h2 = sc[2], h3 = sc[3], h4 = sc[4], h5 = sc[5], h6 = sc[6];
    use_sched = (h0 == kSchedMagic) & (h2 == a.next_n) & (h3 == (VAR == 0 ? 0 : 1)) & (h4 == a.max_context) &
                (h5 == a.batch) & (h6 == s_prefix[a.batch]) & (h1 > 0);
  }
  if (use_sched) {
    // Units come from the schedule's split points (flat item indices); the
    // request and page of each item are re-derived from the current seq_lens,
    // so even a stale schedule cannot address outside the inputs.
    const int U = sc[1];
    for (int u = unit; u < U; u += G) {
      const int32_t* e = sc + kSchedHeader + 3 * u;
      const long long f0 = e[2], f1 = e[5];
      if (f1 > f0) process_range<N, VAR, OUTT>(a, s_prefix, s_pid, ring, f0, (int)(f1 - f0));
      ring_barrier();  // the ring and the page-id table are reused by the next unit
    }
  } else {
    // Equal (round-weighted) static ranges over the first S items; with a
    // work counter, the last P - S items are dealt in chunks to whichever
    // workgroups finish their range first, from one pool per XCD (a
    // contiguous share of the dynamic items, and its own counter, so that
    // the grabs of the 8 XCDs do not queue on one address).
    const long long P = uniform(s_prefix[a.batch]);
    long long S = P, C = 1, D = 0;
    if (work != nullptr) {
      C = a.dyn_chunk > 0 ? a.dyn_chunk : 1;
      D = P * a.dyn_share / 1024;
      S = P - D;
    }
    long long f0 = split_point(unit, G, a.cus, a.split_skew, S);
    long long cnt = split_point(unit + 1, G, a.cus, a.split_skew, S) - f0;
    const int pools = (G % kXcds == 0) ? kXcds : 1;
    const int pool = pools == kXcds ? blockIdx.x % kXcds : 0;
    const long long p0 = S + D * pool / pools, p1 = S + D * (pool + 1) / pools;
    const int NC = (int)((p1 - p0 + C - 1) / C);
    const int last_grab = NC + G / pools - 1;
    while (true) {
      if (cnt > 0) process_range<N, VAR, OUTT>(a, s_prefix, s_pid, ring, f0, (int)cnt);
      if (work == nullptr) break;
      ring_barrier();  // the ring and the page-id table are reused by the next chunk
      const int c = grab_chunk(work + pool, last_grab, &s_wsum[0]);
      if (c >= NC) break;
      f0 = p0 + (long long)c * C;
      cnt = p1 - f0 < C ? p1 - f0 : C;
    }
  }
}

// ------------------------------------------------------------- launchers

template <int N, int VAR, int OUTT>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&mqa_logits_kernel<N, VAR, OUTT>);
}

template <int N, int VAR>
static const void* kernel_ptr(int out_dtype) {
  return out_dtype == 0 ? kernel_ptr<N, VAR, 0>() : kernel_ptr<N, VAR, 1>();
}

template <int N>
static const void* kernel_ptr(int variant, int out_dtype) {
  switch (variant) {
    case 0: return kernel_ptr<N, 0>(out_dtype);
    case 1: return kernel_ptr<N, 1>(out_dtype);
    case 2: return kernel_ptr<N, 2>(out_dtype);
    case 3: return kernel_ptr<N, 3>(out_dtype);
    case 4: return kernel_ptr<N, 4>(out_dtype);
    default: return nullptr;
  }
}

const void* mqa_kernel_symbol(int slots, int variant, int out_dtype) {
  switch (slots) {
    case 1: return kernel_ptr<1>(variant, out_dtype);
    case 2: return kernel_ptr<2>(variant, out_dtype);
    case 3: return kernel_ptr<3>(variant, out_dtype);
    case 4: return kernel_ptr<4>(variant, out_dtype);
    default: return nullptr;
  }
}

size_t mqa_ring_bytes(int variant, int slots) {
  (void)slots;
  switch (variant) {
    case 0: return ring_bytes<1, 0>();
    case 1: return ring_bytes<1, 1>();
    case 2: return ring_bytes<1, 2>();
    case 3: return ring_bytes<1, 3>();
    case 4: return ring_bytes<1, 4>();
    default: return 0;
  }
}

hipError_t launch_mqa(const MqaArgs& a, int slots, int variant, int out_dtype, int grid,
                      size_t lds_bytes, WorkCounter* work, hipStream_t stream) {
  const void* fn = mqa_kernel_symbol(slots, variant, out_dtype);
  if (!fn) return hipErrorInvalidValue;
  const uint8_t* q = a.q;
  const uint8_t* q_sf = a.q_sf;
  const uint8_t* kv = a.kv;
  const float* w = a.w;
  const int32_t* seq_lens = a.seq_lens;
  const int32_t* bt = a.bt;
  const int32_t* sched = a.schedule;
  void* out = a.out;
  void* args[] = {&q,   &q_sf, &kv,   &w,    &seq_lens,
                  &bt,  &sched, &out, &work, const_cast<MqaArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kBlockThreads), args, lds_bytes, stream);
}

hipError_t launch_schedule(const int32_t* seq_lens, int B, int next_n, int variant,
                           int max_context, int U, int cus, int skew, int32_t* sched,
                           hipStream_t stream) {
  const size_t lds = (size_t)(B + 1) * sizeof(int);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kBlockThreads), lds, stream, seq_lens, B,
                     next_n, variant, max_context, U, cus, skew, sched);
  return hipGetLastError();
}

const void* schedule_kernel_symbol() { return reinterpret_cast<const void*>(&schedule_kernel); }

}  // namespace pmqa
