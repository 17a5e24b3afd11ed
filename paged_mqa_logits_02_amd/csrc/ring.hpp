// Pieces shared by the paged logits kernels: the per-call work split over
// (request, 64-token page) items, the LDS page ring fed by direct-to-LDS loads,
// the FP8 key-page layout and operand fragment, and the page-id table.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "pmqa_internal.h"

namespace pmqa {

// LDS ring slots for pages (measured: 5 and 6 slots within noise on the long
// workloads, fewer resident workgroups for the general kernel's wide shapes).
constexpr int kStages = 4;

// --------------------------------------------------------------- schedule

__device__ __forceinline__ int tiles_of(int L, int max_tiles) {
  if (L <= 0) return 0;
  int t = (L + kPage - 1) / kPage;
  return t < max_tiles ? t : max_tiles;
}

// Exclusive prefix of per-request page counts into s_prefix[0..B]
// (s_prefix[B] = total).  Whole workgroup of kBlockThreads threads; ends with
// a barrier.
__device__ void build_prefix(const int32_t* __restrict__ seq_lens, int B, int max_tiles,
                             int* s_prefix, int* s_wsum) {
  const int tid = threadIdx.x, nthr = kBlockThreads;
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwave = nthr / kWave;
  const int per = (B + nthr - 1) / nthr;
  const int lo = tid * per;
  const int hi = min(lo + per, B);
  // seq_lens's address is wanted here, before the per-thread branch: read
  // there, it would be a second round trip to the kernel arguments after the
  // one that brings B, before the first global load of the launch.
  asm volatile("" ::"s"(seq_lens));
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
// lies in request b at page f - prefix[b].  f is wave-uniform and all 64 lanes
// of the wave call it: a binary search narrows [lo, hi] to fewer than 64
// entries (prefix[lo] <= f throughout), then every lane tests one entry at
// once; prefix is non-decreasing, so the lanes whose entry is <= f are lanes
// 0 .. answer - lo.
__device__ __forceinline__ int locate(const int* s_prefix, int B, long long f) {
  int lo = 0, hi = B;
  while (hi - lo >= kWave) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(s_prefix[mid]) <= f) lo = mid; else hi = mid - 1;
  }
  const int i = lo + (int)(threadIdx.x & (kWave - 1));
  const int v = s_prefix[i <= hi ? i : hi];  // every lane reads inside [lo, hi]
  const unsigned long long le = __ballot(i <= hi && v <= f);
  return lo + __builtin_popcountll(le) - 1;
}

// The same for a value of f per lane (a plain binary search per lane).
__device__ __forceinline__ int locate_lane(const int* s_prefix, int B, long long f) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// In-call work split.  Unit u (the workgroups renumbered XCD-major: the
// dispatcher deals blocks to the 8 XCDs round-robin, unit = (block % 8) *
// (G / 8) + block / 8) takes items [split_point(u), split_point(u + 1)).
// When the grid is R workgroups per CU (G = R * cus), the blocks are
// dispatched in R rounds of one per CU (round = block / cus, which is
// (u % (G/8)) / (cus/8) in unit terms), and the hardware's issue priority for
// older waves makes a CU's round-0 workgroup run fastest and its last-round
// workgroup slowest.  Weight w_r = 1024 + skew * (R-1-2r) / (R-1) per unit of
// round r (skew in 1024ths) gives the early rounds more items so that a CU's
// workgroups finish together; skew 0 (or any other grid) is the equal split.
__device__ __forceinline__ long long split_weight_before(int u, int G, int cus, int skew) {
  const int R = G / cus, per = cus / 8, chunk = G / 8;
  long long wchunk = 0;
  for (int r = 0; r < R; ++r) wchunk += (long long)per * (1024 + skew * (R - 1 - 2 * r) / (R - 1));
  const int y = u % chunk, ry = y / per;
  long long c = (long long)(u / chunk) * wchunk;
  for (int r = 0; r < ry; ++r) c += (long long)per * (1024 + skew * (R - 1 - 2 * r) / (R - 1));
  return c + (long long)(y % per) * (1024 + skew * (R - 1 - 2 * ry) / (R - 1));
}
__device__ __forceinline__ long long split_point(int u, int G, int cus, int skew, long long P) {
  if (skew <= 0 || skew >= 1024 || cus < 8 || cus % 8 != 0 || G % cus != 0 || G / cus < 2) {
    // floor(u * P / G) = u * q + floor(u * r / G) with P = q * G + r, in 32-bit
    // arithmetic when P < 2^31 and G < 2^16 (u <= G, so u * r < G^2 < 2^32)
    if (P >= 0 && P < (1ll << 31) && G > 0 && G < (1 << 16) && u >= 0 && u <= G) {
      const unsigned q = (unsigned)P / (unsigned)G, r = (unsigned)P % (unsigned)G;
      return (long long)((unsigned)u * q + (unsigned)u * r / (unsigned)G);
    }
    return (long long)u * P / G;
  }
  return split_weight_before(u, G, cus, skew) * P / split_weight_before(G, G, cus, skew);
}

// ------------------------------------------------------- page staging (LDS)

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Lane i copies 16 (4) bytes from g to lds_base + 16i (4i); lds_base is uniform.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)lds_base, 16, 0, 0);
}

// The same for KV pages, with the non-temporal (evict-first) cache policy.
// A page is read once.  With the default policy its lines push the output
// lines the kernel has just written out of the caches, and their write-backs
// to HBM land in between the page reads; evict-first page lines leave the
// output lines cached (measured: 3% faster on long FP8 workloads, 6% on short
// ones, 11% with few heads; no change in the HBM bytes read).
//
// The page base is wave-uniform and each lane adds a 32-bit offset that stays
// the same from page to page.  The empty asm redefines the caller's offset
// variable in place at every load, so its zero extension stays next to the
// load (a loop-invariant offset would be hoisted as a 64-bit value and added
// to the base with a 64-bit vector add per load) and the load takes the base
// from scalar registers and the offset from one vector register, with no
// copy of it.
constexpr int kPolicyStream = 2;  // cache-policy operand: NT
__device__ __forceinline__ void dma16_page(const uint8_t* page, uint32_t& off, uint8_t* lds_base) {
  asm volatile("" : "+v"(off));
  __builtin_amdgcn_global_load_lds(page + off, (lds_void_ptr)lds_base, 16, 0, kPolicyStream);
}
__device__ __forceinline__ void dma4_page(const uint8_t* page, uint32_t& off, uint8_t* lds_base) {
  asm volatile("" : "+v"(off));
  __builtin_amdgcn_global_load_lds(page + off, (lds_void_ptr)lds_base, 4, 0, kPolicyStream);
}

// Global loads the compiler does not track: it never inserts a wait for
// them.  The query slice is loaded this way so that it can be issued ahead of
// page loads and waited for with an exact count (wait_vmcnt / wait_page);
// every use follows such a wait and settle().
__device__ __forceinline__ v4i ldg_untracked(const void* p) {
  v4i v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ int ldg_untracked_u8(const void* p) {
  int v;
  asm volatile("global_load_ubyte %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Waits until at most N vector-memory loads of this wave are outstanding
// (s_waitcnt vmcnt(N), other counters untouched).  The compiler's own waitcnt
// tracking sees this wait; it does not track loads into LDS by itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the page ring: waits for this wave's LDS reads only.
// Neither __syncthreads() nor a workgroup fence can be used here: both make
// the compiler wait for every load into LDS still in flight, which would drain
// the ring.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Page layout per variant.  Key rows are stored in LDS with their 16-byte
// chunks XOR-permuted by row (chunk c of row r sits in slot c ^ swz(r)).  The
// permutations were chosen by measurement (rocprof SQ_LDS_BANK_CONFLICT = 0)
// for both operand read patterns: 16 consecutive rows per 16 lanes (16x16
// tiles) and 32 consecutive rows per 32 lanes (32x32 tiles).
template <int VAR> struct PageLayout;

template <> struct PageLayout<0> {       // FP8: 64 x 128 B keys, 64 fp32 scales
  static constexpr int kRowBytes = 128;
  static constexpr int kKeyBytes = kPage * kRowBytes;  // 8192
  static constexpr int kStageBytes = kKeyBytes + kPage * 4;
  static constexpr int kLoadsPerWave = 3;  // two 1 KB key chunks, one scale chunk
  __device__ static int swz(int r) { return (r >> 1) & 7; }
  // Wave w loads key rows 16w .. 16w+15 and scales of tokens 16w .. 16w+15.
  // The per-lane byte offsets inside a page do not change from page to page;
  // they are computed once, so a page's loads take a uniform base address and
  // these offsets (no per-page vector arithmetic).
  struct Lanes {
    uint32_t key[2];
    uint32_t scale;
  };
  __device__ static Lanes lanes(int wave, int lane) {
    Lanes o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (2 * wave + i) + (lane >> 3);
      o.key[i] = r * kRowBytes + 16 * ((lane & 7) ^ swz(r));
    }
    o.scale = kKeyBytes + 64 * wave + 4 * (lane & 15);
    return o;
  }
  __device__ static void issue(uint8_t* stage, const uint8_t* page, Lanes& o, int wave,
                               int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_page(page, o.key[i], stage + 8 * (2 * wave + i) * kRowBytes);
    if (lane < 16) dma4_page(page, o.scale, stage + kKeyBytes + 64 * wave);
  }
};

// ------------------------------------------------------------ operands

// MFMA operand fragment of one 16-row tile.  The K dimension (head_dim) is
// split over lanes identically for the query (A) and key (B) operand, so every
// product pairs matching d.
template <int VAR> struct Frag;

// FP8: lane l holds d in [16g, 16g+16) and [64+16g, 64+16g+16), g = l>>4.
template <> struct Frag<0> {
  v8i v;
  __device__ __forceinline__ void load_global(const uint8_t* row, int g) {
    v4i lo = ldg_untracked(row + 16 * g);
    v4i hi = ldg_untracked(row + 64 + 16 * g);
    v = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ __forceinline__ void load_stage(const uint8_t* stage, int r, int g) {
    const int sw = PageLayout<0>::swz(r);
    const uint8_t* row = stage + r * PageLayout<0>::kRowBytes;
    v4i lo = *reinterpret_cast<const v4i*>(row + 16 * (g ^ sw));
    v4i hi = *reinterpret_cast<const v4i*>(row + 16 * ((4 + g) ^ sw));
    v = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// FP8 operands are multiplied in f16 (exact products, fp32-precision sums): a
// key fragment is widened once and used by every head tile; a query fragment
// is widened once per request.
__device__ __forceinline__ Half32 key_operand(const Frag<0>& k) { return widen32(k.v); }
__device__ __forceinline__ v4f mma(const Half32& q, const Half32& k) {
  return mfma_half32(q, k, (v4f){0.f, 0.f, 0.f, 0.f});
}

// Marks x as redefined here: the empty asm reads and rewrites it, so no use
// of x can be scheduled above this point.  Placed after the explicit wait for
// the (untracked) loads of x, it makes every use see the loaded value.
template <typename T>
__device__ __forceinline__ void settle(T& x) {
  asm volatile("" : "+v"(x));
}

// Row of q, w and out for query slot t of request b: the launch scores slots
// slot0 .. slot0+slots-1 of each request's next_n slots.
__device__ __forceinline__ long long row_of(const MqaArgs& a, int b, int t) {
  return (long long)b * a.next_n + a.slot0 + t;
}

// Stores one logit; an output that depends on an out-of-range page id is a
// quiet NaN, written as a bit pattern (this file is compiled without NaN
// semantics for arithmetic, so no NaN is ever produced by arithmetic).
template <int OUTT>
__device__ __forceinline__ void store_logit(void* out, long long idx, float v, bool valid) {
  if constexpr (OUTT == 0) {
    const uint32_t bits = valid ? __float_as_uint(v) : 0x7FC00000u;
    reinterpret_cast<uint32_t*>(out)[idx] = bits;
  } else {
    const uint16_t bits = valid ? f32_to_bf16_rne(v) : (uint16_t)0x7FC0u;
    reinterpret_cast<uint16_t*>(out)[idx] = bits;
  }
}

// The same at element `start + col` of the output, where `start` is
// wave-uniform and `col` (0 .. 63) the lane's column: as for the page loads,
// the store then takes its base from scalar registers and a 32-bit offset
// from one vector register (no 64-bit vector add per store).
template <int OUTT>
__device__ __forceinline__ void store_logit_at(void* out, long long start, uint32_t col, float v,
                                               bool valid) {
  using T = std::conditional_t<OUTT == 0, uint32_t, uint16_t>;
  T* const base = reinterpret_cast<T*>(out) + start;
  uint32_t off = col * (uint32_t)sizeof(T);
  asm volatile("" : "+v"(off));
  T bits;
  if constexpr (OUTT == 0)
    bits = valid ? __float_as_uint(v) : 0x7FC00000u;
  else
    bits = valid ? f32_to_bf16_rne(v) : (uint16_t)0x7FC0u;
  *reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(base) + off) = bits;
}

// Values read from LDS are wave-uniform here; saying so keeps the cursors in
// scalar registers and the page-id fetch a scalar load.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int tiles_at(const int* s_prefix, int b) {
  return uniform(s_prefix[b + 1] - s_prefix[b]);
}

// 1 if 0 <= pg < num_pages, else 0, by integer arithmetic on the scalar unit
// (a comparison result is a lane mask, which costs a vector select and a
// read-back before it can be shifted into a bit set): for pg >= 0,
// pg - num_pages is negative exactly when pg < num_pages; a negative pg has
// its sign bit set, and ~pg clears the result.
__device__ __forceinline__ uint32_t page_ok_bit(const MqaArgs& a, int pg) {
  const uint32_t p = (uint32_t)pg;
  return ((p - (uint32_t)a.num_pages) & ~p) >> 31;
}

// Waits for the loads of the page scored now, given how many pages were
// issued after it (`ahead`, 0 .. kMax).  The steady state (kMax pages ahead)
// is tested first; fewer pages are ahead only at the end of a range.
template <int LPI, int kMax>
__device__ __forceinline__ void wait_page(int ahead) {
  static_assert(kMax * LPI < 64, "vmcnt range");
  if (ahead >= kMax) {
    wait_vmcnt<kMax * LPI>();
  } else if constexpr (kMax > 1) {
    wait_page<LPI, kMax - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

constexpr int kPidTable = 512;  // page ids of the next items, in LDS

// Fills s_pid[0 .. kPidTable) with the page ids of flat items f .. f+kPidTable-1 (up
// to f_end); entries past the end are not written.  (b, j) is item f's
// request and page.  Thread t walks from there to item f+t, request by
// request (a unit spans few requests, so this is a few LDS reads).  Whole
// workgroup; the caller places the barrier.
__device__ __forceinline__ void fill_pid_table(const MqaArgs& a, const int* s_prefix, int* s_pid,
                                               long long f, long long f_end, int b, int j) {
  for (int t = threadIdx.x; t < kPidTable; t += blockDim.x) {
    if (f + t < f_end) {
      int bb = b, jj = j + t, pid = -1;
      while (bb < a.batch) {
        const int tiles = s_prefix[bb + 1] - s_prefix[bb];
        if (jj < tiles) break;
        jj -= tiles;
        ++bb;
      }
      if (bb < a.batch) pid = a.bt[(long long)bb * a.bt_stride + jj];
      s_pid[t] = pid;
    }
  }
}

}  // namespace pmqa
