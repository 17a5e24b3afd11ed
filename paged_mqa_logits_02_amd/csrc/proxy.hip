// Block-max proxy score with NVFP4 query and keys on gfx950.
//
// out[h, t, i] = max over the visible keys k of KV block t (keys 128t ..
// 128t+127 of token i's request) of g * (q[i, h] . k[k, kvh]), g = the
// product of the two global scales, kvh = h / (Hq / Hkv); -inf where the
// block holds no visible key (FlashInfer "flashinfer.msa_ops.
// msa_proxy_score_fp4": description, parameter list and "Returns").  Causal
// visibility: key k is visible to token p of its request iff k <= q_offset +
// p, q_offset defaulting to Lk - Lq.  With reduce_heads the heads are reduced
// by max into one output plane.
//
// Values are e2m1 times the e4m3 scale of their 16-value block.  Such a
// product has at most six significant bits and lies in [2^-10, 2688], so each
// operand is dequantised exactly into f16 (the conversion's scale operand
// applies only a power of two, so the e4m3 scale is a separate packed f16
// multiply) and the 16x16x32 f16 matrix instruction forms exact products
// with fp32 sums.
//
// Work: a unit is (request, KV head, token chunk, KV block).  The query rows
// of a unit are the chunk's tokens x the KV head's group of query heads,
// token-major, up to 16*NT rows (NT row tiles).  Keys are the A operand (16
// keys per tile, eight tiles per block) and the query rows the B operand, so
// lane l of a product holds keys 4(l>>4) .. 4(l>>4)+3 of a tile for query
// row l & 15: the block max is a running element-wise max over the eight
// key tiles, then a max over the four 16-lane rows.  Each wave takes a
// contiguous range of units (units of one request and KV head are adjacent,
// so the query rows are reused across blocks).  Each wave has a private 9 KB
// LDS slot: at the start of a unit it copies the slot (that unit's keys and
// scales) into registers and at once loads the whole next unit into the slot
// with direct-to-LDS copies, so a full unit is in flight while one is scored
// (a unit's 9 KB, 12 waves per CU); page ids are read 64 units ahead (one per
// lane).  With reduce_heads the units of one (token
// chunk, block) run over the KV heads consecutively and the wave keeps the
// per-token max across them.  Blocks past a request's last visible one are
// never read: a final sweep writes their -inf (and every output of a token
// in no request) with coalesced stores along the token axis.
#include "device.hpp"
#include "pmqa_internal.h"

namespace pmqa {
namespace {

constexpr int kBlk = 128;  // keys per KV block
constexpr int kRows = 16;  // query rows per row tile

// Per-request fields, computed identically by the prologue and the walk.
struct ProxyReq {
  int q0, lq;       // first query token, token count
  int lk;           // key count
  int off;          // causal offset
  int tiles;        // blocks with a visible key (at most max_k_tiles)
  int chunks;       // token chunks
  long long kbase;  // flat keys: first key row of the request
  bool bad;         // flat keys: the request's keys lie outside the buffer
};

__device__ __forceinline__ ProxyReq proxy_req(const ProxyArgs& a, int r) {
  ProxyReq q;
  int q0 = a.cu_q[r], q1 = a.cu_q[r + 1];
  q0 = min(max(q0, 0), a.total_q);
  q1 = min(max(q1, q0), a.total_q);
  q.q0 = q0;
  q.lq = q1 - q0;
  long long lk, kb = 0;
  if (a.paged) {
    lk = a.seqused[r];
    lk = max(lk, 0ll);
    lk = min(lk, (long long)a.pt_width * kBlk);
  } else {
    kb = a.cu_k[r];
    lk = (long long)a.cu_k[r + 1] - kb;
    lk = max(lk, 0ll);
  }
  q.lk = (int)lk;
  q.kbase = kb;
  q.bad = !a.paged && (kb < 0 || kb + lk > a.total_k);
  q.off = a.q_offset ? a.q_offset[r] : q.lk - q.lq;
  long long tiles = (lk + kBlk - 1) / kBlk;
  tiles = min(tiles, (long long)a.max_k_tiles);
  if (a.causal) {
    const long long last = (long long)q.off + q.lq - 1;  // the last token's last visible key
    tiles = min(tiles, last < 0 ? 0ll : last / kBlk + 1);
  }
  if (q.lq == 0) tiles = 0;
  q.tiles = (int)tiles;
  q.chunks = (q.lq + a.tc - 1) / a.tc;
  return q;
}

__device__ __forceinline__ int units_of(const ProxyArgs& a, const ProxyReq& q) {
  return q.tiles * q.chunks * a.hkv;
}

// s_cuq[r] = first token of request r (s_cuq[B] = end of the last),
// s_tiles[r] = its blocks with a visible key, and s_prefix = exclusive prefix
// of units per request; whole workgroup.
__device__ void build_tables(const ProxyArgs& a, int* s_cuq, int* s_tiles, int* s_prefix,
                             int* s_wsum) {
  const int B = a.batch;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int per = (B + kBlockThreads - 1) / kBlockThreads;
  const int lo = min(tid * per, B), hi = min(lo + per, B);
  int sum = 0;
  for (int r = lo; r < hi; ++r) {
    const ProxyReq q = proxy_req(a, r);
    const int u = units_of(a, q);
    s_cuq[r] = q.q0;
    if (r == B - 1) s_cuq[B] = q.q0 + q.lq;
    s_tiles[r] = q.tiles;
    s_prefix[r] = u;
    sum += u;
  }
  const int incl = wave_inclusive_scan(sum, lane);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kBlockThreads / kWave; ++w) {
    const int v = s_wsum[w];
    base += w < wave ? v : 0;
    total += v;
  }
  int run = base + incl - sum;
  for (int r = lo; r < hi; ++r) {
    const int u = s_prefix[r];
    s_prefix[r] = run;
    run += u;
  }
  if (tid == 0) {
    s_prefix[B] = total;
    if (B == 0) s_cuq[0] = 0;
  }
  __syncthreads();
}

// Largest r in [0, B] with prefix[r] <= f (the request of unit f).
__device__ __forceinline__ int locate_unit(const int* s_prefix, int B, int f) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(s_prefix[mid]) <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same search per lane (f differs between lanes).
__device__ __forceinline__ int locate_unit_lane(const int* s_prefix, int B, int f) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Page ids of units f .. f+63 (lane k: unit f + k, if below f_end): paged
// keys only.  Block of a unit from its request's position in the walk order.
__device__ __forceinline__ int pids_of(const ProxyArgs& a, const int* s_prefix, const int* s_tiles,
                                       int f, int f_end, int lane) {
  const int fu = f + lane;
  if (!a.paged || fu >= f_end) return 0;
  const int r = locate_unit_lane(s_prefix, a.batch, fu);
  const int local = fu - s_prefix[r];
  const int tiles = s_tiles[r];
  const int t = a.reduce ? (local / a.hkv) % tiles : local % tiles;
  return a.pt[(long long)r * a.pt_stride + t];
}

// One unit of the wave's walk (wave-uniform).
struct Unit {
  int r, j, c, t;
  ProxyReq q;
};

// Unit f of request r (f - prefix[r] units into it).
__device__ __forceinline__ void unit_at(const ProxyArgs& a, Unit& u, int r, int local) {
  u.r = r;
  u.q = proxy_req(a, r);
  if (!a.reduce) {  // KV head, chunk, block; blocks fastest
    u.t = local % u.q.tiles;
    const int x = local / u.q.tiles;
    u.c = x % u.q.chunks;
    u.j = x / u.q.chunks;
  } else {  // chunk, block, KV head; KV heads fastest
    u.j = local % a.hkv;
    const int x = local / a.hkv;
    u.t = x % u.q.tiles;
    u.c = x / u.q.tiles;
  }
}

__device__ __forceinline__ void advance(const ProxyArgs& a, const int* s_prefix, Unit& u) {
  bool next_req;
  if (!a.reduce) {
    next_req = false;
    if (++u.t == u.q.tiles) {
      u.t = 0;
      if (++u.c == u.q.chunks) {
        u.c = 0;
        if (++u.j == a.hkv) next_req = true;
      }
    }
  } else {
    next_req = false;
    if (++u.j == a.hkv) {
      u.j = 0;
      if (++u.t == u.q.tiles) {
        u.t = 0;
        if (++u.c == u.q.chunks) next_req = true;
      }
    }
  }
  if (next_req) {
    int r = u.r + 1;
    while (r < a.batch &&
           __builtin_amdgcn_readfirstlane(s_prefix[r + 1]) ==
               __builtin_amdgcn_readfirstlane(s_prefix[r]))
      ++r;
    if (r < a.batch) unit_at(a, u, r, 0);
    else u.r = a.batch;
  }
}

// Raw operands of one unit, as loaded: the lane's 16 bytes and two scales of
// each of the eight key tiles, and of each query row tile.
template <int NT>
struct Raw {
  v4i k[8];
  uint32_t ks[8];
  v4i q[NT];
  uint32_t qs[NT];
};

// The lane's query row in each row tile, token-major: row 16nt + (l & 15) =
// tok * group + hg.  Fixed for the whole kernel.
template <int NT>
struct LaneRows {
  int tok[NT];  // token within the unit's chunk (>= tc: no row)
  int hg[NT];   // head within the KV head's group
  __device__ __forceinline__ LaneRows(const ProxyArgs& a, int lane) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int m = kRows * nt + (lane & 15);
      tok[nt] = m / a.group;
      hg[nt] = m - tok[nt] * a.group;
    }
  }
};

struct RowOf {
  int p;      // token within the request (valid rows only)
  int hg;     // head within the KV head's group
  bool valid;
};
template <int NT>
__device__ __forceinline__ RowOf row_of_lane(const ProxyArgs& a, const Unit& u,
                                             const LaneRows<NT>& lr, int nt) {
  RowOf o;
  o.hg = lr.hg[nt];
  o.p = u.c * a.tc + lr.tok[nt];
  o.valid = lr.tok[nt] < a.tc && o.p < u.q.lq;
  return o;
}

template <int NT>
__device__ __forceinline__ void issue_query(const ProxyArgs& a, const Unit& u,
                                            const LaneRows<NT>& lr, Raw<NT>& raw, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const RowOf ro = row_of_lane(a, u, lr, nt);
    const long long row = ro.valid ? ((long long)(u.q.q0 + ro.p) * a.hq + u.j * a.group + ro.hg)
                                   : (long long)u.q.q0 * a.hq;
    raw.q[nt] = ldg<v4i>(a.q + row * 64 + 16 * g);
    raw.qs[nt] = ldg<uint16_t>(a.qs + row * 8 + 2 * g);
  }
}

// A wave's LDS slot: the unit's 128 packed key rows (64 B each, the 16-byte
// chunk c of row r stored at chunk position c ^ ((r >> 2) & 3), so that the
// operand reads of 16 rows x 4 chunks meet every bank once per 16 lanes), then
// their 128 scale rows of 8 bytes.
constexpr int kSlotKeyBytes = kBlk * 64;
constexpr int kSlotBytes = kSlotKeyBytes + kBlk * 8;  // 9 KB
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)lds_base, 16, 0, 2);  // non-temporal
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)lds_base, 4, 0, 2);
}

// Loads unit u's keys and scales into the slot (every lane of the wave).
// Load i of the keys fills slot bytes 1024 i + 16 lane: row 16 i + lane / 4,
// chunk position lane % 4, which holds chunk (lane % 4) ^ ((lane >> 4) & 3)
// of that row.  Paged: the block's rows and scale rows are contiguous; flat:
// rows lie Hkv rows apart and rows past the request's last key repeat it.
__device__ __forceinline__ void issue_unit(const ProxyArgs& a, const Unit& u, int pid,
                                           uint8_t* slot, int lane) {
  const int rr = lane >> 2, pos = lane & 3;
  const uint32_t kchunk = 16u * (uint32_t)(pos ^ ((lane >> 4) & 3));
  if (a.paged) {
    const long long page = (pid >= 0 && pid < a.num_pages) ? pid : 0;
    const uint8_t* kb = a.k + page * a.page_stride + (long long)u.j * kBlk * 64;
    const uint8_t* sb = a.ks + ((page * a.hkv + u.j) * kBlk) * 8;
    const uint32_t lo = (uint32_t)rr * 64u + kchunk;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(kb + 1024u * i + lo, slot + 1024 * i);
    dma16(sb + 16u * lane, slot + kSlotKeyBytes);
  } else {
    if (u.q.bad) return;  // keys outside the buffer: never read (outputs NaN)
    const long long first = u.q.kbase + (long long)kBlk * u.t;
    const int last = min(kBlk - 1, u.q.lk - 1 - kBlk * u.t);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const long long row = first + min(16 * i + rr, last);
      dma16(a.k + (row * a.hkv + u.j) * 64 + kchunk, slot + 1024 * i);
    }
    // scale rows: dword (lane & 1) of row 32 i + lane / 2
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long row = first + min(32 * i + (lane >> 1), last);
      dma4(a.ks + (row * a.hkv + u.j) * 8 + 4 * (lane & 1), slot + kSlotKeyBytes + 256 * i);
    }
  }
}

// The lane's operands of all eight key tiles from the slot.
template <int NT>
__device__ __forceinline__ void read_slot(const uint8_t* slot, Raw<NT>& raw, int lane) {
  typedef __attribute__((address_space(3))) const v4i* lds_v4i;
  typedef __attribute__((address_space(3))) const uint16_t* lds_u16;
  const int g = lane >> 4, c = lane & 15;
  const int kpos = 16 * (g ^ ((c >> 2) & 3));
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int row = 16 * s + c;
    raw.k[s] = *(lds_v4i)(slot + row * 64 + kpos);
    raw.ks[s] = *(lds_u16)(slot + kSlotKeyBytes + row * 8 + 2 * g);
  }
}

// Eight values of one packed dword times the f16 scale pair s (both halves
// equal): exact.
__device__ __forceinline__ v8h dequant8(uint32_t packed, v2h s) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * s;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * s;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * s;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * s;
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 values (16 bytes, the scales of its two 16-blocks in the low
// and high byte of sc) as the four K-step fragments, times sign.
__device__ __forceinline__ void dequant32(const v4i& v, uint32_t sc, _Float16 sign, v8h out[4]) {
  const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sc, 1.0f, false);
  const v2h lo = (v2h){s2[0], s2[0]} * sign, hi = (v2h){s2[1], s2[1]} * sign;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) out[ks] = dequant8((uint32_t)v[ks], ks < 2 ? lo : hi);
}

__device__ __forceinline__ float max_over_rows(float x) {
  float y = x;
  swap32(x, y);
  x = __builtin_fmaxf(x, y);
  y = x;
  swap16(x, y);
  return __builtin_fmaxf(x, y);
}

template <int NT>
struct Query {
  v8h b[NT][4];  // B operand fragments of each row tile
};

template <int NT>
__device__ __forceinline__ void dequant_query(const ProxyArgs& a, const Unit& u,
                                              const LaneRows<NT>& lr, const Raw<NT>& raw,
                                              Query<NT>& qf) {
  const _Float16 sign = a.g < 0.0f ? (_Float16)-1.0f : (_Float16)1.0f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    dequant32(raw.q[nt], raw.qs[nt], sign, qf.b[nt]);
    if (!row_of_lane(a, u, lr, nt).valid) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf.b[nt][ks] = (v8h){};
    }
  }
}

// Scores one unit: per row tile, the lane ends with the block max of query
// row (lane & 15) (scaled by |g|; -inf if no key is visible; NaN if the
// block's page id is out of range and a key is visible).
template <int NT>
__device__ __forceinline__ void score_unit(const ProxyArgs& a, const Unit& u, int pid,
                                           const LaneRows<NT>& lr, const Raw<NT>& raw,
                                           const Query<NT>& qf, int lane, float res[NT]) {
  const int g = lane >> 4;
  const float ninf = -__builtin_inff();
  int lim[NT];  // the lane's largest visible key index, per row tile
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const RowOf ro = row_of_lane(a, u, lr, nt);
    int l = u.q.lk - 1;
    if (a.causal) l = min(l, u.q.off + ro.p);
    lim[nt] = ro.valid ? l : -1;
  }
  // every key of the block visible to every row of the unit: its last key
  // is below the key count and within the chunk's first token's limit
  const int last = kBlk * u.t + kBlk - 1;
  const bool masked = !(last < u.q.lk && (!a.causal || last <= u.q.off + u.c * a.tc));
  v4f run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) run[nt] = (v4f){ninf, ninf, ninf, ninf};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    v8h ka[4];
    dequant32(raw.k[s], raw.ks[s], (_Float16)1.0f, ka);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma_f16(ka[ks], qf.b[nt][ks], acc);
      if (masked) {
        const int k0 = kBlk * u.t + 16 * s + 4 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = k0 + v <= lim[nt] ? acc[v] : ninf;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) run[nt][v] = __builtin_fmaxf(run[nt][v], acc[v]);
    }
    // one key tile at a time: keeps the scheduler from dequantising every
    // tile ahead of the products (eight tiles of f16 operands in registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  const float ag = __builtin_fabsf(a.g);
  const bool bad_page = a.paged ? (pid < 0 || pid >= a.num_pages) : u.q.bad;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float m = __builtin_fmaxf(__builtin_fmaxf(run[nt][0], run[nt][1]),
                              __builtin_fmaxf(run[nt][2], run[nt][3]));
    m = max_over_rows(m);
    const bool any = lim[nt] >= kBlk * u.t;  // a visible key in this block
    float v = m == ninf ? ninf : ag * m;
    if (bad_page && any) v = __builtin_nanf("");
    res[nt] = v;
  }
}

template <int NT, bool RED>
__device__ void run_units(const ProxyArgs& a, const int* s_prefix, const int* s_tiles,
                          float* s_red, uint8_t* slot, int f0, int count, int lane) {
  if (count <= 0) return;
  const int f_end = f0 + count;
  Unit u;
  {
    const int r = locate_unit(s_prefix, a.batch, f0);
    unit_at(a, u, r, f0 - __builtin_amdgcn_readfirstlane(s_prefix[r]));
  }
  // page ids of the next 64 units and of the 64 after them
  int pidv = pids_of(a, s_prefix, s_tiles, f0, f_end, lane);
  int pidv_next = pids_of(a, s_prefix, s_tiles, f0 + 64, f_end, lane);
  const LaneRows<NT> lr(a, lane);
  Raw<NT> raw;
  Query<NT> qf;
  int pid = __builtin_amdgcn_readfirstlane(pidv);
  issue_query(a, u, lr, raw, lane);
  issue_unit(a, u, pid, slot, lane);
  bool newq = true;
  // reduce_heads: per-token running max (lane = token of the chunk) and NaN flag
  float tok_max = -__builtin_inff();
  bool tok_nan = false;
  // A unit's results are stored one unit later, after the next unit's loads
  // are issued: the wait at the start of each unit then finds them long done.
  float pval[NT];
  long long pidx[NT];
  bool pvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) pvalid[nt] = false;
  auto flush = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (pvalid[nt]) a.out[pidx[nt]] = pval[nt];
  };

  for (int n = 0; n < count; ++n) {
    const bool has_next = n + 1 < count;
    Unit un = u;
    if (has_next) advance(a, s_prefix, un);
    if (((n + 1) & 63) == 0) {
      pidv = pidv_next;
      pidv_next = pids_of(a, s_prefix, s_tiles, f0 + n + 65, f_end, lane);
    }
    const int pid_next = __builtin_amdgcn_readlane(pidv, (n + 1) & 63);
    const bool newq_next = has_next && (un.r != u.r || un.j != u.j || un.c != u.c);
    // this unit's keys (and query rows, if new) have landed: into registers,
    // then the next unit into the slot
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt untouched
    asm volatile("" ::: "memory");
    read_slot(slot, raw, lane);
    if (newq) dequant_query(a, u, lr, raw, qf);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt untouched: the slot reads are done
    asm volatile("" ::: "memory");
    if (newq_next) issue_query(a, un, lr, raw, lane);
    if (has_next) issue_unit(a, un, pid_next, slot, lane);
    flush();
    float res[NT];
    score_unit(a, u, pid, lr, raw, qf, lane, res);
    if constexpr (!RED) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const RowOf ro = row_of_lane(a, u, lr, nt);
        const long long h = (long long)u.j * a.group + ro.hg;
        pvalid[nt] = lane < kRows && ro.valid;
        pidx[nt] = (h * a.max_k_tiles + u.t) * a.total_q + u.q.q0 + ro.p;
        pval[nt] = res[nt];
      }
    } else {
      // rows to LDS, then lane tk combines the group's rows of token tk
      if (lane < kRows) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s_red[kRows * nt + lane] = res[nt];
      }
      asm volatile("" ::: "memory");
      if (lane < a.tc) {
        for (int hg = 0; hg < a.group; ++hg) {
          const float v = s_red[lane * a.group + hg];
          tok_nan = tok_nan || __builtin_isnan(v);
          tok_max = __builtin_fmaxf(tok_max, v);
        }
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pvalid[nt] = false;
      if (u.j == a.hkv - 1) {
        const int p = u.c * a.tc + lane;
        pvalid[0] = lane < a.tc && p < u.q.lq;
        pidx[0] = (long long)u.t * a.total_q + u.q.q0 + p;
        pval[0] = tok_nan ? __builtin_nanf("") : tok_max;
        tok_max = -__builtin_inff();
        tok_nan = false;
      }
    }
    u = un;
    pid = pid_next;
    newq = newq_next;
  }
  flush();
}

// -inf for every output no unit writes: blocks at or past a request's
// visible-block count and tokens in no request.  Iterations (token chunk of
// 64, head, block), blocks fastest; lane = token.
__device__ void fill_unwritten(const ProxyArgs& a, const int* s_cuq, const int* s_prefix,
                               long long e0, long long e1, int lane) {
  const int hout = a.reduce ? 1 : a.hq;
  const float ninf = -__builtin_inff();
  int ic_cur = -1, tiles = 0;
  bool tok_ok = false;
  for (long long e = e0; e < e1; ++e) {
    const int t = (int)(e % a.max_k_tiles);
    const long long y = e / a.max_k_tiles;
    const int h = (int)(y % hout);
    const int ic = (int)(y / hout);
    if (ic != ic_cur) {
      ic_cur = ic;
      const int i = 64 * ic + lane;
      tok_ok = i < a.total_q;
      tiles = 0;
      // request of token i: largest r with s_cuq[r] <= i, if i < s_cuq[r+1]
      int lo = 0, hi = a.batch;  // search s_cuq[0 .. B]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cuq[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int r = lo;
      if (r < a.batch && s_cuq[r] <= i && i < s_cuq[r + 1]) {
        const int units = s_prefix[r + 1] - s_prefix[r];
        const int lq = s_cuq[r + 1] - s_cuq[r];
        const int chunks = (lq + a.tc - 1) / a.tc;
        tiles = units / (a.hkv * chunks);
      }
    }
    if (tok_ok && t >= tiles)
      a.out[((long long)h * a.max_k_tiles + t) * a.total_q + 64 * ic + lane] = ninf;
  }
}

template <int NT, bool RED>
__global__ void __launch_bounds__(256) proxy_kernel(const ProxyArgs a) {
  extern __shared__ int smem[];
  __shared__ int s_wsum[kBlockThreads / kWave];
  __shared__ float s_red[kBlockThreads / kWave][kRows * 4];
  uint8_t* slots = reinterpret_cast<uint8_t*>(smem);  // 4 waves x kSlotBytes
  int* s_cuq = smem + 4 * kSlotBytes / 4;
  int* s_tiles = s_cuq + a.batch + 1;
  int* s_prefix = s_cuq + 2 * a.batch + 1;
  build_tables(a, s_cuq, s_tiles, s_prefix, s_wsum);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // consecutive waves on one XCD (workgroups are dealt to the 8 XCDs in turn)
  const int G = gridDim.x;
  const int unit = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const long long W = 4ll * G, w = 4ll * unit + wave;

  const long long P = __builtin_amdgcn_readfirstlane(s_prefix[a.batch]);
  // reduce_heads: ranges hold whole groups of the KV heads of one item
  const long long step = RED ? a.hkv : 1;
  const long long items = P / step;
  const long long f0 = step * (items * w / W), f1 = step * (items * (w + 1) / W);
  run_units<NT, RED>(a, s_prefix, s_tiles, s_red[wave], slots + wave * kSlotBytes, (int)f0,
                     (int)(f1 - f0), lane);

  const long long hout = RED ? 1 : a.hq;
  const long long F = hout * a.max_k_tiles * ((a.total_q + 63) / 64);
  fill_unwritten(a, s_cuq, s_prefix, F * w / W, F * (w + 1) / W, lane);
}

template <int NT, bool RED>
const void* proxy_ptr() {
  return reinterpret_cast<const void*>(&proxy_kernel<NT, RED>);
}

}  // namespace

const void* proxy_kernel_symbol(int nt, int reduce) {
  switch (nt) {
    case 1: return reduce ? proxy_ptr<1, true>() : proxy_ptr<1, false>();
    case 2: return reduce ? proxy_ptr<2, true>() : proxy_ptr<2, false>();
    case 4: return reduce ? proxy_ptr<4, true>() : proxy_ptr<4, false>();
    default: return nullptr;
  }
}

size_t proxy_lds_bytes(int batch) { return 4 * kSlotBytes + (size_t)(3 * batch + 2) * sizeof(int); }

hipError_t launch_proxy(const ProxyArgs& a, int nt, int grid, hipStream_t stream) {
  const void* fn = proxy_kernel_symbol(nt, a.reduce);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<ProxyArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kBlockThreads), args, proxy_lds_bytes(a.batch),
                         stream);
}

}  // namespace pmqa
