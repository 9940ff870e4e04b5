// HIP kernel and C ABI of the speculative-decoding verification sampler,
// written for AMD CDNA4 (gfx950, MI355X).
//
// What is computed (velog "6-1편. Speculative Decoding", section 2
// "알고리즘 4단계" steps 2-4 with section 2-1, the min(1, p/q) rule, and
// section 2-2, the residual norm(max(0, p - q)); greedy rule of "How to
// Scale Your Model -- All About Transformer Inference", Appendix D): see
// include/specverify.h.
//
// How.  The logits are read from HBM exactly once.  Every target row is
// split into chunks of 8192 logits.  A work item is one chunk of one target
// row plus, when the position has a draft, the same chunk of the draft row,
// so p_k and q_k of the same token meet in the same registers.
//
// Schedule.  The kernel is persistent: the host launches as many 256-thread
// workgroups as the GPU holds at once.  Rows are dealt round robin to eight
// groups that match the eight XCDs (workgroup b runs on XCD b % 8); inside a
// group, workgroup j takes items j, j + G, j + 2G, ... of the group's
// row-major item list, so the chunks of a row run together, in one round,
// on one XCD.  While a workgroup works on one item, the 16-byte loads of its
// next item are already in flight (double buffering in registers).
//
//   phase 1   chunk max m_c; e_k = 2^(l_k s - m_c s), s = log2(e) / T, kept
//             in registers; chunk sum s_c.  T = 0: chunk argmax.
//   xch 1     (m_c, s_c) of target and draft go into epoch-tagged slots; the
//             row's chunks read all of them and merge (max, sum 2^((m_c-M)s)),
//             the associative combine of an online softmax.
//   phase 2   with a_c = 2^((m_c - M) s) / S for target (t) and draft (d) and
//             rho = a_d / a_t: p_k = a_t e_t and q_k = a_t rho e_d, so
//             min(p, q) = a_t min(e_t, rho e_d) and max(0, p - q) =
//             a_t max(0, e_t - rho e_d); the chunk sums of both go out (beta,
//             velog section 2-3 item 1, and the residual mass Z, item 2), and
//             the chunk holding the drafted token publishes p(x) and q(x).
//   xch 2     every chunk of the row reads every chunk's sums: Z, beta and
//             the chunk whose CDF interval holds u_gamma * Z (or, for the
//             bonus row and for Z = 0, the CDF of p).
//   owner     that chunk finds the token in its registers (block scan), runs
//             the acceptance test u_i q(x) < p(x), writes the diagnostics and
//             the row result, and counts the row in on its sequence.
//   resolve   the last row of a sequence finds the first rejection n and
//             writes accepted_len and the n + 1 tokens; no host sync.
//
// Synchronisation uses no fences: every value that crosses workgroups
// travels in its own 64-bit slot together with a 32-bit epoch tag, written
// and read with agent-scope atomics, so a reader that sees the tag sees the
// value.  Every wait is bounded by a poll budget; an expired wait is
// reported as accepted_len = -2 and the kernel still ends.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <new>

#include "specverify.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = 32;                 // logits per thread per row
constexpr int kChunk = kThreads * kPerThread;  // 8192 logits per chunk
constexpr int kMaxChunks = 64;                 // V <= 524288
constexpr int kGroups = 8;                     // row groups = XCDs of an MI355X
constexpr int kX1 = 4;                         // exchange-1 slots per chunk
constexpr int kX2 = 2;                         // exchange-2 slots per chunk (+2 per row)
constexpr int kDefaultSpin = 1 << 18;          // ~0.3 s of polling; normal waits are microseconds
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMin = 1.17549435e-38f;
constexpr float kFltMax = 3.40282347e38f;
constexpr uint32_t kTokMask = (1u << 23) - 1;
constexpr uint32_t kAccBit = 1u << 23;
constexpr uint32_t kStatusShift = 24;          // 0 ok, 1 invalid data, 2 wait expired

template <int DT> struct Fmt;
template <> struct Fmt<SPECVERIFY_F32> {
  static constexpr int EPV = 4;   // logits per 16-byte vector
  static constexpr int U = 8;     // vectors per thread per row
  static constexpr int ESIZE = 4;
};
template <> struct Fmt<SPECVERIFY_BF16> {
  static constexpr int EPV = 8;
  static constexpr int U = 4;
  static constexpr int ESIZE = 2;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const void* target;
  const void* draft;
  int64_t tstride;
  int64_t dstride;
  const int32_t* tokens;
  const float* uniforms;
  const float* temps;
  const int32_t* cu_draft;   // NULL: uniform gamma
  int32_t gamma;
  int32_t B;
  int32_t R_d;
  int32_t R_t;
  int32_t V;
  int32_t C;                 // chunks per row
  int32_t G;                 // workgroups per row group
  uint32_t epoch;
  int32_t spin_limit;
  int32_t t_aligned;         // target rows start on 16-byte boundaries
  int32_t d_aligned;
  uint64_t* xch1;            // [rows][C][kX1]
  uint64_t* xch2;            // [rows][C * kX2 + 2]
  uint64_t* rowslot;         // [rows]
  uint64_t* seqctr;          // [max_batch]
  int32_t* acc_len;
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* beta;
  float* resid;
};

// ------------------------------------------------------------------ slots

__device__ __forceinline__ void slot_put(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_putf(uint64_t* p, uint32_t tag, float v) {
  slot_put(p, tag, __float_as_uint(v));
}
// Poll one slot until it carries `tag`; false once `limit` polls have failed.
__device__ __forceinline__ bool slot_get(uint64_t* p, uint32_t tag, int limit, uint32_t& v) {
  for (int k = 0;; ++k) {
    const uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) {
      v = (uint32_t)w;
      return true;
    }
    if (k >= limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------ wave primitives (DPP)
// Reductions leave the same value in every lane and use a fixed order, so
// every workgroup that reduces the same data gets the same bits.

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror: every lane holds its 16-lane row sum
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// Inclusive prefix sum over the 64 lanes, fixed association.
__device__ __forceinline__ float wave_scan(float v, int lane) {
  v += dpp<0x111>(v);   // row_shr:1 (bound_ctrl: 0 enters at the row start)
  v += dpp<0x112>(v);   // row_shr:2
  v += dpp<0x114>(v);   // row_shr:4
  v += dpp<0x118>(v);   // row_shr:8
  const float t0 = lane_f(v, 15), t1 = lane_f(v, 31), t2 = lane_f(v, 47);
  const int row = lane >> 4;
  const float off = row == 0 ? 0.0f : row == 1 ? t0 : row == 2 ? (t0 + t1) : ((t0 + t1) + t2);
  return v + off;
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dppi<0xB1>(v, v));
  v = min(v, dppi<0x4E>(v, v));
  v = min(v, dppi<0x141>(v, v));
  v = min(v, dppi<0x140>(v, v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dppi<0xB1>(v, v));
  v = max(v, dppi<0x4E>(v, v));
  v = max(v, dppi<0x141>(v, v));
  v = max(v, dppi<0x140>(v, v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// (value, index): larger value wins, lower index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& k, float v2, int k2) {
  if (v2 > v || (v2 == v && k2 < k)) {
    v = v2;
    k = k2;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& k) {
  const float v2 = __int_as_float(dppi<CTRL>(__float_as_int(v), __float_as_int(v)));
  const int k2 = dppi<CTRL>(k, k);
  argmax_merge(v, k, v2, k2);
}
__device__ __forceinline__ void wave_argmax(float& v, int& k) {
  argmax_step<0xB1>(v, k);
  argmax_step<0x4E>(v, k);
  argmax_step<0x141>(v, k);
  argmax_step<0x140>(v, k);   // every lane holds its row's (max, first index)
  float bv = lane_f(v, 0);
  int bk = __builtin_amdgcn_readlane(k, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16)
    argmax_merge(bv, bk, lane_f(v, l), __builtin_amdgcn_readlane(k, l));
  v = bv;
  k = bk;
}

// ------------------------------------------------------------------ loads

// Issue this thread's loads of one chunk row: vector u holds tokens
// e0 + u*256*EPV + tid*EPV .. +EPV-1.  Tokens >= V read as -inf; rows not on
// 16-byte boundaries are read element by element.
template <int DT>
__device__ __forceinline__ void issue_chunk(const void* base, int64_t row, int64_t stride, int64_t e0,
                                            int V, int tid, bool aligned, u32x4 (&raw)[Fmt<DT>::U]) {
  using F = Fmt<DT>;
  const char* rowp = (const char*)base + row * stride * F::ESIZE;
  if (aligned && e0 + kChunk <= V) {
#pragma unroll
    for (int u = 0; u < F::U; ++u) {
      const int64_t k = e0 + (int64_t)u * kThreads * F::EPV + (int64_t)tid * F::EPV;
      raw[u] = __builtin_nontemporal_load((const u32x4*)(rowp + k * F::ESIZE));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < F::U; ++u) {
    const int64_t k = e0 + (int64_t)u * kThreads * F::EPV + (int64_t)tid * F::EPV;
    if (aligned && k + F::EPV <= V) {
      raw[u] = __builtin_nontemporal_load((const u32x4*)(rowp + k * F::ESIZE));
    } else if (DT == SPECVERIFY_F32) {
      const uint32_t* p = (const uint32_t*)rowp;
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[u][e] = (k + e < V) ? p[k + e] : 0xFF800000u;
    } else {
      const uint16_t* p = (const uint16_t*)rowp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (k + 2 * e < V) ? p[k + 2 * e] : 0xFF80u;
        const uint32_t hi = (k + 2 * e + 1 < V) ? p[k + 2 * e + 1] : 0xFF80u;
        raw[u][e] = lo | (hi << 16);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void unpack(const u32x4 (&raw)[Fmt<DT>::U], float (&x)[kPerThread]) {
  using F = Fmt<DT>;
#pragma unroll
  for (int u = 0; u < F::U; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = raw[u][e];
      if (DT == SPECVERIFY_F32) {
        x[u * 4 + e] = __uint_as_float(w);
      } else {
        x[u * 8 + 2 * e] = __uint_as_float(w << 16);
        x[u * 8 + 2 * e + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
  }
}

// Exponent offset of a chunk: -m s, or 0 for a chunk of only -inf (so that
// its exponentials are 2^-inf = 0 instead of NaN).
__device__ __forceinline__ float chunk_offset(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : -m * s;
}

// ------------------------------------------------------------------ work items

struct Item {
  int r;       // target row
  int c;       // chunk
  int b;       // sequence
  int gam;     // its draft length
  int d0;      // its first draft row
  int i;       // position in the sequence (r - cu_t[b])
  bool ok;     // consistent cu_draft
  bool pair;   // the position has a draft row
  float T;     // temperature of the sequence
  int xtok;    // drafted token (pair rows)
  float ui;    // acceptance uniform of the position
  float ug;    // uniform of the sequence's final sample
};

__device__ __forceinline__ void item_place(const Params& P, int grp, int idx, Item& it) {
  const int rl = idx / P.C;
  it.c = idx - rl * P.C;
  it.r = rl * kGroups + grp;
}

// Sequence of the item's row, and the per-row scalars (their loads overlap
// the work on the current item).
__device__ __forceinline__ void item_lookup(const Params& P, Item& it) {
  if (P.cu_draft == nullptr) {
    it.b = it.r / (P.gamma + 1);
    it.gam = P.gamma;
    it.d0 = it.b * P.gamma;
  } else {
    int lo = 0, hi = P.B - 1;
    while (lo < hi) {   // largest b with cu_t[b] = cu_draft[b] + b <= r
      const int mid = (lo + hi + 1) >> 1;
      if (P.cu_draft[mid] + mid <= it.r) lo = mid;
      else hi = mid - 1;
    }
    it.b = lo;
    it.d0 = P.cu_draft[it.b];
    it.gam = P.cu_draft[it.b + 1] - it.d0;
  }
  it.i = it.r - (it.d0 + it.b);
  it.ok = it.gam >= 0 && it.d0 >= 0 && it.d0 + it.gam <= P.R_d && it.i >= 0 && it.i <= it.gam;
  it.pair = it.ok && it.i < it.gam;
  it.T = 0.0f;
  it.xtok = 0;
  it.ui = 0.0f;
  it.ug = 0.0f;
  if (it.ok) {
    it.T = P.temps[it.b];
    it.ui = P.uniforms[it.r];
    it.ug = P.uniforms[it.d0 + it.b + it.gam];
    if (it.pair) it.xtok = P.tokens[it.d0 + it.i];
  }
}

// ------------------------------------------------------------------ shared state

struct Shared {
  float red[2 * kWaves];
  int redi[2 * kWaves];
  uint32_t x1[kX1 * kMaxChunks];     // exchange-1 payloads of the row
  uint32_t x2[kX2 * kMaxChunks + 2]; // exchange-2 payloads (+ p(x), q(x))
  float scan[8 * kWaves];            // block scan scratch
  float Z, beta, thr, before;
  float Mt, St, Md, Sd;
  int owner;
  int mode;
  int payload;
  int last;
};

__device__ __forceinline__ void block_max2(float& a, float& b, Shared& sh) {
  a = wave_max(a);
  b = wave_max(b);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.red[w] = a;
    sh.red[kWaves + w] = b;
  }
  __syncthreads();
  a = fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
  b = fmaxf(fmaxf(sh.red[4], sh.red[5]), fmaxf(sh.red[6], sh.red[7]));
  __syncthreads();
}
__device__ __forceinline__ void block_sum2(float& a, float& b, Shared& sh) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.red[w] = a;
    sh.red[kWaves + w] = b;
  }
  __syncthreads();
  a = (sh.red[0] + sh.red[1]) + (sh.red[2] + sh.red[3]);
  b = (sh.red[4] + sh.red[5]) + (sh.red[6] + sh.red[7]);
  __syncthreads();
}
__device__ __forceinline__ void block_argmax(float& v, int& k, Shared& sh) {
  wave_argmax(v, k);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.red[w] = v;
    sh.redi[w] = k;
  }
  __syncthreads();
  v = sh.red[0];
  k = sh.redi[0];
#pragma unroll
  for (int j = 1; j < kWaves; ++j) argmax_merge(v, k, sh.red[j], sh.redi[j]);
  __syncthreads();
}

// Gather n <= 256 slots starting at base into dst (every thread calls).
__device__ __forceinline__ bool gather(uint64_t* base, int n, uint32_t tag, int spin, uint32_t* dst) {
  int ok = 1;
  const int tid = threadIdx.x;
  if (tid < n) {
    uint32_t v = 0;
    ok = slot_get(base + tid, tag, spin, v);
    dst[tid] = v;
  }
  return __syncthreads_and(ok) != 0;
}

// Per-thread argmax of a chunk in token order (first maximum wins) plus a
// flag for NaN / +inf.
template <int DT>
__device__ __forceinline__ void thread_argmax(const float (&x)[kPerThread], int64_t e0, int tid,
                                              float& bv, int& bk, int& bad) {
  using F = Fmt<DT>;
  bv = -__builtin_huge_valf();
  int slot = -1;   // u * EPV + e of the best logit so far
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const float v = x[k];
    bad |= (v != v) | (v == __builtin_huge_valf());
    if (v > bv) {
      bv = v;
      slot = k;
    }
  }
  const int u = slot / F::EPV, e = slot - u * F::EPV;
  bk = slot < 0 ? 0x7FFFFFFF : (int)(e0 + u * (kThreads * F::EPV) + tid * F::EPV + e);
}

// Owner selection over n <= 64 non-negative chunk totals, one per lane of
// wave 0: the first j with tot_j > 0 and incl_j > thr, else the last j with
// tot_j > 0 (rounding guard).  Returns j (-1 if all are 0) and the CDF value
// before j.
__device__ __forceinline__ int owner_select(float tot, int n, float thr, int lane, float& before) {
  const float t = lane < n ? tot : 0.0f;
  const float incl = wave_scan(t, lane);
  const uint64_t hit = __ballot(lane < n && t > 0.0f && incl > thr);
  const uint64_t pos = __ballot(lane < n && t > 0.0f);
  int j;
  if (hit) j = __builtin_ctzll(hit);
  else if (pos) j = 63 - __builtin_clzll(pos);
  else j = -1;
  const float prev = __shfl(incl, j > 0 ? j - 1 : 0);
  before = j > 0 ? prev : 0.0f;
  return j;
}

// Inverse CDF inside one chunk held in registers (every thread calls).  w:
// this thread's weights in the layout of issue_chunk; tau: threshold in the
// chunk's own units.  Token order is round u, then thread, then element.
// Returns the chunk-local index of the first logit with w > 0 whose running
// sum exceeds tau, else of the last logit with w > 0, else -1.
template <int DT>
__device__ __forceinline__ int chunk_search(const float (&w)[kPerThread], float tau, Shared& sh) {
  using F = Fmt<DT>;
  constexpr int U = F::U, EPV = F::EPV;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float g[U], incl[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) a += w[u * EPV + e];
    g[u] = a;
    incl[u] = wave_scan(a, lane);
    if (lane == 63) sh.scan[u * kWaves + wv] = incl[u];
  }
  __syncthreads();
  float round_off = 0.0f;   // total of all earlier rounds
  int cslot = -1, lslot = -1;   // u * EPV + e of this thread's first hit / last positive weight
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float off = round_off;
    for (int k = 0; k < wv; ++k) off += sh.scan[u * kWaves + k];
    float run = off + (incl[u] - g[u]);   // exclusive prefix of this thread's group
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float x = w[u * EPV + e];
      run += x;
      if (x > 0.0f) {
        lslot = u * EPV + e;
        if (run > tau && cslot < 0) cslot = u * EPV + e;
      }
    }
    float rt = round_off;
    for (int k = 0; k < kWaves; ++k) rt += sh.scan[u * kWaves + k];
    round_off = rt;
  }
  // token order: round u first, then thread, then element
  int cand = cslot < 0 ? 0x7FFFFFFF : (cslot / EPV) * (kThreads * EPV) + tid * EPV + cslot % EPV;
  int lastpos = lslot < 0 ? -1 : (lslot / EPV) * (kThreads * EPV) + tid * EPV + lslot % EPV;
  cand = wave_min_i(cand);
  lastpos = wave_max_i(lastpos);
  __syncthreads();
  if (lane == 0) {
    sh.redi[wv] = cand;
    sh.redi[kWaves + wv] = lastpos;
  }
  __syncthreads();
  int c2 = 0x7FFFFFFF, l2 = -1;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    c2 = min(c2, sh.redi[k]);
    l2 = max(l2, sh.redi[kWaves + k]);
  }
  __syncthreads();
  return c2 != 0x7FFFFFFF ? c2 : l2;
}

// ------------------------------------------------------------------ row result and sequence

__device__ __forceinline__ uint32_t row_payload(int status, bool acc, int tok) {
  return ((uint32_t)status << kStatusShift) | (acc ? kAccBit : 0u) |
         (status == 0 ? ((uint32_t)tok & kTokMask) : 0u);
}

// Publish the row result and count the row in on its sequence (one thread).
// True for the last of the sequence's gamma + 1 rows.  The counter word holds
// (epoch, count); a stale epoch counts as zero, so no run depends on what
// earlier runs left behind.
__device__ __forceinline__ bool arrive(const Params& P, int r, int b, int gam, uint32_t payload) {
  slot_put(P.rowslot + r, P.epoch, payload);
  uint64_t* ctr = P.seqctr + b;
  uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t cnt = 0;
  for (int k = 0; k < (1 << 20); ++k) {
    cnt = ((uint32_t)(old >> 32) == P.epoch) ? (uint32_t)old + 1u : 1u;
    const uint64_t nw = ((uint64_t)P.epoch << 32) | cnt;
    if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  return cnt == (uint32_t)gam + 1u;
}

// The last row of sequence b to finish: first rejection n, accepted length
// and the n + 1 emitted tokens (wave 0).
__device__ __forceinline__ void resolve(const Params& P, int b, int t0, int d0, int gam, int lane) {
  int n = gam, st = 0;
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    uint32_t v = 0;
    int okj = 1;
    if (j <= gam) okj = slot_get(P.rowslot + t0 + j, P.epoch, P.spin_limit, v);
    const int sj = (j <= gam) ? (okj ? (int)(v >> kStatusShift) : 2) : 0;
    st = max(st, wave_max_i(sj));
    const uint64_t rb = __ballot(j < gam && !(v & kAccBit));
    if (n == gam && rb) n = j0 + __builtin_ctzll(rb);
  }
  uint32_t tn = 0;
  if (st == 0)
    tn = (uint32_t)__hip_atomic_load(P.rowslot + t0 + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
         kTokMask;
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    if (j <= gam) {
      int o = -1;
      if (st == 0) o = (j < n) ? P.tokens[d0 + j] : (j == n ? (int)tn : -1);
      P.out_tokens[t0 + j] = o;
    }
  }
  if (lane == 0) P.acc_len[b] = st == 2 ? -2 : st == 1 ? -1 : n;
}

// Row result of the workgroup that decides a row: publish, arrive, resolve.
__device__ __forceinline__ void finish_row(const Params& P, const Item& it, Shared& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.last = arrive(P, it.r, it.b, it.gam, (uint32_t)sh.payload) ? 1 : 0;
  __syncthreads();
  if (sh.last && tid < 64) resolve(P, it.b, it.d0 + it.b, it.d0, it.gam, tid);
}

// ------------------------------------------------------------------ greedy rows
// T = 0 (or an invalid temperature, which only needs the row to be reported):
// chunk argmax of target and draft; the last chunk decides.
template <int DT>
__device__ __forceinline__ void greedy_item(const Params& P, const Item& it, const float (&xt)[kPerThread],
                                            const float (&xd)[kPerThread], bool t_ok, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, C = P.C;
  const uint32_t tag = P.epoch;
  const bool pair = it.pair;
  const int64_t e0 = (int64_t)it.c * kChunk;
  uint64_t* x1row = P.xch1 + (int64_t)it.r * C * kX1;
  float vt, vd = -__builtin_huge_valf();
  int kt, kd = 0x7FFFFFFF, badt = 0, badd = 0;
  thread_argmax<DT>(xt, e0, tid, vt, kt, badt);
  if (pair) thread_argmax<DT>(xd, e0, tid, vd, kd, badd);
  badt = __syncthreads_or(badt);
  badd = __syncthreads_or(badd);
  block_argmax(vt, kt, sh);
  if (pair) block_argmax(vd, kd, sh);
  if (tid < kX1) {
    const uint32_t v = tid == 0 ? __float_as_uint(vt) : tid == 1 ? (badt ? 0xFFFFFFFFu : (uint32_t)kt)
                     : tid == 2 ? __float_as_uint(vd) : (badd ? 0xFFFFFFFFu : (uint32_t)kd);
    slot_put(x1row + (int64_t)it.c * kX1 + tid, tag, v);
  }
  if (it.c != C - 1) return;
  const bool ok = gather(x1row, kX1 * C, tag, P.spin_limit, sh.x1);
  if (tid < 64) {
    float av = -__builtin_huge_valf(), dv = -__builtin_huge_valf();
    int ak = 0x7FFFFFFF, dk = 0x7FFFFFFF, bad = 0;
    if (lane < C) {
      const uint32_t akk = sh.x1[lane * kX1 + 1], dkk = sh.x1[lane * kX1 + 3];
      av = __uint_as_float(sh.x1[lane * kX1 + 0]);
      dv = __uint_as_float(sh.x1[lane * kX1 + 2]);
      bad = (akk == 0xFFFFFFFFu) || (pair && dkk == 0xFFFFFFFFu);
      ak = (int)akk;
      dk = (int)dkk;
    }
    bad = __any(bad);
    wave_argmax(av, ak);
    wave_argmax(dv, dk);
    int status = !ok ? 2 : 0;
    if (status == 0 && (!t_ok || bad || av == -__builtin_huge_valf() ||
                        (pair && dv == -__builtin_huge_valf())))
      status = 1;
    const int x = it.xtok;
    if (pair && status == 0 && (x < 0 || x >= P.V)) status = 1;
    const bool acc = pair && (x == ak);
    if (lane == 0) {
      const int rd = it.d0 + it.i;
      if (pair && status == 0) {
        if (P.p_draft) P.p_draft[rd] = (x == ak) ? 1.0f : 0.0f;
        if (P.q_draft) P.q_draft[rd] = (x == dk) ? 1.0f : 0.0f;
        if (P.beta) P.beta[rd] = (ak == dk) ? 1.0f : 0.0f;
        if (P.resid) P.resid[rd] = (ak == dk) ? 0.0f : 1.0f;
      }
      sh.payload = (int)row_payload(status, acc, ak);
    }
  }
  __syncthreads();
  finish_row(P, it, sh);
}

// ------------------------------------------------------------------ sampled rows (T > 0)
template <int DT>
__device__ __forceinline__ void sampled_item(const Params& P, const Item& it, float (&xt)[kPerThread],
                                             float (&xd)[kPerThread], Shared& sh) {
  using F = Fmt<DT>;
  constexpr int EPV = F::EPV;
  constexpr int U = F::U;
  const int tid = threadIdx.x, lane = tid & 63, C = P.C;
  const uint32_t tag = P.epoch;
  const int spin = P.spin_limit;
  const bool pair = it.pair;
  const int rd = it.d0 + it.i;
  uint64_t* x1row = P.xch1 + (int64_t)it.r * C * kX1;
  uint64_t* x2row = P.xch2 + (int64_t)it.r * (C * kX2 + 2);
  const float s = kLog2e / it.T;
  const float ninf = -__builtin_huge_valf();
  const bool tok_ok = !pair || (it.xtok >= 0 && it.xtok < P.V);
  const int xchunk = (pair && tok_ok) ? it.xtok / kChunk : -1;

  // ---- phase 1: chunk max, exponentials kept in registers, chunk sum
  float mt = ninf, md = ninf;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) mt = fmaxf(mt, xt[k]);
  if (pair) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) md = fmaxf(md, xd[k]);
  }
  block_max2(mt, md, sh);
  const float ct = chunk_offset(mt, s);
  const float cd = chunk_offset(md, s);
  float st, sd = 0.0f;
  {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; k += 4) {
      xt[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[k], s, ct));
      xt[k + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[k + 1], s, ct));
      xt[k + 2] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[k + 2], s, ct));
      xt[k + 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[k + 3], s, ct));
      a0 += xt[k];
      a1 += xt[k + 1];
      a2 += xt[k + 2];
      a3 += xt[k + 3];
    }
    st = (a0 + a1) + (a2 + a3);
  }
  if (pair) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; k += 4) {
      xd[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[k], s, cd));
      xd[k + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[k + 1], s, cd));
      xd[k + 2] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[k + 2], s, cd));
      xd[k + 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[k + 3], s, cd));
      a0 += xd[k];
      a1 += xd[k + 1];
      a2 += xd[k + 2];
      a3 += xd[k + 3];
    }
    sd = (a0 + a1) + (a2 + a3);
  }
  block_sum2(st, sd, sh);
  if (tid < kX1) {
    const float v = tid == 0 ? mt : tid == 1 ? st : tid == 2 ? md : sd;
    slot_putf(x1row + (int64_t)it.c * kX1 + tid, tag, v);
  }

  // ---- exchange 1: the row's normalisers (M, S) of target and draft
  const bool ok = gather(x1row, kX1 * C, tag, spin, sh.x1);
  if (tid < 64) {
    const bool in = lane < C;
    const float m1 = in ? __uint_as_float(sh.x1[lane * kX1 + 0]) : ninf;
    const float s1 = in ? __uint_as_float(sh.x1[lane * kX1 + 1]) : 0.0f;
    const float m2 = in ? __uint_as_float(sh.x1[lane * kX1 + 2]) : ninf;
    const float s2 = in ? __uint_as_float(sh.x1[lane * kX1 + 3]) : 0.0f;
    const float Mt = wave_max(m1);
    const float Md = wave_max(m2);
    const float St = wave_sum(in ? s1 * __builtin_amdgcn_exp2f((m1 - Mt) * s) : 0.0f);
    const float Sd = wave_sum(in ? s2 * __builtin_amdgcn_exp2f((m2 - Md) * s) : 0.0f);
    if (lane == 0) {
      sh.Mt = Mt;
      sh.St = St;
      sh.Md = Md;
      sh.Sd = Sd;
    }
  }
  __syncthreads();
  const float Mt = sh.Mt, St = sh.St, Md = sh.Md, Sd = sh.Sd;
  const bool norm_ok = ok && Mt > ninf && St == St && St > 0.0f &&
                       (!pair || (Md > ninf && Sd == Sd && Sd > 0.0f));
  const float at = __builtin_amdgcn_exp2f((mt - Mt) * s) / St;   // p_k = at e_t
  const float ad = __builtin_amdgcn_exp2f((md - Md) * s) / Sd;   // q_k = ad e_d
  const float rho = ad / at;                                     // q_k = at rho e_d

  // ---- phase 2 (rows with a draft): sums of min(e_t, rho e_d) and max(0, e_t - rho e_d)
  bool ok2 = true;
  if (pair) {
    if (norm_ok) {
      float bsum = 0.0f, wsum = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float ws = 0.0f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float et = xt[u * EPV + e];
          const float qe = rho * xd[u * EPV + e];
          bsum += fminf(et, qe);
          ws += fmaxf(et - qe, 0.0f);
        }
        wsum += ws;
      }
      block_sum2(wsum, bsum, sh);
      if (tid < kX2) slot_putf(x2row + (int64_t)it.c * kX2 + tid, tag, tid == 0 ? at * wsum : at * bsum);
      if (it.c == xchunk) {   // the chunk holding the drafted token: p(x), q(x)
        const int loc = it.xtok - it.c * kChunk;
        const int u = loc / (kThreads * EPV);
        const int rem = loc - u * kThreads * EPV;
        if (tid == rem / EPV) {
          const int e = rem % EPV;
          float et = 0.0f, ed = 0.0f;
#pragma unroll
          for (int k = 0; k < kPerThread; ++k)
            if (k == u * EPV + e) {
              et = xt[k];
              ed = xd[k];
            }
          slot_putf(x2row + C * kX2 + 0, tag, et * at);
          slot_putf(x2row + C * kX2 + 1, tag, ed * ad);
        }
      }
    }
    // ---- exchange 2: residual mass, beta, p(x), q(x)
    const int n2 = norm_ok ? (tok_ok ? kX2 * C + 2 : kX2 * C) : 0;
    ok2 = gather(x2row, n2, tag, spin, sh.x2);
  }

  // ---- which chunk holds the sampled token
  // weights: the residual max(0, p - q) when it has mass, else p (bonus row,
  // or Z = 0 where the residual is undefined)
  if (tid < 64) {
    float Z = 0.0f, beta = 0.0f;
    if (pair && norm_ok && ok2) {
      Z = wave_sum(lane < C ? __uint_as_float(sh.x2[lane * kX2 + 0]) : 0.0f);
      beta = wave_sum(lane < C ? __uint_as_float(sh.x2[lane * kX2 + 1]) : 0.0f);
    }
    const bool resid_mode = pair && Z > 0.0f;
    float tot;
    if (resid_mode) {
      tot = lane < C ? __uint_as_float(sh.x2[lane * kX2 + 0]) : 0.0f;
    } else {
      const float m1 = lane < C ? __uint_as_float(sh.x1[lane * kX1 + 0]) : ninf;
      const float s1 = lane < C ? __uint_as_float(sh.x1[lane * kX1 + 1]) : 0.0f;
      tot = lane < C ? s1 * __builtin_amdgcn_exp2f((m1 - Mt) * s) / St : 0.0f;
    }
    const float mass = resid_mode ? Z : wave_sum(tot);
    const float thr = it.ug * mass;
    float before = 0.0f;
    const int own = (norm_ok && ok2) ? owner_select(tot, C, thr, lane, before) : -1;
    if (lane == 0) {
      sh.Z = Z;
      sh.beta = beta;
      sh.thr = thr;
      sh.before = before;
      sh.owner = own;
      sh.mode = resid_mode ? 1 : 0;
    }
  }
  __syncthreads();
  const int owner = sh.owner;
  const bool t_ok = it.T >= kFltMin && it.T <= kFltMax;
  int status = (!ok || !ok2) ? 2 : (!t_ok || !norm_ok || !tok_ok) ? 1 : (owner < 0 ? 2 : 0);
  // the owner chunk decides; a row already known bad is reported by its last chunk
  const bool decider = (status == 0) ? (it.c == owner) : (it.c == C - 1);
  if (!decider) return;
  int tok = 0;
  if (status == 0) {
    // weights in this chunk's own units (the sampled weight of token k is at * w_k)
    if (sh.mode) {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) xt[k] = fmaxf(xt[k] - rho * xd[k], 0.0f);
    }
    const float tau = (sh.thr - sh.before) / at;
    const int loc = chunk_search<DT>(xt, tau, sh);
    tok = it.c * kChunk + loc;
    if (loc < 0 || tok >= P.V) status = 2;   // unreachable: the owner chunk has weight > 0
  }
  if (tid == 0) {
    bool acc = false;
    if (pair && status == 0) {
      const float px = __uint_as_float(sh.x2[C * kX2 + 0]);
      const float qx = __uint_as_float(sh.x2[C * kX2 + 1]);
      acc = it.ui * qx < px;
      if (P.p_draft) P.p_draft[rd] = px;
      if (P.q_draft) P.q_draft[rd] = qx;
      if (P.beta) P.beta[rd] = sh.beta;
      if (P.resid) P.resid[rd] = sh.Z;
    }
    sh.payload = (int)row_payload(status, acc, tok);
  }
  __syncthreads();
  finish_row(P, it, sh);
}

// ------------------------------------------------------------------ the kernel
template <int DT>
__global__ __launch_bounds__(kThreads) void verify_kernel(Params P) {
  using F = Fmt<DT>;
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int grp = (int)(blockIdx.x % kGroups);
  if (grp >= P.R_t) return;
  const int n_items = ((P.R_t - grp + kGroups - 1) / kGroups) * P.C;
  int idx = (int)(blockIdx.x / kGroups);
  if (idx >= n_items) return;

  Item it;
  u32x4 rt[F::U], rdr[F::U];
  item_place(P, grp, idx, it);
  issue_chunk<DT>(P.target, it.r, P.tstride, (int64_t)it.c * kChunk, P.V, tid, P.t_aligned, rt);
  item_lookup(P, it);
  if (it.pair)
    issue_chunk<DT>(P.draft, it.d0 + it.i, P.dstride, (int64_t)it.c * kChunk, P.V, tid, P.d_aligned, rdr);
  while (true) {
    float xt[kPerThread], xd[kPerThread];
    unpack<DT>(rt, xt);
    if (it.pair) unpack<DT>(rdr, xd);
    // prefetch the next item while this one is processed
    const int nidx = idx + P.G;
    const bool more = nidx < n_items;
    Item nx = it;
    if (more) {
      item_place(P, grp, nidx, nx);
      issue_chunk<DT>(P.target, nx.r, P.tstride, (int64_t)nx.c * kChunk, P.V, tid, P.t_aligned, rt);
      item_lookup(P, nx);
      if (nx.pair)
        issue_chunk<DT>(P.draft, nx.d0 + nx.i, P.dstride, (int64_t)nx.c * kChunk, P.V, tid, P.d_aligned, rdr);
    }
    if (it.ok) {
      const bool t_ok = (it.T == 0.0f) || (it.T >= kFltMin && it.T <= kFltMax);
      __syncthreads();   // shared state of the previous item is no longer read
      if (t_ok && it.T > 0.0f)
        sampled_item<DT>(P, it, xt, xd, sh);
      else
        greedy_item<DT>(P, it, xt, xd, t_ok, sh);
    }
    if (!more) break;
    idx = nidx;
    it = nx;
  }
}

int chunks_for(int V) { return (V + kChunk - 1) / kChunk; }

}  // namespace

struct specverify_ctx {
  specverify_config cfg;
  int chunks;
  int64_t rows;            // max target rows
  int cap;                 // workgroups resident at once on the device
  uint64_t* ws;
  size_t ws_bytes;
  uint64_t* xch1;
  uint64_t* xch2;
  uint64_t* rowslot;
  uint64_t* seqctr;
  uint32_t epoch;
};

extern "C" {

specverify_status specverify_create(const specverify_config* cfg, specverify_handle* out) {
  if (out) *out = nullptr;
  if (!cfg || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (cfg->max_batch < 1 || cfg->max_gamma < 0 || cfg->vocab < 1 || cfg->spin_limit < 0 ||
      (cfg->dtype != SPECVERIFY_F32 && cfg->dtype != SPECVERIFY_BF16))
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)cfg->max_batch * ((int64_t)cfg->max_gamma + 1);
  if (rows > (int64_t)1 << 24) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (chunks_for(cfg->vocab) > kMaxChunks) return SPECVERIFY_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev)
    return SPECVERIFY_ERR_DEVICE;
  specverify_ctx* h = new (std::nothrow) specverify_ctx();
  if (!h) return SPECVERIFY_ERR_OUT_OF_MEMORY;
  h->cfg = *cfg;
  if (h->cfg.spin_limit == 0) h->cfg.spin_limit = kDefaultSpin;
  h->chunks = chunks_for(cfg->vocab);
  h->rows = rows;
  const size_t n1 = (size_t)rows * h->chunks * kX1;
  const size_t n2 = (size_t)rows * (h->chunks * kX2 + 2);
  const size_t n3 = (size_t)rows;
  const size_t n4 = (size_t)cfg->max_batch;
  h->ws_bytes = (n1 + n2 + n3 + n4) * sizeof(uint64_t);
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(cfg->device) != hipSuccess) {
    delete h;
    return SPECVERIFY_ERR_DEVICE;
  }
  // residency of the persistent grid: workgroups per CU times CUs
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cfg->device);
  if (e == hipSuccess)
    e = cfg->dtype == SPECVERIFY_F32
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<SPECVERIFY_F32>, kThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<SPECVERIFY_BF16>, kThreads, 0);
  h->cap = (e == hipSuccess) ? cus * per_cu : 0;
  void* p = nullptr;
  if (e == hipSuccess && h->cap < kGroups) e = hipErrorInvalidConfiguration;
  if (e == hipSuccess) e = hipMalloc(&p, h->ws_bytes);
  if (e == hipSuccess) e = hipMemset(p, 0, h->ws_bytes);   // tag 0 is never an epoch
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    if (p) (void)hipFree(p);
    delete h;
    return e == hipErrorOutOfMemory ? SPECVERIFY_ERR_OUT_OF_MEMORY : SPECVERIFY_ERR_DEVICE;
  }
  h->ws = (uint64_t*)p;
  h->xch1 = h->ws;
  h->xch2 = h->xch1 + n1;
  h->rowslot = h->xch2 + n2;
  h->seqctr = h->rowslot + n3;
  h->epoch = 0;
  *out = h;
  return SPECVERIFY_OK;
}

specverify_status specverify_run(specverify_handle h, const specverify_inputs* in,
                                 const specverify_outputs* out, void* hip_stream) {
  if (!h || !in || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int B = in->batch;
  if (B < 0 || B > h->cfg.max_batch) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (B == 0) return SPECVERIFY_OK;
  int64_t R_d;
  if (in->cu_draft == nullptr) {
    if (in->gamma < 0 || in->gamma > h->cfg.max_gamma) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = (int64_t)B * in->gamma;
  } else {
    if (in->num_draft_rows < 0) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = in->num_draft_rows;
  }
  const int64_t R_t = R_d + B;
  if (R_t > h->rows) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int V = h->cfg.vocab;
  if (!in->target_logits || !in->uniforms || !in->temperatures || !out->accepted_len ||
      !out->out_tokens)
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (R_d > 0 && (!in->draft_logits || !in->draft_tokens)) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (in->target_stride < V || (R_d > 0 && in->draft_stride < V)) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int esize = h->cfg.dtype == SPECVERIFY_F32 ? 4 : 2;
  if (((uintptr_t)in->target_logits % esize) || (R_d > 0 && ((uintptr_t)in->draft_logits % esize)))
    return SPECVERIFY_ERR_UNSUPPORTED;   // logits must be element aligned
  // Rows that do not start on 16-byte boundaries are read element by element.
  const bool t_aligned = !((uintptr_t)in->target_logits & 15) && !((in->target_stride * esize) & 15);
  const bool d_aligned = R_d > 0 && !((uintptr_t)in->draft_logits & 15) && !((in->draft_stride * esize) & 15);

  // Persistent grid: per row group, as many workgroups as the device holds
  // (a whole number of rows' worth when it holds that many), never more
  // than the group has items.
  const int C = h->chunks;
  const int64_t rows_g = (R_t + kGroups - 1) / kGroups;
  int64_t G = h->cap / kGroups;
  if (G >= C) G = (G / C) * C;
  if (G > rows_g * C) G = rows_g * C;
  if (G < 1) G = 1;

  if (++h->epoch == 0) h->epoch = 1;   // 0 never tags a slot (workspace is zeroed)
  Params P;
  P.target = in->target_logits;
  P.draft = in->draft_logits;
  P.tstride = in->target_stride;
  P.dstride = in->draft_stride;
  P.tokens = in->draft_tokens;
  P.uniforms = in->uniforms;
  P.temps = in->temperatures;
  P.cu_draft = in->cu_draft;
  P.gamma = in->gamma;
  P.B = B;
  P.R_d = (int32_t)R_d;
  P.R_t = (int32_t)R_t;
  P.V = V;
  P.C = C;
  P.G = (int32_t)G;
  P.epoch = h->epoch;
  P.spin_limit = h->cfg.spin_limit;
  P.t_aligned = t_aligned;
  P.d_aligned = d_aligned;
  P.xch1 = h->xch1;
  P.xch2 = h->xch2;
  P.rowslot = h->rowslot;
  P.seqctr = h->seqctr;
  P.acc_len = out->accepted_len;
  P.out_tokens = out->out_tokens;
  P.p_draft = out->p_draft;
  P.q_draft = out->q_draft;
  P.beta = out->beta;
  P.resid = out->resid_mass;

  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  hipStream_t stream = (hipStream_t)hip_stream;
  const dim3 grid((uint32_t)(G * kGroups));
  if (h->cfg.dtype == SPECVERIFY_F32)
    hipLaunchKernelGGL(verify_kernel<SPECVERIFY_F32>, grid, dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(verify_kernel<SPECVERIFY_BF16>, grid, dim3(kThreads), 0, stream, P);
  const hipError_t e = hipGetLastError();
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_destroy(specverify_handle h) {
  if (!h) return SPECVERIFY_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->cfg.device);
  (void)hipFree(h->ws);
  (void)hipSetDevice(prev);
  delete h;
  return SPECVERIFY_OK;
}

int32_t specverify_chunks_per_row(specverify_handle h) { return h ? h->chunks : 0; }
int64_t specverify_workspace_bytes(specverify_handle h) { return h ? (int64_t)h->ws_bytes : 0; }

}  // extern "C"
