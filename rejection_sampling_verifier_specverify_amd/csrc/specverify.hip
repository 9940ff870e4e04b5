// HIP kernels and C ABI of the speculative-decoding verification sampler,
// written for AMD CDNA4 (gfx950, MI355X).
//
// What is computed (velog "6-1편. Speculative Decoding", section 2
// "알고리즘 4단계" steps 2-4 with section 2-1, the min(1, p/q) rule, and
// section 2-2, the residual norm(max(0, p - q)); greedy rule of "How to
// Scale Your Model -- All About Transformer Inference", Appendix D): see
// include/specverify.h.
//
// How.  The logits are read from HBM exactly once.  Every target row is
// split into chunks of 8192 logits; one 256-thread workgroup owns one chunk
// of one target row and, when the row has a draft, the same chunk of the
// draft row, so p_k and q_k of the same token meet in the same registers.
// Workgroup (row r, chunk c) is blockIdx r * C + c.
//
//   phase 1   16-byte coalesced loads -> fp32 registers; chunk max m_c; the
//             exponentials e_k = 2^(l_k * s - m_c * s), s = log2(e) / T,
//             kept in registers; chunk sum s_c.  T = 0: chunk argmax.
//   xch 1     (m_c, s_c) of target and draft are published in epoch-tagged
//             64-bit slots; the chunks of a row that need the row's
//             normalisers poll the row's slots until every tag carries this
//             run's epoch.  The merge (max, sum * 2^((m_c - M) s)) is the
//             associative combine of an online softmax.
//   phase 2   p_k = e_k * 2^((m_c - M_t) s) / S_t, q_k likewise; the chunk
//             sums of min(p, q) (beta, velog section 2-3 item 1) and of
//             w_k = max(0, p_k - q_k) (the residual mass, section 2-3 item 2),
//             plus the sums of w over 32-lane sub-chunks, are published.
//   finish    the last chunk of each row: residual mass Z, beta; inverse CDF
//             of u_gamma * Z over chunk totals -> sub-chunk totals -> the
//             256 or 128 logits of one sub-chunk, re-read and scanned; the
//             acceptance test u_i * q(x) < p(x); diagnostics; the row
//             result in a tagged slot; an arrival on the sequence counter.
//   resolve   the last row of a sequence to arrive finds the first rejection
//             n and writes accepted_len and the n + 1 tokens; no host sync.
//
// Synchronisation uses no fences: every value crossing workgroups travels in
// its own 64-bit slot together with a 32-bit epoch tag, written and read
// with agent-scope atomics, so a reader that sees the tag sees the value.
// Every wait is bounded by a poll budget; an expired wait is reported as
// accepted_len = -2 and the kernel still ends.  Waits only target chunks of
// the same row (consecutive blockIdx), which the in-order dispatch of each
// XCD brings up together.
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
constexpr int kHalf = 32;                      // lanes per sub-chunk
constexpr int kX1 = 4;                         // exchange-1 slots per chunk
constexpr int kX2Head = 2;                     // exchange-2: W_c, B_c, then sub-totals
constexpr int kMaxSub = 64;                    // sub-chunks per chunk (f32: 64, bf16: 32)
constexpr int kDefaultSpin = 1 << 18;   // ~0.3 s of polling; normal waits are microseconds
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMin = 1.17549435e-38f;
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
  int32_t V;
  int32_t C;                 // chunks per row
  uint32_t epoch;
  int32_t spin_limit;
  bool t_aligned;            // target rows start on 16-byte boundaries
  bool d_aligned;
  uint64_t* xch1;            // [rows][C][kX1]
  uint64_t* xch2;            // [rows][C][kX2Head + NSUB]
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

// Poll one slot until it carries `tag`; false once `limit` polls have failed.
__device__ __forceinline__ bool slot_get(uint64_t* p, uint32_t tag, int limit, uint32_t& v) {
  for (int k = 0;; ++k) {
    const uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) {
      v = (uint32_t)w;
      return true;
    }
    if (k >= limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// ------------------------------------------------------------------ reductions
// Butterflies leave the same value in every lane (addition and max are
// commutative), so every workgroup that reduces the same data gets the same
// bits.

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float half_sum(float v) {  // within each 32-lane half
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
// Inclusive prefix sum over the 64 lanes of a wave, fixed association.
__device__ __forceinline__ float wave_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}
// (value, index): larger value wins, lower index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& k, float v2, int k2) {
  if (v2 > v || (v2 == v && k2 < k)) {
    v = v2;
    k = k2;
  }
}
__device__ __forceinline__ void wave_argmax(float& v, int& k) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float v2 = __shfl_xor(v, m);
    const int k2 = __shfl_xor(k, m);
    argmax_merge(v, k, v2, k2);
  }
}
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// ------------------------------------------------------------------ loads

// Load this thread's 32 logits of a chunk as fp32.  Element x[u*EPV + e] is
// token e0 + u*256*EPV + tid*EPV + e; tokens >= V read as -inf.
template <int DT>
__device__ __forceinline__ void load_chunk(const void* base, int64_t row, int64_t stride,
                                           int64_t e0, int V, int tid, bool aligned,
                                           float (&x)[kPerThread]) {
  using F = Fmt<DT>;
  const char* rowp = (const char*)base + row * stride * F::ESIZE;
  u32x4 raw[F::U];
  if (aligned && e0 + kChunk <= V) {
#pragma unroll
    for (int u = 0; u < F::U; ++u) {
      const int64_t k = e0 + (int64_t)u * kThreads * F::EPV + (int64_t)tid * F::EPV;
      raw[u] = __builtin_nontemporal_load((const u32x4*)(rowp + k * F::ESIZE));
    }
  } else {
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

template <int DT>
__device__ __forceinline__ float load_one(const void* base, int64_t row, int64_t stride, int64_t k) {
  if (DT == SPECVERIFY_F32) return ((const float*)base)[row * stride + k];
  const uint16_t b = ((const uint16_t*)base)[row * stride + k];
  return __uint_as_float((uint32_t)b << 16);
}

// Residual weight max(0, p - q) of one logit from its exponentials and the
// chunk scales; phase 2 and the finisher's re-scan both use this, so that
// (built without fp contraction) they produce the same bits.
__device__ __forceinline__ float resid_weight(float et, float at, float ed, float ad) {
  const float p = et * at;
  const float q = ed * ad;
  return fmaxf(p - q, 0.0f);
}

// Exponent offset of a chunk: -m * s, or 0 for a chunk of only -inf (so that
// its exponentials are 2^-inf = 0 instead of NaN).
__device__ __forceinline__ float chunk_offset(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : -m * s;
}

struct Shared {
  float red[2 * kWaves];
  int redi[2 * kWaves];
  uint32_t x1[kX1 * kMaxChunks];     // exchange-1 payloads of the row
  float tot[kMaxChunks];             // chunk weight totals (W_c or P_c)
  float btot[kMaxChunks];            // chunk sums of min(p, q)
  float sub[kMaxSub];                // sub-chunk weight totals of the owner chunk
  float Mt, St, Md, Sd;              // row normalisers
  float scal[8];
  int flag;
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

// Per-thread argmax of a chunk in token order (first maximum wins) plus a
// flag for NaN / +inf.
template <int DT>
__device__ __forceinline__ void thread_argmax(const float (&x)[kPerThread], int64_t e0, int tid,
                                              float& bv, int& bk, int& bad) {
  using F = Fmt<DT>;
  bv = -__builtin_huge_valf();
  bk = 0x7FFFFFFF;
#pragma unroll
  for (int u = 0; u < F::U; ++u) {
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const float v = x[u * F::EPV + e];
      bad |= (v != v) | (v == __builtin_huge_valf());
      if (v > bv) {
        bv = v;
        bk = (int)(e0 + (int64_t)u * kThreads * F::EPV + (int64_t)tid * F::EPV + e);
      }
    }
  }
}

// Inverse CDF inside one sub-chunk (wave 0 only; lanes 0..31 own EPV logits
// each).  w: this lane's weights; base: CDF value before the sub-chunk; thr:
// u * Z.  Returns the sub-chunk-local index of the first logit with w > 0 and
// base + C_k > thr, else of the last logit with w > 0 (rounding guard).
template <int EPV>
__device__ __forceinline__ int subchunk_search(const float (&w)[EPV], float base, float thr, int lane) {
  float loc[EPV];
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    run += w[e];
    loc[e] = run;
  }
  const float lane_tot = lane < kHalf ? run : 0.0f;
  const float incl = wave_scan(lane_tot, lane);
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.0f;
  int first = 0x7FFFFFFF, lastpos = -1;
  if (lane < kHalf) {
#pragma unroll
    for (int e = EPV - 1; e >= 0; --e) {
      const float Ck = base + (excl + loc[e]);
      if (w[e] > 0.0f && Ck > thr) first = lane * EPV + e;
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      if (w[e] > 0.0f) lastpos = lane * EPV + e;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    first = min(first, __shfl_xor(first, m));
    lastpos = max(lastpos, __shfl_xor(lastpos, m));
  }
  return first != 0x7FFFFFFF ? first : lastpos;
}

// Owner selection over n <= 64 non-negative totals held one per lane (wave 0):
// first j with tot_j > 0 and base + incl_j > thr, else the last j with
// tot_j > 0.  Returns j (or -1 if every total is 0) and the CDF value before j.
__device__ __forceinline__ int owner_select(float tot, int n, float base, float thr, int lane,
                                            float& before) {
  const float t = lane < n ? tot : 0.0f;
  const float incl = wave_scan(t, lane);
  const float G = base + incl;
  const uint64_t hit = wave_ballot(lane < n && t > 0.0f && G > thr);
  const uint64_t pos = wave_ballot(lane < n && t > 0.0f);
  int j;
  if (hit) j = __builtin_ctzll(hit);
  else if (pos) j = 63 - __builtin_clzll(pos);
  else j = -1;
  const float prev = __shfl(G, j > 0 ? j - 1 : 0);
  before = j > 0 ? prev : base;
  return j;
}

// Publish the row result and count the row in on its sequence (thread 0).
// Returns true for the last of the sequence's gamma + 1 rows to arrive.  The
// counter word holds (epoch, count); a stale epoch counts as zero, so a run
// never depends on what earlier runs left behind.
__device__ __forceinline__ bool arrive(const Params& P, int r, int b, int gam, uint32_t tag,
                                       uint32_t payload) {
  slot_put(P.rowslot + r, tag, payload);
  uint64_t* ctr = P.seqctr + b;
  uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t cnt = 0;
  for (int k = 0; k < (1 << 20); ++k) {
    cnt = ((uint32_t)(old >> 32) == tag) ? (uint32_t)old + 1u : 1u;
    const uint64_t nw = ((uint64_t)tag << 32) | cnt;
    if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  return cnt == (uint32_t)gam + 1u;
}

// The last row of sequence b to finish: first rejection n, accepted length
// and the n + 1 emitted tokens (wave 0).
__device__ __forceinline__ void resolve(const Params& P, int b, int t0, int d0, int gam, uint32_t tag,
                                        int lane) {
  int n = gam, st = 0;
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    uint32_t v = 0;
    int okj = 1;
    if (j <= gam) okj = slot_get(P.rowslot + t0 + j, tag, P.spin_limit, v);
    int sj = (j <= gam) ? (okj ? (int)(v >> kStatusShift) : 2) : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sj = max(sj, __shfl_xor(sj, m));
    st = max(st, sj);
    const uint64_t rb = wave_ballot(j < gam && !(v & kAccBit));
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

__device__ __forceinline__ uint32_t row_payload(int status, bool acc, int tok) {
  return ((uint32_t)status << kStatusShift) | (acc ? kAccBit : 0u) |
         (status == 0 ? ((uint32_t)tok & kTokMask) : 0u);
}

// Gather the exchange-1 slots of row r into sh.x1 (every thread calls).
__device__ __forceinline__ bool gather_x1(uint64_t* x1row, int C, uint32_t tag, int spin, Shared& sh) {
  int ok = 1;
  const int tid = threadIdx.x;
  if (tid < kX1 * C) {
    uint32_t v = 0;
    ok = slot_get(x1row + tid, tag, spin, v);
    sh.x1[tid] = v;
  }
  return __syncthreads_and(ok) != 0;
}

// ---------------------------------------------------------------- greedy rows
// T = 0 (or an invalid temperature, which only needs the row to be reported):
// chunk argmax of target and draft, and the finisher's greedy decision.
template <int DT>
__device__ __forceinline__ void greedy_row(const Params& P, const float (&xt)[kPerThread], const float (&xd)[kPerThread],
                           int r, int c, int b, int t0, int d0, int gam, int rd, bool pair, bool t_ok,
                           Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, C = P.C;
  const uint32_t tag = P.epoch;
  const int64_t e0 = (int64_t)c * kChunk;
  uint64_t* x1row = P.xch1 + (int64_t)r * C * kX1;
  float vt, vd = -__builtin_huge_valf();
  int kt, kd = 0x7FFFFFFF, badt = 0, badd = 0;
  thread_argmax<DT>(xt, e0, tid, vt, kt, badt);
  if (pair) thread_argmax<DT>(xd, e0, tid, vd, kd, badd);
  badt = __syncthreads_or(badt);
  badd = __syncthreads_or(badd);
  block_argmax(vt, kt, sh);
  if (pair) block_argmax(vd, kd, sh);
  if (tid == 0) {
    uint64_t* s = x1row + (int64_t)c * kX1;
    slot_put(s + 0, tag, __float_as_uint(vt));
    slot_put(s + 1, tag, badt ? 0xFFFFFFFFu : (uint32_t)kt);
    slot_put(s + 2, tag, __float_as_uint(vd));
    slot_put(s + 3, tag, badd ? 0xFFFFFFFFu : (uint32_t)kd);
  }
  if (c != C - 1) return;
  const bool ok = gather_x1(x1row, C, tag, P.spin_limit, sh);
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
    bool acc = false;
    int x = 0;
    if (pair) {
      x = P.tokens[rd];
      if (status == 0 && (x < 0 || x >= P.V)) status = 1;
      acc = (x == ak);
    }
    if (lane == 0) {
      if (pair && status == 0) {
        if (P.p_draft) P.p_draft[rd] = (x == ak) ? 1.0f : 0.0f;
        if (P.q_draft) P.q_draft[rd] = (x == dk) ? 1.0f : 0.0f;
        if (P.beta) P.beta[rd] = (ak == dk) ? 1.0f : 0.0f;
        if (P.resid) P.resid[rd] = (ak == dk) ? 0.0f : 1.0f;
      }
      sh.last = arrive(P, r, b, gam, tag, row_payload(status, acc, ak)) ? 1 : 0;
    }
  }
  __syncthreads();
  if (sh.last && tid < 64) resolve(P, b, t0, d0, gam, tag, lane);
}

// ---------------------------------------------------------------- sampled rows
template <int DT>
__device__ __forceinline__ void sampled_row(const Params& P, float (&xt)[kPerThread], float (&xd)[kPerThread], int r,
                            int c, int b, int t0, int d0, int gam, int rd, bool pair, float T,
                            Shared& sh) {
  using F = Fmt<DT>;
  constexpr int EPV = F::EPV;
  constexpr int U = F::U;
  constexpr int NSUB = (kThreads / kHalf) * U;
  constexpr int SLOTS2 = kX2Head + NSUB;
  const int tid = threadIdx.x, lane = tid & 63, C = P.C;
  const uint32_t tag = P.epoch;
  const int spin = P.spin_limit;
  const bool finisher = (c == C - 1);
  uint64_t* x1row = P.xch1 + (int64_t)r * C * kX1;
  const float s = kLog2e / T;

  // ---- phase 1: chunk max, exponentials kept in registers, chunk sum
  float mt = -__builtin_huge_valf(), md = -__builtin_huge_valf();
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
  if (tid == 0) {
    uint64_t* sl = x1row + (int64_t)c * kX1;
    slot_put(sl + 0, tag, __float_as_uint(mt));
    slot_put(sl + 1, tag, __float_as_uint(st));
    slot_put(sl + 2, tag, __float_as_uint(md));
    slot_put(sl + 3, tag, __float_as_uint(sd));
  }
  if (!pair && !finisher) return;   // the other chunks of a bonus row are done

  // ---- exchange 1: the row's normalisers (M, S) of target and draft
  const bool ok = gather_x1(x1row, C, tag, spin, sh);
  if (!ok && !finisher) return;     // the finisher will time out and report
  if (tid < 64) {
    const bool in = lane < C;
    const float m1 = in ? __uint_as_float(sh.x1[lane * kX1 + 0]) : -__builtin_huge_valf();
    const float s1 = in ? __uint_as_float(sh.x1[lane * kX1 + 1]) : 0.0f;
    const float m2 = in ? __uint_as_float(sh.x1[lane * kX1 + 2]) : -__builtin_huge_valf();
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
  const float ninf = -__builtin_huge_valf();
  const bool norm_ok = ok && Mt > ninf && St == St && St > 0.0f &&
                       (!pair || (Md > ninf && Sd == Sd && Sd > 0.0f));

  // ---- phase 2: beta and residual mass of this chunk, plus sub-chunk sums
  if (pair && ok) {
    const float at = __builtin_amdgcn_exp2f((mt - Mt) * s) / St;
    const float ad = __builtin_amdgcn_exp2f((md - Md) * s) / Sd;
    float bsum = 0.0f, wtot = 0.0f;
    float wsub[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float ws = 0.0f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float p = xt[u * EPV + e] * at;
        const float q = xd[u * EPV + e] * ad;
        bsum += fminf(p, q);
        ws += resid_weight(xt[u * EPV + e], at, xd[u * EPV + e], ad);
      }
      wsub[u] = ws;
      wtot += ws;
    }
    block_sum2(wtot, bsum, sh);
    uint64_t* x2 = P.xch2 + ((int64_t)r * C + c) * SLOTS2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sub = half_sum(wsub[u]);
      if ((tid & (kHalf - 1)) == 0)
        slot_put(x2 + kX2Head + u * (kThreads / kHalf) + tid / kHalf, tag, __float_as_uint(sub));
    }
    if (tid == 0) {
      slot_put(x2 + 0, tag, __float_as_uint(wtot));
      slot_put(x2 + 1, tag, __float_as_uint(bsum));
    }
  }
  if (!finisher) return;

  // ---------------- finisher: residual mass, beta, inverse CDF, acceptance
  int status = ok ? 0 : 2;
  const int xtok = pair ? P.tokens[rd] : 0;
  float Z = 0.0f, beta = 0.0f;
  if (pair && status == 0) {
    int ok2 = 1;
    if (tid < 2 * C) {
      uint32_t v = 0;
      const int cc = tid >> 1;
      ok2 = slot_get(P.xch2 + ((int64_t)r * C + cc) * SLOTS2 + (tid & 1), tag, spin, v);
      if (tid & 1) sh.btot[cc] = __uint_as_float(v);
      else sh.tot[cc] = __uint_as_float(v);
    }
    ok2 = __syncthreads_and(ok2);
    if (tid < 64) {
      const float wz = wave_sum(lane < C ? sh.tot[lane] : 0.0f);
      const float bz = wave_sum(lane < C ? sh.btot[lane] : 0.0f);
      if (lane == 0) {
        sh.scal[0] = wz;
        sh.scal[1] = bz;
      }
    }
    __syncthreads();
    Z = sh.scal[0];
    beta = sh.scal[1];
    if (!ok2) status = 2;
  }
  const bool t_ok = T >= kFltMin && T <= 3.40282347e38f;
  if (status == 0 && (!t_ok || !norm_ok || (pair && (xtok < 0 || xtok >= P.V)))) status = 1;
  // sampled weights: the residual max(0, p - q) if it has mass, else p
  // (the bonus row, or Z = 0 where the residual is undefined)
  const bool resid_mode = pair && Z > 0.0f;
  int tok = 0;
  if (status == 0) {
    const float ug = P.uniforms[t0 + gam];
    if (!resid_mode) {
      if (tid < 64) {   // chunk totals of p: s_c 2^((m_c - M) s) / S
        const bool in = lane < C;
        const float m1 = in ? __uint_as_float(sh.x1[lane * kX1 + 0]) : ninf;
        const float s1 = in ? __uint_as_float(sh.x1[lane * kX1 + 1]) : 0.0f;
        const float pc = in ? s1 * __builtin_amdgcn_exp2f((m1 - Mt) * s) / St : 0.0f;
        if (in) sh.tot[lane] = pc;
        const float tz = wave_sum(pc);
        if (lane == 0) sh.scal[2] = tz;
      }
      __syncthreads();
    }
    const float thr = ug * (resid_mode ? Z : sh.scal[2]);
    if (tid < 64) {   // owner chunk
      float before;
      const int cs = owner_select(lane < C ? sh.tot[lane] : 0.0f, C, 0.0f, thr, lane, before);
      if (lane == 0) {
        sh.scal[3] = before;
        sh.flag = cs;
      }
    }
    __syncthreads();
    const int cs = sh.flag;
    const float Pc = sh.scal[3];
    if (cs < 0 || cs >= C) {
      status = 2;   // unreachable for a valid row: the row maximum has weight > 0
    } else {
      const float mtc = __uint_as_float(sh.x1[cs * kX1 + 0]);
      const float mdc = __uint_as_float(sh.x1[cs * kX1 + 2]);
      const float atc = __builtin_amdgcn_exp2f((mtc - Mt) * s) / St;
      const float adc = resid_mode ? __builtin_amdgcn_exp2f((mdc - Md) * s) / Sd : 0.0f;
      const float ctc = chunk_offset(mtc, s);
      const float cdc = chunk_offset(mdc, s);
      const int64_t ce0 = (int64_t)cs * kChunk;
      int ok3 = 1;
      if (resid_mode) {   // published sub-chunk sums of the owner chunk
        if (tid < NSUB) {
          uint32_t v = 0;
          ok3 = slot_get(P.xch2 + ((int64_t)r * C + cs) * SLOTS2 + kX2Head + tid, tag, spin, v);
          sh.sub[tid] = __uint_as_float(v);
        }
        ok3 = __syncthreads_and(ok3);
      } else {            // p weights: re-read the owner chunk, sum per sub-chunk
        float xo[kPerThread];
        load_chunk<DT>(P.target, r, P.tstride, ce0, P.V, tid, P.t_aligned, xo);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float ws = 0.0f;
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            ws += __builtin_amdgcn_exp2f(__builtin_fmaf(xo[u * EPV + e], s, ctc)) * atc;
          const float sub = half_sum(ws);
          if ((tid & (kHalf - 1)) == 0) sh.sub[u * (kThreads / kHalf) + tid / kHalf] = sub;
        }
        __syncthreads();
      }
      if (!ok3) {
        status = 2;
      } else {
        if (tid < 64) {
          float before;
          const int ss = owner_select(lane < NSUB ? sh.sub[lane] : 0.0f, NSUB, Pc, thr, lane, before);
          int found = -1;
          if (ss >= 0) {
            const int su = ss / (kThreads / kHalf);
            const int sg = ss % (kThreads / kHalf);
            const int64_t kb = ce0 + (int64_t)su * kThreads * EPV + (int64_t)sg * kHalf * EPV;
            const int64_t k0 = kb + (int64_t)lane * EPV;
            float w[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              float wv = 0.0f;
              if (lane < kHalf && k0 + e < P.V) {
                const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(
                    load_one<DT>(P.target, r, P.tstride, k0 + e), s, ctc));
                if (resid_mode) {
                  const float ed = __builtin_amdgcn_exp2f(__builtin_fmaf(
                      load_one<DT>(P.draft, rd, P.dstride, k0 + e), s, cdc));
                  wv = resid_weight(et, atc, ed, adc);
                } else {
                  wv = et * atc;
                }
              }
              w[e] = wv;
            }
            const int loc = subchunk_search<EPV>(w, before, thr, lane);
            if (loc >= 0) found = (int)(kb + loc);
          }
          if (lane == 0) sh.flag = found;
        }
        __syncthreads();
        tok = sh.flag;
        if (tok < 0 || tok >= P.V) status = 2;
      }
    }
  }
  if (tid == 0) {
    bool acc = false;
    if (pair && status == 0) {
      const float lt = load_one<DT>(P.target, r, P.tstride, xtok);
      const float ld = load_one<DT>(P.draft, rd, P.dstride, xtok);
      const float px = __builtin_amdgcn_exp2f(__builtin_fmaf(lt, s, -Mt * s)) / St;
      const float qx = __builtin_amdgcn_exp2f(__builtin_fmaf(ld, s, -Md * s)) / Sd;
      acc = P.uniforms[r] * qx < px;
      if (P.p_draft) P.p_draft[rd] = px;
      if (P.q_draft) P.q_draft[rd] = qx;
      if (P.beta) P.beta[rd] = beta;
      if (P.resid) P.resid[rd] = Z;
    }
    sh.last = arrive(P, r, b, gam, tag, row_payload(status, acc, tok)) ? 1 : 0;
  }
  __syncthreads();
  if (sh.last && tid < 64) resolve(P, b, t0, d0, gam, tag, lane);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void verify_kernel(Params P) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int C = P.C;
  const int r = (int)(blockIdx.x / (uint32_t)C);   // target row
  const int c = (int)(blockIdx.x - (uint32_t)r * (uint32_t)C);

  // ---- target row -> (sequence b, position i)
  int b, gam, d0;
  if (P.cu_draft == nullptr) {
    b = r / (P.gamma + 1);
    gam = P.gamma;
    d0 = b * P.gamma;
  } else {
    int lo = 0, hi = P.B - 1;
    while (lo < hi) {   // largest b with cu_t[b] = cu_draft[b] + b <= r
      const int mid = (lo + hi + 1) >> 1;
      if (P.cu_draft[mid] + mid <= r) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    d0 = P.cu_draft[b];
    gam = P.cu_draft[b + 1] - d0;
  }
  const int t0 = d0 + b;   // cu_t[b]
  const int i = r - t0;
  if (gam < 0 || d0 < 0 || d0 + gam > P.R_d || i < 0 || i > gam) return;   // inconsistent cu_draft
  const bool pair = i < gam;
  const int rd = d0 + i;
  const float T = P.temps[b];
  const bool t_ok = (T == 0.0f) || (T >= kFltMin && T <= 3.40282347e38f);

  float xt[kPerThread], xd[kPerThread];
  const int64_t e0 = (int64_t)c * kChunk;
  load_chunk<DT>(P.target, r, P.tstride, e0, P.V, tid, P.t_aligned, xt);
  if (pair) load_chunk<DT>(P.draft, rd, P.dstride, e0, P.V, tid, P.d_aligned, xd);
  if (t_ok && T > 0.0f)
    sampled_row<DT>(P, xt, xd, r, c, b, t0, d0, gam, rd, pair, T, sh);
  else
    greedy_row<DT>(P, xt, xd, r, c, b, t0, d0, gam, rd, pair, t_ok, sh);
}

int chunks_for(int V) { return (V + kChunk - 1) / kChunk; }
int nsub_for(int dtype) { return (kThreads / kHalf) * (dtype == SPECVERIFY_F32 ? Fmt<SPECVERIFY_F32>::U : Fmt<SPECVERIFY_BF16>::U); }

}  // namespace

struct specverify_ctx {
  specverify_config cfg;
  int chunks;
  int nsub;
  int64_t rows;            // max target rows
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
  h->nsub = nsub_for(cfg->dtype);
  h->rows = rows;
  const size_t n1 = (size_t)rows * h->chunks * kX1;
  const size_t n2 = (size_t)rows * h->chunks * (kX2Head + h->nsub);
  const size_t n3 = (size_t)rows;
  const size_t n4 = (size_t)cfg->max_batch;
  h->ws_bytes = (n1 + n2 + n3 + n4) * sizeof(uint64_t);
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(cfg->device) != hipSuccess) {
    delete h;
    return SPECVERIFY_ERR_DEVICE;
  }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, h->ws_bytes);
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
  const int64_t blocks = R_t * h->chunks;
  if (blocks > 0x7FFFFFFF) return SPECVERIFY_ERR_INVALID_ARGUMENT;

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
  P.V = V;
  P.C = h->chunks;
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
  if (h->cfg.dtype == SPECVERIFY_F32)
    hipLaunchKernelGGL(verify_kernel<SPECVERIFY_F32>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(verify_kernel<SPECVERIFY_BF16>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, P);
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
