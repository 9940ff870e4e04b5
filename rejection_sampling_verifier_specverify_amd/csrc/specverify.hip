// HIP kernels and C ABI of the speculative-decoding verification sampler,
// written for AMD CDNA4 (gfx950, MI355X).
//
// What is computed (velog "6-1편. Speculative Decoding", section 2
// "알고리즘 4단계" steps 2-4 with section 2-1, the min(1, p/q) rule, and
// section 2-2, the residual norm(max(0, p - q)); greedy rule of "How to
// Scale Your Model -- All About Transformer Inference", Appendix D): see
// include/specverify.h.
//
// Two kernels run back to back on the caller's stream.
//
// stream_kernel reads every logit from HBM exactly once.  Target rows are
// split into chunks of 8192 logits; a work item is one chunk of one target
// row plus, when the position has a draft, the same chunk of the draft row,
// so p_k and q_k of the same token meet in the same registers.  The kernel
// is persistent: as many 256-thread workgroups as the GPU holds at once.
// Rows are dealt round robin to eight groups that match the eight XCDs
// (workgroup b runs on XCD b % 8); inside a group, workgroup j takes items
// j, j + G, j + 2G, ... of the group's row-major item list, so the chunks of
// a row run together, in one round, on one XCD, and the 16-byte loads of a
// workgroup's next item are in flight while it works on the current one.
//   phase 1   chunk max m_c; e_k = 2^(l_k s - m_c s), s = log2(e) / T, kept
//             in registers; chunk sum s_c and sums over 32-lane sub-chunks.
//             T = 0: chunk argmax.
//   xch 1     (m_c, s_c) of target and draft go into epoch-tagged slots.
//             Rows with a draft read all of their row's slots and merge
//             them, (max, sum 2^((m_c - M) s)): the row normalisers M, S.
//   phase 2   with a_c = 2^((m_c - M) s) / S for target (t) and draft (d) and
//             rho = a_d / a_t: p_k = a_t e_t and q_k = a_t rho e_d, so
//             min(p, q) = a_t min(e_t, rho e_d) and max(0, p - q) =
//             a_t max(0, e_t - rho e_d).  Chunk sums of both (beta, velog
//             section 2-3 item 1; residual mass Z, item 2) and sub-chunk sums
//             of the residual go out; the chunk holding the drafted token
//             writes p(x) and q(x).
// finish_kernel, one workgroup per sequence and one wave per row, then
// merges the partials: Z and beta; the chunk, then the 32-lane sub-chunk,
// whose CDF interval holds u_gamma * Z (or the CDF of p for the bonus row and
// when Z = 0); the 256 (bf16) or 128 (fp32) logits of that sub-chunk are
// re-read and scanned for the token; the acceptance test u_i q(x) < p(x);
// finally the sequence's first rejection n, accepted_len and the n + 1
// tokens.  The accepted length never leaves the device.
//
// Inside stream_kernel, values cross workgroups only in 64-bit slots that
// carry a 32-bit epoch tag next to the value, written and read with
// agent-scope atomics, so a reader that sees the tag sees the value; no
// fences.  Every wait is bounded; an expired wait is reported as
// accepted_len = -2 and the kernels still end.  finish_kernel reads what
// stream_kernel wrote after the kernel boundary.
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
constexpr int kHalf = 32;                      // lanes per sub-chunk
constexpr int kHalves = kThreads / kHalf;      // sub-chunks per load round
constexpr int kMaxSub = 64;                    // sub-chunks per chunk (fp32 64, bf16 32)
constexpr int kX1 = 4;                         // exchange-1 slots per chunk
constexpr int kPart = 4 + 2 * kMaxSub;         // floats of partials per chunk
constexpr int kMaxGamma = 255;                 // rows per sequence <= 256
constexpr int kFinishWaves = 16;
constexpr int kDefaultSpin = 1 << 18;          // ~0.3 s of polling; normal waits are microseconds
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMin = 1.17549435e-38f;
constexpr float kFltMax = 3.40282347e38f;
constexpr uint32_t kTokMask = (1u << 23) - 1;
constexpr uint32_t kAccBit = 1u << 23;
constexpr uint32_t kStatusShift = 24;          // 0 ok, 1 invalid data, 2 wait expired

// partials of one (row, chunk), floats
constexpr int kPDone = 0;                      // epoch that completed the item (bits)
constexpr int kPW = 1;                         // sum of max(0, e_t - rho e_d)
constexpr int kPB = 2;                         // sum of min(e_t, rho e_d)
constexpr int kPWsub = 4;                      // [kMaxSub] residual sub-chunk sums
constexpr int kPPsub = 4 + kMaxSub;            // [kMaxSub] sub-chunk sums of e_t

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
  int32_t G;                 // stream workgroups per row group
  int32_t max_gamma;
  uint32_t epoch;
  int32_t spin_limit;
  int32_t t_aligned;         // target rows start on 16-byte boundaries
  int32_t d_aligned;
  uint64_t* xch1;            // [rows][C][kX1] tagged slots
  float* part;               // [rows][C][kPart]
  float* rowpart;            // [rows][2]: p(x), q(x)
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
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------ wave primitives (DPP)
// Reductions leave the same value in every lane and use a fixed order, so
// the two kernels, and every workgroup, reduce the same data to the same bits.

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sums of the four 16-lane rows, left in every lane of each row.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
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
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dppi<0xB1>(v));
  v = min(v, dppi<0x4E>(v));
  v = min(v, dppi<0x141>(v));
  v = min(v, dppi<0x140>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dppi<0xB1>(v));
  v = max(v, dppi<0x4E>(v));
  v = max(v, dppi<0x141>(v));
  v = max(v, dppi<0x140>(v));
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
  const float v2 = __int_as_float(dppi<CTRL>(__float_as_int(v)));
  const int k2 = dppi<CTRL>(k);
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
  for (int l = 16; l < 64; l += 16) argmax_merge(bv, bk, lane_f(v, l), __builtin_amdgcn_readlane(k, l));
  v = bv;
  k = bk;
}

// Row normalisers of a softmax split into chunks: lane c (< C) holds chunk c's
// (max m, sum s of 2^(l s_T - m s_T)); the merge is (max, sum 2^((m - M) s_T)).
// Both kernels call this with the same lane layout.
__device__ __forceinline__ void merge_chunks(float m, float sum, bool in, float sT, float& M, float& S) {
  M = wave_max(in ? m : -__builtin_huge_valf());
  S = wave_sum(in ? sum * __builtin_amdgcn_exp2f((m - M) * sT) : 0.0f);
}

// Exponent offset of a chunk: -m s, or 0 for a chunk of only -inf (so that
// its exponentials are 2^-inf = 0 instead of NaN).
__device__ __forceinline__ float chunk_offset(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : -m * s;
}
// Scale of a chunk: p_k = scale * e_k.
__device__ __forceinline__ float chunk_scale(float m, float M, float S, float s) {
  return __builtin_amdgcn_exp2f((m - M) * s) / S;
}
// Weight of one logit pair in the residual, in the chunk's units; the stream
// and finish kernels both use this (built without fp contraction) so the
// finisher's re-scan sees the stream kernel's bits.
__device__ __forceinline__ float resid_w(float et, float ed, float rho) {
  return fmaxf(et - rho * ed, 0.0f);
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

// EPV logits starting at token k (fewer near V: -inf), as fp32.
template <int DT>
__device__ __forceinline__ void load_group(const void* base, int64_t row, int64_t stride, int64_t k,
                                           int V, bool aligned, float (&x)[Fmt<DT>::EPV]) {
  using F = Fmt<DT>;
  const char* rowp = (const char*)base + row * stride * F::ESIZE;
  u32x4 raw;
  if (aligned && k + F::EPV <= V) {
    raw = *(const u32x4*)(rowp + k * F::ESIZE);
  } else if (DT == SPECVERIFY_F32) {
    const uint32_t* p = (const uint32_t*)rowp;
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = (k + e < V) ? p[k + e] : 0xFF800000u;
  } else {
    const uint16_t* p = (const uint16_t*)rowp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (k + 2 * e < V) ? p[k + 2 * e] : 0xFF80u;
      const uint32_t hi = (k + 2 * e + 1 < V) ? p[k + 2 * e + 1] : 0xFF80u;
      raw[e] = lo | (hi << 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (DT == SPECVERIFY_F32) {
      x[e] = __uint_as_float(raw[e]);
    } else {
      x[2 * e] = __uint_as_float(raw[e] << 16);
      x[2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
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

// ------------------------------------------------------------------ sequence layout

struct Seq {
  int b, gam, d0;
  bool ok;
};
// The sequence owning target row r (binary search of cu_t[b] = cu_draft[b] + b).
__device__ __forceinline__ Seq seq_of_row(const Params& P, int r) {
  Seq q;
  if (P.cu_draft == nullptr) {
    q.b = r / (P.gamma + 1);
    q.gam = P.gamma;
    q.d0 = q.b * P.gamma;
  } else {
    int lo = 0, hi = P.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P.cu_draft[mid] + mid <= r) lo = mid;
      else hi = mid - 1;
    }
    q.b = lo;
    q.d0 = P.cu_draft[lo];
    q.gam = P.cu_draft[lo + 1] - q.d0;
  }
  const int i = r - (q.d0 + q.b);
  q.ok = q.gam >= 0 && q.gam <= P.max_gamma && q.d0 >= 0 && q.d0 + q.gam <= P.R_d && i >= 0 && i <= q.gam;
  return q;
}

// ================================================================== stream kernel

struct Item {
  int r, c;       // target row, chunk
  int b, i, rd;   // sequence, position, draft row
  bool ok, pair;
  float T;
  int xtok;
};

__device__ __forceinline__ void item_place(const Params& P, int grp, int idx, Item& it) {
  const int rl = idx / P.C;
  it.c = idx - rl * P.C;
  it.r = rl * kGroups + grp;
}
// Sequence of the item's row and its per-row scalars; the loads overlap the
// work on the current item.
__device__ __forceinline__ void item_lookup(const Params& P, Item& it) {
  const Seq q = seq_of_row(P, it.r);
  it.b = q.b;
  it.i = it.r - (q.d0 + q.b);
  it.rd = q.d0 + it.i;
  it.ok = q.ok;
  it.pair = q.ok && it.i < q.gam;
  it.T = q.ok ? P.temps[q.b] : 0.0f;
  it.xtok = it.pair ? P.tokens[it.rd] : 0;
}

struct StreamShared {
  float red[2 * kWaves];
  int redi[2 * kWaves];
  uint32_t x1[kX1 * kMaxChunks];
  float Mt, St, Md, Sd;
};

__device__ __forceinline__ void block_max2(float& a, float& b, StreamShared& sh) {
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
__device__ __forceinline__ void block_sum2(float& a, float& b, StreamShared& sh) {
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
__device__ __forceinline__ void block_argmax(float& v, int& k, StreamShared& sh) {
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

// Sums over each 32-lane half of the wave; lane 0 of the wave writes the two
// halves of the u-th load round to dst[u * kHalves + 2 * wave + {0, 1}].
__device__ __forceinline__ void store_halves(float v, float* dst, int u) {
  const float r = row_sum16(v);
  const float h0 = lane_f(r, 0) + lane_f(r, 16);
  const float h1 = lane_f(r, 32) + lane_f(r, 48);
  if ((threadIdx.x & 63) == 0) {
    const int w = threadIdx.x >> 6;
    dst[u * kHalves + 2 * w] = h0;
    dst[u * kHalves + 2 * w + 1] = h1;
  }
}

// Per-thread argmax of a chunk in token order (first maximum wins) plus a
// flag for NaN / +inf.
template <int DT>
__device__ __forceinline__ void thread_argmax(const float (&x)[kPerThread], int64_t e0, int tid,
                                              float& bv, int& bk, int& bad) {
  using F = Fmt<DT>;
  bv = -__builtin_huge_valf();
  int slot = -1;
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

// Greedy rows (T = 0, or an invalid temperature that only needs reporting):
// chunk argmax of target and draft into the exchange-1 slots.
template <int DT>
__device__ __forceinline__ void stream_greedy(const Params& P, const Item& it, const float (&xt)[kPerThread],
                                              const float (&xd)[kPerThread], StreamShared& sh) {
  const int tid = threadIdx.x;
  const int64_t e0 = (int64_t)it.c * kChunk;
  float vt, vd = -__builtin_huge_valf();
  int kt, kd = 0x7FFFFFFF, badt = 0, badd = 0;
  thread_argmax<DT>(xt, e0, tid, vt, kt, badt);
  if (it.pair) thread_argmax<DT>(xd, e0, tid, vd, kd, badd);
  badt = __syncthreads_or(badt);
  badd = __syncthreads_or(badd);
  block_argmax(vt, kt, sh);
  if (it.pair) block_argmax(vd, kd, sh);
  if (tid < kX1) {
    const uint32_t v = tid == 0 ? __float_as_uint(vt) : tid == 1 ? (badt ? 0xFFFFFFFFu : (uint32_t)kt)
                     : tid == 2 ? __float_as_uint(vd) : (badd ? 0xFFFFFFFFu : (uint32_t)kd);
    slot_put(P.xch1 + ((int64_t)it.r * P.C + it.c) * kX1 + tid, P.epoch, v);
  }
}

// Sampled rows (T > 0): phases 1 and 2 of one chunk.
template <int DT>
__device__ __forceinline__ void stream_sampled(const Params& P, const Item& it, float (&xt)[kPerThread],
                                               float (&xd)[kPerThread], StreamShared& sh) {
  using F = Fmt<DT>;
  constexpr int EPV = F::EPV;
  constexpr int U = F::U;
  const int tid = threadIdx.x, lane = tid & 63, C = P.C;
  const uint32_t tag = P.epoch;
  const bool pair = it.pair;
  uint64_t* x1row = P.xch1 + (int64_t)it.r * C * kX1;
  float* part = P.part + ((int64_t)it.r * C + it.c) * kPart;
  const float s = kLog2e / it.T;
  const float ninf = -__builtin_huge_valf();

  // ---- phase 1: chunk max, exponentials kept in registers, sums
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
  float gt[U];
  float st = 0.0f, sd = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int k = u * EPV + e;
      xt[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(xt[k], s, ct));
      a += xt[k];
    }
    gt[u] = a;
    st += a;
  }
  if (pair) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int k = u * EPV + e;
        xd[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[k], s, cd));
        a += xd[k];
      }
      sd += a;
    }
  }
  block_sum2(st, sd, sh);
  if (tid < kX1) {
    const float v = tid == 0 ? mt : tid == 1 ? st : tid == 2 ? md : sd;
    slot_put(x1row + (int64_t)it.c * kX1 + tid, tag, __float_as_uint(v));
  }
#pragma unroll
  for (int u = 0; u < U; ++u) store_halves(gt[u], part + kPPsub, u);
  if (!pair) {
    if (tid == 0) part[kPDone] = __uint_as_float(tag);
    return;
  }

  // ---- exchange 1: the row's normalisers (M, S) of target and draft
  int ok = 1;
  if (tid < kX1 * C) {
    uint32_t v = 0;
    ok = slot_get(x1row + tid, tag, P.spin_limit, v);
    sh.x1[tid] = v;
  }
  if (!__syncthreads_and(ok)) return;   // the finisher sees no completion mark and reports
  if (tid < 64) {
    const bool in = lane < C;
    float Mt, St, Md, Sd;
    merge_chunks(__uint_as_float(sh.x1[lane * kX1 + 0]), __uint_as_float(sh.x1[lane * kX1 + 1]), in, s, Mt, St);
    merge_chunks(__uint_as_float(sh.x1[lane * kX1 + 2]), __uint_as_float(sh.x1[lane * kX1 + 3]), in, s, Md, Sd);
    if (lane == 0) {
      sh.Mt = Mt;
      sh.St = St;
      sh.Md = Md;
      sh.Sd = Sd;
    }
  }
  __syncthreads();
  const float Mt = sh.Mt, St = sh.St, Md = sh.Md, Sd = sh.Sd;
  const bool norm_ok = Mt > ninf && St == St && St > 0.0f && Md > ninf && Sd == Sd && Sd > 0.0f;
  if (!norm_ok) {   // invalid data: the finisher reports it from the slots
    if (tid == 0) part[kPDone] = __uint_as_float(tag);
    return;
  }
  const float at = chunk_scale(mt, Mt, St, s);   // p_k = at e_t
  const float ad = chunk_scale(md, Md, Sd, s);   // q_k = ad e_d
  const float rho = ad / at;                     // q_k = at rho e_d

  // ---- phase 2: sums of min(e_t, rho e_d) and max(0, e_t - rho e_d)
  float wsub[U];
  float bsum = 0.0f, wsum = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float ws = 0.0f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int k = u * EPV + e;
      bsum += fminf(xt[k], rho * xd[k]);
      ws += resid_w(xt[k], xd[k], rho);
    }
    wsub[u] = ws;
    wsum += ws;
  }
  block_sum2(wsum, bsum, sh);
#pragma unroll
  for (int u = 0; u < U; ++u) store_halves(wsub[u], part + kPWsub, u);
  // the chunk holding the drafted token: p(x) and q(x)
  const int x = it.xtok;
  if (x >= it.c * kChunk && x < (it.c + 1) * kChunk && x < P.V) {
    const int loc = x - it.c * kChunk;
    const int u = loc / (kThreads * EPV);
    const int rem = loc - u * kThreads * EPV;
    if (tid == rem / EPV) {
      const int e = rem - (rem / EPV) * EPV;
      float et = 0.0f, ed = 0.0f;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (k == u * EPV + e) {
          et = xt[k];
          ed = xd[k];
        }
      P.rowpart[(int64_t)it.r * 2 + 0] = et * at;
      P.rowpart[(int64_t)it.r * 2 + 1] = ed * ad;
    }
  }
  if (tid == 0) {
    part[kPW] = wsum;
    part[kPB] = bsum;
    part[kPDone] = __uint_as_float(tag);
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void stream_kernel(Params P) {
  using F = Fmt<DT>;
  __shared__ StreamShared sh;
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
    issue_chunk<DT>(P.draft, it.rd, P.dstride, (int64_t)it.c * kChunk, P.V, tid, P.d_aligned, rdr);
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
      if (nx.pair) issue_chunk<DT>(P.draft, nx.rd, P.dstride, (int64_t)nx.c * kChunk, P.V, tid, P.d_aligned, rdr);
    }
    if (it.ok) {
      __syncthreads();   // shared state of the previous item is no longer read
      const bool sampled = it.T >= kFltMin && it.T <= kFltMax;
      if (sampled) stream_sampled<DT>(P, it, xt, xd, sh);
      else stream_greedy<DT>(P, it, xt, xd, sh);
    }
    if (!more) break;
    idx = nidx;
    it = nx;
  }
}

// ================================================================== finish kernel

struct FinishShared {
  uint32_t res[kMaxGamma + 1];   // row results of the sequence
  int bad_layout;
};

__device__ __forceinline__ uint32_t row_payload(int status, bool acc, int tok) {
  return ((uint32_t)status << kStatusShift) | (acc ? kAccBit : 0u) |
         (status == 0 ? ((uint32_t)tok & kTokMask) : 0u);
}

// Owner selection over n <= 64 non-negative totals, one per lane: the first j
// with tot_j > 0 and base + incl_j > thr, else the last j with tot_j > 0
// (rounding guard).  Returns j (-1 if all are 0) and the CDF value before j.
__device__ __forceinline__ int owner_select(float tot, int n, float base, float thr, int lane,
                                            float& before) {
  const float t = lane < n ? tot : 0.0f;
  const float G = base + wave_scan(t, lane);
  const uint64_t hit = __ballot(lane < n && t > 0.0f && G > thr);
  const uint64_t pos = __ballot(lane < n && t > 0.0f);
  int j;
  if (hit) j = __builtin_ctzll(hit);
  else if (pos) j = 63 - __builtin_clzll(pos);
  else j = -1;
  const float prev = lane_f(G, j > 0 ? j - 1 : 0);
  before = j > 0 ? prev : base;
  return j;
}

// One row of a sampled sequence, on one wave.  Returns the row result.
template <int DT>
__device__ __forceinline__ uint32_t finish_sampled(const Params& P, int r, int rd, bool pair, float T,
                                                   float ui, float ug, int lane) {
  using F = Fmt<DT>;
  constexpr int EPV = F::EPV;
  const int C = P.C;
  const uint32_t tag = P.epoch;
  const float s = kLog2e / T;
  const float ninf = -__builtin_huge_valf();
  const bool in = lane < C;
  const int NSUB = kHalves * F::U;
  // chunk statistics and partials
  float m1 = ninf, s1 = 0.0f, m2 = ninf, s2 = 0.0f, W = 0.0f, Bs = 0.0f;
  int ok = 1;
  if (in) {
    const uint64_t* x1 = P.xch1 + ((int64_t)r * C + lane) * kX1;
    const uint64_t a = __hip_atomic_load(x1 + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t bb = __hip_atomic_load(x1 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t c = __hip_atomic_load(x1 + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t d = __hip_atomic_load(x1 + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = ((uint32_t)(a >> 32) == tag) & ((uint32_t)(bb >> 32) == tag) & ((uint32_t)(c >> 32) == tag) &
         ((uint32_t)(d >> 32) == tag);
    m1 = __uint_as_float((uint32_t)a);
    s1 = __uint_as_float((uint32_t)bb);
    m2 = __uint_as_float((uint32_t)c);
    s2 = __uint_as_float((uint32_t)d);
    const float* pt = P.part + ((int64_t)r * C + lane) * kPart;
    ok &= __float_as_uint(pt[kPDone]) == tag;
    W = pt[kPW];
    Bs = pt[kPB];
  }
  if (!__all(ok)) return row_payload(2, false, 0);
  float Mt, St, Md = ninf, Sd = 0.0f;
  merge_chunks(m1, s1, in, s, Mt, St);
  if (pair) merge_chunks(m2, s2, in, s, Md, Sd);
  const bool norm_ok = Mt > ninf && St == St && St > 0.0f &&
                       (!pair || (Md > ninf && Sd == Sd && Sd > 0.0f));
  const int x = pair ? P.tokens[rd] : 0;
  if (!norm_ok || (pair && (x < 0 || x >= P.V))) return row_payload(1, false, 0);
  // chunk scales, residual mass and beta
  const float at = in ? chunk_scale(m1, Mt, St, s) : 0.0f;
  const float ad = (in && pair) ? chunk_scale(m2, Md, Sd, s) : 0.0f;
  const float rho = (in && pair) ? ad / at : 0.0f;
  float Z = 0.0f, beta = 0.0f;
  if (pair) {
    Z = wave_sum(in ? at * W : 0.0f);
    beta = wave_sum(in ? at * Bs : 0.0f);
  }
  const bool resid = pair && Z > 0.0f;
  const float tot = in ? (resid ? at * W : at * s1) : 0.0f;
  const float mass = resid ? Z : wave_sum(tot);
  const float thr = ug * mass;
  float before;
  const int cs = owner_select(tot, C, 0.0f, thr, lane, before);
  if (cs < 0) return row_payload(2, false, 0);   // unreachable for a valid row
  const float a_s = lane_f(at, cs);
  const float rho_s = lane_f(rho, cs);
  const float ct = chunk_offset(lane_f(m1, cs), s);
  const float cd = chunk_offset(lane_f(m2, cs), s);
  // sub-chunk sums of the owner chunk, in p units
  const float* pc = P.part + ((int64_t)r * C + cs) * kPart + (resid ? kPWsub : kPPsub);
  const float sub = lane < NSUB ? a_s * pc[lane] : 0.0f;
  float before2;
  const int ss = owner_select(sub, NSUB, before, thr, lane, before2);
  if (ss < 0) return row_payload(2, false, 0);
  // re-read the sub-chunk: 32 lanes x EPV logits, token order lane then element
  const int su = ss / kHalves, sg = ss - su * kHalves;
  const int64_t kb = (int64_t)cs * kChunk + (int64_t)su * kThreads * EPV + (int64_t)sg * kHalf * EPV;
  const int64_t k0 = kb + (int64_t)lane * EPV;
  float w[EPV];
  {
    float lt[EPV], ld[EPV];
    if (lane < kHalf) {
      load_group<DT>(P.target, r, P.tstride, k0, P.V, P.t_aligned, lt);
      if (resid) load_group<DT>(P.draft, rd, P.dstride, k0, P.V, P.d_aligned, ld);
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      float wv = 0.0f;
      if (lane < kHalf) {
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(lt[e], s, ct));
        wv = resid ? resid_w(et, __builtin_amdgcn_exp2f(__builtin_fmaf(ld[e], s, cd)), rho_s) : et;
      }
      w[e] = wv;
    }
  }
  // running sums in the chunk's units against tau = (thr - before2) / a_s
  const float tau = (thr - before2) / a_s;
  float loc[EPV];
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    run += w[e];
    loc[e] = run;
  }
  const float incl = wave_scan(lane < kHalf ? run : 0.0f, lane);
  const float excl = incl - (lane < kHalf ? run : 0.0f);
  int first = 0x7FFFFFFF, lastpos = -1;
  if (lane < kHalf) {
#pragma unroll
    for (int e = EPV - 1; e >= 0; --e)
      if (w[e] > 0.0f && excl + loc[e] > tau) first = lane * EPV + e;
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      if (w[e] > 0.0f) lastpos = lane * EPV + e;
  }
  first = wave_min_i(first);
  lastpos = wave_max_i(lastpos);
  const int pick = first != 0x7FFFFFFF ? first : lastpos;
  if (pick < 0) return row_payload(2, false, 0);   // unreachable: the sub-chunk has weight > 0
  const int tok = (int)(kb + pick);
  if (tok >= P.V) return row_payload(2, false, 0);
  bool acc = false;
  if (pair) {
    const float px = P.rowpart[(int64_t)r * 2 + 0];
    const float qx = P.rowpart[(int64_t)r * 2 + 1];
    acc = ui * qx < px;
    if (lane == 0) {
      if (P.p_draft) P.p_draft[rd] = px;
      if (P.q_draft) P.q_draft[rd] = qx;
      if (P.beta) P.beta[rd] = beta;
      if (P.resid) P.resid[rd] = Z;
    }
  }
  return row_payload(0, acc, tok);
}

// One row of a greedy (or invalid-temperature) sequence, on one wave.
__device__ __forceinline__ uint32_t finish_greedy(const Params& P, int r, int rd, bool pair, bool t_ok,
                                                  int lane) {
  const int C = P.C;
  const uint32_t tag = P.epoch;
  const bool in = lane < C;
  float av = -__builtin_huge_valf(), dv = -__builtin_huge_valf();
  int ak = 0x7FFFFFFF, dk = 0x7FFFFFFF, bad = 0, ok = 1;
  if (in) {
    const uint64_t* x1 = P.xch1 + ((int64_t)r * C + lane) * kX1;
    const uint64_t a = __hip_atomic_load(x1 + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t bb = __hip_atomic_load(x1 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t c = __hip_atomic_load(x1 + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t d = __hip_atomic_load(x1 + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = ((uint32_t)(a >> 32) == tag) & ((uint32_t)(bb >> 32) == tag) & ((uint32_t)(c >> 32) == tag) &
         ((uint32_t)(d >> 32) == tag);
    av = __uint_as_float((uint32_t)a);
    dv = __uint_as_float((uint32_t)c);
    bad = ((uint32_t)bb == 0xFFFFFFFFu) || (pair && (uint32_t)d == 0xFFFFFFFFu);
    ak = (int)(uint32_t)bb;
    dk = (int)(uint32_t)d;
  }
  if (!__all(ok)) return row_payload(2, false, 0);
  bad = __any(bad);
  wave_argmax(av, ak);
  wave_argmax(dv, dk);
  if (!t_ok || bad || av == -__builtin_huge_valf() || (pair && dv == -__builtin_huge_valf()))
    return row_payload(1, false, 0);
  bool acc = false;
  if (pair) {
    const int x = P.tokens[rd];
    if (x < 0 || x >= P.V) return row_payload(1, false, 0);
    acc = (x == ak);
    if (lane == 0) {
      if (P.p_draft) P.p_draft[rd] = (x == ak) ? 1.0f : 0.0f;
      if (P.q_draft) P.q_draft[rd] = (x == dk) ? 1.0f : 0.0f;
      if (P.beta) P.beta[rd] = (ak == dk) ? 1.0f : 0.0f;
      if (P.resid) P.resid[rd] = (ak == dk) ? 0.0f : 1.0f;
    }
  }
  return row_payload(0, acc, ak);
}

template <int DT>
__global__ __launch_bounds__(64 * kFinishWaves) void finish_kernel(Params P) {
  __shared__ FinishShared sh;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int d0, gam;
  bool layout_ok;
  if (P.cu_draft == nullptr) {
    d0 = b * P.gamma;
    gam = P.gamma;
    layout_ok = true;
  } else {
    d0 = P.cu_draft[b];
    gam = P.cu_draft[b + 1] - d0;
    layout_ok = d0 >= 0 && gam >= 0 && gam <= P.max_gamma && d0 + gam <= P.R_d &&
                P.cu_draft[0] == 0 && P.cu_draft[P.B] == P.R_d;
  }
  if (!layout_ok) {   // the rows of this sequence are unknown: report only
    if (threadIdx.x == 0) P.acc_len[b] = -1;
    return;
  }
  const int t0 = d0 + b;
  const float T = P.temps[b];
  const bool t_ok = (T == 0.0f) || (T >= kFltMin && T <= kFltMax);
  const bool sampled = t_ok && T > 0.0f;
  const float ug = P.uniforms[t0 + gam];
  for (int j = wv; j <= gam; j += nw) {
    const bool pair = j < gam;
    const int r = t0 + j, rd = d0 + j;
    const uint32_t res = sampled ? finish_sampled<DT>(P, r, rd, pair, T, P.uniforms[r], ug, lane)
                                 : finish_greedy(P, r, rd, pair, t_ok, lane);
    if (lane == 0) sh.res[j] = res;
  }
  __syncthreads();
  if (wv != 0) return;
  // first rejection n, accepted length and the n + 1 tokens
  int n = gam, st = 0;
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t v = j <= gam ? sh.res[j] : 0u;
    st = max(st, wave_max_i((int)(v >> kStatusShift)));
    const uint64_t rb = __ballot(j < gam && !(v & kAccBit));
    if (n == gam && rb) n = j0 + __builtin_ctzll(rb);
  }
  const int tn = (int)(sh.res[n] & kTokMask);
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    if (j <= gam) {
      int o = -1;
      if (st == 0) o = (j < n) ? P.tokens[d0 + j] : (j == n ? tn : -1);
      P.out_tokens[t0 + j] = o;
    }
  }
  if (lane == 0) P.acc_len[b] = st == 2 ? -2 : st == 1 ? -1 : n;
}

int chunks_for(int V) { return (V + kChunk - 1) / kChunk; }

}  // namespace

struct specverify_ctx {
  specverify_config cfg;
  int chunks;
  int64_t rows;            // max target rows
  int cap;                 // stream workgroups resident at once on the device
  void* ws;
  size_t ws_bytes;
  uint64_t* xch1;
  float* part;
  float* rowpart;
  uint32_t epoch;
  int timing;              // recording events
  int trec;                // runs recorded since the measurement started
  hipEvent_t* ev;          // [SPECVERIFY_TIMING_RUNS][3], created on first use
};

extern "C" {

specverify_status specverify_create(const specverify_config* cfg, specverify_handle* out) {
  if (out) *out = nullptr;
  if (!cfg || !out) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (cfg->max_batch < 1 || cfg->max_gamma < 0 || cfg->max_gamma > kMaxGamma || cfg->vocab < 1 ||
      cfg->spin_limit < 0 || (cfg->dtype != SPECVERIFY_F32 && cfg->dtype != SPECVERIFY_BF16))
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
  const size_t n1 = (size_t)rows * h->chunks * kX1 * sizeof(uint64_t);
  const size_t n2 = (size_t)rows * h->chunks * kPart * sizeof(float);
  const size_t n3 = (size_t)rows * 2 * sizeof(float);
  h->ws_bytes = n1 + n2 + n3;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(cfg->device) != hipSuccess) {
    delete h;
    return SPECVERIFY_ERR_DEVICE;
  }
  // residency of the persistent stream grid: workgroups per CU times CUs
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cfg->device);
  if (e == hipSuccess)
    e = cfg->dtype == SPECVERIFY_F32
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<SPECVERIFY_F32>, kThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<SPECVERIFY_BF16>, kThreads, 0);
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
  h->ws = p;
  h->xch1 = (uint64_t*)p;
  h->part = (float*)((char*)p + n1);
  h->rowpart = (float*)((char*)p + n1 + n2);
  h->epoch = 0;
  h->timing = 0;
  h->trec = 0;
  h->ev = nullptr;
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
  const int gmax = in->cu_draft == nullptr ? in->gamma : h->cfg.max_gamma;
  const int fwaves = gmax + 1 < kFinishWaves ? gmax + 1 : kFinishWaves;

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
  P.max_gamma = h->cfg.max_gamma;
  P.epoch = h->epoch;
  P.spin_limit = h->cfg.spin_limit;
  P.t_aligned = t_aligned;
  P.d_aligned = d_aligned;
  P.xch1 = h->xch1;
  P.part = h->part;
  P.rowpart = h->rowpart;
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
  hipError_t e = hipSuccess;
  hipEvent_t* ev = nullptr;
  if (h->timing && h->trec < SPECVERIFY_TIMING_RUNS) ev = h->ev + 3 * h->trec++;
  if (ev) e = hipEventRecord(ev[0], stream);
  if (h->cfg.dtype == SPECVERIFY_F32) {
    hipLaunchKernelGGL(stream_kernel<SPECVERIFY_F32>, grid, dim3(kThreads), 0, stream, P);
    if (ev && e == hipSuccess) e = hipEventRecord(ev[1], stream);
    hipLaunchKernelGGL(finish_kernel<SPECVERIFY_F32>, dim3(B), dim3(64 * fwaves), 0, stream, P);
  } else {
    hipLaunchKernelGGL(stream_kernel<SPECVERIFY_BF16>, grid, dim3(kThreads), 0, stream, P);
    if (ev && e == hipSuccess) e = hipEventRecord(ev[1], stream);
    hipLaunchKernelGGL(finish_kernel<SPECVERIFY_BF16>, dim3(B), dim3(64 * fwaves), 0, stream, P);
  }
  if (ev && e == hipSuccess) e = hipEventRecord(ev[2], stream);
  const hipError_t e2 = hipGetLastError();
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return (e == hipSuccess && e2 == hipSuccess) ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_destroy(specverify_handle h) {
  if (!h) return SPECVERIFY_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->cfg.device);
  if (h->ev)
    for (int k = 0; k < 3 * SPECVERIFY_TIMING_RUNS; ++k) (void)hipEventDestroy(h->ev[k]);
  delete[] h->ev;
  (void)hipFree(h->ws);
  (void)hipSetDevice(prev);
  delete h;
  return SPECVERIFY_OK;
}

specverify_status specverify_set_timing(specverify_handle h, int32_t enable) {
  if (!h) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (enable && !h->ev) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
    hipEvent_t* ev = new (std::nothrow) hipEvent_t[3 * SPECVERIFY_TIMING_RUNS];
    int n = 0;
    hipError_t e = ev ? hipSuccess : hipErrorOutOfMemory;
    for (; e == hipSuccess && n < 3 * SPECVERIFY_TIMING_RUNS; ++n) e = hipEventCreate(&ev[n]);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      for (int k = 0; k < n - 1; ++k) (void)hipEventDestroy(ev[k]);
      delete[] ev;
      return SPECVERIFY_ERR_DEVICE;
    }
    h->ev = ev;
  }
  h->timing = enable ? 1 : 0;
  if (enable) h->trec = 0;
  return SPECVERIFY_OK;
}

specverify_status specverify_timing_totals(specverify_handle h, int32_t* runs, float* stream_ms,
                                           float* finish_ms) {
  if (!h || !runs || !stream_ms || !finish_ms) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  *runs = 0;
  *stream_ms = 0.0f;
  *finish_ms = 0.0f;
  if (h->trec == 0) return SPECVERIFY_OK;
  const hipEvent_t* ev = h->ev;
  if (hipEventSynchronize(ev[3 * (h->trec - 1) + 2]) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  double a = 0.0, f = 0.0;
  for (int k = 0; k < h->trec; ++k) {
    float x = 0.0f, y = 0.0f;
    if (hipEventElapsedTime(&x, ev[3 * k], ev[3 * k + 1]) != hipSuccess ||
        hipEventElapsedTime(&y, ev[3 * k + 1], ev[3 * k + 2]) != hipSuccess)
      return SPECVERIFY_ERR_DEVICE;
    a += x;
    f += y;
  }
  *runs = h->trec;
  *stream_ms = (float)a;
  *finish_ms = (float)f;
  h->trec = 0;
  return SPECVERIFY_OK;
}

int32_t specverify_chunks_per_row(specverify_handle h) { return h ? h->chunks : 0; }
int64_t specverify_workspace_bytes(specverify_handle h) { return h ? (int64_t)h->ws_bytes : 0; }

}  // extern "C"
