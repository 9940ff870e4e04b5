// HIP kernels and C ABI of the speculative-decoding verification sampler,
// written for AMD CDNA4 (gfx950, MI355X).
//
// What is computed (velog "6-1편. Speculative Decoding", section 2
// "알고리즘 4단계" steps 2-4 with section 2-1, the min(1, p/q) rule, and
// section 2-2, the residual norm(max(0, p - q)); greedy rule of "How to
// Scale Your Model -- All About Transformer Inference", Appendix D): see
// include/specverify.h.
//
// A run launches up to three kernels on the caller's stream.
//
// layout_kernel (ragged batches only) checks cu_draft and writes one
// record per target row: sequence, draft row, whether the position has a
// draft, temperature.
//
// stream_kernel reads every logit from HBM exactly once.  Its unit of work
// is an item: 4 KB of one target row (a chunk of 2048 bf16 or 1024 fp32
// logits) plus the same chunk of the draft row when the position has one,
// so p_k and q_k of a token meet in the same lane.  One wave owns one item
// at a time; the four waves of a workgroup are independent (no barriers,
// no LDS).  The grid is persistent (what the GPU holds at once).  Rows are
// dealt round robin to eight groups matching the eight XCDs (workgroup b
// runs on XCD b % 8); wave j of a group takes items j, j + Gw, j + 2 Gw, ...
// of the group's row-major item list, so the chunks of a row are handled in
// one round by waves of one XCD.
//   phase 1   chunk max m_c (DPP), e_k = 2^(l_k s - m_c s) with s = log2(e)/T
//             kept in registers, chunk sum s_c; (m_c, s_c) of target and
//             draft go out in epoch-tagged slots.  T = 0: chunk argmax.
//   phase 2   once every chunk of the row has published: the row normalisers
//             (M, S) = merge of (m_c, s_c); with a_c = 2^((m_c - M) s) / S and
//             rho = a_d / a_t, p_k = a_t e_t and q_k = a_t rho e_d, so
//             min(p, q) = a_t min(e_t, rho e_d) and max(0, p - q) =
//             a_t (e_t - min(e_t, rho e_d)); the chunk sums of both (beta,
//             velog section 2-3 item 1; residual mass Z, item 2) go out.
// The waves are software pipelined: a step runs phase 1 of item k + 1, then
// polls item k's row and runs its phase 2, with the 16-byte loads of items
// k + 2 and k + 3 in flight.  Logits are read with buffer loads: a row
// without a draft gets a zero-sized buffer, so every item issues the same
// loads and none of them touches memory it should not.
//
// stream_t_kernel replaces stream_kernel when a run has no draft logits
// (token-only drafts, q = delta_x; or no drafts at all): phase 1 only, one
// item per wave, no exchange.  The chunk that holds a drafted token x also
// publishes e_t at x.
//
// finish_kernel, one workgroup per sequence and one wave per row, then
// merges the partials: Z and beta; the chunk whose CDF interval holds
// u_gamma * Z (or the CDF of p for the bonus row and when Z = 0), whose
// logits it re-reads; p(x) and q(x) from the two logits of the drafted token
// (a token-only draft: e_t at x from the slots, q(x) = 1); the acceptance
// test u_i q(x) < p(x); for a rejected row, the scan of the re-read chunk
// in token order for the token; finally the sequence's first rejection n,
// accepted_len and the n + 1 tokens.  The accepted length never leaves the
// device.
//
// commit_kernel (its own call, specverify_commit) appends each sequence's
// n + 1 emitted tokens to its token row on the device.
//
// Inside stream_kernel, values cross waves only in 64-bit slots that carry a
// 32-bit epoch tag next to the value.  A slot is written with one aligned
// 64-bit store (the CU's L1 writes through to the XCD's L2) and polled with
// loads that skip L1 and read that L2; the waves that meet over a row all run
// on one XCD, so a reader that sees the tag sees the value, without fences or
// atomics.  Nothing guarantees that every workgroup of the grid is resident
// at once, so a wave that has polled spin_limit times reads the chunks that
// are still missing and computes their statistics itself (bit-identical to
// what their owners publish); every wait therefore ends.  finish_kernel reads
// what stream_kernel wrote after the kernel boundary.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <new>

#include "specverify.h"

namespace {

constexpr int kStreamWaves = 4;                // independent waves per stream workgroup
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kU = 4;                          // 16-byte loads per lane and row of an item
constexpr int kRowBytes = kU * 64 * 16;        // bytes of one row in one item (4 KB)
constexpr int kMaxChunks = 256;                // chunks per fp32 row (V <= 262144)
constexpr int kMaxChunksBf16 = 128;            // chunks per bf16 row (V <= 262144)
constexpr int kGroups = 8;                     // row groups = XCDs of an MI355X
constexpr int kX1 = 4;                         // exchange slots per (row, chunk)
constexpr int kPart = 4;                       // floats of partials per (row, chunk)
constexpr int kMaxGamma = 255;                 // rows per sequence <= 256
constexpr int kFinishWaves = 8;
constexpr int kLayoutThreads = 1024;
constexpr int kDefaultSpin = 64;               // polls (~1 us each) before a wave computes missing chunks itself
constexpr int kMaxSpin = 1 << 20;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMin = 1.17549435e-38f;
constexpr float kFltMax = 3.40282347e38f;
constexpr uint32_t kTokMask = (1u << 23) - 1;
constexpr uint32_t kAccBit = 1u << 23;
constexpr uint32_t kStatusShift = 24;          // 0 ok, 1 invalid data, 2 wait expired
constexpr int kRsrcWord3 = 0x00020000;         // raw (untyped) buffer, gfx9 family
constexpr int kNT = 2;                         // buffer-load cache policy: nontemporal

// Partials of one (row, chunk), kPart floats: the epoch that completed the
// item (bits), the sum of e_t - min(e_t, rho e_d), the sum of
// min(e_t, rho e_d), unused.

template <int DT> struct Fmt;
template <> struct Fmt<SPECVERIFY_F32> {
  static constexpr int EPV = 4;   // logits per 16-byte vector
  static constexpr int ESIZE = 4;
  static constexpr int L = kU * EPV;   // logits per lane and row of an item
  static constexpr int CH = 64 * L;    // logits per chunk
};
template <> struct Fmt<SPECVERIFY_BF16> {
  static constexpr int EPV = 8;
  static constexpr int ESIZE = 2;
  static constexpr int L = kU * EPV;
  static constexpr int CH = 64 * L;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

struct Params {
  const char* target;
  const char* draft;
  int64_t tstride_b;         // row strides in bytes
  int64_t dstride_b;
  const int32_t* tokens;
  const float* uniforms;
  const float* temps;
  const int32_t* cu_draft;   // NULL: uniform gamma
  const int4* rowinfo;       // ragged: per target row {sequence (<0: bad layout), draft row, has draft, T bits}
  const uint32_t* layout;    // ragged: epoch * 2 + (layout invalid)
  int32_t gamma;
  int32_t B;
  int32_t R_d;
  int32_t R_t;
  int32_t V;
  int32_t C;                 // chunks per row
  int32_t Gw;                // stream waves per row group
  int32_t max_gamma;
  uint32_t epoch;
  int32_t spin_limit;
  int32_t token_only;        // drafts come without logits: q_i = delta_{x_i}
  uint32_t div_c[3];         // unsigned division by C: multiplier and two shifts
  uint32_t div_g[3];         // unsigned division by gamma + 1 (uniform gamma)
  uint64_t* xch1;            // [rows][C][kX1] tagged slots
  uint64_t* dummy;           // [stream waves][8]: where a wave's step with nothing to publish writes
  float* part;               // [rows][C][kPart]
  int32_t* acc_len;
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* beta;
  float* resid;
};

// ------------------------------------------------------------------ slots

// One 64-bit store (single-copy atomic); the CU's L1 writes it through to
// the XCD's L2, where the sc0 loads of the other waves of the row find it.
__device__ __forceinline__ void slot_put(uint64_t* p, uint32_t tag, uint32_t v) {
  *p = ((uint64_t)tag << 32) | v;
}
__device__ __forceinline__ uint32_t slot_tag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float slot_f(uint64_t w) { return __uint_as_float((uint32_t)w); }

// ------------------------------------------------------------------ wave primitives (DPP)
// Reductions use a fixed order, so the two kernels, and every wave, reduce
// the same data to the same bits.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK,
                                                    0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum over the 64 lanes: a butterfly inside each 16-lane row, then
// row_bcast:15 and row_bcast:31 fold the rows as (r3 + r2) + (r1 + r0).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  v += dpp_rows<0x142, 0xa>(v, 0.0f);   // rows 1, 3 += last lane of rows 0, 2
  v += dpp_rows<0x143, 0xc>(v, 0.0f);   // rows 2, 3 += lane 31
  return lane_f(v, 63);
}
// Max over the 64 lanes on order-preserving integer keys of the floats
// (integer max needs no NaN quieting, so each step is one DPP max); a
// positive NaN would win, which only makes an invalid row invalid.
__device__ __forceinline__ int f2key(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key2f(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
template <int CTRL>
__device__ __forceinline__ int dpp_all(int v) {    // every lane has a source lane
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ float wave_max(float f) {
  int v = f2key(f);
  v = max(v, dpp_all<0xB1>(v));
  v = max(v, dpp_all<0x4E>(v));
  v = max(v, dpp_all<0x141>(v));
  v = max(v, dpp_all<0x140>(v));
  // every lane holds its row's max: fold the four rows on the scalar unit
  const int a = max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
  const int b = max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48));
  return key2f(max(a, b));
}
// Inclusive prefix sum over the 64 lanes, fixed association.
__device__ __forceinline__ float wave_scan(float v, int lane) {
  v += dpp<0x111>(v);   // row_shr:1 (bound_ctrl: 0 enters at the row start)
  v += dpp<0x112>(v);   // row_shr:2
  v += dpp<0x114>(v);   // row_shr:4
  v += dpp<0x118>(v);   // row_shr:8
  const float t0 = lane_f(v, 15), t1 = lane_f(v, 31), t2 = lane_f(v, 47);
  const float t01 = t0 + t1, t012 = t01 + t2;
  // the offset of the lane's row of 16, by selects (a chained conditional
  // here compiled to branches on the lane)
  const int row = lane >> 4;
  float off = row >= 1 ? t0 : 0.0f;
  off = row >= 2 ? t01 : off;
  off = row >= 3 ? t012 : off;
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
// (v2, k2) wins over (v, k) if larger, or equal with a lower index.  Written
// without short-circuit evaluation: selects, not branches.
__device__ __forceinline__ void argmax_merge(float& v, int& k, float v2, int k2) {
  const bool take = (v2 > v) | ((v2 == v) & (k2 < k));
  v = take ? v2 : v;
  k = take ? k2 : k;
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

// Exponent offset of a chunk: -m s, or 0 for a chunk of only -inf (so that
// its exponentials are 2^-inf = 0 instead of NaN).
__device__ __forceinline__ float chunk_offset(float m, float s) {
  return (m == -__builtin_huge_valf()) ? 0.0f : -m * s;
}
// Scale of a chunk: p_k = scale * e_k.
__device__ __forceinline__ float chunk_scale(float m, float M, float S, float s) {
  return __builtin_amdgcn_exp2f((m - M) * s) / S;
}
// rho = a_d / a_t of a chunk (q_k = a_t rho e_d), from the chunk maxima and
// the row normalisers: 2^(((m_d - M_d) - (m_t - M_t)) s) S_t / S_d.  Both
// kernels take it from this function, so a chunk's residual weights
// e_t - min(e_t, rho e_d) have the same bits in both.
__device__ __forceinline__ float chunk_rho(float mt, float Mt, float St, float md, float Md, float Sd, float s) {
  return __builtin_amdgcn_exp2f(((md - Md) - (mt - Mt)) * s) * (St * __builtin_amdgcn_rcpf(Sd));
}
// min(a, b) of two floats that are >= 0 (+0, positive, +inf or a positive
// NaN): the unsigned order of their bit patterns is their order, NaN above
// everything, as fminf treats it.  One integer instruction; fminf would add
// a canonicalisation of each operand.
__device__ __forceinline__ float min_nonneg(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}
// Weight of one logit pair in the residual, in the chunk's units: e_t minus
// min(e_t, rho e_d).
__device__ __forceinline__ float resid_w(float et, float ed, float rho) {
  return et - min_nonneg(et, rho * ed);
}

// ------------------------------------------------------------------ chunk slots of a row

// The exchange slots of every chunk of row r, lane-major: lane l holds
// chunks l, l + 64, ...  Lanes past the last chunk read the dummy slots.
template <int NPER>
struct RowSlots {
  uint64_t w[NPER][kX1];
};
// Byte offsets of a lane's slots inside a row (loop invariant; lanes past
// the last chunk re-read the last one, whose values they never use).
template <int NPER>
__device__ __forceinline__ void slot_offsets(int C, int lane, uint32_t (&off)[NPER]) {
#pragma unroll
  for (int j = 0; j < NPER; ++j) off[j] = (uint32_t)min(lane + 64 * j, C - 1) * (kX1 * sizeof(uint64_t));
}
// The slots of row r, read two at a time with 16-byte buffer loads that miss
// the CU's L1 (sc1) and are served by the XCD's L2 (0.5 us per launch faster
// than one 8-byte load per slot), through a buffer over the row's slots:
// a uniform base and loop-invariant lane offsets, so no vector register is
// written before the loads issue.  `real` false: a zero-sized buffer, the
// loads read zeros (tag 0 is never an epoch) and touch no memory.
constexpr int kSC0 = 16;   // sc1: the load misses L1 and reads L2
template <int NPER>
__device__ __forceinline__ void slots_issue(const Params& P, int r, bool real, const uint32_t (&off)[NPER],
                                            RowSlots<NPER>& q) {
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc((void*)(P.xch1 + (int64_t)(real ? r : 0) * P.C * kX1),
                                                    (short)0, real ? P.C * kX1 * (int)sizeof(uint64_t) : 0,
                                                    kRsrcWord3);
#pragma unroll
  for (int j = 0; j < NPER; ++j)
#pragma unroll
    for (int k = 0; k < kX1; k += 2) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off[j] + k * 8, 0, kSC0);
      q.w[j][k] = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
      q.w[j][k + 1] = (uint64_t)v[2] | ((uint64_t)v[3] << 32);
    }
}
// Every chunk's first `n` slots carry `tag` (wave-uniform answer).
template <int NPER>
__device__ __forceinline__ bool slots_ready(const RowSlots<NPER>& q, int C, uint32_t tag, int n, int lane) {
  bool ok = true;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) {
#pragma unroll
      for (int k = 0; k < kX1; ++k)
        if (k < n) ok &= slot_tag(q.w[j][k]) == tag;
    }
  return __all(ok);
}
// Row normalisers of a softmax split into chunks from slots (m_c, s_c) at
// slot index `at`: M = max m_c, S = sum s_c 2^((m_c - M) s).  Both kernels
// call this with the same lane layout.
template <int NPER>
__device__ __forceinline__ void merge_row(const RowSlots<NPER>& q, int C, int at, float s, int lane, float& M,
                                          float& S) {
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) m = fmaxf(m, slot_f(q.w[j][at]));
  M = wave_max(m);
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (lane + 64 * j < C) a += slot_f(q.w[j][at + 1]) * __builtin_amdgcn_exp2f((slot_f(q.w[j][at]) - M) * s);
  S = wave_sum(a);
}
__device__ __forceinline__ bool norm_ok(float M, float S) {
  return M > -__builtin_huge_valf() && S == S && S > 0.0f && S <= kFltMax;
}

// ------------------------------------------------------------------ loads

__device__ __forceinline__ Rsrc row_rsrc(const char* base, int64_t row, int64_t stride_b, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row * stride_b), (short)0, nbytes, kRsrcWord3);
}

// Loads of one row of chunk c: vector u of lane `lane` holds tokens
// c*CH + u*64*EPV + lane*EPV .. +EPV-1.  VEC: 16-byte loads (rows and V*esize
// on 16-byte boundaries); otherwise element loads.  Bytes past the buffer
// read as 0 (the caller turns tokens >= V into -inf).
template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_vec(Rsrc rs, int c, int u, int lane) {
  using F = Fmt<DT>;
  u32x4 w;
  if (VEC) {
    // the lane's offset is loop invariant; the chunk's goes into the scalar offset
    w = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + u * 1024, c * kRowBytes, kNT);
  } else {
    const int t0 = c * F::CH + u * 64 * F::EPV + lane * F::EPV;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (DT == SPECVERIFY_F32) {
        w[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, (t0 + e) * 4, 0, kNT);
      } else {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, (t0 + 2 * e) * 2, 0, kNT);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, (t0 + 2 * e + 1) * 2, 0, kNT);
        w[e] = lo | (hi << 16);
      }
    }
  }
  return w;
}
template <int DT, bool VEC>
__device__ __forceinline__ void issue_row(Rsrc rs, int c, int lane, u32x4 (&raw)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) raw[u] = load_vec<DT, VEC>(rs, c, u, lane);
}

template <int DT>
__device__ __forceinline__ void unpack(const u32x4 (&raw)[kU], float (&x)[Fmt<DT>::L]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
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
// Tokens >= V of the last chunk become -inf, in two rows of the same chunk
// at once: one comparison per token, and one at a time (each comparison's
// lane mask is used at once), which keeps the scalar registers of this rare
// path from crowding the common one.
// TWO false: only x is masked (y may alias it).
template <int DT, bool TWO = true>
__device__ __forceinline__ void mask_tail2(float (&x)[Fmt<DT>::L], float (&y)[Fmt<DT>::L], int c, int V, int lane) {
  using F = Fmt<DT>;
  const int lim = V - (c * F::CH + lane * F::EPV);
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const bool out = u * 64 * F::EPV + e >= lim;
      x[u * F::EPV + e] = out ? -__builtin_huge_valf() : x[u * F::EPV + e];
      if (TWO) y[u * F::EPV + e] = out ? -__builtin_huge_valf() : y[u * F::EPV + e];
      __builtin_amdgcn_sched_barrier(0);
    }
}
// Token of element (u, e) of a lane.
template <int DT>
__device__ __forceinline__ int token_of(int c, int k, int lane) {
  using F = Fmt<DT>;
  const int u = k / F::EPV, e = k - u * F::EPV;
  return c * F::CH + u * 64 * F::EPV + lane * F::EPV + e;
}
// Element e of vector u of a lane, as unpack and mask_tail2 leave it; `lim`
// is V minus the token of element 0 of the vector (tokens >= V are -inf).
template <int DT>
__device__ __forceinline__ float elem(const u32x4& w, int e, int lim) {
  float x;
  if (DT == SPECVERIFY_F32) {
    x = __uint_as_float(w[e]);
  } else {
    const uint32_t h = w[e >> 1];
    x = __uint_as_float((e & 1) ? (h & 0xFFFF0000u) : (h << 16));
  }
  return e >= lim ? -__builtin_huge_valf() : x;
}

// Element e of a lane's 16-byte vector w, as unpack leaves it.
template <int DT>
__device__ __forceinline__ float vec_elem(const u32x4& w, int e) {
  if (DT == SPECVERIFY_F32) return __uint_as_float(w[e]);
  const uint32_t h = w[e >> 1];
  return __uint_as_float((e & 1) ? (h & 0xFFFF0000u) : (h << 16));
}
// Tokens >= V of the last chunk become -inf in the raw words of a row (one
// comparison per token, as in mask_tail2).
template <int DT>
__device__ __forceinline__ void mask_raw(u32x4 (&raw)[kU], int c, int V, int lane) {
  using F = Fmt<DT>;
  const int lim = V - (c * F::CH + lane * F::EPV);
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      const bool out = u * 64 * F::EPV + e >= lim;
      if (DT == SPECVERIFY_F32) {
        raw[u][e] = out ? 0xFF800000u : raw[u][e];
      } else {
        const uint32_t w = raw[u][e >> 1];
        const uint32_t m = (e & 1) ? ((w & 0x0000FFFFu) | 0xFF800000u) : ((w & 0xFFFF0000u) | 0x0000FF80u);
        raw[u][e >> 1] = out ? m : w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ------------------------------------------------------------------ sequence layout

// Read-only inputs that a wave reads at a uniform address go through the
// constant address space, so they become scalar loads (counted apart from
// the vector loads that the pipeline keeps in flight).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Unsigned division of n by a run-time constant d with the constants
// {m, s1, s2} of Granlund and Montgomery ("Division by Invariant Integers
// using Multiplication", 1994, unsigned case): l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1), s2 = max(l - 1, 0);
// then t = mulhi(m, n) and n / d = (t + ((n - t) >> s1)) >> s2 for every
// 32-bit n.  Wave-uniform operands make this a few scalar instructions.
__device__ __forceinline__ uint32_t udiv(uint32_t n, const uint32_t (&k)[3]) {
  const uint32_t t = __umulhi(k[0], n);
  return (t + ((n - t) >> k[1])) >> k[2];
}

struct RowMeta {
  int b;      // sequence (< 0: the batch layout is invalid)
  int rd;     // draft row
  int pair;   // position has a draft
  float T;
};
__device__ __forceinline__ RowMeta row_meta(const Params& P, int r) {
  RowMeta m;
  if (P.rowinfo == nullptr) {
    const int g1 = P.gamma + 1;
    m.b = (int)udiv((uint32_t)r, P.div_g);
    const int i = r - m.b * g1;
    m.pair = i < P.gamma;
    m.rd = m.b * P.gamma + i;
    m.T = ld_const(P.temps, m.b);
  } else {
    const int* info = (const int*)(P.rowinfo + r);
    m.b = ld_const(info, 0);
    m.rd = ld_const(info, 1);
    m.pair = ld_const(info, 2);
    m.T = __int_as_float(ld_const(info, 3));
  }
  return m;
}
__device__ __forceinline__ bool t_sampled(float T) { return T >= kFltMin && T <= kFltMax; }

// ================================================================== layout kernel (ragged batches)

// One workgroup: checks that cu_draft is a layout (cu_draft[0] = 0,
// cu_draft[B] = R_d, 0 <= gamma_b <= max_gamma) and writes every target row's
// record; an invalid layout marks every row.
__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(Params P, int4* rowinfo, uint32_t* flag) {
  const int tid = threadIdx.x;
  int bad = 0;
  for (int b = tid; b < P.B; b += blockDim.x) {
    const int g = P.cu_draft[b + 1] - P.cu_draft[b];
    bad |= g < 0 || g > P.max_gamma;
  }
  if (tid == 0) bad |= P.cu_draft[0] != 0 || P.cu_draft[P.B] != P.R_d;
  bad = __syncthreads_or(bad);
  if (bad) {
    for (int r = tid; r < P.R_t; r += blockDim.x) rowinfo[r] = make_int4(-1, 0, 0, 0);
  } else {
    for (int b = tid; b < P.B; b += blockDim.x) {
      const int d0 = P.cu_draft[b], g = P.cu_draft[b + 1] - d0;
      const int Tb = __float_as_int(P.temps[b]);
      for (int i = 0; i <= g; ++i) rowinfo[d0 + b + i] = make_int4(b, d0 + i, i < g ? 1 : 0, Tb);
    }
  }
  if (tid == 0) *flag = P.epoch * 2u + (bad ? 1u : 0u);
}

// ================================================================== stream kernel

// An item in three scalar registers: target row (bits 0-23) and chunk (bits
// 24-31); draft row (bits 0-23), mode (bits 24-25: 0 nothing to do,
// 1 sampled, 2 greedy) and whether the position has a draft (bit 26);
// log2(e) / T.  Rows < 2^24 and chunks <= 256 fit.
struct Item {
  uint32_t rc, rdf;
  float s;
  __device__ __forceinline__ int r() const { return (int)(rc & 0xFFFFFFu); }
  __device__ __forceinline__ int c() const { return (int)(rc >> 24); }
  __device__ __forceinline__ int rd() const { return (int)(rdf & 0xFFFFFFu); }
  __device__ __forceinline__ int mode() const { return (int)((rdf >> 24) & 3u); }
  __device__ __forceinline__ bool pair() const { return (rdf >> 26) & 1u; }
};

__device__ __forceinline__ Item make_item(const Params& P, int grp, int idx, int n_items) {
  Item it;
  it.rc = 0;
  it.rdf = 0;
  it.s = 0.0f;
  if (idx >= n_items) return it;
  const int rl = (int)udiv((uint32_t)idx, P.div_c);
  const int c = idx - rl * P.C;
  const int r = grp + kGroups * rl;
  it.rc = (uint32_t)r | ((uint32_t)c << 24);
  const RowMeta m = row_meta(P, r);
  if (m.b < 0) return it;   // invalid layout: nothing is read
  uint32_t mode = 0;
  if (t_sampled(m.T)) {
    mode = 1;
    it.s = kLog2e / m.T;
  } else if (m.T == 0.0f) {
    mode = 2;
  }   // any other temperature is invalid data: nothing is read
  // a token-only draft has no logits: its position streams like one without a draft
  it.rdf = (uint32_t)m.rd | (mode << 24) | ((uint32_t)(m.pair != 0 && !P.token_only) << 26);
  return it;
}

// The item's loads: always the same 2 kU (VEC) instructions; absent rows
// read through zero-sized buffers.  issue_target: the target row alone, for
// launches without draft logits.
template <int DT, bool VEC>
__device__ __forceinline__ void issue_item(const Params& P, const Item& it, int lane, u32x4 (&R)[2][kU]) {
  const int nb = P.V * Fmt<DT>::ESIZE;
  const bool live = it.mode() != 0;
  const Rsrc rt = row_rsrc(P.target, live ? it.r() : 0, P.tstride_b, live ? nb : 0);
  const Rsrc rd = row_rsrc(P.draft, (live && it.pair()) ? it.rd() : 0, P.dstride_b, (live && it.pair()) ? nb : 0);
  issue_row<DT, VEC>(rt, it.c(), lane, R[0]);
  issue_row<DT, VEC>(rd, it.c(), lane, R[1]);
}
template <int DT, bool VEC>
__device__ __forceinline__ void issue_target(const Params& P, const Item& it, int lane, u32x4 (&R)[kU]) {
  const bool live = it.mode() != 0;
  const Rsrc rt = row_rsrc(P.target, live ? it.r() : 0, P.tstride_b, live ? P.V * Fmt<DT>::ESIZE : 0);
  issue_row<DT, VEC>(rt, it.c(), lane, R);
}

// Phase 1 of a sampled row: chunk max, exponentials in place, chunk sum.
template <int DT>
__device__ __forceinline__ void p1_row(float (&x)[Fmt<DT>::L], float s, float& m, float& sum) {
  float mm = -__builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < Fmt<DT>::L; ++k) mm = fmaxf(mm, x[k]);
  m = wave_max(mm);
  const float c = chunk_offset(m, s);
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < Fmt<DT>::L; ++k) {
    x[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], s, c));
    a += x[k];
  }
  sum = wave_sum(a);
}

// The statistics p1_row computes for chunk c of a row, read again from
// memory one vector at a time (few registers; a rare path): the same
// operations on the same values in the same order, hence the same bits.
template <int DT, bool VEC>
__device__ __forceinline__ void stats_mem(Rsrc rs, int c, int V, int lane, float s, float& m, float& sum) {
  using F = Fmt<DT>;
  const int lim0 = V - (c * F::CH + lane * F::EPV);
  float mm = -__builtin_huge_valf();
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    const u32x4 w = load_vec<DT, VEC>(rs, c, u, lane);
    const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) mm = fmaxf(mm, elem<DT>(w, e, lim));
  }
  m = wave_max(mm);
  const float off = chunk_offset(m, s);
  float a = 0.0f;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    const u32x4 w = load_vec<DT, VEC>(rs, c, u, lane);
    const int lim = lim0 - u * 64 * F::EPV;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) a += __builtin_amdgcn_exp2f(__builtin_fmaf(elem<DT>(w, e, lim), s, off));
  }
  sum = wave_sum(a);
}

// Chunk argmax of a greedy row (first maximum in token order) and a flag for
// NaN / +inf.
template <int DT>
__device__ __forceinline__ void greedy_row(const float (&x)[Fmt<DT>::L], int c, int lane, float& v, int& k,
                                           int& bad) {
  float bv = -__builtin_huge_valf();
  int slot = -1, b = 0;
#pragma unroll
  for (int j = 0; j < Fmt<DT>::L; ++j) {
    const float y = x[j];
    b |= (y != y) | (y == __builtin_huge_valf());
    if (y > bv) {
      bv = y;
      slot = j;
    }
  }
  int bk = slot < 0 ? 0x7FFFFFFF : token_of<DT>(c, slot, lane);
  wave_argmax(bv, bk);
  v = bv;
  k = bk;
  bad = __any(b);
}

// Phase 1 of an item; publishes the chunk statistics.  `mt`, `md` keep the
// chunk maxima for phase 2.
// Both rows are unpacked whatever the item is, so that on every path the
// compiler sees the item's loads consumed here and never waits for them
// later (rows that were not read hold zeros).  Likewise every path ends in
// the same one store (items with nothing to publish write the dummy slots),
// so the count of memory operations in flight is the same on all paths.
// D false: the launch has no draft logits; only row 0 exists.  `x` (D
// false, sampled rows): a drafted token; if this chunk holds it, slot 2
// carries e_t at x instead of the absent draft's maximum.
template <int DT, bool D = true>
__device__ __forceinline__ void p1_item(const Params& P, const Item& it, int lane, uint64_t* wdummy,
                                        const u32x4 (&R)[2][kU], float (&E)[2][Fmt<DT>::L], float& mt,
                                        float& md, float& st, int x = -1) {
  unpack<DT>(R[0], E[0]);
  if (D) unpack<DT>(R[1], E[1]);
  uint32_t v0 = 0, v1 = 0, v2 = 0, v3 = 0;
  uint64_t* dst = wdummy;
  if (it.mode() != 0) {
    dst = P.xch1 + ((int64_t)it.r() * P.C + it.c()) * kX1;
    if ((it.c() + 1) * Fmt<DT>::CH > P.V) mask_tail2<DT, D>(E[0], E[1], it.c(), P.V, lane);
    if (it.mode() == 1) {
      float sd = 0.0f;
      md = -__builtin_huge_valf();
      p1_row<DT>(E[0], it.s, mt, st);
      if (D && it.pair()) p1_row<DT>(E[1], it.s, md, sd);
      v0 = __float_as_uint(mt);
      v1 = __float_as_uint(st);
      v2 = __float_as_uint(md);
      v3 = __float_as_uint(sd);
      const int t = x - it.c() * Fmt<DT>::CH;   // x's position in the chunk
      if (!D && x >= 0 && x < P.V && t >= 0 && t < Fmt<DT>::CH) {
        using F = Fmt<DT>;
        const int k = (t / (64 * F::EPV)) * F::EPV + t % F::EPV;   // element of lane (t / EPV) % 64
        float ex = 0.0f;
#pragma unroll
        for (int i = 0; i < F::L; ++i) ex = i == k ? E[0][i] : ex;
        v2 = __float_as_uint(lane_f(ex, (t / F::EPV) & 63));
      }
    } else {
      float vt, vd = -__builtin_huge_valf();
      int kt, kd = 0x7FFFFFFF, bt, bd = 0;
      greedy_row<DT>(E[0], it.c(), lane, vt, kt, bt);
      if (D && it.pair()) greedy_row<DT>(E[1], it.c(), lane, vd, kd, bd);
      v0 = __float_as_uint(vt);
      v1 = bt ? 0xFFFFFFFFu : (uint32_t)kt;
      v2 = __float_as_uint(vd);
      v3 = bd ? 0xFFFFFFFFu : (uint32_t)kd;
    }
  }
  uint32_t v = lane == 2 ? v2 : v3;   // selects, not a chain of branches on the lane
  v = lane == 1 ? v1 : v;
  v = lane == 0 ? v0 : v;
  if (lane < kX1) slot_put(dst + lane, P.epoch, v);
}

// A wave that has polled long enough for the slots of its row computes the
// missing chunks' statistics itself (their owners may not even be running:
// nothing guarantees that every workgroup of the grid is resident at once)
// and publishes them; the owners later write the same bits.  The caller
// polls again afterwards.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void help_row(const Params& P, const Item& it, int lane, const RowSlots<NPER>& q) {
  const uint32_t tag = P.epoch;
  uint64_t miss[NPER];   // the slots are not needed past these masks
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    bool m = false;
    if (lane + 64 * j < P.C) {
#pragma unroll
      for (int k = 0; k < kX1; ++k) m |= slot_tag(q.w[j][k]) != tag;
    }
    miss[j] = __ballot(m);
  }
  const int nb = P.V * Fmt<DT>::ESIZE;
  const Rsrc rt = row_rsrc(P.target, it.r(), P.tstride_b, nb);
  const Rsrc rd = row_rsrc(P.draft, it.rd(), P.dstride_b, nb);
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    uint64_t mask = miss[j];
    while (mask) {
      const int c = __builtin_ctzll(mask) + 64 * j;
      mask &= mask - 1;
      float mt, st, md, sd;
      stats_mem<DT, VEC>(rt, c, P.V, lane, it.s, mt, st);
      stats_mem<DT, VEC>(rd, c, P.V, lane, it.s, md, sd);
      if (lane < kX1) {
        float y = lane == 2 ? md : sd;
        y = lane == 1 ? st : y;
        const uint32_t x = __float_as_uint(lane == 0 ? mt : y);
        slot_put(P.xch1 + ((int64_t)it.r() * P.C + c) * kX1 + lane, tag, x);
      }
    }
  }
}

// Phase 2 of a sampled item with a draft, once its row's slots are in `q`
// (`ready`: they all carry this run's tag).  Leaves the partials in `o` and
// their address in `dst`; the caller stores them.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void p2_item(const Params& P, const Item& it, int lane, const uint32_t (&soff)[NPER],
                                        RowSlots<NPER>& q, bool ready,
                                        const float (&E)[2][Fmt<DT>::L], float mt, float md, float st, float4& o,
                                        float*& dst) {
  const uint32_t tag = P.epoch;
  if (!ready) {
    for (int k = 0;; ++k) {
      // the help makes the next poll succeed; the bound only guards that
      if (k > 2 * P.spin_limit + 16) return;   // no completion mark: the finisher reports it
      if (k == P.spin_limit) {
        help_row<DT, VEC, NPER>(P, it, lane, q);
        __builtin_amdgcn_s_waitcnt(0);   // its stores are in L2 before the poll below
      } else {
        __builtin_amdgcn_s_sleep(2);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the loads below are read again on every turn
      slots_issue(P, it.r(), true, soff, q);
      if (slots_ready(q, P.C, tag, kX1, lane)) break;
    }
  }
  float Mt, St, Md, Sd;
  merge_row(q, P.C, 0, it.s, lane, Mt, St);
  merge_row(q, P.C, 2, it.s, lane, Md, Sd);
  // invalid data gives NaN or inf here; the finisher checks the normalisers
  const float rho = chunk_rho(mt, Mt, St, md, Md, Sd, it.s);   // q_k = a_t rho e_d
  // sum of min(e_t, rho e_d); the residual's sum is the chunk sum of e_t
  // (phase 1's st, the same values added in the same order) minus it
  float b = 0.0f;
#pragma unroll
  for (int k = 0; k < Fmt<DT>::L; ++k) b += min_nonneg(E[0][k], rho * E[1][k]);
  const float bs = wave_sum(b);
  o.x = __uint_as_float(tag);
  o.y = fmaxf(st - bs, 0.0f);
  o.z = bs;
  dst = P.part + ((int64_t)it.r() * P.C + it.c()) * kPart;
}

// One pipeline step:
//   phase 1 of n1 (its loads were issued two steps ago; exponentials into
//   Efree), then the poll of cur's row, phase 2 of cur (exponentials in
//   Ecur), then the loads of n3 into n1's buffer, now free.
// The poll goes out after phase 1 of n1, a whole phase after cur's own
// phase 1, so that the other chunks of its row have mostly published by
// then.  Vector memory operations complete in order, so waiting for it also
// waits for n2's loads, issued a step earlier: those are needed next step
// anyway.  (Issuing the poll a step earlier, before n3's loads, measured
// 1 us slower per launch: it more often found the row incomplete.)
// Every path through a step issues the same memory operations (items that
// do not exist read zero-sized buffers and write the dummy slots), so the
// compiler's count of operations in flight is exact at every wait.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ void step(const Params& P, int lane, uint64_t* wdummy, const uint32_t (&soff)[NPER],
                                     RowSlots<NPER>& q,
                                     const Item& cur, const float (&Ecur)[2][Fmt<DT>::L], float cmt, float cmd,
                                     float cst, const Item& n1, u32x4 (&R1)[2][kU], float (&Efree)[2][Fmt<DT>::L],
                                     float& nmt, float& nmd, float& nst, const Item& n3) {
  // Phase 1 publishes what other waves' phase 2 polls for: it runs at a
  // higher issue priority than the other wave of its SIMD (1.2 us faster per
  // launch than equal priorities).
  __builtin_amdgcn_s_setprio(3);
  p1_item<DT>(P, n1, lane, wdummy, R1, Efree, nmt, nmd, nst);
  __builtin_amdgcn_s_setprio(0);
  slots_issue(P, cur.r(), cur.mode() == 1 && cur.pair(), soff, q);
  const bool ready = slots_ready(q, P.C, P.epoch, kX1, lane);   // consumes the poll on every path
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float* dst = (float*)(wdummy + kX1);
  if (cur.mode() == 1 && cur.pair()) p2_item<DT, VEC, NPER>(P, cur, lane, soff, q, ready, Ecur, cmt, cmd, cst, o, dst);
  if (lane == 0) *(float4*)dst = o;
  __builtin_amdgcn_sched_barrier(0);
  issue_item<DT, VEC>(P, n3, lane, R1);
  __builtin_amdgcn_sched_barrier(0);
}

template <int DT, bool VEC, int NPER>
__global__ __launch_bounds__(kStreamThreads, 2) void stream_kernel(Params P) {
  using F = Fmt<DT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = (int)(blockIdx.x % kGroups);
  const int j = (int)(blockIdx.x / kGroups) * kStreamWaves + wave;
  const int n_items = ((P.R_t - grp + kGroups - 1) / kGroups) * P.C;
  if (j >= n_items) return;
  const int G = P.Gw;
  uint32_t soff[NPER];
  slot_offsets(P.C, lane, soff);
  // the wave's own dummy slots: waves never contend for a dummy cache line
  uint64_t* wdummy = P.dummy + ((int64_t)blockIdx.x * kStreamWaves + wave) * 8;

  u32x4 RA[2][kU], RB[2][kU];
  float EA[2][F::L], EB[2][F::L];
  float amt = 0.0f, amd = 0.0f, ast = 0.0f, bmt = 0.0f, bmd = 0.0f, bst = 0.0f;
  RowSlots<NPER> q;
  // prologue: items 0 and 1 in flight, phase 1 of item 0, item 2 in flight
  Item ia = make_item(P, grp, j, n_items);
  Item ib = make_item(P, grp, j + G, n_items);
  issue_item<DT, VEC>(P, ia, lane, RA);
  __builtin_amdgcn_sched_barrier(0);
  issue_item<DT, VEC>(P, ib, lane, RB);
  __builtin_amdgcn_sched_barrier(0);
  p1_item<DT>(P, ia, lane, wdummy, RA, EA, amt, amd, ast);
  __builtin_amdgcn_sched_barrier(0);
  Item ic = make_item(P, grp, j + 2 * G, n_items);
  issue_item<DT, VEC>(P, ic, lane, RA);
  __builtin_amdgcn_sched_barrier(0);
  // Two steps per turn, one exit at the top: when the first step's item is
  // the wave's last, the second step runs on nothing (no waits, dummy writes).
  for (int idx = j; idx < n_items; idx += 2 * G) {
    // cur = ia (EA), n1 = ib (RB), n2 = ic (RA, in flight)
    const Item id = make_item(P, grp, idx + 3 * G, n_items);
    step<DT, VEC, NPER>(P, lane, wdummy, soff, q, ia, EA, amt, amd, ast, ib, RB, EB, bmt, bmd, bst, id);
    // cur = ib (EB), n1 = ic (RA), n2 = id (RB, in flight)
    const Item ie = make_item(P, grp, idx + 4 * G, n_items);
    step<DT, VEC, NPER>(P, lane, wdummy, soff, q, ib, EB, bmt, bmd, bst, ic, RA, EA, amt, amd, ast, ie);
    ia = ic;
    ib = id;
    ic = ie;
  }
  // loads of items past the end read zero-sized buffers; let them land
  __builtin_amdgcn_s_waitcnt(0);
}

// The streaming pass of a launch without draft logits (token-only drafts,
// or gamma = 0 everywhere): phase 1 alone, one item per wave.  No item reads
// another's statistics, so nothing waits on other waves and the grid need
// not be resident at once: it covers every item, and the dispatcher starts
// new waves as others end (measured faster than persistent waves with one to
// four items in flight each).
template <int DT, bool VEC>
__global__ __launch_bounds__(kStreamThreads) void stream_t_kernel(Params P) {
  using F = Fmt<DT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = (int)(blockIdx.x % kGroups);
  const int j = (int)(blockIdx.x / kGroups) * kStreamWaves + wave;
  const int n_items = ((P.R_t - grp + kGroups - 1) / kGroups) * P.C;
  if (j >= n_items) return;
  const Item it = make_item(P, grp, j, n_items);
  if (it.mode() == 0) return;   // nothing to read or publish
  u32x4 R[2][kU];               // row 1 is never loaded or read
  float E[2][F::L];
  issue_target<DT, VEC>(P, it, lane, R[0]);
  // a token-only draft x of this row: the chunk that holds it also publishes
  // e_t at x (slot 2, unused without draft logits), so that the finish needs
  // no dependent read of the logit at x
  int x = -1;
  if (P.token_only && it.mode() == 1) {
    const RowMeta m = row_meta(P, it.r());
    if (m.pair) x = ld_const(P.tokens, m.rd);
  }
  float mt, md, st;
  p1_item<DT, false>(P, it, lane, P.dummy, R, E, mt, md, st, x);
}

// ================================================================== finish kernel

struct FinishShared {
  uint32_t res[kMaxGamma + 1];   // row results of the sequence
};

__device__ __forceinline__ uint32_t row_payload(int status, bool acc, int tok) {
  return ((uint32_t)status << kStatusShift) | (acc ? kAccBit : 0u) |
         (status == 0 ? ((uint32_t)tok & kTokMask) : 0u);
}

template <int NPER>
__device__ __forceinline__ float pick(const float (&a)[NPER], int j) {
  float v = a[0];
#pragma unroll
  for (int i = 1; i < NPER; ++i)
    if (i == j) v = a[i];
  return v;
}

// One logit of a row as fp32 (token t < V).
template <int DT>
__device__ __forceinline__ float load_logit(const char* base, int64_t row, int64_t stride_b, int t) {
  const char* p = base + row * stride_b;
  if (DT == SPECVERIFY_F32) return ((const float*)p)[t];
  return __uint_as_float((uint32_t)((const uint16_t*)p)[t] << 16);
}

// What a row's resolution reads first: its chunk slots, its partials and
// the drafted token.  finish_kernel issues these before the row's
// temperature is known, so that their latency overlaps the scalar loads.
template <int NPER>
struct RowIn {
  RowSlots<NPER> q;
  float4 pt[NPER];   // {tag, W_c, B_c} of the lane's chunks (rows with draft logits)
  int x;             // drafted token (rows with a draft)
};
template <int NPER>
__device__ __forceinline__ void row_loads(const Params& P, int r, int rd, bool pair, int lane, RowIn<NPER>& in) {
  uint32_t soff[NPER];
  slot_offsets(P.C, lane, soff);
  slots_issue(P, r, true, soff, in.q);
  const bool dp = pair && !P.token_only;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int c = lane + 64 * j;
    in.pt[j] = (dp && c < P.C) ? *(const float4*)(P.part + ((int64_t)r * P.C + c) * kPart)
                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  in.x = pair ? ld_const(P.tokens, rd) : 0;
}

// One row of a sampled sequence, on one wave.  Returns the row result.
template <int DT, bool VEC, int NPER>
__device__ __forceinline__ uint32_t finish_sampled(const Params& P, int r, int rd, bool pair, float T, float ui,
                                                   float ug, int lane, const RowIn<NPER>& in) {
  using F = Fmt<DT>;
  const int C = P.C;
  const uint32_t tag = P.epoch;
  const float s = kLog2e / T;
  const float ninf = -__builtin_huge_valf();
  // dp: the draft's logits are there; tk: a token-only draft, q = delta_x
  const bool dp = pair && !P.token_only, tk = pair && P.token_only;
  const int x = in.x;
  const bool x_ok = x >= 0 && x < P.V;
  const RowSlots<NPER>& q = in.q;
  float W[NPER], Bp[NPER];
  int done = 1;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    W[j] = 0.0f;
    Bp[j] = 0.0f;
    if (dp && lane + 64 * j < C) {
      done &= __float_as_uint(in.pt[j].x) == tag;
      W[j] = in.pt[j].y;
      Bp[j] = in.pt[j].z;
    }
  }
  float lx = 0.0f, dx = 0.0f;
  if (dp && x_ok) {   // token-only rows read e_t at x from the slots instead
    lx = load_logit<DT>(P.target, r, P.tstride_b, x);
    dx = load_logit<DT>(P.draft, rd, P.dstride_b, x);
  }
  if (!slots_ready(q, C, tag, dp ? 4 : 2, lane) || !__all(done)) return row_payload(2, false, 0);
  float Mt, St, Md = ninf, Sd = 0.0f;
  merge_row(q, C, 0, s, lane, Mt, St);
  if (dp) merge_row(q, C, 2, s, lane, Md, Sd);
  if (!norm_ok(Mt, St) || (dp && !norm_ok(Md, Sd)) || (pair && !x_ok)) return row_payload(1, false, 0);
  const int cx = x / F::CH;              // the chunk that holds x
  const int lxl = cx & 63, jx = cx >> 6;
  // per-chunk scales, residual mass, beta, and the masses the final sample reads
  float at[NPER], tot[NPER], mt[NPER], md[NPER], rho[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool in = lane + 64 * j < C;
    mt[j] = in ? slot_f(q.w[j][0]) : ninf;
    md[j] = (in && dp) ? slot_f(q.w[j][2]) : ninf;
    at[j] = in ? chunk_scale(mt[j], Mt, St, s) : 0.0f;
    rho[j] = (in && dp) ? chunk_rho(mt[j], Mt, St, md[j], Md, Sd, s) : 0.0f;
  }
  const float mtx = lane_f(pick(mt, jx), lxl);
  // e at x as phase 1 computed it (the same operations on the same values);
  // for a token-only draft phase 1 published it in slot 2 of x's chunk
  float ex;
  if (tk) {
    uint32_t tgx = 0, vx = 0;   // slot 2 of chunk cx, read from its lane
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const uint32_t tj = (uint32_t)__builtin_amdgcn_readlane((int)slot_tag(q.w[j][2]), lxl);
      const uint32_t vj = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)q.w[j][2], lxl);
      tgx = j == jx ? tj : tgx;
      vx = j == jx ? vj : vx;
    }
    if (tgx != tag) return row_payload(2, false, 0);   // not published: internal error
    ex = __uint_as_float(vx);
  } else {
    ex = __builtin_amdgcn_exp2f(__builtin_fmaf(lx, s, chunk_offset(mtx, s)));
  }
  if (tk) {
    // the residual p - delta_x is p without x: the chunk sums of e_t, less
    // x's own e in its chunk
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const bool in = lane + 64 * j < C;
      W[j] = in ? slot_f(q.w[j][1]) : 0.0f;
      if (lane + 64 * j == cx) W[j] = fmaxf(W[j] - ex, 0.0f);
    }
  }
  float zl = 0.0f, bl = 0.0f;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool in = lane + 64 * j < C;
    zl += in ? at[j] * W[j] : 0.0f;
    bl += in ? at[j] * Bp[j] : 0.0f;
  }
  float Z = 0.0f, beta = 0.0f;
  if (pair) {
    Z = wave_sum(zl);
    beta = wave_sum(bl);
  }
  const bool resid = pair && Z > 0.0f;
  float ml = 0.0f;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool in = lane + 64 * j < C;
    tot[j] = !in ? 0.0f : resid ? at[j] * W[j] : at[j] * slot_f(q.w[j][1]);
    ml += tot[j];
  }
  const float mass = resid ? Z : wave_sum(ml);
  const float thr = ug * mass;
  // the owner chunk: first chunk whose cumulative mass exceeds thr (chunks
  // with zero mass never own); rounding guard: the last chunk with mass
  int cs = -1, last = -1;
  float before = 0.0f, last_before = 0.0f, base = 0.0f;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool in = lane + 64 * j < C;
    const float t = in ? tot[j] : 0.0f;
    const float G = base + wave_scan(t, lane);
    const float Gex = G - t;
    const uint64_t hit = __ballot(in && t > 0.0f && G > thr);
    const uint64_t pos = __ballot(in && t > 0.0f);
    if (cs < 0 && hit) {
      const int l = __builtin_ctzll(hit);
      cs = 64 * j + l;
      before = lane_f(Gex, l);
    }
    if (pos) {
      const int l = 63 - __builtin_clzll(pos);
      last = 64 * j + l;
      last_before = lane_f(Gex, l);
    }
    base = lane_f(G, 63);
  }
  if (cs < 0) {
    cs = last;
    before = last_before;
  }
  const bool no_owner = cs < 0;   // unreachable for a valid row
  if (no_owner) cs = 0;
  const int ls = cs & 63, js = cs >> 6;
  const float a_s = lane_f(pick(at, js), ls);
  const float rho_s = lane_f(pick(rho, js), ls);
  const float ct = chunk_offset(lane_f(pick(mt, js), ls), s);
  const float cd = chunk_offset(lane_f(pick(md, js), ls), s);
  // re-read the owner chunk and scan its weights in token order
  const int nb = P.V * F::ESIZE;
  u32x4 R[2][kU];
  issue_row<DT, VEC>(row_rsrc(P.target, r, P.tstride_b, nb), cs, lane, R[0]);
  const bool rd_read = resid && dp;
  issue_row<DT, VEC>(row_rsrc(P.draft, rd_read ? rd : 0, P.dstride_b, rd_read ? nb : 0), cs, lane, R[1]);
  // The owner chunk needs only the slots and partials (and, for a token-only
  // draft, x's logit): its loads go out before the acceptance test, whose
  // logits at x may still be in flight.
  // p(x), q(x): the logits at x with their chunk's offset and scale; the
  // acceptance test u q(x) < p(x)
  if (pair) {
    const float mdx = lane_f(pick(md, jx), lxl);
    const float px = chunk_scale(mtx, Mt, St, s) * ex;
    const float qx = tk ? 1.0f : chunk_scale(mdx, Md, Sd, s) * __builtin_amdgcn_exp2f(__builtin_fmaf(dx, s, chunk_offset(mdx, s)));
    if (tk) beta = px;   // sum min(p, delta_x) = p(x)
    if (lane == 0) {
      if (P.p_draft) P.p_draft[rd] = px;
      if (P.q_draft) P.q_draft[rd] = qx;
      if (P.beta) P.beta[rd] = beta;
      if (P.resid) P.resid[rd] = Z;
    }
    // an accepted draft emits itself: its row's residual token is never used
    // (the owner chunk's loads land before the wave goes on)
    if (ui * qx < px) {
      __builtin_amdgcn_s_waitcnt(0);
      return row_payload(0, true, x);   // an accepted row emits its draft
    }
  }
  if (no_owner) return row_payload(2, false, 0);
  if ((cs + 1) * F::CH > P.V) {   // tokens >= V: weight 0
    mask_raw<DT>(R[0], cs, P.V, lane);
    mask_raw<DT>(R[1], cs, P.V, lane);
  }
  // Running sums in the chunk's units against tau = (thr - before) / a_s.
  // Token order inside the chunk is round u (one 16-byte vector per lane),
  // then lane, then element.  Per round: the weights (recomputed with the
  // same functions as phase 2, one branch per row around straight-line
  // code), a wave scan of the lane sums and the first position whose running
  // sum exceeds tau.  Rounds go in order and stop at the first with a hit.
  const float tau = (thr - before) / a_s;
  int first = 0x7FFFFFFF, lastpos = -1;
  float rbase = 0.0f;
#pragma unroll 1
  for (int u = 0; u < kU; ++u) {
    // the round's two vectors, picked by selects (u is wave-uniform)
    u32x4 vt = R[0][0], vd = R[1][0];
#pragma unroll
    for (int i = 1; i < kU; ++i) {
      vt = i == u ? R[0][i] : vt;
      vd = i == u ? R[1][i] : vd;
    }
    float w[F::EPV];
    if (tk && resid) {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e) {   // p without x
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, ct));
        w[e] = token_of<DT>(cs, u * F::EPV + e, lane) == x ? 0.0f : et;
      }
    } else if (resid) {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e)
        w[e] = resid_w(__builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, ct)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vd, e), s, cd)), rho_s);
    } else {
#pragma unroll
      for (int e = 0; e < F::EPV; ++e) w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(vt, e), s, ct));
    }
    float loc[F::EPV];
    float run = 0.0f;
#pragma unroll
    for (int e = 0; e < F::EPV; ++e) {
      run += w[e];
      loc[e] = run;
    }
    const float incl = wave_scan(run, lane);
    const float excl = rbase + (incl - run);
    int cand = 0x7FFFFFFF;
#pragma unroll
    for (int e = F::EPV - 1; e >= 0; --e) {
      const int k = u * 64 * F::EPV + lane * F::EPV + e;   // position inside the chunk
      if (w[e] > 0.0f) {
        if (excl + loc[e] > tau) cand = k;
        lastpos = max(lastpos, k);
      }
    }
    if (__ballot(cand != 0x7FFFFFFF)) {   // positions grow with the round: this round's least hit is the first
      first = wave_min_i(cand);
      break;
    }
    rbase = rbase + lane_f(incl, 63);
  }
  if (first == 0x7FFFFFFF) lastpos = wave_max_i(lastpos);   // every round was scanned
  const int pickk = first != 0x7FFFFFFF ? first : lastpos;
  if (pickk < 0) return row_payload(2, false, 0);   // unreachable: the chunk has weight > 0
  const int tok = cs * F::CH + pickk;
  if (tok >= P.V) return row_payload(2, false, 0);
  return row_payload(0, false, tok);
}

// One row of a greedy sequence, on one wave.
template <int NPER>
__device__ __forceinline__ uint32_t finish_greedy(const Params& P, int r, int rd, bool pair, int lane,
                                                  const RowIn<NPER>& in) {
  const int C = P.C;
  const uint32_t tag = P.epoch;
  // dp: the draft's logits are there; a token-only draft's argmax is x itself
  const bool dp = pair && !P.token_only;
  const RowSlots<NPER>& q = in.q;
  if (!slots_ready(q, C, tag, dp ? 4 : 2, lane)) return row_payload(2, false, 0);
  float av = -__builtin_huge_valf(), dv = -__builtin_huge_valf();
  int ak = 0x7FFFFFFF, dk = 0x7FFFFFFF, bad = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    if (lane + 64 * j < C) {
      argmax_merge(av, ak, slot_f(q.w[j][0]), (int)(uint32_t)q.w[j][1]);
      bad |= (uint32_t)q.w[j][1] == 0xFFFFFFFFu;
      if (dp) {
        argmax_merge(dv, dk, slot_f(q.w[j][2]), (int)(uint32_t)q.w[j][3]);
        bad |= (uint32_t)q.w[j][3] == 0xFFFFFFFFu;
      }
    }
  }
  bad = __any(bad);
  wave_argmax(av, ak);
  wave_argmax(dv, dk);
  if (bad || av == -__builtin_huge_valf() || (dp && dv == -__builtin_huge_valf()))
    return row_payload(1, false, 0);
  bool acc = false;
  if (pair) {
    const int x = in.x;
    if (x < 0 || x >= P.V) return row_payload(1, false, 0);
    if (!dp) dk = x;
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

template <int DT, bool VEC, int NPER>
__global__ __launch_bounds__(64 * kFinishWaves) void finish_kernel(Params P) {
  __shared__ FinishShared sh;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // rows are wave-uniform
  const int nw = blockDim.x >> 6;
  int d0, gam;
  if (P.cu_draft == nullptr) {
    d0 = b * P.gamma;
    gam = P.gamma;
  } else {
    if (*P.layout != P.epoch * 2u) {   // cu_draft is not a layout: every sequence and token is invalid
      if (threadIdx.x == 0) P.acc_len[b] = -1;
      for (int t = b + P.B * (int)threadIdx.x; t < P.R_t; t += P.B * (int)blockDim.x) P.out_tokens[t] = -1;
      return;
    }
    d0 = ld_const(P.cu_draft, b);
    gam = ld_const(P.cu_draft, b + 1) - d0;
  }
  const int t0 = d0 + b;
  const float T = ld_const(P.temps, b);
  const bool sampled = t_sampled(T);
  const bool t_ok = sampled || T == 0.0f;
  const float ug = ld_const(P.uniforms, t0 + gam);
  for (int j = wv; j <= gam; j += nw) {
    const bool pair = j < gam;
    const int r = t0 + j, rd = d0 + j;
    RowIn<NPER> in;
    row_loads(P, r, rd, pair, lane, in);
    uint32_t res;
    if (!t_ok) res = row_payload(1, false, 0);
    else if (sampled) res = finish_sampled<DT, VEC, NPER>(P, r, rd, pair, T, ld_const(P.uniforms, r), ug, lane, in);
    else res = finish_greedy<NPER>(P, r, rd, pair, lane, in);
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
  // rows up to n carry their emitted token: the draft when accepted, the
  // residual or bonus token at n
  for (int j0 = 0; j0 <= gam; j0 += 64) {
    const int j = j0 + lane;
    if (j <= gam) P.out_tokens[t0 + j] = (st == 0 && j <= n) ? (int)(sh.res[j] & kTokMask) : -1;
  }
  if (lane == 0) P.acc_len[b] = st == 2 ? -2 : st == 1 ? -1 : n;
}

// ================================================================== commit kernel

// The commit of a verification step (see specverify_commit in the header):
// one wave per sequence appends its n + 1 emitted tokens to its token row.
struct CommitParams {
  int32_t B, gamma, R_d, capacity;
  const int32_t* cu_draft;   // NULL: uniform gamma
  const int32_t* acc_len;
  const int32_t* out_tokens;
  int32_t* seq_tokens;
  int64_t seq_stride;
  int32_t* seq_lens;
  int32_t* appended;         // may be NULL
  int32_t* next_token;       // may be NULL
};
constexpr int kCommitWaves = 4;

__global__ __launch_bounds__(64 * kCommitWaves) void commit_kernel(CommitParams C) {
  const int lane = threadIdx.x & 63;
  const int b = (int)blockIdx.x * kCommitWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (b >= C.B) return;
  int d0, gam;
  if (C.cu_draft == nullptr) {
    d0 = b * C.gamma;
    gam = C.gamma;
  } else {
    d0 = ld_const(C.cu_draft, b);
    gam = ld_const(C.cu_draft, b + 1) - d0;
  }
  const int n = ld_const(C.acc_len, b);
  // a length the layout does not allow, or a layout outside the run's rows,
  // counts as an invalid sequence: nothing outside the buffers is read
  const bool valid = n >= 0 && n <= gam && d0 >= 0 && d0 + gam <= C.R_d;
  const int k = n + 1;
  const int start = ld_const(C.seq_lens, b);
  const bool fits = valid && start >= 0 && start <= C.capacity - k;
  const int t0 = d0 + b;   // first target row of the sequence
  if (fits) {
    int32_t* row = C.seq_tokens + (int64_t)b * C.seq_stride + start;
    for (int j = lane; j < k; j += 64) row[j] = C.out_tokens[t0 + j];
  }
  if (lane == 0) {
    if (fits) C.seq_lens[b] = start + k;
    if (C.appended) C.appended[b] = fits ? k : valid ? -1 : 0;
    if (C.next_token) C.next_token[b] = fits ? C.out_tokens[t0 + n] : -1;
  }
}

// ================================================================== launch table

typedef void (*KernelFn)(Params);
struct Kernels {
  KernelFn stream, stream_t, finish;   // stream_t: launches without draft logits
};
template <int DT, bool VEC>
Kernels kernels_for(int nper) {
  if (nper == 1) return {stream_kernel<DT, VEC, 1>, stream_t_kernel<DT, VEC>, finish_kernel<DT, VEC, 1>};
  if (nper == 2) return {stream_kernel<DT, VEC, 2>, stream_t_kernel<DT, VEC>, finish_kernel<DT, VEC, 2>};
  // more than 128 chunks per row: fp32 only (the bf16 build would not fit
  // its registers)
  if constexpr (DT == SPECVERIFY_F32)
    return {stream_kernel<DT, VEC, 4>, stream_t_kernel<DT, VEC>, finish_kernel<DT, VEC, 4>};
  return {nullptr, nullptr, nullptr};
}
Kernels kernels_for(int dtype, bool vec, int nper) {
  if (dtype == SPECVERIFY_F32) return vec ? kernels_for<SPECVERIFY_F32, true>(nper) : kernels_for<SPECVERIFY_F32, false>(nper);
  return vec ? kernels_for<SPECVERIFY_BF16, true>(nper) : kernels_for<SPECVERIFY_BF16, false>(nper);
}
int chunk_len(int dtype) { return dtype == SPECVERIFY_F32 ? Fmt<SPECVERIFY_F32>::CH : Fmt<SPECVERIFY_BF16>::CH; }
int chunks_for(int V, int dtype) { return (V + chunk_len(dtype) - 1) / chunk_len(dtype); }
int max_chunks(int dtype) { return dtype == SPECVERIFY_F32 ? kMaxChunks : kMaxChunksBf16; }
int nper_for(int C) { return C <= 64 ? 1 : C <= 128 ? 2 : 4; }
// Constants of udiv for the divisor d >= 1.
void udiv_consts(uint32_t d, uint32_t (&k)[3]) {
  int l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  k[0] = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  k[1] = l < 1 ? l : 1;
  k[2] = l > 1 ? l - 1 : 0;
}

}  // namespace

struct specverify_ctx {
  specverify_config cfg;
  int chunks;
  int nper;
  int64_t rows;            // max target rows
  int cap[2];              // stream workgroups resident at once: [element loads, vector loads]
  void* ws;
  size_t ws_bytes;
  uint64_t* xch1;
  uint64_t* dummy;
  float* part;
  int4* rowinfo;
  uint32_t* layout;
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
  const int C = chunks_for(cfg->vocab, cfg->dtype);
  if (C > max_chunks(cfg->dtype)) return SPECVERIFY_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev)
    return SPECVERIFY_ERR_DEVICE;
  specverify_ctx* h = new (std::nothrow) specverify_ctx();
  if (!h) return SPECVERIFY_ERR_OUT_OF_MEMORY;
  h->cfg = *cfg;
  if (h->cfg.spin_limit == 0) h->cfg.spin_limit = kDefaultSpin;
  if (h->cfg.spin_limit > kMaxSpin) h->cfg.spin_limit = kMaxSpin;
  h->chunks = C;
  h->nper = nper_for(C);
  h->rows = rows;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(cfg->device) != hipSuccess) {
    delete h;
    return SPECVERIFY_ERR_DEVICE;
  }
  // Residency of the persistent stream grid: workgroups per CU times CUs.
  // A row group needs at least C waves, so that the chunks of a row fall
  // into one round or two consecutive ones and their waves meet in time.
  int cus = 0;
  h->cap[0] = h->cap[1] = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cfg->device);
  // A kernel that spilled to scratch would make the runtime allocate scratch
  // at its first launch and spill in its inner loop: such a build is refused
  // rather than run.  (The kernel without draft logits never waits
  // on other waves: its grid is not persistent and needs no residency.)
  int capmax = 0;
  for (int v = 0; v < 6 && e == hipSuccess; ++v) {
    const Kernels K = kernels_for(cfg->dtype, (v & 1) == 1, h->nper);
    const void* fn = (const void*)(v < 2 ? K.stream : v < 4 ? K.stream_t : K.finish);
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, fn);
    if (e == hipSuccess && fa.localSizeBytes > 0) e = hipErrorInvalidConfiguration;
    if (v >= 2) continue;
    int per_cu = 0;
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kStreamThreads, 0);
    h->cap[v] = cus * per_cu;
    if (h->cap[v] > capmax) capmax = h->cap[v];
    if (e == hipSuccess && (h->cap[v] / kGroups) * kStreamWaves < C) e = hipErrorInvalidConfiguration;
  }
  const size_t n1 = (size_t)rows * C * kX1 * sizeof(uint64_t);
  const size_t nd = (size_t)capmax * kStreamWaves * 8 * sizeof(uint64_t);   // dummy slots, per stream wave
  const size_t n2 = (size_t)rows * C * kPart * sizeof(float);
  const size_t n3 = (size_t)rows * sizeof(int4);
  const size_t n4 = 256;                                   // layout flag
  h->ws_bytes = n1 + nd + n2 + n3 + n4;
  void* p = nullptr;
  if (e == hipSuccess) e = hipMalloc(&p, h->ws_bytes);
  if (e == hipSuccess) e = hipMemset(p, 0, h->ws_bytes);   // tag 0 is never an epoch
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    if (p) (void)hipFree(p);
    delete h;
    return e == hipErrorOutOfMemory ? SPECVERIFY_ERR_OUT_OF_MEMORY
           : e == hipErrorInvalidConfiguration ? SPECVERIFY_ERR_UNSUPPORTED
                                               : SPECVERIFY_ERR_DEVICE;
  }
  h->ws = p;
  char* q = (char*)p;
  h->xch1 = (uint64_t*)q;
  h->dummy = (uint64_t*)(q + n1);
  h->part = (float*)(q + n1 + nd);
  h->rowinfo = (int4*)(q + n1 + nd + n2);
  h->layout = (uint32_t*)(q + n1 + nd + n2 + n3);
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
  if (R_d > 0 && !in->draft_tokens) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  // drafts without logits are token-only drafts: q_i = delta_{x_i}
  const bool has_dl = R_d > 0 && in->draft_logits != nullptr;
  if (in->target_stride < V || (has_dl && in->draft_stride < V)) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int esize = h->cfg.dtype == SPECVERIFY_F32 ? 4 : 2;
  if (((uintptr_t)in->target_logits % esize) || (has_dl && ((uintptr_t)in->draft_logits % esize)))
    return SPECVERIFY_ERR_UNSUPPORTED;   // logits must be element aligned
  // 16-byte loads need rows and the row length on 16-byte boundaries;
  // otherwise the kernels read element by element.
  const bool vec = !((uintptr_t)in->target_logits & 15) && !((in->target_stride * esize) & 15) &&
                   !(((int64_t)V * esize) & 15) &&
                   (!has_dl || (!((uintptr_t)in->draft_logits & 15) && !((in->draft_stride * esize) & 15)));

  // Persistent grid: per row group, as many waves as the device holds, never
  // more than the busiest group has items.  Without draft logits: one wave
  // per item.
  const int C = h->chunks;
  const int64_t items_g = ((R_t + kGroups - 1) / kGroups) * C;
  const int64_t need = (items_g + kStreamWaves - 1) / kStreamWaves;
  int64_t wg = has_dl ? h->cap[vec ? 1 : 0] / kGroups : need;
  if (wg > need) wg = need;
  if (wg < 1) wg = 1;
  const int gmax = in->cu_draft == nullptr ? in->gamma : h->cfg.max_gamma;
  const int fwaves = gmax + 1 < kFinishWaves ? gmax + 1 : kFinishWaves;

  if (++h->epoch == 0) h->epoch = 1;   // 0 never tags a slot (workspace is zeroed)
  if (h->epoch >= 0x80000000u) h->epoch = 1;   // the layout flag holds epoch * 2
  Params P;
  P.target = (const char*)in->target_logits;
  P.draft = (const char*)in->draft_logits;
  P.tstride_b = in->target_stride * esize;
  P.dstride_b = in->draft_stride * esize;
  P.tokens = in->draft_tokens;
  P.uniforms = in->uniforms;
  P.temps = in->temperatures;
  P.cu_draft = in->cu_draft;
  P.rowinfo = in->cu_draft ? h->rowinfo : nullptr;
  P.layout = h->layout;
  P.gamma = in->gamma;
  P.B = B;
  P.R_d = (int32_t)R_d;
  P.R_t = (int32_t)R_t;
  P.V = V;
  P.C = C;
  P.Gw = (int32_t)(wg * kStreamWaves);
  P.max_gamma = h->cfg.max_gamma;
  P.epoch = h->epoch;
  P.spin_limit = h->cfg.spin_limit;
  P.token_only = R_d > 0 && !has_dl;
  udiv_consts((uint32_t)C, P.div_c);
  udiv_consts((uint32_t)(in->cu_draft ? 1 : in->gamma + 1), P.div_g);
  P.xch1 = h->xch1;
  P.dummy = h->dummy;
  P.part = h->part;
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
  const Kernels K = kernels_for(h->cfg.dtype, vec, h->nper);
  hipError_t e = hipSuccess;
  hipEvent_t* ev = nullptr;
  if (h->timing && h->trec < SPECVERIFY_TIMING_RUNS) ev = h->ev + 3 * h->trec++;
  if (ev) e = hipEventRecord(ev[0], stream);
  if (in->cu_draft) hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, P, h->rowinfo, h->layout);
  hipLaunchKernelGGL(has_dl ? K.stream : K.stream_t, dim3((uint32_t)(wg * kGroups)), dim3(kStreamThreads), 0, stream, P);
  if (ev && e == hipSuccess) e = hipEventRecord(ev[1], stream);
  hipLaunchKernelGGL(K.finish, dim3(B), dim3(64 * fwaves), 0, stream, P);
  if (ev && e == hipSuccess) e = hipEventRecord(ev[2], stream);
  const hipError_t e2 = hipGetLastError();
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return (e == hipSuccess && e2 == hipSuccess) ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
}

specverify_status specverify_commit(specverify_handle h, const specverify_commit_args* a, void* hip_stream) {
  if (!h || !a) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  const int B = a->batch;
  if (B < 0 || B > h->cfg.max_batch) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (B == 0) return SPECVERIFY_OK;
  int64_t R_d;
  if (a->cu_draft == nullptr) {
    if (a->gamma < 0 || a->gamma > h->cfg.max_gamma) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = (int64_t)B * a->gamma;
  } else {
    if (a->num_draft_rows < 0) return SPECVERIFY_ERR_INVALID_ARGUMENT;
    R_d = a->num_draft_rows;
  }
  if (R_d + B > h->rows) return SPECVERIFY_ERR_INVALID_ARGUMENT;
  if (!a->accepted_len || !a->out_tokens || !a->seq_tokens || !a->seq_lens || a->capacity < 0 ||
      a->seq_stride < a->capacity)
    return SPECVERIFY_ERR_INVALID_ARGUMENT;
  CommitParams C;
  C.B = B;
  C.gamma = a->cu_draft ? 0 : a->gamma;
  C.R_d = (int32_t)R_d;
  C.capacity = a->capacity;
  C.cu_draft = a->cu_draft;
  C.acc_len = a->accepted_len;
  C.out_tokens = a->out_tokens;
  C.seq_tokens = a->seq_tokens;
  C.seq_stride = a->seq_stride;
  C.seq_lens = a->seq_lens;
  C.appended = a->appended;
  C.next_token = a->next_token;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return SPECVERIFY_ERR_DEVICE;
  hipLaunchKernelGGL(commit_kernel, dim3((uint32_t)((B + kCommitWaves - 1) / kCommitWaves)),
                     dim3(64 * kCommitWaves), 0, (hipStream_t)hip_stream, C);
  const hipError_t e = hipGetLastError();
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_ERR_DEVICE;
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
